// BF16 -> MXFP4 weight quantiser (the dense-layer weights the pages keep in
// bf16: gpt-oss page, "MXFP4 Tensor Structure"; spark-vllm page, MXFP4 for
// qkv/o/lm_head).
//
// The steps are those of the gpt-oss page's "Conversion Methodology" (per
// block: amax, scale, E2M1 rounding, packing), with the OCP MX scale rule for
// E8M0: shared exponent X = floor(log2 amax) - 2 (2 = exponent of the largest
// E2M1 magnitude, 6), clamped to [kMxExpMin, kMxExpMax] = [-116, 125] (scale bytes 11..252); codes are
// the nearest E2M1 magnitude of |v| / 2^X with ties to the even mantissa and
// saturation at 6; the sign bit is the input's.
//
// One thread per 32-element block: 64 bytes in (a wave reads 4 KB
// contiguous), 16 bytes of packed nibbles and one scale byte out.  The work
// is a pure stream (HBM-bound); everything is exact integer/power-of-two
// arithmetic, so the codes are bit-exact.
#include "common.hpp"
#include "launch.hpp"
#include "code_rows.hpp"

namespace mx {

__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ w, int64_t nblocks,
                                                          uint8_t* __restrict__ blocks,
                                                          uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
    const uint4* src = reinterpret_cast<const uint4*>(w + b * kBlockElems);
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t = src[i];
      v[4 * i] = t.x;
      v[4 * i + 1] = t.y;
      v[4 * i + 2] = t.z;
      v[4 * i + 3] = t.w;
    }
    // max |v| on the bit patterns: for finite bf16, magnitude order is the
    // order of the low 15 bits
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, max(v[i] & 0x7fffu, (v[i] >> 16) & 0x7fffu));
    // floor(log2 amax) is the bf16 exponent field - 127 for normal amax; zero
    // and subnormal blocks land below the clamp
    const int x = min(max((int)(amax >> 7) - 127 - 2, kMxExpMin), kMxExpMax);
    const float inv = __uint_as_float((uint32_t)(127 - x) << 23);   // 2^-X, a normal fp32
    // elements 2i (low half of v[i]) and 2i + 1 scaled by 2^-X (exact, below
    // 8 in magnitude) -> byte i of the block, element 2i in the low nibble.
    // The hardware conversion rounds exactly as e2m1_round_mag and keeps
    // the sign bit (checked on every fp32 below 8 in magnitude).
    uint32_t packed[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[4 * d + i] << 16) * inv;
        f[2 * i + 1] = __uint_as_float(v[4 * d + i] & 0xffff0000u) * inv;
      }
      packed[d] = e2m1_pack8(f);
    }
    *reinterpret_cast<uint4*>(blocks + b * kBlockBytes) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    scales[b] = (uint8_t)(x + 127);
  }
}

// ---------------------------------------------------------------------------
// MXFP4 activations (FP4 x FP4 MoE mode): the same block rule on x (bf16);
// h is quantised in the gate_up GEMM's epilogue.  Scales are stored step-major: block b of
// row r at ((b / 4) * rows + r) * 4 + b % 4, so one 128-element K step's
// scales of consecutive rows are contiguous; blocks past K (up to the whole
// step) hold 127 (2^0).

// 32 finite fp32 values -> E2M1 nibbles (element 2i in the low nibble of
// byte i) and the E8M0 byte.  For fp32, floor(log2 amax) is the exponent
// field - 127 for a normal amax; zero and subnormal blocks land below the
// clamp.  |v| * 2^-X is exact (a power-of-two scaling that stays below 8).
__device__ __forceinline__ uint32_t mx_encode32(const float* v, uint4& out) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, __float_as_uint(v[i]) & 0x7fffffffu);
  const int x = min(max((int)(amax >> 23) - 127 - 2, kMxExpMin), kMxExpMax);
  const float inv = __uint_as_float((uint32_t)(127 - x) << 23);
  // elements 2j, 2j + 1 -> byte j, by the hardware conversion (rounding and
  // sign as e2m1_round_mag, checked on every fp32 below 8 in magnitude)
  uint32_t packed[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = v[8 * d + i] * inv;
    packed[d] = e2m1_pack8(f);
  }
  out = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  return (uint32_t)(x + 127);
}

// One thread per (token, scale slot c < nbp = whole steps of blocks): block c
// of the token's row (c < H/32) or a pad byte, written to every sorted row
// the token's pairs occupy (inv[t*k + j] >= 0).
__global__ __launch_bounds__(256) void quant_x_mxfp4_sorted_kernel(
    const uint16_t* __restrict__ x, int T, int H, int k, int nbp, const int* __restrict__ inv,
    uint8_t* __restrict__ xb, int64_t ld, uint8_t* __restrict__ xs) {
  const int64_t rows = (int64_t)T * k;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * nbp) return;
  const int t = (int)(idx / nbp), c = (int)(idx - (int64_t)t * nbp);
  const bool real = c < H / kBlockElems;
  uint4 packed = make_uint4(0u, 0u, 0u, 0u);
  uint32_t sc = 127u;
  if (real) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H + c * kBlockElems);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = src[i];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
        v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
    sc = mx_encode32(v, packed);
  }
  for (int j = 0; j < k; ++j) {
    const int r = inv[(int64_t)t * k + j];
    if (r < 0) continue;
    if (real) *reinterpret_cast<uint4*>(xb + (int64_t)r * ld + c * kBlockBytes) = packed;
    xs[((c >> 2) * rows + r) * 4 + (c & 3)] = (uint8_t)sc;
  }
}

hipError_t launch_quant_x_mxfp4_sorted(const uint16_t* x, const MoeShape& sh, const WsPtrs& ws,
                                       hipStream_t s) {
  const int nbp = 4 * ((sh.H + 127) / 128);
  const int64_t n = (int64_t)sh.T * nbp;
  if (n <= 0) return hipSuccess;
  quant_x_mxfp4_sorted_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
      x, sh.T, sh.H, sh.k, nbp, ws.inv, ws.x_codes, code_row_bytes(sh.H, true), ws.x_scales);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4(const uint16_t* w, int64_t nblocks, uint8_t* blocks, uint8_t* scales,
                              hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  const int64_t want = (nblocks + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  quant_mxfp4_kernel<<<grid, 256, 0, s>>>(w, nblocks, blocks, scales);
  return hipGetLastError();
}

}  // namespace mx
