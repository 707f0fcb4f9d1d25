// BF16 -> MXFP4 weight quantiser (the dense-layer weights the pages keep in
// bf16: gpt-oss page, "MXFP4 Tensor Structure"; spark-vllm page, MXFP4 for
// qkv/o/lm_head).
//
// The steps are those of the gpt-oss page's "Conversion Methodology" (per
// block: amax, scale, E2M1 rounding, packing), with the OCP MX scale rule for
// E8M0: shared exponent X = floor(log2 amax) - 2 (2 = exponent of the largest
// E2M1 magnitude, 6), clamped to [-125, 125] (scale bytes 2..252); codes are
// the nearest E2M1 magnitude of |v| / 2^X with ties to the even mantissa and
// saturation at 6; the sign bit is the input's.
//
// One thread per 32-element block: 64 bytes in (a wave reads 4 KB
// contiguous), 16 bytes of packed nibbles and one scale byte out.  The work
// is a pure stream (HBM-bound); everything is exact integer/power-of-two
// arithmetic, so the codes are bit-exact.
#include "common.hpp"
#include "launch.hpp"

namespace mx {

// Magnitude code of q in [0, 8): count of rounding thresholds passed.  A tie
// at a threshold goes to the code whose mantissa bit is 0, so the boundary
// below an odd code is exclusive (q > t) and below an even code inclusive.
__device__ __forceinline__ uint32_t e2m1_round_mag(float q) {
  return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) +
         (uint32_t)(q >= 1.75f) + (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) +
         (uint32_t)(q > 5.0f);
}

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
    const int x = min(max((int)(amax >> 7) - 127 - 2, -125), 125);
    const float inv = __uint_as_float((uint32_t)(127 - x) << 23);   // 2^-X, a normal fp32
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t bits = (v[i] >> (16 * h)) & 0xffffu;
        const float q = __uint_as_float((bits & 0x7fffu) << 16) * inv;   // exact
        const uint32_t code = e2m1_round_mag(q) | ((bits >> 15) << 3);
        const int e = 2 * i + h;                    // element index in the block
        packed[e >> 3] |= code << (4 * (e & 7));    // element 2k low nibble, 2k+1 high
      }
    }
    *reinterpret_cast<uint4*>(blocks + b * kBlockBytes) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    scales[b] = (uint8_t)(x + 127);
  }
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
