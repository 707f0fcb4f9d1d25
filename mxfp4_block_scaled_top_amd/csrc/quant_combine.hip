// FP8 E4M3 per-tensor quantisation (amax pass + encode pass) and the
// weighted combine of the per-pair expert outputs.
//
// The pages run the MoE contraction with FP8 activations against FP4 weights
// (spark-vllm page, "What's Included") and list full-scale activation
// quantisation as open work ("Numerical Accuracy").  Scale s = fp32(amax/448),
// code = E4M3 round-to-nearest-even, saturating, of the correctly rounded
// fp32 quotient v / s.  This translation unit must be built without fast-math
// so that `/` on float stays correctly rounded.
#include "common.hpp"
#include "launch.hpp"
#include "code_rows.hpp"

namespace mx {

template <bool BF16>
__device__ __forceinline__ void load8(const void* in, int64_t i, float v[8]) {
  if (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
      v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(in) + i);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* in, int64_t i) {
  if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(in)[i]);
  return static_cast<const float*>(in)[i];
}

template <bool BF16>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ in, int64_t n,
                                                   uint32_t* __restrict__ amax_bits) {
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    float v[8];
    load8<BF16>(in, i * 8, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, fabsf(load1<BF16>(in, i)));
  m = wave_max(m);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    // |v| bit patterns order like unsigned integers
    atomicMax(amax_bits, __float_as_uint(b));
  }
}

__device__ __forceinline__ float scale_from_amax(uint32_t bits) {
  const float amax = __uint_as_float(bits);
  return amax > 0.0f ? amax / 448.0f : 1.0f;      // correctly rounded divide
}

// Codes of n values; with row_len < ld (row_len a multiple of 16, n a
// multiple of row_len) value e goes to byte (e / row_len) * ld + e % row_len.
template <bool BF16>
__global__ __launch_bounds__(256) void encode_kernel(const void* __restrict__ in, int64_t n,
                                                     uint8_t* __restrict__ codes,
                                                     const uint32_t* __restrict__ amax_bits,
                                                     float* __restrict__ scale_out, int64_t row_len, int64_t ld) {
  const float s = scale_from_amax(*amax_bits);
  if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out) *scale_out = s;
  const int64_t n16 = n / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    float v[16];
    load8<BF16>(in, i * 16, v);
    load8<BF16>(in, i * 16 + 8, v + 8);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = e4m3_pack4(v[4 * q] / s, v[4 * q + 1] / s, v[4 * q + 2] / s, v[4 * q + 3] / s);
    }
    const int64_t e0 = i * 16;
    const int64_t o = ld == row_len ? e0 : (e0 / row_len) * ld + e0 % row_len;
    *reinterpret_cast<uint4*>(codes + o) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (blockIdx.x == 0)
    for (int64_t i = n16 * 16 + threadIdx.x; i < n; i += blockDim.x)
      codes[i] = (uint8_t)e4m3_encode(load1<BF16>(in, i) / s);
}

// Codes of the activation rows in expert-sorted order (the layout both
// prefill GEMMs read): sorted row inv[t*k + j] holds the codes of token t.
// One block per token: each thread encodes 16 elements once and writes them
// to the token's k sorted rows (pairs whose expert id was skipped have no
// row, inv < 0).
__global__ __launch_bounds__(256) void encode_sorted_rows_kernel(
    const uint16_t* __restrict__ x, int H, int k, const int* __restrict__ inv, uint8_t* __restrict__ codes,
    int64_t ld, const uint32_t* __restrict__ amax_bits, float* __restrict__ scale_out) {
  const float s = scale_from_amax(*amax_bits);
  if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out) *scale_out = s;
  const int64_t t = blockIdx.x;
  for (int c = (int)threadIdx.x * 16; c < H; c += (int)blockDim.x * 16) {
    float v[16];
    load8<true>(x, t * H + c, v);
    load8<true>(x, t * H + c + 8, v + 8);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = e4m3_pack4(v[4 * q] / s, v[4 * q + 1] / s, v[4 * q + 2] / s, v[4 * q + 3] / s);
    }
    const uint4 o = make_uint4(w[0], w[1], w[2], w[3]);
    for (int j = 0; j < k; ++j) {
      const int r = inv[t * k + j];
      if (r >= 0) *reinterpret_cast<uint4*>(codes + (int64_t)r * ld + c) = o;
    }
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

static int grid_for(int64_t units) {
  int64_t b = (units + 255) / 256;
  if (b < 1) b = 1;
  if (b > 4096) b = 4096;
  return (int)b;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t s) {
  fill_u32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

hipError_t launch_amax(const void* in, bool in_bf16, int64_t n, uint32_t* amax_bits,
                       hipStream_t s) {
  // few blocks: every block ends in an atomic on the same word
  int grid = grid_for(n / 8);
  if (grid > 512) grid = 512;
  if (in_bf16) amax_kernel<true><<<grid, 256, 0, s>>>(in, n, amax_bits);
  else amax_kernel<false><<<grid, 256, 0, s>>>(in, n, amax_bits);
  return hipGetLastError();
}

hipError_t launch_encode_fp8(const void* in, bool in_bf16, int64_t n, uint8_t* codes,
                             const uint32_t* amax_bits, float* scale_out, hipStream_t s) {
  const int grid = grid_for(n / 16);
  if (in_bf16) encode_kernel<true><<<grid, 256, 0, s>>>(in, n, codes, amax_bits, scale_out, n, n);
  else encode_kernel<false><<<grid, 256, 0, s>>>(in, n, codes, amax_bits, scale_out, n, n);
  return hipGetLastError();
}

hipError_t launch_encode_fp8_rows(const void* in, bool in_bf16, int64_t rows, int64_t row_len, int64_t ld,
                                  uint8_t* codes, const uint32_t* amax_bits, float* scale_out, hipStream_t s) {
  if (row_len % 16 != 0 || ld < row_len) return hipErrorInvalidValue;
  const int64_t n = rows * row_len;
  const int grid = grid_for(n / 16);
  if (in_bf16) encode_kernel<true><<<grid, 256, 0, s>>>(in, n, codes, amax_bits, scale_out, row_len, ld);
  else encode_kernel<false><<<grid, 256, 0, s>>>(in, n, codes, amax_bits, scale_out, row_len, ld);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_rows(const void* in, bool in_bf16, int64_t rows, int64_t row_len, int64_t ld,
                                 uint8_t* codes, uint32_t* amax_bits, float* scale_out, hipStream_t s) {
  hipError_t e = launch_amax(in, in_bf16, rows * row_len, amax_bits, s);
  if (e != hipSuccess) return e;
  return launch_encode_fp8_rows(in, in_bf16, rows, row_len, ld, codes, amax_bits, scale_out, s);
}

hipError_t launch_encode_sorted_rows(const uint16_t* x, const MoeShape& sh, const WsPtrs& ws,
                                    hipStream_t s) {
  if (sh.T <= 0) return hipSuccess;
  encode_sorted_rows_kernel<<<sh.T, 256, 0, s>>>(
      x, sh.H, sh.k, ws.inv, ws.x_codes, code_row_bytes(sh.H, false),
      reinterpret_cast<const uint32_t*>(ws.status + kStAmaxX),
      reinterpret_cast<float*>(ws.status + kStScaleX));
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* in, bool in_bf16, int64_t n, uint8_t* codes,
                            uint32_t* amax_bits, float* scale_out, hipStream_t s) {
  hipError_t e = launch_amax(in, in_bf16, n, amax_bits, s);
  if (e != hipSuccess) return e;
  return launch_encode_fp8(in, in_bf16, n, codes, amax_bits, scale_out, s);
}

// ------------------------------------------------------------- combine ----
// One thread per (token, 8 consecutive outputs); k slots summed in order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int* __restrict__ inv,
                                                      const float* __restrict__ w, int T,
                                                      int H, int k, uint16_t* __restrict__ out) {
  const int per_row = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per_row) return;
  const int t = (int)(idx / per_row);
  const int n0 = (int)(idx % per_row) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    if (r < 0) continue;
    const float wt = w[(size_t)t * k + j];
    const float4* p = reinterpret_cast<const float4*>(y + (size_t)r * H + n0);
    const float4 a = p[0], b = p[1];
    acc[0] = fmaf(wt, a.x, acc[0]); acc[1] = fmaf(wt, a.y, acc[1]);
    acc[2] = fmaf(wt, a.z, acc[2]); acc[3] = fmaf(wt, a.w, acc[3]);
    acc[4] = fmaf(wt, b.x, acc[4]); acc[5] = fmaf(wt, b.y, acc[5]);
    acc[6] = fmaf(wt, b.z, acc[6]); acc[7] = fmaf(wt, b.w, acc[7]);
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + n0) = o;
}

// The same sums for a fixed k: the k row indices, then all 2k y loads, are
// issued before the first FMA (a skipped pair loads row 0 and is not
// added), so a lane waits for memory twice instead of twice per slot.
template <int K>
__global__ __launch_bounds__(256) void combine_k_kernel(const float* __restrict__ y,
                                                        const int* __restrict__ inv,
                                                        const float* __restrict__ w, int T, int H,
                                                        uint16_t* __restrict__ out) {
  const int per_row = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per_row) return;
  const int t = (int)(idx / per_row);
  const int n0 = (int)(idx % per_row) * 8;
  int r[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    r[j] = inv[(size_t)t * K + j];
    wt[j] = w[(size_t)t * K + j];
  }
  float4 a[K], b[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float4* p = reinterpret_cast<const float4*>(y + (size_t)(r[j] < 0 ? 0 : r[j]) * H + n0);
    a[j] = p[0];
    b[j] = p[1];
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (r[j] < 0) continue;
    acc[0] = fmaf(wt[j], a[j].x, acc[0]); acc[1] = fmaf(wt[j], a[j].y, acc[1]);
    acc[2] = fmaf(wt[j], a[j].z, acc[2]); acc[3] = fmaf(wt[j], a[j].w, acc[3]);
    acc[4] = fmaf(wt[j], b[j].x, acc[4]); acc[5] = fmaf(wt[j], b[j].y, acc[5]);
    acc[6] = fmaf(wt[j], b[j].z, acc[6]); acc[7] = fmaf(wt[j], b[j].w, acc[7]);
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + n0) = o;
}

hipError_t launch_combine(const MoeShape& sh, const float* topk_weights, const WsPtrs& ws,
                          uint16_t* out, hipStream_t s) {
  const int64_t threads = (int64_t)sh.T * (sh.H / 8);
  const int grid = (int)((threads + 255) / 256);
  if (sh.k == 4) combine_k_kernel<4><<<grid, 256, 0, s>>>(ws.y, ws.inv, topk_weights, sh.T, sh.H, out);
  else combine_kernel<<<grid, 256, 0, s>>>(ws.y, ws.inv, topk_weights, sh.T, sh.H, sh.k, out);
  return hipGetLastError();
}

}  // namespace mx
