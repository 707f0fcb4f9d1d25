// Device helpers shared by the gfx950 kernels of the MXFP4 MoE library.
//
// Formats (gpt-oss page, "MXFP4 Tensor Structure"): E2M1 nibbles, two per
// byte with the even element in the low nibble, 32 elements per 16-byte
// block, one E8M0 scale byte 2^(s-127) per block.  Activations in the FP8
// path use the OCP E4M3 encoding (bias 7, largest finite 448).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace mx {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kBlockElems = 32;   // elements per MX block
// Shared-exponent range of the library's MXFP4 quantisers (scale bytes
// 11..252).  Below 11 the scaled FP4 -> bf16 conversion the bf16 and FP8
// contractions use does not give E2M1 * 2^(s-127) (measured: it gives
// E2M1 * (2^s + 3) * 2^-127 for s <= 10), so no quantiser writes such bytes.
constexpr int kMxExpMin = -116;
constexpr int kMxExpMax = 125;
constexpr int kBlockBytes = 16;   // bytes per MX block of E2M1 nibbles

// Indices of the int32 status words at the head of the MoE workspace.
enum StatusWord {
  kStFlags = 0,      // bit 0: a top-k id outside [0, E) was skipped
  kStAmaxX = 1,      // fp32 bits of max|x| (FP8 mode)
  kStAmaxH = 2,      // fp32 bits of max|h| (FP8 mode)
  kStScaleX = 3,     // fp32 bits of the x scale
  kStScaleH = 4,     // fp32 bits of the h scale
  kStNumTiles = 5,   // number of (expert, row-tile) entries in the tile list
  kStWords = 16
};

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// E8M0 byte s -> 2^(s-127) as fp32, exact for s in [1, 254].
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s << 23);
}

// Two OCP E4M3 codes (the low two bytes of c) -> fp32, by the gfx950
// conversion at unit scale: exact for every finite code (subnormals m * 2^-9
// included); the NaN codes S.1111.111 are not expected here.
__device__ __forceinline__ v2f e4m3x2_to_f32(uint32_t c) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
}

// OCP E4M3 code of an fp32 value q: round to nearest, ties to even mantissa,
// saturating to +-448, sign of zero kept.  q must not be NaN.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;          // |q| >= 448
  if (a >= 0x3c800000u) {                               // |q| >= 2^-6: normal
    // keep 3 mantissa bits: round the fp32 pattern at bit 20, ties to even
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    const uint32_t e = (r >> 23) - 120u;                // 127 - 7
    const uint32_t m = (r >> 20) & 7u;
    return sign | (e << 3) | m;
  }
  // subnormal: multiples of 2^-9; |q| * 512 is exact, rintf ties to even
  const float n = rintf(__uint_as_float(a) * 512.0f);
  return sign | (uint32_t)n;
}

// Four E4M3 codes (q0 in the low byte) of fp32 values below 464 in
// magnitude: the hardware conversion equals e4m3_encode on every such fp32
// pattern, both signs (checked exhaustively).  The codec's quotients v / s
// stay within 448 (1 + 2^-23) of zero.
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
}

// E2M1 magnitude code of q >= 0 (|v| / 2^X of the MX block rule): the count
// of rounding thresholds passed.  A tie at a threshold goes to the code whose
// mantissa bit is 0, so the boundary below an odd code is exclusive (q > t)
// and below an even code inclusive; q past 6 saturates at code 7.
__device__ __forceinline__ uint32_t e2m1_round_mag(float q) {
  return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) +
         (uint32_t)(q >= 1.75f) + (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) +
         (uint32_t)(q > 5.0f);
}

// Eight fp32 values already scaled by 2^-X (|q| < 8) -> eight E2M1 nibbles,
// value i in nibble i (low nibble first).  The hardware conversion rounds
// exactly as e2m1_round_mag (nearest, ties to the even mantissa bit,
// saturating at 6) and keeps the sign bit, -0 included: checked on every fp32
// pattern below 8 in magnitude.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* q) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
}

// silu(z) = z / (1 + exp(-z)); exp overflow gives -0 for very negative z.
__device__ __forceinline__ float silu(float z) {
  return __fdividef(z, 1.0f + __expf(-z));
}

// Four E2M1 nibbles pairs (one dword = 8 elements) -> 8 bf16 scaled by `scale`
// (a power of two), element order preserved (low nibble first).
__device__ __forceinline__ v8bf fp4x8_to_bf16(uint32_t w, float scale) {
  v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  v8bf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight E2M1 nibbles (one dword) times a full fp32 factor, as bf16.  The
// scaled FP4 conversions apply only the exponent field of their scale
// operand, so an E4M3 block scale (four significant bits) cannot ride on
// them: the nibbles are converted at unit scale, multiplied in fp32 and
// rounded to bf16.  Every step is exact: an E2M1 value times an E4M3 value
// has at most six significant bits and stays inside bf16's normal range.
__device__ __forceinline__ v8bf fp4x8_times_bf16(uint32_t w, float f) {
  const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v8bf r;
  r[0] = (__bf16)(p0[0] * f); r[1] = (__bf16)(p0[1] * f);
  r[2] = (__bf16)(p1[0] * f); r[3] = (__bf16)(p1[1] * f);
  r[4] = (__bf16)(p2[0] * f); r[5] = (__bf16)(p2[1] * f);
  r[6] = (__bf16)(p3[0] * f); r[7] = (__bf16)(p3[1] * f);
  return r;
}

// An E4M3 block scale f (as fp32) split for the f16 expansion: the power of
// two 2^e the scaled FP4 conversion applies (|f| with its mantissa cleared)
// and the f16 pair (M, M), M = f / 2^e with f's sign (1 <= |M| < 2, three
// mantissa bits: exact in f16); f = 0 gives M = 0.
struct NvScale {
  float pow2;
  uint32_t m2;
};
__device__ __forceinline__ NvScale nv_scale(float f) {
  const uint32_t u = __float_as_uint(f);
  NvScale s;
  s.pow2 = __uint_as_float(u & 0x7f800000u);
  const uint32_t m = (u & 0x7fffffffu) ? (((u >> 16) & 0x8000u) | 0x3c00u | ((u >> 13) & 0x3ffu)) : 0u;
  s.m2 = m | (m << 16);
  return s;
}

// Eight E2M1 nibbles times an E4M3 block scale, as f16, exactly: the scaled
// conversion applies 2^e (E2M1 x 2^e lies in [2^-10, 1536] for the finite
// E4M3 scales) and v_pk_mul_f16 the mantissa M (a product of at most six
// significant bits, below 2^12).  Two instructions per pair of weights,
// against four for the bf16 form.
__device__ __forceinline__ v8h fp4x8_times_f16(uint32_t w, const NvScale& s) {
  const v2h m = __builtin_bit_cast(v2h, s.m2);
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 0) * m;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 1) * m;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 2) * m;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 3) * m;
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ v4f mfma16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma16x16x32(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(uint4 v) {
  return __builtin_bit_cast(v8bf, v);
}

// Streaming (nontemporal) loads for data read exactly once per call, such as
// the weights: on gfx950 they keep the read stream from thrashing the caches
// (measured: 6.3 TB/s for a plain 2 GiB read, against 5.0-5.4 TB/s with
// ordinary loads).
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
  const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream1(const uint8_t* p) {
  return __builtin_nontemporal_load(p);
}

// Wave64 reductions (deterministic xor trees).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace mx
