// bf16-activation MXFP4 contractions for small token counts: the MoE decode
// path (gate_up + SwiGLU, down) and the dense projections (qkv_proj, o_proj,
// lm_head at a few tokens).
//
// These are HBM-bound weight streams (gpt-oss page, "MXFP4 Tensor
// Structure" for the layout; forum page, 59 tok/s "close to" the bandwidth
// ceiling: decode is a bandwidth problem).  Design for gfx950:
//   * each wave owns 16 weight rows (gate_up: 16 gate + the matching 16 up
//     rows) and streams them with 16-byte loads, one MX block per lane per
//     K-group of four blocks;
//   * the E2M1 nibbles are expanded in registers with the scaled FP4->bf16
//     convert (the E8M0 block scale folded in, exact for scale bytes 2..252)
//     and fed to v_mfma_f32_16x16x32_bf16 with the routed tokens as the 16
//     columns; a K-group is four MFMAs, each taking 8 elements of the lane's
//     own block, so the K order inside an MFMA is permuted identically for
//     weights and activations;
//   * fp32 accumulation; SwiGLU, bias and the output rounding are fused into
//     the epilogue.  The SwiGLU output is kept as two bf16 halves hi + lo so
//     that the down projection runs on bf16 MFMAs without a second rounding
//     of h (hi = bf16(h), lo = bf16(h - hi)).
#include "common.hpp"
#include "launch.hpp"

namespace mx {

enum GemvMode { kGateUp = 0, kDown = 1, kDense = 2 };

struct GemvArgs {
  const uint8_t* wb;        // blocks [E, R, nb, 16]
  const uint8_t* ws;        // scales [E, R, nb]
  const uint16_t* bias;     // [E, R] or null
  int64_t rows_per_expert;  // R
  int nout;                 // output rows per expert: I (gate_up), H (down), N (dense)
  int nb;                   // K / 32
  const uint16_t* act;      // gate_up: x [T, K]; dense: x [M, K]; down: h hi [rows, K]
  const uint16_t* act_lo;   // down: h lo [rows, K]
  const int* sorted_pairs;
  int topk;
  const int* tiles;
  const int* offsets;
  const int* status;
  int M;                    // dense rows
  uint16_t* out_hi;         // gate_up: h hi / dense: out bf16
  uint16_t* out_lo;         // gate_up: h lo
  float* y;                 // down
};

template <int MODE>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(GemvArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;   // weight row inside the 16-row group / token column
  const int g = lane >> 4;   // which of the K-group's four blocks this lane loads

  int e, row_begin, row_end;
  if (MODE == kDense) {
    e = 0;
    row_begin = blockIdx.y * 16;
    row_end = min(row_begin + 16, a.M);
  } else {
    if ((int)blockIdx.y >= a.status[kStNumTiles]) return;
    e = a.tiles[2 * blockIdx.y];
    row_begin = a.tiles[2 * blockIdx.y + 1];
    row_end = min(row_begin + kDecodeBM, a.offsets[e + 1]);
  }
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= a.nout) return;

  // activation row feeding MFMA column r
  const int row = row_begin + r;
  const bool col_ok = row < row_end;
  const uint16_t* act0 = a.act;
  const uint16_t* act1 = a.act_lo;
  if (col_ok) {
    if (MODE == kGateUp) {
      const int t = a.sorted_pairs[row] / a.topk;
      act0 += (size_t)t * a.nb * kBlockElems;
    } else {
      act0 += (size_t)row * a.nb * kBlockElems;
      if (MODE == kDown) act1 += (size_t)row * a.nb * kBlockElems;
    }
  }

  const size_t wrow0 = (size_t)e * a.rows_per_expert + n0 + r;
  const size_t wrow1 = wrow0 + a.nout;  // matching up row (gate_up only)
  const uint8_t* wb0 = a.wb + wrow0 * a.nb * kBlockBytes;
  const uint8_t* ws0 = a.ws + wrow0 * a.nb;
  const uint8_t* wb1 = a.wb + wrow1 * a.nb * kBlockBytes;
  const uint8_t* ws1 = a.ws + wrow1 * a.nb;

  v4f acc0 = {0.f, 0.f, 0.f, 0.f};
  v4f acc1 = {0.f, 0.f, 0.f, 0.f};
  const int ngroups = (a.nb + 3) >> 2;

  // software pipeline: group grp+1 is loaded while grp is computed
  uint4 w0n = {0, 0, 0, 0}, w1n = {0, 0, 0, 0};
  uint32_t s0n = 0, s1n = 0;
  uint4 bn[4], bln[4];
  auto load_group = [&](int grp, uint4& w0, uint4& w1, uint32_t& s0, uint32_t& s1, uint4* b,
                        uint4* bl) {
    const int j = grp * 4 + g;
    const bool jok = j < a.nb;
    w0 = make_uint4(0, 0, 0, 0);
    w1 = make_uint4(0, 0, 0, 0);
    s0 = 0;
    s1 = 0;
    if (jok) {
      w0 = *reinterpret_cast<const uint4*>(wb0 + (size_t)j * kBlockBytes);
      s0 = ws0[j];
      if (MODE == kGateUp) {
        w1 = *reinterpret_cast<const uint4*>(wb1 + (size_t)j * kBlockBytes);
        s1 = ws1[j];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[q] = make_uint4(0, 0, 0, 0);
      if (MODE == kDown) bl[q] = make_uint4(0, 0, 0, 0);
    }
    if (jok && col_ok) {
      const uint4* p = reinterpret_cast<const uint4*>(act0 + (size_t)j * kBlockElems);
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = p[q];
      if (MODE == kDown) {
        const uint4* pl = reinterpret_cast<const uint4*>(act1 + (size_t)j * kBlockElems);
#pragma unroll
        for (int q = 0; q < 4; ++q) bl[q] = pl[q];
      }
    }
  };

  load_group(0, w0n, w1n, s0n, s1n, bn, bln);
  for (int grp = 0; grp < ngroups; ++grp) {
    const uint4 w0 = w0n, w1 = w1n;
    const uint32_t s0 = s0n, s1 = s1n;
    uint4 b[4], bl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[q] = bn[q];
      if (MODE == kDown) bl[q] = bln[q];
    }
    if (grp + 1 < ngroups) load_group(grp + 1, w0n, w1n, s0n, s1n, bn, bln);

    const float f0 = e8m0_to_f32(s0);
    const uint32_t wv0[4] = {w0.x, w0.y, w0.z, w0.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v8bf A0 = fp4x8_to_bf16(wv0[q], f0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, as_v8bf(b[q]), acc0, 0, 0, 0);
      if (MODE == kDown)
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, as_v8bf(bl[q]), acc0, 0, 0, 0);
    }
    if (MODE == kGateUp) {
      const float f1 = e8m0_to_f32(s1);
      const uint32_t wv1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v8bf A1 = fp4x8_to_bf16(wv1[q], f1);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, as_v8bf(b[q]), acc1, 0, 0, 0);
      }
    }
  }

  if (!col_ok) return;
  // lane holds output rows n0 + 4g + jj (jj = 0..3) of token column r
  const int nbase = n0 + 4 * g;
  const uint16_t* bias_e = a.bias ? a.bias + (size_t)e * a.rows_per_expert : nullptr;
  if (MODE == kGateUp) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = nbase + jj;
      float gate = acc0[jj], up = acc1[jj];
      if (bias_e) {
        gate += bf16_bits_to_f32(bias_e[i]);
        up += bf16_bits_to_f32(bias_e[a.nout + i]);
      }
      const float h = silu(gate) * up;
      hi[jj] = f32_to_bf16_bits(h);
      lo[jj] = f32_to_bf16_bits(h - bf16_bits_to_f32(hi[jj]));
    }
    const size_t o = (size_t)row * a.nout + nbase;
    *reinterpret_cast<uint2*>(a.out_hi + o) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    *reinterpret_cast<uint2*>(a.out_lo + o) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  } else if (MODE == kDown) {
    float4 v = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
    if (bias_e) {
      v.x += bf16_bits_to_f32(bias_e[nbase + 0]);
      v.y += bf16_bits_to_f32(bias_e[nbase + 1]);
      v.z += bf16_bits_to_f32(bias_e[nbase + 2]);
      v.w += bf16_bits_to_f32(bias_e[nbase + 3]);
    }
    *reinterpret_cast<float4*>(a.y + (size_t)row * a.nout + nbase) = v;
  } else {
    uint32_t o[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v = acc0[jj];
      if (bias_e) v += bf16_bits_to_f32(bias_e[nbase + jj]);
      o[jj] = f32_to_bf16_bits(v);
    }
    *reinterpret_cast<uint2*>(a.out_hi + (size_t)row * a.nout + nbase) =
        make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
  }
}

static dim3 gemv_grid(int nout, int64_t ytiles) {
  return dim3((unsigned)((nout + 63) / 64), (unsigned)ytiles);
}

hipError_t launch_moe_gateup_bf16(const uint16_t* x, const MoeShape& sh, const MoeWeights& w,
                                  const WsPtrs& ws, int64_t ntile_bound, hipStream_t s) {
  GemvArgs a{};
  a.wb = w.w13_blocks;
  a.ws = w.w13_scales;
  a.bias = w.w13_bias;
  a.rows_per_expert = 2 * (int64_t)sh.I;
  a.nout = sh.I;
  a.nb = sh.H / kBlockElems;
  a.act = x;
  a.sorted_pairs = ws.sorted_pairs;
  a.topk = sh.k;
  a.tiles = ws.tiles;
  a.offsets = ws.offsets;
  a.status = ws.status;
  uint16_t* h = static_cast<uint16_t*>(ws.h);
  a.out_hi = h;
  a.out_lo = h + (size_t)sh.T * sh.k * sh.I;
  gemv_bf16_kernel<kGateUp><<<gemv_grid(sh.I, ntile_bound), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_moe_down_bf16(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                int64_t ntile_bound, hipStream_t s) {
  GemvArgs a{};
  a.wb = w.w2_blocks;
  a.ws = w.w2_scales;
  a.bias = w.w2_bias;
  a.rows_per_expert = sh.H;
  a.nout = sh.H;
  a.nb = sh.I / kBlockElems;
  const uint16_t* h = static_cast<const uint16_t*>(ws.h);
  a.act = h;
  a.act_lo = h + (size_t)sh.T * sh.k * sh.I;
  a.tiles = ws.tiles;
  a.offsets = ws.offsets;
  a.status = ws.status;
  a.y = ws.y;
  gemv_bf16_kernel<kDown><<<gemv_grid(sh.H, ntile_bound), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_linear_bf16(const uint16_t* x, int M, int N, int K, const uint8_t* wb,
                              const uint8_t* wsc, const uint16_t* bias, uint16_t* out,
                              hipStream_t s) {
  GemvArgs a{};
  a.wb = wb;
  a.ws = wsc;
  a.bias = bias;
  a.rows_per_expert = N;
  a.nout = N;
  a.nb = K / kBlockElems;
  a.act = x;
  a.M = M;
  a.out_hi = out;
  gemv_bf16_kernel<kDense><<<gemv_grid(N, (M + 15) / 16), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mx
