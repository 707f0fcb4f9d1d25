// FP8 x FP4 block-scaled grouped GEMM of the MoE layer (prefill-sized token
// counts): gate_up + SwiGLU (+ max|h|) and down.
//
// spark-vllm page, "What's Included": the MoE layers are an FP8 x FP4
// grouped GEMM whose tile shape and schedule depend on the workload; those
// CUTLASS choices target another GPU and are not reused.  On gfx950 the
// contraction is v_mfma_scale_f32_16x16x128_f8f6f4 with the weights as the
// FP4 (E2M1) operand carrying their own E8M0 block scales straight from the
// checkpoint layout (gpt-oss page, "MXFP4 Tensor Structure") and the
// activations as the OCP E4M3 operand with unit block scale; the per-tensor
// activation scale is applied in the epilogue.
//
// The MFMA used for the gate_up contraction is a template choice.  The
// F8F6F4 instructions sum each 128-long dot product with reduced internal
// precision (measured: errors up to ~2.4e-5 of the sum of |products|), which
// perturbs h enough to move a small fraction of its FP8 codes.  So gate_up,
// whose output is quantised again, expands the FP8 codes and the FP4 weights
// (with their E8M0 block scale) exactly to bf16 and runs
// v_mfma_f32_16x16x32_bf16 (fp32-accurate); down, whose output is not
// quantised, keeps the block-scaled FP8 x FP4 instruction.
//
// Tile: 128 sorted rows (tokens) x 128 weight rows x 128 K per step, 256
// threads.  Both operands are staged through LDS, double buffered, with the
// next K step's global loads in flight while the current one is multiplied.
// Operand layouts of the 16x16x128 instruction (measured): an FP4 lane holds
// 32 consecutive K (= one MX block, matching its scale); an FP8 lane of lane
// group g holds K [16g, 16g+16) and [64+16g, 64+16g+16) of the step.
#include "common.hpp"
#include "launch.hpp"

namespace mx {

constexpr int kBM = kPrefillBM;    // sorted rows per tile
constexpr int kBN = 128;           // weight rows per tile
constexpr int kBK = 128;           // K per step (four MX blocks)
constexpr int kActStride = kBK + 16;        // bytes per activation row in LDS
constexpr int kWStride = kBK / 2 + 16;      // bytes per weight row in LDS
constexpr int kActBytes = kBM * kActStride;
constexpr int kWBytes = kBN * kWStride;
constexpr int kScBytes = kBN * 4;
constexpr int kStageBytes = kActBytes + kWBytes + kScBytes;

struct Fp8Args {
  const uint8_t* wb;        // [E, R, nb, 16]
  const uint8_t* ws;        // [E, R, nb]
  const uint16_t* bias;     // [E, R] or null
  int64_t rows_per_expert;  // R
  int nout;                 // I (gate_up) or H (down)
  int nb;                   // K / 32
  int K;
  const uint8_t* act;       // gate_up: x codes [T, K]; down: h codes [rows, K]
  const int* sorted_pairs;
  int topk;
  const int* tiles;
  const int* offsets;
  int* status;
  int scale_word;           // status word holding the activation scale
  float* h;                 // gate_up output fp32 [rows, I]
  float* y;                 // down output fp32 [rows, H]
};

// Accurate silu for the FP8 path: h is quantised afterwards, so the fast
// exp/divide of the bf16 path would move codes.
__device__ __forceinline__ float silu_accurate(float z) { return z / (1.0f + expf(-z)); }

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact: every E4M3 value is a bf16).
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  v8bf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// GATEUP: gate_up + SwiGLU epilogue, else down.  EXACT: bf16 MFMA on exactly
// expanded operands, else the block-scaled FP4 x FP8 MFMA.
template <bool GATEUP, bool EXACT>
__global__ __launch_bounds__(256, 2) void gemm_fp8_kernel(Fp8Args a) {
  const int4 tile = *reinterpret_cast<const int4*>(a.tiles + kTileInts * blockIdx.y);
  if (tile.x < 0) return;
  const int e = tile.x;
  const int row_begin = tile.y;
  const int row_end = tile.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  // gate_up: 64 gate rows + the 64 matching up rows; down: 128 rows
  const int n0 = blockIdx.x * (GATEUP ? kBN / 2 : kBN);

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- per-thread global source rows (fixed for the whole K loop)
  // activations: 4 chunks of 16 B per thread: row = (tid >> 3) + 32*i, part = tid & 7
  const uint8_t* asrc[4];
  bool aok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row_begin + (tid >> 3) + 32 * i;
    aok[i] = row < row_end;
    size_t src_row = 0;
    if (aok[i]) src_row = GATEUP ? (size_t)(a.sorted_pairs[row] / a.topk) : (size_t)row;
    asrc[i] = a.act + src_row * a.K + (tid & 7) * 16;
  }
  // weights: 2 chunks of 16 B per thread: lds row = (tid >> 2) + 64*i, block = tid & 3
  const uint8_t* wsrc[2];
  bool wok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lr = (tid >> 2) + 64 * i;
    int wr;
    if (GATEUP) {
      const int ii = n0 + (lr & 63);
      wok[i] = ii < a.nout;
      wr = (lr < 64 ? 0 : a.nout) + ii;
    } else {
      wr = n0 + lr;
      wok[i] = wr < a.nout;
    }
    const size_t grow = (size_t)e * a.rows_per_expert + (wok[i] ? wr : 0);
    wsrc[i] = a.wb + (grow * a.nb + (tid & 3)) * kBlockBytes;
  }
  // scales: threads 0..127 fetch the 4 scale bytes of lds row tid
  const uint8_t* ssrc = nullptr;
  bool sok = false;
  if (tid < kBN) {
    int wr;
    if (GATEUP) {
      const int ii = n0 + (tid & 63);
      sok = ii < a.nout;
      wr = (tid < 64 ? 0 : a.nout) + ii;
    } else {
      wr = n0 + tid;
      sok = wr < a.nout;
    }
    ssrc = a.ws + ((size_t)e * a.rows_per_expert + (sok ? wr : 0)) * a.nb;
  }

  const int nsteps = (a.nb + 3) >> 2;
  uint4 ra[4], rw[2];
  uint32_t rs = 0;
  auto gload = [&](int step) {
    const int k0 = step * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + (tid & 7) * 16;
      ra[i] = (aok[i] && kk < a.K) ? *reinterpret_cast<const uint4*>(asrc[i] + k0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = step * 4 + (tid & 3);
      rw[i] = (wok[i] && blk < a.nb)
                  ? *reinterpret_cast<const uint4*>(wsrc[i] + (size_t)step * 4 * kBlockBytes)
                  : make_uint4(0, 0, 0, 0);
    }
    if (tid < kBN) {
      uint32_t v = 0x7f7f7f7fu;
      if (sok) {
        v = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int blk = step * 4 + q;
          const uint32_t sb = blk < a.nb ? ssrc[blk] : 127u;
          v |= sb << (8 * q);
        }
      }
      rs = v;
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(base + ((tid >> 3) + 32 * i) * kActStride + (tid & 7) * 16) = ra[i];
    uint8_t* wbase = base + kActBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(wbase + ((tid >> 2) + 64 * i) * kWStride + (tid & 3) * 16) = rw[i];
    if (tid < kBN) reinterpret_cast<uint32_t*>(base + kActBytes + kWBytes)[tid] = rs;
  };

  // lds weight rows of this wave's four 16-row groups
  int wrow[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
    wrow[rg] = GATEUP ? ((rg >> 1) * 64 + 32 * wn + 16 * (rg & 1)) : (64 * wn + 16 * rg);

  v4f acc[4][4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = {0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
    const uint8_t* base = smem + buf * kStageBytes;
    const uint8_t* wbase = base + kActBytes;
    const uint32_t* sbase = reinterpret_cast<const uint32_t*>(base + kActBytes + kWBytes);
    if (EXACT) {
      // activation fragments: lane group g takes K [32g, 32g+32) of the step;
      // MFMA q of the group uses elements 8q..8q+7 (same order for weights)
      v8bf Bx[4][4];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        const uint8_t* p = base + (64 * wm + 16 * tg + r) * kActStride + 32 * g;
        const uint4 c0 = *reinterpret_cast<const uint4*>(p);
        const uint4 c1 = *reinterpret_cast<const uint4*>(p + 16);
        Bx[tg][0] = fp8x8_to_bf16(c0.x, c0.y);
        Bx[tg][1] = fp8x8_to_bf16(c0.z, c0.w);
        Bx[tg][2] = fp8x8_to_bf16(c1.x, c1.y);
        Bx[tg][3] = fp8x8_to_bf16(c1.z, c1.w);
      }
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int lr = wrow[rg] + r;
        const uint4 w = *reinterpret_cast<const uint4*>(wbase + lr * kWStride + 16 * g);
        const float f = e8m0_to_f32((sbase[lr] >> (8 * g)) & 0xffu);
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v8bf A = fp4x8_to_bf16(wv[q], f);
#pragma unroll
          for (int tg = 0; tg < 4; ++tg)
            acc[rg][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bx[tg][q], acc[rg][tg], 0, 0, 0);
        }
      }
    } else {
      v8i B[4];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        const uint8_t* p = base + (64 * wm + 16 * tg + r) * kActStride;
        const uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * g);
        const uint4 hi = *reinterpret_cast<const uint4*>(p + 64 + 16 * g);
        B[tg] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int lr = wrow[rg] + r;
        const uint4 w = *reinterpret_cast<const uint4*>(wbase + lr * kWStride + 16 * g);
        const v8i A = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        const int sa = (int)((sbase[lr] >> (8 * g)) & 0xffu);
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
          acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[tg], acc[rg][tg], 4, 0, 0,
                                                                         sa, 0, 127);
      }
    }
    if (step + 1 < nsteps) {
      sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows 4g + jj of each 16-row group, token column r
  const float sx = __uint_as_float((uint32_t)a.status[a.scale_word]);
  const uint16_t* bias_e = a.bias ? a.bias + (size_t)e * a.rows_per_expert : nullptr;
  if (GATEUP) {
    float amax = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int i0 = n0 + 32 * wn + 16 * half;     // gate/up rows of groups half, half+2
      if (i0 >= a.nout) continue;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        const int row = row_begin + 64 * wm + 16 * tg + r;
        if (row >= row_end) continue;
        float hv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = i0 + 4 * g + jj;
          float gate = acc[half][tg][jj] * sx;
          float up = acc[half + 2][tg][jj] * sx;
          if (bias_e) {
            gate += bf16_bits_to_f32(bias_e[i]);
            up += bf16_bits_to_f32(bias_e[a.nout + i]);
          }
          hv[jj] = silu_accurate(gate) * up;
          amax = fmaxf(amax, fabsf(hv[jj]));
        }
        *reinterpret_cast<float4*>(a.h + (size_t)row * a.nout + i0 + 4 * g) =
            make_float4(hv[0], hv[1], hv[2], hv[3]);
      }
    }
    amax = wave_max(amax);
    if (lane == 0) atomicMax(reinterpret_cast<uint32_t*>(&a.status[kStAmaxH]), __float_as_uint(amax));
  } else {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int nb0 = n0 + 64 * wn + 16 * rg;
      if (nb0 >= a.nout) continue;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        const int row = row_begin + 64 * wm + 16 * tg + r;
        if (row >= row_end) continue;
        float v[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          v[jj] = acc[rg][tg][jj] * sx;
          if (bias_e) v[jj] += bf16_bits_to_f32(bias_e[nb0 + 4 * g + jj]);
        }
        *reinterpret_cast<float4*>(a.y + (size_t)row * a.nout + nb0 + 4 * g) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

static Fp8Args common_args(const MoeShape& sh, const WsPtrs& ws) {
  Fp8Args a{};
  a.sorted_pairs = ws.sorted_pairs;
  a.topk = sh.k;
  a.tiles = ws.tiles;
  a.offsets = ws.offsets;
  a.status = ws.status;
  return a;
}

hipError_t launch_moe_gateup_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                 int64_t ntile_bound, hipStream_t s) {
  Fp8Args a = common_args(sh, ws);
  a.wb = w.w13_blocks;
  a.ws = w.w13_scales;
  a.bias = w.w13_bias;
  a.rows_per_expert = 2 * (int64_t)sh.I;
  a.nout = sh.I;
  a.nb = sh.H / kBlockElems;
  a.K = sh.H;
  a.act = ws.x_codes;
  a.scale_word = kStScaleX;
  a.h = static_cast<float*>(ws.h);
  const dim3 grid((unsigned)((sh.I + 63) / 64), (unsigned)ntile_bound);
  gemm_fp8_kernel<true, true><<<grid, 256, 2 * kStageBytes, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_moe_down_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                               int64_t ntile_bound, hipStream_t s) {
  Fp8Args a = common_args(sh, ws);
  a.wb = w.w2_blocks;
  a.ws = w.w2_scales;
  a.bias = w.w2_bias;
  a.rows_per_expert = sh.H;
  a.nout = sh.H;
  a.nb = sh.I / kBlockElems;
  a.K = sh.I;
  a.act = ws.h_codes;
  a.scale_word = kStScaleH;
  a.y = ws.y;
  const dim3 grid((unsigned)((sh.H + kBN - 1) / kBN), (unsigned)ntile_bound);
  gemm_fp8_kernel<false, false><<<grid, 256, 2 * kStageBytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace mx
