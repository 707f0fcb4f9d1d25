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
// The MFMA used for the gate_up contraction differs.  The F8F6F4
// instructions sum each 128-long dot product with reduced internal precision
// (measured: errors up to ~2.4e-5 of the sum of |products|), which perturbs h
// enough to move a small fraction of its FP8 codes.  So gate_up, whose output
// is quantised again, expands the FP8 codes and the FP4 weights (with their
// E8M0 block scale) exactly to bf16 and runs v_mfma_f32_16x16x32_bf16
// (fp32-accurate); down, whose output is not quantised, keeps the
// block-scaled FP8 x FP4 instruction.
//
// Schedule (gfx950):
//   * Persistent grid, one block per compute unit.  A unit of work is one row
//     tile (up to BM expert-sorted rows of one expert, from the tile list the
//     permutation builds) times one n-tile of 256 weight rows (gate_up: 128
//     gate rows and the matching 128 up rows).  Block b takes units b, b + G,
//     b + 2G, ...; a unit is nsteps K steps of 128.
//   * Four loader waves copy every K step's activations (BM x 128 B of E4M3
//     codes, rows in expert-sorted order), weights (256 x 64 B of E2M1) and
//     E8M0 scales from global memory into one slot of an LDS ring by DMA
//     (global -> LDS), and run STAGES-1 steps ahead of the compute waves.
//     The DMA issue rate is a per-wave limit (measured: about 12.5 GB/s per
//     wave whether the data comes from L2 or HBM, scaling with the number of
//     issuing waves), so the copies are spread over four waves.
//     Each loader issues the same number of DMA instructions every step, so
//     it waits for exactly the slot the next step needs with an explicit
//     vector-memory count.  The loaders read the tile list through the scalar
//     cache, so no other vector-memory operation enters those counts.
//   * The compute waves issue no vector-memory loads in the K loop, so the
//     counter wait the compiler places before LDS reads that may alias a DMA
//     never stalls them.
//   * One barrier per K step: after it the slot of step t has landed and the
//     slot of step t-1 is free; the loaders then refill it with step
//     t+STAGES-1.
//   * BM/16 compute waves, each 64 sorted rows x 64 weight rows (4 x 4 MFMA
//     tiles of 16 x 16).
//   * LDS layouts are XOR-swizzled at 16-byte granularity, chosen through
//     each lane's DMA source address, so that the MFMA-layout reads of a
//     group of 8 lanes hit distinct banks.
//   * K tails: chunks past K are loaded from a valid address and the weight
//     operand of MX blocks past K is forced to zero in the compute waves.
#include "common.hpp"
#include "launch.hpp"

namespace mx {

constexpr int kBN = 256;               // weight rows per unit
constexpr int kBK = 128;               // K per step (four MX blocks)
constexpr int kWTile = kBN * kBK / 2;  // E2M1 bytes per step
constexpr int kScTile = kBN * 8;       // two aligned scale dwords per weight row

template <int BM>
struct Ring {
  static constexpr int kCompute = BM / 16;              // compute waves
  static constexpr int kLoaders = 4;                    // DMA issue rate is per wave
  static constexpr int kThreads = 64 * (kCompute + kLoaders);
  static constexpr int kStages = BM == 128 ? 4 : 5;
  static constexpr int kAct = BM * kBK;                 // activation bytes per slot
  static constexpr int kW = kAct;                       // offsets inside a slot
  static constexpr int kSc = kAct + kWTile;
  static constexpr int kSlot = kSc + kScTile;
  static constexpr int kActDma = BM / 8 / kLoaders;     // 1 KB activation DMAs per loader per step
  static constexpr int kWDma = 16 / kLoaders;           // 1 KB weight DMAs per loader per step
  static constexpr int kScDma = 8 / kLoaders;           // 256 B scale DMAs per loader per step
  static constexpr int kDma = kActDma + kWDma + kScDma; // DMA instructions per loader per step
  static_assert(kActDma * kLoaders * 8 == BM, "activation rows split over the loaders");
  static_assert(3 * kDma <= 63, "vector-memory count range");
  static_assert(kStages - 2 <= 3, "waits cover up to three steps ahead");
  static_assert(kStages * kSlot <= 160 * 1024, "LDS");
};

struct PrefillArgs {
  const uint8_t* wb;       // [E, R, nb, 16]
  const uint8_t* ws;       // [E, R, nb]
  const uint16_t* bias;    // [E, R] or null
  int64_t sc_total;        // E * R * nb (scale bytes; a multiple of 4)
  int R;                   // rows per expert: 2I (gate_up) or H (down)
  int nout;                // I (gate_up) or H (down)
  int nb;                  // K / 32
  int K;
  int NT;                  // n-tiles
  int nsteps;              // ceil(nb / 4)
  const uint8_t* act;      // [sorted rows, K] E4M3 codes
  int scale_word;          // status word holding the activation scale
  float* out;              // h [rows, I] (gate_up) or y [rows, H] (down), fp32
};

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

// Accurate silu for the FP8 path: h is quantised afterwards, so the fast
// exp/divide of the bf16 path would move codes.
__device__ __forceinline__ float silu_accurate(float z) { return z / (1.0f + expf(-z)); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding (the other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Tile-list entry (expert, first row, end row) through the scalar cache:
// `p` is wave-uniform, and the load is counted by lgkmcnt, not vmcnt.
__device__ __forceinline__ int3 tile_entry(const int* p) {
  typedef int v4i_t __attribute__((ext_vector_type(4)));
  v4i_t v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
  return make_int3(v.x, v.y, v.z);
}

// Weight row (within the expert) held in LDS row lr of n-tile nt, clamped
// into the matrix (clamped rows are loaded but never stored).
template <bool GATEUP>
__device__ __forceinline__ int weight_row(int lr, int nt, int nout) {
  if (GATEUP) {
    const int i = min(nt * (kBN / 2) + (lr & (kBN / 2 - 1)), nout - 1);
    return (lr < kBN / 2 ? 0 : nout) + i;
  }
  return min(nt * kBN + lr, nout - 1);
}

template <bool GATEUP, int BM>
__device__ __forceinline__ void prefill_loader(const PrefillArgs& a, const int* __restrict__ tiles,
                                               uint8_t* smem, int l, int lane, int total, int u0,
                                               int G) {
  using C = Ring<BM>;
  constexpr int NL = C::kLoaders;
  // Per-lane parts fixed for the whole kernel.  Activation DMA i of loader l
  // fills slot rows 8j..8j+7 (j = NL*i + l): lane -> row 8j + lane/8, 16-byte
  // slot lane%8, which holds logical chunk (lane%8) ^ (row%8).
  const int a_row = lane >> 3;
  const int a_chunk = (lane & 7) ^ a_row;
  // Weight DMA i fills rows 16j..16j+15: lane -> row 16j + lane/4, slot
  // lane%4, which holds MX block (lane%4) ^ ((row/2)%4).
  const int w_row = lane >> 2;
  const int w_blk = (lane & 3) ^ ((lane >> 3) & 3);
  // Scale DMA i fills rows 32j..32j+31: lane -> row 32j + lane/2, aligned
  // dword lane%2 of the 8 bytes that hold the row's four scales of the step.
  const int s_row = lane >> 1;
  const int s_dw = lane & 1;
  const int my_units = total / a.nsteps;

  const uint8_t* aptr[C::kActDma];
  const uint8_t* wptr[C::kWDma];
  int64_t sofs[C::kScDma];

  auto setup = [&](int u) __attribute__((always_inline)) {
    const int tile = u / a.NT;
    const int nt = u - tile * a.NT;
    const int3 te = tile_entry(tiles + kTileInts * tile);
#pragma unroll
    for (int i = 0; i < C::kActDma; ++i) {
      int row = te.y + 8 * (NL * i + l) + a_row;
      row = row < te.z ? row : te.y;
      aptr[i] = a.act + (int64_t)row * a.K;
    }
    const int64_t ebase = (int64_t)te.x * a.R;
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i) {
      const int wr = weight_row<GATEUP>(16 * (NL * i + l) + w_row, nt, a.nout);
      wptr[i] = a.wb + (ebase + wr) * a.nb * kBlockBytes;
    }
#pragma unroll
    for (int i = 0; i < C::kScDma; ++i) {
      const int wr = weight_row<GATEUP>(32 * (NL * i + l) + s_row, nt, a.nout);
      sofs[i] = (ebase + wr) * a.nb;
    }
  };

  int k = 0, step = 0, slot = 0;   // local unit index, step and ring slot of the next issue
  auto issue = [&]() __attribute__((always_inline)) {
    uint8_t* dst = smem + slot * C::kSlot;
    const bool tail = step == a.nsteps - 1;
    const int kb = step * kBK;
#pragma unroll
    for (int i = 0; i < C::kActDma; ++i) {
      const int off = kb + 16 * a_chunk;           // past K: the row's first 16 bytes
      __builtin_amdgcn_global_load_lds(aptr[i] + (!tail || off < a.K ? off : 0), dst + 1024 * (NL * i + l),
                                       16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i) {
      const int blk = 4 * step + w_blk;            // past K: the row's first block
      __builtin_amdgcn_global_load_lds(wptr[i] + (!tail || blk < a.nb ? blk * kBlockBytes : 0),
                                       dst + C::kW + 1024 * (NL * i + l), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::kScDma; ++i) {
      int64_t q = ((sofs[i] + 4 * step) & ~(int64_t)3) + 4 * s_dw;
      q = q < a.sc_total - 4 ? q : a.sc_total - 4;
      __builtin_amdgcn_global_load_lds(a.ws + q, dst + C::kSc + 256 * (NL * i + l), 4, 0, 0);
    }
    slot = slot + 1 == C::kStages ? 0 : slot + 1;
    if (++step == a.nsteps) {
      step = 0;
      if (++k < my_units) setup(u0 + k * G);
    }
  };

  setup(u0);
  const int pro = total < C::kStages - 1 ? total : C::kStages - 1;
  for (int p = 0; p < pro; ++p) issue();
  for (int t = 0; t < total; ++t) {
    // steps issued beyond t: min(STAGES - 2, total - 1 - t); wait for the rest
    int ahead = total - 1 - t;
    ahead = ahead < C::kStages - 2 ? ahead : C::kStages - 2;
    if (ahead >= 3) wait_vm<3 * C::kDma>();
    else if (ahead == 2) wait_vm<2 * C::kDma>();
    else if (ahead == 1) wait_vm<C::kDma>();
    else wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");
    if (t + C::kStages - 1 < total) issue();
  }
}

template <bool GATEUP, int BM>
__global__ __launch_bounds__(Ring<BM>::kThreads) void prefill_gemm_kernel(PrefillArgs a,
                                                                          const int* __restrict__ tiles,
                                                                          int* status) {
  using C = Ring<BM>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kStages * C::kSlot];
  const int num_units = status[kStNumTiles] * a.NT;
  const float sx = __uint_as_float((uint32_t)status[a.scale_word]);
  const int G = gridDim.x;
  const int u0 = blockIdx.x;
  if (u0 >= num_units) return;
  const int total = ((num_units - 1 - u0) / G + 1) * a.nsteps;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= C::kCompute) {
    prefill_loader<GATEUP, BM>(a, tiles, smem, wave - C::kCompute, lane, total, u0, G);
    return;
  }

  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  // LDS weight rows of this lane in the wave's four 16-row groups (gate_up:
  // groups 0, 1 gate rows, 2, 3 the matching up rows)
  int lrow[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
    lrow[rg] = (GATEUP ? (rg >> 1) * (kBN / 2) + 32 * wn + 16 * (rg & 1) : 64 * wn + 16 * rg) + r;
  const int wslot = g ^ ((r >> 1) & 3);    // slot of MX block g in these rows
  // activation chunks: the bf16 path takes K [32g, 32g+32) = chunks 2g, 2g+1,
  // the block-scaled path chunks g and 4+g; the row's swizzle is row%8 = r%8
  const int c0 = (GATEUP ? 2 * g : g) ^ (r & 7);
  const int c1 = (GATEUP ? 2 * g + 1 : 4 + g) ^ (r & 7);

  int unit = u0, step = 0, slot = 0;
  int e = 0, rb = 0, re = 0, nt = 0;
  int sphase[4];
  // bias of the lane's four output rows of each epilogue group, as bf16
  // pairs; loaded when a unit starts so that its epilogue does not wait on
  // memory (gate_up: gate and up rows of groups 0 and 1; down: groups 0..3)
  uint2 bq[4];
  auto setup = [&](int u) __attribute__((always_inline)) {
    const int tile = u / a.NT;
    nt = u - tile * a.NT;
    const int4 te = *reinterpret_cast<const int4*>(tiles + kTileInts * tile);
    e = te.x; rb = te.y; re = te.z;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int wr = weight_row<GATEUP>(lrow[rg], nt, a.nout);
      sphase[rg] = (int)((((int64_t)e * a.R + wr) * a.nb) & 3);
    }
    const uint16_t* bias_e = a.bias + (size_t)e * a.R;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n0 = GATEUP ? nt * (kBN / 2) + 32 * wn + 16 * (j >> 1) : nt * kBN + 64 * wn + 16 * j;
      const int off = (GATEUP && (j & 1) ? a.nout : 0) + n0 + 4 * g;
      bq[j] = a.bias && n0 < a.nout ? *reinterpret_cast<const uint2*>(bias_e + off) : make_uint2(0, 0);
    }
  };
  setup(unit);

  v4f acc[4][4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = {0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < total; ++t) {
    // slot of step t landed; everyone is done with step t-1's slot
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const uint8_t* base = smem + slot * C::kSlot;
    const bool valid = 4 * step + g < a.nb;    // this lane's MX block lies inside K
    uint4 wq[4];
    uint32_t sb[4];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      wq[rg] = *reinterpret_cast<const uint4*>(base + C::kW + lrow[rg] * 64 + 16 * wslot);
      sb[rg] = base[C::kSc + lrow[rg] * 8 + sphase[rg] + g];
    }
    if (GATEUP) {
      uint4 xa[4], xb[4];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        const uint8_t* p = base + (64 * wm + 16 * tg + r) * kBK;
        xa[tg] = *reinterpret_cast<const uint4*>(p + 16 * c0);
        xb[tg] = *reinterpret_cast<const uint4*>(p + 16 * c1);
      }
      // lane group g holds K [32g, 32g+32) of the step (its own MX block);
      // MFMA q takes elements 8q..8q+7 of it, in the same order for both
      // operands
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v8bf B[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const uint4 c = q < 2 ? xa[tg] : xb[tg];
          B[tg] = (q & 1) ? fp8x8_to_bf16(c.z, c.w) : fp8x8_to_bf16(c.x, c.y);
        }
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float f = valid ? e8m0_to_f32(sb[rg]) : 0.0f;
          const uint32_t wv = q == 0 ? wq[rg].x : q == 1 ? wq[rg].y : q == 2 ? wq[rg].z : wq[rg].w;
          const v8bf A = fp4x8_to_bf16(wv, f);
#pragma unroll
          for (int tg = 0; tg < 4; ++tg)
            acc[rg][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[tg], acc[rg][tg], 0, 0, 0);
        }
      }
    } else {
      typedef int v4i_t __attribute__((ext_vector_type(4)));
      v8i B[4];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        const uint8_t* p = base + (64 * wm + 16 * tg + r) * kBK;
        const v4i_t lo = *reinterpret_cast<const v4i_t*>(p + 16 * c0);
        const v4i_t hi = *reinterpret_cast<const v4i_t*>(p + 16 * c1);
        B[tg] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const v8i A = valid ? v8i{(int)wq[rg].x, (int)wq[rg].y, (int)wq[rg].z, (int)wq[rg].w, 0, 0, 0, 0}
                            : v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
          acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[tg], acc[rg][tg], 4, 0, 0,
                                                                         (int)sb[rg], 0, 127);
      }
    }
    slot = slot + 1 == C::kStages ? 0 : slot + 1;
    if (++step < a.nsteps) continue;

    // ---- epilogue of the unit: the lane holds rows 4g + jj of each 16-row
    // weight group and sorted row r of each 16-row token group
    if (GATEUP) {
      float amax = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int i0 = nt * (kBN / 2) + 32 * wn + 16 * half;
        if (i0 >= a.nout) continue;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const int row = rb + 64 * wm + 16 * tg + r;
          if (row >= re) continue;
          float hv[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint2 bg = bq[2 * half], bu = bq[2 * half + 1];
            const uint32_t wg = jj < 2 ? bg.x : bg.y, wu = jj < 2 ? bu.x : bu.y;
            const float gate = acc[half][tg][jj] * sx + bf16_bits_to_f32(jj & 1 ? wg >> 16 : wg & 0xffffu);
            const float up = acc[half + 2][tg][jj] * sx + bf16_bits_to_f32(jj & 1 ? wu >> 16 : wu & 0xffffu);
            hv[jj] = silu_accurate(gate) * up;
            amax = fmaxf(amax, fabsf(hv[jj]));
          }
          *reinterpret_cast<float4*>(a.out + (size_t)row * a.nout + i0 + 4 * g) =
              make_float4(hv[0], hv[1], hv[2], hv[3]);
        }
      }
      amax = wave_max(amax);
      if (lane == 0) atomicMax(reinterpret_cast<uint32_t*>(&status[kStAmaxH]), __float_as_uint(amax));
    } else {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n0 = nt * kBN + 64 * wn + 16 * rg;
        if (n0 >= a.nout) continue;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const int row = rb + 64 * wm + 16 * tg + r;
          if (row >= re) continue;
          float v[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t wb = jj < 2 ? bq[rg].x : bq[rg].y;
            v[jj] = acc[rg][tg][jj] * sx + bf16_bits_to_f32(jj & 1 ? wb >> 16 : wb & 0xffffu);
          }
          *reinterpret_cast<float4*>(a.out + (size_t)row * a.nout + n0 + 4 * g) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = {0.f, 0.f, 0.f, 0.f};
    step = 0;
    unit += G;
    if (t + 1 < total) setup(unit);
  }
}

template <bool GATEUP>
static hipError_t launch_prefill(const PrefillArgs& a, const WsPtrs& ws, hipStream_t s) {
  // one block per compute unit: the LDS ring takes most of a unit's LDS
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  prefill_gemm_kernel<GATEUP, kPrefillBM><<<cus, Ring<kPrefillBM>::kThreads, 0, s>>>(a, ws.tiles, ws.status);
  return hipGetLastError();
}

hipError_t launch_moe_gateup_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                 int64_t /*ntile_bound*/, hipStream_t s) {
  PrefillArgs a{};
  a.wb = w.w13_blocks;
  a.ws = w.w13_scales;
  a.bias = w.w13_bias;
  a.R = 2 * sh.I;
  a.nout = sh.I;
  a.nb = sh.H / kBlockElems;
  a.K = sh.H;
  a.sc_total = (int64_t)sh.E * a.R * a.nb;
  a.NT = (sh.I + kBN / 2 - 1) / (kBN / 2);
  a.nsteps = (a.nb + 3) / 4;
  a.act = ws.x_codes;
  a.scale_word = kStScaleX;
  a.out = static_cast<float*>(ws.h);
  return launch_prefill<true>(a, ws, s);
}

hipError_t launch_moe_down_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                               int64_t /*ntile_bound*/, hipStream_t s) {
  PrefillArgs a{};
  a.wb = w.w2_blocks;
  a.ws = w.w2_scales;
  a.bias = w.w2_bias;
  a.R = sh.H;
  a.nout = sh.H;
  a.nb = sh.I / kBlockElems;
  a.K = sh.I;
  a.sc_total = (int64_t)sh.E * a.R * a.nb;
  a.NT = (sh.H + kBN - 1) / kBN;
  a.nsteps = (a.nb + 3) / 4;
  a.act = ws.h_codes;
  a.scale_word = kStScaleH;
  a.out = ws.y;
  return launch_prefill<false>(a, ws, s);
}

}  // namespace mx
