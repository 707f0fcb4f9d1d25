// bf16-activation MXFP4 contractions for small token counts: the MoE decode
// path (gate_up + SwiGLU, down) and the dense projections (qkv_proj, o_proj,
// lm_head at a few tokens).
//
// These are HBM-bound weight streams (gpt-oss page, "MXFP4 Tensor
// Structure" for the layout; forum page: decode runs close to the bandwidth
// ceiling).  Design for gfx950:
//   * a wave owns 16 weight rows (gate_up: 16 gate + the matching 16 up rows)
//     and streams them with 16-byte loads, one MX block per lane per K-group
//     of four blocks;
//   * loads run DEPTH groups ahead through a statically indexed register
//     ring, so a wave keeps several KB in flight and only waits for the group
//     it is about to multiply;
//   * when a launch has few row tiles (qkv/o projections, a handful of
//     routed tokens) the K range of a row tile is split across KSPLIT waves
//     of the block and the partial sums are added in LDS in a fixed order;
//   * the E2M1 nibbles are expanded in registers with the scaled FP4->bf16
//     convert (the E8M0 block scale folded in; exact for scale bytes 11..252)
//     and fed to v_mfma_f32_16x16x32_bf16 with the routed tokens as the 16
//     columns; a K-group is four MFMAs, each taking 8 elements of the lane's
//     own block, so the K order inside an MFMA is permuted identically for
//     weights and activations;
//   * fp32 accumulation; SwiGLU, bias and the output rounding are fused into
//     the epilogue.  The SwiGLU output is kept as two bf16 halves hi + lo so
//     that the down projection runs on bf16 MFMAs without a second rounding
//     of h (hi = bf16(h), lo = bf16(h - hi)).
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "route_small.hpp"

namespace mx {

enum GemvMode { kGateUp = 0, kDown = 1, kDense = 2 };
constexpr int kDepth = 3;   // K-groups in flight per wave

struct GemvArgs {
  const uint8_t* wb;        // blocks [E, R, nb, 16]
  const uint8_t* ws;        // scales [E, R, nb]
  const uint16_t* bias;     // [E, R] or null
  int64_t rows_per_expert;  // R
  int nout;                 // output rows per expert: I (gate_up), H (down), N (dense)
  int nb;                   // K / 32
  const uint16_t* act;      // gate_up: x [T, K]; dense: x [M, K]; down: h hi [rows, K]
  const uint16_t* act_lo;   // down: h lo [rows, K]
  uint32_t act_bytes;       // bytes of act (and of act_lo); < 2^31
  const int* sorted_pairs;
  int topk;
  const int* tiles;
  const int* offsets;
  const int* status;
  int M;                    // dense rows
  uint16_t* out_hi;         // gate_up: h hi / dense: out bf16
  uint16_t* out_lo;         // gate_up: h lo
  float* y;                 // down
  float gscale;             // NVFP4: the weight tensor's global scale (MXFP4: 1)
  // gate_up that routes the batch itself (decode batches): router logits
  // [T, E] and the outputs block 0 writes (top-k ids and weights, and the
  // permutation for the down and combine kernels)
  const float* logits;
  int T, E, bound;
  int* ids_out;
  float* w_out;
  int* g_status;
  int* g_offsets;
  int* g_sorted;
  int* g_inv;
  int* g_tiles;
};

// LDS of a routing gate_up block beyond the GEMV's: ids, expert offsets,
// sorted pairs (128 each), status words, then the row-tile list.
constexpr int kRouteLdsInts = 3 * kSmallMaxPairs + kStWords;
static_assert(kSmallMaxExperts <= kSmallMaxPairs, "expert offsets share the pair-sized slot");
inline size_t route_lds_bytes(int bound) { return (size_t)(kRouteLdsInts + kTileInts * bound) * 4; }

// One K-group's operands for one lane.
template <int MODE>
struct Group {
  uint4 w0, w1;        // 16 B of the lane's block: main/gate row, up row
  uint32_t s0, s1;     // their E8M0 scales
  uint4 b[4];          // 32 activations (bf16) of the lane's column
  uint4 bl[4];         // down: the lo halves
};

template <int MODE, int KSPLIT>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(GemvArgs a) {
  constexpr int kTilesPerBlock = 4 / KSPLIT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;   // weight row inside the 16-row group / token column
  const int g = lane >> 4;   // which of the K-group's four blocks this lane loads
  const int kpart = wave % KSPLIT;
  const int rt = wave / KSPLIT;

  int e, row_begin, row_end;
  if (MODE == kDense) {
    e = 0;
    row_begin = blockIdx.y * 16;
    row_end = min(row_begin + 16, a.M);
  } else {
    const int4 tile = *reinterpret_cast<const int4*>(a.tiles + kTileInts * blockIdx.y);
    if (tile.x < 0) return;
    e = tile.x;
    row_begin = tile.y;
    row_end = tile.z;
  }
  const int n0 = (blockIdx.x * kTilesPerBlock + rt) * 16;
  const bool tile_ok = n0 < a.nout;   // uniform per wave; no early return (LDS reduction below)

  // activation row feeding MFMA column r
  const int row = row_begin + r;
  const bool col_ok = row < row_end;
  const int arow = col_ok ? row : row_begin;   // inactive columns read a valid row
  const uint16_t* act0 = a.act;
  const uint16_t* act1 = a.act_lo;
  if (MODE == kGateUp) {
    const int t = a.sorted_pairs[arow] / a.topk;
    act0 += (size_t)t * a.nb * kBlockElems;
  } else {
    act0 += (size_t)arow * a.nb * kBlockElems;
    if (MODE == kDown) act1 += (size_t)arow * a.nb * kBlockElems;
  }

  const size_t wrow0 = (size_t)e * a.rows_per_expert + (tile_ok ? n0 + r : 0);
  const size_t wrow1 = wrow0 + a.nout;  // matching up row (gate_up only)
  const uint8_t* wb0 = a.wb + wrow0 * a.nb * kBlockBytes;
  const uint8_t* ws0 = a.ws + wrow0 * a.nb;
  const uint8_t* wb1 = a.wb + wrow1 * a.nb * kBlockBytes;
  const uint8_t* ws1 = a.ws + wrow1 * a.nb;

  // this wave's share of the K-groups
  const int ngroups = (a.nb + 3) >> 2;
  const int g_begin = tile_ok ? (kpart * ngroups) / KSPLIT : 0;
  const int g_end = tile_ok ? ((kpart + 1) * ngroups) / KSPLIT : 0;

  // Loads are issued unconditionally so the outstanding-load count is the
  // same on every path: a block past the end of K reads the last block with
  // its scale forced to 0 (the expanded weights are then 0), and a column
  // past the tile's rows reads a valid row whose results are discarded.
  auto load = [&](int grp, Group<MODE>& G) {
    const int j = grp * 4 + g;
    const int jc = j < a.nb ? j : a.nb - 1;
    G.w0 = ld_stream16(wb0 + (size_t)jc * kBlockBytes);
    G.s0 = ld_stream1(ws0 + jc);
    if (MODE == kGateUp) {
      G.w1 = ld_stream16(wb1 + (size_t)jc * kBlockBytes);
      G.s1 = ld_stream1(ws1 + jc);
    }
    const uint4* p = reinterpret_cast<const uint4*>(act0 + (size_t)jc * kBlockElems);
#pragma unroll
    for (int q = 0; q < 4; ++q) G.b[q] = p[q];
    if (MODE == kDown) {
      const uint4* pl = reinterpret_cast<const uint4*>(act1 + (size_t)jc * kBlockElems);
#pragma unroll
      for (int q = 0; q < 4; ++q) G.bl[q] = pl[q];
    }
  };

  v4f acc0 = {0.f, 0.f, 0.f, 0.f};
  v4f acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int grp, const Group<MODE>& G) {
    const bool jok = grp * 4 + g < a.nb;     // tail blocks: scale 0 zeroes the weights
    const float f0 = jok ? e8m0_to_f32(G.s0) : 0.0f;
    const uint32_t wv0[4] = {G.w0.x, G.w0.y, G.w0.z, G.w0.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v8bf A0 = fp4x8_to_bf16(wv0[q], f0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, as_v8bf(G.b[q]), acc0, 0, 0, 0);
      if (MODE == kDown)
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, as_v8bf(G.bl[q]), acc0, 0, 0, 0);
    }
    if (MODE == kGateUp) {
      const float f1 = jok ? e8m0_to_f32(G.s1) : 0.0f;
      const uint32_t wv1[4] = {G.w1.x, G.w1.y, G.w1.z, G.w1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v8bf A1 = fp4x8_to_bf16(wv1[q], f1);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, as_v8bf(G.b[q]), acc1, 0, 0, 0);
      }
    }
  };

  // prefetch ring: group grp lives in ring[(grp - g_begin) % kDepth].  The
  // steady-state loop refills after every multiply with no condition, so the
  // compiler can keep kDepth groups outstanding; the tail drains the ring.
  Group<MODE> ring[kDepth];
  if (g_end - g_begin >= kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) load(g_begin + u, ring[u]);
    int grp = g_begin;
    for (; grp + 2 * kDepth <= g_end; grp += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        compute(grp + u, ring[u]);
        load(grp + u + kDepth, ring[u]);
      }
    }
    // kDepth <= g_end - grp < 2 * kDepth groups remain, kDepth of them loaded
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      compute(grp + u, ring[u]);
      if (grp + u + kDepth < g_end) load(grp + u + kDepth, ring[u]);
    }
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
      if (grp + kDepth + u < g_end) compute(grp + kDepth + u, ring[u]);
  } else {
    for (int grp = g_begin; grp < g_end; ++grp) {
      load(grp, ring[0]);
      compute(grp, ring[0]);
    }
  }

  if (KSPLIT > 1) {
    // fixed-order reduction of the K parts of each row tile
    __shared__ v4f part[4][2][64];
    part[wave][0][lane] = acc0;
    part[wave][1][lane] = acc1;
    __syncthreads();
    if (kpart != 0) return;
    for (int kp = 1; kp < KSPLIT; ++kp) {
      acc0 += part[wave + kp][0][lane];
      acc1 += part[wave + kp][1][lane];
    }
  }
  if (!col_ok || !tile_ok) return;

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

// ---------------------------------------------------------------------------
// Persistent streaming variant (decode-sized MoE GEMMs, lm_head).
//   * A unit is one m-tile (at most 4 activation rows: routed pairs of one
//     expert, or dense rows) times 16 weight rows (down, dense) or 8 gate rows
//     plus the matching 8 up rows (gate_up).  The grid is the number of blocks
//     resident at once; each block walks a contiguous range of units, so
//     consecutive units share their m-tile and the activations stay in
//     registers.
//   * Loading: wave w of the block's two waves copies the unit's weight rows
//     8w..8w+7 (one contiguous run of whole 128-byte lines: no line is shared
//     with another wave or unit) and their E8M0 scales by DMA (global -> LDS,
//     1 KB / 256 B per instruction, nontemporal; measured 6.7 TB/s for this
//     pattern, against 3.7 TB/s for 16 rows x 64 B per register load) into the
//     block's LDS buffer.  As soon as both waves have copied the buffer into
//     registers, the DMA of the next unit is issued, so the buffer stays in
//     flight while the unit is multiplied -- the bytes in flight per CU, which
//     loaded HBM latency calls for, are the LDS the resident blocks hold (six
//     blocks of 27 KB per CU).
//   * Multiplying: the waves split K: wave h takes K-groups [HG*h, HG*h + HG)
//     of all 16 rows (HG a compile-time count; groups past K are zero).
//   * Activations use the compact layout: register set j holds in lane
//     t + 4q + 16g the 8 activations [128j + 32g + 8q, +8) of m-tile column t,
//     one 16-byte load per lane bringing 256 contiguous bytes of each column.
//     MFMA step q rotates the set by 4q lanes inside each 16-lane row (DPP),
//     which puts column t's values in lane t + 16g; lanes of columns 4..15 then
//     hold other columns' values and their MFMA outputs are never stored.
//     Columns past the m-tile's rows and blocks past K read through a
//     range-checked buffer descriptor with an out-of-range offset, which
//     returns zeros without touching memory.
//   * Wave 1 hands its partial sums to wave 0 through LDS; wave 0 adds them,
//     adds bias, applies SwiGLU (gate_up: one 16-row MFMA holds 8 gate rows and
//     their 8 up rows, the up result moves to the gate lane, lane ^ 32) and
//     stores.  Three barriers per unit: data landed, buffer read, partial sums
//     written.
constexpr int kUnitRows = 16;          // weight rows per unit
constexpr int kRunRows = 8;            // rows per wave's DMA run
constexpr int kCols = 4;               // activation rows per unit
constexpr int kMaxHG = 12;             // K-groups per wave: K <= 3072 on this path
constexpr int kRunDma = 12;            // 1 KB weight DMA instructions per run (8 x 1536 B max)
// 256 B scale DMA instructions per run: MXFP4 8 x 96 B max, NVFP4 (two
// scales per 32 elements) 8 x 192 B max
template <bool NV> struct RunLayout {
  static constexpr int kScDma = NV ? 6 : 3;
  // (a run's region also covers reads of blocks up to 95 of its last row:
  // 7 * 1536 + 96 * 16 <= 12 KB; scales 7 * 96 + 96 <= 768, NVFP4
  // 7 * 192 + 192 <= 1536)
  static constexpr int kRunBytes = kRunDma * 1024 + kScDma * 256;   // LDS per run
  static constexpr int kBufBytes = 2 * kRunBytes;                  // LDS per unit buffer
  // buffer, partial sums; NVFP4: the two waves' per-column activation maxima
  static constexpr int kLds = kBufBytes + 64 * 16 + (NV ? 2 * kCols * 4 : 0);
};
static_assert(kCols == kDecodeBM, "a decode row tile is one m-tile");

struct PersistPlan {
  int run_rows;      // rows per contiguous weight run of a unit: 8
  int row_tiles;     // units per m-tile
};

static PersistPlan persist_plan(int mode, int nout) {
  PersistPlan p{};
  p.run_rows = kRunRows;
  p.row_tiles = nout / (mode == kGateUp ? kRunRows : kUnitRows);
  return p;
}

// K-groups per wave for nb blocks (0: K outside this path)
static int persist_hg(int nb) {
  const int ng = (nb + 3) / 4;
  if (ng < 2 || ng > 2 * kMaxHG) return 0;
  for (int hg : {1, 2, 3, 6, 12})
    if (2 * hg >= ng) return hg;
  return 0;
}

static bool persist_fits(int nb, uint32_t act_bytes) {
  return act_bytes != 0 && persist_hg(nb) != 0;
}

// Lane i of each 16-lane row takes lane (i + 4q) mod 16 of the same row.
template <int Q>
__device__ __forceinline__ uint4 row_rotate4(uint4 v) {
  if (Q == 0) return v;
  constexpr int ctrl = 0x120 + 16 - 4 * Q;   // DPP row_ror:(16 - 4Q)
  return make_uint4((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, ctrl, 0xf, 0xf, true),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, ctrl, 0xf, 0xf, true),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, ctrl, 0xf, 0xf, true),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, ctrl, 0xf, 0xf, true));
}

template <int Q>
__device__ __forceinline__ float rot4_f32(float v) {
  constexpr int ctrl = 0x120 + 16 - 4 * Q;   // DPP row_ror:(16 - 4Q)
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, true));
}

// NV: NVFP4 weights (16-element blocks with E4M3 scales: two scales per
// 32-element chunk; the tensor's global scale is applied to the sums).  The
// NVFP4 kernels multiply f16 operands: the weights expand exactly to f16
// (fp4x8_times_f16, half the instructions of the bf16 form), and each m-tile
// column's bf16 activations are scaled by a power of two 2^-k that puts the
// column's max |x| in [2^14, 2^15) and converted to f16, exactly for every
// value of at least max|x| * 2^-32 (smaller ones round to f16 subnormals:
// at most max|x| * 2^-40 each); the sums are multiplied by 2^k.
// RT (gate_up of decode batches only): every block first routes the whole
// batch itself (T <= 8 tokens, T * k <= 128 pairs, E <= 128) with the router
// and permutation of the stand-alone route + permutation kernel, into its
// LDS; block 0 also writes the router outputs and the permutation to global
// memory for the down and combine kernels.  This replaces a single-block
// launch (about 8 us plus a launch gap) by a prologue of about 5 us.
template <int MODE, int HG, bool NV, bool RT = false>
__global__ __launch_bounds__(128) void gemv_persist_kernel(
    GemvArgs a, PersistPlan P, const int* __restrict__ tiles, const int* __restrict__ sorted_pairs,
    const int* __restrict__ status) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  constexpr bool kPair = MODE == kGateUp;
  static_assert(!RT || (MODE == kGateUp && !NV), "only the MXFP4 gate_up routes");
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  using RL = RunLayout<NV>;

  int64_t mtiles;
  if constexpr (RT) {
    int* rl = reinterpret_cast<int*>(smem + RL::kLds);
    int* ids_l = rl;
    int* eoff_l = rl + kSmallMaxPairs;
    int* sorted_l = rl + 2 * kSmallMaxPairs;
    int* st_l = rl + 3 * kSmallMaxPairs;
    int* tiles_l = rl + kRouteLdsInts;
    // 16 lanes per token, 8 tokens per round; every round's logits are
    // loaded first, so the rounds wait for memory once
    constexpr int kRounds = kGateUpRouteMaxTokens / 8;
    const int l16 = lane & 15, tw = lane >> 4;
    uint32_t keys[kRounds][8];
#pragma unroll
    for (int rd = 0; rd < kRounds; ++rd) {
      const int t = 8 * rd + 4 * kh + tw;
      const bool live = t < a.T;
      route16_keys(a.logits + (size_t)(live ? t : 0) * a.E, live, a.E, l16, keys[rd]);
    }
#pragma unroll
    for (int rd = 0; rd < kRounds; ++rd) {
      if (8 * rd >= a.T) break;
      const int t = 8 * rd + 4 * kh + tw;
      int id;
      float w;
      route16_pick(keys[rd], a.topk, l16, id, w);
      if (t < a.T && l16 < a.topk) {
        ids_l[t * a.topk + l16] = id;
        if (blockIdx.x == 0) {
          a.ids_out[t * a.topk + l16] = id;
          a.w_out[t * a.topk + l16] = w;
        }
      }
    }
    __syncthreads();
    if (kh == 0) {
      const PermDst dl{nullptr, sorted_l, nullptr, tiles_l, st_l};
      const PermDst dg = blockIdx.x == 0 ? PermDst{a.g_offsets, a.g_sorted, a.g_inv, a.g_tiles, a.g_status}
                                          : PermDst{nullptr, nullptr, nullptr, nullptr, nullptr};
      permute_wave(ids_l, a.T * a.topk, a.E, kCols, a.bound, eoff_l, dl, dg);
    }
    __syncthreads();
    tiles = tiles_l;
    sorted_pairs = sorted_l;
    mtiles = st_l[kStNumTiles];
  } else {
    mtiles = MODE == kDense ? (a.M + kCols - 1) / kCols : status[kStNumTiles];
  }

  // this block's units
  const int64_t U = mtiles * P.row_tiles;
  const int64_t u_begin = U * blockIdx.x / gridDim.x;
  const int64_t u_end = U * (blockIdx.x + 1) / gridDim.x;
  if (u_begin >= u_end) return;   // the same for both waves: no barrier is skipped by one

  const int64_t rb = (int64_t)a.nb * kBlockBytes;
  constexpr int kRunBytes = RL::kRunBytes;
  v4f* red = reinterpret_cast<v4f*>(smem + RL::kBufBytes);
  const int nsr = NV ? 2 * a.nb : a.nb;               // scale bytes per weight row

  // DMA of this wave's run (rows 8kh..8kh+7 of a unit) into buffer `buf`; the
  // tail lanes of the last instruction re-read the run's last 16 bytes
  const int64_t wrun = kRunRows * rb;                 // weight bytes of the run
  const int64_t srun = (int64_t)kRunRows * nsr;       // scale bytes (4-byte aligned run)
  const uint32_t wlast = (uint32_t)(wrun - 16), slast = (uint32_t)(srun - 4);
  const uint32_t lane16 = 16u * lane, lane4 = 4u * lane;
  auto issue_dma = [&](int e, int n0) {
    // first row of the run: gate_up wave 1 takes the matching up rows
    const size_t row0 = (size_t)e * a.rows_per_expert + n0 + (kPair ? (size_t)kh * a.nout : (size_t)kh * kRunRows);
    const uint8_t* gw = a.wb + row0 * rb;
    const uint8_t* gs = a.ws + row0 * nsr;
    uint8_t* dst = smem + kh * kRunBytes;
#pragma unroll
    for (int c = 0; c < kRunDma; ++c) {
      const uint32_t off = min((uint32_t)(c * 1024) + lane16, wlast);
      __builtin_amdgcn_global_load_lds(gw + off, dst + c * 1024, 16, 0, 2);
    }
#pragma unroll
    for (int c = 0; c < RL::kScDma; ++c) {
      const uint32_t off = min((uint32_t)(c * 256) + lane4, slast);
      __builtin_amdgcn_global_load_lds(gs + off, dst + kRunDma * 1024 + c * 256, 4, 0, 2);
    }
  };

  // m-tile of a unit: expert, first sorted row, end row
  auto tile_of = [&](int64_t m, int& e, int& rbeg, int& rend) {
    if (MODE == kDense) {
      e = 0;
      rbeg = (int)m * kCols;
      rend = min(rbeg + kCols, a.M);
    } else {
      const int4 t = *reinterpret_cast<const int4*>(tiles + kTileInts * m);
      e = t.x;
      rbeg = t.y;
      rend = t.z;
    }
  };
  constexpr int kUnitStep = kPair ? kRunRows : kUnitRows;   // first rows of consecutive units

  // activations of an m-tile (compact layout), this wave's groups only
  const int gl = kh * HG;
  const int xt = lane & 3;
  const int xq = (lane >> 2) & 3;
  const uint32_t rowb = (uint32_t)(a.nb * kBlockElems * 2);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, (int)a.act_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(MODE == kDown ? a.act_lo : a.act), (short)0,
                                        (int)a.act_bytes, 0x00020000);
  uint4 xa[HG];
  uint4 xl[MODE == kDown ? HG : 1];
  bool x_new = true;   // NVFP4: xa (xl) hold a new m-tile's bf16 values
  int xk = 0;          // NVFP4: the lane's column exponent k
  auto load_x = [&](int rbeg, int rend) {
    x_new = true;
    const int ncols = rend - rbeg;
    int arow = rbeg + min(xt, ncols - 1);
    if (MODE == kGateUp) {   // token of the lane's column
      int p = sorted_pairs[rbeg];
#pragma unroll
      for (int c = 1; c < kCols; ++c) {
        const int pc = sorted_pairs[rbeg + min(c, ncols - 1)];
        p = xt == c ? pc : p;
      }
      arow = p / a.topk;
    }
    const bool xt_ok = xt < ncols;
    const uint32_t xoff = (uint32_t)arow * rowb + (uint32_t)(32 * g + 8 * xq) * 2;
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      const int j = gl + jj;
      const bool ok = xt_ok && 4 * j + g < a.nb;
      const uint32_t off = ok ? xoff + 256u * j : 0x80000000u;
      const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
      xa[jj] = make_uint4(v.x, v.y, v.z, v.w);
      if (MODE == kDown) {
        const v4u_t vl = __builtin_amdgcn_raw_buffer_load_b128(lrs, off, 0, 0);
        xl[jj] = make_uint4(vl.x, vl.y, vl.z, vl.w);
      }
    }
  };

  // bias of the rows wave 0's lane stores (rows n0 + 4g .. +3; gate_up: the
  // gate lanes g < 2 also need the matching up rows)
  uint2 bias_a = make_uint2(0, 0), bias_b = make_uint2(0, 0);
  auto load_bias = [&](int e, int n0) {
    if (kh == 0 && a.bias) {
      const uint16_t* be = a.bias + (size_t)e * a.rows_per_expert + n0 + 4 * (kPair ? (g & 1) : g);
      bias_a = *reinterpret_cast<const uint2*>(be);
      if (kPair) bias_b = *reinterpret_cast<const uint2*>(be + a.nout);
    }
  };

  // staging reads: lane (r, g), group jj -> block 4(gl + jj) + g of unit row r
  // (run r / 8, row r % 8 of the run)
  const int lrun = r / kRunRows, lrr = r % kRunRows;
  const int wrow_off = lrun * kRunBytes + lrr * (int)rb;
  const int srow_off = lrun * kRunBytes + kRunDma * 1024 + lrr * nsr;

  auto step = [&](v4f& acc, const v8bf& A, const uint4& b, const uint4& bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_v8bf(b), acc, 0, 0, 0);
    if (MODE == kDown) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_v8bf(bl), acc, 0, 0, 0);
  };
  auto step_h = [&](v4f& acc, const v8h& A, const uint4& b, const uint4& bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(v8h, b), acc, 0, 0, 0);
    if (MODE == kDown)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(v8h, bl), acc, 0, 0, 0);
  };
  // NVFP4: max |x| over the lane's chunks (bf16 magnitude bits), then over
  // the wave's 16 lanes of the same column (lane % 4)
  uint32_t* xmax_l = reinterpret_cast<uint32_t*>(smem + RL::kBufBytes + 64 * 16);
  auto column_max = [&]() {
    uint32_t mx = 0;
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      const uint32_t d[4] = {xa[jj].x, xa[jj].y, xa[jj].z, xa[jj].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = max(mx, max(d[i] & 0x7fffu, (d[i] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int sh = 4; sh < 64; sh <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, sh, 64));
    return mx;
  };
  // NVFP4: the m-tile's activations (both waves' maxima in LDS) as f16 times
  // 2^-k, in place
  auto to_f16 = [&]() {
    const uint32_t mx = max(xmax_l[xt], xmax_l[kCols + xt]);
    const int ex = (int)(mx >> 7);                 // bf16 exponent field (finite x)
    xk = ex == 0 ? 0 : ex - 141;                   // max|x| * 2^-k in [2^14, 2^15)
    auto cvt = [&](uint32_t d) {
      const v2h p = {(_Float16)ldexpf(__uint_as_float(d << 16), -xk),
                     (_Float16)ldexpf(__uint_as_float(d & 0xffff0000u), -xk)};
      return __builtin_bit_cast(uint32_t, p);
    };
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      xa[jj] = make_uint4(cvt(xa[jj].x), cvt(xa[jj].y), cvt(xa[jj].z), cvt(xa[jj].w));
      if (MODE == kDown) xl[jj] = make_uint4(cvt(xl[jj].x), cvt(xl[jj].y), cvt(xl[jj].z), cvt(xl[jj].w));
    }
  };
  // The activations stay in the compact layout: lane (c, g) holds K chunk
  // (c / 4) % 4 of column c % 4.  MFMA step Q multiplies weight chunk Q, so
  // in accumulator Q only columns 4Q .. 4Q+3 hold valid sums (those of
  // columns 0-3); the epilogue rotates them into place once per unit.

  // unit u = m-tile m, row tile nt (stepped without dividing)
  int64_t u = u_begin;
  int64_t m = u_begin / P.row_tiles;
  int nt = (int)(u_begin - m * P.row_tiles);
  int e, rbeg, rend;
  tile_of(m, e, rbeg, rend);
  int n0 = nt * kUnitStep;
  issue_dma(e, n0);
  load_x(rbeg, rend);
  load_bias(e, n0);
  for (;;) {
    // Blocks sharing a compute unit do not progress alike (its waves are
    // issued oldest first: with equal shares a CU's first-dispatched block
    // ended, on average, 18 us before its last at 32 tokens).  A wave's issue
    // priority follows the share of its block's units still ahead of it:
    // blocks that are behind get the higher priority and catch up.
    {
      const int64_t left = u_end - u;
      const int64_t n = u_end - u_begin;
      if (4 * left > 3 * n) __builtin_amdgcn_s_setprio(3);
      else if (2 * left > n) __builtin_amdgcn_s_setprio(2);
      else if (4 * left > n) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(0);            // this wave's run of unit u, activations, bias
    if constexpr (NV) {
      if (x_new) {
        const uint32_t mx = column_max();
        if (lane < kCols) xmax_l[kh * kCols + lane] = mx;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    asm volatile("s_barrier" ::: "memory");   // both runs of unit u have landed
    if constexpr (NV) {
      if (x_new) {
        to_f16();
        x_new = false;
      }
    }
    // blocks past K (up to 8 HG - 1 < 96) read bytes inside the run's region
    // (finite FP4 codes or stale scales); their scale is forced to 0 below
    // scale bytes of groups jj: MXFP4 one per group, packed four per
    // register; NVFP4 two per group (the chunk's two 16-element blocks),
    // packed two groups per register
    constexpr int kSpk = NV ? (HG + 1) / 2 : (HG + 3) / 4;
    uint32_t spk[kSpk];
    if (NV) {
      const uint8_t* ssrc = smem + srow_off + 2 * (4 * gl + g);
#pragma unroll
      for (int k2 = 0; k2 < kSpk; ++k2) {
        uint32_t p = *reinterpret_cast<const uint16_t*>(ssrc + 8 * (2 * k2));
        if (2 * k2 + 1 < HG) p |= (uint32_t)*reinterpret_cast<const uint16_t*>(ssrc + 8 * (2 * k2 + 1)) << 16;
        spk[k2] = p;
      }
    } else {
      const uint8_t* ssrc = smem + srow_off + 4 * gl + g;
#pragma unroll
      for (int k4 = 0; k4 < kSpk; ++k4) {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 4 && 4 * k4 + i < HG; ++i) p |= (uint32_t)ssrc[4 * (4 * k4 + i)] << (8 * i);
        spk[k4] = p;
      }
    }
    uint4 wreg[HG];
    const uint8_t* wsrc = smem + wrow_off + (4 * gl + g) * kBlockBytes;
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) wreg[jj] = *reinterpret_cast<const uint4*>(wsrc + jj * 4 * kBlockBytes);
    // both waves have read the buffer: the next unit's DMA may overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool more = u + 1 < u_end;
    const bool next_tile = nt + 1 == P.row_tiles;
    int e1 = e, rbeg1 = rbeg, rend1 = rend;
    const int n01 = next_tile ? 0 : n0 + kUnitStep;
    if (more) {
      if (next_tile) tile_of(m + 1, e1, rbeg1, rend1);
      issue_dma(e1, n01);
    }
    v4f acc0 = {0.f, 0.f, 0.f, 0.f};
    v4f acc1 = {0.f, 0.f, 0.f, 0.f};
    v4f acc2 = {0.f, 0.f, 0.f, 0.f};
    v4f acc3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      const uint4 w = wreg[jj];
      // blocks past K (factor 0) contribute 0
      const bool in_k = 4 * (gl + jj) + g < a.nb;
      float f0, f1;   // factors of elements 0-15 and 16-31 of the lane's chunk
      if (NV) {
        // E4M3 block scales, applied whole (mantissa included) below
        const uint32_t sw = (spk[jj / 2] >> (16 * (jj % 2))) & 0xffffu;
        const v2f fs = e4m3x2_to_f32(sw);
        f0 = in_k ? fs[0] : 0.0f;
        f1 = in_k ? fs[1] : 0.0f;
      } else {
        const uint32_t sc = (spk[jj / 4] >> (8 * (jj % 4))) & 0xffu;
        f0 = f1 = e8m0_to_f32(in_k ? sc : 0u);
      }
      const uint4 lo = MODE == kDown ? xl[jj] : xa[jj];
      if constexpr (NV) {
        const NvScale s0 = nv_scale(f0), s1 = nv_scale(f1);
        step_h(acc0, fp4x8_times_f16(w.x, s0), xa[jj], lo);
        step_h(acc1, fp4x8_times_f16(w.y, s0), xa[jj], lo);
        step_h(acc2, fp4x8_times_f16(w.z, s1), xa[jj], lo);
        step_h(acc3, fp4x8_times_f16(w.w, s1), xa[jj], lo);
      } else {
        step(acc0, fp4x8_to_bf16(w.x, f0), xa[jj], lo);
        step(acc1, fp4x8_to_bf16(w.y, f0), xa[jj], lo);
        step(acc2, fp4x8_to_bf16(w.z, f1), xa[jj], lo);
        step(acc3, fp4x8_to_bf16(w.w, f1), xa[jj], lo);
      }
    }
    // lane c of each 16-lane row takes chunk Q's sums from lane c + 4Q
    v4f acc;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      acc[jj] = (acc0[jj] + rot4_f32<1>(acc1[jj])) + (rot4_f32<2>(acc2[jj]) + rot4_f32<3>(acc3[jj]));
    if (kh == 1) red[lane] = acc;
    // wave 1's partial sums are in LDS; the next unit's DMA stays in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kh == 0) {
      acc += red[lane];
      if constexpr (NV) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[jj] = ldexpf(acc[jj], xk) * a.gscale;
      }
      // lane (column r, group g) holds rows 4g + jj of column r
      const int row = rbeg + r;
      const bool col_ok = r < rend - rbeg;
      const int nbase = n0 + 4 * (kPair ? (g & 1) : g);
      const float bia[4] = {bf16_bits_to_f32(bias_a.x & 0xffffu), bf16_bits_to_f32(bias_a.x >> 16),
                            bf16_bits_to_f32(bias_a.y & 0xffffu), bf16_bits_to_f32(bias_a.y >> 16)};
      if (MODE == kGateUp) {
        float upv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) upv[jj] = __shfl_xor(acc[jj], 32, 64);
        if (g < 2 && col_ok) {
          const float bib[4] = {bf16_bits_to_f32(bias_b.x & 0xffffu), bf16_bits_to_f32(bias_b.x >> 16),
                                bf16_bits_to_f32(bias_b.y & 0xffffu), bf16_bits_to_f32(bias_b.y >> 16)};
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float gate = acc[jj] + bia[jj], up = upv[jj] + bib[jj];
            const float h = silu(gate) * up;
            hi[jj] = f32_to_bf16_bits(h);
            lo[jj] = f32_to_bf16_bits(h - bf16_bits_to_f32(hi[jj]));
          }
          const size_t o = (size_t)row * a.nout + nbase;
          *reinterpret_cast<uint2*>(a.out_hi + o) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
          *reinterpret_cast<uint2*>(a.out_lo + o) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        }
      } else if (col_ok) {
        float v[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = acc[jj] + bia[jj];
        if (MODE == kDown) {
          *reinterpret_cast<float4*>(a.y + (size_t)row * a.nout + nbase) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          const uint32_t o0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          const uint32_t o1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(a.out_hi + (size_t)row * a.nout + nbase) = make_uint2(o0, o1);
        }
      }
    }
    if (!more) break;
    if (rbeg1 != rbeg || rend1 != rend) load_x(rbeg1, rend1);
    load_bias(e1, n01);
    ++u;
    if (next_tile) {
      ++m;
      nt = 0;
    } else {
      ++nt;
    }
    e = e1; rbeg = rbeg1; rend = rend1; n0 = n01;
  }
}

// Blocks of the persistent kernel: as many as are resident at once on the
// device (compute units x resident blocks per unit, queried per kernel and
// LDS size).
template <int MODE, int HG, bool NV, bool RT = false>
static hipError_t launch_persist_hg(const GemvArgs& a, const PersistPlan& P, const int* tiles,
                                    const int* sorted_pairs, const int* status, hipStream_t s,
                                    size_t extra_lds = 0) {
  const size_t lds = RunLayout<NV>::kLds + extra_lds;
  // (device + 1) << 48 | lds << 24 | blocks, cached per kernel; threads may
  // race to fill it, but every writer stores the same value for its key
  static std::atomic<uint64_t> cache{0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t key = ((uint64_t)(dev + 1) << 48) | ((uint64_t)lds << 24);
  uint64_t c = cache.load(std::memory_order_relaxed);
  if ((c & ~0xffffffull) != key) {
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemv_persist_kernel<MODE, HG, NV, RT>, 128,
                                                       lds);
    if (err != hipSuccess) return err;
    c = key | (uint64_t)(cus * (per_cu > 0 ? per_cu : 1));
    cache.store(c, std::memory_order_relaxed);
  }
  const unsigned blocks = (unsigned)(c & 0xffffffu);
  gemv_persist_kernel<MODE, HG, NV, RT><<<blocks, 128, lds, s>>>(a, P, tiles, sorted_pairs, status);
  return hipGetLastError();
}

template <int MODE, bool NV = false, bool RT = false>
static hipError_t launch_persist(const GemvArgs& a, const PersistPlan& P, const int* tiles,
                                 const int* sorted_pairs, const int* status, hipStream_t s,
                                 size_t extra_lds = 0) {
  switch (persist_hg(a.nb)) {
    case 1: return launch_persist_hg<MODE, 1, NV, RT>(a, P, tiles, sorted_pairs, status, s, extra_lds);
    case 2: return launch_persist_hg<MODE, 2, NV, RT>(a, P, tiles, sorted_pairs, status, s, extra_lds);
    case 3: return launch_persist_hg<MODE, 3, NV, RT>(a, P, tiles, sorted_pairs, status, s, extra_lds);
    case 6: return launch_persist_hg<MODE, 6, NV, RT>(a, P, tiles, sorted_pairs, status, s, extra_lds);
    case 12: return launch_persist_hg<MODE, 12, NV, RT>(a, P, tiles, sorted_pairs, status, s, extra_lds);
    default: return hipErrorInvalidValue;
  }
}

// Row tiles of 16 rows; KSPLIT waves per row tile, 4 waves per block.
template <int MODE>
static hipError_t launch_gemv(const GemvArgs& a, int nout, int64_t ytiles, int ksplit, hipStream_t s) {
  const int per_block = 4 / ksplit;
  const dim3 grid((unsigned)((nout / 16 + per_block - 1) / per_block), (unsigned)ytiles);
  switch (ksplit) {
    case 1: gemv_bf16_kernel<MODE, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: gemv_bf16_kernel<MODE, 2><<<grid, 256, 0, s>>>(a); break;
    default: gemv_bf16_kernel<MODE, 4><<<grid, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

// Split K when the launch would have fewer than ~8 waves per CU otherwise.
static int pick_ksplit(int64_t row_tiles) {
  if (row_tiles >= 2048) return 1;
  if (row_tiles >= 1024) return 2;
  return 4;
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
  const size_t xbytes = (size_t)sh.T * sh.H * 2;
  a.act_bytes = (uint32_t)(xbytes < (1u << 31) ? xbytes : 0);
  a.sorted_pairs = ws.sorted_pairs;
  a.topk = sh.k;
  a.tiles = ws.tiles;
  a.offsets = ws.offsets;
  a.status = ws.status;
  uint16_t* h = static_cast<uint16_t*>(ws.h);
  a.out_hi = h;
  a.out_lo = h + (size_t)sh.T * sh.k * sh.I;
  // expected busy row tiles: one m-tile per routed pair at most
  const int64_t pairs = (int64_t)sh.T * sh.k;
  const int64_t busy = (pairs < sh.E ? pairs : sh.E) * (sh.I / 16);
  if (w.nvfp4) {
    // NVFP4 runs on the persistent kernel only
    if (!persist_fits(a.nb, a.act_bytes)) return hipErrorInvalidValue;
    a.gscale = w.w13_global;
    return launch_persist<kGateUp, true>(a, persist_plan(kGateUp, sh.I), ws.tiles, ws.sorted_pairs,
                                         ws.status, s);
  }
  a.gscale = 1.0f;
  if (persist_fits(a.nb, a.act_bytes))
    return launch_persist<kGateUp>(a, persist_plan(kGateUp, sh.I), ws.tiles, ws.sorted_pairs,
                                   ws.status, s);
  return launch_gemv<kGateUp>(a, sh.I, ntile_bound, pick_ksplit(busy), s);
}

bool gateup_routes_batch(const MoeShape& sh, bool nvfp4) {
  const int64_t pairs = (int64_t)sh.T * sh.k;
  const size_t xbytes = (size_t)sh.T * sh.H * 2;
  return !nvfp4 && sh.T >= 1 && sh.T <= kGateUpRouteMaxTokens && pairs <= kSmallMaxPairs &&
         sh.E <= kSmallMaxExperts && sh.k <= kSmallMaxK && xbytes < (1u << 31) &&
         persist_fits(sh.H / kBlockElems, (uint32_t)xbytes);
}

hipError_t launch_moe_gateup_bf16_routed(const uint16_t* x, const float* logits, int* ids, float* wts,
                                         const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                         int64_t ntile_bound, hipStream_t s) {
  if (!gateup_routes_batch(sh, w.nvfp4)) return hipErrorInvalidValue;
  GemvArgs a{};
  a.wb = w.w13_blocks;
  a.ws = w.w13_scales;
  a.bias = w.w13_bias;
  a.rows_per_expert = 2 * (int64_t)sh.I;
  a.nout = sh.I;
  a.nb = sh.H / kBlockElems;
  a.act = x;
  a.act_bytes = (uint32_t)((size_t)sh.T * sh.H * 2);
  a.topk = sh.k;
  uint16_t* h = static_cast<uint16_t*>(ws.h);
  a.out_hi = h;
  a.out_lo = h + (size_t)sh.T * sh.k * sh.I;
  a.gscale = 1.0f;
  a.logits = logits;
  a.T = sh.T;
  a.E = sh.E;
  a.bound = (int)ntile_bound;
  a.ids_out = ids;
  a.w_out = wts;
  a.g_status = ws.status;
  a.g_offsets = ws.offsets;
  a.g_sorted = ws.sorted_pairs;
  a.g_inv = ws.inv;
  a.g_tiles = ws.tiles;
  return launch_persist<kGateUp, false, true>(a, persist_plan(kGateUp, sh.I), nullptr, nullptr, nullptr, s,
                                              route_lds_bytes((int)ntile_bound));
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
  const size_t hbytes = (size_t)sh.T * sh.k * sh.I * 2;
  a.act_bytes = (uint32_t)(hbytes < (1u << 31) ? hbytes : 0);
  a.tiles = ws.tiles;
  a.offsets = ws.offsets;
  a.status = ws.status;
  a.y = ws.y;
  const int64_t pairs = (int64_t)sh.T * sh.k;
  const int64_t busy = (pairs < sh.E ? pairs : sh.E) * (sh.H / 16);
  if (w.nvfp4) {
    if (!persist_fits(a.nb, a.act_bytes)) return hipErrorInvalidValue;
    a.gscale = w.w2_global;
    return launch_persist<kDown, true>(a, persist_plan(kDown, sh.H), ws.tiles, ws.sorted_pairs,
                                       ws.status, s);
  }
  a.gscale = 1.0f;
  if (persist_fits(a.nb, a.act_bytes))
    return launch_persist<kDown>(a, persist_plan(kDown, sh.H), ws.tiles, ws.sorted_pairs,
                                 ws.status, s);
  return launch_gemv<kDown>(a, sh.H, ntile_bound, pick_ksplit(busy), s);
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
  const size_t xbytes = (size_t)M * K * 2;
  a.act_bytes = (uint32_t)(xbytes < (1u << 31) ? xbytes : 0);
  a.M = M;
  a.out_hi = out;
  const int64_t mt = (M + 15) / 16;
  const int64_t row_tiles = (int64_t)(N / 16) * mt;
  if (persist_fits(a.nb, a.act_bytes) && row_tiles >= 2048)
    return launch_persist<kDense>(a, persist_plan(kDense, N), nullptr, nullptr, nullptr, s);
  return launch_gemv<kDense>(a, N, mt, pick_ksplit(row_tiles), s);
}

}  // namespace mx
