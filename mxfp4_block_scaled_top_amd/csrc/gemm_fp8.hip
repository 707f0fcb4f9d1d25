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
//     b + 2G, ...; a unit is nsteps K steps of 128 (256 with MXFP4
//     activations).  (Placing the n-tiles of
//     one row tile on one XCD, to share its activations in that XCD's L2, made
//     no measurable difference.)
//   * Every K step's activations (BM x 128 B of E4M3 codes, rows in
//     expert-sorted order), weights (256 x 64 B of E2M1) and E8M0 scales are
//     copied from global memory into one slot of an LDS ring by DMA (global ->
//     LDS), STAGES-1 steps ahead of their use.  All waves of the block share
//     the copies: the DMA issue rate is a per-wave limit (measured: about
//     12.5 GB/s per wave whether the data comes from L2 or HBM, scaling with
//     the number of issuing waves).  Each wave issues the same number of DMA
//     instructions every step, so before the step's barrier it waits for
//     exactly its part of the slot that step needs, with an explicit
//     vector-memory count.
//   * The compute reads of the ring are inline-assembly LDS loads with their
//     own lgkmcnt wait.  The compiler does not track which ring slot a DMA
//     writes and would otherwise wait for every DMA in flight before any LDS
//     read, which serialises the ring.  Tile-list entries and biases come
//     through the scalar cache, so no other load enters the vector-memory
//     counts.
//   * One barrier per K step: after it the slot of step t has landed and the
//     slot of step t-1 is free to be refilled with step t+STAGES-1.
//   * BM/16 waves (two per SIMD at BM = 128), each 64 sorted rows x 64 weight
//     rows (4 x 4 MFMA tiles of 16 x 16).
//   * LDS layouts are XOR-swizzled at 16-byte granularity, chosen through
//     each lane's DMA source address, so that the MFMA-layout reads hit
//     distinct banks in each pass of a 16-byte read (lanes 0-7 with 16-23,
//     8-15 with 24-31, ..., over 64 four-byte banks; the bank-conflict
//     counter reads zero for every read here).
//   * K tails: chunks past K are loaded from a valid address and the weight
//     operand of MX blocks past K is forced to zero.
#include "common.hpp"
#include "launch.hpp"
#include "code_rows.hpp"

namespace mx {

constexpr int kBN = 256;               // weight rows per unit
constexpr int kBK = 128;               // K per step (four MX blocks)
constexpr int kCodeChunk = kBN * kBK / 2;  // restaged codes per (n-tile, step): 16 KB
constexpr int kSchedRows = 4;          // row tiles of one expert per group of the unit schedule

// A4: MXFP4 activations, K steps of 256 (eight MX blocks): 128 B of E2M1
// codes per activation and weight row, so every 1 KB copy covers 8 whole
// 128-byte lines, plus two dwords of E8M0 scales per row.  Otherwise E4M3
// activations, K steps of 128: 128 B per activation row, 64 B per weight
// row, one dword of scales per weight row.
// NV: NVFP4 weights (E4M3 activations only): the same 64 B of E2M1 codes per
// weight row and step, two E4M3 scales per 32 elements (8 bytes per row and
// step instead of 4).
// WN (wide-N units, BM = 64, E4M3 activations): a unit is 64 sorted rows x
// two n-tiles (512 weight rows); waves 0-3 take the first n-tile, 4-7 the
// second, each 64 rows x 64 weight rows as in the 128-row tiles; three
// slots of 42 KB (NVFP4: 44 KB).
template <int BM, bool A4 = false, bool NV = false, bool WN = false>
struct Ring {
  static constexpr int kWaves = 8;                      // each 64 sorted rows x 64 weight rows
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBNu = WN ? 2 * kBN : kBN;       // weight rows per unit
  static constexpr int kK = A4 ? 2 * kBK : kBK;         // K per step
  static constexpr int kSub = kK / kBK;                 // 128-element sub-steps per step (scale dwords per row)
  static constexpr int kStages = A4 || WN ? 3 : 4;
  static constexpr int kActRow = A4 ? kK / 2 : kK;      // activation bytes per row per step
  static constexpr int kWRow = kK / 2;                  // weight bytes per row per step
  static constexpr int kAct = BM * kActRow;             // activation bytes per slot
  static constexpr int kW = kAct;                       // offsets inside a slot
  static constexpr int kSc = kAct + kBNu * kWRow;
  static constexpr int kScRow = NV ? 8 : 4;             // weight-scale bytes per row and 128-element step
  static constexpr int kASc = kSc + kBNu * kScRow * kSub; // A4: activation scales, 4 B per row and sub-step
  static constexpr int kSlot = kASc + (A4 ? BM * 4 * kSub : 0);
  static constexpr int kActDma = BM * kActRow / 1024 / kWaves;  // 1 KB activation DMAs per wave per step
  static constexpr int kWDma = kBNu * kWRow / 1024 / kWaves;    // 1 KB weight DMAs per wave per step
  // the step's weight scales: E4M3 activations, the wave's 1/8; A4 (two
  // 128-element sub-steps), whole 1 KB copies by waves 0 and 1, and both
  // sub-steps' activation scales (512 B each) by wave 2
  static constexpr int kScDma = 1;                      // at most, per wave and step
  static constexpr int kAScDma = 0;
  static constexpr int kDma = kActDma + kWDma + kScDma + kAScDma;  // DMA instructions per wave per step
  static constexpr int kLds = kStages * kSlot;
  static_assert(kActDma * kWaves * 1024 == BM * kActRow, "copies split over the waves");
  static_assert(kWDma * kWaves * 1024 == kBNu * kWRow, "copies split over the waves");
  static_assert(WN ? BM == 64 && !A4 : BM == 128, "tile heights: 128 rows, wide-N units 64");
  static_assert(!(A4 && NV), "NVFP4 weights take E4M3 activations");
  static_assert((kStages - 2) * kDma <= 63, "vector-memory count range");
  static_assert(kStages - 2 <= 4, "waits cover up to four steps ahead");
  static_assert(kLds <= 160 * 1024, "LDS");
};

struct PrefillArgs {
  const uint8_t* wb;       // [E, R, nb, 16]
  const uint8_t* wcs;      // the codes restaged by launch_code_stream, or null (copies then read wb)
  const uint8_t* wsp;      // the weight scales restaged by launch_scale_stream
  const uint16_t* bias;    // [E, R] or null
  int R;                   // rows per expert: 2I (gate_up) or H (down)
  int nout;                // I (gate_up) or H (down)
  int nb;                  // K / 32
  int K;
  int NT;                  // n-tile units per row tile (wide-N: pairs of n-tiles)
  int NTs;                 // n-tiles of the restaged scale stream
  int nsteps;              // K steps: ceil(nb / 4), MXFP4 activations ceil(nb / 8)
  int nsteps_s;            // 128-element steps of the scale streams: ceil(nb / 4)
  const uint8_t* act;      // [sorted rows, K] E4M3 codes, or [sorted rows, K/32, 16] E2M1 blocks
  int act_ld;              // activation row stride in bytes (code_row_bytes: K or K/2, whole 128-B lines)
  const uint8_t* asc;      // E2M1 activations: E8M0 [nsteps, sorted rows, 4] (step-major)
  int64_t asc_step;        // bytes per step of asc (4 * sorted rows)
  int scale_word;          // status word holding the per-tensor activation scale (E4M3)
  float* out;              // h [rows, I] (gate_up, E4M3 mode) or y [rows, H] (down), fp32
  uint16_t* out_bf16;      // down: y rounded once to bf16 [rows, H] in place of out, or null
  float gscale;            // NVFP4 weights: the tensor's global scale (applied to the sums)
  // gate_up with E2M1 activations: h quantised in the epilogue into E2M1
  // blocks [rows, I/32, 16] and step-major E8M0 scales [ceil(I/128), rows, 4]
  uint8_t* h_codes;
  uint8_t* h_scales;
  int64_t h_rows;          // rows of the step-major scale array (T*k)
  int sched_xcd;           // units in expert-major order, one contiguous share per XCD (see unit_tile)
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

// 8 E4M3 codes (two dwords) -> 8 f16 (exact: every E4M3 value is an f16).
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// silu with the hardware exp and reciprocal: a few 1e-7 relative error (at
// most about 3e-6 for |z| <= 50; beyond, silu is z or negligible), inside the
// h error both quantised modes are specified against.
__device__ __forceinline__ float silu_rcp(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }


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

// Word 3 of a tile-list entry (the expert's first entry and entry count).
__device__ __forceinline__ int tile_word_at(const int* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0xc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
  return v;
}

// Unit v of the schedule -> (row tile, n-tile).  Plain order: v = tile * NT
// + nt.  Expert-major order (sched_xcd): the units of expert e, whose row
// tiles are entries [f, f + c) of the list, are v in [NT f, NT (f + c)), in
// groups of kSchedRows row tiles (the last group the remainder), n-tile-major
// inside a group: v = NT (f + g) + nt G + i for tile f + g + i of a group
// of G tiles starting at g.  The grid hands each XCD (blocks b with the same
// b mod 8, the hardware's round-robin placement) one contiguous eighth of
// that order, round-robin over its blocks, so the blocks of one XCD stream
// the same weight n-tile for different row tiles of a hot expert and share
// it in that XCD's L2, while the group's activation rows (kSchedRows tiles,
// read once per n-tile) stay in it too.  Same box at 8192 skewed tokens:
// groups of 4, 8, 16 and one group per expert 1118, 1118, 1118 and 1124 us
// (FP4 x FP4), 1905, 1902, 1907 and 1920 us (FP8).
__device__ __forceinline__ void unit_tile(const PrefillArgs& a, const int* tiles, int v, int& tile, int& nt) {
  if (a.sched_xcd) {
    const int w = tile_word_at(tiles + kTileInts * (v / a.NT));
    const int f = w & 0xffff, c = w >> 16;
    const int local = v - a.NT * f;
    constexpr int G = kSchedRows;
    const int full = c - c % G;     // tiles in whole groups
    if (local < full * a.NT) {
      const int g = local / (G * a.NT), r = local - g * G * a.NT;
      nt = r / G;
      tile = f + g * G + (r - nt * G);
    } else {
      const int rem = c - full, r = local - full * a.NT;
      nt = r / rem;
      tile = f + full + (r - nt * rem);
    }
  } else {
    tile = v / a.NT;
    nt = v - tile * a.NT;
  }
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

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

// bf16 numbers 4g .. 4g+3 of the 16 held in v, for the lane's g (0..3), as
// two dwords picked by a select chain on g
__device__ __forceinline__ uint2 bias_quad(const v8i_t& v, int g) {
  const uint32_t lo = (uint32_t)(g == 0 ? v[0] : g == 1 ? v[2] : g == 2 ? v[4] : v[6]);
  const uint32_t hi = (uint32_t)(g == 0 ? v[1] : g == 1 ? v[3] : g == 2 ? v[5] : v[7]);
  return make_uint2(lo, hi);
}

// 2 x 16 bf16 through the scalar cache in one round trip; p0, p1 wave-uniform
// and 4-byte aligned
__device__ __forceinline__ void sload_bias2(const uint16_t* p0, const uint16_t* p1, v8i_t& v0, v8i_t& v1) {
  asm volatile("s_load_dwordx8 %0, %2, 0x0\n\ts_load_dwordx8 %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1)
               : "s"(p0), "s"(p1));
}

__device__ __forceinline__ float bf16_of(uint2 q, int jj) {
  const uint32_t w = jj < 2 ? q.x : q.y;
  return bf16_bits_to_f32(jj & 1 ? w >> 16 : w & 0xffffu);
}

// A wave's share of the copies of every K step (global -> LDS DMA).
// Activation DMA i fills slot rows 8j..8j+7 (j = NW*i + wave): lane -> row
// 8j + lane/8, 16-byte slot lane%8, which holds logical chunk
// (lane%8) ^ (row%8).  Weight DMA i fills rows 16j..16j+15: lane -> row
// 16j + lane/4, slot lane%4, which holds MX block (lane%4) ^ ((row/2)%4).
// The weight scales come from the restaged stream (launch_scale_stream),
// where a unit's step is 1 KB: the four scale bytes of each of its 256 LDS
// rows in row order.  Wave w copies bytes [128w, 128w + 128) with lanes 0-7,
// one cache line per instruction (the checkpoint layout would need a
// scattered 4-byte read per row: rows are K/32 bytes apart).
//
// A4 (E2M1 activations): activation DMA i fills slot rows 16j..16j+15 like a
// weight DMA (lane -> row 16j + lane/4, slot lane%4 holding MX block
// (lane%4) ^ ((row/2)%4)).  The activation scales are stored step-major, so a
// step's scales of the tile's 128 rows are 512 contiguous bytes; wave w
// copies rows 16w .. 16w+15 with lanes 0-3.
template <bool GATEUP, int BM, bool A4 = false, bool NV = false, bool WN = false>
struct PrefillCopier {
  using C = Ring<BM, A4, NV, WN>;
  static constexpr int NW = C::kWaves;
  const int* tiles;
  uint8_t* smem;
  int wave, u0, G, my_units;
  int lane, a_chunk, a_row, w_row, w_blk;
  const uint8_t* aptr[C::kActDma];
  const uint8_t* wptr[C::kWDma];   // codes of weight copy i: the row (wb), or step 0's 16 bytes (wcs)
  int wback;            // restaged A4 codes: bytes back to the lane's K-tail substitute
  const uint8_t* wsp;   // this lane's 16 bytes of the unit's first step in the scale stream
  const uint8_t* ascp;  // A4: this lane's 16 bytes of the tile's scales at step 0
  int k, step, slot;    // next copy: local unit, step, ring slot

  __device__ __forceinline__ void init(const PrefillArgs& a, const int* t, uint8_t* sm, int w, int lane, int first,
                                       int grid, int units) {
    tiles = t; smem = sm; wave = w; u0 = first; G = grid; my_units = units;
    this->lane = lane;
    // a 1 KB copy fills 8 LDS rows of 128 B (E4M3 activations; A4 activations
    // and weights) or 16 rows of 64 B (E4M3-mode weights); the lane's 16 B
    // slot in its row is fixed, the block fetched into it is slot ^ (row % 8)
    // (128 B rows) or slot ^ ((row / 2) % 4) (64 B rows)
    a_row = lane >> 3;
    a_chunk = (lane & 7) ^ a_row;
    w_row = A4 ? lane >> 3 : lane >> 2;
    w_blk = A4 ? (lane & 7) ^ (lane >> 3) : (lane & 3) ^ ((lane >> 3) & 3);
    k = 0; step = 0; slot = 0;
    setup(a, u0);
  }

  __device__ __forceinline__ void setup(const PrefillArgs& a, int u) {
    int tile, nt;
    unit_tile(a, tiles, u, tile, nt);
    const int3 te = tile_entry(tiles + kTileInts * tile);
#pragma unroll
    for (int i = 0; i < C::kActDma; ++i) {
      int row = te.y + 8 * (NW * i + wave) + a_row;
      row = row < te.z ? row : te.y;
      aptr[i] = a.act + (int64_t)row * a.act_ld;
    }
    // rows past the tile end read other rows' scales (never stored)
    // A4: wave 2 copies the tile's 128 rows of both sub-steps
    if (A4) ascp = a.asc + (int64_t)te.y * 4 + 16 * (lane & 31);
    const int64_t ebase = (int64_t)te.x * a.R;
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i) {
      const int lr = (A4 ? 8 : 16) * (NW * i + wave) + w_row;
      if (a.wcs) {
        // restaged codes: 16 KB per (n-tile, 128-element step) in LDS order
        // (E4M3 activations: copy c takes bytes 1 KB c of the chunk).  A4
        // rows of 128 B take their two 64-byte halves from the chunks of
        // steps 2s and 2s + 1: slot j of row lr holds block 8s + jx, jx =
        // j ^ (lr % 8), which chunk 2s + jx / 4 keeps at slot (jx % 4) ^
        // ((lr / 2) % 4) of the row
        const int h = WN ? lr >> 8 : 0;
        const int ntr = WN ? min(2 * nt + h, a.NTs - 1) : nt;
        const uint8_t* chunk0 = a.wcs + ((int64_t)te.x * a.NTs + ntr) * a.nsteps_s * kCodeChunk;
        if (A4) {
          const int jx = w_blk, hi = jx >> 2;
          wptr[i] = chunk0 + hi * kCodeChunk + lr * 64 + 16 * ((jx & 3) ^ ((lr >> 1) & 3));
          wback = hi * kCodeChunk;
        } else {
          wptr[i] = chunk0 + 1024 * ((NW * i + wave) & 15) + 16 * lane;
        }
      } else {
        // wide-N: LDS rows 256 h .. 256 h + 255 hold n-tile 2 nt + h
        const int wr = WN ? weight_row<GATEUP>(lr & (kBN - 1), 2 * nt + (lr >> 8), a.nout)
                          : weight_row<GATEUP>(lr, nt, a.nout);
        wptr[i] = a.wb + (ebase + wr) * a.nb * kBlockBytes;
      }
    }
    // the unit's stream: 1 KB per 128-element sub-step; A4: wave w copies 256 B
    // (lanes 0-15) of sub-step w / 4, else 128 B (lanes 0-7).  Wide-N: waves
    // 0-3 copy the first n-tile's 1 KB (NVFP4 2 KB), 4-7 the second's (an odd
    // last n-tile re-reads the stream's last one: its outputs are never
    // stored), 256 B (512 B) each
    if (WN) {
      const int ntr = min(2 * nt + (wave >> 2), a.NTs - 1);
      wsp = a.wsp + ((int64_t)te.x * a.NTs + ntr) * a.nsteps_s * (kBN * C::kScRow) +
            (kBN * C::kScRow / 4) * (wave & 3) + 16 * lane;
    } else {
      wsp = a.wsp + ((int64_t)te.x * a.NTs + nt) * a.nsteps_s * (kBN * C::kScRow) +
            (A4 ? 16 * lane : NV ? 256 * wave + 16 * (lane & 15) : 128 * wave + 16 * (lane & 7));
    }
  }

  // copies of the next step into its slot, then advance
  __device__ __forceinline__ void issue(const PrefillArgs& a) {
    issue_act(a);
    issue_w(a);
    advance(a);
  }
  // the activation copies (and the scale copies) of the next step
  __device__ __forceinline__ void issue_act(const PrefillArgs& a) {
    uint8_t* dst = smem + slot * C::kSlot;
    const bool tail = step == a.nsteps - 1;
    const int kb = step * kBK;
#pragma unroll
    for (int i = 0; i < C::kActDma; ++i) {
      if (A4) {
        const int blk = 8 * step + a_chunk;        // past K: the row's first block
        __builtin_amdgcn_global_load_lds(aptr[i] + (!tail || blk < a.nb ? blk * kBlockBytes : 0),
                                         dst + 1024 * (NW * i + wave), 16, 0, 0);
      } else {
        const int off = kb + 16 * a_chunk;         // past K: the row's first 16 bytes
        __builtin_amdgcn_global_load_lds(aptr[i] + (!tail || off < a.K ? off : 0), dst + 1024 * (NW * i + wave),
                                         16, 0, 0);
      }
    }
    if (A4) {
      // sub-step wave / 4 of this step; past the last one (K tail) the last
      // sub-step again (its values are masked)
      const int ss0 = min(2 * step, a.nsteps_s - 1), ss1 = min(2 * step + 1, a.nsteps_s - 1);
      if (wave < 2)
        __builtin_amdgcn_global_load_lds(wsp + (wave ? ss1 : ss0) * 1024, dst + C::kSc + 1024 * wave, 16, 0, 0);
      else if (wave == 2)
        __builtin_amdgcn_global_load_lds(ascp + (lane < 32 ? ss0 : ss1) * a.asc_step, dst + C::kASc, 16, 0, 0);
    } else if (lane < C::kBNu * C::kScRow / C::kWaves / 16) {
      // the scale bytes of rows (kBNu / 8) w .. (kBNu / 8)(w + 1) - 1 (NVFP4:
      // 8 per row)
      __builtin_amdgcn_global_load_lds(wsp + step * (kBN * C::kScRow),
                                       dst + C::kSc + (C::kBNu / C::kWaves) * C::kScRow * wave, 16, 0, 0);
    }
  }
  // the weight copies of the next step
  __device__ __forceinline__ void issue_w(const PrefillArgs& a) {
    uint8_t* dst = smem + slot * C::kSlot;
    const bool tail = step == a.nsteps - 1;
    const int blk = C::kSub * 4 * step + w_blk;    // past K: the row's first block
    if (a.wcs) {
      // restaged: the step's chunk (zeros past K); A4 past K: chunk 2s
      const int64_t off = (int64_t)step * C::kSub * kCodeChunk - (A4 && tail && blk >= a.nb ? wback : 0);
#pragma unroll
      for (int i = 0; i < C::kWDma; ++i)
        __builtin_amdgcn_global_load_lds(wptr[i] + off, dst + C::kW + 1024 * (NW * i + wave), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < C::kWDma; ++i)
        __builtin_amdgcn_global_load_lds(wptr[i] + (!tail || blk < a.nb ? blk * kBlockBytes : 0),
                                         dst + C::kW + 1024 * (NW * i + wave), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void advance(const PrefillArgs& a) {
    slot = slot + 1 == C::kStages ? 0 : slot + 1;
    if (++step == a.nsteps) {
      step = 0;
      if (++k < my_units) setup(a, u0 + k * G);
    }
  }
};

// One K step's operands of a wave from its LDS slot: 8 activation reads
// (two chunks of 4 token-row groups, 2 KB apart), 4 weight reads and 4 scale
// bytes (gate_up: weight groups at LDS rows +0, +16, +128, +144; down: +0,
// +16, +32, +48), issued and waited for in one assembly block so that no
// compiler-generated code sees the registers while the loads are in flight.
#define MX_RD_ACT                                                                    \
  "ds_read_b128 %0, %16\n\tds_read_b128 %4, %17\n\t"                               \
  "ds_read_b128 %1, %16 offset:2048\n\tds_read_b128 %5, %17 offset:2048\n\t"       \
  "ds_read_b128 %2, %16 offset:4096\n\tds_read_b128 %6, %17 offset:4096\n\t"       \
  "ds_read_b128 %3, %16 offset:6144\n\tds_read_b128 %7, %17 offset:6144\n\t"
#define MX_RD_OUTS                                                                   \
  "=&v"(xa0), "=&v"(xa1), "=&v"(xa2), "=&v"(xa3), "=&v"(xb0), "=&v"(xb1), "=&v"(xb2), "=&v"(xb3), \
      "=&v"(wq0), "=&v"(wq1), "=&v"(wq2), "=&v"(wq3), "=&v"(sb0), "=&v"(sb1), "=&v"(sb2), "=&v"(sb3)
// NV (NVFP4 weights): 2 scale bytes per row (the step's 16-element blocks 2g
// and 2g+1), rows 8 B apart.
template <bool GATEUP, bool NV = false>
__device__ __forceinline__ void lds_step_reads(uint32_t aa0, uint32_t aa1, uint32_t ww, uint32_t ss,
                                               v4u_t& xa0, v4u_t& xa1, v4u_t& xa2, v4u_t& xa3,
                                               v4u_t& xb0, v4u_t& xb1, v4u_t& xb2, v4u_t& xb3,
                                               v4u_t& wq0, v4u_t& wq1, v4u_t& wq2, v4u_t& wq3,
                                               uint32_t& sb0, uint32_t& sb1, uint32_t& sb2, uint32_t& sb3) {
  if (NV && GATEUP) {
    asm volatile(MX_RD_ACT
                 "ds_read_b128 %8, %18\n\tds_read_b128 %9, %18 offset:1024\n\t"
                 "ds_read_b128 %10, %18 offset:8192\n\tds_read_b128 %11, %18 offset:9216\n\t"
                 "ds_read_u16 %12, %19\n\tds_read_u16 %13, %19 offset:128\n\t"
                 "ds_read_u16 %14, %19 offset:1024\n\tds_read_u16 %15, %19 offset:1152\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MX_RD_OUTS
                 : "v"(aa0), "v"(aa1), "v"(ww), "v"(ss));
  } else if (NV) {
    asm volatile(MX_RD_ACT
                 "ds_read_b128 %8, %18\n\tds_read_b128 %9, %18 offset:1024\n\t"
                 "ds_read_b128 %10, %18 offset:2048\n\tds_read_b128 %11, %18 offset:3072\n\t"
                 "ds_read_u16 %12, %19\n\tds_read_u16 %13, %19 offset:128\n\t"
                 "ds_read_u16 %14, %19 offset:256\n\tds_read_u16 %15, %19 offset:384\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MX_RD_OUTS
                 : "v"(aa0), "v"(aa1), "v"(ww), "v"(ss));
  } else if (GATEUP) {
    asm volatile(MX_RD_ACT
                 "ds_read_b128 %8, %18\n\tds_read_b128 %9, %18 offset:1024\n\t"
                 "ds_read_b128 %10, %18 offset:8192\n\tds_read_b128 %11, %18 offset:9216\n\t"
                 "ds_read_u8 %12, %19\n\tds_read_u8 %13, %19 offset:64\n\t"
                 "ds_read_u8 %14, %19 offset:512\n\tds_read_u8 %15, %19 offset:576\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MX_RD_OUTS
                 : "v"(aa0), "v"(aa1), "v"(ww), "v"(ss));
  } else {
    asm volatile(MX_RD_ACT
                 "ds_read_b128 %8, %18\n\tds_read_b128 %9, %18 offset:1024\n\t"
                 "ds_read_b128 %10, %18 offset:2048\n\tds_read_b128 %11, %18 offset:3072\n\t"
                 "ds_read_u8 %12, %19\n\tds_read_u8 %13, %19 offset:64\n\t"
                 "ds_read_u8 %14, %19 offset:128\n\tds_read_u8 %15, %19 offset:192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MX_RD_OUTS
                 : "v"(aa0), "v"(aa1), "v"(ww), "v"(ss));
  }
}
#undef MX_RD_ACT
#undef MX_RD_OUTS




// A4, one half (four MX blocks) of a 256-element step: 4 activation reads
// (token-row groups 16 rows = 2 KB apart), 4 weight reads (gate_up: weight
// groups at LDS rows +0, +16, +128, +144; down: +0, +16, +32, +48; rows of
// 128 B), 4 weight-scale bytes and 4 activation-scale bytes, waited for in
// the same assembly block.
__device__ __forceinline__ void lds_half_reads_a4(bool gateup, uint32_t aa, uint32_t ww, uint32_t ss, uint32_t as,
                                                  v4u_t& xa0, v4u_t& xa1, v4u_t& xa2, v4u_t& xa3,
                                                  v4u_t& wq0, v4u_t& wq1, v4u_t& wq2, v4u_t& wq3,
                                                  uint32_t& sb0, uint32_t& sb1, uint32_t& sb2, uint32_t& sb3,
                                                  uint32_t& ab0, uint32_t& ab1, uint32_t& ab2, uint32_t& ab3) {
  if (gateup) {
    asm volatile("ds_read_u8 %8, %18\n\tds_read_u8 %9, %18 offset:64\n\t"
                 "ds_read_u8 %10, %18 offset:512\n\tds_read_u8 %11, %18 offset:576\n\t"
                 "ds_read_u8 %12, %19\n\tds_read_u8 %13, %19 offset:64\n\t"
                 "ds_read_u8 %14, %19 offset:128\n\tds_read_u8 %15, %19 offset:192\n\t"
                 "ds_read_b128 %4, %17\n\tds_read_b128 %5, %17 offset:2048\n\t"
                 "ds_read_b128 %6, %17 offset:16384\n\tds_read_b128 %7, %17 offset:18432\n\t"
                 "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:2048\n\t"
                 "ds_read_b128 %2, %16 offset:4096\n\tds_read_b128 %3, %16 offset:6144\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(xa0), "=&v"(xa1), "=&v"(xa2), "=&v"(xa3), "=&v"(wq0), "=&v"(wq1), "=&v"(wq2),
                   "=&v"(wq3), "=&v"(sb0), "=&v"(sb1), "=&v"(sb2), "=&v"(sb3), "=&v"(ab0), "=&v"(ab1),
                   "=&v"(ab2), "=&v"(ab3)
                 : "v"(aa), "v"(ww), "v"(ss), "v"(as));
  } else {
    asm volatile("ds_read_u8 %8, %18\n\tds_read_u8 %9, %18 offset:64\n\t"
                 "ds_read_u8 %10, %18 offset:128\n\tds_read_u8 %11, %18 offset:192\n\t"
                 "ds_read_u8 %12, %19\n\tds_read_u8 %13, %19 offset:64\n\t"
                 "ds_read_u8 %14, %19 offset:128\n\tds_read_u8 %15, %19 offset:192\n\t"
                 "ds_read_b128 %4, %17\n\tds_read_b128 %5, %17 offset:2048\n\t"
                 "ds_read_b128 %6, %17 offset:4096\n\tds_read_b128 %7, %17 offset:6144\n\t"
                 "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:2048\n\t"
                 "ds_read_b128 %2, %16 offset:4096\n\tds_read_b128 %3, %16 offset:6144\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(xa0), "=&v"(xa1), "=&v"(xa2), "=&v"(xa3), "=&v"(wq0), "=&v"(wq1), "=&v"(wq2),
                   "=&v"(wq3), "=&v"(sb0), "=&v"(sb1), "=&v"(sb2), "=&v"(sb3), "=&v"(ab0), "=&v"(ab1),
                   "=&v"(ab2), "=&v"(ab3)
                 : "v"(aa), "v"(ww), "v"(ss), "v"(as));
  }
}

// A4: E2M1 activations with E8M0 block scales; both operands of the
// block-scaled MFMA are FP4 and carry their own scales, and the epilogue has
// no per-tensor factor.
// NV: NVFP4 weights with E4M3 activations; both GEMMs then expand their
// operands exactly to bf16 (an E4M3 block scale cannot ride on the
// block-scaled MFMA, whose scales are E8M0) and the global scale joins the
// per-tensor activation scale in the epilogue.
// CW (copy waves; gate_up on E4M3 activations with MXFP4 weights, 128-row
// tiles): waves 4-7 issue every copy of the block (two waves' shares each)
// and waves 0-3 none, so that the waves of rows 0-63, which carry the MFMAs
// while the experts average at most 64 rows, never stall behind the copy
// issue.
template <bool GATEUP, int BM, bool A4, bool NV, bool WN, bool CW>
__device__ __forceinline__ void prefill_gemm_body(PrefillArgs a, const int* __restrict__ tiles,
                                                  int* status) {
  using C = Ring<BM, A4, NV, WN>;
  constexpr bool EXP = GATEUP || NV;   // operands expanded to bf16, v_mfma_f32_16x16x32_bf16
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds];
  const int num_units = status[kStNumTiles] * a.NT;
  float sx = A4 ? 1.0f : __uint_as_float((uint32_t)status[a.scale_word]);
  if constexpr (NV) sx *= a.gscale;
  // this block's units: u0, u0 + G, ... (my_units of them) in the schedule
  int u0, G, my_units;
  if (a.sched_xcd) {
    const int x = blockIdx.x & 7, gx = gridDim.x >> 3;
    const int s0 = (int)((int64_t)num_units * x / 8), s1 = (int)((int64_t)num_units * (x + 1) / 8);
    u0 = s0 + (int)(blockIdx.x >> 3);
    G = gx;
    my_units = u0 < s1 ? (s1 - 1 - u0) / gx + 1 : 0;
  } else {
    u0 = blockIdx.x;
    G = gridDim.x;
    my_units = u0 < num_units ? (num_units - 1 - u0) / G + 1 : 0;
  }
  if (my_units == 0) return;
  const int total = my_units * a.nsteps;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // down: the waves of rows 64-127 (the second wave of each SIMD) issue
  // first (same box, 8192 skewed tokens: FP4 x FP4 down 378 -> 369 us, FP8
  // 459 -> 456 us; the gate_up kernels gained nothing)
  if (!GATEUP && wave >= 4) __builtin_amdgcn_s_setprio(2);

  static_assert(!CW || (GATEUP && BM == kPrefillBM && !A4 && !NV && !WN), "copy waves: MXFP4 x E4M3 gate_up");
  static_assert(!CW || (C::kStages - 2) * 2 * C::kDma <= 63, "vector-memory count range");
  const bool copies = !CW || wave >= 4;   // this wave issues copies
  PrefillCopier<GATEUP, BM, A4, NV, WN> cp, cp2;
  cp.init(a, tiles, smem, CW ? wave & 3 : wave, lane, u0, G, my_units);
  if (CW) cp2.init(a, tiles, smem, (wave & 3) + 4, lane, u0, G, my_units);

  // ---------------- compute: 64 sorted rows x 64 weight rows ----------------
  constexpr int kRG = 4;                            // 16-row weight groups per wave
  // wave (wm, wn): 128-row tiles, sorted rows 64 wm .. 64 wm + 63; wide-N
  // units, the unit's n-tile wm; weight rows 64 wn .. 64 wn + 63 of it
  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  // LDS weight row of this lane in the wave's first 16-row group; the others
  // follow at fixed offsets (gate_up: groups 0, 1 gate rows, 2, 3 the
  // matching up rows)
  const int lrow0 = (WN ? kBN * wm : 0) + (GATEUP ? 32 : 64) * wn + r;
  // first sorted row of the wave's 64 (wide-N: every wave takes rows 0-63)
  const int arow = WN ? 0 : 64 * wm;
  const int wslot = g ^ ((r >> 1) & 3);             // slot of MX block g in these rows
  // activation chunks: the bf16 path takes K [32g, 32g+32) = chunks 2g, 2g+1,
  // the block-scaled path chunks g and 4+g; the row's swizzle is row%8 = r%8.
  // A 16-byte LDS read serves lanes 0-7 with 16-23 (and 8-15 with 24-31, ...)
  // in one pass over 64 four-byte banks; for those pairs to hit distinct
  // banks the bf16 path's odd lane groups read chunk 2g+1 first (their K
  // order within the block is then 16..31, 0..15, for both operands).
  const int c0 = (EXP ? 2 * g + (g & 1) : g) ^ (r & 7);
  const int c1 = (EXP ? 2 * g + 1 - (g & 1) : 4 + g) ^ (r & 7);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t a0 = lds0 + (arow + r) * kBK + 16 * c0;
  const uint32_t a1 = lds0 + (arow + r) * kBK + 16 * c1;
  const uint32_t w0 = lds0 + C::kW + lrow0 * 64 + 16 * wslot;
  // scale of MX block g of the step (NVFP4: of its 16-element blocks 2g, 2g+1)
  const uint32_t s0 = lds0 + C::kSc + lrow0 * C::kScRow + (NV ? 2 * g : g);
  // A4 (rows of 128 B, eight 16-byte slots swizzled by row % 8 = r % 8):
  // MX block 4h + g of a row sits in slot (4h + g) ^ (r % 8); the scales of
  // half h sit in the step's second 128-element scale chunk (weights: 1 KB
  // on, activations: 512 B on)
  const uint32_t ax[2] = {lds0 + (64 * wm + r) * 128 + 16 * (g ^ (r & 7)),
                          lds0 + (64 * wm + r) * 128 + 16 * ((4 + g) ^ (r & 7))};
  const uint32_t wx[2] = {lds0 + C::kW + lrow0 * 128 + 16 * (g ^ (r & 7)),
                          lds0 + C::kW + lrow0 * 128 + 16 * ((4 + g) ^ (r & 7))};
  const uint32_t as0 = lds0 + C::kASc + (64 * wm + r) * 4 + g;

  int cstep = 0, cslot = 0, ck = 0;
  int e = 0, rb = 0, re = 0, nt = 0;
  int ntr = 0;   // the wave's n-tile (wide-N units: 2 nt + wm)
  // 16-row groups of this wave's 64 sorted rows that hold rows of the tile:
  // in the FP8 kernels the MFMAs (and activation expansions) of groups
  // wholly past the tile's end are skipped (their outputs are never stored).
  // A tile of an expert with ~64 rows fills only wm = 0's half of the 128
  // rows (same-box A/B: 2048-token FP8 call 781 -> 720 us).  The FP4 x FP4
  // kernels, bound by their copies, gained nothing from it and keep every
  // MFMA.
  int ntg = 4;
  // bias of the lane's four output rows of each epilogue group, as bf16
  // pairs (gate_up: gate and up rows of groups 0 and 1; down: groups 0..3)
  uint2 bq[4];
  auto comp_setup = [&](int u) __attribute__((always_inline)) {
    int tile;
    unit_tile(a, tiles, u, tile, nt);
    ntr = WN ? 2 * nt + wm : nt;
    const int3 te = tile_entry(tiles + kTileInts * tile);
    e = te.x; rb = te.y; re = te.z;
    {
      const int v = re - rb - arow;
      ntg = v <= 0 ? 0 : v >= 64 ? 4 : (v + 15) >> 4;
    }
    // through the scalar cache, 16 rows at a time (a group past nout is
    // never stored and not loaded)
    const uint16_t* bias_e = a.bias + (size_t)e * a.R;
#pragma unroll
    for (int jp = 0; jp < kRG; jp += 2) {
      // groups jp and jp + 1 (16 rows each); a group past nout reads group jp's
      // rows again and is zeroed (never stored)
      int n0[2], off[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = jp + h;
        n0[h] = GATEUP ? ntr * (kBN / 2) + 32 * wn + 16 * (j >> 1) : ntr * kBN + 64 * wn + 16 * j;
        off[h] = (GATEUP && (j & 1) ? a.nout : 0) + n0[h];
      }
      if (a.bias && n0[0] < a.nout) {
        v8i_t v0, v1;
        sload_bias2(bias_e + off[0], bias_e + (n0[1] < a.nout ? off[1] : off[0]), v0, v1);
        bq[jp] = bias_quad(v0, g);
        bq[jp + 1] = n0[1] < a.nout ? bias_quad(v1, g) : make_uint2(0u, 0u);
      } else {
        bq[jp] = bq[jp + 1] = make_uint2(0u, 0u);
      }
    }
  };

  comp_setup(u0);
  const int pro = total < C::kStages - 1 ? total : C::kStages - 1;
  if (copies)
    for (int p = 0; p < pro; ++p) {
      cp.issue(a);
      if (CW) cp2.issue(a);
    }

  v4f acc[kRG][4];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = {0.f, 0.f, 0.f, 0.f};
  float amax = 0.0f;     // gate_up: max |h| of the lane's outputs

  // one K step; NTG: the wave's 16-row groups that hold rows of the tile,
  // fixed per unit (-1: taken from ntg at run time).  The expanding kernels
  // run a separate step loop for each value, so that the step holds no
  // branch on it: the compiler then keeps the accumulators in place (a
  // merge of full and partial paths inside the step cost 24-72 register
  // copies per step)
  // TAIL: the unit's last K step, the only one whose blocks can lie past K
  // (the other steps take no masking of weights and scales)
  auto step = [&](const int t, auto ntg_c, auto tail_c) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tail_c)::value;
    constexpr int NTG = decltype(ntg_c)::value;
    const int nrg = NTG < 0 ? ntg : NTG;
    // this wave's copies of step t have landed (steps issued beyond t:
    // min(STAGES - 2, total - 1 - t)); after the barrier everybody's have,
    // and everybody is done reading step t-1's slot
    // (copy waves: two shares per step; the other waves have none to wait for)
    constexpr int kD = CW ? 2 * C::kDma : C::kDma;
    int ahead = total - 1 - t;
    ahead = ahead < C::kStages - 2 ? ahead : C::kStages - 2;
    if (A4) {
      constexpr int kA = C::kActDma + C::kWDma;   // + one scale copy in waves 0-2
      static_assert(!A4 || C::kStages == 3, "one step ahead");
      if (wave < 3) {
        if (ahead >= 1) wait_vm<kA + 1>(); else wait_vm<0>();
      } else {
        if (ahead >= 1) wait_vm<kA>(); else wait_vm<0>();
      }
    } else if (!copies) {
    } else if (ahead >= 4) wait_vm<4 * kD>();
    else if (ahead == 3) wait_vm<3 * kD>();
    else if (ahead == 2) wait_vm<2 * kD>();
    else if (ahead == 1) wait_vm<kD>();
    else wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // refill the slot freed by the barrier.  A4: the activation and scale
    // copies here, the weight copies (16 rows, 8 lines per instruction)
    // halfway through the step's MFMAs, so the matrix core works while this
    // wave issues them (measured 4-5% faster than all copies here; weights
    // first was 15% slower).  The FP8 steps were not faster with any split.
    const bool refill = t + C::kStages - 1 < total;
    if (refill && copies) {
      if (A4) {
        cp.issue_act(a);
      } else {
        cp.issue(a);
        if (CW) cp2.issue(a);
      }
    }
    // step t's operands
    const uint32_t so = (uint32_t)(cslot * C::kSlot);
    const uint32_t aa0 = a0 + so, aa1 = a1 + so, ww = w0 + so, ss = s0 + so;
    v4u_t xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3, wq0, wq1, wq2, wq3;
    uint32_t sb0, sb1, sb2, sb3;
    if constexpr (A4) {
      // two halves of four MX blocks: the reads of half 1 overlap the MFMAs
      // of half 0; lane group g holds MX block 4h + g of the step in both
      // operands; past K the weights are zero and both scales 2^0
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t ab0, ab1, ab2, ab3;
        lds_half_reads_a4(GATEUP, ax[h] + so, wx[h] + so, ss + 1024 * h, as0 + so + 512 * h, xa0, xa1, xa2, xa3,
                          wq0, wq1, wq2, wq3, sb0, sb1, sb2, sb3, ab0, ab1, ab2, ab3);
        const v4u_t xa[4] = {xa0, xa1, xa2, xa3};
        const v4u_t wq[4] = {wq0, wq1, wq2, wq3};
        const uint32_t sb[4] = {sb0, sb1, sb2, sb3};
        const uint32_t ab[4] = {ab0, ab1, ab2, ab3};
        const bool valid = !TAIL || 8 * cstep + 4 * h + g < a.nb;
        v8i B[4];
        int bsc[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          B[tg] = v8i{(int)xa[tg].x, (int)xa[tg].y, (int)xa[tg].z, (int)xa[tg].w, 0, 0, 0, 0};
          bsc[tg] = valid ? (int)ab[tg] : 127;
        }
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) {
          const v4u_t wz = valid ? wq[rg] : v4u_t{0u, 0u, 0u, 0u};
          const v8i A = v8i{(int)wz.x, (int)wz.y, (int)wz.z, (int)wz.w, 0, 0, 0, 0};
          const int asc = valid ? (int)sb[rg] : 127;
#pragma unroll
          for (int tg = 0; tg < 4; ++tg)
            acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[tg], acc[rg][tg], 4, 4, 0, asc, 0,
                                                                           bsc[tg]);
        }
        if (h == 0) {
          __builtin_amdgcn_sched_barrier(0);
          if (refill) {
            cp.issue_w(a);
            cp.advance(a);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (nrg > 0) {
      // (a wave whose rows all lie past the tile neither reads nor computes:
      // at ~64 rows per expert that is half the waves of a 128-row tile)
      // all 16 reads and their wait in one assembly block: no register of a
      // read in flight is ever visible to compiler-generated code (variants
      // that waited for the reads in two or four phases were no faster)
      lds_step_reads<GATEUP, NV>(aa0, aa1, ww, ss, xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3, wq0, wq1, wq2, wq3, sb0,
                                 sb1, sb2, sb3);
      const v4u_t xa[4] = {xa0, xa1, xa2, xa3};
      v4u_t wq[4] = {wq0, wq1, wq2, wq3};
      if (EXP && (g & 1)) {
        // odd lane groups hold activation K 16..31 of the block in xa: take
        // the weight dwords in the same order
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) wq[rg] = v4u_t{wq[rg].z, wq[rg].w, wq[rg].x, wq[rg].y};
      }
      const uint32_t sb[4] = {sb0, sb1, sb2, sb3};
      const bool valid = !TAIL || 4 * cstep + g < a.nb;   // this lane's MX block lies inside K
      // weights of chunk q (elements 8q..8q+7 of the lane's block, 8(q^2).. for
      // odd g) of weight group rg, exactly: MXFP4 as bf16 through the scaled
      // conversion with the block's E8M0 scale; NVFP4 as f16, times the E4M3
      // scale of the chunk's 16-element block (the low byte of sb holds block
      // 2g).  The NVFP4 kernels run the f16 MFMA on f16 operands (E4M3 codes
      // are f16 values too), the MXFP4 gate_up the bf16 one.
      auto expand_w = [&](int rg, int q) __attribute__((always_inline)) {
        if constexpr (NV) {
          const uint32_t sub = (uint32_t)((q >> 1) ^ (g & 1));
          const v2f fs = e4m3x2_to_f32(sb[rg]);
          const float f = valid ? (sub ? fs[1] : fs[0]) : 0.0f;
          return fp4x8_times_f16(wq[rg][q], nv_scale(f));
        } else {
          const float f = valid ? e8m0_to_f32(sb[rg]) : 0.0f;
          return fp4x8_to_bf16(wq[rg][q], f);
        }
      };
      using XT = std::conditional_t<NV, v8h, v8bf>;
      auto expand_x = [&](uint32_t lo, uint32_t hi) __attribute__((always_inline)) {
        if constexpr (NV) return fp8x8_to_f16(lo, hi);
        else return fp8x8_to_bf16(lo, hi);
      };
      if (EXP) {
        // lane group g holds K [32g, 32g+32) of the step (its own MX block);
        // MFMA q takes elements 8q..8q+7 of it (8(q^2).. for odd g), in the
        // same order for both operands; MFMAs 2-3 take the second chunks
        if (nrg == 4) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4u_t xb[4] = {xb0, xb1, xb2, xb3};
            XT B[4];
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
              const v4u_t c = q < 2 ? xa[tg] : xb[tg];
              B[tg] = (q & 1) ? expand_x(c.z, c.w) : expand_x(c.x, c.y);
            }
#pragma unroll
            for (int rg = 0; rg < kRG; ++rg) {
              const XT A = expand_w(rg, q);
#pragma unroll
              for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = mfma16x16x32(A, B[tg], acc[rg][tg]);
            }
          }
        } else {
          // part of the wave's rows lie past the tile: only the groups that
          // hold rows of it (none: no expansion either)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4u_t xb[4] = {xb0, xb1, xb2, xb3};
            XT A[4];
#pragma unroll
            for (int rg = 0; rg < kRG; ++rg) A[rg] = expand_w(rg, q);
#pragma unroll
            for (int tg = 0; tg < 3; ++tg) {
              if (tg >= nrg) break;
              const v4u_t c = q < 2 ? xa[tg] : xb[tg];
              const XT B = (q & 1) ? expand_x(c.z, c.w) : expand_x(c.x, c.y);
#pragma unroll
              for (int rg = 0; rg < kRG; ++rg) acc[rg][tg] = mfma16x16x32(A[rg], B, acc[rg][tg]);
            }
          }
        }
      } else {
        const v4u_t xb[4] = {xb0, xb1, xb2, xb3};
        v8i A[4];
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) {
          const v4u_t wz = valid ? wq[rg] : v4u_t{0u, 0u, 0u, 0u};
          A[rg] = v8i{(int)wz.x, (int)wz.y, (int)wz.z, (int)wz.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          if (tg >= nrg) break;   // rows past the tile (never stored)
          const v8i B = __builtin_bit_cast(v8i, __builtin_shufflevector(xa[tg], xb[tg], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rg = 0; rg < kRG; ++rg)
            acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rg], B, acc[rg][tg], 4, 0, 0,
                                                                           (int)sb[rg], 0, 127);
        }
      }
    }
    cslot = cslot + 1 == C::kStages ? 0 : cslot + 1;
    ++cstep;
  };

  for (int t = 0; t < total;) {
    // the unit's steps
    const int t_end = t + a.nsteps;
    if constexpr (EXP && !A4) {
      switch (ntg) {
        case 0: for (; t < t_end; ++t) step(t, std::integral_constant<int, 0>{}, std::true_type{}); break;
        case 1: for (; t < t_end; ++t) step(t, std::integral_constant<int, 1>{}, std::true_type{}); break;
        case 2: for (; t < t_end; ++t) step(t, std::integral_constant<int, 2>{}, std::true_type{}); break;
        case 3: for (; t < t_end; ++t) step(t, std::integral_constant<int, 3>{}, std::true_type{}); break;
        default: for (; t < t_end; ++t) step(t, std::integral_constant<int, 4>{}, std::true_type{}); break;
      }
    } else {
      // the steps before the last without the K-tail masking
      for (; t < t_end - 1; ++t) step(t, std::integral_constant<int, -1>{}, std::false_type{});
      step(t, std::integral_constant<int, -1>{}, std::true_type{});
      ++t;
    }

    // ---- epilogue of the unit: the lane holds rows 4g + jj of each 16-row
    // weight group and sorted row r of each 16-row token group
    if constexpr (GATEUP && A4) {
      // the wave's 32 h columns [ib, ib + 32) are MX block b of each token
      // row: lane (r, g) holds columns 4g..4g+3 (half 0) and 16+4g..16+4g+3
      // (half 1).  The block is quantised here (the rule of
      // quant_x_mxfp4_sorted_kernel): amax over the row's four lanes, shared
      // exponent, codes; no fp32 h is written.  Every lane takes part in the
      // shuffles; only real rows store.  SwiGLU uses the hardware exp and
      // reciprocal (a few 1e-7 relative, far inside the h error the codes
      // are specified against), not the correctly rounded ones of the FP8
      // path.
      const int ib = nt * (kBN / 2) + 32 * wn;
      if (ib < a.nout) {
        const int b = ib / kBlockElems, nbh = a.nout / kBlockElems;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const int row = rb + arow + 16 * tg + r;
          float hv[8];
          uint32_t am = 0;
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const float gate = acc[half][tg][jj] + bf16_of(bq[2 * half], jj);
              const float up = acc[half + 2][tg][jj] + bf16_of(bq[2 * half + 1], jj);
              hv[4 * half + jj] = silu_rcp(gate) * up;
              am = max(am, __float_as_uint(hv[4 * half + jj]) & 0x7fffffffu);
            }
          am = max(am, (uint32_t)__shfl_xor((int)am, 16, 64));
          am = max(am, (uint32_t)__shfl_xor((int)am, 32, 64));
          const int x = min(max((int)(am >> 23) - 127 - 2, kMxExpMin), kMxExpMax);
          const float inv = __uint_as_float((uint32_t)(127 - x) << 23);
          // codes of h * 2^-X (|.| < 8): the hardware conversion rounds exactly
          // as e2m1_round_mag with the sign bit kept (checked on every fp32
          // below 8 in magnitude); value 2i in the low nibble of byte i
          uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, hv[0] * inv, hv[1] * inv, 1.0f, 0);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[2] * inv, hv[3] * inv, 1.0f, 1);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[4] * inv, hv[5] * inv, 1.0f, 2);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[6] * inv, hv[7] * inv, 1.0f, 3);
          // nibbles of columns 4g.. (half 0) and 16+4g.. (half 1)
          const uint32_t q[2] = {w & 0xffffu, w >> 16};
          if (row < re) {
            uint8_t* hb = a.h_codes + (int64_t)row * code_row_bytes(a.nout, true) + b * kBlockBytes;
            *reinterpret_cast<uint16_t*>(hb + 2 * g) = (uint16_t)q[0];
            *reinterpret_cast<uint16_t*>(hb + 8 + 2 * g) = (uint16_t)q[1];
            if (g == 0) {
              a.h_scales[((int64_t)(b >> 2) * a.h_rows + row) * 4 + (b & 3)] = (uint8_t)(x + 127);
              if (b == nbh - 1)   // the pad bytes of the row's last step
                for (int p = nbh; p < 4 * ((nbh + 3) / 4); ++p)
                  a.h_scales[((int64_t)(p >> 2) * a.h_rows + row) * 4 + (p & 3)] = 127;
            }
          }
        }
      }
    } else if constexpr (GATEUP) {
      // halves 0, 1 take gate groups 0, 1 and up groups 2, 3
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int i0 = ntr * (kBN / 2) + 32 * wn + 16 * half;
        if (i0 >= a.nout) continue;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const int row = rb + arow + 16 * tg + r;
          if (row >= re) continue;
          float hv[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float gate = acc[half][tg][jj] * sx + bf16_of(bq[2 * half], jj);
            const float up = acc[half + 2][tg][jj] * sx + bf16_of(bq[2 * half + 1], jj);
            hv[jj] = silu_rcp(gate) * up;
            amax = fmaxf(amax, fabsf(hv[jj]));
          }
          *reinterpret_cast<float4*>(a.out + (size_t)row * a.nout + i0 + 4 * g) =
              make_float4(hv[0], hv[1], hv[2], hv[3]);
        }
      }
    } else {
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
        const int n0 = ntr * kBN + 64 * wn + 16 * rg;
        if (n0 >= a.nout) continue;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const int row = rb + arow + 16 * tg + r;
          if (row >= re) continue;
          float v[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[jj] = acc[rg][tg][jj] * sx + bf16_of(bq[rg], jj);
          if (a.out_bf16) {
            *reinterpret_cast<uint2*>(a.out_bf16 + (size_t)row * a.nout + n0 + 4 * g) =
                make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                           f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
          } else {
            *reinterpret_cast<float4*>(a.out + (size_t)row * a.nout + n0 + 4 * g) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = {0.f, 0.f, 0.f, 0.f};
    cstep = 0;
    if (++ck < my_units) comp_setup(u0 + ck * G);
  }
  if (GATEUP && !A4) {
    // max |h| over all of this wave's units: one atomic per wave
    amax = wave_max(amax);
    if (lane == 0) atomicMax(reinterpret_cast<uint32_t*>(&status[kStAmaxH]), __float_as_uint(amax));
  }
}

template <bool GATEUP, int BM, bool A4 = false, bool NV = false, bool WN = false>
__global__ __launch_bounds__((Ring<BM, A4, NV, WN>::kThreads)) void prefill_gemm_kernel(PrefillArgs a,
                                                                                  const int* __restrict__ tiles,
                                                                                  int* status) {
  prefill_gemm_body<GATEUP, BM, A4, NV, WN, false>(a, tiles, status);
}

// gate_up on E4M3 activations with MXFP4 weights, copy waves
__global__ __launch_bounds__((Ring<kPrefillBM>::kThreads)) void prefill_gemm_cw_kernel(PrefillArgs a,
                                                                                 const int* __restrict__ tiles,
                                                                                 int* status) {
  prefill_gemm_body<true, kPrefillBM, false, false, false, true>(a, tiles, status);
}

// The E2M1 codes of one weight tensor in the order the E4M3-activation copies
// take them (launch_code_stream): for expert e, n-tile nt and 128-element
// step s, 16 KB holding, for LDS row lr = 0..255, 64 bytes whose 16-byte slot
// j is block 4s + (j ^ ((lr / 2) % 4)) of weight row weight_row(lr), zeros
// past K.  One thread per 16 bytes, stores contiguous.
template <bool GATEUP>
__global__ __launch_bounds__(256) void code_stream_kernel(const uint8_t* __restrict__ wb, int R, int nout, int nb,
                                                          int NT, int nsteps, int64_t n16, uint8_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n16) return;
  const int within = (int)(q & 1023);                  // 16-byte piece of the chunk
  const int64_t c = q >> 10;                           // chunk (e, nt, s)
  const int st = (int)(c % nsteps);
  const int64_t u = c / nsteps;
  const int nt = (int)(u % NT), e = (int)(u / NT);
  const int lr = within >> 2, j = within & 3;
  const int b = 4 * st + (j ^ ((lr >> 1) & 3));
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (b < nb)
    v = *reinterpret_cast<const uint4*>(wb + (((int64_t)e * R + weight_row<GATEUP>(lr, nt, nout)) * nb + b) *
                                                 kBlockBytes);
  reinterpret_cast<uint4*>(out)[q] = v;
}

hipError_t launch_code_stream(const uint8_t* wb, int E, int R, int nout, int K, bool gateup, uint8_t* out,
                              hipStream_t s) {
  const int nb = K / kBlockElems, nsteps = (nb + 3) / 4;
  const int NT = gateup ? (nout + kBN / 2 - 1) / (kBN / 2) : (nout + kBN - 1) / kBN;
  const int64_t n16 = (int64_t)E * NT * nsteps * (kCodeChunk / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  if (gateup) code_stream_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(wb, R, nout, nb, NT, nsteps, n16, out);
  else code_stream_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(wb, R, nout, nb, NT, nsteps, n16, out);
  return hipGetLastError();
}

// The weight scales of every unit in the order the copies take them: for
// expert e, n-tile nt and K step s, 1 KB holding, for each of the unit's 256
// LDS rows lr, the scale bytes of MX blocks 4s .. 4s+3 of weight row
// weight_row(lr) (127, i.e. 2^0, past K, and for LDS rows past the last
// weight row, whose outputs are never stored).  A block takes CPB chunks of
// 32 LDS rows of one unit: the chunk's rows are read into LDS, then written
// out step by step.
__device__ __forceinline__ int lds_row_index(bool gateup, int lr, int nt) {
  return gateup ? nt * (kBN / 2) + (lr & (kBN / 2 - 1)) : nt * kBN + lr;   // before clamping
}

template <bool GATEUP>
__global__ __launch_bounds__(256) void scale_stream_kernel(const uint8_t* __restrict__ ws, int R, int nout, int nb,
                                                           int NT, int nsteps, int cpb, uint32_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t rows[];   // 32 * cpb x nb bytes, row-major
  const int per_unit = 8 / cpb;
  const int unit = blockIdx.x / per_unit;     // e * NT + nt
  const int c0 = (blockIdx.x - unit * per_unit) * cpb;
  const int e = unit / NT, nt = unit - e * NT;
  const int t = threadIdx.x;
  const int chunk_dw = 8 * nb;                // dwords of 32 rows
  if (cpb == 8 && chunk_dw <= 768) {
    // chunk c holds LDS rows 32c .. 32c+31, i.e. weight rows row0 .. row0+31
    // of which the first nv are real (row index below nout); those are
    // nv * nb contiguous bytes at an offset that is a multiple of 32 from the
    // 4-byte aligned scales.  A thread loads dwords t, t + 256, t + 512 of
    // it, an index past the real bytes taking the chunk's last dword that
    // holds real bytes (inside the tensor: its size is a multiple of 4).
    // The loads are straight-line code, all issued before the first store to
    // LDS (loads under branches get a full wait at each branch).
    uint32_t v[8][3];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int i0 = lds_row_index(GATEUP, 32 * c, nt);
      const int half = GATEUP && c >= 4 ? nout : 0;   // first weight row of the chunk's half
      // a chunk with no real rows reads its half's first row (32-aligned,
      // unused: written as 127)
      const int row0 = half + (i0 < nout ? i0 : 0);
      const int nv = max(1, min(32, nout - i0));
      const int last = (nv * nb - 1) >> 2;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(ws + ((int64_t)e * R + row0) * nb);
#pragma unroll
      for (int q = 0; q < 3; ++q) v[c][q] = src[min(t + 256 * q, last)];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (t + 256 * q < chunk_dw) reinterpret_cast<uint32_t*>(rows)[c * chunk_dw + t + 256 * q] = v[c][q];
    }
  } else {
    // K > 3072: one byte per thread and step, rows clamped as the GEMM does
    for (int i = t; i < 32 * cpb * nb; i += blockDim.x) {
      const int l = i / nb, b = i - l * nb;
      rows[i] = ws[((int64_t)e * R + weight_row<GATEUP>(32 * c0 + l, nt, nout)) * nb + b];
    }
  }
  __syncthreads();
  // thread l writes LDS row l's word of every step (consecutive threads,
  // consecutive words)
  const int l = t;
  if (l < 32 * cpb) {
    const bool real = lds_row_index(GATEUP, 32 * c0 + l, nt) < nout;
    const uint8_t* src = rows + l * nb;
    uint32_t* dst = out + (int64_t)unit * nsteps * 256 + 32 * c0 + l;
    int st = 0;
    if (!real) {
      for (; st < nsteps; ++st) dst[st * 256] = 0x7f7f7f7fu;
    } else if ((nb & 1) == 0) {
      // even nb: a step's four bytes start 2-byte aligned, two halfword reads
      const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
      for (; st < nb / 4; ++st) dst[st * 256] = (uint32_t)s16[2 * st] | ((uint32_t)s16[2 * st + 1] << 16);
    }
    for (; st < nsteps; ++st) {   // the tail step (past K: 127), or odd nb
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = 4 * st + j;
        word |= (uint32_t)(b < nb ? src[b] : 127u) << (8 * j);
      }
      dst[st * 256] = word;
    }
  }
}

// NVFP4 weights: per (expert, n-tile, 128-element K step) 2 KB holding the 8
// E4M3 scale bytes (16-element blocks 8 step .. 8 step + 7) of each of the
// unit's 256 LDS rows in row order; blocks past K are 0.  One thread per
// (unit, LDS row) walks the row's scale bytes in order (dword loads when the
// row's K/16 bytes keep them aligned, else 16-bit ones) and writes each step's
// 8 bytes, the 256 threads of a block writing 2 KB contiguously per step.
template <bool GATEUP>
__global__ __launch_bounds__(256) void scale_stream_nv_kernel(const uint8_t* __restrict__ ws, int R, int nout,
                                                              int nb16, int NT, int nsteps, int64_t n,
                                                              uint2* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int lr = (int)(i & (kBN - 1));
  const int64_t unit = i >> 8;                // e * NT + nt
  const int e = (int)(unit / NT), nt = (int)(unit - (int64_t)e * NT);
  const uint8_t* src = ws + ((int64_t)e * R + weight_row<GATEUP>(lr, nt, nout)) * nb16;
  uint2* dst = out + unit * nsteps * kBN + lr;
  const bool dw = (nb16 & 3) == 0;            // rows start 4-byte aligned
  for (int step = 0; step < nsteps; ++step) {
    const int b0 = 8 * step;
    uint32_t lo, hi;
    if (b0 + 8 <= nb16) {
      if (dw) {
        lo = *reinterpret_cast<const uint32_t*>(src + b0);
        hi = *reinterpret_cast<const uint32_t*>(src + b0 + 4);
      } else {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(src + b0);
        lo = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        hi = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
      }
    } else {                                  // the step past K: its real blocks, then 0
      lo = hi = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint32_t v = b0 + b < nb16 ? src[b0 + b] : 0u;
        if (b < 4) lo |= v << (8 * b);
        else hi |= v << (8 * (b - 4));
      }
    }
    dst[(int64_t)step * kBN] = make_uint2(lo, hi);
  }
}

// The same stream, one block per (expert, n-tile) with the unit's rows staged
// in LDS (K <= 3072: 256 rows x K/16 bytes <= 48 KB): the rows of a half
// (gate_up: 128 gate rows, 128 up rows; down: 256 rows) are contiguous in
// the tensor, so they are loaded with consecutive 16-bit or 32-bit loads;
// LDS rows past the matrix are zero (never stored).  Then every step's 2 KB
// is written by the block's 256 threads, one LDS row each.
constexpr int kNvStageMaxNb16 = 192;   // 48 KB of LDS: K <= 3072
template <bool GATEUP>
__global__ __launch_bounds__(256) void scale_stream_nv_lds_kernel(const uint8_t* __restrict__ ws, int R, int nout,
                                                                  int nb16, int NT, int nsteps,
                                                                  uint2* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t rows[];   // 256 x nb16 bytes
  const int unit = blockIdx.x, e = unit / NT, nt = unit - e * NT;
  const int t = threadIdx.x;
  constexpr int kHalves = GATEUP ? 2 : 1, kHalfRows = kBN / kHalves;
#pragma unroll
  for (int h = 0; h < kHalves; ++h) {
    const int first = nt * kHalfRows;                                  // first row of the half's block
    const int nv = max(0, min(kHalfRows, nout - first));               // rows inside the matrix
    const uint8_t* src = ws + ((int64_t)e * R + (h ? nout : 0) + first) * nb16;
    uint8_t* dst = rows + h * kHalfRows * nb16;
    const int bytes = nv * nb16, all = kHalfRows * nb16;
    // batches of 12 loads per thread issued before their LDS stores
    constexpr int kB = 12;
    if ((bytes & 3) == 0) {     // whole dwords (the block start is 4-byte aligned: nb16 is even)
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
      uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
      const int nd = all / 4;
      for (int d0 = t; d0 < nd; d0 += 256 * kB) {
        uint32_t v[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int d = d0 + 256 * j;
          v[j] = d < nd && 4 * d < bytes ? s32[d] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kB; ++j)
          if (d0 + 256 * j < nd) d32[d0 + 256 * j] = v[j];
      }
    } else {
      const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
      uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
      const int nd = all / 2;
      for (int d0 = t; d0 < nd; d0 += 256 * kB) {
        uint16_t v[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int d = d0 + 256 * j;
          v[j] = d < nd && 2 * d < bytes ? s16[d] : (uint16_t)0;
        }
#pragma unroll
        for (int j = 0; j < kB; ++j)
          if (d0 + 256 * j < nd) d16[d0 + 256 * j] = v[j];
      }
    }
  }
  __syncthreads();
  const uint8_t* row = rows + t * nb16;
  uint2* dst = out + (int64_t)unit * nsteps * kBN + t;
  for (int step = 0; step < nsteps; ++step) {
    const int b0 = 8 * step;
    uint32_t lo = 0, hi = 0;
    if (b0 + 8 <= nb16 && (nb16 & 3) == 0) {
      lo = *reinterpret_cast<const uint32_t*>(row + b0);
      hi = *reinterpret_cast<const uint32_t*>(row + b0 + 4);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint32_t v = b0 + b < nb16 ? row[b0 + b] : 0u;
        if (b < 4) lo |= v << (8 * b);
        else hi |= v << (8 * (b - 4));
      }
    }
    dst[(int64_t)step * kBN] = make_uint2(lo, hi);
  }
}

hipError_t launch_scale_stream(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws, bool gateup,
                               hipStream_t s) {
  if (w.nvfp4) {
    const int R = gateup ? 2 * sh.I : sh.H, nout = gateup ? sh.I : sh.H;
    const int K = gateup ? sh.H : sh.I;
    const int NT = gateup ? (sh.I + kBN / 2 - 1) / (kBN / 2) : (sh.H + kBN - 1) / kBN;
    const int nsteps = (K / kBlockElems + 3) / 4;
    uint2* out = reinterpret_cast<uint2*>(gateup ? ws.w13_stream : ws.w2_stream);
    const int nb16 = K / 16;
    if (sh.E * NT <= 0) return hipSuccess;
    if (nb16 <= kNvStageMaxNb16) {
      const size_t lds = (size_t)kBN * nb16;
      if (gateup)
        scale_stream_nv_lds_kernel<true><<<sh.E * NT, 256, lds, s>>>(w.w13_scales, R, nout, nb16, NT, nsteps, out);
      else
        scale_stream_nv_lds_kernel<false><<<sh.E * NT, 256, lds, s>>>(w.w2_scales, R, nout, nb16, NT, nsteps, out);
      return hipGetLastError();
    }
    const int64_t n = (int64_t)sh.E * NT * kBN;   // one thread per (unit, LDS row)
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (gateup)
      scale_stream_nv_kernel<true><<<grid, 256, 0, s>>>(w.w13_scales, R, nout, K / 16, NT, nsteps, n, out);
    else
      scale_stream_nv_kernel<false><<<grid, 256, 0, s>>>(w.w2_scales, R, nout, K / 16, NT, nsteps, n, out);
    return hipGetLastError();
  }
  const int R = gateup ? 2 * sh.I : sh.H, nout = gateup ? sh.I : sh.H;
  const int K = gateup ? sh.H : sh.I, nb = K / kBlockElems;
  const int NT = gateup ? (sh.I + kBN / 2 - 1) / (kBN / 2) : (sh.H + kBN - 1) / kBN;
  const int nsteps = (nb + 3) / 4;
  // chunks of 32 rows per block: a whole unit while its rows fit in 48 KB
  int cpb = 8;
  while (cpb > 1 && (size_t)32 * cpb * nb > 48 * 1024) cpb /= 2;
  const unsigned grid = (unsigned)(sh.E * NT * (8 / cpb));
  const size_t lds = (size_t)32 * cpb * nb;
  if (gateup)
    scale_stream_kernel<true><<<grid, 256, lds, s>>>(w.w13_scales, R, nout, nb, NT, nsteps, cpb,
                                                     reinterpret_cast<uint32_t*>(ws.w13_stream));
  else
    scale_stream_kernel<false><<<grid, 256, lds, s>>>(w.w2_scales, R, nout, nb, NT, nsteps, cpb,
                                                      reinterpret_cast<uint32_t*>(ws.w2_stream));
  return hipGetLastError();
}

template <bool GATEUP, int BM, bool NV, bool A4 = false, bool WN = false>
static hipError_t launch_prefill_bm(const PrefillArgs& args, const MoeShape& sh, const WsPtrs& ws, hipStream_t s,
                                    bool cw = false) {
  // one block per compute unit: the LDS ring takes most of a unit's LDS
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  PrefillArgs a = args;
  if (WN) a.NT = (args.NT + 1) / 2;   // units of two n-tiles
  // the expert-major XCD schedule needs the tile words (bounded list) and
  // a grid of whole XCDs
  a.sched_xcd = cus % 8 == 0 && max_tiles((int64_t)sh.T * sh.k, sh.E, BM) <= kTileWordMaxBound;
  if (GATEUP && BM == kPrefillBM && !A4 && !NV && !WN && cw)
    prefill_gemm_cw_kernel<<<cus, Ring<BM, A4, NV, WN>::kThreads, 0, s>>>(a, ws.tiles, ws.status);
  else
    prefill_gemm_kernel<GATEUP, BM, A4, NV, WN><<<cus, Ring<BM, A4, NV, WN>::kThreads, 0, s>>>(a, ws.tiles,
                                                                                         ws.status);
  return hipGetLastError();
}

// The tile height follows prefill_bm, the rule the tile list was built with.
template <bool GATEUP, bool A4 = false, bool NV = false>
static hipError_t launch_prefill(const PrefillArgs& args, const MoeShape& sh, const WsPtrs& ws, hipStream_t s) {
  if constexpr (NV) {
    if (prefill_bm((int64_t)sh.T * sh.k, sh.E, true) == kPrefillNarrowBM)
      return launch_prefill_bm<GATEUP, kPrefillNarrowBM, NV, false, true>(args, sh, ws, s);
  }
  // MXFP4 gate_up on E4M3 activations: copy waves while the experts average
  // at most 64 rows (same-box A/B at 2048 tokens: gate_up 374 -> 357 us)
  const bool cw = GATEUP && !NV && !A4 && (int64_t)sh.T * sh.k <= (int64_t)kPrefillNarrowBM * sh.E;
  return launch_prefill_bm<GATEUP, kPrefillBM, NV, A4>(args, sh, ws, s, cw);
}

hipError_t launch_moe_gateup_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                 int64_t /*ntile_bound*/, hipStream_t s) {
  PrefillArgs a{};
  a.wb = w.w13_blocks;
  a.wcs = w.w13_codes;
  a.wsp = ws.w13_stream;
  a.bias = w.w13_bias;
  a.R = 2 * sh.I;
  a.nout = sh.I;
  a.nb = sh.H / kBlockElems;
  a.K = sh.H;
  a.NT = a.NTs = (sh.I + kBN / 2 - 1) / (kBN / 2);
  a.nsteps = (a.nb + 3) / 4;
  a.nsteps_s = a.nsteps;
  a.act = ws.x_codes;
  a.act_ld = (int)code_row_bytes(sh.H, false);
  a.scale_word = kStScaleX;
  a.out = static_cast<float*>(ws.h);
  if (w.nvfp4) {
    a.gscale = w.w13_global;
    return launch_prefill<true, false, true>(a, sh, ws, s);
  }
  return launch_prefill<true>(a, sh, ws, s);
}

hipError_t launch_moe_down_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                               int64_t /*ntile_bound*/, hipStream_t s, uint16_t* out_bf16) {
  PrefillArgs a{};
  a.wb = w.w2_blocks;
  a.wcs = w.w2_codes;
  a.wsp = ws.w2_stream;
  a.bias = w.w2_bias;
  a.R = sh.H;
  a.nout = sh.H;
  a.nb = sh.I / kBlockElems;
  a.K = sh.I;
  a.NT = a.NTs = (sh.H + kBN - 1) / kBN;
  a.nsteps = (a.nb + 3) / 4;
  a.nsteps_s = a.nsteps;
  a.act = ws.h_codes;
  a.act_ld = (int)code_row_bytes(sh.I, false);
  a.scale_word = kStScaleH;
  a.out = ws.y;
  a.out_bf16 = out_bf16;
  if (w.nvfp4) {
    a.gscale = w.w2_global;
    return launch_prefill<false, false, true>(a, sh, ws, s);
  }
  return launch_prefill<false>(a, sh, ws, s);
}

hipError_t launch_moe_gateup_fp4(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws, hipStream_t s) {
  PrefillArgs a{};
  a.wb = w.w13_blocks;
  a.wcs = w.w13_codes;
  a.wsp = ws.w13_stream;
  a.bias = w.w13_bias;
  a.R = 2 * sh.I;
  a.nout = sh.I;
  a.nb = sh.H / kBlockElems;
  a.K = sh.H;
  a.NT = a.NTs = (sh.I + kBN / 2 - 1) / (kBN / 2);
  a.nsteps = (a.nb + 7) / 8;        // K steps of 256
  a.nsteps_s = (a.nb + 3) / 4;
  a.act = ws.x_codes;
  a.act_ld = (int)code_row_bytes(sh.H, true);
  a.asc = ws.x_scales;
  a.asc_step = (int64_t)4 * sh.T * sh.k;
  a.scale_word = -1;
  a.out = nullptr;
  a.h_codes = ws.h_codes;
  a.h_scales = ws.h_scales;
  a.h_rows = (int64_t)sh.T * sh.k;
  return launch_prefill<true, true>(a, sh, ws, s);
}

hipError_t launch_moe_down_fp4(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws, hipStream_t s,
                               uint16_t* out_bf16) {
  PrefillArgs a{};
  a.wb = w.w2_blocks;
  a.wcs = w.w2_codes;
  a.wsp = ws.w2_stream;
  a.bias = w.w2_bias;
  a.R = sh.H;
  a.nout = sh.H;
  a.nb = sh.I / kBlockElems;
  a.K = sh.I;
  a.NT = a.NTs = (sh.H + kBN - 1) / kBN;
  a.nsteps = (a.nb + 7) / 8;        // K steps of 256
  a.nsteps_s = (a.nb + 3) / 4;
  a.act = ws.h_codes;
  a.act_ld = (int)code_row_bytes(sh.I, true);
  a.asc = ws.h_scales;
  a.asc_step = (int64_t)4 * sh.T * sh.k;
  a.scale_word = -1;
  a.out = ws.y;
  a.out_bf16 = out_bf16;
  return launch_prefill<false, true>(a, sh, ws, s);
}

}  // namespace mx
