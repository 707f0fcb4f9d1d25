// Host-side launch wrappers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

constexpr int kFusedPermuteMaxPairs = 4096;  // single-block permutation up to here
constexpr int kFusedRouteMaxTokens = 32;     // single-block route + permute up to here
constexpr int kDecodeBM = 4;                 // sorted rows per tile, bf16 path
constexpr int kPrefillBM = 128;              // sorted rows per tile, FP8 and FP4 x FP4 paths
constexpr int kPrefillNarrowBM = 64;         // NVFP4 weights when experts average <= 64 rows
// Row-tile height of the prefill GEMMs for npairs routed rows over E experts:
// with NVFP4 weights (E4M3 activations), while the experts average at most
// 64 rows, units of 64 rows x two n-tiles (all eight waves busy: in 128-row
// tiles the lower half's waves would hold no rows), else 128-row tiles.
// With MXFP4 weights the 64-row units were no faster for gate_up and slower
// for down (2048-token FP8 layer 720 -> 761 us, same-box A/B).
inline int prefill_bm(int64_t npairs, int64_t E, bool nv) {
  return nv && npairs <= (int64_t)kPrefillNarrowBM * E ? kPrefillNarrowBM : kPrefillBM;
}
// A row tile is 4 ints: expert, first sorted row, end row (exclusive), and
// a word locating the expert's entries (tile_word).  Entries past the number
// of tiles (up to max_tiles) hold expert -1.
constexpr int kTileInts = 4;
// tile_word: (index of the expert's first entry) | (its entry count << 16),
// or 0 when the list bound exceeds kTileWordMaxBound
constexpr int kTileWordMaxBound = 32768;
__host__ __device__ inline int tile_word(int first, int count, int bound) {
  return bound <= kTileWordMaxBound ? (first | (count << 16)) : 0;
}

// Typed pointers into the caller's MoE workspace.
struct WsPtrs {
  int* status;
  int* offsets;
  int* sorted_pairs;
  int* inv;
  int* chunk_counts;
  int* chunk_ranks;
  int* tiles;
  uint8_t* x_codes;  // FP8: E4M3 codes; MXFP4 activations: E2M1 blocks
  void* h;           // bf16 hi|lo (BF16 mode) or fp32 (FP8 mode)
  uint8_t* h_codes;
  float* y;
  uint8_t* x_scales;  // MXFP4 activations: E8M0 [ceil(H/128), T*k, 4] (step-major)
  uint8_t* h_scales;  // MXFP4 activations: E8M0 [ceil(I/128), T*k, 4]
  uint8_t* w13_stream;  // prefill modes: w13 scales restaged by launch_scale_stream
  uint8_t* w2_stream;   // prefill modes: w2 scales restaged
};

// Bytes of MXFP4 activation scales for `rows` rows of K elements: per
// 128-element K step, the four E8M0 bytes of every row (pad bytes 127), plus
// 512 bytes so that a step's read of a partial last row tile stays inside.
inline int64_t act_scale_bytes(int64_t rows, int K) { return (int64_t)((K + 127) / 128) * rows * 4 + 512; }

// Bytes of a restaged weight-code stream: 16 KB per (expert, n-tile, K step).
inline int64_t code_stream_bytes(int E, int nout_tiles, int K) { return (int64_t)E * nout_tiles * ((K + 127) / 128) * 16384; }
// The E2M1 codes of one expert tensor [E, R, K/2 bytes] restaged for the
// prefill GEMMs' copies (gateup: R = 2 nout rows, gate then up; else R = nout).
hipError_t launch_code_stream(const uint8_t* wb, int E, int R, int nout, int K, bool gateup, uint8_t* out,
                              hipStream_t s);

// Bytes of a restaged weight-scale stream: 1 KB per (expert, n-tile, K step).
inline int64_t scale_stream_bytes(int E, int nout_tiles, int K) { return (int64_t)E * nout_tiles * ((K + 127) / 128) * 1024; }
inline int gateup_ntiles(int I) { return (I + 127) / 128; }
inline int down_ntiles(int H) { return (H + 255) / 256; }

// Upper bound of the number of (expert, row-tile) entries.
inline int64_t max_tiles(int64_t npairs, int64_t E, int BM) {
  const int64_t busy = npairs < E ? npairs : E;
  return npairs / BM + busy + 1;
}

struct MoeShape {
  int T, H, I, E, k;
};

struct MoeWeights {
  const uint8_t* w13_blocks;
  const uint8_t* w13_scales;
  const uint16_t* w13_bias;
  const uint8_t* w2_blocks;
  const uint8_t* w2_scales;
  const uint16_t* w2_bias;
  // NVFP4 weights (16-element blocks, E4M3 scales [., ., K/16], one global
  // scale per tensor); bf16-activation path only
  bool nvfp4 = false;
  float w13_global = 1.0f;
  float w2_global = 1.0f;
  // E4M3 and MXFP4 activations: the codes restaged by launch_code_stream
  // (null: the prefill copies read the blocks above)
  const uint8_t* w13_codes = nullptr;
  const uint8_t* w2_codes = nullptr;
};

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int* ids, float* w,
                             hipStream_t s);
hipError_t launch_permute(const int* ids, int npairs, int E, int BM, int tile_bound,
                          const WsPtrs& ws, hipStream_t s);
// route + permute in one single-block launch, for T*k <= kFusedPermuteMaxPairs
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* ids, float* w, int BM,
                                int tile_bound, const WsPtrs& ws, hipStream_t s);

// FP8 quantisation of n values (fp32 or bf16 input); amax accumulates into
// *amax_bits (must be zero beforehand), the scale is written to *scale_out.
hipError_t launch_quant_fp8(const void* in, bool in_bf16, int64_t n, uint8_t* codes,
                            uint32_t* amax_bits, float* scale_out, hipStream_t s);
hipError_t launch_amax(const void* in, bool in_bf16, int64_t n, uint32_t* amax_bits,
                       hipStream_t s);
hipError_t launch_encode_fp8(const void* in, bool in_bf16, int64_t n, uint8_t* codes,
                             const uint32_t* amax_bits, float* scale_out, hipStream_t s);
// x codes in expert-sorted row order ([T*k, H], rows up to offsets[E]),
// scale from status[kStAmaxX] into status[kStScaleX].
hipError_t launch_encode_sorted_rows(const uint16_t* x, const MoeShape& sh, const WsPtrs& ws,
                                     hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t s);

// bf16-activation path (MFMA bf16 with weights expanded from FP4 in registers).
hipError_t launch_moe_gateup_bf16(const uint16_t* x, const MoeShape& sh, const MoeWeights& w,
                                  const WsPtrs& ws, int64_t ntile_bound, hipStream_t s);
hipError_t launch_moe_down_bf16(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                int64_t ntile_bound, hipStream_t s);
// Decode batches: the gate_up kernel routes the batch itself (top-k of
// `logits`, writing ids / wts and the permutation into the workspace), in
// place of the route + permutation launch.  Applies when
// gateup_routes_batch() holds.
// One routing round of 8 tokens (16 lanes each) per block; measured, each
// further round costs the gate_up kernel about 3 us, more than the route +
// permutation launch it replaces (about 8 us plus a launch gap) at 32 tokens.
constexpr int kGateUpRouteMaxTokens = 8;
bool gateup_routes_batch(const MoeShape& sh, bool nvfp4);
hipError_t launch_moe_gateup_bf16_routed(const uint16_t* x, const float* logits, int* ids, float* wts,
                                         const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                         int64_t ntile_bound, hipStream_t s);
hipError_t launch_linear_bf16(const uint16_t* x, int M, int N, int K, const uint8_t* wb,
                              const uint8_t* ws, const uint16_t* bias, uint16_t* out,
                              hipStream_t s);

// FP8 x FP4 block-scaled MFMA path.
hipError_t launch_moe_gateup_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                 int64_t ntile_bound, hipStream_t s);
// With out_bf16, down writes y rounded once to bf16 there instead of fp32 y
// (the dense projection: one expert, rows in order, routing weight 1).
hipError_t launch_moe_down_fp8(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                               int64_t ntile_bound, hipStream_t s, uint16_t* out_bf16 = nullptr);

// MXFP4 activations: x in expert-sorted row order as E2M1 blocks + step-major
// E8M0 scales (h is quantised by the gate_up GEMM's epilogue).
hipError_t launch_quant_x_mxfp4_sorted(const uint16_t* x, const MoeShape& sh, const WsPtrs& ws,
                                       hipStream_t s);

// Restage one weight tensor's E8M0 scales (w13 when gateup, else w2) into
// the order the prefill GEMM copies them.
hipError_t launch_scale_stream(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws, bool gateup,
                               hipStream_t s);

// FP4 x FP4 block-scaled MFMA path (MXFP4 activations).
hipError_t launch_moe_gateup_fp4(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                                 hipStream_t s);
hipError_t launch_moe_down_fp4(const MoeShape& sh, const MoeWeights& w, const WsPtrs& ws,
                               hipStream_t s, uint16_t* out_bf16 = nullptr);

// Dense rows as one expert (the prefill-sized dense projection): zeroes the
// status words and writes the tile list of M rows in BM-row tiles (bound
// entries) and, when inv is not null, the identity row map inv[m] = m.
hipError_t launch_dense_tiles(int M, int BM, int bound, int* status, int* tiles, int* inv, hipStream_t s);

// bf16 [nblocks * 32] -> MXFP4 blocks [nblocks, 16] + E8M0 scales [nblocks]
hipError_t launch_quant_mxfp4(const uint16_t* w, int64_t nblocks, uint8_t* blocks, uint8_t* scales,
                              hipStream_t s);

// Streaming read of `bytes` (rounded down to whole 16 KB rounds of the
// grid: stream_read_bytes gives the bytes actually read) for ceiling
// measurements; dma selects direct-to-LDS copies over register loads.
hipError_t launch_stream_read(const void* buf, int64_t bytes, bool dma, uint32_t* sink, hipStream_t s);
int64_t stream_read_bytes(int64_t bytes);

// out[t] = sum_j w[t,j] * y[inv[t*k+j]]  -> bf16
hipError_t launch_combine(const MoeShape& sh, const float* topk_weights, const WsPtrs& ws,
                          uint16_t* out, hipStream_t s);

}  // namespace mx
