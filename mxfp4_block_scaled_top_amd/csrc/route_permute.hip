// Router top-k and the token-by-expert permutation (histogram, scan, stable
// scatter) that regroups the T*k (token, slot) pairs by expert.
//
// gpt-oss page, "GPT-OSS-120B Architecture": each token is routed to 4 of
// 128 experts.  gptoss-spark page, "What produced it, ranked": a MoE support
// kernel that aligns tokens to experts was one of the measured wins; this is
// the gfx950 version of that step.  Everything here is integer work except
// the fp32 softmax of the k chosen logits.
#include "common.hpp"
#include "launch.hpp"
#include "route_small.hpp"

namespace mx {

// ---------------------------------------------------------------- top-k ----
// W lanes (a wave, or half a wave) route one token; lane l of the group
// holds logits l, l+W, ... (PER_LANE of them).  Lanes j < k of the group end
// with the j-th choice (id, softmax weight over the k chosen logits).
template <int PER_LANE, int W = 64>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int lane,
                                            int& out_id, float& out_w) {
  float v[PER_LANE];
  bool avail[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int idx = lane + W * i;
    avail[i] = idx < E;
    v[i] = avail[i] ? row[idx] : 0.0f;
  }
  float my_val = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    // best (largest value, then smallest index) among this lane's free entries
    float bv = 0.0f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int idx = lane + W * i;
      if (avail[i] && (bi == 0x7fffffff || v[i] > bv)) { bv = v[i]; bi = idx; }
    }
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, W);
      const int oi = __shfl_xor(bi, off, W);
      const bool take = oi != 0x7fffffff &&
                        (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
      if (take) { bv = ov; bi = oi; }
    }
    // the owner marks its entry as taken
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (lane + W * i == bi) avail[i] = false;
    if (lane == j) { my_val = bv; my_id = bi; }
  }
  // softmax over the k chosen logits (lane 0 of the group holds the largest)
  const float vmax = __shfl(my_val, 0, W);
  const float z = lane < k ? expf(my_val - vmax) : 0.0f;
  float s = z;
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, W);
  out_id = my_id;
  out_w = z / s;
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int T, int E, int k,
                                                         int* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int id;
  float w;
  route_token<PER_LANE>(logits + (size_t)t * E, E, k, lane, id, w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    weights[(size_t)t * k + lane] = w;
  }
}

// ---------------------------------------------------------- permutation ----
constexpr int kChunk = 1024;          // pairs ranked together by one block
constexpr int kChunkWaves = kChunk / 64;

// Exclusive scan of one int per thread over a 1024-thread block.
// `tmp` holds kChunkWaves ints of LDS.  Returns the exclusive prefix; *total
// receives the block sum.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kChunkWaves ? tmp[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(wi, off, 64);
      if (lane >= off) wi += o;
    }
    if (lane < kChunkWaves) tmp[lane] = wi - w;    // exclusive wave offsets
    if (lane == kChunkWaves - 1) tmp[kChunkWaves] = wi;
  }
  __syncthreads();
  const int res = tmp[wave] + incl - v;
  *total = tmp[kChunkWaves];
  __syncthreads();
  return res;
}

// Lanes of this wave holding the same expert id e (valid lanes only).
__device__ __forceinline__ uint64_t match_lanes(int e, bool valid, int id_bits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    same &= bit ? bb : ~bb;
  }
  return valid ? same : 0ull;
}

// Within-chunk stable ranks.  Each of the 1024 threads holds pair base+tid
// with expert e (valid only if in range).  wcnt is [kChunkWaves][E] LDS.
// Returns the rank of the pair among the chunk's pairs of the same expert
// (ascending pair index); afterwards wcnt[w][e] holds wave w's count of e.
__device__ int chunk_rank(int e, bool valid, int E, int id_bits, int* wcnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kChunkWaves * E; i += kChunk) wcnt[i] = 0;
  __syncthreads();
  const uint64_t same = match_lanes(e, valid, id_bits);
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int rank_in_wave = __popcll(same & below);
  const bool leader = valid && (same & below) == 0;
  if (leader) wcnt[wave * E + e] = __popcll(same);
  __syncthreads();
  int pre = 0;
  if (valid)
    for (int w = 0; w < wave; ++w) pre += wcnt[w * E + e];
  return pre + rank_in_wave;
}

__device__ __forceinline__ bool id_ok(int e, int E) { return e >= 0 && e < E; }

// Tile list: expert e with n_e sorted rows contributes ceil(n_e / BM) entries
// (e, offsets[e] + i*BM, min(offsets[e] + (i+1)*BM, offsets[e] + n_e), w)
// with w = (index of e's first entry) | (e's entry count << 16) while the
// list bound is at most kTileWordMaxBound entries, else 0;
// entries from the tile count up to `bound` get expert -1, so a GEMM block
// learns everything about its tile from one 16-byte read.  Called by a whole
// 1024-thread block with cnt and off valid in LDS (E <= 1024).
__device__ void write_tiles(const int* cnt, const int* off, int E, int BM, int bound,
                            int* scan_tmp, int* tiles, int* status) {
  const int e = threadIdx.x;
  const int nt = (e < E) ? (cnt[e] + BM - 1) / BM : 0;
  int total;
  const int first = block_exclusive_scan(nt, scan_tmp, &total);
  const int w = tile_word(first, nt, bound);
  for (int i = 0; i < nt; ++i) {
    const int b = off[e] + i * BM;
    const int end = off[e] + cnt[e];
    *reinterpret_cast<int4*>(tiles + kTileInts * (first + i)) = make_int4(e, b, min(b + BM, end), w);
  }
  for (int t = total + (int)threadIdx.x; t < bound; t += (int)blockDim.x)
    *reinterpret_cast<int4*>(tiles + kTileInts * t) = make_int4(-1, 0, 0, 0);
  if (threadIdx.x == 0) status[kStNumTiles] = total;
}

// Single-block permutation for small pair counts (decode): counts, offsets,
// stable scatter and tile list, run by a whole 1024-thread block.  `ids` may
// live in global memory or LDS.  lds: cnt[E], off[E], run[E], wcnt[16*E] ints.
__device__ void permute_block(const int* ids, int npairs, int E, int id_bits, int BM, int bound,
                              int* __restrict__ status, int* __restrict__ offsets,
                              int* __restrict__ sorted_pairs, int* __restrict__ inv,
                              int* __restrict__ tiles, int* lds, int* scan_tmp) {
  int* cnt = lds;
  int* off = lds + E;
  int* run = lds + 2 * E;
  int* wcnt = lds + 3 * E;
  const int tid = threadIdx.x;
  if (tid < kStWords && tid != kStNumTiles) status[tid] = 0;
  for (int e = tid; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int p = tid; p < npairs; p += kChunk) {
    const int e = ids[p];
    if (id_ok(e, E)) atomicAdd(&cnt[e], 1); else bad = true;
  }
  __syncthreads();
  int total;
  const int ex = block_exclusive_scan(tid < E ? cnt[tid] : 0, scan_tmp, &total);
  if (tid < E) { off[tid] = ex; run[tid] = ex; offsets[tid] = ex; }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  for (int base = 0; base < npairs; base += kChunk) {
    const int p = base + tid;
    const int e = p < npairs ? ids[p] : -1;
    const bool valid = p < npairs && id_ok(e, E);
    const int r = chunk_rank(e, valid, E, id_bits, wcnt);
    if (valid) {
      const int pos = run[e] + r;
      sorted_pairs[pos] = p;
      inv[p] = pos;
    } else if (p < npairs) {
      inv[p] = -1;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kChunk) {
      int c = 0;
      for (int w = 0; w < kChunkWaves; ++w) c += wcnt[w * E + ee];
      run[ee] += c;
    }
    __syncthreads();
  }
  if (bad) atomicOr(&status[kStFlags], 1);
  write_tiles(cnt, off, E, BM, bound, scan_tmp, tiles, status);
}

__global__ __launch_bounds__(1024) void permute_fused_kernel(
    const int* __restrict__ ids, int npairs, int E, int id_bits, int BM, int bound,
    int* __restrict__ status, int* __restrict__ offsets, int* __restrict__ sorted_pairs,
    int* __restrict__ inv, int* __restrict__ tiles) {
  extern __shared__ int lds[];
  __shared__ int scan_tmp[kChunkWaves + 1];
  permute_block(ids, npairs, E, id_bits, BM, bound, status, offsets, sorted_pairs, inv, tiles, lds,
                scan_tmp);
}

// Router and permutation in one 1024-thread block (decode-sized batches):
// each half wave routes one token (32 per round: tokens h, h + 32, ... for
// half wave h) into LDS and the caller's id/weight outputs, then the block
// permutes from LDS.  One launch instead of two.
// lds: ids[npairs] ints, then the permutation's cnt/off/run/wcnt arrays.
template <int PER_LANE>
__global__ __launch_bounds__(1024) void route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int id_bits, int BM, int bound,
    int* __restrict__ ids_out, float* __restrict__ w_out, int* __restrict__ status,
    int* __restrict__ offsets, int* __restrict__ sorted_pairs, int* __restrict__ inv,
    int* __restrict__ tiles) {
  extern __shared__ int lds[];
  __shared__ int scan_tmp[kChunkWaves + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int npairs = T * k;
  int* ids = lds;
  const int hl = lane & 31;
  for (int t = 2 * wave + (lane >> 5); t - (lane >> 5) < T; t += 2 * kChunkWaves) {
    // both halves of a wave stay in the loop together (the shuffles are
    // wave instructions); a half past T routes a clamped row and stores nothing
    const int tt = t < T ? t : T - 1;
    int id;
    float w;
    route_token<2 * PER_LANE, 32>(logits + (size_t)tt * E, E, k, hl, id, w);
    if (t < T && hl < k) {
      ids[t * k + hl] = id;
      ids_out[(size_t)t * k + hl] = id;
      w_out[(size_t)t * k + hl] = w;
    }
  }
  __syncthreads();
  permute_block(ids, npairs, E, id_bits, BM, bound, status, offsets, sorted_pairs, inv, tiles,
                lds + ((npairs + 3) & ~3), scan_tmp);
}

// ------------------------------------------------ small decode batches ----
// Route + permutation for at most 128 pairs and 128 experts (k <= 16): 16
// lanes route one token (8 logits each; 4 tokens per wave, 32 per round of
// 8 waves), then a single wave builds the permutation from ballots, so the
// block needs one barrier instead of a dozen.  Results are bitwise those of
// route_topk_kernel and permute_block: the same choices (largest logit,
// lower index on ties, -0 equal to +0) and the same softmax arithmetic
// (exp of the difference to the largest chosen logit, the k terms summed in
// the order of a 32-lane butterfly, then one division).
constexpr int kSmallThreads = 512;

__global__ __launch_bounds__(kSmallThreads) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int BM, int bound,
    int* __restrict__ ids_out, float* __restrict__ w_out, int* __restrict__ status,
    int* __restrict__ offsets, int* __restrict__ sorted_pairs, int* __restrict__ inv,
    int* __restrict__ tiles) {
  __shared__ int ids[kSmallMaxPairs];
  __shared__ int eoff[kSmallMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, tw = lane >> 4;
  const int npairs = T * k;
  for (int t0 = 0; t0 < T; t0 += 4 * (kSmallThreads / 64)) {
    const int t = t0 + 4 * wave + tw;
    const bool live = t < T;   // the whole 16-lane row agrees
    int id;
    float w;
    route16_token(logits + (size_t)(live ? t : 0) * E, live, E, k, l16, id, w);
    if (live && l16 < k) {
      ids[t * k + l16] = id;
      ids_out[(size_t)t * k + l16] = id;
      w_out[(size_t)t * k + l16] = w;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const PermDst d0{offsets, sorted_pairs, inv, tiles, status};
  const PermDst none{nullptr, nullptr, nullptr, nullptr, nullptr};
  permute_wave(ids, npairs, E, BM, bound, eoff, d0, none);
}

// Multi-block path, phase 1: per-chunk ranks and per-chunk expert counts
// (a pair whose id lies outside [0, E) gets rank -1 and is not counted).
__global__ __launch_bounds__(1024) void permute_count_kernel(
    const int* __restrict__ ids, int npairs, int E, int id_bits,
    int* __restrict__ chunk_counts, int* __restrict__ chunk_ranks) {
  extern __shared__ int wcnt[];
  const int c = blockIdx.x;
  const int p = c * kChunk + threadIdx.x;
  const int e = p < npairs ? ids[p] : -1;
  const bool valid = p < npairs && id_ok(e, E);
  const int r = chunk_rank(e, valid, E, id_bits, wcnt);
  if (p < npairs) chunk_ranks[p] = valid ? r : -1;
  for (int ee = threadIdx.x; ee < E; ee += kChunk) {
    int s = 0;
    for (int w = 0; w < kChunkWaves; ++w) s += wcnt[w * E + ee];
    chunk_counts[(size_t)c * E + ee] = s;
  }
}

// Phase 2 (one block): per-expert totals, offsets, per-chunk bases, tiles,
// and every status word of the call (the skipped-id flag from the count of
// pairs that were kept; the words later steps accumulate into start at 0).
__global__ __launch_bounds__(1024) void permute_scan_kernel(
    int npairs, int nchunks, int E, int BM, int bound, int* __restrict__ status, int* __restrict__ offsets,
    int* __restrict__ chunk_counts, int* __restrict__ tiles) {
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  __shared__ int scan_tmp[kChunkWaves + 1];
  const int e = threadIdx.x;
  // chunks in batches of 8, each batch's loads issued before its stores
  // (the stores go to the same array, so a load cannot pass the previous
  // chunk's store: one memory round trip per batch instead of per chunk)
  constexpr int kB = 8;
  int running = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (c0 + u < nchunks) chunk_counts[(size_t)(c0 + u) * E + e] = running;
        running += v[u];
      }
    }
    cnt[e] = running;
  }
  int total;
  const int ex = block_exclusive_scan(e < E ? running : 0, scan_tmp, &total);
  if (e < E) {
    off[e] = ex;
    offsets[e] = ex;
    for (int c0 = 0; c0 < nchunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (c0 + u < nchunks) chunk_counts[(size_t)(c0 + u) * E + e] = v[u] + ex;
    }
  }
  if (e == 0) offsets[E] = total;
  if (e < kStWords && e != kStNumTiles) status[e] = e == kStFlags ? (total != npairs ? 1 : 0) : 0;
  __syncthreads();
  write_tiles(cnt, off, E, BM, bound, scan_tmp, tiles, status);
}

// Phase 3: scatter each pair to its sorted row.
__global__ __launch_bounds__(1024) void permute_scatter_kernel(
    const int* __restrict__ ids, int npairs, int E, const int* __restrict__ chunk_counts,
    const int* __restrict__ chunk_ranks, int* __restrict__ sorted_pairs, int* __restrict__ inv) {
  const int c = blockIdx.x;
  const int p = c * kChunk + threadIdx.x;
  if (p >= npairs) return;
  const int e = ids[p];
  const int r = chunk_ranks[p];
  if (!id_ok(e, E) || r < 0) { inv[p] = -1; return; }
  const int pos = chunk_counts[(size_t)c * E + e] + r;
  sorted_pairs[pos] = p;
  inv[p] = pos;
}

// ------------------------------------------------------------- launchers ----
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int* ids, float* w,
                             hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64) route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128) route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256) route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

static int id_bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* ids, float* w, int BM,
                                int tile_bound, const WsPtrs& ws, hipStream_t s) {
  const int npairs = T * k;
  if (npairs <= kSmallMaxPairs && E <= kSmallMaxExperts && k <= kSmallMaxK) {
    route_permute_small_kernel<<<1, kSmallThreads, 0, s>>>(logits, T, E, k, BM, tile_bound, ids, w, ws.status,
                                                          ws.offsets, ws.sorted_pairs, ws.inv, ws.tiles);
    return hipGetLastError();
  }
  const int bits = id_bits_for(E);
  const size_t lds = ((size_t)((npairs + 3) & ~3) + (size_t)(3 + kChunkWaves) * E) * sizeof(int);
  if (E <= 64)
    route_permute_kernel<1><<<1, kChunk, lds, s>>>(logits, T, E, k, bits, BM, tile_bound, ids, w, ws.status,
                                                    ws.offsets, ws.sorted_pairs, ws.inv, ws.tiles);
  else if (E <= 128)
    route_permute_kernel<2><<<1, kChunk, lds, s>>>(logits, T, E, k, bits, BM, tile_bound, ids, w, ws.status,
                                                    ws.offsets, ws.sorted_pairs, ws.inv, ws.tiles);
  else if (E <= 256)
    route_permute_kernel<4><<<1, kChunk, lds, s>>>(logits, T, E, k, bits, BM, tile_bound, ids, w, ws.status,
                                                    ws.offsets, ws.sorted_pairs, ws.inv, ws.tiles);
  else
    route_permute_kernel<8><<<1, kChunk, lds, s>>>(logits, T, E, k, bits, BM, tile_bound, ids, w, ws.status,
                                                    ws.offsets, ws.sorted_pairs, ws.inv, ws.tiles);
  return hipGetLastError();
}

// ------------------------------------------------- dense rows, one expert ----
// The prefill-sized dense projection runs the down GEMM with one expert whose
// rows are the M activation rows in order: tiles of BM rows, the tile count
// and zeroed status words, and (MXFP4 activations) the identity row map.
__global__ __launch_bounds__(256) void dense_tiles_kernel(int M, int BM, int bound, int* __restrict__ status,
                                                          int* __restrict__ tiles, int* __restrict__ inv) {
  const int ntiles = (M + BM - 1) / BM;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < kStWords) status[threadIdx.x] = threadIdx.x == kStNumTiles ? ntiles : 0;
  if (i < bound) {
    const int t = (int)i;
    *reinterpret_cast<int4*>(tiles + kTileInts * i) =
        t < ntiles ? make_int4(0, t * BM, min(t * BM + BM, M), tile_word(0, ntiles, bound)) : make_int4(-1, 0, 0, 0);
  }
  if (inv && i < M) inv[i] = (int)i;
}

hipError_t launch_dense_tiles(int M, int BM, int bound, int* status, int* tiles, int* inv, hipStream_t s) {
  const int64_t n = M > bound ? M : bound;
  const unsigned grid = (unsigned)((n + 255) / 256);
  dense_tiles_kernel<<<grid > 0 ? grid : 1, 256, 0, s>>>(M, BM, bound, status, tiles, inv);
  return hipGetLastError();
}

hipError_t launch_permute(const int* ids, int npairs, int E, int BM, int tile_bound,
                          const WsPtrs& ws, hipStream_t s) {
  const int bits = id_bits_for(E);
  if (npairs <= kFusedPermuteMaxPairs) {
    const size_t lds = (size_t)(3 + kChunkWaves) * E * sizeof(int);
    permute_fused_kernel<<<1, kChunk, lds, s>>>(ids, npairs, E, bits, BM, tile_bound, ws.status,
                                                 ws.offsets, ws.sorted_pairs, ws.inv, ws.tiles);
    return hipGetLastError();
  }
  const int nchunks = (npairs + kChunk - 1) / kChunk;
  permute_count_kernel<<<nchunks, kChunk, (size_t)kChunkWaves * E * sizeof(int), s>>>(
      ids, npairs, E, bits, ws.chunk_counts, ws.chunk_ranks);
  permute_scan_kernel<<<1, kChunk, 0, s>>>(npairs, nchunks, E, BM, tile_bound, ws.status, ws.offsets,
                                           ws.chunk_counts, ws.tiles);
  permute_scatter_kernel<<<nchunks, kChunk, 0, s>>>(ids, npairs, E, ws.chunk_counts,
                                                    ws.chunk_ranks, ws.sorted_pairs, ws.inv);
  return hipGetLastError();
}

}  // namespace mx
