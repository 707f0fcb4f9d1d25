// Router top-k of one token by 16 lanes, and the permutation of up to 128
// (token, slot) pairs over up to 128 experts by one wave.  Shared by the
// stand-alone route + permutation kernel and the decode gate_up kernel that
// routes the batch itself, so that both make bitwise the same choices.
//
// gpt-oss page, "GPT-OSS-120B Architecture": each token goes to 4 of 128
// experts.  Choices: largest fp32 logit first, the lower expert index on ties,
// -0 equal to +0; the weights are the softmax over the k chosen logits (exp of
// the difference to the largest chosen logit, the k terms summed in the order
// of a 32-lane butterfly, then one division), the arithmetic of
// route_topk_kernel.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mx {

constexpr int kSmallMaxPairs = 128;
constexpr int kSmallMaxExperts = 128;
constexpr int kSmallMaxK = 16;

// Order-preserving map of a non-NaN float to uint32 (larger float, larger
// key; -0 and +0 map to the same key); 0 is below every mapped value.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b << 1) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}
// maximum over the 16 lanes of a DPP row, in every lane of the row
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, dpp_u32<0x121>(v));   // row_ror:1
  v = max(v, dpp_u32<0x122>(v));   // row_ror:2
  v = max(v, dpp_u32<0x124>(v));   // row_ror:4
  v = max(v, dpp_u32<0x128>(v));   // row_ror:8
  return v;
}
__device__ __forceinline__ uint32_t row16_min(uint32_t v) {
  v = min(v, dpp_u32<0x121>(v));
  v = min(v, dpp_u32<0x122>(v));
  v = min(v, dpp_u32<0x124>(v));
  v = min(v, dpp_u32<0x128>(v));
  return v;
}
// lanes holding expert e among the lanes of mask `valid`, given the wave's
// ballots of each id bit
__device__ __forceinline__ uint64_t lanes_with(int e, const uint64_t* bits, uint64_t valid) {
  uint64_t m = valid;
#pragma unroll
  for (int b = 0; b < 7; ++b) m &= ((e >> b) & 1) ? bits[b] : ~bits[b];
  return m;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Keys of one token's logits for the 16 lanes of a DPP row (l16 = lane %
// 16): lane l16 holds logits l16 + 16 i (E <= 128); 0 where taken, past E,
// or for a padding row (`live` false, the same in all 16 lanes).
__device__ __forceinline__ void route16_keys(const float* __restrict__ row, bool live, int E, int l16,
                                             uint32_t (&key)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = l16 + 16 * i;
    key[i] = live && idx < E ? order_key(row[idx]) : 0u;
  }
}

// The row's top k (k <= 16) of those keys: lane l16 < k ends with slot
// l16's expert and weight.  Each lane computes the exp of its own slot; the
// k terms are summed across the row by DPP in the order of a 32-lane
// butterfly over 16 slots (z[l] + z[l+8], then + 4 apart, then
// (c[0] + c[2]) + (c[1] + c[3])), slots past k being 0, then one division.
__device__ __forceinline__ void route16_pick(uint32_t (&key)[8], int k, int l16, int& out_id, float& out_w) {
  int my_id = 0;
  float my_val = 0.0f, val0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = max(m, key[i]);
    m = row16_max(m);
    // lowest index holding the maximum: the lane's first i with that key,
    // then the row minimum
    uint32_t cand = 0xffffffffu;
#pragma unroll
    for (int i = 7; i >= 0; --i) cand = key[i] == m ? (uint32_t)(l16 + 16 * i) : cand;
    const uint32_t win = row16_min(cand);
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = (uint32_t)(l16 + 16 * i) == win ? 0u : key[i];
    const float v = key_value(m);
    if (j == 0) val0 = v;
    if (j == l16) {
      my_id = (int)win;
      my_val = v;
    }
  }
  const float z = l16 < k ? expf(my_val - val0) : 0.0f;
  const float b8 = z + __int_as_float((int)dpp_u32<0x128>((uint32_t)__float_as_int(z)));     // + z[l+8]
  const float c4 = b8 + __int_as_float((int)dpp_u32<0x12c>((uint32_t)__float_as_int(b8)));   // + b8[l+4]
  const float d2 = c4 + __int_as_float((int)dpp_u32<0x12e>((uint32_t)__float_as_int(c4)));   // + c4[l+2]
  const float e1 = d2 + __int_as_float((int)dpp_u32<0x12f>((uint32_t)__float_as_int(d2)));   // + d2[l+1]
  // lane 0 of the row holds (c4[0] + c4[2]) + (c4[1] + c4[3]); every lane takes it
  const float ssum = __shfl(e1, (int)(threadIdx.x & 63) & ~15, 64);
  out_id = my_id;
  out_w = z / ssum;
}

// route16_keys then route16_pick.
__device__ __forceinline__ void route16_token(const float* __restrict__ row, bool live, int E, int k, int l16,
                                              int& out_id, float& out_w) {
  uint32_t key[8];
  route16_keys(row, live, E, l16, key);
  route16_pick(key, k, l16, out_id, out_w);
}

// Where the permutation goes; any pointer may be null (not written).  The
// pointers may address LDS or global memory.
struct PermDst {
  int* offsets;       // [E+1]
  int* sorted_pairs;  // [npairs]
  int* inv;           // [npairs]
  int* tiles;         // [bound * kTileInts], entries past the tile count: expert -1
  int* status;        // [kStWords]: the tile count, every other word 0
};

// One wave (all 64 lanes call it): the stable regrouping of the npairs
// (<= 128) pairs with ids `ids` (valid ids < E <= 128) by expert, the row
// tiles of BM rows, written to both destinations.  eoff: LDS scratch of E
// ints.  Pairs lane and lane + 64, experts 2 lane and 2 lane + 1.
__device__ __forceinline__ void permute_wave(const int* ids, int npairs, int E, int BM, int bound, int* eoff,
                                             const PermDst& d0, const PermDst& d1) {
  const int lane = threadIdx.x & 63;
  const int p0 = lane, p1 = lane + 64;
  const bool v0 = p0 < npairs, v1 = p1 < npairs;
  const int e0 = v0 ? ids[p0] : 0, e1 = v1 ? ids[p1] : 0;
  uint64_t B0[7], B1[7];
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    B0[b] = __ballot(v0 && ((e0 >> b) & 1));
    B1[b] = __ballot(v1 && ((e1 >> b) & 1));
  }
  const uint64_t V0 = __ballot(v0), V1 = __ballot(v1);
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int r0 = __popcll(lanes_with(e0, B0, V0) & below);
  const int r1 = __popcll(lanes_with(e1, B0, V0)) + __popcll(lanes_with(e1, B1, V1) & below);
  const int ea = 2 * lane, eb = 2 * lane + 1;
  const int ca = ea < E ? __popcll(lanes_with(ea, B0, V0)) + __popcll(lanes_with(ea, B1, V1)) : 0;
  const int cb = eb < E ? __popcll(lanes_with(eb, B0, V0)) + __popcll(lanes_with(eb, B1, V1)) : 0;
  const int pincl = wave_incl_scan(ca + cb);
  const int offa = pincl - ca - cb, offb = offa + ca;
  if (ea < E) eoff[ea] = offa;
  if (eb < E) eoff[eb] = offb;
  const PermDst* dst[2] = {&d0, &d1};
#pragma unroll
  for (int di = 0; di < 2; ++di) {
    int* off = dst[di]->offsets;
    if (!off) continue;
    if (ea < E) off[ea] = offa;
    if (eb < E) off[eb] = offb;
    if (lane == 63) off[E] = pincl;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  const int pos0 = v0 ? eoff[e0] + r0 : 0, pos1 = v1 ? eoff[e1] + r1 : 0;
  // row tiles: expert e contributes ceil(n_e / BM) entries, in expert order
  const int na = (ca + BM - 1) / BM, nb2 = (cb + BM - 1) / BM;
  const int tincl = wave_incl_scan(na + nb2);
  const int fa = tincl - na - nb2, fb = fa + na;
  const int ntiles = __shfl(tincl, 63, 64);
  const int wa = tile_word(fa, na, bound), wb = tile_word(fb, nb2, bound);
#pragma unroll
  for (int di = 0; di < 2; ++di) {
    const PermDst& d = *dst[di];
    if (d.sorted_pairs) {
      if (v0) d.sorted_pairs[pos0] = p0;
      if (v1) d.sorted_pairs[pos1] = p1;
    }
    if (d.inv) {
      if (v0) d.inv[p0] = pos0;
      if (v1) d.inv[p1] = pos1;
    }
    if (d.tiles) {
      for (int i = 0; i < na; ++i) {
        const int b = offa + i * BM;
        *reinterpret_cast<int4*>(d.tiles + kTileInts * (fa + i)) = make_int4(ea, b, min(b + BM, offa + ca), wa);
      }
      for (int i = 0; i < nb2; ++i) {
        const int b = offb + i * BM;
        *reinterpret_cast<int4*>(d.tiles + kTileInts * (fb + i)) = make_int4(eb, b, min(b + BM, offb + cb), wb);
      }
      for (int t = ntiles + lane; t < bound; t += 64)
        *reinterpret_cast<int4*>(d.tiles + kTileInts * t) = make_int4(-1, 0, 0, 0);
    }
    if (d.status && lane < kStWords) d.status[lane] = lane == kStNumTiles ? ntiles : 0;
  }
}

}  // namespace mx
