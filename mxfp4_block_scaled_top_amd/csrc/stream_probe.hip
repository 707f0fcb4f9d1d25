// Streaming-read ceiling of the device: reads a buffer once with the two
// access forms the library's weight streams use, so that measurements can be
// stated against what a plain read reaches on the same device (not against
// the nominal 8 TB/s alone).  Not on the layer's path.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace mx {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;    // 1 KB wave copies in flight per wave per round
constexpr int kProbeChunk = kProbeThreads * 16 * kProbeUnroll;   // 16 KB per block round

// DMA: each wave copies its 1 KB pieces global -> LDS with the nontemporal
// DMA the decode GEMV uses; registers: nontemporal 16-byte vector loads.
// Either way the block walks a contiguous slab of `per_block` bytes.  The
// words read are folded into one value that is stored only if it equals a
// value the caller passes (so the loads cannot be dropped).
template <bool DMA>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint8_t* __restrict__ buf,
                                                                     int64_t per_block, uint32_t magic,
                                                                     uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kProbeChunk];
  const uint8_t* base = buf + (int64_t)blockIdx.x * per_block;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t fold = 0;
  for (int64_t o = 0; o < per_block; o += kProbeChunk) {
    if (DMA) {
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t piece = o + (int64_t)(u * 4 + wave) * 1024;
        __builtin_amdgcn_global_load_lds(base + piece + 16 * lane, lds + (u * 4 + wave) * 1024, 16, 0, 2);
      }
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      uint4 v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u)
        v[u] = ld_stream16(base + o + (int64_t)(u * 4 + wave) * 1024 + 16 * lane);
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (DMA) {
    __syncthreads();
    fold = reinterpret_cast<const uint32_t*>(lds)[threadIdx.x];
  }
  if (fold == magic) sink[0] = fold;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, bool dma, uint32_t* sink, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // 4 blocks per compute unit, each a whole number of 16 KB rounds
  int64_t nblocks = (int64_t)cus * 4;
  const int64_t rounds = bytes / kProbeChunk;
  if (rounds < nblocks) nblocks = rounds > 0 ? rounds : 1;
  const int64_t per_block = rounds / nblocks * kProbeChunk;
  if (per_block == 0) return hipSuccess;
  if (dma)
    stream_read_kernel<true><<<(int)nblocks, kProbeThreads, 0, s>>>(static_cast<const uint8_t*>(buf), per_block,
                                                                    0x9e3779b9u, sink);
  else
    stream_read_kernel<false><<<(int)nblocks, kProbeThreads, 0, s>>>(static_cast<const uint8_t*>(buf), per_block,
                                                                     0x9e3779b9u, sink);
  return hipGetLastError();
}

int64_t stream_read_bytes(int64_t bytes) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int64_t nblocks = (int64_t)cus * 4;
  const int64_t rounds = bytes / kProbeChunk;
  if (rounds < nblocks) nblocks = rounds > 0 ? rounds : 1;
  return rounds / nblocks * kProbeChunk * nblocks;
}

}  // namespace mx
