// C ABI of the MXFP4 MoE library: argument validation, workspace plan and
// launch sequencing.  Declarations and the contract are in
// include/mxfp4_moe.h.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/mxfp4_moe.h"
#include "common.hpp"
#include "launch.hpp"
#include "code_rows.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MXFP4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Cached per-device architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch[64];

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MXFP4_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MXFP4_E_DEVICE, "device index %d out of range", dev);
  int state = g_arch[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MXFP4_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(state, std::memory_order_relaxed);
    if (state == 2) return fail(MXFP4_E_DEVICE, "device %d is %s, only gfx950 is supported", dev, prop.gcnArchName);
  }
  if (state != 1) return fail(MXFP4_E_DEVICE, "device %d is not gfx950", dev);
  return MXFP4_OK;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int moe_shape_check(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, int32_t act_mode) {
  if (act_mode != MXFP4_ACT_BF16 && act_mode != MXFP4_ACT_FP8_E4M3 && act_mode != MXFP4_ACT_MXFP4)
    return fail(MXFP4_E_MODE, "unknown act_mode %d", act_mode);
  if (T < 0 || T > (1 << 22)) return fail(MXFP4_E_SHAPE, "T=%lld outside [0, 2^22]", (long long)T);
  if (H <= 0 || H % 32 || H > (1 << 16)) return fail(MXFP4_E_SHAPE, "H=%lld must be a positive multiple of 32 (<= 65536)", (long long)H);
  if (I <= 0 || I % 32 || I > (1 << 16)) return fail(MXFP4_E_SHAPE, "I=%lld must be a positive multiple of 32 (<= 65536)", (long long)I);
  if (E < 1 || E > 512) return fail(MXFP4_E_SHAPE, "E=%d outside [1, 512]", E);
  if (k < 1 || k > 16 || k > E) return fail(MXFP4_E_SHAPE, "k=%d outside [1, min(E, 16)]", k);
  const int64_t npairs = T * k;
  // (64-row tiles are taken only below 64 E pairs: far inside the limit)
  const int bm = act_mode == MXFP4_ACT_BF16 ? mx::kDecodeBM : mx::kPrefillBM;
  if (mx::max_tiles(npairs, E, bm) > 65535) return fail(MXFP4_E_SHAPE, "T*k=%lld gives too many row tiles", (long long)npairs);
  return MXFP4_OK;
}

// nv: NVFP4 weights, whose restaged scale streams take 8 bytes per row and
// 128-element step instead of 4.
void plan(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, int32_t act_mode,
          mxfp4_moe_workspace_layout* L, bool nv = false) {
  const int64_t np = T * k;
  const int64_t nchunks = (np + 1023) / 1024;
  // E4M3 activations: room for the 64-row tiles of NVFP4 weights with
  // either weight format, so that both share the layout up to the scale
  // streams
  const int bm = act_mode == MXFP4_ACT_BF16       ? mx::kDecodeBM
                 : act_mode == MXFP4_ACT_FP8_E4M3 ? mx::prefill_bm(np, E, true)
                                                  : mx::kPrefillBM;
  size_t o = 0;
  memset(L, 0, sizeof(*L));
  L->status = o; o = up(o + mx::kStWords * 4);
  L->expert_offsets = o; o = up(o + (size_t)(E + 1) * 4);
  L->sorted_pairs = o; o = up(o + (size_t)np * 4);
  L->inv_pairs = o; o = up(o + (size_t)np * 4);
  L->chunk_counts = o; o = up(o + (size_t)nchunks * E * 4);
  L->chunk_ranks = o; o = up(o + (size_t)np * 4);
  L->tiles = o; o = up(o + (size_t)mx::max_tiles(np, E, bm) * mx::kTileInts * 4);
  if (act_mode == MXFP4_ACT_FP8_E4M3) {
    L->x_codes = o; o = up(o + (size_t)np * mx::code_row_bytes(H, false));
    L->h = o; o = up(o + (size_t)np * I * 4);
    L->h_codes = o; o = up(o + (size_t)np * mx::code_row_bytes(I, false));
  } else if (act_mode == MXFP4_ACT_MXFP4) {
    L->x_codes = o; o = up(o + (size_t)np * mx::code_row_bytes(H, true));
    L->x_scales = o; o = up(o + (size_t)mx::act_scale_bytes(np, (int)H));
    L->h = o;                      // h is quantised in the GEMM epilogue: no fp32 copy
    L->h_codes = o; o = up(o + (size_t)np * mx::code_row_bytes(I, true));
    L->h_scales = o; o = up(o + (size_t)mx::act_scale_bytes(np, (int)I));
  } else {
    L->x_codes = o;
    L->h = o; o = up(o + (size_t)np * I * 2 * 2);
    L->h_codes = o;
  }
  L->y = o; o = up(o + (size_t)np * H * 4);
  if (act_mode != MXFP4_ACT_BF16) {
    const size_t f = nv ? 2 : 1;
    L->w13_scale_stream = o; o = up(o + f * (size_t)mx::scale_stream_bytes(E, mx::gateup_ntiles((int)I), (int)H));
    L->w2_scale_stream = o; o = up(o + f * (size_t)mx::scale_stream_bytes(E, mx::down_ntiles((int)H), (int)I));
  }
  L->total_bytes = o;
}

// Workspace of the quantised-activation dense projection (one expert, M
// rows in order): status words, tile list, identity row map (MXFP4), the
// activation codes (and MXFP4 scales, step-major), the restaged weight
// scales.  BF16 activations need none.
struct LinearLayout {
  size_t status, tiles, inv, codes, scales, w_stream, total;
};

int linear_shape_check(int64_t M, int64_t N, int64_t K, int32_t act_mode) {
  if (act_mode != MXFP4_ACT_BF16 && act_mode != MXFP4_ACT_FP8_E4M3 && act_mode != MXFP4_ACT_MXFP4)
    return fail(MXFP4_E_MODE, "unknown act_mode %d", act_mode);
  if (M < 0 || M > (1 << 20)) return fail(MXFP4_E_SHAPE, "M=%lld outside [0, 2^20]", (long long)M);
  if (N <= 0 || N % 16 || N > (1LL << 26)) return fail(MXFP4_E_SHAPE, "N=%lld must be a positive multiple of 16", (long long)N);
  if (K <= 0 || K % 32 || K > (1 << 20)) return fail(MXFP4_E_SHAPE, "K=%lld must be a positive multiple of 32", (long long)K);
  if (act_mode != MXFP4_ACT_BF16) {
    if (K > (1 << 16)) return fail(MXFP4_E_SHAPE, "K=%lld above 65536 with quantised activations", (long long)K);
    // (row tiles) x (256-row n-tiles) work units in an int
    if ((M / mx::kPrefillBM + 1) * (N / 256 + 1) >= (1LL << 30))
      return fail(MXFP4_E_SHAPE, "M=%lld x N=%lld too large with quantised activations", (long long)M, (long long)N);
  }
  return MXFP4_OK;
}

void linear_plan(int64_t M, int64_t N, int64_t K, int32_t act_mode, LinearLayout* L) {
  memset(L, 0, sizeof(*L));
  if (act_mode == MXFP4_ACT_BF16) return;
  const bool a4 = act_mode == MXFP4_ACT_MXFP4;
  size_t o = 0;
  L->status = o; o = up(o + mx::kStWords * 4);
  L->tiles = o; o = up(o + (size_t)mx::max_tiles(M, 1, mx::kPrefillBM) * mx::kTileInts * 4);
  L->inv = o; if (a4) o = up(o + (size_t)M * 4);
  L->codes = o; o = up(o + (size_t)M * mx::code_row_bytes(K, a4));
  L->scales = o; if (a4) o = up(o + (size_t)mx::act_scale_bytes(M, (int)K));
  L->w_stream = o; o = up(o + (size_t)mx::scale_stream_bytes(1, mx::down_ntiles((int)N), (int)K));
  L->total = o;
}

mx::WsPtrs ws_ptrs(void* base, const mxfp4_moe_workspace_layout& L) {
  uint8_t* b = static_cast<uint8_t*>(base);
  mx::WsPtrs w;
  w.status = reinterpret_cast<int*>(b + L.status);
  w.offsets = reinterpret_cast<int*>(b + L.expert_offsets);
  w.sorted_pairs = reinterpret_cast<int*>(b + L.sorted_pairs);
  w.inv = reinterpret_cast<int*>(b + L.inv_pairs);
  w.chunk_counts = reinterpret_cast<int*>(b + L.chunk_counts);
  w.chunk_ranks = reinterpret_cast<int*>(b + L.chunk_ranks);
  w.tiles = reinterpret_cast<int*>(b + L.tiles);
  w.x_codes = b + L.x_codes;
  w.h = b + L.h;
  w.h_codes = b + L.h_codes;
  w.y = reinterpret_cast<float*>(b + L.y);
  w.x_scales = b + L.x_scales;
  w.h_scales = b + L.h_scales;
  w.w13_stream = b + L.w13_scale_stream;
  w.w2_stream = b + L.w2_scale_stream;
  return w;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MXFP4_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// Fixed device scratch of mxfp4_moe_layer_noalloc: every device the library
// runs on holds one copy for the life of the process, shared by all calls on
// that device.  Host code never uses this name as an address: the device
// address of each device's copy comes from hipGetSymbolAddress (see
// scratch_ptr) and only that pointer is passed to kernels.
static __device__ __align__(256) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void*> g_scratch[64];

// Device address of the current device's scratch, looked up on the first call
// on that device (with that device current) and kept per device.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MXFP4_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MXFP4_E_DEVICE, "device index %d out of range", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MXFP4_E_HIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MXFP4_OK;
}

}  // namespace

extern "C" {

int mxfp4_abi_version(void) { return MXFP4_ABI_VERSION; }

const char* mxfp4_status_string(int status) {
  switch (status) {
    case MXFP4_OK: return "ok";
    case MXFP4_E_NULL: return "null pointer";
    case MXFP4_E_SHAPE: return "bad shape";
    case MXFP4_E_ALIGN: return "misaligned pointer";
    case MXFP4_E_MODE: return "unknown mode";
    case MXFP4_E_WORKSPACE: return "workspace too small";
    case MXFP4_E_DEVICE: return "unsupported or missing device";
    case MXFP4_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mxfp4_last_error(void) { return g_err; }

int mxfp4_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_weights, void* stream) {
  if (T < 0 || T > (1 << 24)) return fail(MXFP4_E_SHAPE, "T=%lld outside [0, 2^24]", (long long)T);
  if (E < 1 || E > 512) return fail(MXFP4_E_SHAPE, "E=%d outside [1, 512]", E);
  if (k < 1 || k > 16 || k > E) return fail(MXFP4_E_SHAPE, "k=%d outside [1, min(E, 16)]", k);
  if (T == 0) return ok();
  if (!logits || !topk_ids || !topk_weights) return fail(MXFP4_E_NULL, "route_topk: null pointer");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MXFP4_E_ALIGN, "route_topk: pointers must be 4-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = mx::launch_route_topk(logits, (int)T, E, k, topk_ids, topk_weights,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route_topk launch");
  return ok();
}

int mxfp4_moe_workspace_layout_query(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                                     int32_t act_mode, mxfp4_moe_workspace_layout* layout) {
  if (!layout) return fail(MXFP4_E_NULL, "layout is null");
  int rc = moe_shape_check(T, H, I, E, k, act_mode);
  if (rc) return rc;
  plan(T, H, I, E, k, act_mode, layout);
  return ok();
}

int mxfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                             int32_t act_mode, size_t* bytes) {
  if (!bytes) return fail(MXFP4_E_NULL, "bytes is null");
  mxfp4_moe_workspace_layout L;
  int rc = mxfp4_moe_workspace_layout_query(T, H, I, E, k, act_mode, &L);
  if (rc) return rc;
  *bytes = L.total_bytes;
  return ok();
}

namespace {

// The layer after validation of the shared arguments.  With `logits`, the
// router runs first (writing topk_ids / topk_weights); otherwise they are
// inputs.
int moe_run(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I, int32_t E,
            int32_t k, int32_t* topk_ids, float* topk_weights, const uint8_t* w13_blocks,
            const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_blocks,
            const uint8_t* w2_scales, const uint16_t* w2_bias, int32_t act_mode, uint16_t* out,
            void* workspace, size_t workspace_bytes, const mxfp4_moe_opts* opts, void* stream,
            const char* fn, const float* nv_globals = nullptr) {
  int rc = moe_shape_check(T, H, I, E, k, act_mode);
  if (rc) return rc;
  if (nv_globals) {
    if (act_mode == MXFP4_ACT_MXFP4)
      return fail(MXFP4_E_MODE, "%s: NVFP4 weights take bf16 or E4M3 activations", fn);
    if (!std::isfinite(nv_globals[0]) || !std::isfinite(nv_globals[1]))
      return fail(MXFP4_E_SHAPE, "%s: global scales must be finite", fn);
    if (act_mode == MXFP4_ACT_BF16) {
      if (H < 160 || I < 160 || H > 3072 || I > 3072)
        return fail(MXFP4_E_SHAPE, "%s: NVFP4 weights with bf16 activations need 160 <= H, I <= 3072", fn);
      if ((int64_t)T * k * (I > H ? I : H) * 2 >= (1LL << 31))
        return fail(MXFP4_E_SHAPE, "%s: NVFP4 weights with bf16 activations need T*k*max(H, I)*2 < 2^31", fn);
    }
  }
  if (T == 0) return ok();
  if (!x || !topk_ids || !topk_weights || !w13_blocks || !w13_scales || !w2_blocks ||
      !w2_scales || !out)
    return fail(MXFP4_E_NULL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w13_blocks, 16) ||
      !aligned(w2_blocks, 16) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(w13_scales, 4) || !aligned(w2_scales, 4) || (logits && !aligned(logits, 4)) ||
      (w13_bias && !aligned(w13_bias, 8)) || (w2_bias && !aligned(w2_bias, 8)))
    return fail(MXFP4_E_ALIGN, "%s: x/out/blocks need 16-byte, biases 8-byte, logits/ids/weights/scales 4-byte alignment", fn);
  if (opts && (!aligned(opts->w13_codes, 16) || !aligned(opts->w2_codes, 16)))
    return fail(MXFP4_E_ALIGN, "%s: restaged code streams need 16-byte alignment", fn);
  mxfp4_moe_workspace_layout L;
  plan(T, H, I, E, k, act_mode, &L, nv_globals != nullptr);
  if (!workspace) return fail(MXFP4_E_WORKSPACE, "workspace is null");
  if (!aligned(workspace, 256)) return fail(MXFP4_E_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total_bytes)
    return fail(MXFP4_E_WORKSPACE, "workspace %zu bytes < required %llu", workspace_bytes,
                (unsigned long long)L.total_bytes);
  rc = check_device();
  if (rc) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const mx::WsPtrs ws = ws_ptrs(workspace, L);
  const mx::MoeShape sh{(int)T, (int)H, (int)I, E, k};
  mx::MoeWeights w{w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias};
  if (nv_globals) {
    w.nvfp4 = true;
    w.w13_global = nv_globals[0];
    w.w2_global = nv_globals[1];
  }
  const bool fp8 = act_mode == MXFP4_ACT_FP8_E4M3;
  const bool a4 = act_mode == MXFP4_ACT_MXFP4;
  if ((fp8 || a4) && opts) {
    w.w13_codes = static_cast<const uint8_t*>(opts->w13_codes);
    w.w2_codes = static_cast<const uint8_t*>(opts->w2_codes);
  }
  const int64_t npairs = T * k;
  const int bm = act_mode == MXFP4_ACT_BF16 ? mx::kDecodeBM : mx::prefill_bm(npairs, E, nv_globals != nullptr);
  const int64_t bound = mx::max_tiles(npairs, E, bm);

  auto mark = [&](int stage) -> hipError_t {
    if (opts && opts->events[stage])
      return hipEventRecord(static_cast<hipEvent_t>(opts->events[stage]), s);
    return hipSuccess;
  };
  hipError_t e;
#define MX_STEP(call, what)                      \
  do {                                           \
    e = (call);                                  \
    if (e != hipSuccess) return hip_fail(e, what); \
  } while (0)

  MX_STEP(mark(MXFP4_STAGE_BEGIN), "event record");
  // decode batches with bf16 activations: the gate_up kernel routes the batch
  // itself (no route + permutation launch; the permute stage is then empty)
  const bool route_in_gateup = logits && act_mode == MXFP4_ACT_BF16 && !nv_globals &&
                               mx::gateup_routes_batch(sh, false);
  // one launch for route + permute while the block routes the whole batch in
  // one round (a half wave per token)
  if (route_in_gateup) {
    // (routed in the gate_up launch below)
  } else if (logits && T <= mx::kFusedRouteMaxTokens && npairs <= mx::kFusedPermuteMaxPairs) {
    MX_STEP(mx::launch_route_permute(logits, (int)T, E, k, topk_ids, topk_weights, bm, (int)bound, ws, s),
            "route+permute launch");
  } else {
    if (logits) MX_STEP(mx::launch_route_topk(logits, (int)T, E, k, topk_ids, topk_weights, s), "route launch");
    MX_STEP(mx::launch_permute(topk_ids, (int)npairs, E, bm, (int)bound, ws, s), "permute launch");
  }
  MX_STEP(mark(MXFP4_STAGE_PERMUTE), "event record");
  if (fp8) {
    // per-tensor scale over all of x, codes written in expert-sorted row order
    MX_STEP(mx::launch_amax(x, true, T * H, reinterpret_cast<uint32_t*>(ws.status + mx::kStAmaxX), s),
            "amax x launch");
    MX_STEP(mx::launch_encode_sorted_rows(x, sh, ws, s), "quant x launch");
  } else if (a4) {
    MX_STEP(mx::launch_quant_x_mxfp4_sorted(x, sh, ws, s), "quant x launch");
  }
  const bool restage = (fp8 || a4) && !(opts && (opts->flags & MXFP4_OPT_SCALE_STREAMS_READY));
  if (restage) MX_STEP(mx::launch_scale_stream(sh, w, ws, true, s), "w13 scale stream launch");
  MX_STEP(mark(MXFP4_STAGE_QUANT_X), "event record");
  if (fp8) MX_STEP(mx::launch_moe_gateup_fp8(sh, w, ws, bound, s), "gate_up launch");
  else if (a4) MX_STEP(mx::launch_moe_gateup_fp4(sh, w, ws, s), "gate_up launch");
  else if (route_in_gateup)
    MX_STEP(mx::launch_moe_gateup_bf16_routed(x, logits, topk_ids, topk_weights, sh, w, ws, bound, s),
            "gate_up launch");
  else MX_STEP(mx::launch_moe_gateup_bf16(x, sh, w, ws, bound, s), "gate_up launch");
  MX_STEP(mark(MXFP4_STAGE_GEMM1), "event record");
  if (fp8) {
    MX_STEP(mx::launch_encode_fp8_rows(ws.h, false, npairs, I, mx::code_row_bytes(I, false), ws.h_codes,
                                       reinterpret_cast<const uint32_t*>(ws.status + mx::kStAmaxH),
                                       reinterpret_cast<float*>(ws.status + mx::kStScaleH), s),
            "quant h launch");
  }
  if (restage) MX_STEP(mx::launch_scale_stream(sh, w, ws, false, s), "w2 scale stream launch");
  MX_STEP(mark(MXFP4_STAGE_QUANT_H), "event record");
  if (fp8) MX_STEP(mx::launch_moe_down_fp8(sh, w, ws, bound, s), "down launch");
  else if (a4) MX_STEP(mx::launch_moe_down_fp4(sh, w, ws, s), "down launch");
  else MX_STEP(mx::launch_moe_down_bf16(sh, w, ws, bound, s), "down launch");
  MX_STEP(mark(MXFP4_STAGE_GEMM2), "event record");
  MX_STEP(mx::launch_combine(sh, topk_weights, ws, out, s), "combine launch");
  MX_STEP(mark(MXFP4_STAGE_COMBINE), "event record");
#undef MX_STEP
  return ok();
}

}  // namespace

int mxfp4_moe_forward(const uint16_t* x, int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                      const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13_blocks, const uint8_t* w13_scales,
                      const uint16_t* w13_bias, const uint8_t* w2_blocks,
                      const uint8_t* w2_scales, const uint16_t* w2_bias, int32_t act_mode,
                      uint16_t* out, void* workspace, size_t workspace_bytes,
                      const mxfp4_moe_opts* opts, void* stream) {
  return moe_run(x, nullptr, T, H, I, E, k, const_cast<int32_t*>(topk_ids),
                 const_cast<float*>(topk_weights), w13_blocks, w13_scales, w13_bias, w2_blocks,
                 w2_scales, w2_bias, act_mode, out, workspace, workspace_bytes, opts, stream,
                 "moe_forward");
}

int mxfp4_moe_layer(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I,
                    int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                    const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                    const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias,
                    int32_t act_mode, uint16_t* out, void* workspace, size_t workspace_bytes,
                    const mxfp4_moe_opts* opts, void* stream) {
  if (T > 0 && !logits) return fail(MXFP4_E_NULL, "moe_layer: logits is null");
  return moe_run(x, logits, T, H, I, E, k, topk_ids, topk_weights, w13_blocks, w13_scales, w13_bias,
                 w2_blocks, w2_scales, w2_bias, act_mode, out, workspace, workspace_bytes, opts,
                 stream, "moe_layer");
}

int mxfp4_moe_layer_noalloc(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I,
                            int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                            const uint8_t* w13_blocks, const uint8_t* w13_scales,
                            const uint16_t* w13_bias, const uint8_t* w2_blocks,
                            const uint8_t* w2_scales, const uint16_t* w2_bias, int32_t act_mode,
                            uint16_t* out, const mxfp4_moe_opts* opts, void* stream) {
  if (T > 0 && !logits) return fail(MXFP4_E_NULL, "moe_layer_noalloc: logits is null");
  int rc = moe_shape_check(T, H, I, E, k, act_mode);
  if (rc) return rc;
  mxfp4_moe_workspace_layout L;
  plan(T, H, I, E, k, act_mode, &L);
  if (L.total_bytes > MXFP4_NOALLOC_SCRATCH_BYTES)
    return fail(MXFP4_E_WORKSPACE,
                "moe_layer_noalloc: these sizes need %llu bytes of scratch; the fixed scratch holds %llu "
                "(use mxfp4_moe_layer with a workspace)",
                (unsigned long long)L.total_bytes, (unsigned long long)MXFP4_NOALLOC_SCRATCH_BYTES);
  if (T == 0) return ok();
  rc = check_device();
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc) return rc;
  // restaged scale streams in the shared scratch may belong to another call:
  // always restage
  mxfp4_moe_opts o;
  if (opts) {
    o = *opts;
    o.flags &= ~(uint32_t)MXFP4_OPT_SCALE_STREAMS_READY;
  }
  return moe_run(x, logits, T, H, I, E, k, topk_ids, topk_weights, w13_blocks, w13_scales, w13_bias,
                 w2_blocks, w2_scales, w2_bias, act_mode, out, ws, MXFP4_NOALLOC_SCRATCH_BYTES,
                 opts ? &o : nullptr, stream, "moe_layer_noalloc");
}

int nvfp4_moe_forward(const uint16_t* x, int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                      const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13_blocks, const uint8_t* w13_scales, float w13_global,
                      const uint16_t* w13_bias, const uint8_t* w2_blocks, const uint8_t* w2_scales,
                      float w2_global, const uint16_t* w2_bias, int32_t act_mode, uint16_t* out,
                      void* workspace, size_t workspace_bytes, const mxfp4_moe_opts* opts, void* stream) {
  const float g[2] = {w13_global, w2_global};
  return moe_run(x, nullptr, T, H, I, E, k, const_cast<int32_t*>(topk_ids),
                 const_cast<float*>(topk_weights), w13_blocks, w13_scales, w13_bias, w2_blocks,
                 w2_scales, w2_bias, act_mode, out, workspace, workspace_bytes, opts, stream,
                 "nvfp4_moe_forward", g);
}

int nvfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, int32_t act_mode,
                             size_t* bytes) {
  if (!bytes) return fail(MXFP4_E_NULL, "bytes is null");
  int rc = moe_shape_check(T, H, I, E, k, act_mode);
  if (rc) return rc;
  if (act_mode == MXFP4_ACT_MXFP4)
    return fail(MXFP4_E_MODE, "nvfp4_moe_workspace_size: NVFP4 weights take bf16 or E4M3 activations");
  mxfp4_moe_workspace_layout L;
  plan(T, H, I, E, k, act_mode, &L, true);
  *bytes = L.total_bytes;
  return ok();
}

int mxfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t act_mode, size_t* bytes) {
  if (!bytes) return fail(MXFP4_E_NULL, "bytes is null");
  int rc = linear_shape_check(M, N, K, act_mode);
  if (rc) return rc;
  LinearLayout L;
  linear_plan(M, N, K, act_mode, &L);
  *bytes = L.total;
  return ok();
}

int mxfp4_linear(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_blocks,
                 const uint8_t* w_scales, const uint16_t* bias, int32_t act_mode, uint16_t* out,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = linear_shape_check(M, N, K, act_mode);
  if (rc) return rc;
  if (M == 0) return ok();
  if (!x || !w_blocks || !w_scales || !out) return fail(MXFP4_E_NULL, "linear: null pointer");
  if (!aligned(x, 16) || !aligned(w_blocks, 16) || !aligned(out, 16) || !aligned(w_scales, 4) ||
      (bias && !aligned(bias, 8)))
    return fail(MXFP4_E_ALIGN, "linear: x, w_blocks and out need 16-byte, bias 8-byte, w_scales 4-byte alignment");
  LinearLayout L;
  linear_plan(M, N, K, act_mode, &L);
  if (L.total) {
    if (!workspace) return fail(MXFP4_E_WORKSPACE, "linear: workspace is null");
    if (!aligned(workspace, 256)) return fail(MXFP4_E_ALIGN, "linear: workspace must be 256-byte aligned");
    if (workspace_bytes < L.total)
      return fail(MXFP4_E_WORKSPACE, "linear: workspace %zu bytes < required %llu", workspace_bytes,
                  (unsigned long long)L.total);
  }
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (act_mode == MXFP4_ACT_BF16) {
    e = mx::launch_linear_bf16(x, (int)M, (int)N, (int)K, w_blocks, w_scales, bias, out, s);
    if (e != hipSuccess) return hip_fail(e, "linear launch");
    return ok();
  }
  // quantised activations: the MoE down GEMM with one expert whose rows are
  // the M activation rows in order, written straight to bf16
  const bool a4 = act_mode == MXFP4_ACT_MXFP4;
  uint8_t* b = static_cast<uint8_t*>(workspace);
  mx::WsPtrs ws{};
  ws.status = reinterpret_cast<int*>(b + L.status);
  ws.tiles = reinterpret_cast<int*>(b + L.tiles);
  ws.inv = a4 ? reinterpret_cast<int*>(b + L.inv) : nullptr;
  ws.x_codes = ws.h_codes = b + L.codes;
  ws.x_scales = ws.h_scales = a4 ? b + L.scales : nullptr;
  ws.w2_stream = b + L.w_stream;
  const mx::MoeShape sh{(int)M, (int)N, (int)K, 1, 1};
  mx::MoeWeights w{};
  w.w2_blocks = w_blocks;
  w.w2_scales = w_scales;
  w.w2_bias = bias;
  const int bm = mx::kPrefillBM;
  const int64_t bound = mx::max_tiles(M, 1, bm);
#define MX_STEP(call, what)                      \
  do {                                           \
    e = (call);                                  \
    if (e != hipSuccess) return hip_fail(e, what); \
  } while (0)
  MX_STEP(mx::launch_dense_tiles((int)M, bm, (int)bound, ws.status, ws.tiles, ws.inv, s),
          "linear tiles launch");
  if (a4) {
    // per-row 32-element blocks of x (the rows' K is the quantiser's H)
    const mx::MoeShape shq{(int)M, (int)K, (int)N, 1, 1};
    MX_STEP(mx::launch_quant_x_mxfp4_sorted(x, shq, ws, s), "linear quant x launch");
  } else {
    MX_STEP(mx::launch_quant_fp8_rows(x, true, M, K, mx::code_row_bytes(K, false), ws.h_codes,
                                      reinterpret_cast<uint32_t*>(ws.status + mx::kStAmaxH),
                                      reinterpret_cast<float*>(ws.status + mx::kStScaleH), s),
            "linear quant x launch");
  }
  MX_STEP(mx::launch_scale_stream(sh, w, ws, false, s), "linear scale stream launch");
  if (a4) MX_STEP(mx::launch_moe_down_fp4(sh, w, ws, s, out), "linear GEMM launch");
  else MX_STEP(mx::launch_moe_down_fp8(sh, w, ws, bound, s, out), "linear GEMM launch");
#undef MX_STEP
  return ok();
}

int mxfp4_quant_fp8_e4m3(const void* in, int32_t in_dtype, int64_t n, uint8_t* codes, float* scale,
                         float* amax, void* stream) {
  if (in_dtype != 0 && in_dtype != 1) return fail(MXFP4_E_MODE, "unknown in_dtype %d", in_dtype);
  if (n < 0 || n > (1LL << 40)) return fail(MXFP4_E_SHAPE, "n=%lld out of range", (long long)n);
  if (!scale || !amax) return fail(MXFP4_E_NULL, "quant: scale/amax null");
  if (n > 0 && (!in || !codes)) return fail(MXFP4_E_NULL, "quant: null pointer");
  if (!aligned(in, 16) || !aligned(codes, 16) || !aligned(scale, 4) || !aligned(amax, 4))
    return fail(MXFP4_E_ALIGN, "quant: in/codes need 16-byte alignment");
  int rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mx::launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 0u, 1, s);
  if (e != hipSuccess) return hip_fail(e, "quant init");
  e = mx::launch_quant_fp8(in, in_dtype == 1, n, codes, reinterpret_cast<uint32_t*>(amax), scale, s);
  if (e != hipSuccess) return hip_fail(e, "quant launch");
  return ok();
}

int mxfp4_quantize_weights(const uint16_t* w, int64_t N, int64_t K, uint8_t* blocks,
                           uint8_t* scales, void* stream) {
  if (K <= 0 || K % 32) return fail(MXFP4_E_SHAPE, "K=%lld must be a positive multiple of 32", (long long)K);
  if (N < 0 || (N > 0 && N > (1LL << 40) / K)) return fail(MXFP4_E_SHAPE, "N=%lld out of range", (long long)N);
  if (N == 0) return ok();
  if (!w || !blocks || !scales) return fail(MXFP4_E_NULL, "quantize_weights: null pointer");
  if (!aligned(w, 16) || !aligned(blocks, 16))
    return fail(MXFP4_E_ALIGN, "quantize_weights: w and blocks need 16-byte alignment");
  int rc = check_device();
  if (rc) return rc;
  const hipError_t e = mx::launch_quant_mxfp4(w, N * (K / 32), blocks, scales, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize_weights launch");
  return ok();
}

namespace {
// rows, K and row tiles of one expert tensor (which: 0 w13, 1 w2)
void code_stream_shape(int64_t H, int64_t I, int32_t which, int& R, int& nout, int& K, int& tiles) {
  const bool gu = which == 0;
  R = (int)(gu ? 2 * I : H);
  nout = (int)(gu ? I : H);
  K = (int)(gu ? H : I);
  tiles = gu ? (nout + 127) / 128 : (nout + 255) / 256;
}
int code_stream_check(int64_t H, int64_t I, int32_t E, int32_t which, const char* fn) {
  if (which != 0 && which != 1) return fail(MXFP4_E_MODE, "%s: which must be 0 (w13) or 1 (w2)", fn);
  if (H <= 0 || I <= 0 || H % 32 || I % 32 || H > 65536 || I > 65536)
    return fail(MXFP4_E_SHAPE, "%s: H, I must be positive multiples of 32 up to 65536", fn);
  if (E < 1 || E > 512) return fail(MXFP4_E_SHAPE, "%s: E=%d out of [1, 512]", fn, E);
  return MXFP4_OK;
}
}  // namespace

int mxfp4_moe_code_stream_size(int64_t H, int64_t I, int32_t E, int32_t which, size_t* bytes) {
  int rc = code_stream_check(H, I, E, which, "code_stream_size");
  if (rc) return rc;
  if (!bytes) return fail(MXFP4_E_NULL, "code_stream_size: bytes is null");
  int R, nout, K, tiles;
  code_stream_shape(H, I, which, R, nout, K, tiles);
  *bytes = (size_t)mx::code_stream_bytes(E, tiles, K);
  return ok();
}

int mxfp4_moe_prepare_code_stream(const uint8_t* blocks, int64_t H, int64_t I, int32_t E, int32_t which,
                                  void* out, size_t out_bytes, void* stream) {
  int rc = code_stream_check(H, I, E, which, "prepare_code_stream");
  if (rc) return rc;
  if (!blocks || !out) return fail(MXFP4_E_NULL, "prepare_code_stream: null pointer");
  if (!aligned(blocks, 16) || !aligned(out, 16))
    return fail(MXFP4_E_ALIGN, "prepare_code_stream: blocks and out need 16-byte alignment");
  int R, nout, K, tiles;
  code_stream_shape(H, I, which, R, nout, K, tiles);
  const int64_t need = mx::code_stream_bytes(E, tiles, K);
  if ((int64_t)out_bytes < need)
    return fail(MXFP4_E_WORKSPACE, "prepare_code_stream: out %zu bytes < required %lld", out_bytes, (long long)need);
  rc = check_device();
  if (rc) return rc;
  const hipError_t e = mx::launch_code_stream(blocks, E, R, nout, K, which == 0, static_cast<uint8_t*>(out),
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prepare_code_stream launch");
  return ok();
}

int mxfp4_stream_read(const void* buf, uint64_t bytes, int32_t mode, uint32_t* sink,
                      uint64_t* bytes_read, void* stream) {
  if (mode != 0 && mode != 1) return fail(MXFP4_E_MODE, "stream_read: unknown mode %d", mode);
  if (!bytes_read) return fail(MXFP4_E_NULL, "stream_read: bytes_read is null");
  if (bytes > (1ULL << 40)) return fail(MXFP4_E_SHAPE, "stream_read: %llu bytes out of range",
                                        (unsigned long long)bytes);
  if (bytes > 0 && (!buf || !sink)) return fail(MXFP4_E_NULL, "stream_read: null pointer");
  if (!aligned(buf, 1024) || !aligned(sink, 4))
    return fail(MXFP4_E_ALIGN, "stream_read: buf needs 1024-byte, sink 4-byte alignment");
  int rc = check_device();
  if (rc) return rc;
  *bytes_read = (uint64_t)mx::stream_read_bytes((int64_t)bytes);
  if (*bytes_read == 0) return ok();
  hipError_t e = mx::launch_stream_read(buf, (int64_t)bytes, mode == 1, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  return ok();
}

int mxfp4_event_create(void** event) {
  if (!event) return fail(MXFP4_E_NULL, "event is null");
  hipEvent_t ev;
  hipError_t e = hipEventCreate(&ev);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  *event = ev;
  return ok();
}

int mxfp4_event_destroy(void* event) {
  if (!event) return fail(MXFP4_E_NULL, "event is null");
  hipError_t e = hipEventDestroy(static_cast<hipEvent_t>(event));
  if (e != hipSuccess) return hip_fail(e, "hipEventDestroy");
  return ok();
}

int mxfp4_event_elapsed_ms(void* start, void* end, float* ms) {
  if (!start || !end || !ms) return fail(MXFP4_E_NULL, "event/ms is null");
  hipError_t e = hipEventSynchronize(static_cast<hipEvent_t>(end));
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  e = hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(end));
  if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  return ok();
}

}  // extern "C"
