/*
 * mxfp4_moe.h - C ABI of the MI355X (gfx950) MXFP4 block-scaled MoE layer and
 * dense projections.
 *
 * What is computed (source pages):
 *   - Weights are MXFP4 as the gpt-oss page describes them in "MXFP4 Tensor
 *     Structure": *_blocks uint8 [E, N, K/32, 16] hold two E2M1 codes per
 *     byte (32 elements per 16-byte block), *_scales uint8 [E, N, K/32] one
 *     E8M0 power-of-two scale per block with bias 127, *_bias bfloat16.  An
 *     element's value is E2M1(code) * 2^(scale - 127) ("Conversion
 *     Methodology", step 1).  Element 2i of a block sits in the low nibble of
 *     byte i, element 2i+1 in its high nibble.
 *   - The MoE layer of gpt-oss-120b ("GPT-OSS-120B Architecture": 128
 *     experts, 4 active per token, hidden 2880) run as an FP8 x FP4 grouped
 *     GEMM (spark-vllm page, "What's Included") or, for small token counts,
 *     with bf16 activations; dense MXFP4 qkv_proj, o_proj and lm_head
 *     (spark-vllm page, full MXFP4 stack; gptoss-spark page, "What produced
 *     it, ranked").
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major
 *     and contiguous.  bfloat16 is passed as uint16_t bit patterns.  `stream`
 *     is a hipStream_t (NULL = the default stream).
 *   - Calls are asynchronous: they validate, enqueue kernels on `stream` and
 *     return.  Faults inside kernels surface at the caller's next
 *     synchronisation of the stream.
 *   - Validation is complete before anything is enqueued: on any non-zero
 *     return nothing has been launched and no output has been written.
 *   - The library allocates no device memory; scratch comes from the caller's
 *     `workspace`, sized with mxfp4_moe_workspace_size().
 *   - No C++ exception crosses this boundary.  Functions are thread-safe; the
 *     only state is a per-device cache of the architecture check and a
 *     thread-local error message.
 *   - Only gfx950 devices are accepted (MXFP4_E_DEVICE otherwise).
 */
#ifndef MXFP4_MOE_H
#define MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP4_ABI_VERSION 5

/* Status codes.  0 is success; every failure leaves outputs untouched. */
enum {
  MXFP4_OK = 0,
  MXFP4_E_NULL = 1,      /* a required pointer is NULL */
  MXFP4_E_SHAPE = 2,     /* bad size: K/H/I not a positive multiple of 32, k > E, ... */
  MXFP4_E_ALIGN = 3,     /* a pointer is not aligned as documented */
  MXFP4_E_MODE = 4,      /* unknown enum value (never silently ignored) */
  MXFP4_E_WORKSPACE = 5, /* workspace NULL or smaller than required */
  MXFP4_E_DEVICE = 6,    /* no HIP device, or the current device is not gfx950 */
  MXFP4_E_HIP = 7        /* a HIP runtime call or kernel launch failed */
};

/* Activation precision of the MoE contraction. */
enum {
  MXFP4_ACT_BF16 = 0,         /* x used as given (bf16), fp32 accumulation */
  MXFP4_ACT_FP8_E4M3 = 1,     /* x and the SwiGLU output h each quantised to
                                 OCP FP8 E4M3 with one per-tensor fp32 scale
                                 amax/448; FP8 x FP4 block-scaled MFMA */
  MXFP4_ACT_MXFP4 = 2         /* x and h each quantised to MXFP4 (E2M1 codes,
                                 one E8M0 scale per 32-element block of a
                                 row); FP4 x FP4 block-scaled MFMA (the
                                 native FP4 x FP4 contraction the spark-vllm
                                 page lists under "Performance
                                 Optimizations") */
};

/* Stage boundaries at which mxfp4_moe_forward can record caller events. */
enum {
  MXFP4_STAGE_BEGIN = 0,      /* before the first kernel */
  MXFP4_STAGE_PERMUTE = 1,    /* after the token-by-expert permutation (in
                                 mxfp4_moe_layer with bf16 activations and at
                                 most 8 tokens the gate_up kernel routes the
                                 batch itself: this stage is then empty and
                                 GEMM1 includes the routing) */
  MXFP4_STAGE_QUANT_X = 2,    /* after quantisation of x and the restaging of the
                                 w13 scales (FP8, MXFP4 activations) */
  MXFP4_STAGE_GEMM1 = 3,      /* after gate_up GEMM + SwiGLU */
  MXFP4_STAGE_QUANT_H = 4,    /* after quantisation of h and the restaging of the
                                 w2 scales (FP8, MXFP4 activations) */
  MXFP4_STAGE_GEMM2 = 5,      /* after the down GEMM */
  MXFP4_STAGE_COMBINE = 6,    /* after the weighted combine (end) */
  MXFP4_NUM_STAGES = 7
};

/* Bits of mxfp4_moe_opts.flags. */
enum {
  /* FP8 and MXFP4-activation modes: the workspace already holds the restaged
     weight scales (w13_scale_stream, w2_scale_stream) of exactly these
     w13_scales / w2_scales, written by an earlier call with the same weights,
     shapes, act_mode and workspace, and not overwritten since; the restaging
     is skipped.  For callers whose weights stay fixed (prepared once, as a
     load-time step).  Ignored in BF16 mode.  If the promise does not hold the
     result is undefined (but every access stays inside the workspace). */
  MXFP4_OPT_SCALE_STREAMS_READY = 1
};

/* Optional per-call options for mxfp4_moe_forward (pass NULL for none). */
typedef struct {
  /* events[i], if non-NULL, is a hipEvent_t recorded on `stream` at stage
     boundary i (0 <= i < MXFP4_NUM_STAGES).  Used for per-kernel timing. */
  void* events[MXFP4_NUM_STAGES];
  uint32_t flags;             /* MXFP4_OPT_* bits; 0 for none */
  /* FP8 and MXFP4-activation modes: NULL, or the E2M1 codes of w13_blocks /
     w2_blocks restaged by mxfp4_moe_prepare_code_stream for exactly these
     weights and shapes (16-byte aligned); the prefill GEMMs then copy the
     codes from there (contiguous 16 KB per tile and step) instead of the
     blocks.  The results are bitwise those without them.  Ignored in BF16
     mode.  A stale or foreign stream gives undefined results (every access
     stays inside the stream's mxfp4_moe_code_stream_size bytes). */
  const void* w13_codes;
  const void* w2_codes;
} mxfp4_moe_opts;

/* Byte offsets of the intermediate results inside the MoE workspace, for
   inspection by tests and profilers (all offsets are 256-byte aligned). */
typedef struct {
  uint64_t total_bytes;
  uint64_t status;          /* int32[16]: [0] error flags (bit 0: an expert id was
                               outside [0,E) and its pair was skipped),
                               [1] amax(x) fp32 bits, [2] amax(h) fp32 bits,
                               [3] x scale fp32 bits, [4] h scale fp32 bits,
                               [5] number of row tiles */
  uint64_t expert_offsets;  /* int32 [E+1]: sorted rows of expert e are
                               [offsets[e], offsets[e+1]) */
  uint64_t sorted_pairs;    /* int32 [T*k]: pair index p = t*k + j per sorted row,
                               ascending p within an expert */
  uint64_t inv_pairs;       /* int32 [T*k]: sorted row of pair p */
  uint64_t chunk_counts;    /* int32 scratch of the permutation */
  uint64_t chunk_ranks;     /* int32 scratch of the permutation */
  uint64_t tiles;           /* int32 [4 * max_tiles]: (expert, first sorted row, end row, 0);
                               entries past the tile count have expert -1 */
  uint64_t x_codes;         /* FP8 mode: uint8 [T*k, H] E4M3 codes of x in sorted
                               row order: row r holds token sorted_pairs[r] / k
                               (rows past expert_offsets[E] unused);
                               MXFP4-activation mode: uint8 [T*k, H/32, 16]
                               E2M1 blocks of x in the same row order.  Rows
                               are padded to whole 128-byte lines: row r starts
                               at r * ceil(H / 128) * 128 bytes (FP8) or
                               r * ceil(H / 256) * 128 (E2M1); pad bytes are
                               unspecified */
  uint64_t h;               /* BF16 mode: bf16 hi [T*k, I] then bf16 lo [T*k, I]
                               with h = hi + lo; FP8 mode: fp32 [T*k, I]; rows
                               in sorted order.  MXFP4-activation mode: no
                               bytes (h is quantised in the gate_up GEMM) */
  uint64_t h_codes;         /* FP8 mode: uint8 [T*k, I] E4M3 codes of h;
                               MXFP4-activation mode: uint8 [T*k, I/32, 16]
                               E2M1 blocks of h; rows padded as in x_codes
                               (with I for H) */
  uint64_t y;               /* fp32 [T*k, H] per-pair expert outputs, sorted rows */
  uint64_t x_scales;        /* MXFP4-activation mode: uint8 [ceil(H/128), T*k, 4]
                               E8M0 scales of the x blocks, step-major: block b
                               of sorted row r at ((b/4)*T*k + r)*4 + b%4;
                               bytes of blocks past H/32 hold 127; 0 in the
                               other modes */
  uint64_t h_scales;        /* MXFP4-activation mode: uint8 [ceil(I/128), T*k, 4]
                               E8M0 scales of the h blocks, likewise; 0 in the
                               other modes */
  uint64_t w13_scale_stream; /* FP8 and MXFP4-activation modes: the w13 E8M0
                               scales restaged in the order the prefill GEMM
                               copies them (internal layout); 0 in BF16 mode */
  uint64_t w2_scale_stream; /* the same for w2 */
} mxfp4_moe_workspace_layout;

/*
 * Load-time restaging of an expert weight tensor's E2M1 codes for the prefill
 * GEMMs (E4M3 and MXFP4 activations).  Not a step of the method: a layout of
 * this library, for callers whose weights stay fixed.  The GEMMs read each
 * weight tile 64 bytes per row and 128-element step (rows 1440 bytes apart at
 * the gpt-oss shape), which the memory system serves at about two thirds of
 * the rate of contiguous reads; restaged, a tile's step is one contiguous
 * 16 KB chunk.  For expert e, row tile nt (gate_up: 128 gate rows and the
 * matching 128 up rows; down: 256 rows) and step s, the chunk holds for each
 * of the tile's 256 rows 64 bytes: four 16-byte blocks of 32 codes, blocks
 * 4s..4s+3 of the row in an order of this library, zeros past K.
 *   which   0: w13 (E x 2I rows of H codes, gate rows [0, I) then up rows),
 *           1: w2 (E x H rows of I codes)
 *   blocks  the codes as mxfp4_moe_forward takes them ([E, R, K/32, 16]) or as
 *           nvfp4_moe_forward takes them ([E, R, K/16, 8]): the same K/2
 *           bytes per row; 16-byte aligned
 *   out     mxfp4_moe_code_stream_size() bytes, 16-byte aligned, caller-owned
 * Limits: H, I positive multiples of 32 (<= 65536); 1 <= E <= 512.  The size:
 * E * ceil(rows / 256) * ceil(K / 128) * 16 KB (gate_up counts ceil(I / 128)
 * tiles), about 4.5% above the blocks at the gpt-oss shape.
 */
int mxfp4_moe_code_stream_size(int64_t H, int64_t I, int32_t E, int32_t which, size_t* bytes);
int mxfp4_moe_prepare_code_stream(const uint8_t* blocks, int64_t H, int64_t I, int32_t E, int32_t which,
                                  void* out, size_t out_bytes, void* stream);

/* Library ABI version (MXFP4_ABI_VERSION of the compiled library). */
int mxfp4_abi_version(void);

/* Static text for a status code. */
const char* mxfp4_status_string(int status);

/* Detail text of the last failing call on this thread ("" if none). */
const char* mxfp4_last_error(void);

/*
 * Router top-k (gpt-oss page, "GPT-OSS-120B Architecture": 4 of 128 experts
 * per token).  For each token t: ids are the k experts with the largest fp32
 * logit, in descending logit order, equal logits going to the lower index
 * (-0 equals +0); weights are the softmax over the k chosen logits, in fp32.
 *   logits        fp32 [T, E]           input (NaN logits are not supported)
 *   topk_ids      int32 [T, k]          output
 *   topk_weights  fp32 [T, k]           output
 * Limits: 1 <= E <= 512, 1 <= k <= min(E, 16), T >= 0 (T == 0 is a no-op).
 * Alignment: 4 bytes for every pointer.
 */
int mxfp4_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_weights, void* stream);

/* Workspace bytes mxfp4_moe_forward needs for these sizes (written to *bytes). */
int mxfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                             int32_t act_mode, size_t* bytes);

/* Offsets of the intermediates inside that workspace (see the struct). */
int mxfp4_moe_workspace_layout_query(int64_t T, int64_t H, int64_t I, int32_t E,
                                     int32_t k, int32_t act_mode,
                                     mxfp4_moe_workspace_layout* layout);

/*
 * One MoE layer (gpt-oss page, "GPT-OSS-120B Architecture" and "MXFP4 Tensor
 * Structure"; spark-vllm page, FP8 x FP4 grouped GEMM).  For each token t and
 * slot j, with e = topk_ids[t, j]:
 *     g      = W13[e] a_t + b13[e]                 (2I values)
 *     h      = silu(g[0:I]) * g[I:2I],  silu(z) = z / (1 + exp(-z))
 *     y[t,j] = W2[e] h' + b2[e]                    (H values)
 *     out[t] = sum_j topk_weights[t, j] * y[t, j]  (fp32, j ascending, then one
 *                                                   round-to-nearest-even to bf16)
 * where a_t = x_t and h' = h in MXFP4_ACT_BF16 mode; in MXFP4_ACT_FP8_E4M3
 * mode a_t and h' are the E4M3-dequantised values with per-tensor scales
 * s = fp32(amax/448) computed over all of x, and over all T*k*I values of h,
 * codes = E4M3 round-to-nearest-even, saturating, of the correctly rounded
 * fp32 quotient v / s.  In MXFP4_ACT_MXFP4 mode a_t and h' are the
 * MXFP4-dequantised values, each 32-element block of a row of x (and of each
 * pair's fp32 h) quantised on its own: shared exponent X = floor(log2 amax)
 * - 2 clamped to [-116, 125], codes = the E2M1 value nearest to |v| / 2^X
 * (ties to the even code, saturating at 6), sign kept (the rule of
 * mxfp4_quantize_weights).  W13 rows [0, I) are the gate rows, [I, 2I) the up
 * rows.
 *
 *   x            bf16 [T, H]                 16-byte aligned
 *   topk_ids     int32 [T, k]                values in [0, E); a pair with an
 *                                            id outside is skipped (contributes
 *                                            0) and status bit 0 is set
 *   topk_weights fp32 [T, k]
 *   w13_blocks   uint8 [E, 2I, H/32, 16]     16-byte aligned
 *   w13_scales   uint8 [E, 2I, H/32]      4-byte aligned
 *   w13_bias     bf16 [E, 2I] or NULL (zero bias), 8-byte aligned
 *   w2_blocks    uint8 [E, H, I/32, 16]      16-byte aligned
 *   w2_scales    uint8 [E, H, I/32]       4-byte aligned
 *   w2_bias      bf16 [E, H] or NULL, 8-byte aligned
 *   act_mode     MXFP4_ACT_BF16, MXFP4_ACT_FP8_E4M3 or MXFP4_ACT_MXFP4
 *   out          bf16 [T, H]                 16-byte aligned, must not alias
 *                                            any input or the workspace
 *   workspace    >= mxfp4_moe_workspace_size() bytes, 256-byte aligned
 *   opts         NULL or per-call options (stage events)
 * Limits: H, I positive multiples of 32 (<= 65536); 1 <= E <= 512;
 * 1 <= k <= min(E, 16); 0 <= T <= 2^22 (T == 0 is a no-op).
 * E8M0 scale bytes (the gpt-oss page's range is 2^-127 .. 2^127; 255 is not a
 * scale in any mode):
 *   - MXFP4_ACT_BF16 and MXFP4_ACT_FP8_E4M3: bytes in [11, 252] for w13
 *     and w2.  These paths form each weight in bf16 with the hardware's
 *     scaled FP4 conversion, which is exact for bytes 11..252 only (measured
 *     on gfx950: for a byte s <= 10 it gives E2M1 * (2^s + 3) * 2^-127, and
 *     253, 254 overflow bf16 at 6 * 2^126).  In FP8 mode the sums are
 *     moreover taken over the E4M3 codes (up to 448) and the per-tensor
 *     scales applied after them, so a row whose sum of |weight| * 448
 *     exceeds the fp32 range overflows even where the scaled result would not
 *     (with K = 2880 this needs weights of magnitude 2^104 or more).
 *   - MXFP4_ACT_MXFP4: every byte except 255 (the block-scaled MFMA applies
 *     both operands' E8M0 scales itself).
 * Bytes outside these ranges are not rejected (that would need a pass over
 * the scales on every call); the result is then undefined.  The same holds
 * for NaN or infinite bf16 values in x or the biases.
 */
int mxfp4_moe_forward(const uint16_t* x, int64_t T, int64_t H, int64_t I, int32_t E,
                      int32_t k, const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13_blocks, const uint8_t* w13_scales,
                      const uint16_t* w13_bias, const uint8_t* w2_blocks,
                      const uint8_t* w2_scales, const uint16_t* w2_bias,
                      int32_t act_mode, uint16_t* out, void* workspace,
                      size_t workspace_bytes, const mxfp4_moe_opts* opts, void* stream);

/*
 * The router and the layer in one call: mxfp4_route_topk on `logits` (fp32
 * [T, E], 4-byte aligned) writing topk_ids / topk_weights (outputs here, same
 * layout and values as mxfp4_route_topk), then mxfp4_moe_forward on them, on
 * one stream in one call.  Every other
 * argument, limit and error is that of mxfp4_moe_forward; the result is
 * bitwise the same as the two calls in sequence.
 */
int mxfp4_moe_layer(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I,
                    int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                    const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                    const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias,
                    int32_t act_mode, uint16_t* out, void* workspace, size_t workspace_bytes,
                    const mxfp4_moe_opts* opts, void* stream);

/* Bytes of the fixed device scratch mxfp4_moe_layer_noalloc works in. */
#define MXFP4_NOALLOC_SCRATCH_BYTES (32ull << 20)

/*
 * mxfp4_moe_layer for callers that cannot allocate device memory, or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results (bitwise), limits and
 * errors as mxfp4_moe_layer, without workspace / workspace_bytes: the
 * intermediates live in a fixed scratch array of the library, of
 * MXFP4_NOALLOC_SCRATCH_BYTES (32 MiB), one per device, held from the first
 * call on a device until the process ends.  The call allocates nothing.
 *   - Sizes whose workspace (mxfp4_moe_workspace_size) exceeds the scratch
 *     are rejected with MXFP4_E_WORKSPACE before anything is enqueued: the
 *     gpt-oss shape (hidden 2880, 128 experts, top-4) fits up to 363 tokens
 *     with bf16 activations (decode);
 *     the FP8 and MXFP4-activation modes need their restaged weight scales
 *     in the workspace (about 100 MB at that shape) and do not fit it.
 *   - All calls on one device share its scratch, which keeps the last
 *     call's contents: calls that overlap on one device (other streams,
 *     other threads) race and must be ordered by the caller.  Nothing in it
 *     needs to start at zero (every call writes what it reads).
 *   - opts->flags MXFP4_OPT_SCALE_STREAMS_READY is ignored (another call may
 *     have overwritten the restaged scales): the scales are restaged on
 *     every call.
 */
int mxfp4_moe_layer_noalloc(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I,
                            int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                            const uint8_t* w13_blocks, const uint8_t* w13_scales,
                            const uint16_t* w13_bias, const uint8_t* w2_blocks,
                            const uint8_t* w2_scales, const uint16_t* w2_bias, int32_t act_mode,
                            uint16_t* out, const mxfp4_moe_opts* opts, void* stream);

/*
 * The MoE layer of mxfp4_moe_forward with NVFP4 expert weights (gpt-oss page,
 * "The MXFP4 -> NVFP4 Conversion": the same E2M1 element code, 16-element
 * blocks, one E4M3 scale per block, one global scale per tensor; spark-vllm
 * page, "New Features": NVFP4 with group size 16).  A weight is
 * E2M1(code) * E4M3(block scale) * global.
 *   w13_blocks   uint8 [E, 2I, H/16, 8]      16-byte aligned; element 2i of a
 *                                            block in the low nibble of byte i
 *   w13_scales   uint8 [E, 2I, H/16]         4-byte aligned; finite OCP E4M3
 *                                            codes (not S.1111.111)
 *   w13_global   fp32 global scale of w13 (finite)
 *   w2_blocks    uint8 [E, H, I/16, 8]       16-byte aligned
 *   w2_scales    uint8 [E, H, I/16]          4-byte aligned
 *   w2_global    fp32 global scale of w2 (finite)
 *   act_mode     MXFP4_ACT_BF16 (decode: the persistent weight stream) or
 *                MXFP4_ACT_FP8_E4M3 (prefill: x and h quantised exactly as
 *                in mxfp4_moe_forward, both GEMMs on the bf16 MFMA with the
 *                E4M3 codes and the weights expanded exactly to bf16: an
 *                E4M3 block scale cannot ride on the block-scaled MFMA,
 *                whose scales are E8M0); MXFP4_ACT_MXFP4: MXFP4_E_MODE
 *   workspace    nvfp4_moe_workspace_size() bytes (its restaged scale
 *                streams take 8 bytes per weight row and 128-element step)
 * Every other argument is that of mxfp4_moe_forward.  Each weight is formed
 * exactly in bf16 (E2M1 x E4M3 has at most 6 significant bits) and the global
 * scale multiplies the fp32 sums (with the activation scale) before the bias.
 * Limits as mxfp4_moe_forward; with bf16 activations also 160 <= H, I <= 3072
 * (five to 96 32-element chunks per weight row, the span of the persistent
 * decode kernel) and T*k*max(H, I)*2 < 2^31; outside them MXFP4_E_SHAPE.
 */
int nvfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, int32_t act_mode,
                             size_t* bytes);
int nvfp4_moe_forward(const uint16_t* x, int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                      const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13_blocks, const uint8_t* w13_scales, float w13_global,
                      const uint16_t* w13_bias, const uint8_t* w2_blocks, const uint8_t* w2_scales,
                      float w2_global, const uint16_t* w2_bias, int32_t act_mode, uint16_t* out,
                      void* workspace, size_t workspace_bytes, const mxfp4_moe_opts* opts, void* stream);

/*
 * Dense MXFP4 projection out = x W^T + b (spark-vllm page, MXFP4 qkv/o/lm_head,
 * and "Performance Optimizations": FP8 activations on the block-scaled MMA for
 * the dense layers; gptoss-spark page: qkv_proj, o_proj and the 201k-row
 * lm_head in MXFP4), fp32 accumulation, one round-to-nearest-even to bf16.
 *   x         bf16 [M, K]          16-byte aligned
 *   w_blocks  uint8 [N, K/32, 16]  16-byte aligned
 *   w_scales  uint8 [N, K/32]      4-byte aligned; E8M0 bytes in [11, 252]
 *                                  (with bf16 and E4M3 activations the
 *                                  weight is formed with the scaled FP4
 *                                  conversion, exact for these bytes only;
 *                                  others are not rejected and give
 *                                  undefined results; MXFP4 activations
 *                                  take every byte except 255)
 *   bias      bf16 [N] or NULL, 8-byte aligned
 *   act_mode  MXFP4_ACT_BF16: out = bf16(x W^T + b) with x used as given
 *               (a weight stream for decode-sized M; any M is correct);
 *             MXFP4_ACT_FP8_E4M3: x is quantised with the codec of
 *               mxfp4_quant_fp8_e4m3 (one scale s over all of x) and
 *               out = bf16(s (codes W^T) + b) on the FP8 x FP4 block-scaled
 *               MFMA, whose internal sums carry about 2.4e-5 of the sum of
 *               |products| per 128 elements (prefill-sized M);
 *             MXFP4_ACT_MXFP4: each 32-element block of each row of x is
 *               quantised to MXFP4 with the weight quantiser's rule
 *               (mxfp4_quantize_weights) and out = bf16(xq W^T + b) on the
 *               FP4 x FP4 block-scaled MFMA;
 *             anything else: MXFP4_E_MODE
 *   out       bf16 [M, N]          16-byte aligned, must not alias the inputs
 *   workspace device memory of mxfp4_linear_workspace_size() bytes, 256-byte
 *             aligned, caller-owned (contents undefined after the call); may
 *             be NULL when that size is 0 (MXFP4_ACT_BF16); too small:
 *             MXFP4_E_WORKSPACE
 * Limits: K a positive multiple of 32, N a positive multiple of 16,
 * 0 <= M <= 2^20 (M == 0 is a no-op); with quantised activations also
 * K <= 65536 and (M/128 + 1)(N/256 + 1) < 2^30 (MXFP4_E_SHAPE otherwise).
 */
int mxfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t act_mode, size_t* bytes);
int mxfp4_linear(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                 const uint8_t* w_blocks, const uint8_t* w_scales, const uint16_t* bias,
                 int32_t act_mode, uint16_t* out, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Per-tensor FP8 E4M3 quantiser, exactly the codec the FP8 MoE mode applies to
 * x and h, exported for bit-exact tests.  The pages run the MoE as FP8
 * activations times FP4 weights (spark-vllm page, "What's Included") and list
 * real activation scales as open work ("Numerical Accuracy"); this codec is
 * the OCP E4M3 encoding with the per-tensor scale amax/448 the FP8 workloads
 * specify:
 *   amax = max |v|; s = fp32(amax / 448) (1 if amax == 0);
 *   code = E4M3 round-to-nearest-even, saturating to +-448, of fp32(v / s).
 *   in        fp32 [n] (in_dtype 0) or bf16 [n] (in_dtype 1), 16-byte aligned
 *   codes     uint8 [n] output
 *   scale     fp32 [1] output s
 *   amax      fp32 [1] output amax (also used as the accumulator)
 * n >= 0 (n == 0 writes s = 1, amax = 0).  NaN inputs are not supported.
 */
int mxfp4_quant_fp8_e4m3(const void* in, int32_t in_dtype, int64_t n, uint8_t* codes,
                         float* scale, float* amax, void* stream);

/*
 * BF16 -> MXFP4 weight quantiser, for dense weights kept in bf16 (gpt-oss
 * page, "MXFP4 Tensor Structure": attention projections and the LM head are
 * stored bf16; spark-vllm page: MXFP4 for qkv/o/lm_head).  The steps follow
 * the gpt-oss page's "Conversion Methodology" (per-block amax, scale, E2M1
 * rounding, packing) with 32-element blocks and the OCP MX scale rule:
 *   X = floor(log2(max |v| of the block)) - 2, clamped to [-116, 125] (the
 *       lower clamp is this library's departure from the OCP rule, which
 *       would go down to -127: it keeps every byte written inside what all
 *       entry points apply exactly; it only affects blocks with max |v|
 *       below 2^-114);
 *   scale byte = X + 127 (so 11..252, what mxfp4_linear takes);
 *   code = E2M1 value nearest to |v| / 2^X, ties to the even mantissa,
 *          saturating at 6, with the sign bit of v;
 *   nibbles packed as mxfp4_linear reads them (element 2i low, 2i+1 high).
 *   w       bf16 [N, K], 16-byte aligned; finite values (NaN/Inf unsupported)
 *   blocks  uint8 [N, K/32, 16] output, 16-byte aligned
 *   scales  uint8 [N, K/32] output
 * Limits: K a positive multiple of 32, 0 <= N, N * K < 2^40 (N == 0 is a no-op).
 */
int mxfp4_quantize_weights(const uint16_t* w, int64_t N, int64_t K, uint8_t* blocks,
                           uint8_t* scales, void* stream);

/*
 * Measurement helper, not part of the layer: reads `bytes` of device memory
 * once, so that a caller timing it gets the device's streaming-read rate, the
 * ceiling against which the weight streams of the layer are judged (the
 * forum page compares its decode rate with the "bandwidth ceiling" of its
 * GPU the same way).
 *   buf        device memory, 1024-byte aligned, at least `bytes` long
 *   mode       0: 16-byte nontemporal loads into registers; 1: 16-byte
 *              nontemporal direct-to-LDS copies, 1 KB per wave instruction
 *              (the decode GEMV's access)
 *   sink       uint32 [1] device word; written only in the (practically
 *              impossible) case that the folded data equals a fixed value
 *   bytes_read host output: bytes actually read (the grid reads whole 16 KB
 *              rounds per block: `bytes` rounded down, 0 below 16 KB)
 * Limits: bytes <= 2^40.
 */
int mxfp4_stream_read(const void* buf, uint64_t bytes, int32_t mode, uint32_t* sink,
                      uint64_t* bytes_read, void* stream);

/* Thin hipEvent helpers so callers can time stages without their own HIP
   bindings: create (timing enabled), destroy, and elapsed milliseconds between
   two recorded events (synchronises on `end`). */
int mxfp4_event_create(void** event);
int mxfp4_event_destroy(void* event);
int mxfp4_event_elapsed_ms(void* start, void* end, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_MOE_H */
