"""ctypes binding of libmxfp4moe.so (include/mxfp4_moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the shared library.  PyTorch provides device memory and the stream.  There is
no fallback: if the library is missing the first call raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxfp4moe.so")

ACT_BF16 = 0
ACT_FP8_E4M3 = 1
ACT_MXFP4 = 2
ABI_VERSION = 5
NUM_STAGES = 7
STAGES = ("begin", "permute", "quant_x", "gemm1", "quant_h", "gemm2", "combine")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "total_bytes", "status", "expert_offsets", "sorted_pairs", "inv_pairs",
        "chunk_counts", "chunk_ranks", "tiles", "x_codes", "h", "h_codes", "y", "x_scales",
        "h_scales", "w13_scale_stream", "w2_scale_stream")]


OPT_SCALE_STREAMS_READY = 1


class MoeOpts(ctypes.Structure):
    _fields_ = [("events", _c_void_p * NUM_STAGES), ("flags", ctypes.c_uint32),
                ("w13_codes", _c_void_p), ("w2_codes", _c_void_p)]


def _opts(events, scale_streams_ready, code_streams=None):
    if events is None and not scale_streams_ready and code_streams is None:
        return None
    opts = MoeOpts()
    for i, ev in enumerate(events or ()):
        opts.events[i] = ev
    opts.flags = OPT_SCALE_STREAMS_READY if scale_streams_ready else 0
    if code_streams is not None:
        w13c, w2c = code_streams
        for t, name in ((w13c, "w13 code stream"), (w2c, "w2 code stream")):
            if t is not None:
                _need(t, name, torch.uint8, 1)
        opts.w13_codes = None if w13c is None else w13c.data_ptr()
        opts.w2_codes = None if w2c is None else w2c.data_ptr()
    return opts


class Mxfp4Error(RuntimeError):
    def __init__(self, func, status, detail):
        super().__init__("%s failed with status %d: %s" % (func, status, detail))
        self.status = status


_lib = None


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmxfp4moe.so is not built (run __graft_entry__.build()): %s" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.mxfp4_abi_version.restype = ctypes.c_int
        if L.mxfp4_abi_version() != ABI_VERSION:
            raise RuntimeError("libmxfp4moe.so has ABI version %d, the binding expects %d (rebuild it)"
                               % (L.mxfp4_abi_version(), ABI_VERSION))
        L.mxfp4_status_string.restype = ctypes.c_char_p
        L.mxfp4_status_string.argtypes = [ctypes.c_int]
        L.mxfp4_last_error.restype = ctypes.c_char_p
        L.mxfp4_route_topk.argtypes = [_c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]
        L.mxfp4_moe_workspace_size.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32,
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.mxfp4_moe_workspace_layout_query.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32,
                                                       ctypes.POINTER(WorkspaceLayout)]
        L.mxfp4_moe_forward.argtypes = [
            _c_void_p, _i64, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p,
            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
            _i32, _c_void_p, _c_void_p, ctypes.c_size_t, ctypes.POINTER(MoeOpts), _c_void_p]
        L.mxfp4_moe_layer.argtypes = [
            _c_void_p, _c_void_p, _i64, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p,
            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
            _i32, _c_void_p, _c_void_p, ctypes.c_size_t, ctypes.POINTER(MoeOpts), _c_void_p]
        L.mxfp4_moe_layer_noalloc.argtypes = [
            _c_void_p, _c_void_p, _i64, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p,
            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
            _i32, _c_void_p, ctypes.POINTER(MoeOpts), _c_void_p]
        L.nvfp4_moe_forward.argtypes = [
            _c_void_p, _i64, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p,
            _c_void_p, _c_void_p, ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, ctypes.c_float,
            _c_void_p, _i32, _c_void_p, _c_void_p, ctypes.c_size_t, ctypes.POINTER(MoeOpts), _c_void_p]
        L.nvfp4_moe_workspace_size.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32,
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.mxfp4_linear_workspace_size.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(ctypes.c_size_t)]
        L.mxfp4_linear.argtypes = [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                   _i32, _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p]
        L.mxfp4_quant_fp8_e4m3.argtypes = [_c_void_p, _i32, _i64, _c_void_p, _c_void_p, _c_void_p,
                                           _c_void_p]
        L.mxfp4_quantize_weights.argtypes = [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]
        L.mxfp4_stream_read.argtypes = [_c_void_p, ctypes.c_uint64, _i32, _c_void_p,
                                        ctypes.POINTER(ctypes.c_uint64), _c_void_p]
        L.mxfp4_moe_code_stream_size.argtypes = [_i64, _i64, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]
        L.mxfp4_moe_prepare_code_stream.argtypes = [_c_void_p, _i64, _i64, _i32, _i32, _c_void_p,
                                                    ctypes.c_size_t, _c_void_p]
        L.mxfp4_event_create.argtypes = [ctypes.POINTER(_c_void_p)]
        L.mxfp4_event_destroy.argtypes = [_c_void_p]
        L.mxfp4_event_elapsed_ms.argtypes = [_c_void_p, _c_void_p, ctypes.POINTER(ctypes.c_float)]
        for name in ("mxfp4_route_topk", "mxfp4_moe_workspace_size", "mxfp4_moe_workspace_layout_query",
                     "mxfp4_moe_forward", "mxfp4_moe_layer", "mxfp4_moe_layer_noalloc", "nvfp4_moe_forward",
                     "nvfp4_moe_workspace_size",
                     "mxfp4_linear_workspace_size", "mxfp4_linear",
                     "mxfp4_quant_fp8_e4m3",
                     "mxfp4_quantize_weights", "mxfp4_stream_read", "mxfp4_moe_code_stream_size",
                     "mxfp4_moe_prepare_code_stream", "mxfp4_event_create",
                     "mxfp4_event_destroy", "mxfp4_event_elapsed_ms"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(func, status):
    if status != 0:
        raise Mxfp4Error(func, status, lib().mxfp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims" % (name, ndim))


def mxfp4_abi_version():
    return lib().mxfp4_abi_version()


def mxfp4_route_topk(logits, k, topk_ids=None, topk_weights=None, stream=None):
    """Top-k expert ids (int32 [T,k]) and softmax-of-k weights (fp32 [T,k])."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    if tuple(topk_ids.shape) != (T, k) or tuple(topk_weights.shape) != (T, k):
        raise ValueError("topk outputs must be [T, k]")
    _check("mxfp4_route_topk", lib().mxfp4_route_topk(
        _ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_weights), _stream(stream)))
    return topk_ids, topk_weights


def mxfp4_moe_workspace_size(T, H, I, E, k, act_mode):
    n = ctypes.c_size_t(0)
    _check("mxfp4_moe_workspace_size",
           lib().mxfp4_moe_workspace_size(T, H, I, E, k, act_mode, ctypes.byref(n)))
    return n.value


def mxfp4_moe_workspace_layout_query(T, H, I, E, k, act_mode):
    L = WorkspaceLayout()
    _check("mxfp4_moe_workspace_layout_query",
           lib().mxfp4_moe_workspace_layout_query(T, H, I, E, k, act_mode, ctypes.byref(L)))
    return {name: getattr(L, name) for name, _ in WorkspaceLayout._fields_}


def mxfp4_moe_forward(x, topk_ids, topk_weights, w13_blocks, w13_scales, w13_bias,
                      w2_blocks, w2_scales, w2_bias, act_mode, out=None, workspace=None,
                      events=None, stream=None, scale_streams_ready=False, code_streams=None):
    """One MoE layer; returns out (bf16 [T, H]).  `workspace` is a uint8 device
    tensor of at least mxfp4_moe_workspace_size() bytes (allocated here if None);
    `events` is an optional list of NUM_STAGES event handles (or None entries);
    `scale_streams_ready` sets MXFP4_OPT_SCALE_STREAMS_READY (the workspace
    already holds these weights' restaged scales from an earlier call);
    `code_streams` is None or (w13, w2) code streams from
    mxfp4_moe_prepare_code_stream (either may be None)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    _need(w13_blocks, "w13_blocks", torch.uint8, 4)
    _need(w13_scales, "w13_scales", torch.uint8, 3)
    _need(w2_blocks, "w2_blocks", torch.uint8, 4)
    _need(w2_scales, "w2_scales", torch.uint8, 3)
    if w13_bias is not None:
        _need(w13_bias, "w13_bias", torch.bfloat16, 2)
    if w2_bias is not None:
        _need(w2_bias, "w2_bias", torch.bfloat16, 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    E, twoI = w13_blocks.shape[0], w13_blocks.shape[1]
    I = twoI // 2
    if (tuple(w13_blocks.shape) != (E, 2 * I, H // 32, 16) or tuple(w13_scales.shape) != (E, 2 * I, H // 32)
            or tuple(w2_blocks.shape) != (E, H, I // 32, 16) or tuple(w2_scales.shape) != (E, H, I // 32)
            or tuple(topk_ids.shape) != (T, k) or tuple(topk_weights.shape) != (T, k)
            or (w13_bias is not None and tuple(w13_bias.shape) != (E, 2 * I))
            or (w2_bias is not None and tuple(w2_bias.shape) != (E, H))):
        raise ValueError("inconsistent MoE tensor shapes")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if workspace is None:
        workspace = torch.empty(max(mxfp4_moe_workspace_size(T, H, I, E, k, act_mode), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    opts = _opts(events, scale_streams_ready, code_streams)
    _check("mxfp4_moe_forward", lib().mxfp4_moe_forward(
        _ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_weights),
        _ptr(w13_blocks), _ptr(w13_scales), _ptr(w13_bias),
        _ptr(w2_blocks), _ptr(w2_scales), _ptr(w2_bias), act_mode, _ptr(out),
        _ptr(workspace), workspace.numel(), ctypes.byref(opts) if opts is not None else None,
        _stream(stream)))
    return out


def nvfp4_moe_workspace_size(T, H, I, E, k, act_mode=ACT_BF16):
    n = ctypes.c_size_t()
    _check("nvfp4_moe_workspace_size",
           lib().nvfp4_moe_workspace_size(T, H, I, E, k, act_mode, ctypes.byref(n)))
    return n.value


def nvfp4_moe_forward(x, topk_ids, topk_weights, w13_blocks, w13_scales, w13_global, w13_bias,
                      w2_blocks, w2_scales, w2_global, w2_bias, out=None, workspace=None, events=None,
                      stream=None, act_mode=ACT_BF16, scale_streams_ready=False, code_streams=None):
    """MoE layer with NVFP4 expert weights (blocks [E, N, K/16, 8], E4M3 scales
    [E, N, K/16], one fp32 global scale per tensor), bf16 or (act_mode
    ACT_FP8_E4M3) per-tensor E4M3 activations; returns out (bf16 [T, H])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    _need(w13_blocks, "w13_blocks", torch.uint8, 4)
    _need(w13_scales, "w13_scales", torch.uint8, 3)
    _need(w2_blocks, "w2_blocks", torch.uint8, 4)
    _need(w2_scales, "w2_scales", torch.uint8, 3)
    if w13_bias is not None:
        _need(w13_bias, "w13_bias", torch.bfloat16, 2)
    if w2_bias is not None:
        _need(w2_bias, "w2_bias", torch.bfloat16, 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    E, twoI = w13_blocks.shape[0], w13_blocks.shape[1]
    I = twoI // 2
    if (tuple(w13_blocks.shape) != (E, 2 * I, H // 16, 8) or tuple(w13_scales.shape) != (E, 2 * I, H // 16)
            or tuple(w2_blocks.shape) != (E, H, I // 16, 8) or tuple(w2_scales.shape) != (E, H, I // 16)
            or tuple(topk_ids.shape) != (T, k) or tuple(topk_weights.shape) != (T, k)
            or (w13_bias is not None and tuple(w13_bias.shape) != (E, 2 * I))
            or (w2_bias is not None and tuple(w2_bias.shape) != (E, H))):
        raise ValueError("inconsistent NVFP4 MoE tensor shapes")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if workspace is None:
        workspace = torch.empty(max(nvfp4_moe_workspace_size(T, H, I, E, k, act_mode), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    opts = _opts(events, scale_streams_ready, code_streams)
    _check("nvfp4_moe_forward", lib().nvfp4_moe_forward(
        _ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_weights),
        _ptr(w13_blocks), _ptr(w13_scales), float(w13_global), _ptr(w13_bias),
        _ptr(w2_blocks), _ptr(w2_scales), float(w2_global), _ptr(w2_bias), act_mode, _ptr(out),
        _ptr(workspace), workspace.numel(), ctypes.byref(opts) if opts is not None else None,
        _stream(stream)))
    return out


def _layer_args(x, logits, k, w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias, out, topk_ids,
                topk_weights):
    """Shape and dtype checks of the router + layer entry points; outputs
    created when not given.  Returns (T, H, I, E, out, topk_ids, topk_weights)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2)
    T, H = x.shape
    E = logits.shape[1]
    if logits.shape[0] != T or w13_blocks.shape[0] != E:
        raise ValueError("logits must be [T, E]")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    for t, name, nd in ((w13_blocks, "w13_blocks", 4), (w13_scales, "w13_scales", 3),
                        (w2_blocks, "w2_blocks", 4), (w2_scales, "w2_scales", 3)):
        _need(t, name, torch.uint8, nd)
    I = w13_blocks.shape[1] // 2
    if (tuple(w13_blocks.shape) != (E, 2 * I, H // 32, 16) or tuple(w13_scales.shape) != (E, 2 * I, H // 32)
            or tuple(w2_blocks.shape) != (E, H, I // 32, 16) or tuple(w2_scales.shape) != (E, H, I // 32)
            or tuple(topk_ids.shape) != (T, k) or tuple(topk_weights.shape) != (T, k)
            or (w13_bias is not None and tuple(w13_bias.shape) != (E, 2 * I))
            or (w2_bias is not None and tuple(w2_bias.shape) != (E, H))):
        raise ValueError("inconsistent MoE tensor shapes")
    if w13_bias is not None:
        _need(w13_bias, "w13_bias", torch.bfloat16, 2)
    if w2_bias is not None:
        _need(w2_bias, "w2_bias", torch.bfloat16, 2)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    return T, H, I, E, out, topk_ids, topk_weights


def mxfp4_moe_layer(x, logits, k, w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias,
                    act_mode, out=None, topk_ids=None, topk_weights=None, workspace=None, events=None,
                    stream=None, scale_streams_ready=False, code_streams=None):
    """Router + MoE layer in one call; returns (out, topk_ids, topk_weights)."""
    T, H, I, E, out, topk_ids, topk_weights = _layer_args(
        x, logits, k, w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias, out, topk_ids,
        topk_weights)
    if workspace is None:
        workspace = torch.empty(max(mxfp4_moe_workspace_size(T, H, I, E, k, act_mode), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    opts = _opts(events, scale_streams_ready, code_streams)
    _check("mxfp4_moe_layer", lib().mxfp4_moe_layer(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_weights),
        _ptr(w13_blocks), _ptr(w13_scales), _ptr(w13_bias),
        _ptr(w2_blocks), _ptr(w2_scales), _ptr(w2_bias), act_mode, _ptr(out),
        _ptr(workspace), workspace.numel(), ctypes.byref(opts) if opts is not None else None,
        _stream(stream)))
    return out, topk_ids, topk_weights


def mxfp4_moe_layer_noalloc(x, logits, k, w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias,
                            act_mode, out, topk_ids, topk_weights, events=None, stream=None):
    """Router + MoE layer in the library's fixed device scratch (no workspace);
    the caller passes every output.  Returns (out, topk_ids, topk_weights)."""
    if out is None or topk_ids is None or topk_weights is None:
        raise ValueError("mxfp4_moe_layer_noalloc takes caller-owned outputs")
    T, H, I, E, out, topk_ids, topk_weights = _layer_args(
        x, logits, k, w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias, out, topk_ids,
        topk_weights)
    opts = _opts(events, False)
    _check("mxfp4_moe_layer_noalloc", lib().mxfp4_moe_layer_noalloc(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_weights),
        _ptr(w13_blocks), _ptr(w13_scales), _ptr(w13_bias),
        _ptr(w2_blocks), _ptr(w2_scales), _ptr(w2_bias), act_mode, _ptr(out),
        ctypes.byref(opts) if opts is not None else None, _stream(stream)))
    return out, topk_ids, topk_weights


def mxfp4_linear_workspace_size(M, N, K, act_mode=ACT_BF16):
    n = ctypes.c_size_t()
    _check("mxfp4_linear_workspace_size", lib().mxfp4_linear_workspace_size(M, N, K, act_mode, ctypes.byref(n)))
    return n.value


def mxfp4_linear(x, w_blocks, w_scales, bias=None, out=None, stream=None, act_mode=ACT_BF16, workspace=None):
    """Dense MXFP4 projection out = x W^T + b, bf16 [M, N].  With act_mode
    ACT_FP8_E4M3 or ACT_MXFP4 x is quantised first; `workspace` is a uint8
    device tensor of at least mxfp4_linear_workspace_size() bytes (allocated
    here if None)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_blocks, "w_blocks", torch.uint8, 3)
    _need(w_scales, "w_scales", torch.uint8, 2)
    M, K = x.shape
    N = w_blocks.shape[0]
    if tuple(w_blocks.shape) != (N, K // 32, 16) or tuple(w_scales.shape) != (N, K // 32):
        raise ValueError("w_blocks/w_scales shape does not match x")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must be [N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    need = mxfp4_linear_workspace_size(M, N, K, act_mode)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
    _check("mxfp4_linear", lib().mxfp4_linear(
        _ptr(x), M, N, K, _ptr(w_blocks), _ptr(w_scales), _ptr(bias), act_mode, _ptr(out),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out


def mxfp4_quant_fp8_e4m3(inp, codes=None, scale=None, amax=None, stream=None):
    """Per-tensor E4M3 codes (uint8, same shape), scale and amax (fp32 [1])."""
    if inp.dtype == torch.float32:
        dt = 0
    elif inp.dtype == torch.bfloat16:
        dt = 1
    else:
        raise TypeError("inp must be float32 or bfloat16")
    _need(inp, "inp", inp.dtype)
    if codes is None:
        codes = torch.empty(inp.shape, dtype=torch.uint8, device=inp.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=inp.device)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=inp.device)
    _need(codes, "codes", torch.uint8)
    _check("mxfp4_quant_fp8_e4m3", lib().mxfp4_quant_fp8_e4m3(
        _ptr(inp), dt, inp.numel(), _ptr(codes), _ptr(scale), _ptr(amax), _stream(stream)))
    return codes, scale, amax


def mxfp4_quantize_weights(w, blocks=None, scales=None, stream=None):
    """bf16 weights [N, K] -> MXFP4 blocks uint8 [N, K/32, 16] and E8M0 scales [N, K/32]."""
    _need(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if blocks is None:
        blocks = torch.empty((N, K // 32, 16), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    _need(blocks, "blocks", torch.uint8, 3)
    _need(scales, "scales", torch.uint8, 2)
    if tuple(blocks.shape) != (N, K // 32, 16) or tuple(scales.shape) != (N, K // 32):
        raise ValueError("blocks/scales shape does not match w")
    _check("mxfp4_quantize_weights", lib().mxfp4_quantize_weights(
        _ptr(w), N, K, _ptr(blocks), _ptr(scales), _stream(stream)))
    return blocks, scales


def mxfp4_stream_read(buf, mode, sink=None, stream=None):
    """Read the device buffer `buf` once (mode 0: register loads, 1: direct-to-LDS
    copies); returns the bytes actually read.  For ceiling measurements."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    n = ctypes.c_uint64()
    _check("mxfp4_stream_read", lib().mxfp4_stream_read(
        _ptr(buf), buf.numel() * buf.element_size(), mode, _ptr(sink), ctypes.byref(n), _stream(stream)))
    return n.value


def mxfp4_event_create():
    ev = ctypes.c_void_p()
    _check("mxfp4_event_create", lib().mxfp4_event_create(ctypes.byref(ev)))
    return ev.value


def mxfp4_event_destroy(ev):
    _check("mxfp4_event_destroy", lib().mxfp4_event_destroy(ctypes.c_void_p(ev)))


def mxfp4_event_elapsed_ms(start, end):
    ms = ctypes.c_float()
    _check("mxfp4_event_elapsed_ms",
           lib().mxfp4_event_elapsed_ms(ctypes.c_void_p(start), ctypes.c_void_p(end), ctypes.byref(ms)))
    return ms.value


def mxfp4_moe_code_stream_size(H, I, E, which):
    """Bytes of the restaged code stream of w13 (which=0) or w2 (which=1)."""
    n = ctypes.c_size_t(0)
    _check("mxfp4_moe_code_stream_size", lib().mxfp4_moe_code_stream_size(H, I, E, which, ctypes.byref(n)))
    return n.value


def mxfp4_moe_prepare_code_stream(blocks, H, I, which, out=None, stream=None):
    """The E2M1 codes of w13 (which=0, blocks [E, 2I, ...]) or w2 (which=1,
    blocks [E, H, ...]) restaged for the prefill GEMMs; a uint8 device tensor."""
    _need(blocks, "blocks", torch.uint8)
    E = blocks.shape[0]
    n = mxfp4_moe_code_stream_size(H, I, E, which)
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.uint8, device=blocks.device)
    _need(out, "out", torch.uint8, 1)
    _check("mxfp4_moe_prepare_code_stream", lib().mxfp4_moe_prepare_code_stream(
        _ptr(blocks), H, I, E, which, _ptr(out), out.numel(), _stream(stream)))
    return out

