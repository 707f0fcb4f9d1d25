"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching a device (runs without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4_moe.h")

E_NULL, E_SHAPE, E_ALIGN, E_MODE, E_WORKSPACE, E_DEVICE = 1, 2, 3, 4, 5, 6


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mxfp4|nvfp4)_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from mxfp4_block_scaled_top_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmxfp4moe.so is not built; run __graft_entry__.build()")
    return _lib.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("mxfp4_route_topk", "mxfp4_moe_forward", "mxfp4_linear",
                 "mxfp4_quant_fp8_e4m3", "mxfp4_moe_workspace_size"):
        assert must in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.mxfp4_abi_version() == 5
    assert L.mxfp4_status_string(0) == b"ok"
    assert L.mxfp4_status_string(E_WORKSPACE) == b"workspace too small"
    assert L.mxfp4_status_string(99) == b"unknown status"


def _size(L, T, H, I, E, k, mode):
    n = ctypes.c_size_t(0)
    rc = L.mxfp4_moe_workspace_size(T, H, I, E, k, mode, ctypes.byref(n))
    return rc, n.value


def test_workspace_size_validation(L):
    rc, n = _size(L, 32, 2880, 2880, 128, 4, 0)
    assert rc == 0 and n > 32 * 4 * 2880 * 4
    rc8, n8 = _size(L, 2048, 2880, 2880, 128, 4, 1)
    assert rc8 == 0 and n8 > n
    rc4, n4 = _size(L, 2048, 2880, 2880, 128, 4, 2)                # MXFP4 activations
    assert rc4 == 0 and n < n4 < n8
    assert _size(L, 4, 2880, 2880, 128, 4, 3)[0] == E_MODE          # unknown act_mode
    assert _size(L, 4, 2880 + 16, 2880, 128, 4, 0)[0] == E_SHAPE    # H % 32
    assert _size(L, 4, 2880, 0, 128, 4, 0)[0] == E_SHAPE
    assert _size(L, 4, 2880, 2880, 128, 0, 0)[0] == E_SHAPE         # k < 1
    assert _size(L, 4, 2880, 2880, 3, 4, 0)[0] == E_SHAPE           # k > E
    assert _size(L, 4, 2880, 2880, 513, 4, 0)[0] == E_SHAPE
    assert _size(L, -1, 2880, 2880, 128, 4, 0)[0] == E_SHAPE
    assert L.mxfp4_moe_workspace_size(4, 2880, 2880, 128, 4, 0, None) == E_NULL
    assert b"act_mode" in L.mxfp4_last_error() or L.mxfp4_last_error() != b""


def test_layout_offsets_are_ordered_and_aligned(L):
    from mxfp4_block_scaled_top_amd._lib import WorkspaceLayout
    lay = WorkspaceLayout()
    assert L.mxfp4_moe_workspace_layout_query(8192, 2880, 2880, 128, 4, 1, ctypes.byref(lay)) == 0
    offs = [lay.status, lay.expert_offsets, lay.sorted_pairs, lay.inv_pairs, lay.chunk_counts,
            lay.chunk_ranks, lay.tiles, lay.x_codes, lay.h, lay.h_codes, lay.y]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and lay.total_bytes > lay.y
    # code rows are padded to whole 128-byte lines: 2880 E4M3 codes -> 2944 bytes
    assert lay.y - lay.h >= 8192 * 4 * (2880 * 4 + 2944)  # fp32 h + u8 codes
    assert lay.y - lay.h_codes >= 8192 * 4 * 2944
    assert lay.h - lay.x_codes >= 8192 * 4 * 2944        # x codes per routed pair (sorted rows)
    assert lay.x_scales == 0 and lay.h_scales == 0
    # restaged scale streams: 1 KB per (expert, n-tile, K step)
    assert lay.y < lay.w13_scale_stream < lay.w2_scale_stream < lay.total_bytes
    assert lay.w2_scale_stream - lay.w13_scale_stream >= 128 * 23 * 23 * 1024
    assert lay.total_bytes - lay.w2_scale_stream >= 128 * 12 * 23 * 1024


def test_layout_of_mxfp4_activations(L):
    from mxfp4_block_scaled_top_amd._lib import WorkspaceLayout
    lay = WorkspaceLayout()
    T, H, I = 2048, 2880, 2880
    np_ = T * 4
    assert L.mxfp4_moe_workspace_layout_query(T, H, I, 128, 4, 2, ctypes.byref(lay)) == 0
    offs = [lay.x_codes, lay.x_scales, lay.h, lay.h_codes, lay.h_scales, lay.y, lay.w13_scale_stream,
            lay.w2_scale_stream]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert lay.x_scales - lay.x_codes >= np_ * 1536      # E2M1 blocks per sorted row, 1440 -> 1536 B
    assert lay.h - lay.x_scales >= 23 * np_ * 4 + 512    # 23 steps x 4 scales per row, + read slack
    assert lay.h_codes == lay.h                          # h is quantised in the GEMM: no fp32 copy
    assert lay.h_scales - lay.h_codes >= np_ * 1536
    assert lay.y - lay.h_scales >= 23 * np_ * 4 + 512
    assert lay.w13_scale_stream - lay.y >= np_ * H * 4
    assert lay.total_bytes - lay.w2_scale_stream >= 128 * 12 * 23 * 1024


def _fake(n=1):
    return ctypes.c_void_p(0x1000 * n)     # never dereferenced: validation fails first


def test_moe_forward_rejects_bad_arguments_without_touching_memory(L):
    a = dict(x=_fake(1), T=4, H=2880, I=2880, E=128, k=4, ids=_fake(2), w=_fake(3), b13=_fake(4),
             s13=_fake(5), bias13=None, b2=_fake(6), s2=_fake(7), bias2=None, mode=0, out=_fake(8),
             ws=_fake(9), wsb=1 << 40, opts=None, stream=None)

    def call(**kw):
        d = dict(a, **kw)
        return L.mxfp4_moe_forward(d["x"], d["T"], d["H"], d["I"], d["E"], d["k"], d["ids"], d["w"],
                                   d["b13"], d["s13"], d["bias13"], d["b2"], d["s2"], d["bias2"],
                                   d["mode"], d["out"], d["ws"], d["wsb"], d["opts"], d["stream"])
    assert call(mode=7) == E_MODE
    assert call(H=100) == E_SHAPE
    assert call(k=17) == E_SHAPE
    assert call(x=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(x=ctypes.c_void_p(0x1008)) == E_ALIGN
    assert call(ws=ctypes.c_void_p(0x1010)) == E_ALIGN
    assert call(bias13=ctypes.c_void_p(0x1002)) == E_ALIGN   # biases are read 4 rows at a time
    assert call(bias2=ctypes.c_void_p(0x1004)) == E_ALIGN
    assert call(ws=None) == E_WORKSPACE
    assert call(wsb=100) == E_WORKSPACE
    assert call(T=0) == 0                       # empty batch: a no-op
    # the router + layer call: same checks, plus the logits
    assert L.mxfp4_moe_layer(_fake(1), None, 4, 2880, 2880, 128, 4, _fake(2), _fake(3), _fake(4), _fake(5),
                             None, _fake(6), _fake(7), None, 0, _fake(8), _fake(9), 1 << 40, None,
                             None) == E_NULL
    assert L.mxfp4_moe_layer(_fake(1), _fake(10), 4, 2880, 2880, 128, 4, _fake(2), _fake(3), _fake(4),
                             _fake(5), None, _fake(6), _fake(7), None, 9, _fake(8), _fake(9), 1 << 40,
                             None, None) == E_MODE


def _lin(L, x, M, N, K, bias=None, mode=0, ws=None, ws_bytes=0):
    return L.mxfp4_linear(x, M, N, K, _fake(), _fake(), bias, mode, _fake(), ws, ws_bytes, None)


def test_linear_and_quant_and_route_validation(L):
    assert _lin(L, _fake(), 1, 100, 2880) == E_SHAPE
    assert _lin(L, _fake(), 1, 128, 2881) == E_SHAPE
    assert _lin(L, None, 1, 128, 2880) == E_NULL
    assert _lin(L, _fake(), 0, 128, 2880) == 0
    assert _lin(L, _fake(), 1, 128, 2880, bias=ctypes.c_void_p(0x1002)) == E_ALIGN
    assert _lin(L, _fake(), 1, 128, 2880, mode=7) == E_MODE
    # quantised activations need the workspace the size query gives
    for mode in (1, 2):
        assert _lin(L, _fake(), 4, 128, 2880, mode=mode) == E_WORKSPACE
        assert _lin(L, _fake(), 4, 128, 2880, mode=mode, ws=_fake(), ws_bytes=1024) == E_WORKSPACE
        assert _lin(L, _fake(), 4, 128, 2880, mode=mode, ws=ctypes.c_void_p(0x1010),
                    ws_bytes=1 << 40) == E_ALIGN
        assert _lin(L, _fake(), 4, 128, 1 << 17, mode=mode) == E_SHAPE
    assert _lin(L, _fake(), 4, 128, 1 << 17, mode=9) == E_MODE
    assert L.mxfp4_quant_fp8_e4m3(_fake(), 5, 10, _fake(), _fake(), _fake(), None) == E_MODE
    assert L.mxfp4_quant_fp8_e4m3(_fake(), 0, 10, _fake(), None, _fake(), None) == E_NULL
    assert L.mxfp4_route_topk(_fake(), 4, 128, 0, _fake(), _fake(), None) == E_SHAPE
    assert L.mxfp4_route_topk(_fake(), 4, 600, 4, _fake(), _fake(), None) == E_SHAPE
    assert L.mxfp4_route_topk(None, 4, 128, 4, _fake(), _fake(), None) == E_NULL
    assert L.mxfp4_route_topk(None, 0, 128, 4, None, None, None) == 0
    assert L.mxfp4_quantize_weights(_fake(), 4, 33, _fake(), _fake(), None) == E_SHAPE
    assert L.mxfp4_quantize_weights(_fake(), -1, 32, _fake(), _fake(), None) == E_SHAPE
    assert L.mxfp4_quantize_weights(None, 4, 32, _fake(), _fake(), None) == E_NULL
    assert L.mxfp4_quantize_weights(ctypes.c_void_p(0x1008), 4, 32, _fake(), _fake(), None) == E_ALIGN
    assert L.mxfp4_quantize_weights(None, 0, 32, None, None, None) == 0


def test_valid_call_without_a_gpu_reports_no_device(L):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert L.mxfp4_route_topk(_fake(), 4, 128, 4, _fake(), _fake(), None) == E_DEVICE
    assert L.mxfp4_last_error() != b""


def test_nvfp4_moe_forward_rejects_bad_arguments_without_touching_memory(L):
    f = L.nvfp4_moe_forward
    fake = _fake
    args = [fake(1), 4, 2880, 2880, 128, 4, fake(2), fake(3), fake(4), fake(5), ctypes.c_float(1.0), None,
            fake(6), fake(7), ctypes.c_float(1.0), None, 0, fake(8), fake(9), ctypes.c_size_t(1 << 30), None,
            None]
    a = list(args); a[8] = None                       # null w13_blocks
    assert f(*a) == E_NULL
    a = list(args); a[2] = 4096; a[3] = 4096          # beyond the bf16-activation NVFP4 limit
    assert f(*a) == E_SHAPE
    a = list(args); a[2] = 128                        # below the bf16-activation NVFP4 limit
    assert f(*a) == E_SHAPE
    a = list(args); a[10] = ctypes.c_float(float("nan"))
    assert f(*a) == E_SHAPE
    a = list(args); a[2] = 2880 + 16                  # H % 32
    assert f(*a) == E_SHAPE
    a = list(args); a[16] = 2                         # MXFP4 activations: not with NVFP4 weights
    assert f(*a) == E_MODE
    a = list(args); a[16] = 5
    assert f(*a) == E_MODE
    # E4M3 activations lift the decode kernel's 3072 limit; a small workspace is then the error
    a = list(args); a[16] = 1; a[2] = 4096; a[3] = 4096; a[19] = ctypes.c_size_t(1024)
    assert f(*a) == E_WORKSPACE


def test_nvfp4_workspace_size_doubles_the_scale_streams(L):
    n_mx, n_nv, n_bf = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.mxfp4_moe_workspace_size(2048, 2880, 2880, 128, 4, 1, ctypes.byref(n_mx)) == 0
    assert L.nvfp4_moe_workspace_size(2048, 2880, 2880, 128, 4, 1, ctypes.byref(n_nv)) == 0
    streams = 128 * (23 + 12) * 23 * 1024      # w13 (23 n-tiles) + w2 (12), 23 K steps, 1 KB each
    assert n_nv.value - n_mx.value >= streams
    assert L.nvfp4_moe_workspace_size(32, 2880, 2880, 128, 4, 0, ctypes.byref(n_bf)) == 0
    assert L.mxfp4_moe_workspace_size(32, 2880, 2880, 128, 4, 0, ctypes.byref(n_mx)) == 0
    assert n_bf.value == n_mx.value
    assert L.nvfp4_moe_workspace_size(32, 2880, 2880, 128, 4, 2, ctypes.byref(n_bf)) == E_MODE


def test_stream_read_validation(L):
    n = ctypes.c_uint64(0)
    assert L.mxfp4_stream_read(_fake(), 1 << 20, 2, _fake(), ctypes.byref(n), None) == E_MODE
    assert L.mxfp4_stream_read(_fake(), 1 << 20, 0, _fake(), None, None) == E_NULL
    assert L.mxfp4_stream_read(None, 1 << 20, 1, _fake(), ctypes.byref(n), None) == E_NULL
    assert L.mxfp4_stream_read(ctypes.c_void_p(0x1010), 1 << 20, 0, _fake(), ctypes.byref(n), None) == E_ALIGN
    assert L.mxfp4_stream_read(_fake(), 1 << 41, 0, _fake(), ctypes.byref(n), None) == E_SHAPE


def test_moe_layer_noalloc_rejects_bad_arguments_without_touching_memory(L):
    f = L.mxfp4_moe_layer_noalloc
    args = lambda T, H, I, E, k, act, logits=_fake(2): (  # noqa: E731
        _fake(), logits, T, H, I, E, k, _fake(3), _fake(4), _fake(5), _fake(6), None, _fake(7), _fake(8), None,
        act, _fake(9), None, None)
    # 400 tokens x top-4 at 2880 x 2880 need more than the 32 MiB scratch
    assert f(*args(400, 2880, 2880, 4, 4, 0)) == E_WORKSPACE
    assert f(*args(2048, 2880, 2880, 128, 4, 1)) == E_WORKSPACE
    assert f(*args(32, 2880, 2880, 128, 4, 7)) == E_MODE
    assert f(*args(32, 2880, 2880, 128, 4, 0, logits=None)) == E_NULL
    assert f(*args(32, 33, 2880, 128, 4, 0)) == E_SHAPE
    assert f(*args(0, 2880, 2880, 128, 4, 0)) == 0          # T == 0: no-op


def test_linear_workspace_size(L):
    n = ctypes.c_size_t()
    assert L.mxfp4_linear_workspace_size(4, 5120, 2880, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert L.mxfp4_linear_workspace_size(4, 5120, 2880, 3, ctypes.byref(n)) == E_MODE
    assert L.mxfp4_linear_workspace_size(4, 5120, 2880, 1, None) == E_NULL
    sizes = {}
    for mode in (1, 2):
        for M in (1, 2048):
            assert L.mxfp4_linear_workspace_size(M, 5120, 2880, mode, ctypes.byref(n)) == 0
            sizes[mode, M] = n.value
    # codes (1 byte, MXFP4 half a byte, per element of x) plus the restaged
    # weight scales (1 KB per 256-row n-tile and 128-element K step)
    stream = 20 * 23 * 1024
    assert sizes[1, 2048] >= 2048 * 2880 + stream
    assert sizes[2, 2048] >= 2048 * 1440 + stream + 23 * 2048 * 4
    assert sizes[1, 2048] - sizes[1, 1] >= 2047 * 2880
    assert sizes[2, 2048] < sizes[1, 2048]
