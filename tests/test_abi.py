"""C-ABI contract checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments with a status code before any HIP call
(the pointers passed below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import ternary_weight_linear_w1_amd as bl
from ternary_weight_linear_w1_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_ALIAS, ERR_HIP = range(7)


@pytest.fixture(scope="module")
def L():
    if not _build.up_to_date():
        _build.build()
    return bl.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z0-9_]+)\s*\(", src)))


def P(addr):
    return ctypes.c_void_p(addr)


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(bl.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(7):
        assert bl.status_string(s)
    assert bl.status_string(99) == "unknown status"


def test_pack_workspace_bytes(L):
    def expect(n):
        total, cur = 0, n
        while True:
            cur = -(-cur // 4096)
            total += cur
            if cur == 1:
                return total * 8
    for N, K in [(1, 4), (64, 64), (2560, 2560), (28672, 8192), (4096, 4100)]:
        assert bl.bitlinear_pack_workspace_bytes(N, K) == expect(N * K)
    assert bl.bitlinear_pack_workspace_bytes(3, 6) == 0
    assert bl.bitlinear_pack_workspace_bytes(0, 4) == 0


def test_forward_rejects_before_launch(L):
    f = L.bitlinear_forward
    a = 1 << 20
    args = dict(Xq=P(a), s=P(2 * a), M=1, K=64, W=P(3 * a), g=P(4 * a), N=8, Y=P(5 * a), acc=None, st=None)

    def call(**kw):
        d = dict(args, **kw)
        return f(d["Xq"], d["s"], d["M"], d["K"], d["W"], d["g"], d["N"], d["Y"], d["acc"], d["st"])
    assert call(Xq=None) == ERR_NULL
    assert call(Y=None) == ERR_NULL
    assert call(g=None) == ERR_NULL
    assert call(K=6) == ERR_SHAPE
    assert call(K=0) == ERR_SHAPE
    assert call(M=0) == ERR_SHAPE
    assert call(N=0) == ERR_SHAPE
    assert call(N=1 << 31) == ERR_SHAPE
    assert call(K=(1 << 20) + 4) == ERR_SHAPE
    assert call(Y=P(5 * a + 2)) == ERR_ALIGN
    assert call(Xq=P(a + 1)) == ERR_ALIGN
    assert call(Y=P(3 * a)) == ERR_ALIAS
    assert call(acc=P(5 * a)) == ERR_ALIAS


def test_forward_f32_rejects_before_launch(L):
    f = L.bitlinear_forward_f32
    a = 1 << 20
    assert f(None, 1, 64, None, 1e-5, 0, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_NULL
    assert f(P(a), 1, 62, None, 1e-5, 0, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_SHAPE
    assert f(P(a + 4), 1, 64, None, 1e-5, 0, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_ALIGN
    assert f(P(a), 1, 64, P(2 * a + 8), 1e-5, 0, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_ALIGN
    assert f(P(a), 1, 64, None, 1e-5, 0, P(3 * a), P(4 * a), 8, P(a), None) == ERR_ALIAS
    # activation mode outside {0, 1, 2}; gated rows are 2K floats long (Y inside the up half)
    assert f(P(a), 1, 64, None, 1e-5, 3, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_SHAPE
    assert f(P(a), 1, 64, None, 1e-5, -1, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_SHAPE
    assert f(P(a), 1, 64, None, 1e-5, 2, P(3 * a), P(4 * a), 8, P(a + 300), None) == ERR_ALIAS


def test_forward_workspace_bytes(L):
    f = bl.bitlinear_forward_workspace_bytes
    # K split for 10..32 tokens (8 on >= 64M weights) and K >= 16384: up to 8 slices of >= 4 K steps of 256,
    # about 1024 blocks; slices x M x N int32 partials
    assert f(16, 8192, 28672) == 8 * 16 * 8192 * 4      # 64 tiles of 32 x 128: capped at 8
    assert f(32, 8192, 28672) == 8 * 32 * 8192 * 4
    assert f(32, 40000, 16384) == 3 * 32 * 40000 * 4    # 313 tiles: 1024 / 313 = 3 slices
    assert f(32, 20000, 16384) == 6 * 32 * 20000 * 4    # 157 tiles: 6 slices
    assert f(20, 64, 16384) == 8 * 20 * 64 * 4          # 64 K steps: 16 of 4, capped at 8
    assert f(16, 96, 2560) == 0 and f(32, 10240, 8192) == 0            # short rows: no split
    assert f(7, 8192, 28672) == 0 and f(33, 8192, 28672) == 0          # token range
    assert f(8, 8192, 28672) == 8 * 8 * 8192 * 4        # 8 tokens on >= 64M weights
    assert f(8, 2560, 16384) == 0                       # ... not on smaller matrices
    assert f(12, 2560, 16384) == 8 * 12 * 2560 * 4      # from 10 tokens on any
    assert f(16, 128, 16400) == 0                       # K % 64
    assert f(0, 64, 64) == 0 and f(16, 64, 62) == 0                    # out of range


def test_forward_f32_workspace_bytes(L):
    f = bl.bitlinear_forward_f32_workspace_bytes
    assert f(1, 96, 64) == 0 and f(2, 96, 256) == 0     # one-launch sizes need none
    assert f(15, 96, 256) == 3840 + 256                 # 3..15 tokens: the matrix-core product
    assert f(2, 28672, 8192) == 16384 + 256             # 2 tokens on the largest matrices
    assert f(16, 8, 256) == 4096 + 256                  # codes, then scales, each on 256 bytes
    assert f(100, 130, 260) == 26112 + 512
    assert f(2048, 6912, 6912) == 2048 * 6912 + 8192
    assert f(32, 8192, 28672) == 32 * 28672 + 256 + 8 * 32 * 8192 * 4   # and the K-split partials
    assert f(16, 8, 62) == 0 and f(0, 8, 64) == 0 and f(16, 8, (1 << 20) + 4) == 0   # out of range


def test_forward_f32_ws_rejects_before_launch(L):
    f = L.bitlinear_forward_f32_ws
    a = 1 << 24
    M, K, N = 16, 256, 8
    need = bl.bitlinear_forward_f32_workspace_bytes(M, N, K)

    def call(ws, nbytes, X=P(a), k=K):
        return f(X, M, k, None, 1e-5, 0, P(3 * a), P(4 * a), N, P(5 * a), 0, ws, nbytes, None)

    assert call(None, need) == ERR_NULL
    assert call(P(6 * a), need - 1) == ERR_WORKSPACE
    assert call(P(6 * a + 8), need) == ERR_ALIGN
    assert call(P(5 * a - 64), need) == ERR_ALIAS      # runs into Y
    assert call(P(a + 16), need) == ERR_ALIAS          # inside X (M*K*4 bytes)
    # the one-launch call's own checks come first
    assert call(P(6 * a), need, k=62) == ERR_SHAPE
    assert call(P(6 * a), need, X=None) == ERR_NULL
    # the one-launch call's checks come before the workspace's
    g = f(P(a), 1, K, None, 1e-5, 7, P(3 * a), P(4 * a), N, P(5 * a), 0, None, 0, None)
    assert g == ERR_SHAPE


def test_forward_f32_noalloc_rejects_before_launch(L):
    """The no-allocation call checks its arguments like the workspace call, and rejects
    sizes that need more than its fixed scratch (the header's limit) before any HIP call."""
    m = re.search(r"#define BITLINEAR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == bl.NOALLOC_SCRATCH_BYTES
    a = 1 << 40
    f = L.bitlinear_forward_f32_noalloc
    args = lambda **kw: [kw.get("X", P(a)), kw.get("M", 64), kw.get("K", 2560), kw.get("g", None), 1e-5,
                         kw.get("act", 0), kw.get("W", P(2 * a)), kw.get("gm", P(3 * a)), kw.get("N", 256),
                         kw.get("Y", P(4 * a)), 0, None]
    assert f(*args(X=None)) == ERR_NULL
    assert f(*args(K=2562)) == ERR_SHAPE
    assert f(*args(act=3)) == ERR_SHAPE
    assert f(*args(X=P(a + 4))) == ERR_ALIGN
    assert f(*args(Y=P(2 * a))) == ERR_ALIAS
    # 4096 tokens x 16384: 64 MiB of codes, more than the scratch
    assert f(*args(M=4096, K=16384, N=64)) == ERR_WORKSPACE
    assert bl.bitlinear_forward_f32_workspace_bytes(2048, 28672, 8192) <= bl.NOALLOC_SCRATCH_BYTES


def test_forward_ws_rejects_before_launch(L):
    f = L.bitlinear_forward_ws
    a = 1 << 26
    M, K, N = 32, 16384, 256
    need = bl.bitlinear_forward_workspace_bytes(M, N, K)
    assert need > 0

    def call(ws, nbytes, Xq=P(a), acc=None):
        return f(Xq, P(2 * a), M, K, P(3 * a), P(4 * a), N, P(5 * a), acc, 0, ws, nbytes, None)

    assert call(None, need) == ERR_NULL
    assert call(P(6 * a), need - 4) == ERR_WORKSPACE
    assert call(P(6 * a + 4), need) == ERR_ALIGN
    assert call(P(5 * a + 128), need) == ERR_ALIAS     # inside Y
    assert call(P(6 * a), need, acc=P(6 * a + 4096)) == ERR_ALIAS   # acc inside the workspace
    assert call(P(6 * a), need, Xq=None) == ERR_NULL  # the product's own checks come first


def test_residual_forms_reject_before_launch(L):
    a = 1 << 20
    f = L.bitlinear_forward_residual
    assert f(None, P(2 * a), 1, 64, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_NULL
    assert f(P(a), P(2 * a), 1, 62, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_SHAPE
    assert f(P(a), P(2 * a), 1, 64, P(3 * a), P(4 * a), 8, P(5 * a + 2), None) == ERR_ALIGN
    assert f(P(a), P(2 * a), 1, 64, P(3 * a), P(4 * a), 8, P(3 * a), None) == ERR_ALIAS
    g = L.bitlinear_forward_f32_residual
    assert g(P(a), 1, 64, None, 1e-5, 0, None, P(4 * a), 8, P(5 * a), None) == ERR_NULL
    assert g(P(a), 1, 64, None, 1e-5, 5, P(3 * a), P(4 * a), 8, P(5 * a), None) == ERR_SHAPE
    assert g(P(a), 1, 64, None, 1e-5, 0, P(3 * a), P(4 * a), 8, P(a), None) == ERR_ALIAS


def test_quantize_act_rejects_before_launch(L):
    f = L.bitlinear_quantize_act
    a = 1 << 20
    assert f(None, 1, 64, None, 1e-5, 0, P(2 * a), P(3 * a), None) == ERR_NULL
    assert f(P(a), 1, 66, None, 1e-5, 0, P(2 * a), P(3 * a), None) == ERR_SHAPE
    assert f(P(a), 0, 64, None, 1e-5, 0, P(2 * a), P(3 * a), None) == ERR_SHAPE
    assert f(P(a + 8), 1, 64, None, 1e-5, 0, P(2 * a), P(3 * a), None) == ERR_ALIGN
    assert f(P(a), 1, 64, None, 1e-5, 0, P(a + 16), P(3 * a), None) == ERR_ALIAS
    assert f(P(a), 1, 64, None, 1e-5, 3, P(2 * a), P(3 * a), None) == ERR_SHAPE
    assert f(P(a), 1, 64, None, 1e-5, 2, P(a + 300), P(3 * a), None) == ERR_ALIAS
    assert f(P(a), 1, 64, None, 1e-5, 2, P(2 * a), P(a + 400), None) == ERR_ALIAS


def test_pack_rejects_before_launch(L):
    f = L.bitlinear_pack_weights
    a = 1 << 24
    ws = bl.bitlinear_pack_workspace_bytes(16, 64)
    assert f(None, 16, 64, P(2 * a), P(3 * a), P(4 * a), ws, None) == ERR_NULL
    assert f(P(a), 16, 64, P(2 * a), P(3 * a), None, ws, None) == ERR_NULL
    assert f(P(a), 16, 66, P(2 * a), P(3 * a), P(4 * a), ws, None) == ERR_SHAPE
    assert f(P(a), 16, 64, P(2 * a), P(3 * a), P(4 * a), ws - 8, None) == ERR_WORKSPACE
    assert f(P(a + 4), 16, 64, P(2 * a), P(3 * a), P(4 * a), ws, None) == ERR_ALIGN
    assert f(P(a), 16, 64, P(a + 64), P(3 * a), P(4 * a), ws, None) == ERR_ALIAS


def test_binding_without_gpu_fails_loudly():
    """Without a device the binding must raise, never compute on the CPU."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    w = torch.zeros((4, 8))
    with pytest.raises(ValueError):
        bl.bitlinear_pack_weights(w)


def test_packed5_row_bytes(L):
    f = L.bitlinear_packed5_row_bytes
    assert f(2560) == 512 and f(6912) == 1392 and f(8192) == 1648 and f(80) == 16 and f(84) == 32
    assert f(0) == 0 and f(6) == 0


def test_five_per_byte_calls_reject_before_launch(L):
    a = 1 << 20
    r = L.bitlinear_repack5
    assert r(None, 8, 64, P(2 * a), None) == ERR_NULL
    assert r(P(a), 8, 66, P(2 * a), None) == ERR_SHAPE
    assert r(P(a), 8, 64, P(2 * a + 2), None) == ERR_ALIGN
    assert r(P(a), 8, 64, P(a + 64), None) == ERR_ALIAS
    f = L.bitlinear_forward5
    args = lambda **kw: [kw.get("Xq", P(a)), kw.get("s", P(2 * a)), kw.get("M", 1), kw.get("K", 64),
                         kw.get("W", P(3 * a)), kw.get("g", P(4 * a)), kw.get("N", 8), kw.get("Y", P(5 * a)),
                         kw.get("acc", None), None]
    assert f(*args(W=None)) == ERR_NULL
    assert f(*args(K=68)) == ERR_SHAPE                 # K % 16 != 0
    assert f(*args(K=131072 + 16)) == ERR_SHAPE        # a token's codes no longer fit in LDS
    assert f(*args(Xq=P(a + 4))) == ERR_ALIGN
    assert f(*args(W=P(3 * a + 4))) == ERR_ALIGN
    assert f(*args(Y=P(3 * a))) == ERR_ALIAS
    # a 4-token tile of outputs (4 N floats) must end at or before the offset that masked
    # lanes store to (2^31 - 16), so N = 2^27 is out of range and 2^27 - 1 passes the size
    # checks (and then fails the overlap check of these fake buffers, still before a launch)
    assert f(*args(N=1 << 27)) == ERR_SHAPE
    assert f(*args(N=(1 << 27) - 1)) == ERR_ALIAS


def test_attention_workspace_bytes(L):
    # (M, heads, capacity) -> per (sequence, head): ceil(capacity / 64) chunk records of 128 + 2
    # floats
    for M, H, C in [(1, 20, 4096), (3, 64, 100), (1, 1, 1), (65535, 1, 64)]:
        assert bl.bitlinear_attention_workspace_bytes(M, H, C) == M * H * (-(-C // 64)) * 130 * 4
    for bad in [(0, 20, 64), (1, 0, 64), (1, 20, 0), (65536, 1, 64), (1, 4097, 64), (1, 1, (1 << 24) + 1)]:
        assert bl.bitlinear_attention_workspace_bytes(*bad) == 0


def test_attention_rejects_before_launch(L):
    A = 1 << 20
    qkv, kc, vc, pos, out, ws = P(1 * A), P(64 * A), P(128 * A), P(192 * A), P(200 * A), P(256 * A)
    need = bl.bitlinear_attention_workspace_bytes(1, 20, 4096)
    f = L.bitlinear_attention_decode

    def call(**kw):
        a = dict(qkv=qkv, kc=kc, vc=vc, pos=pos, M=1, H=20, KVH=5, D=128, C=4096, theta=10000.0, out=out, ws=ws,
                 wsb=need)
        a.update(kw)
        return f(a["qkv"], a["kc"], a["vc"], a["pos"], a["M"], a["H"], a["KVH"], a["D"], a["C"], a["theta"],
                 a["out"], a["ws"], a["wsb"], None)

    assert call(qkv=None) == ERR_NULL
    assert call(pos=None) == ERR_NULL
    assert call(ws=None) == ERR_NULL
    assert call(D=64) == ERR_SHAPE
    assert call(KVH=3) == ERR_SHAPE                 # 20 % 3 != 0
    assert call(M=0) == ERR_SHAPE
    assert call(M=65536) == ERR_SHAPE
    assert call(C=0) == ERR_SHAPE
    assert call(C=(1 << 24) + 1) == ERR_SHAPE
    assert call(theta=0.0) == ERR_SHAPE
    assert call(theta=float("nan")) == ERR_SHAPE
    assert call(theta=float("inf")) == ERR_SHAPE
    assert call(wsb=need - 1) == ERR_WORKSPACE
    assert call(qkv=P(A + 4)) == ERR_ALIGN
    assert call(kc=P(64 * A + 8)) == ERR_ALIGN
    assert call(pos=P(192 * A + 2)) == ERR_ALIGN
    assert call(out=P(qkv.value)) == ERR_ALIAS       # output on the input
    assert call(vc=P(kc.value + 4096)) == ERR_ALIAS  # value cache inside the key cache
    assert call(ws=P(out.value)) == ERR_ALIAS
    assert call(pos=P(ws.value + 16)) == ERR_ALIAS   # device pos inside the workspace


def test_peaks_library_exports_and_rejects():
    """The benchmark's calibration kernels: every entry exported; invalid arguments are
    rejected before any launch (no GPU needed)."""
    if not os.path.exists(_build.PEAKS_LIB):
        _build.build()
    K = ctypes.CDLL(_build.PEAKS_LIB)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    K.bl_peak_stream_read.argtypes = [vp, i64, ci, ci, vp, vp]
    K.bl_peak_mfma_i8.argtypes = [ci, ci, vp, vp]
    a = P(1 << 24)
    assert K.bl_peak_stream_read(None, 1024, 256, 4, a, None) == 1
    assert K.bl_peak_stream_read(a, 1000, 256, 4, a, None) == 1           # not a multiple of 16
    assert K.bl_peak_stream_read(P((1 << 24) + 8), 1024, 256, 4, a, None) == 1   # misaligned
    assert K.bl_peak_stream_read(a, 1024, 256, 3, a, None) == 1           # unroll 2, 4 or 8
    assert K.bl_peak_stream_read(a, 1024, 0, 4, a, None) == 1
    assert K.bl_peak_mfma_i8(0, 256, a, None) == 1 and K.bl_peak_mfma_i8(10, 256, None, None) == 1
    K.bl_peak_mfma_valu.argtypes = [ci, ci, ci, vp, vp]
    K.bl_peak_empty.argtypes = [ci, vp, vp]
    assert K.bl_peak_mfma_valu(3, 10, 256, a, None) == 1                  # vector ops 0, 2, 4, 6, 8, 12
    assert K.bl_peak_mfma_valu(4, 0, 256, a, None) == 1 and K.bl_peak_mfma_valu(4, 10, 0, a, None) == 1
    assert K.bl_peak_mfma_valu(4, 10, 256, None, None) == 1
    assert K.bl_peak_empty(0, a, None) == 1 and K.bl_peak_empty(256, None, None) == 1
    K.bl_peak_lds_read.argtypes = [ci, ci, vp, vp]
    assert K.bl_peak_lds_read(0, 256, a, None) == 1 and K.bl_peak_lds_read(10, 0, a, None) == 1
    assert K.bl_peak_lds_read(10, 256, None, None) == 1
