"""W1.58A8 BitLinear forward on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/bitlinear.h`` (``libbitlinear.so``,
built in-tree by ``ternary_weight_linear_w1_amd._build``). Every function here only
checks and marshals arguments; all arithmetic runs in the HIP kernels. PyTorch is used
for device memory and the current stream.

The library must be built; importing works without a GPU, and every call that would
launch work needs a ROCm device. There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIB as _LIB_PATH

__all__ = [
    "BitLinearError", "lib", "status_string", "bitlinear_pack_workspace_bytes", "bitlinear_pack_weights",
    "bitlinear_quantize_act", "bitlinear_forward", "bitlinear_forward_f32", "bitlinear_forward_f32_workspace_bytes",
    "bitlinear_forward_workspace_bytes", "bitlinear_forward_f32_noalloc", "NOALLOC_SCRATCH_BYTES",
    "bitlinear_attention_workspace_bytes",
    "bitlinear_attention_decode", "EXPORTED",
]

EXPORTED = (
    "bitlinear_status_string",
    "bitlinear_pack_workspace_bytes",
    "bitlinear_pack_weights",
    "bitlinear_quantize_act",
    "bitlinear_forward",
    "bitlinear_forward_f32",
    "bitlinear_forward_residual",
    "bitlinear_forward_f32_residual",
    "bitlinear_forward_f32_workspace_bytes",
    "bitlinear_forward_f32_ws",
    "bitlinear_forward_f32_noalloc",
    "bitlinear_forward_workspace_bytes",
    "bitlinear_forward_ws",
    "bitlinear_packed5_row_bytes",
    "bitlinear_repack5",
    "bitlinear_forward5",
    "bitlinear_attention_workspace_bytes",
    "bitlinear_attention_decode",
)

_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def lib() -> ctypes.CDLL:
    """Load ``libbitlinear.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libbitlinear.so is not built; run ternary_weight_linear_w1_amd._build.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        L.bitlinear_status_string.argtypes = [ci]
        L.bitlinear_status_string.restype = ctypes.c_char_p
        L.bitlinear_pack_workspace_bytes.argtypes = [i64, i64]
        L.bitlinear_pack_workspace_bytes.restype = ctypes.c_size_t
        L.bitlinear_pack_weights.argtypes = [vp, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
        L.bitlinear_pack_weights.restype = ci
        L.bitlinear_quantize_act.argtypes = [vp, i64, i64, vp, f32, ci, vp, vp, vp]
        L.bitlinear_quantize_act.restype = ci
        L.bitlinear_forward.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp]
        L.bitlinear_forward.restype = ci
        L.bitlinear_forward_f32.argtypes = [vp, i64, i64, vp, f32, ci, vp, vp, i64, vp, vp]
        L.bitlinear_forward_f32.restype = ci
        L.bitlinear_forward_residual.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp]
        L.bitlinear_forward_residual.restype = ci
        L.bitlinear_forward_f32_residual.argtypes = [vp, i64, i64, vp, f32, ci, vp, vp, i64, vp, vp]
        L.bitlinear_forward_f32_residual.restype = ci
        L.bitlinear_forward_f32_workspace_bytes.argtypes = [i64, i64, i64]
        L.bitlinear_forward_f32_workspace_bytes.restype = ctypes.c_size_t
        L.bitlinear_forward_f32_ws.argtypes = [vp, i64, i64, vp, f32, ci, vp, vp, i64, vp, ci, vp, ctypes.c_size_t, vp]
        L.bitlinear_forward_f32_ws.restype = ci
        L.bitlinear_forward_f32_noalloc.argtypes = [vp, i64, i64, vp, f32, ci, vp, vp, i64, vp, ci, vp]
        L.bitlinear_forward_f32_noalloc.restype = ci
        L.bitlinear_forward_workspace_bytes.argtypes = [i64, i64, i64]
        L.bitlinear_forward_workspace_bytes.restype = ctypes.c_size_t
        L.bitlinear_forward_ws.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, ci, vp, ctypes.c_size_t, vp]
        L.bitlinear_forward_ws.restype = ci
        L.bitlinear_packed5_row_bytes.argtypes = [i64]
        L.bitlinear_packed5_row_bytes.restype = i64
        L.bitlinear_repack5.argtypes = [vp, i64, i64, vp, vp]
        L.bitlinear_repack5.restype = ci
        L.bitlinear_forward5.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp]
        L.bitlinear_forward5.restype = ci
        L.bitlinear_attention_workspace_bytes.argtypes = [i64, i64, i64]
        L.bitlinear_attention_workspace_bytes.restype = ctypes.c_size_t
        L.bitlinear_attention_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_double, vp, vp,
                                                 ctypes.c_size_t, vp]
        L.bitlinear_attention_decode.restype = ci
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bitlinear_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise BitLinearError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A tensor allocated here for the call's outputs or scratch. The caching allocator
    ties a block to the stream that was current at allocation; when the work goes to
    another stream, the block is marked as used there too, so that it is not handed out
    again before that stream's kernels are done with it."""
    import torch
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _need(t, dtype, name, ndim=None, shape=None):
    """Device, dtype, contiguity and (when given) rank and exact shape of a tensor argument:
    the library trusts the sizes it is given, so a short buffer must not get through."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def bitlinear_pack_workspace_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_pack_workspace_bytes(int(N), int(K)))


def bitlinear_pack_weights(W, packed=None, gamma=None, workspace=None, stream=None):
    """Latent fp32 weights [N][K] -> (packed uint8 [N][K/4], gamma fp32 [1])."""
    import torch
    _need(W, torch.float32, "W", 2)
    N, K = W.shape
    if packed is None:
        packed = _empty((N, K // 4), torch.uint8, W.device, stream)
    _need(packed, torch.uint8, "packed", shape=(N, K // 4))
    if gamma is None:
        gamma = _empty((1,), torch.float32, W.device, stream)
    _need(gamma, torch.float32, "gamma", shape=(1,))
    nbytes = bitlinear_pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = _empty((max(nbytes, 8),), torch.uint8, W.device, stream)
    _check(lib().bitlinear_pack_weights(_ptr(W), N, K, _ptr(packed), _ptr(gamma), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)),
           "bitlinear_pack_weights")
    return packed, gamma


def _act_mode(act, X):
    """Activation mode (0 none, 1 squared ReLU, 2 gated: X rows are [gate | up]) and K."""
    act = int(act)
    if act not in (0, 1, 2):
        raise ValueError("act must be 0, 1 or 2")
    M, K = X.shape
    if act == 2:
        if K % 2:
            raise ValueError("gated input needs rows of 2K values")
        K //= 2
    return act, M, K


def bitlinear_quantize_act(X, gain=None, eps: float = 1e-5, act=0, xq=None, scale=None, stream=None):
    """fp32 activations [M][K] ([M][2K] when act == 2) -> (int8 codes [M][K], scale fp32 [M])."""
    import torch
    _need(X, torch.float32, "X", 2)
    act, M, K = _act_mode(act, X)
    if gain is not None:
        _need(gain, torch.float32, "gain", shape=(K,))
    if xq is None:
        xq = _empty((M, K), torch.int8, X.device, stream)
    _need(xq, torch.int8, "xq", shape=(M, K))
    if scale is None:
        scale = _empty((M,), torch.float32, X.device, stream)
    _need(scale, torch.float32, "scale", shape=(M,))
    _check(lib().bitlinear_quantize_act(_ptr(X), M, K, _ptr(gain), float(eps), act, _ptr(xq),
                                        _ptr(scale), _stream(stream)), "bitlinear_quantize_act")
    return xq, scale


def bitlinear_forward_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes of bitlinear_forward_ws (0: no split for these sizes)."""
    return int(lib().bitlinear_forward_workspace_bytes(int(M), int(N), int(K)))


def bitlinear_forward(Xq, x_scale, W_packed, gamma, y=None, acc=None, stream=None, residual=False,
                      workspace=None, split=True):
    """int8 activations + packed ternary weights -> fp32 y [M][N] (and int32 acc if given).
    residual=True adds the product to the given y (no acc). With 10 to 32 tokens (8 on matrices of >= 64M weights) and
    long rows the call goes through bitlinear_forward_ws (K split across blocks; the workspace, uint8 of at least
    bitlinear_forward_workspace_bytes(M, N, K), is allocated here when not given);
    split=False calls bitlinear_forward / bitlinear_forward_residual (same result)."""
    import torch
    _need(Xq, torch.int8, "Xq", 2)
    _need(W_packed, torch.uint8, "W_packed", 2)
    M, K = Xq.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must have K/4 columns")
    _need(x_scale, torch.float32, "x_scale", shape=(M,))
    _need(gamma, torch.float32, "gamma", shape=(1,))
    if residual:
        if y is None or acc is not None:
            raise ValueError("residual needs y and takes no acc")
        _need(y, torch.float32, "y", shape=(M, N))
    else:
        if y is None:
            y = _empty((M, N), torch.float32, Xq.device, stream)
        _need(y, torch.float32, "y", shape=(M, N))
        if acc is True:
            acc = _empty((M, N), torch.int32, Xq.device, stream)
        if isinstance(acc, torch.Tensor):
            _need(acc, torch.int32, "acc", shape=(M, N))
    accp = _ptr(acc if isinstance(acc, torch.Tensor) else None)
    need = bitlinear_forward_workspace_bytes(M, N, K)
    if split and (need > 0 or workspace is not None):
        if workspace is None:
            workspace = _empty((need,), torch.uint8, Xq.device, stream)
        _need(workspace, torch.uint8, "workspace", 1)
        if workspace.numel() < need:
            raise ValueError("workspace must hold %d bytes" % need)
        _check(lib().bitlinear_forward_ws(_ptr(Xq), _ptr(x_scale), M, K, _ptr(W_packed), _ptr(gamma), N, _ptr(y), accp,
                                          int(bool(residual)), _ptr(workspace), workspace.numel(), _stream(stream)),
               "bitlinear_forward_ws")
    elif residual:
        _check(lib().bitlinear_forward_residual(_ptr(Xq), _ptr(x_scale), M, K, _ptr(W_packed), _ptr(gamma), N,
                                                _ptr(y), _stream(stream)), "bitlinear_forward_residual")
    else:
        _check(lib().bitlinear_forward(_ptr(Xq), _ptr(x_scale), M, K, _ptr(W_packed), _ptr(gamma), N, _ptr(y), accp,
                                       _stream(stream)), "bitlinear_forward")
    return (y, acc) if isinstance(acc, torch.Tensor) else y


def bitlinear_forward_f32_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes of bitlinear_forward_f32_ws (0: none needed)."""
    return int(lib().bitlinear_forward_f32_workspace_bytes(int(M), int(N), int(K)))


def bitlinear_forward_f32(X, W_packed, gamma, gain=None, eps: float = 1e-5, act=0, y=None, stream=None,
                          residual=False, workspace=None, one_launch=False):
    """Fused quantize + product from fp32 activations [M][K] ([M][2K] when act == 2) -> fp32 y [M][N].
    residual=True adds the product to the given y. Where the product runs on the matrix cores
    (from 16 tokens; 3..15 tokens; 2 on the largest matrices) the call goes through
    bitlinear_forward_f32_ws (quantize into a workspace, then the matrix-core product); the
    workspace (uint8, at least bitlinear_forward_f32_workspace_bytes(M, N, K)) is allocated here
    when not given. one_launch=True calls the one-launch entry whatever M (same result)."""
    import torch
    _need(X, torch.float32, "X", 2)
    _need(W_packed, torch.uint8, "W_packed", 2)
    _need(gamma, torch.float32, "gamma", shape=(1,))
    act, M, K = _act_mode(act, X)
    if gain is not None:
        _need(gain, torch.float32, "gain", shape=(K,))
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must have K/4 columns")
    if residual:
        if y is None:
            raise ValueError("residual needs y")
        _need(y, torch.float32, "y", shape=(M, N))
        fn, name = lib().bitlinear_forward_f32_residual, "bitlinear_forward_f32_residual"
    else:
        if y is None:
            y = _empty((M, N), torch.float32, X.device, stream)
        _need(y, torch.float32, "y", shape=(M, N))
        fn, name = lib().bitlinear_forward_f32, "bitlinear_forward_f32"
    need = bitlinear_forward_f32_workspace_bytes(M, N, K)
    if not one_launch and (need > 0 or workspace is not None):
        if workspace is None:
            workspace = _empty((need,), torch.uint8, X.device, stream)
        _need(workspace, torch.uint8, "workspace", 1)
        if workspace.numel() < need:
            raise ValueError("workspace must hold %d bytes" % need)
        _check(lib().bitlinear_forward_f32_ws(_ptr(X), M, K, _ptr(gain), float(eps), act, _ptr(W_packed), _ptr(gamma),
                                              N, _ptr(y), int(bool(residual)), _ptr(workspace), workspace.numel(),
                                              _stream(stream)), "bitlinear_forward_f32_ws")
        return y
    _check(fn(_ptr(X), M, K, _ptr(gain), float(eps), act, _ptr(W_packed), _ptr(gamma), N, _ptr(y), _stream(stream)),
           name)
    return y


# Fixed scratch of bitlinear_forward_f32_noalloc (BITLINEAR_NOALLOC_SCRATCH_BYTES in the header).
NOALLOC_SCRATCH_BYTES = 32 << 20


def bitlinear_forward_f32_noalloc(X, W_packed, gamma, y, gain=None, eps: float = 1e-5, act=0, stream=None,
                                  residual=False):
    """The fused call without any allocation, here or in the library: the library's fixed
    per-device scratch serves as the workspace (sizes needing more than
    NOALLOC_SCRATCH_BYTES are rejected). y must be given. Calls that may overlap on one
    device share that scratch and must be ordered by the caller."""
    import torch
    _need(X, torch.float32, "X", 2)
    _need(W_packed, torch.uint8, "W_packed", 2)
    _need(gamma, torch.float32, "gamma", shape=(1,))
    act, M, K = _act_mode(act, X)
    if gain is not None:
        _need(gain, torch.float32, "gain", shape=(K,))
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must have K/4 columns")
    _need(y, torch.float32, "y", shape=(M, N))
    _check(lib().bitlinear_forward_f32_noalloc(_ptr(X), M, K, _ptr(gain), float(eps), act, _ptr(W_packed), _ptr(gamma),
                                               N, _ptr(y), int(bool(residual)), _stream(stream)),
           "bitlinear_forward_f32_noalloc")
    return y


def bitlinear_packed5_row_bytes(K: int) -> int:
    """Bytes per row of the five-codes-per-byte format: 16 * ceil(K / 80)."""
    return int(lib().bitlinear_packed5_row_bytes(int(K)))


def bitlinear_repack5(W_packed, out=None, stream=None):
    """2-bit packed weights [N][K/4] -> five codes per byte [N][16 * ceil(K/80)]."""
    import torch
    _need(W_packed, torch.uint8, "W_packed", 2)
    N, K = W_packed.shape[0], W_packed.shape[1] * 4
    rb = bitlinear_packed5_row_bytes(K)
    if out is None:
        out = _empty((N, rb), torch.uint8, W_packed.device, stream)
    _need(out, torch.uint8, "out", shape=(N, rb))
    _check(lib().bitlinear_repack5(_ptr(W_packed), N, K, _ptr(out), _stream(stream)), "bitlinear_repack5")
    return out


def bitlinear_forward5(Xq, x_scale, W_packed5, gamma, y=None, acc=None, stream=None):
    """bitlinear_forward on weights packed five codes per byte."""
    import torch
    _need(Xq, torch.int8, "Xq", 2)
    _need(W_packed5, torch.uint8, "W_packed5", 2)
    M, K = Xq.shape
    N = W_packed5.shape[0]
    if W_packed5.shape[1] != bitlinear_packed5_row_bytes(K):
        raise ValueError("W_packed5 must have 16 * ceil(K/80) columns")
    _need(x_scale, torch.float32, "x_scale", shape=(M,))
    _need(gamma, torch.float32, "gamma", shape=(1,))
    if y is None:
        y = _empty((M, N), torch.float32, Xq.device, stream)
    _need(y, torch.float32, "y", shape=(M, N))
    if acc is True:
        acc = _empty((M, N), torch.int32, Xq.device, stream)
    if isinstance(acc, torch.Tensor):
        _need(acc, torch.int32, "acc", shape=(M, N))
    _check(lib().bitlinear_forward5(_ptr(Xq), _ptr(x_scale), M, K, _ptr(W_packed5), _ptr(gamma), N, _ptr(y),
                                    _ptr(acc if isinstance(acc, torch.Tensor) else None), _stream(stream)),
           "bitlinear_forward5")
    return (y, acc) if isinstance(acc, torch.Tensor) else y


def bitlinear_attention_workspace_bytes(M: int, heads: int, capacity: int) -> int:
    return int(lib().bitlinear_attention_workspace_bytes(int(M), int(heads), int(capacity)))


def bitlinear_attention_decode(qkv, k_cache, v_cache, pos, heads: int, kv_heads: int, theta: float = 10000.0,
                               out=None, workspace=None, stream=None):
    """Decode attention of one new token per sequence over its bf16 key/value cache
    (rotary positions, grouped-query heads, head_dim 128).

    qkv fp32 [M][(heads + 2 kv_heads) * 128]; k_cache, v_cache bfloat16
    [M][kv_heads][capacity][128] (slot pos[t] is written); pos int32 [M] on the device.
    Returns out fp32 [M][heads * 128]. ``workspace`` (uint8, at least
    bitlinear_attention_workspace_bytes bytes) is allocated when not given."""
    import torch
    _need(qkv, torch.float32, "qkv", 2)
    M = qkv.shape[0]
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    d = 128
    capacity = k_cache.shape[2]
    _need(qkv, torch.float32, "qkv", shape=(M, (heads + 2 * kv_heads) * d))
    _need(k_cache, torch.bfloat16, "k_cache", shape=(M, kv_heads, capacity, d))
    _need(v_cache, torch.bfloat16, "v_cache", shape=(M, kv_heads, capacity, d))
    _need(pos, torch.int32, "pos", shape=(M,))
    if out is None:
        out = _empty((M, heads * d), torch.float32, qkv.device, stream)
    _need(out, torch.float32, "out", shape=(M, heads * d))
    need = bitlinear_attention_workspace_bytes(M, heads, capacity)
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, qkv.device, stream)
    _need(workspace, torch.uint8, "workspace", 1)
    _check(lib().bitlinear_attention_decode(_ptr(qkv), _ptr(k_cache), _ptr(v_cache), _ptr(pos), M, int(heads),
                                            int(kv_heads), d, capacity, float(theta), _ptr(out), _ptr(workspace),
                                            workspace.numel(), _stream(stream)),
           "bitlinear_attention_decode")
    return out

