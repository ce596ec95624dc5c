"""Plain CPU oracle of the W1.58A8 BitLinear forward (ctypes wrapper over
``bitlinear_oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` import this package. The product library never uses it.

Every function takes and returns numpy arrays. The BitLinear arithmetic is in the C
file, whose header lists the passages each step follows; the decode attention (rotary
positions, bf16 key/value cache, softmax attention) is plain numpy at the end of this
file, each function citing its passage.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, f32, f64, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
        L.ora_abs_sum.argtypes = [vp, i64]
        L.ora_abs_sum.restype = f64
        L.ora_weight_scale.argtypes = [vp, i64]
        L.ora_weight_scale.restype = f32
        L.ora_weight_codes.argtypes = [vp, i64, f32, vp]
        L.ora_weight_codes.restype = None
        L.ora_pack.argtypes = [vp, i64, i64, vp]
        L.ora_pack.restype = None
        L.ora_unpack.argtypes = [vp, i64, i64, vp]
        L.ora_unpack.restype = i64
        L.ora_pack5_row_bytes.argtypes = [i64]
        L.ora_pack5_row_bytes.restype = i64
        L.ora_pack5.argtypes = [vp, i64, i64, vp]
        L.ora_pack5.restype = None
        L.ora_unpack5.argtypes = [vp, i64, i64, vp]
        L.ora_unpack5.restype = i64
        L.ora_quantize_act.argtypes = [vp, i64, i64, vp, vp]
        L.ora_quantize_act.restype = None
        L.ora_quantize_act_norm.argtypes = [vp, i64, i64, vp, f32, ctypes.c_int, vp, vp, vp]
        L.ora_quantize_act_norm.restype = None
        L.ora_forward.argtypes = [vp, vp, i64, i64, vp, f32, i64, vp, vp]
        L.ora_forward.restype = i64
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def abs_sum(w: np.ndarray) -> float:
    """Pairwise binary64 sum of |w| over the flattened array (see O1 in the C file)."""
    w = _c(w, np.float32).reshape(-1)
    return float(lib().ora_abs_sum(_ptr(w), w.size))


def weight_scale(w: np.ndarray) -> np.float32:
    """gamma = max(fl32(pairwise_sum|W| / numel), 1e-8)."""
    w = _c(w, np.float32).reshape(-1)
    return np.float32(lib().ora_weight_scale(_ptr(w), w.size))


def weight_codes(w: np.ndarray, gamma) -> np.ndarray:
    w = _c(w, np.float32)
    q = np.empty(w.shape, dtype=np.int8)
    lib().ora_weight_codes(_ptr(w), w.size, np.float32(gamma), _ptr(q))
    return q


def pack(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    n, k = q.shape
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    out = np.empty((n, k // 4), dtype=np.uint8)
    lib().ora_pack(_ptr(q), n, k, _ptr(out))
    return out


def unpack(packed: np.ndarray, k: int):
    """Returns (codes [N][K] int8, number of unused 0b11 fields seen)."""
    packed = _c(packed, np.uint8)
    n = packed.shape[0]
    q = np.empty((n, k), dtype=np.int8)
    bad = lib().ora_unpack(_ptr(packed), n, k, _ptr(q))
    return q, int(bad)


def pack5_row_bytes(k: int) -> int:
    return int(lib().ora_pack5_row_bytes(int(k)))


def pack5(q: np.ndarray) -> np.ndarray:
    """Codes int8 [N][K] -> five codes per byte, uint8 [N][16 * ceil(K/80)] (O3b in the C file)."""
    q = _c(q, np.int8)
    n, k = q.shape
    out = np.empty((n, pack5_row_bytes(k)), dtype=np.uint8)
    lib().ora_pack5(_ptr(q), n, k, _ptr(out))
    return out


def unpack5(packed: np.ndarray, k: int):
    """Returns (codes int8 [N][K], number of invalid bytes or non-zero padding digits)."""
    packed = _c(packed, np.uint8)
    n = packed.shape[0]
    if packed.shape[1] != pack5_row_bytes(k):
        raise ValueError("row length must be 16 * ceil(K/80)")
    q = np.empty((n, k), dtype=np.int8)
    bad = lib().ora_unpack5(_ptr(packed), n, k, _ptr(q))
    return q, int(bad)


def pack_weights(w: np.ndarray):
    """Latent fp32 W [N][K] -> (packed uint8 [N][K/4], gamma fp32, codes int8 [N][K])."""
    gamma = weight_scale(w)
    q = weight_codes(w, gamma)
    return pack(q), gamma, q


def quantize_act(x: np.ndarray):
    """x fp32 [M][K] -> (xq int8 [M][K], s fp32 [M])."""
    x = _c(x, np.float32)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    lib().ora_quantize_act(_ptr(x), m, k, _ptr(xq), _ptr(s))
    return xq, s


def quantize_act_norm(u: np.ndarray, gain, eps: float, relu2):
    """Fused [activation] -> RMSNorm(gain, eps) -> absmax quant; gain None = no norm.

    relu2: 0/False = none, 1/True = squared ReLU, 2 = gated squared ReLU (u holds
    [gate | up], 2K values per token)."""
    act = int(relu2)
    u = _c(u, np.float32)
    m, k = u.shape
    if act == 2:
        if k % 2:
            raise ValueError("gated input needs an even row length")
        k //= 2
    xq = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    work = np.empty(k, dtype=np.float32)
    g = None if gain is None else _c(gain, np.float32)
    lib().ora_quantize_act_norm(_ptr(u), m, k, None if g is None else _ptr(g), np.float32(eps),
                                act, _ptr(xq), _ptr(s), _ptr(work))
    return xq, s


def forward(xq: np.ndarray, s: np.ndarray, q: np.ndarray, gamma):
    """xq [M][K] int8, s [M], q [N][K] int8 codes, gamma -> (acc int32 [M][N], y fp32 [M][N])."""
    xq = _c(xq, np.int8)
    s = _c(s, np.float32)
    q = _c(q, np.int8)
    m, k = xq.shape
    n, k2 = q.shape
    if k != k2:
        raise ValueError("K mismatch")
    acc = np.empty((m, n), dtype=np.int32)
    y = np.empty((m, n), dtype=np.float32)
    ovf = lib().ora_forward(_ptr(xq), _ptr(s), m, k, _ptr(q), np.float32(gamma), n, _ptr(acc), _ptr(y))
    if ovf:
        raise OverflowError("%d accumulators exceed int32" % ovf)
    return acc, y


def bitlinear(x: np.ndarray, w: np.ndarray, gain=None, eps: float = 1e-5, relu2=False):
    """Whole path on latent inputs: quantize W and x, accumulate, rescale.
    relu2 as in quantize_act_norm (0, 1, or 2 = gated with x = [gate | up])."""
    packed, gamma, q = pack_weights(w)
    if gain is None and not relu2:
        xq, s = quantize_act(x)
    else:
        xq, s = quantize_act_norm(x, gain, eps, relu2)
    acc, y = forward(xq, s, q, gamma)
    return dict(packed=packed, gamma=gamma, q=q, xq=xq, s=s, acc=acc, y=y)


def attention_ctx1(qkv: np.ndarray, heads: int, kv_heads: int, head_dim: int) -> np.ndarray:
    """Scaled dot-product attention over a single position (BitNet b1.58 深度解析 s.2.4 block
    diagram; grouped-query heads): the softmax over one key is exactly 1 and rotary
    embedding at position 0 is the identity, so each query head outputs the value vector
    of its KV group. Written out literally as softmax-weighted values (no shortcut)."""
    m = qkv.shape[0]
    q_end, k_end = heads * head_dim, (heads + kv_heads) * head_dim
    v = qkv[:, k_end:].reshape(m, kv_heads, head_dim)
    k = qkv[:, q_end:k_end].reshape(m, kv_heads, head_dim)
    q = qkv[:, :q_end].reshape(m, heads, head_dim)
    out = np.empty((m, heads, head_dim), dtype=np.float32)
    group = heads // kv_heads
    for t in range(m):
        for hh in range(heads):
            g = hh // group
            score = np.array([np.dot(q[t, hh].astype(np.float64), k[t, g].astype(np.float64))]) / np.sqrt(head_dim)
            p = np.exp(score - score.max())
            p /= p.sum()                                  # one key: p == [1.0]
            out[t, hh] = (p[0] * v[t, g].astype(np.float64)).astype(np.float32)
    return out.reshape(m, heads * head_dim)


def decode_layer(h: np.ndarray, mats: dict, gains: dict, dims: dict, gated: bool, eps: float = 1e-5,
                 cache=None):
    """One BitNet decode layer on fp32 h [M][H] (standard Transformer block with BitLinear
    in place of nn.Linear: BitNet b1.58 深度解析 s.2.4; subln before O and down and ReLU^2:
    微软AI大模型炸场 s.1-2). mats[name] = (codes int8 [N][K], gamma) for qkv, o, up
    ([2F][K] gate rows then up rows when gated), down; gains g_in, g_attn, g_post, g_ffn.
    Residual adds are fp32. Attention runs at context length 1 (attention_ctx1) unless
    cache = dict(k, v, pos, theta) is given: then attention_decode over that cache, whose
    updated arrays are returned among the intermediates as k and v.
    Returns the new h and the intermediates."""
    def lin(x, name, gain, act):
        q, gamma = mats[name]
        xq, s = quantize_act_norm(x, gain, eps, act)
        return forward(xq, s, q, gamma)[1]

    f32 = np.float32
    qkv = lin(h, "qkv", gains["g_in"], 0)
    extra = {}
    if cache is None:
        o = attention_ctx1(qkv, dims["heads"], dims["kv_heads"], dims["head_dim"])
    else:
        o, extra["k"], extra["v"] = attention_decode(qkv, cache["k"], cache["v"], cache["pos"], dims["heads"],
                                                     dims["kv_heads"], cache["theta"])
        o = o.astype(f32)
    h1 = (h.astype(f32) + lin(o, "o", gains["g_attn"], 0)).astype(f32)
    u = lin(h1, "up", gains["g_post"], 0)
    h2 = (h1 + lin(u, "down", gains["g_ffn"], 2 if gated else 1)).astype(f32)
    return h2, dict(qkv=qkv, o=o, h1=h1, u=u, **extra)


# --------------------------------------------------------------------------------------
# Decode attention at real context length: rotary positions, a bf16 key/value cache and
# grouped-query softmax attention. Plain numpy, binary64 unless a step states otherwise.
# --------------------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotation frequency of pair i: theta^(-2i/D), i = 0 .. D/2-1, in binary64 (rotary
    position embedding, 微软AI大模型炸场 s.2 "特殊设计"; the pages name the method only:
    the original rotary frequencies and base are taken)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -(2.0 * i) / head_dim)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary embedding of head vectors x [..., D] at position pos, binary64: dimension i
    and dimension i + D/2 form a plane rotated by the angle pos * theta^(-2i/D)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    a = pos * rope_inv_freq(2 * h, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_f32(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """The same rotation evaluated in binary32, for keys whose rotated value is rounded
    into the bf16 cache (a rounding decision taken in the kernel's precision): cos and
    sin of the binary64 angle rounded once to binary32, then x1*c - x2*s and x2*c + x1*s
    with every product and the sum rounded to binary32 (no fused multiply-add)."""
    x = np.asarray(x, dtype=np.float32)
    h = x.shape[-1] // 2
    a = pos * rope_inv_freq(2 * h, theta)
    c, s = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    x1, x2 = x[..., :h], x[..., h:]
    lo = np.subtract(np.multiply(x1, c, dtype=np.float32), np.multiply(x2, s, dtype=np.float32), dtype=np.float32)
    hi = np.add(np.multiply(x2, c, dtype=np.float32), np.multiply(x1, s, dtype=np.float32), dtype=np.float32)
    return np.concatenate([lo, hi], axis=-1)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Finite binary32 values to bfloat16 bit patterns (uint16), rounding to nearest with
    ties to even: bfloat16 keeps 8 significant bits and binary32's exponent range, so a
    value m * 2^e (0.5 <= |m| < 1) is rounded to a multiple of 2^(e-8), never finer than
    the smallest bfloat16 step 2^-133."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / quantum) * quantum           # x / quantum is exact; rint is half-even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Value of bfloat16 bit patterns, as binary64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def attention_decode(qkv: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos, heads: int,
                     kv_heads: int, theta: float):
    """One decode step of scaled dot-product attention (BitNet b1.58 深度解析 s.2.4 block
    diagram) with rotary positions (微软AI大模型炸场 s.2) over a key/value cache.

    qkv [M][(heads + 2 kv_heads) D] fp32 holds the new token's query heads, then key heads,
    then value heads. k_cache / v_cache are bf16 bit patterns [M][kv_heads][C][D]; pos [M]
    is the new token's position. For each sequence b with 0 <= pos[b] < C:
      1. the new key is rotated at pos (rope_f32) and it and the new value are rounded
         to bf16 into slot pos of the caches;
      2. query head h (of group h // (heads / kv_heads)) is rotated at pos in binary64
         and scores s_j = q . k_j / sqrt(D) over cached positions j = 0 .. pos;
      3. out_h = sum_j softmax(s)_j v_j.
    A sequence with pos outside [0, C) gets NaN outputs and leaves its caches untouched.
    Returns (out float64 [M][heads D], new k_cache, new v_cache)."""
    qkv = np.asarray(qkv, dtype=np.float32)
    m = qkv.shape[0]
    _, _, cap, d = k_cache.shape
    kc, vc = k_cache.copy(), v_cache.copy()
    group = heads // kv_heads
    out = np.full((m, heads, d), np.nan)
    for b in range(m):
        p = int(pos[b])
        if not 0 <= p < cap:
            continue
        q = qkv[b, :heads * d].reshape(heads, d)
        k = qkv[b, heads * d:(heads + kv_heads) * d].reshape(kv_heads, d)
        v = qkv[b, (heads + kv_heads) * d:(heads + 2 * kv_heads) * d].reshape(kv_heads, d)
        kc[b, :, p, :] = round_bf16(rope_f32(k, p, theta))
        vc[b, :, p, :] = round_bf16(v)
        qr = rope(q, p, theta)
        for h in range(heads):
            g = h // group
            keys = bf16_value(kc[b, g, :p + 1])
            vals = bf16_value(vc[b, g, :p + 1])
            s = keys @ qr[h] / np.sqrt(d)
            w = np.exp(s - s.max())
            out[b, h] = (w / w.sum()) @ vals
    return out.reshape(m, heads * d), kc, vc
