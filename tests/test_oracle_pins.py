"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived examples (tests/golden/hand_examples.json), closed forms, library
routines (math.fsum, numpy integer matmul, scipy special functions), brute force in
fp64, and invariants of the definitions. Each test names the mistake it would catch.
"""
import math

import numpy as np
import pytest
from scipy.special import gammainc, gammaln, ndtr

import datagen

F32 = np.float32


# ----------------------------------------------------------------------------- O1 gamma

def test_gamma_gaussian_closed_form(ora):
    """E|W| = sigma*sqrt(2/pi) for W ~ N(0, sigma^2). Catches a dropped abs, a wrong
    divisor (N instead of N*K) or a per-row mean."""
    w = datagen.gaussian_weights(2560, 2560, datagen.stream_id(1, role=1))
    g = float(ora.weight_scale(w))
    expect = 0.02 * math.sqrt(2.0 / math.pi)
    se = expect * math.sqrt(math.pi / 2.0 - 1.0) / math.sqrt(w.size)
    assert abs(g - expect) < 5 * se, (g, expect, se)


def test_abs_sum_vs_fsum_bound(ora):
    """Pairwise binary64 sum against the correctly rounded sum (math.fsum) within the
    pairwise error bound ceil(log2 n) * 2^-53 * sum|x|."""
    rng = datagen.rng(99)
    for n in (1, 2, 3, 7, 1000, 65537, 1 << 20):
        w = (rng.standard_normal(n) * rng.uniform(0.01, 100.0)).astype(np.float32)
        s = ora.abs_sum(w)
        exact = math.fsum(abs(float(v)) for v in w)
        bound = max(1, math.ceil(math.log2(max(n, 2)))) * 2.0 ** -53 * exact
        assert abs(s - exact) <= bound, (n, s, exact)


def test_abs_sum_is_pairwise_not_sequential(ora):
    """[1, 0, 0, 0, 2^-53, 2^-53] (n = 6, tree padded to 8): the pairwise tree adds the
    two 2^-53 first, giving 1 + 2^-52 exactly; a left-to-right sum loses both (1.0)."""
    t = 2.0 ** -53
    w = np.array([1.0, 0.0, 0.0, 0.0, t, t], dtype=np.float32)
    assert ora.abs_sum(w) == 1.0 + 2.0 ** -52
    seq = 0.0
    for v in w:
        seq += abs(float(v))
    assert seq == 1.0


def test_gamma_floor_and_sign_pattern(ora):
    """All-zero W takes the 1e-8 floor; W = c * sign pattern gives gamma = c and q = sign."""
    z = np.zeros((4, 8), dtype=np.float32)
    assert ora.weight_scale(z) == F32(1e-8)
    packed, gamma, q = ora.pack_weights(z)
    assert (q == 0).all()
    signs = np.where(datagen.rng(5).random((16, 64)) < 0.5, -1.0, 1.0).astype(np.float32)
    w = signs * F32(0.0123)
    packed, gamma, q = ora.pack_weights(w)
    assert gamma == F32(0.0123)
    assert (q == signs.astype(np.int8)).all()


def test_gamma_final_rounding_golden(ora, golden):
    """gamma = fl32(S / n) with the binary64 quotient rounded once: two hand cases in which
    rounding the sum (and n) to binary32 before dividing gives another binary32 value, one
    with n = 3 and one with n = 2^24 + 1, where n itself is not a binary32 value. Catches
    (float)S / (float)n and (float)S / n."""
    cases = golden["gamma_final_rounding"]["cases"]
    w = np.array(cases[0]["W"], np.float32)
    assert ora.weight_scale(w) == F32(cases[0]["gamma"])
    assert F32(cases[0]["gamma"]) != F32(cases[0]["gamma_if_sum_rounded_to_fp32_first"])
    big = cases[1]
    w = np.full(big["n"], F32(1.0) + F32(2.0 ** -23), np.float32)
    assert ora.abs_sum(w) == 2.0 ** 24 + 3.0 + 2.0 ** -23
    assert ora.weight_scale(w) == F32(big["gamma"])
    assert F32(big["gamma"]) != F32(big["gamma_if_sum_and_n_rounded_to_fp32_first"])


# ----------------------------------------------------------------------------- O2 codes

def test_weight_ties_golden(ora, golden):
    """Hand example: ties go to even and codes are clipped to [-1, 1]."""
    g = golden["weight_ties"]
    w = np.array(g["W"], dtype=np.float32)
    packed, gamma, q = ora.pack_weights(w)
    assert gamma == F32(g["gamma"])
    assert q.tolist() == g["codes"]
    assert packed.tolist() == g["packed"]


def test_codes_brute_force_tiny(ora):
    """Codes against a direct restatement on python floats (fp32 quotient through numpy
    scalars, round-half-even through Python's round) on a tiny matrix."""
    w = datagen.gaussian_weights(7, 12, 77)
    gamma = ora.weight_scale(w)
    q = ora.weight_codes(w, gamma)
    for i in range(7):
        for k in range(12):
            r = round(float(F32(w[i, k]) / F32(gamma)))
            assert q[i, k] == max(-1, min(1, r))


def test_gaussian_split_closed_form(ora):
    """For Gaussian latents P(q=0) = 2*Phi(sqrt(2/pi)/2) - 1 = 0.31006. Catches the
    threshold-at-mean variant (57.5% zeros) and a half-away rounding of the ratio."""
    w = datagen.gaussian_weights(2048, 2048, datagen.stream_id(1, role=2))
    _, gamma, q = ora.pack_weights(w)
    p0 = float((q == 0).mean())
    expect = 2.0 * ndtr(math.sqrt(2.0 / math.pi) / 2.0) - 1.0
    assert abs(p0 - expect) < 2e-3, (p0, expect)
    assert abs(float((q == 1).mean()) - (1 - expect) / 2) < 2e-3
    threshold_variant = 2.0 * ndtr(math.sqrt(2.0 / math.pi)) - 1.0
    assert abs(p0 - threshold_variant) > 0.2


def test_trained_like_split_matches_pages(ora):
    """Generalized-Gaussian (beta = 0.846) latents: closed form through the regularized
    incomplete gamma, and the pages' trained-weight split 42% / 29% / 29%
    (BitNet b1.58 深度解析 s.2.3) within half a percent."""
    b = datagen.GG_BETA_TRAINED
    w = datagen.gg_weights(1024, 4096, datagen.stream_id(2, role=3))
    _, gamma, q = ora.pack_weights(w)
    p0 = float((q == 0).mean())
    pp = float((q == 1).mean())
    pm = float((q == -1).mean())
    t = math.exp(gammaln(2 / b) - gammaln(1 / b)) / 2
    expect0 = gammainc(1 / b, t ** b)
    assert abs(p0 - expect0) < 2e-3
    assert abs(p0 - 0.42) < 0.005 and abs(pp - 0.29) < 0.005 and abs(pm - 0.29) < 0.005


# ----------------------------------------------------------------------------- O3 pack

def test_pack_golden_and_roundtrip(ora, golden):
    g = golden["pack_order"]
    q = np.array(g["codes"], dtype=np.int8)
    p = ora.pack(q)
    assert p.tolist() == g["packed"]
    w = datagen.gaussian_weights(33, 260, 3)
    packed, gamma, q = ora.pack_weights(w)
    q2, bad = ora.unpack(packed, 260)
    assert bad == 0 and (q2 == q).all()
    fields = np.stack([(packed >> (2 * i)) & 3 for i in range(4)])
    assert (fields != 3).all()


def test_pack_rejects_ragged_k(ora):
    with pytest.raises(ValueError):
        ora.pack(np.zeros((2, 6), dtype=np.int8))


# ----------------------------------------------------------------------------- O4 act quant

def test_act_quant_golden(ora, golden):
    g = golden["act_quant"]
    xq, s = ora.quantize_act(np.array(g["X"], dtype=np.float32))
    assert s.tolist() == g["scale"]
    assert xq.tolist() == g["codes"]


def test_act_quant_invariants(ora):
    """Per-token max|xq| = 127 exactly; odd symmetry; power-of-two scale invariance;
    tokens with different ranges get different scales (per token, not per tensor)."""
    x = datagen.outlier_acts(64, 2560, 11)
    x[3] *= 1000.0
    xq, s = ora.quantize_act(x)
    assert (np.abs(xq.astype(np.int32)).max(axis=1) == 127).all()
    assert (xq != -128).all()
    assert s[3] < s[2] / 100.0
    xq2, s2 = ora.quantize_act(-x)
    assert (xq2 == -xq).all() and (s2 == s).all()
    xq3, s3 = ora.quantize_act(x * F32(8.0))
    assert (xq3 == xq).all() and (s3 == s / F32(8.0)).all()


def test_act_quant_brute_force(ora):
    """Every code against a restatement with numpy fp32 scalars and round-half-even."""
    x = datagen.outlier_acts(3, 300, 12)
    xq, s = ora.quantize_act(x)
    for t in range(3):
        m = max(float(np.abs(x[t]).max()), 1e-8)
        st = F32(127.0) / F32(m)
        assert s[t] == st
        for k in range(300):
            r = round(float(F32(x[t, k]) * st))
            assert xq[t, k] == max(-128, min(127, r))


def test_act_quant_zero_row(ora):
    x = np.zeros((2, 8), dtype=np.float32)
    xq, s = ora.quantize_act(x)
    assert (xq == 0).all() and s[0] == F32(127.0) / F32(1e-8)


# ----------------------------------------------------------------------------- O5 prologue

def test_prologue_golden(ora, golden):
    g = golden["relu2_norm"]
    u = np.array(g["U"], dtype=np.float32)
    xq, s = ora.quantize_act_norm(u, np.array(g["gain"], np.float32), g["eps"], True)
    assert xq.tolist() == g["codes"]
    expect = F32(31.75 * math.sqrt(4.015625 + float(F32(g["eps"]))))
    assert s[0] == expect


def test_prologue_constant_row_closed_form(ora):
    """u_k = a, g = 1: RMSNorm output is a/sqrt(a^2+eps) for every k, so codes are
    127*sign(a) and the stored scale is (127/|a|) * sqrt(a^2 + eps)."""
    for a in (2.0, -0.75, 1e-3):
        u = np.full((1, 256), a, dtype=np.float32)
        xq, s = ora.quantize_act_norm(u, np.ones(256, np.float32), 1e-5, False)
        assert (xq == (127 if a > 0 else -127)).all()
        ref = (127.0 / abs(a)) * math.sqrt(a * a + float(F32(1e-5)))
        assert abs(float(s[0]) - ref) <= 2 * abs(ref) * 2.0 ** -24


def test_prologue_matches_normalize_then_quantize(ora):
    """Independent check of the reading that the norm's per-token factor cancels:
    normalize in fp64 (v/sqrt(mean v^2 + eps) * g), quantize in fp64, and compare.
    Codes may differ only where x*s lands within rounding noise of a .5 boundary
    (at most by 1, very rarely); scales agree to a few fp32 ulps."""
    u = datagen.outlier_acts(32, 6912, 21)
    g = datagen.gains(6912, 22)
    for relu2 in (False, True):
        xq, s = ora.quantize_act_norm(u, g, 1e-5, relu2)
        v = u.astype(np.float64)
        if relu2:
            v = np.maximum(v, 0.0) ** 2
        r = 1.0 / np.sqrt((v * v).mean(axis=1, keepdims=True) + float(F32(1e-5)))
        xn = v * r * g.astype(np.float64)
        sn = 127.0 / np.abs(xn).max(axis=1, keepdims=True)
        ref = np.clip(np.round(xn * sn), -128, 127).astype(np.int32)
        diff = np.abs(ref - xq.astype(np.int32))
        assert diff.max() <= 1
        assert (diff > 0).mean() < 1e-4
        assert np.allclose(s.astype(np.float64), sn[:, 0], rtol=3e-7, atol=0)


def test_prologue_codes_equal_plain_quant_of_gained_input(ora):
    """The codes of the fused path are the plain absmax codes of fl(v * g) and do not
    depend on eps or on a power-of-two scaling of u (without ReLU^2)."""
    u = datagen.outlier_acts(8, 2560, 31)
    g = datagen.gains(2560, 32)
    xq, s = ora.quantize_act_norm(u, g, 1e-5, False)
    xq_plain, _ = ora.quantize_act((u * g).astype(np.float32))
    assert (xq == xq_plain).all()
    xq2, s2 = ora.quantize_act_norm(u * F32(4.0), g, 1e-5, False)
    assert (xq2 == xq).all()
    xq3, _ = ora.quantize_act_norm(u, g, 0.5, False)
    assert (xq3 == xq).all()
    ur = datagen.outlier_acts(8, 2560, 33)
    xq4, _ = ora.quantize_act_norm(ur, g, 1e-5, True)
    pos = np.maximum(ur, 0)
    xq5, _ = ora.quantize_act((pos * pos * g).astype(np.float32))
    assert (xq4 == xq5).all()
    assert (xq4[ur <= 0] == 0).all()


def test_prologue_without_gain_is_plain(ora):
    u = datagen.outlier_acts(4, 512, 41)
    xq, s = ora.quantize_act_norm(u, None, 1e-5, False)
    xq2, s2 = ora.quantize_act(u)
    assert (xq == xq2).all() and (s == s2).all()


# ----------------------------------------------------------------------------- O6/O7 forward

def test_forward_golden(ora, golden):
    g = golden["forward"]
    r = ora.bitlinear(np.array(g["X"], np.float32), np.array(g["W"], np.float32))
    assert r["acc"].tolist() == g["acc"]
    c = F32(1.0) / F32(127.0)
    assert r["y"][0, 0] == F32(32.0) * c and r["y"][0, 1] == F32(-191.0) * c


def test_forward_rescale_order_golden(ora, golden):
    """y = fl32(fl32(acc) * fl32(gamma / s)): a hand case (gamma = 1, s = 3, acc = 5) where
    scaling by gamma and then dividing by s lands one unit lower. Catches the other
    association and a product with an unrounded gamma / s."""
    g = golden["rescale_order"]
    acc, y = ora.forward(np.array(g["xq"], np.int8), np.array(g["s"], np.float32), np.array(g["codes"], np.int8),
                         F32(g["gamma"]))
    assert acc.tolist() == g["acc"]
    assert y.tolist() == [[float(F32(v)) for v in row] for row in g["y"]]
    assert y[0, 0] != F32(g["y0_if_scaled_by_gamma_then_divided_by_s"])


def test_forward_acc_vs_integer_matmul(ora):
    """Accumulators against numpy's int64 matmul (a library primitive), non-square and
    ragged shapes so that a transposed operand cannot pass."""
    for (m, n, k) in ((1, 37, 260), (5, 64, 68), (3, 19, 1024)):
        w = datagen.gg_weights(n, k, 100 + k)
        x = datagen.outlier_acts(m, k, 200 + k)
        r = ora.bitlinear(x, w)
        ref = r["xq"].astype(np.int64) @ r["q"].astype(np.int64).T
        assert (r["acc"].astype(np.int64) == ref).all()


def test_forward_vs_dense_fp64_dequantized(ora):
    """y against a dense fp64 product of the dequantized operands, (q*gamma) and
    (xq/s): relative error within 3e-7 (two fp32 roundings) and exact zeros."""
    m, n, k = 4, 96, 2560
    w = datagen.gg_weights(n, k, 301)
    x = datagen.outlier_acts(m, k, 302)
    r = ora.bitlinear(x, w)
    wd = r["q"].astype(np.float64) * float(r["gamma"])
    xd = r["xq"].astype(np.float64) / r["s"].astype(np.float64)[:, None]
    ref = xd @ wd.T
    y = r["y"].astype(np.float64)
    # fp64 round-off of the dense sum, used only where the exact result is zero
    noise = 1e-13 * (np.abs(xd) @ np.abs(wd).T)
    zero = np.abs(ref) <= noise
    assert (y[zero] == 0).all()
    rel = np.abs(y[~zero] - ref[~zero]) / np.abs(ref[~zero])
    assert rel.max() < 3e-7
    # and the quantized product approximates the latent product
    latent = x.astype(np.float64) @ w.astype(np.float64).T
    cos = (latent * ref).sum() / np.sqrt((latent ** 2).sum() * (ref ** 2).sum())
    assert cos > 0.6


def test_forward_one_hot(ora):
    """A single nonzero activation x_k: xq = +-127 at k and y_n = gamma * q_nk * x_k
    (the textbook special case) within a few ulp."""
    n, k = 32, 64
    w = datagen.gaussian_weights(n, k, 401)
    x = np.zeros((1, k), dtype=np.float32)
    x[0, 17] = F32(-3.25)
    r = ora.bitlinear(x, w)
    assert r["xq"][0, 17] == -127 and (np.delete(r["xq"][0], 17) == 0).all()
    expect = float(r["gamma"]) * r["q"][:, 17].astype(np.float64) * -3.25
    assert np.allclose(r["y"][0].astype(np.float64), expect, rtol=4e-7, atol=0)


def test_forward_bound(ora):
    """|acc| <= 127 * nnz(row of q)."""
    w = datagen.gg_weights(64, 512, 501)
    x = datagen.heavy_channel_acts(8, 512, 502)
    r = ora.bitlinear(x, w)
    nnz = (r["q"] != 0).sum(axis=1)
    assert (np.abs(r["acc"]) <= 127 * nnz[None, :]).all()


# ----------------------------------------------------------------------------- gated FFN input

def test_gated_golden(ora, golden):
    g = golden["gated_relu2"]
    xq, s = ora.quantize_act_norm(np.array(g["U"], np.float32), None, 1e-5, 2)
    assert xq.tolist() == g["codes"]
    assert s[0] == F32(127.0) / F32(9.0)


def test_gated_reduces_to_relu2_when_up_is_one(ora):
    """relu(gate)^2 * 1 is relu(gate)^2: the gated mode with up = 1 equals mode 1."""
    gate = datagen.outlier_acts(6, 2560, 51)
    g = datagen.gains(2560, 52)
    u = np.concatenate([gate, np.ones_like(gate)], axis=1)
    xq1, s1 = ora.quantize_act_norm(gate, g, 1e-5, True)
    xq2, s2 = ora.quantize_act_norm(u, g, 1e-5, 2)
    assert (xq1 == xq2).all() and (s1 == s2).all()


def test_gated_codes_are_plain_codes_of_the_product(ora):
    """Codes of the gated input equal plain absmax codes of fl(fl(p^2) * up) * g."""
    gate = datagen.outlier_acts(5, 6912, 53)
    up = datagen.outlier_acts(5, 6912, 54)
    g = datagen.gains(6912, 55)
    xq, s = ora.quantize_act_norm(np.concatenate([gate, up], axis=1), g, 1e-5, 2)
    p = np.maximum(gate, 0).astype(np.float32)
    v = ((p * p).astype(np.float32) * up).astype(np.float32)
    xq_plain, _ = ora.quantize_act((v * g).astype(np.float32))
    assert (xq == xq_plain).all()
    ms = (v.astype(np.float64) ** 2).mean(axis=1)
    sp = F32(127.0) / np.maximum(np.abs((v * g).astype(np.float32)).max(axis=1), F32(1e-8))
    ref = sp.astype(np.float64) * np.sqrt(ms + float(F32(1e-5)))
    assert np.allclose(s.astype(np.float64), ref, rtol=2e-7, atol=0)


# ----------------------------------------------------------------------------- decode layer

def test_attention_ctx1_hand_example(ora):
    """heads 4, kv_heads 2, head_dim 1: qkv = [q0..q3 | k0 k1 | v0 v1]; query heads 0, 1
    share KV head 0 and heads 2, 3 share KV head 1, and one key gets softmax weight 1,
    so o = [v0, v0, v1, v1] whatever q and k are."""
    qkv = np.array([[9.0, -3.0, 0.5, 7.0, 2.0, -8.0, 1.25, -6.5]], np.float32)
    assert ora.attention_ctx1(qkv, 4, 2, 1).tolist() == [[1.25, 1.25, -6.5, -6.5]]


def test_attention_ctx1_ignores_q_and_k_and_reduces_to_v_for_mha(ora):
    rng = np.random.default_rng(61)
    qkv = rng.standard_normal((3, (6 + 2 * 6) * 16)).astype(np.float32)
    o = ora.attention_ctx1(qkv, 6, 6, 16)
    assert np.array_equal(o, qkv[:, 12 * 16:])          # one KV head per query head: o = v
    qkv2 = qkv.copy()
    qkv2[:, :12 * 16] = rng.standard_normal((3, 12 * 16)) * 50
    assert np.array_equal(ora.attention_ctx1(qkv2, 6, 6, 16), o)


def _layer(ora, H, F, heads, kv, hd, gated, seed, zero=()):
    mats = {}
    shapes = {"qkv": ((heads + 2 * kv) * hd, H), "o": (H, H), "up": ((2 if gated else 1) * F, H), "down": (H, F)}
    for i, (name, (n, k)) in enumerate(shapes.items()):
        w = np.zeros((n, k), np.float32) if name in zero else datagen.gg_weights(n, k, seed + i)
        packed, gamma, q = ora.pack_weights(w)
        mats[name] = (q, gamma)
    gains = {g: datagen.gains(H if g != "g_ffn" else F, seed + 10 + j)
             for j, g in enumerate(("g_in", "g_attn", "g_post", "g_ffn"))}
    return mats, gains, dict(heads=heads, kv_heads=kv, head_dim=hd)


def test_decode_layer_with_zero_weights_is_identity(ora):
    """All-zero weights give gamma = 1e-8, codes 0 and products 0, so both residual adds
    leave h unchanged; the intermediates are exact zeros."""
    mats, gains, dims = _layer(ora, 64, 96, 4, 2, 16, False, 70, zero=("qkv", "o", "up", "down"))
    h = datagen.outlier_acts(2, 64, 71)
    h2, mid = ora.decode_layer(h, mats, gains, dims, gated=False)
    assert np.array_equal(h2, h) and not mid["qkv"].any() and not mid["u"].any()


def test_decode_layer_zero_up_rows_skip_the_ffn(ora):
    """Gated: with the gate|up matrix zero the FFN input relu(gate)^2 * up is 0, down adds
    exactly 0 and h after the layer equals h after attention; with O also zero it equals
    the input."""
    mats, gains, dims = _layer(ora, 64, 96, 4, 1, 16, True, 80, zero=("up",))
    h = datagen.outlier_acts(3, 64, 81)
    h2, mid = ora.decode_layer(h, mats, gains, dims, gated=True)
    assert np.array_equal(h2, mid["h1"])
    assert not np.array_equal(mid["h1"], h)
    mats, gains, dims = _layer(ora, 64, 96, 4, 1, 16, True, 80, zero=("up", "o"))
    h2, _ = ora.decode_layer(h, mats, gains, dims, gated=True)
    assert np.array_equal(h2, h)


def test_decode_layer_matches_dense_fp64_of_dequantized_operands(ora):
    """Each sublayer of the layer is within the output tolerance of dense fp64 arithmetic on
    the dequantized operands (codes * gamma) . (xq / s), evaluated on the oracle's own
    intermediates: checks the residual wiring, the gains and the attention copy."""
    H, F = 128, 192
    mats, gains, dims = _layer(ora, H, F, 4, 2, 32, False, 90)
    h = datagen.outlier_acts(2, H, 91)
    h2, mid = ora.decode_layer(h, mats, gains, dims, gated=False)

    def dense(x, name, gain, act):
        q, gamma = mats[name]
        xq, s = ora.quantize_act_norm(x, gain, 1e-5, act)
        return (xq.astype(np.float64) / s.astype(np.float64)[:, None]) @ (q.astype(np.float64) * float(gamma)).T

    def close(a, b, scale):
        return (np.abs(a.astype(np.float64) - b) <= 1e-5 * scale + 1e-6 * np.abs(b)).all()

    qkv = dense(h, "qkv", gains["g_in"], 0)
    assert close(mid["qkv"], qkv, np.abs(qkv).max())
    assert np.array_equal(mid["o"][:, :32], mid["qkv"][:, 192:224])    # head 0 <- KV head 0's v
    d_o = dense(mid["o"], "o", gains["g_attn"], 0)
    assert close(mid["h1"], h.astype(np.float64) + d_o, np.abs(d_o).max())
    d_u = dense(mid["h1"], "up", gains["g_post"], 0)      # the FFN reads h after attention
    assert close(mid["u"], d_u, np.abs(d_u).max())
    d_d = dense(mid["u"], "down", gains["g_ffn"], 1)
    assert close(h2, mid["h1"].astype(np.float64) + d_d, np.abs(d_d).max())


def test_decode_layer_cache_branch_at_position_one(ora):
    """The real-context branch at position 1 with the QKV matrix's key rows zero: the new key
    is exactly 0, as is the cached key of slot 0, so both scores are 0 and each softmax
    weight is exactly 1/2. Query head h then outputs the mean of its group's cached value
    (slot 0) and of the new value rounded to bf16; slot 1 of the key cache holds zeros and
    slot 1 of the value cache the new value; h1 and the FFN read what the dense fp64 sublayers
    give. Catches a dropped cache position, a wrong head-to-group map, the caches not updated
    or updated at the wrong slot, and the FFN wired to the layer input."""
    H, F, heads, kv, hd = 128, 192, 4, 2, 32
    mats, gains, dims = _layer(ora, H, F, heads, kv, hd, False, 95)
    w = datagen.gg_weights((heads + 2 * kv) * hd, H, 95)
    w[heads * hd:(heads + kv) * hd] = 0.0                  # key rows
    _, gamma, q = ora.pack_weights(w)
    mats["qkv"] = (q, gamma)
    M, cap = 2, 3
    h = datagen.outlier_acts(M, H, 96)
    kc = np.zeros((M, kv, cap, hd), np.uint16)
    vc = ora.round_bf16(datagen.outlier_acts(M * kv * cap, hd, 97)).reshape(M, kv, cap, hd)
    h2, mid = ora.decode_layer(h, mats, gains, dims, gated=False,
                               cache=dict(k=kc, v=vc, pos=[1, 1], theta=10000.0))
    assert not mid["qkv"][:, heads * hd:(heads + kv) * hd].any()
    v_new = mid["qkv"][:, (heads + kv) * hd:].reshape(M, kv, hd)
    v16 = ora.round_bf16(v_new)
    expect = (ora.bf16_value(vc[:, :, 0]) + ora.bf16_value(v16)) / 2.0     # [M][kv][hd], exact in binary64
    o = mid["o"].reshape(M, heads, hd)
    for hh in range(heads):
        assert (o[:, hh] == expect[:, hh // (heads // kv)].astype(np.float32)).all()
    assert (mid["k"][:, :, 1] == 0).all() and (mid["v"][:, :, 1] == v16).all()
    assert (mid["v"][:, :, 0] == vc[:, :, 0]).all() and (mid["v"][:, :, 2] == vc[:, :, 2]).all()

    def dense(x, name, gain, act):
        qq, gm = mats[name]
        xq, s = ora.quantize_act_norm(x, gain, 1e-5, act)
        return (xq.astype(np.float64) / s.astype(np.float64)[:, None]) @ (qq.astype(np.float64) * float(gm)).T

    def close(a, b):
        return (np.abs(a.astype(np.float64) - b) <= 1e-5 * np.abs(b - 0).max() + 1e-6 * np.abs(b)).all()

    d_o = dense(mid["o"], "o", gains["g_attn"], 0)
    assert close(mid["h1"] - h.astype(np.float64), d_o)
    assert close(mid["u"], dense(mid["h1"], "up", gains["g_post"], 0))
    assert close(h2 - mid["h1"].astype(np.float64), dense(mid["u"], "down", gains["g_ffn"], 1))


# ----------------------------------------------------------------------------- 5 codes per byte

def test_pack5_golden(ora, golden):
    g = golden["pack5_order"]
    q = np.array(g["codes"], np.int8)
    packed = ora.pack5(q)
    assert packed.tolist() == g["packed"]
    back, bad = ora.unpack5(packed, q.shape[1])
    assert bad == 0 and (back == q).all()


def test_pack5_is_the_base3_numeral_of_every_pattern(ora):
    """All 3^5 five-code groups: the byte equals the base-3 numeral of the digits (code + 1,
    first code least significant) as Python's int(., 3) parses it, and the 243 bytes are
    distinct, i.e. the code is a bijection onto 0..242."""
    import itertools
    pats = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)    # [243][5]
    packed = ora.pack5(pats.reshape(1, -1))[0, :243]
    for pat, byte in zip(pats, packed):
        numeral = "".join(str(c + 1) for c in pat[::-1])
        assert int(byte) == int(numeral, 3)
    assert sorted(packed.tolist()) == list(range(243))


@pytest.mark.parametrize("K", [1, 4, 5, 79, 80, 81, 2560, 6912])
def test_pack5_round_trip_and_row_length(ora, K):
    q = ora.weight_codes(datagen.gg_weights(7, K, 600 + K), np.float32(0.02))
    packed = ora.pack5(q)
    assert packed.shape == (7, 16 * ((K + 79) // 80))
    assert packed.max() <= 242
    back, bad = ora.unpack5(packed, K)
    assert bad == 0 and (back == q).all()
    # bytes past the last five-code group encode five zero codes
    assert (packed[:, (K + 4) // 5:] == 121).all()
    # 1.6 bits per weight instead of 2 (plus at most one 16-byte chunk per row)
    assert packed.shape[1] <= (K * 2 // 8) * 0.8 + 16


def test_unpack5_flags_invalid_bytes_and_padding(ora):
    packed = np.full((1, 16), 121, np.uint8)
    packed[0, 1] = 243                    # above the largest numeral (codes 5..9, inside K)
    packed[0, 2] = 0                      # covers codes 10..14: 12..14 lie past K = 12
    _, bad = ora.unpack5(packed, 12)
    assert bad == 1 + 3


# ----------------------------------------------------------------------------- attention at real context

def test_rope_golden(ora, golden):
    """Hand example at D = 4: catches a swapped pairing ((2i, 2i+1) instead of (i, i+D/2)),
    a wrong frequency exponent or a sign flip in the rotation."""
    g = golden["rope_hand"]
    x = np.array(g["x"])
    got = ora.rope(x, g["pos"], g["theta"])
    assert np.allclose(got, g["expect"], rtol=0, atol=1e-15)
    got32 = ora.rope_f32(x, g["pos"], g["theta"])
    assert np.allclose(got32, g["expect"], rtol=2 ** -22, atol=0)


def test_rope_position_zero_and_norms(ora):
    """Position 0 rotates by 0 (identity, also in binary32); every pair keeps its length."""
    x = datagen.outlier_acts(5, 128, 801)
    assert (ora.rope(x, 0, 10000.0) == x.astype(np.float64)).all()
    assert (ora.rope_f32(x, 0, 10000.0) == x).all()
    y = ora.rope(x, 4095, 10000.0)
    n0 = np.hypot(x[:, :64].astype(np.float64), x[:, 64:].astype(np.float64))
    n1 = np.hypot(y[:, :64], y[:, 64:])
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)


def test_rope_scores_depend_on_relative_position_only(ora):
    """The defining property of rotary embedding: <R(a) q, R(b) k> = <R(a+t) q, R(b+t) k>.
    Catches per-dimension (not per-pair) angles or a frequency that varies with position."""
    q = datagen.outlier_acts(3, 128, 802).astype(np.float64)
    k = datagen.outlier_acts(3, 128, 803).astype(np.float64)
    for a, b, t in ((7, 3, 100), (0, 4000, 95), (1234, 1234, 2000)):
        s0 = np.sum(ora.rope(q, a, 10000.0) * ora.rope(k, b, 10000.0), axis=1)
        s1 = np.sum(ora.rope(q, a + t, 10000.0) * ora.rope(k, b + t, 10000.0), axis=1)
        scale = np.sum(np.abs(q) * np.abs(k), axis=1)
        assert (np.abs(s0 - s1) <= 1e-10 * scale).all()


def test_rope_f32_within_binary32_bound_of_rope(ora):
    """The binary32 evaluation differs from the binary64 rotation by at most the rounding
    of c, s, two products and a sum: 3 * 2^-24 * (|x1| + |x2|) per output."""
    x = datagen.outlier_acts(16, 128, 804)
    for pos in (1, 17, 4095, 131071):
        y64 = ora.rope(x, pos, 10000.0)
        y32 = ora.rope_f32(x, pos, 10000.0).astype(np.float64)
        mag = np.abs(x[:, :64]).astype(np.float64) + np.abs(x[:, 64:])
        bound = 3 * 2.0 ** -24 * np.concatenate([mag, mag], axis=1)
        assert (np.abs(y64 - y32) <= bound).all(), pos


def test_round_bf16_golden_and_torch(ora, golden):
    """Hand cases (ties to even, just above a tie, subnormal) and torch's float32 to
    bfloat16 conversion (round to nearest even) on random values, exact ties included."""
    import torch
    g = golden["bf16_round"]
    assert ora.round_bf16(np.array(g["x"], np.float32)).tolist() == g["bits"]
    rng = datagen.rng(805)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ties = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ora.round_bf16(x) == ref).all()
    assert (ora.bf16_value(ref) == torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy()).all()


def _one_seq(q, k, v, heads, kv_heads, d):
    return np.concatenate([np.ravel(q), np.ravel(k), np.ravel(v)]).astype(np.float32)[None, :]


def test_attention_golden(ora, golden):
    """Two positions with hand-computed softmax weights: catches a missing 1/sqrt(D), a
    query left unrotated, or the new key/value not entering the softmax."""
    g = golden["attention_hand"]
    qkv = _one_seq(g["q"], g["k_new"], g["v_new"], 1, 1, 2)
    kc = np.zeros((1, 1, 4, 2), np.uint16)
    vc = np.zeros((1, 1, 4, 2), np.uint16)
    kc[0, 0, 0] = ora.round_bf16(np.array(g["k0"], np.float32))
    vc[0, 0, 0] = ora.round_bf16(np.array(g["v0"], np.float32))
    out, kc2, vc2 = ora.attention_decode(qkv, kc, vc, [g["pos"]], 1, 1, g["theta"])
    assert np.allclose(out[0], g["expect"], rtol=1e-14, atol=0)
    assert (ora.bf16_value(vc2[0, 0, 1]) == np.array(g["v_new"])).all()
    assert (kc2[0, 0, 1] == 0).all() and (kc2[0, 0, 2:] == 0).all()


def test_attention_first_position_copies_value_per_group(ora):
    """At position 0 the softmax has one term, so query head h returns its group's new
    value (bf16-rounded): with 4 query heads on 2 KV heads the output is v0, v0, v1, v1.
    Catches a wrong head-to-group map (h % kv_heads instead of h // group)."""
    d = 8
    q = datagen.outlier_acts(4, d, 806)
    k = datagen.outlier_acts(2, d, 807)
    v = datagen.outlier_acts(2, d, 808)
    kc = np.zeros((1, 2, 3, d), np.uint16)
    out, _, vc = ora.attention_decode(_one_seq(q, k, v, 4, 2, d), kc, kc.copy(), [0], 4, 2, 10000.0)
    v16 = ora.bf16_value(ora.round_bf16(v))
    assert (out[0].reshape(4, d) == v16[[0, 0, 1, 1]]).all()
    assert (vc[0, :, 0] == ora.round_bf16(v)).all()


def test_attention_equal_keys_average_values(ora):
    """Every cached key equal to the new rotated key: all scores tie and the output is
    the plain mean of the value rows 0..pos (numpy mean)."""
    d, pos, cap = 16, 37, 50
    rng = datagen.rng(809)
    q = rng.standard_normal((2, d)).astype(np.float32)
    k = rng.standard_normal((1, d)).astype(np.float32)
    v = rng.standard_normal((1, d)).astype(np.float32)
    krot = ora.round_bf16(ora.rope_f32(k, pos, 10000.0))
    kc = np.broadcast_to(krot, (1, 1, cap, d)).copy()
    vc = ora.round_bf16(rng.standard_normal((1, 1, cap, d)).astype(np.float32))
    out, _, vc2 = ora.attention_decode(_one_seq(q, k, v, 2, 1, d), kc, vc, [pos], 2, 1, 10000.0)
    mean = ora.bf16_value(vc2[0, 0, :pos + 1]).mean(axis=0)
    assert np.allclose(out[0].reshape(2, d), mean[None, :], rtol=1e-13, atol=1e-15)


def test_attention_dominant_key_and_extent(ora):
    """A cached key along the rotated query with score about 77 (the others stay near 0,
    so their weights are below e^-70) returns its value; slots after pos hold NaN here
    and must never be read."""
    d, pos, cap, hot = 32, 20, 30, 9
    rng = datagen.rng(810)
    q = rng.standard_normal((1, d)).astype(np.float32)
    k = rng.standard_normal((1, d)).astype(np.float32)
    v = rng.standard_normal((1, d)).astype(np.float32)
    kc = ora.round_bf16(0.1 * rng.standard_normal((1, 1, cap, d)).astype(np.float32))
    vc = ora.round_bf16(rng.standard_normal((1, 1, cap, d)).astype(np.float32))
    qr = ora.rope(q, pos, 10000.0)[0]
    kc[0, 0, hot] = ora.round_bf16((60.0 * qr / np.linalg.norm(qr)).astype(np.float32))
    nan16 = np.uint16(0x7FC0)
    kc[0, 0, pos + 1:] = nan16
    vc[0, 0, pos + 1:] = nan16
    out, kc2, vc2 = ora.attention_decode(_one_seq(q, k, v, 1, 1, d), kc, vc, [pos], 1, 1, 10000.0)
    assert np.allclose(out[0], ora.bf16_value(vc[0, 0, hot]), rtol=0, atol=1e-28)
    assert (kc2[0, 0, pos + 1:] == nan16).all() and (vc2[0, 0, :pos] == vc[0, 0, :pos]).all()


def test_attention_invalid_position(ora):
    """A position outside [0, C) gives NaN outputs and leaves both caches as they were."""
    d = 8
    qkv = datagen.outlier_acts(2, 3 * d, 811)
    kc = ora.round_bf16(datagen.outlier_acts(2 * 4, d, 812)).reshape(2, 1, 4, d)
    vc = kc.copy()
    out, kc2, vc2 = ora.attention_decode(qkv, kc, vc, [4, -1], 1, 1, 10000.0)
    assert np.isnan(out).all()
    assert (kc2 == kc).all() and (vc2 == vc).all()
