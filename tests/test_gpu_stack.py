"""GPU parity of the decode stack: BitNet-2B-shaped layers (hidden 2560, 20 query heads,
5 KV heads of 128, FFN 6912) at decode, plain and gated FFN.

Teacher-forced: every launch of a layer is checked against the oracle computed from the
GPU's own input to that launch (the attention copy bit for bit, every BitLinear within
the fp32 output tolerance plus the residual add's rounding). End to end: a captured
graph of the whole stack equals the eager launches bit for bit on every replay, and the
stack's output stays within a small relative error of the oracle's layer chain.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_linear_w1_amd as bl
from ternary_weight_linear_w1_amd import _build
from ternary_weight_linear_w1_amd.decode_stack import DecodeStack, LayerWeights

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-5
H, HEADS, KV, HD, F = 2560, 20, 5, 128, 6912
DIMS = dict(heads=HEADS, kv_heads=KV, head_dim=HD)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not _build.up_to_date():
        _build.build()
    bl.lib()
    oracle.lib()
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def build(n_layers, gated, cfg, M=1):
    """Stack on the device plus the oracle's (codes, gamma) and gains of every layer."""
    layers, host = [], []
    shapes = {"qkv": ((HEADS + 2 * KV) * HD, H), "o": (H, H), "up": ((2 if gated else 1) * F, H), "down": (H, F)}
    for li in range(n_layers):
        dev, mats = {}, {}
        for mi, (name, (n, k)) in enumerate(shapes.items()):
            w = datagen.gg_weights_torch(n, k, datagen.stream_id(cfg, li, mi, 0), DEV)
            packed, gamma = bl.bitlinear_pack_weights(w)
            wh = w.cpu().numpy()
            del w
            ogamma = oracle.weight_scale(wh)
            assert float(gamma.cpu()[0]) == float(ogamma)
            mats[name] = (oracle.weight_codes(wh, ogamma), ogamma)
            dev[name] = (packed, gamma)
        gains = {g: datagen.gains_torch(F if g == "g_ffn" else H, datagen.stream_id(cfg, li, 4 + j, 2), DEV)
                 for j, g in enumerate(("g_in", "g_attn", "g_post", "g_ffn"))}
        layers.append(LayerWeights(dev["qkv"], dev["o"], dev["up"], dev["down"], **gains))
        host.append((mats, {g: t.cpu().numpy() for g, t in gains.items()}))
    stack = DecodeStack(layers, H, HEADS, KV, HD, F, gated, M=M, eps=EPS, device=DEV)
    return stack, host


def lin(mats, x, name, gain, act):
    q, gamma = mats[name]
    xq, s = oracle.quantize_act_norm(x, gain, EPS, act)
    return oracle.forward(xq, s, q, gamma)[1]


def within(gpu, expect, y):
    """|gpu - expect| <= 1e-6 |y| + 2^-23 |expect|: the product's tolerance plus the add."""
    tol = 1e-6 * np.abs(y.astype(np.float64)) + 2.0 ** -23 * np.abs(expect.astype(np.float64))
    return (np.abs(gpu.astype(np.float64) - expect.astype(np.float64)) <= tol).all()


@pytest.mark.parametrize("gated,M,n_layers", [(False, 1, 3), (True, 1, 2), (False, 3, 1)])
def test_stack_teacher_forced(gated, M, n_layers):
    stack, host = build(n_layers, gated, 30 + int(gated) + 2 * M, M)
    stack.h.copy_(datagen.outlier_acts_torch(M, H, datagen.stream_id(3, 99, 0, 1), DEV))
    act = 2 if gated else 1
    for li in range(n_layers):
        mats, gains = host[li]
        ops = dict(stack.ops(li))
        h0 = stack.h.cpu().numpy()
        ops["qkv"]()
        qkv = stack.qkv.cpu().numpy()
        y = lin(mats, h0, "qkv", gains["g_in"], 0)
        assert within(qkv, y, y), "layer %d qkv" % li
        ops["attn"]()
        assert np.array_equal(stack.o.cpu().numpy(), oracle.attention_ctx1(qkv, HEADS, KV, HD)), "layer %d attn" % li
        ops["o"]()
        h1 = stack.h.cpu().numpy()
        y = lin(mats, stack.o.cpu().numpy(), "o", gains["g_attn"], 0)
        assert within(h1, (h0 + y).astype(np.float32), y), "layer %d o" % li
        ops["up"]()
        u = stack.u.cpu().numpy()
        y = lin(mats, h1, "up", gains["g_post"], 0)
        assert within(u, y, y), "layer %d up" % li
        ops["down"]()
        h2 = stack.h.cpu().numpy()
        y = lin(mats, u, "down", gains["g_ffn"], act)
        assert within(h2, (h1 + y).astype(np.float32), y), "layer %d down" % li


@pytest.mark.parametrize("gated", [False, True])
def test_stack_graph_replays_and_end_to_end(gated):
    n_layers = 4
    stack, host = build(n_layers, gated, 40 + int(gated))
    x0 = datagen.outlier_acts_torch(1, H, datagen.stream_id(3, 98, 0, 1), DEV)
    stack.h.copy_(x0)
    stack.step()
    eager = stack.h.clone()
    stack.h.copy_(x0)
    g = stack.capture()               # runs one eager pass first, then records
    for _ in range(3):
        stack.h.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(stack.h, eager)
        stack.u.zero_()               # eager work between replays
    h = x0.cpu().numpy()
    for li in range(n_layers):
        h, _ = oracle.decode_layer(h, host[li][0], host[li][1], DIMS, gated, EPS)
    got = eager.cpu().numpy().astype(np.float64)
    err = np.abs(got - h).max() / np.abs(h).max()
    print("end-to-end max error / max|h| over %d layers: %.3g" % (n_layers, err))
    assert err <= 1e-4
