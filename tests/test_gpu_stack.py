"""GPU parity of the decode stack: BitNet-2B-shaped layers (hidden 2560, 20 query heads,
5 KV heads of 128, FFN 6912) at decode with a bf16 key/value cache, plain and gated FFN.

Per launch: each op of a layer runs alone on seeded inputs written into exactly the
buffers it reads, and its output is checked against the oracle on those inputs (every
BitLinear within the fp32 output tolerance plus the residual add's rounding; attention
within its derived bound and its cache slot bit for bit). This checks the wiring of every
launch (buffers, weights, gains, activation mode, residual) with no GPU output feeding
the oracle. End to end: from a seeded hidden state and seeded prior context, a captured
graph of the whole stack equals the eager launches bit for bit on every replay, advancing
positions in the graph matches eager steps, and the output stays within a small relative
error of the oracle's layer chain.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_linear_w1_amd as bl
from ternary_weight_linear_w1_amd import _build
from ternary_weight_linear_w1_amd.decode_stack import DecodeStack, LayerWeights
from tolerances import attention_bound

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


def build(n_layers, gated, cfg, M=1, capacity=256):
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
    stack = DecodeStack(layers, H, HEADS, KV, HD, F, gated, M=M, eps=EPS, device=DEV, capacity=capacity)
    return stack, host


def lin(mats, x, name, gain, act):
    q, gamma = mats[name]
    xq, s = oracle.quantize_act_norm(x, gain, EPS, act)
    return oracle.forward(xq, s, q, gamma)[1]


def within(gpu, expect, y):
    """|gpu - expect| <= 1e-6 |y| + 2^-23 |expect|: the product's tolerance plus the add."""
    tol = 1e-6 * np.abs(y.astype(np.float64)) + 2.0 ** -23 * np.abs(expect.astype(np.float64))
    return (np.abs(gpu.astype(np.float64) - expect.astype(np.float64)) <= tol).all()


def seeded(shape, cfg, tag):
    m, n = shape
    return datagen.outlier_acts(m, n, datagen.stream_id(cfg, 200 + tag, 0, 1))


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def as_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def from_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("gated,M", [(False, 1), (True, 1), (False, 3)])
def test_stack_ops_on_seeded_inputs(gated, M):
    cfg = 30 + int(gated) + 2 * M
    n_layers, C = 2, 200
    stack, host = build(n_layers, gated, cfg, M, capacity=C)
    act = 2 if gated else 1
    nqkv = (HEADS + 2 * KV) * HD
    for li in range(n_layers):
        mats, gains = host[li]
        ops = dict(stack.ops(li))
        tag = 10 * li
        print("stack op check gated=%s M=%d layer %d" % (gated, M, li), flush=True)
        # qkv reads h
        h = seeded((M, H), cfg, tag + 0)
        stack.h.copy_(to_dev(h))
        ops["qkv"]()
        y = lin(mats, h, "qkv", gains["g_in"], 0)
        assert within(stack.qkv.cpu().numpy(), y, y), "layer %d qkv" % li
        # attention reads qkv, the layer's caches and pos
        qkv = seeded((M, nqkv), cfg, tag + 1)
        kc = datagen.bf16_cache((M, KV, C, HD), datagen.stream_id(cfg, 210 + li, 1, 1))
        vc = datagen.bf16_cache((M, KV, C, HD), datagen.stream_id(cfg, 210 + li, 2, 1))
        pos = [(37 * (li + 1) + 61 * b) % C for b in range(M)]
        stack.qkv.copy_(to_dev(qkv))
        stack.k_cache[li].copy_(from_u16(kc))
        stack.v_cache[li].copy_(from_u16(vc))
        stack.pos.copy_(torch.tensor(pos, dtype=torch.int32))
        ops["attn"]()
        ref, okc, ovc = oracle.attention_decode(qkv, kc, vc, pos, HEADS, KV, 10000.0)
        assert (as_u16(stack.k_cache[li]) == okc).all() and (as_u16(stack.v_cache[li]) == ovc).all()
        tol = attention_bound(qkv, okc, ovc, pos, HEADS, KV)
        assert (np.abs(stack.o.cpu().numpy() - ref) <= tol).all(), "layer %d attn" % li
        # o reads o and h (residual)
        o = seeded((M, H), cfg, tag + 2)
        h = seeded((M, H), cfg, tag + 3)
        stack.o.copy_(to_dev(o))
        stack.h.copy_(to_dev(h))
        ops["o"]()
        y = lin(mats, o, "o", gains["g_attn"], 0)
        assert within(stack.h.cpu().numpy(), (h + y).astype(np.float32), y), "layer %d o" % li
        # up reads h
        h = seeded((M, H), cfg, tag + 4)
        stack.h.copy_(to_dev(h))
        ops["up"]()
        y = lin(mats, h, "up", gains["g_post"], 0)
        assert within(stack.u.cpu().numpy(), y, y), "layer %d up" % li
        # down reads u and h (residual)
        u = seeded((M, stack.u.shape[1]), cfg, tag + 5)
        h = seeded((M, H), cfg, tag + 6)
        stack.u.copy_(to_dev(u))
        stack.h.copy_(to_dev(h))
        ops["down"]()
        y = lin(mats, u, "down", gains["g_ffn"], act)
        assert within(stack.h.cpu().numpy(), (h + y).astype(np.float32), y), "layer %d down" % li


def seed_context(stack, n_layers, cfg):
    """Seeded prior context in every layer's caches; returns the host copies."""
    caches = []
    for li in range(n_layers):
        shape = tuple(stack.k_cache[li].shape)
        kc = datagen.bf16_cache(shape, datagen.stream_id(cfg, 220 + li, 1, 1))
        vc = datagen.bf16_cache(shape, datagen.stream_id(cfg, 220 + li, 2, 1))
        stack.k_cache[li].copy_(from_u16(kc))
        stack.v_cache[li].copy_(from_u16(vc))
        caches.append((kc, vc))
    return caches


@pytest.mark.parametrize("gated", [False, True])
def test_stack_graph_replays_and_end_to_end(gated):
    n_layers, cfg, p = 4, 40 + int(gated), 150
    stack, host = build(n_layers, gated, cfg)
    caches = seed_context(stack, n_layers, cfg)
    x0 = datagen.outlier_acts_torch(1, H, datagen.stream_id(3, 98, 0, 1), DEV)
    stack.pos.fill_(p)
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
        kc, vc = caches[li]
        h, _ = oracle.decode_layer(h, host[li][0], host[li][1], DIMS, gated, EPS,
                                   cache=dict(k=kc, v=vc, pos=[p], theta=10000.0))
    got = eager.cpu().numpy().astype(np.float64)
    err = np.abs(got - h).max() / np.abs(h).max()
    print("end-to-end max error / max|h| over %d layers at position %d: %.3g" % (n_layers, p, err))
    assert err <= 1e-4


def test_stack_graph_advances_positions():
    """A graph captured with advance=True decodes successive tokens: two replays give the
    same hidden state, caches and positions as two eager steps with advance."""
    n_layers, cfg = 2, 45
    stack, _ = build(n_layers, False, cfg, M=2)
    seed_context(stack, n_layers, cfg)
    start = torch.tensor([10, 63], dtype=torch.int32)
    x0 = datagen.outlier_acts_torch(2, H, datagen.stream_id(3, 97, 0, 1), DEV)
    k0 = [t.clone() for t in stack.k_cache]
    v0 = [t.clone() for t in stack.v_cache]

    def reset():
        stack.h.copy_(x0)
        stack.pos.copy_(start)
        for li in range(n_layers):
            stack.k_cache[li].copy_(k0[li])
            stack.v_cache[li].copy_(v0[li])

    reset()
    stack.step(advance=True)
    stack.step(advance=True)
    torch.cuda.synchronize()
    want = (stack.h.clone(), stack.pos.clone(), [t.clone() for t in stack.k_cache], [t.clone() for t in stack.v_cache])
    assert stack.pos.cpu().tolist() == [12, 65]
    reset()
    g = stack.capture(advance=True)
    reset()
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(stack.h, want[0]) and torch.equal(stack.pos, want[1])
    for li in range(n_layers):
        assert torch.equal(stack.k_cache[li].view(torch.int16), want[2][li].view(torch.int16))
        assert torch.equal(stack.v_cache[li].view(torch.int16), want[3][li].view(torch.int16))
