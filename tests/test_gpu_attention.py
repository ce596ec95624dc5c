"""GPU parity of decode attention at real context length (rotary positions, bf16
key/value cache, grouped-query softmax attention) against the CPU oracle.

Every case draws the new token's q/k/v and the whole cache from the seeded generators.
The cache must come back bit-identical to the oracle's (slot pos holds the rotated,
bf16-rounded new key and value; every other slot is untouched), and the output must lie
within the error bound derived below from the kernel's fp32 arithmetic.

The output bound is tolerances.attention_bound (derived there from the kernel's fp32
arithmetic). The tie test needs no bound: all scores are exactly 0, so the output is the
mean of integer values, which both sides round once.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_linear_w1_amd as bl
from ternary_weight_linear_w1_amd import _build
from tolerances import attention_bound

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not _build.up_to_date():
        _build.build()
    bl.lib()
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def make(M, H, KVH, C, seed, qscale=1.0):
    qkv = datagen.outlier_acts(M, (H + 2 * KVH) * D, datagen.stream_id(40, seed, 0, 1))
    qkv[:, :H * D] *= np.float32(qscale)
    kc = datagen.bf16_cache((M, KVH, C, D), datagen.stream_id(40, seed, 1, 1))
    vc = datagen.bf16_cache((M, KVH, C, D), datagen.stream_id(40, seed, 2, 1))
    return qkv, kc, vc


def run_gpu(qkv, kc, vc, pos, H, KVH, theta=10000.0):
    g_qkv = torch.from_numpy(qkv).to(DEV)
    g_kc = torch.from_numpy(kc.view(np.int16)).to(DEV).view(torch.bfloat16)
    g_vc = torch.from_numpy(vc.view(np.int16)).to(DEV).view(torch.bfloat16)
    g_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    out = bl.bitlinear_attention_decode(g_qkv, g_kc, g_vc, g_pos, H, KVH, theta)
    torch.cuda.synchronize()
    as16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.cpu().numpy(), as16(g_kc), as16(g_vc)


def check(M, H, KVH, C, pos, seed, qscale=1.0):
    qkv, kc, vc = make(M, H, KVH, C, seed, qscale)
    print("attention case M=%d H=%d KVH=%d C=%d pos=%s seed=%d" % (M, H, KVH, C, pos, seed), flush=True)
    out, gkc, gvc = run_gpu(qkv, kc, vc, pos, H, KVH)
    ref, okc, ovc = oracle.attention_decode(qkv, kc, vc, pos, H, KVH, 10000.0)
    assert (gkc == okc).all(), np.argwhere(gkc != okc)[:5]
    assert (gvc == ovc).all(), np.argwhere(gvc != ovc)[:5]
    tol = attention_bound(qkv, okc, ovc, pos, H, KVH)
    valid = ~np.isnan(ref)
    assert (np.isnan(out) == ~valid).all()
    err = np.abs(out.astype(np.float64) - ref)
    worst = np.max(np.where(valid, err / tol, 0.0))
    print("  max error / bound = %.3g" % worst)
    assert worst <= 1.0
    return worst


CASES = [
    # M, H, KVH, C, pos
    (1, 4, 1, 64, [0]),                  # only the new token: out = its value
    (1, 20, 5, 300, [63]),               # last position of the first chunk
    (1, 20, 5, 300, [64]),               # first position of the second chunk
    (1, 20, 5, 300, [65]),
    (1, 20, 5, 100, [99]),               # last slot of a capacity that is not a chunk multiple
    (1, 20, 5, 4096, [4095]),            # 2B shape, full 4096-token context
    (3, 8, 2, 130, [5, 129, 64]),        # sequences at different positions
    (2, 64, 8, 1000, [999, 17]),         # 100B shape: 8 query heads per KV head
    (1, 6, 2, 100, [77]),                # 3 query heads per KV head
    (1, 16, 8, 128, [100]),              # 2 per KV head
    (1, 2, 2, 70, [69]),                 # plain multi-head
    (1, 32, 2, 200, [150]),              # 16 per KV head: two blocks per KV head
    (1, 1, 1, 1, [0]),                   # capacity 1
    # more blocks than two per compute unit: blocks walk several 64-position sub-chunks
    # with a running maximum, two sub-chunks' loads in flight
    (1, 20, 5, 32768, [32767]),          # 2B heads, long context
    (8, 20, 5, 4096, [4095, 4000, 3000, 2047, 1024, 700, 64, 5]),   # 8 sequences at mixed positions
    (2, 64, 8, 4096, [4095, 2222]),      # 100B heads: 8 query heads per KV head split in two blocks
]


@pytest.mark.parametrize("M,H,KVH,C,pos", CASES)
def test_attention_parity(M, H, KVH, C, pos):
    check(M, H, KVH, C, pos, seed=C % 97 + H)


def test_attention_peaked_scores():
    """Queries scaled by 6: scores spread over tens of units, most weight on a few keys."""
    check(1, 20, 5, 2048, [2047], seed=3, qscale=6.0)
    check(2, 64, 8, 600, [599, 300], seed=4, qscale=6.0)


def test_attention_invalid_positions_leave_cache():
    """pos = capacity and pos = -1: NaN outputs, caches untouched; the valid sequence in
    the same call is unaffected."""
    check(3, 8, 2, 200, [200, 57, -1], seed=5)


@pytest.mark.parametrize("C,p", [(512, 300), (512, 0), (32768, 20000), (32768, 191)])
def test_attention_ignores_slots_past_pos(C, p):
    """NaN bit patterns in slot pos and every slot after it never reach the output (slot
    pos is overwritten with the new key and value), in the one-sub-chunk form (512) and in
    the form whose blocks walk several sub-chunks (32768)."""
    M, H, KVH = 1, 20, 5
    qkv, kc, vc = make(M, H, KVH, C, 6)
    kc[:, :, p:] = 0x7FC0
    vc[:, :, p:] = 0x7FC0
    print("attention NaN past pos: C=%d pos=%d" % (C, p), flush=True)
    out, gkc, gvc = run_gpu(qkv, kc, vc, [p], H, KVH)
    ref, okc, ovc = oracle.attention_decode(qkv, kc, vc, [p], H, KVH, 10000.0)
    assert np.isfinite(out).all()
    assert (gkc == okc).all() and (gvc == ovc).all()
    assert (np.abs(out - ref) <= attention_bound(qkv, okc, ovc, [p], H, KVH)).all()


@pytest.mark.parametrize("M,H,KVH,C,pos", [(1, 20, 5, 32768, [100]), (1, 20, 5, 4096, [70]),
                                           (3, 8, 2, 2000, [1999, 0, 640]), (8, 20, 5, 4096, [4095] + [9] * 7)])
def test_attention_stale_workspace_is_never_read(M, H, KVH, C, pos):
    """The merge requests its first batch of chunk records before it has read pos; records
    past the live ones hold whatever an earlier call left. With every workspace byte 0xFF
    (NaN floats) beforehand the output still matches the oracle."""
    qkv, kc, vc = make(M, H, KVH, C, 11)
    print("attention stale workspace: M=%d H=%d KVH=%d C=%d pos=%s" % (M, H, KVH, C, pos), flush=True)
    g_qkv = torch.from_numpy(qkv).to(DEV)
    g_kc = torch.from_numpy(kc.view(np.int16)).to(DEV).view(torch.bfloat16)
    g_vc = torch.from_numpy(vc.view(np.int16)).to(DEV).view(torch.bfloat16)
    g_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    ws = torch.full((bl.bitlinear_attention_workspace_bytes(M, H, C),), 0xFF, dtype=torch.uint8, device=DEV)
    out = bl.bitlinear_attention_decode(g_qkv, g_kc, g_vc, g_pos, H, KVH, workspace=ws).cpu().numpy()
    ref, okc, ovc = oracle.attention_decode(qkv, kc, vc, pos, H, KVH, 10000.0)
    assert np.isfinite(out).all()
    assert (np.abs(out - ref) <= attention_bound(qkv, okc, ovc, pos, H, KVH)).all()


@pytest.mark.parametrize("M,H,KVH,C,pos", [(1, 20, 5, 4096, [4095]), (2, 64, 8, 4096, [4000, 1234]),
                                           (1, 6, 3, 129, [128])])
def test_attention_ties_count_every_position_once(M, H, KVH, C, pos):
    """All keys zero: every score is exactly 0, every weight exactly 1, and the output is
    the mean of small-integer values. Sum and count are exact in fp32, so the GPU must
    return the correctly rounded quotient S / (pos + 1) bit for bit. That is
    float32(float64(S) / n): S / n is not dyadic unless n is a power of two (then it is
    exact), and a non-dyadic quotient lies at least 2^-24 / n relative away from every
    binary32 rounding midpoint, far beyond the binary64 division's 2^-53, so the double
    rounding cannot go wrong. The oracle's binary64 softmax path (whose sum of 1/n-weighted
    values can cancel) must agree with the exact mean within 1e-12 absolute.
    A position dropped, counted twice or read from the wrong head or dim changes it."""
    qkv = np.zeros((M, (H + 2 * KVH) * D), np.float32)
    qkv[:, :H * D] = datagen.outlier_acts(M, H * D, datagen.stream_id(41, C, 0, 1))
    qkv[:, (H + KVH) * D:] = datagen.small_ints((M, KVH * D), datagen.stream_id(41, C, 1, 1), -3, 3)
    kc = np.zeros((M, KVH, C, D), np.uint16)
    vals = datagen.small_ints((M, KVH, C, D), datagen.stream_id(41, C, 2, 1), -3, 3)
    vc = (vals.view(np.uint32) >> 16).astype(np.uint16)     # small integers are exact in bf16
    out, gkc, gvc = run_gpu(qkv, kc, vc, pos, H, KVH)
    ref, okc, ovc = oracle.attention_decode(qkv, kc, vc, pos, H, KVH, 10000.0)
    assert (gkc == okc).all() and (gvc == ovc).all()
    G = H // KVH
    for b in range(M):
        n = pos[b] + 1
        sums = oracle.bf16_value(ovc[b, :, :n]).sum(axis=1)           # [KVH][D], exact integers
        mean = np.repeat(sums / n, G, axis=0).reshape(-1)             # head h -> group h // G
        assert (out[b] == mean.astype(np.float32)).all(), (b, np.argwhere(out[b] != mean.astype(np.float32))[:5])
        assert np.abs(ref[b] - mean).max() <= 1e-12


def test_attention_graph_replay_matches_eager():
    """A captured graph of the two launches gives the eager result on every replay, with
    eager work between replays."""
    M, H, KVH, C, p = 1, 20, 5, 1024, 700
    qkv, kc, vc = make(M, H, KVH, C, 7)
    eager, _, _ = run_gpu(qkv, kc, vc, [p], H, KVH)
    g_qkv = torch.from_numpy(qkv).to(DEV)
    g_kc = torch.from_numpy(kc.view(np.int16)).to(DEV).view(torch.bfloat16)
    g_vc = torch.from_numpy(vc.view(np.int16)).to(DEV).view(torch.bfloat16)
    g_pos = torch.tensor([p], dtype=torch.int32, device=DEV)
    out = torch.empty((M, H * D), dtype=torch.float32, device=DEV)
    ws = torch.empty((bl.bitlinear_attention_workspace_bytes(M, H, C),), dtype=torch.uint8, device=DEV)
    bl.bitlinear_attention_decode(g_qkv, g_kc, g_vc, g_pos, H, KVH, out=out, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            bl.bitlinear_attention_decode(g_qkv, g_kc, g_vc, g_pos, H, KVH, out=out, workspace=ws, stream=s)
    for _ in range(3):
        out.fill_(0.0)
        ws.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert (out.cpu().numpy() == eager).all()
