"""The no-allocation fused call (bitlinear_forward_f32_noalloc) through the C ABI against
bitlinear_forward_f32_ws with a caller workspace: the same kernels, so every output must
match bit for bit. Two calls in a row on one stream share the library's fixed scratch,
the second with a smaller input; a split-K size (int32 partials in the scratch) and the
residual form are covered, and a size beyond the scratch is rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import ternary_weight_linear_w1_amd as bl
from ternary_weight_linear_w1_amd import _build

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-5
ERR_WORKSPACE = 4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not _build.up_to_date():
        _build.build()
    bl.lib()
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def case(M, N, K, mode, seed):
    w = torch.from_numpy(datagen.gg_weights(N, K, seed)).to(DEV)
    packed, gamma = bl.bitlinear_pack_weights(w)
    width = 2 * K if mode == "gated" else K
    x = torch.from_numpy(datagen.outlier_acts(M, width, seed + 1)).to(DEV)
    gain = torch.from_numpy(datagen.gains(K, seed + 2)).to(DEV) if mode != "plain" else None
    act = {"plain": 0, "norm": 0, "relu2norm": 1, "gated": 2}[mode]
    y0 = torch.from_numpy(datagen.outlier_acts(M, N, seed + 3)).to(DEV)   # residual input
    return dict(M=M, N=N, K=K, packed=packed, gamma=gamma, x=x, gain=gain, act=act, y0=y0)


def with_workspace(c, residual):
    y = c["y0"].clone() if residual else torch.empty((c["M"], c["N"]), dtype=torch.float32, device=DEV)
    need = bl.bitlinear_forward_f32_workspace_bytes(c["M"], c["N"], c["K"])
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=DEV)
    st = bl.lib().bitlinear_forward_f32_ws(P(c["x"]), c["M"], c["K"], P(c["gain"]), EPS, c["act"], P(c["packed"]),
                                           P(c["gamma"]), c["N"], P(y), int(residual), P(ws), ws.numel(), None)
    assert st == 0
    torch.cuda.synchronize()
    return y, need


def no_alloc(c, residual, y):
    return bl.lib().bitlinear_forward_f32_noalloc(P(c["x"]), c["M"], c["K"], P(c["gain"]), EPS, c["act"],
                                                  P(c["packed"]), P(c["gamma"]), c["N"], P(y), int(residual), None)


PAIRS = [
    # (first, second): the second call is smaller than the first
    ((64, 2560, 6912, "relu2norm", 0), (20, 2560, 2560, "plain", 0)),
    ((12, 8192, 28672, "plain", 0), (10, 4096, 16384, "norm", 0)),        # K split: partials in the scratch
    ((256, 3840, 2560, "norm", 1), (17, 1024, 2560, "gated", 1)),          # residual forms
    ((2048, 2560, 6912, "relu2norm", 0), (1, 6912, 2560, "plain", 0)),     # 14 MB of codes; one token: no scratch
    ((16, 4096, 28672, "relu2norm", 0), (1, 8192, 28672, "relu2norm", 1)),  # one token, long rows: two-role kernel
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_no_alloc_matches_workspace_call_twice_in_a_row(first, second):
    print("no-alloc pair", first, second, flush=True)
    c1 = case(*first[:4], seed=500 + first[0])
    c2 = case(*second[:4], seed=700 + second[0])
    r1, r2 = bool(first[4]), bool(second[4])
    ref1, need1 = with_workspace(c1, r1)
    ref2, need2 = with_workspace(c2, r2)
    assert need1 > 0 and need1 <= bl.NOALLOC_SCRATCH_BYTES and need2 <= need1
    y1 = c1["y0"].clone() if r1 else torch.full((c1["M"], c1["N"]), float("nan"), device=DEV)
    y2 = c2["y0"].clone() if r2 else torch.full((c2["M"], c2["N"]), float("nan"), device=DEV)
    torch.cuda.synchronize()
    assert no_alloc(c1, r1, y1) == 0
    assert no_alloc(c2, r2, y2) == 0          # same stream, right after: reuses the scratch
    torch.cuda.synchronize()
    assert torch.equal(y1, ref1)
    assert torch.equal(y2, ref2)
    # and once more in the other order, through the Python binding
    y1b = c1["y0"].clone() if r1 else torch.empty_like(ref1)
    y2b = c2["y0"].clone() if r2 else torch.empty_like(ref2)
    bl.bitlinear_forward_f32_noalloc(c2["x"], c2["packed"], c2["gamma"], y2b, c2["gain"], EPS, c2["act"], residual=r2)
    bl.bitlinear_forward_f32_noalloc(c1["x"], c1["packed"], c1["gamma"], y1b, c1["gain"], EPS, c1["act"], residual=r1)
    torch.cuda.synchronize()
    assert torch.equal(y1b, ref1) and torch.equal(y2b, ref2)


def test_no_alloc_rejects_sizes_beyond_its_scratch():
    M, N, K = 4096, 64, 16384                 # 64 MiB of codes > 32 MiB
    assert bl.bitlinear_forward_f32_workspace_bytes(M, N, K) > bl.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    packed = torch.zeros((N, K // 4), dtype=torch.uint8, device=DEV)
    gamma = torch.ones((1,), dtype=torch.float32, device=DEV)
    y = torch.full((M, N), 7.0, device=DEV)
    st = bl.lib().bitlinear_forward_f32_noalloc(P(x), M, K, None, EPS, 0, P(packed), P(gamma), N, P(y), 0, None)
    torch.cuda.synchronize()
    assert st == ERR_WORKSPACE
    assert bool((y == 7.0).all())             # nothing was enqueued


def test_no_alloc_inside_a_captured_graph():
    """The use the entry point is for: after a first call outside capture (which looks up
    the device's scratch address), calls captured in a graph allocate nothing and every
    replay, with eager work between replays, gives the workspace call's bits."""
    c1 = case(64, 2560, 6912, "relu2norm", seed=900)
    c2 = case(12, 8192, 28672, "plain", seed=901)      # K split: partials in the scratch
    ref1, _ = with_workspace(c1, False)
    ref2, _ = with_workspace(c2, False)
    y1 = torch.empty_like(ref1)
    y2 = torch.empty_like(ref2)
    assert no_alloc(c1, False, y1) == 0                 # outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            st = ctypes.c_void_p(side.cuda_stream)
            r1 = bl.lib().bitlinear_forward_f32_noalloc(P(c1["x"]), c1["M"], c1["K"], P(c1["gain"]), EPS, c1["act"],
                                                         P(c1["packed"]), P(c1["gamma"]), c1["N"], P(y1), 0, st)
            r2 = bl.lib().bitlinear_forward_f32_noalloc(P(c2["x"]), c2["M"], c2["K"], P(c2["gain"]), EPS, c2["act"],
                                                         P(c2["packed"]), P(c2["gamma"]), c2["N"], P(y2), 0, st)
    assert r1 == 0 and r2 == 0
    for _ in range(3):
        y1.fill_(float("nan"))
        y2.fill_(float("nan"))
        with_workspace(c2, False)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, ref1) and torch.equal(y2, ref2)
