"""GPU parity at the benchmark's full sizes, through the same entry points and launch
configurations bench.py times.

Latent weights are drawn on the device (datagen's Philox generators) and copied to the
host for the oracle, which recomputes gamma over the whole matrix and packs it; packed
bytes and gamma are compared in full. Outputs are compared in full where the oracle is
fast enough (M <= 8) and on sampled output rows otherwise (every token, 48 rows spread
over N including the last).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_linear_w1_amd as bl
from ternary_weight_linear_w1_amd import _build

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-5

LAYER_2B = [("qkv", 3840, 2560, "plain"), ("o", 2560, 2560, "norm"), ("up", 6912, 2560, "plain"),
            ("down", 2560, 6912, "relu2norm")]
LAYER_100B = [("qkv", 10240, 8192, "plain"), ("o", 8192, 8192, "norm"), ("up", 28672, 8192, "plain"),
              ("down", 8192, 28672, "relu2norm")]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not _build.up_to_date():
        _build.build()
    bl.lib()
    oracle.lib()
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def sample_rows(n, count=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(n, size=min(count, n), replace=False), [0, n - 1]]))
    return rows


def check_matrix(cfg, idx, N, K, mode, M, fused, heavy=False, sampled=False):
    w = datagen.gg_weights_torch(N, K, datagen.stream_id(cfg, 9, idx, 0), DEV)
    if heavy:
        x = datagen.heavy_channel_acts_torch(M, K, datagen.stream_id(cfg, 9, idx, 1), DEV)
    else:
        x = datagen.outlier_acts_torch(M, K, datagen.stream_id(cfg, 9, idx, 1), DEV)
    gain = datagen.gains_torch(K, datagen.stream_id(cfg, 9, idx, 2), DEV) if "norm" in mode else None
    relu2 = mode == "relu2norm"
    packed, gamma = bl.bitlinear_pack_weights(w)
    if fused:
        y = bl.bitlinear_forward_f32(x, packed, gamma, gain, EPS, relu2)
        acc = None
    else:
        xq, s = bl.bitlinear_quantize_act(x, gain, EPS, relu2)
        y, acc = bl.bitlinear_forward(xq, s, packed, gamma, acc=True)
        # without the int32 copy the product takes another store path: same output bits
        assert torch.equal(bl.bitlinear_forward(xq, s, packed, gamma).view(torch.int32), y.view(torch.int32))
    torch.cuda.synchronize()
    wh = w.cpu().numpy()
    xh = x.cpu().numpy()
    gh = None if gain is None else gain.cpu().numpy()
    del w
    # full weight-side parity
    opacked, ogamma, _ = oracle.pack_weights(wh)
    assert float(gamma.cpu()[0]) == float(ogamma)
    assert np.array_equal(packed.cpu().numpy(), opacked)
    # activation side
    if gh is None and not relu2:
        oxq, os_ = oracle.quantize_act(xh)
    else:
        oxq, os_ = oracle.quantize_act_norm(xh, gh, EPS, relu2)
    rows = sample_rows(N, seed=idx) if sampled else np.arange(N)
    q_rows = oracle.weight_codes(wh[rows], ogamma)
    oacc, oy = oracle.forward(oxq, os_, q_rows, ogamma)
    yh = y.cpu().numpy()[:, rows]
    if acc is not None:
        assert np.array_equal(acc.cpu().numpy()[:, rows], oacc)
    if gh is None:
        assert np.array_equal(yh.view(np.int32), oy.view(np.int32))
    else:
        err = np.abs(yh.astype(np.float64) - oy.astype(np.float64))
        assert (err <= 1e-6 * np.abs(oy.astype(np.float64))).all()


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("i", range(4))
def test_2b_layer_decode(M, i):
    """Both entries at every token count: the fused call and the product on pre-quantized
    codes (at one token the two take different launch shapes)."""
    name, N, K, mode = LAYER_2B[i]
    check_matrix(2, i + 10 * M, N, K, mode, M, fused=(M == 1))
    check_matrix(2, i + 10 * M + 100, N, K, mode, M, fused=(M != 1))


@pytest.mark.parametrize("M", [512, 2048])
@pytest.mark.parametrize("i", range(4))
def test_2b_prefill(M, i):
    name, N, K, mode = LAYER_2B[i]
    check_matrix(4, i + M, N, K, "plain", M, fused=False, heavy=True, sampled=True)


@pytest.mark.parametrize("i", range(4))
def test_100b_decode_m1(i):
    name, N, K, mode = LAYER_100B[i]
    check_matrix(5, i, N, K, mode, 1, fused=True)


@pytest.mark.parametrize("i", range(4))
def test_100b_small_batch_m64(i):
    name, N, K, mode = LAYER_100B[i]
    check_matrix(5, i + 64, N, K, mode, 64, fused=False, sampled=True)


@pytest.mark.parametrize("i", range(4))
def test_100b_decode_m1_prequantized(i):
    """The two-call path (quantize, then the product) at M = 1, full outputs and
    accumulators: the launch shapes the pre-quantized dispatch picks for long rows."""
    name, N, K, mode = LAYER_100B[i]
    check_matrix(5, i + 16, N, K, mode, 1, fused=False)


@pytest.mark.parametrize("M", [8, 32])
@pytest.mark.parametrize("i", range(4))
def test_100b_few_tokens(M, i):
    """8 tokens (the few-token matrix-core kernel; down with its K split) and 32 tokens (the
    tiled product; down with its K split), as bench.py times them; sampled outputs."""
    name, N, K, mode = LAYER_100B[i]
    check_matrix(5, i + 8 * M, N, K, mode, M, fused=False, sampled=True)


LAYER_100B_TP8 = [("qkv", 1280, 8192, "plain"), ("o", 8192, 1024, "norm"), ("up", 3584, 8192, "plain"),
                  ("down", 8192, 3584, "relu2norm")]


@pytest.mark.parametrize("i", range(4))
def test_100b_tp8_shard_m1(i):
    """One GPU's share of the 100B slice under 8-way tensor parallelism at one token: the
    fused call and the pre-quantized product, full outputs."""
    name, N, K, mode = LAYER_100B_TP8[i]
    check_matrix(6, i, N, K, mode, 1, fused=True)
    check_matrix(6, i + 4, N, K, mode, 1, fused=False)


def test_max_output_width_four_token_tiles():
    """The widest output the chunked product takes, N = 2^27 - 1 rows, with four-token tiles
    (M = 4, K = 64): a tile's output buffer is then 4 N floats = 2^31 - 16 bytes, ending
    exactly at the out-of-range offset that masked lanes store to, so those stores must be
    dropped and every output row, the last ones included, must hold the oracle's values.
    Checked on sampled rows and on the last 64 rows of every token."""
    M, N, K = 4, (1 << 27) - 1, 64
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2027)
    codes = torch.randint(0, 3, (N, K // 4, 4), generator=gen, device=DEV, dtype=torch.int32)
    packed = (codes[..., 0] | (codes[..., 1] << 2) | (codes[..., 2] << 4) | (codes[..., 3] << 6)).to(torch.uint8)
    del codes
    gamma = torch.tensor([0.0123], dtype=torch.float32, device=DEV)
    x = datagen.outlier_acts(M, K, 2028)
    xq, s = bl.bitlinear_quantize_act(torch.from_numpy(x).to(DEV))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    bl.bitlinear_forward(xq, s, packed, gamma, y=y, split=False)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(N, seed=5), np.arange(N - 64, N)]))
    q, bad = oracle.unpack(packed[torch.from_numpy(rows).to(DEV)].cpu().numpy(), K)
    assert bad == 0
    oxq, os_ = oracle.quantize_act(x)
    assert np.array_equal(xq.cpu().numpy(), oxq)
    _, oy = oracle.forward(oxq, os_, q, np.float32(0.0123))
    yh = y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(yh.view(np.int32), oy.view(np.int32))


def test_max_k_one_and_two_tokens():
    """K at the API maximum (2^20): the product on the generic path, plain and subln input,
    full outputs against the oracle."""
    K = 1 << 20
    for M, N, mode in ((1, 3, None), (2, 5, "norm")):
        w = datagen.gg_weights(N, K, 2030 + M)
        x = datagen.outlier_acts(M, K, 2031 + M)
        gain = datagen.gains(K, 2032) if mode else None
        packed, gamma = bl.bitlinear_pack_weights(torch.from_numpy(w).to(DEV))
        y = bl.bitlinear_forward_f32(torch.from_numpy(x).to(DEV), packed, gamma,
                                     None if gain is None else torch.from_numpy(gain).to(DEV), EPS, 0)
        torch.cuda.synchronize()
        o = oracle.bitlinear(x, w, gain=gain, eps=EPS) if mode else oracle.bitlinear(x, w)
        assert np.array_equal(packed.cpu().numpy(), o["packed"])
        yh = y.cpu().numpy()
        if mode is None:
            assert np.array_equal(yh.view(np.int32), o["y"].view(np.int32))
        else:
            assert (np.abs(yh.astype(np.float64) - o["y"]) <= 1e-6 * np.abs(o["y"].astype(np.float64))).all()
