"""GPU parity of the five-codes-per-byte format (1.6 bits per weight).

The GPU repacker is compared byte for byte with the oracle's packer on the same codes;
bitlinear_forward5 is compared with the oracle's product (int32 accumulators and fp32
outputs bit for bit) and with bitlinear_forward on the 2-bit layout of the same
weights, at ragged K (partial last group, partial last 80-code chunk), every token-tile
shape and the 2B / 100B layer shapes.
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


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not _build.up_to_date():
        _build.build()
    bl.lib()
    oracle.lib()
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def down(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("N,K", [(3, 4), (5, 68), (7, 80), (9, 84), (33, 260), (40, 2560), (17, 6912),
                                 (3, 28672)])
def test_repack5_matches_oracle_packer(N, K):
    w = datagen.gg_weights(N, K, 7100 + K)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    p5 = bl.bitlinear_repack5(packed)
    _, ogamma, q = oracle.pack_weights(w)
    assert float(down(gamma)[0]) == float(ogamma)
    assert np.array_equal(down(p5), oracle.pack5(q))


CASES = [
    # (M, N, K): K % 16 == 0; chunk tails (K % 80 != 0), 1/2/4-token tiles and token tails,
    # lanes per row from 16 to 256 and the 8-chunk tile of the longest rows
    (1, 7, 16), (1, 33, 80), (2, 20, 96), (3, 17, 2560), (5, 70, 2560), (8, 129, 6912), (1, 300, 8192),
    (4, 40, 8192), (2, 61, 16384), (1, 50, 28672), (7, 9, 28672), (1, 5, 131072), (17, 23, 1040),
]


@pytest.mark.parametrize("M,N,K", CASES)
def test_forward5_parity(M, N, K):
    w = datagen.gg_weights(N, K, 7200 + N + K)
    x = datagen.outlier_acts(M, K, 7300 + M + K)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    p5 = bl.bitlinear_repack5(packed)
    xq, s = bl.bitlinear_quantize_act(up(x))
    y5, acc5 = bl.bitlinear_forward5(xq, s, p5, gamma, acc=True)
    y2, acc2 = bl.bitlinear_forward(xq, s, packed, gamma, acc=True)
    o = oracle.bitlinear(x, w)
    assert np.array_equal(down(acc5), o["acc"])
    assert np.array_equal(down(y5).view(np.int32), o["y"].view(np.int32))
    assert torch.equal(acc5, acc2) and torch.equal(y5, y2)


@pytest.mark.parametrize("N,K", [(3840, 2560), (2560, 6912), (28672, 8192), (8192, 28672)])
def test_forward5_full_layer_shapes_match_2bit(N, K):
    """Full 2B / 100B matrices at M = 1 and 4: identical to the 2-bit path everywhere,
    and to the oracle on sampled rows."""
    w = datagen.gg_weights_torch(N, K, datagen.stream_id(6, 0, K % 7, 0), DEV)
    packed, gamma = bl.bitlinear_pack_weights(w)
    p5 = bl.bitlinear_repack5(packed)
    rows = np.unique(np.concatenate([np.random.default_rng(K).choice(N, 40, replace=False), [0, N - 1]]))
    wh = w[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    q_rows = oracle.weight_codes(wh, np.float32(down(gamma)[0]))
    del w
    for M in (1, 4):
        x = datagen.outlier_acts_torch(M, K, datagen.stream_id(6, 1, M, 1), DEV)
        xq, s = bl.bitlinear_quantize_act(x)
        y5, acc5 = bl.bitlinear_forward5(xq, s, p5, gamma, acc=True)
        y2, acc2 = bl.bitlinear_forward(xq, s, packed, gamma, acc=True)
        assert torch.equal(acc5, acc2) and torch.equal(y5, y2)
        oacc, _ = oracle.forward(down(xq), down(s), q_rows, down(gamma)[0])
        assert np.array_equal(down(acc5)[:, rows], oacc)
