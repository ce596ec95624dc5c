"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Bar: packed bytes, gamma, activation codes, plain-path scales and int32 accumulators
bit-exact; fp32 outputs bit-exact on the plain path; on the RMSNorm (subln) path the
scale's binary64 sum is summed in a different order than the oracle's, so scales may
differ by an ulp and y is held to 1e-6 relative (the tolerance the method's target
states). The fused entry point must equal quantize + forward bit for bit.
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
F32 = np.float32


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


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def latents(n, k, seed, kind="gg"):
    if kind == "gauss":
        return datagen.gaussian_weights(n, k, seed)
    return datagen.gg_weights(n, k, seed)


# ------------------------------------------------------------------------------ packing

PACK_SHAPES = [(1, 4, "gauss"), (3, 64, "gg"), (37, 260, "gg"), (64, 2560, "gauss"), (5, 4100, "gg"),
               (2560, 2560, "gauss"), (3840, 2560, "gg"), (4096, 4100, "gg")]


@pytest.mark.parametrize("N,K,kind", PACK_SHAPES)
def test_pack_parity(N, K, kind):
    w = latents(N, K, 1000 + N + K, kind)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    opacked, ogamma, _ = oracle.pack_weights(w)
    assert down(gamma)[0] == ogamma
    assert np.array_equal(down(packed), opacked)


def test_pack_golden_and_degenerate(golden):
    g = golden["weight_ties"]
    packed, gamma = bl.bitlinear_pack_weights(up(np.array(g["W"], np.float32)))
    assert down(gamma)[0] == F32(g["gamma"])
    assert down(packed).tolist() == g["packed"]
    z = np.zeros((9, 36), np.float32)
    packed, gamma = bl.bitlinear_pack_weights(up(z))
    assert down(gamma)[0] == F32(1e-8)
    assert (down(packed) == 0x55).all()          # every field is code 0 -> 0b01
    # huge dynamic range: a single large weight dominates gamma
    w = latents(16, 64, 7)
    w[3, 5] = 1e6
    opacked, ogamma, _ = oracle.pack_weights(w)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    assert down(gamma)[0] == ogamma and np.array_equal(down(packed), opacked)


def test_pack_reuses_workspace_and_is_deterministic():
    w = up(latents(300, 520, 8))
    ws = torch.empty((bl.bitlinear_pack_workspace_bytes(300, 520),), dtype=torch.uint8, device=DEV)
    p1, g1 = bl.bitlinear_pack_weights(w, workspace=ws)
    p2, g2 = bl.bitlinear_pack_weights(w, workspace=ws)
    assert torch.equal(p1, p2) and torch.equal(g1, g2)


# ------------------------------------------------------------------------------ activations

QUANT_CASES = [
    (1, 4, None), (3, 260, None), (5, 2560, "norm"), (7, 6912, "relu2norm"), (4, 64, "relu2"),
    (64, 2560, None), (512, 6912, None), (16, 28672, "relu2norm"), (33, 8192, "norm"),
    # gated squared ReLU: rows of [gate | up], 2K values per token
    (3, 2560, "gated"), (5, 6912, "gatednorm"), (2, 28672, "gatednorm"), (6, 260, "gatednorm"),
]


def make_acts(M, K, seed, heavy=False):
    return datagen.heavy_channel_acts(M, K, seed) if heavy else datagen.outlier_acts(M, K, seed)


def pro_args(mode, K, seed):
    """(gain or None, activation mode 0/1/2) for a test mode name."""
    gain = datagen.gains(K, seed) if mode in ("norm", "relu2norm", "gatednorm") else None
    act = 2 if mode in ("gated", "gatednorm") else int(mode in ("relu2", "relu2norm"))
    return gain, act


def row_len(mode, K):
    return 2 * K if mode in ("gated", "gatednorm") else K


@pytest.mark.parametrize("M,K,mode", QUANT_CASES)
def test_quantize_act_parity(M, K, mode):
    x = make_acts(M, row_len(mode, K), 2000 + M + K, heavy=(M >= 64))
    if M > 2:
        x[0, :] = 0.0                           # an all-zero token takes the 1e-8 floor
    gain, relu2 = pro_args(mode, K, 3000 + K)
    xq, s = bl.bitlinear_quantize_act(up(x), None if gain is None else up(gain), EPS, relu2)
    if mode is None:
        oxq, os_ = oracle.quantize_act(x)
    else:
        oxq, os_ = oracle.quantize_act_norm(x, gain, EPS, relu2)
    assert np.array_equal(down(xq), oxq)
    if gain is None:
        assert np.array_equal(down(s), os_)
    else:
        assert ulp_diff(down(s), os_).max() <= 2


def test_quantize_act_golden(golden):
    g = golden["act_quant"]
    xq, s = bl.bitlinear_quantize_act(up(np.array(g["X"], np.float32)))
    assert down(xq).tolist() == g["codes"] and down(s).tolist() == g["scale"]
    g = golden["relu2_norm"]
    xq, s = bl.bitlinear_quantize_act(up(np.array(g["U"], np.float32)), up(np.array(g["gain"], np.float32)),
                                      g["eps"], True)
    assert down(xq).tolist() == g["codes"]
    g = golden["gated_relu2"]
    xq, s = bl.bitlinear_quantize_act(up(np.array(g["U"], np.float32)), None, EPS, 2)
    assert down(xq).tolist() == g["codes"]


# ------------------------------------------------------------------------------ forward

def run_gpu(x, w, mode=None, gain=None, relu2=False):
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xg = up(x)
    gg = None if gain is None else up(gain)
    if mode is None:
        xq, s = bl.bitlinear_quantize_act(xg)
    else:
        xq, s = bl.bitlinear_quantize_act(xg, gg, EPS, relu2)
    y, acc = bl.bitlinear_forward(xq, s, packed, gamma, acc=True)
    yf = bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, relu2)
    y1 = bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, relu2, one_launch=True)
    return dict(packed=down(packed), gamma=down(gamma)[0], xq=down(xq), s=down(s), y=down(y), acc=down(acc),
                yf=down(yf), y1=down(y1))


def compare(r, o, norm):
    assert r["gamma"] == o["gamma"]
    assert np.array_equal(r["packed"], o["packed"])
    assert np.array_equal(r["xq"], o["xq"])
    assert np.array_equal(r["acc"], o["acc"])
    assert np.array_equal(r["y"].view(np.int32), r["yf"].view(np.int32)), "fused != quantize+forward"
    assert np.array_equal(r["y"].view(np.int32), r["y1"].view(np.int32)), "one-launch fused != quantize+forward"
    if not norm:
        assert np.array_equal(r["s"], o["s"])
        assert np.array_equal(r["y"].view(np.int32), o["y"].view(np.int32))
    else:
        yo = o["y"].astype(np.float64)
        err = np.abs(r["y"].astype(np.float64) - yo)
        assert (err <= 1e-6 * np.abs(yo)).all()


FWD_CASES = [
    # (M, N, K, mode)  small shapes: several tiles and ragged tails
    (1, 1, 4, None), (1, 7, 64, None), (2, 37, 260, None), (3, 96, 2560, None), (4, 64, 6912, "norm"),
    (5, 33, 128, "relu2"), (8, 129, 2560, "relu2norm"), (16, 100, 1024, None), (64, 70, 8192, "norm"),
    (1, 300, 28672, "relu2norm"), (2, 17, 16384, None), (3, 5, 65536, None), (6, 40, 192, None),
    (1, 2560, 2560, None),
    (1, 2560, 6912, "gatednorm"), (4, 70, 2560, "gatednorm"), (2, 33, 260, "gatednorm"),
    (1, 50, 28672, "gatednorm"), (3, 17, 128, "gated"), (8, 300, 6912, "gatednorm"),
    # one-token tiles of the fused prologue: 4 and 8 units per thread kept in registers,
    # rows past 8 units re-read for their codes, every activation kind with and without norm
    (1, 33, 16384, "norm"), (1, 40, 65536, "relu2norm"), (1, 24, 65536, "gatednorm"), (1, 20, 65536, "gated"),
    (1, 40, 28672, "gated"), (1, 50, 8192, "relu2"), (1, 30, 32768, "norm"),
    # pre-quantized rows of 257..448 chunks (one wave per row, 7 chunks per lane, some lanes
    # holding fewer) and of 449..512 (four waves per row)
    (1, 77, 20480, None), (1, 45, 16448, None), (1, 9, 28672, None), (1, 21, 30720, None),
    # fused rows of 257..448 chunks at one token: the two-role kernel (waves 0-3 derive the
    # codes, waves 4-7 stream weights); one pass per block, a ragged last pass, 8-9 passes
    # (6-7 streamed, 2 by the prologue waves) and 13 (10 and 3: an odd count in turns of two)
    (1, 1, 28672, None), (1, 5, 20480, "norm"), (1, 1030, 24576, "relu2"), (1, 8200, 16448, "gated"),
    (1, 12300, 16448, "relu2norm"), (1, 4101, 28672, "gatednorm"),
    # the two-role kernel with 32 lanes per row (K <= 8192 on >= 128M weights, two blocks
    # per CU): 8 rows per pass, 8-9 passes per block
    (1, 16400, 8192, "norm"), (1, 17000, 7936, "gatednorm"),
]


@pytest.mark.parametrize("M,N,K,mode", FWD_CASES)
def test_forward_parity(M, N, K, mode):
    w = latents(N, K, 4000 + N * 7 + K)
    x = make_acts(M, row_len(mode, K), 5000 + M + K)
    gain, relu2 = pro_args(mode, K, 6000 + K)
    r = run_gpu(x, w, mode, gain, relu2)
    o = oracle.bitlinear(x, w, gain=gain, eps=EPS, relu2=relu2) if mode else oracle.bitlinear(x, w)
    compare(r, o, gain is not None)


def test_forward_degenerate():
    """All-zero activations give y = 0; all-zero weights give y = 0; one-hot input."""
    w = latents(40, 256, 11)
    x = np.zeros((3, 256), np.float32)
    x[1, 17] = -3.25
    r = run_gpu(x, w)
    o = oracle.bitlinear(x, w)
    compare(r, o, False)
    assert (r["y"][0] == 0).all() and (r["y"][2] == 0).all()
    r = run_gpu(make_acts(2, 256, 12), np.zeros((40, 256), np.float32))
    assert (r["y"] == 0).all() and (r["acc"] == 0).all()


def test_forward_misaligned_views():
    """Row strides that are not multiples of 16 bytes and offset views take the generic path."""
    w = latents(21, 68, 13)
    x = make_acts(3, 68, 14)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    big = torch.zeros(packed.numel() + 1, dtype=torch.uint8, device=DEV)
    off = big[1:].view(packed.shape)
    off.copy_(packed)
    xq, s = bl.bitlinear_quantize_act(up(x))
    y1 = bl.bitlinear_forward(xq, s, packed, gamma)
    y2 = bl.bitlinear_forward(xq, s, off, gamma)
    assert torch.equal(y1, y2)
    o = oracle.bitlinear(x, w)
    assert np.array_equal(down(y1), o["y"])


# ------------------------------------------------------------------------------ MFMA path (M >= 16)

GEMM_CASES = [
    # (M, N, K): token and feature tails, K steps of 64 and 128, all block shapes; whole
    # 64 x 256 and 32 x 128 tiles (the store epilogue without bounds checks) with K tails
    (16, 33, 64), (17, 129, 192), (64, 256, 2560), (100, 70, 6912), (255, 300, 128), (256, 384, 2560),
    (300, 257, 1024), (512, 128, 8192), (2048, 96, 2560), (40, 1000, 28672),
    (512, 512, 2560), (1024, 768, 1024), (2048, 512, 192), (600, 1024, 64), (32, 1024, 6912),
]


# Many tiles of 64 x 256 (at least 40% of a round of two blocks on each of 256 CUs): the
# two-role kernel (activation loader waves). Ragged M and N, K tails of 64, a single K step.
ROLES_CASES = [(1216, 2600, 2624), (1000, 6912, 192), (2048, 2560, 64), (1280, 3840, 6912)]


@pytest.mark.parametrize("M,N,K", ROLES_CASES)
def test_gemm_roles_parity(M, N, K):
    """Codes, accumulators and outputs bit-exact against the oracle on sampled output
    columns (every row), with and without the int32 copy, and the residual form equal to
    the plain output added in fp32."""
    w = latents(N, K, 7100 + N + K)
    x = make_acts(M, K, 8100 + M + K, heavy=True)
    print("roles GEMM case M=%d N=%d K=%d" % (M, N, K), flush=True)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xq, s = bl.bitlinear_quantize_act(up(x))
    y, acc = bl.bitlinear_forward(xq, s, packed, gamma, acc=True)
    y_plain = bl.bitlinear_forward(xq, s, packed, gamma)
    y0 = datagen.outlier_acts(M, N, 8200 + M + N)
    yr = up(y0)
    bl.bitlinear_forward(xq, s, packed, gamma, y=yr, residual=True)
    rng = np.random.default_rng(N + K)
    cols = np.unique(np.concatenate([rng.choice(N, size=40, replace=False), [0, 255, 256, N - 1]]))
    opacked, ogamma, _ = oracle.pack_weights(w)
    oxq, os_ = oracle.quantize_act(x)
    assert np.array_equal(down(xq), oxq)
    oacc, oy = oracle.forward(oxq, os_, oracle.weight_codes(w[cols], ogamma), ogamma)
    assert np.array_equal(down(acc)[:, cols], oacc)
    assert np.array_equal(down(y)[:, cols].view(np.int32), oy.view(np.int32))
    assert np.array_equal(down(y_plain).view(np.int32), down(y).view(np.int32))
    assert np.array_equal(down(yr).view(np.int32), oracle_residual(y0, down(y)).view(np.int32))
    # the fused call (quantize into a workspace, then this product) gives the same bits,
    # plain and with a gated subln input
    assert np.array_equal(down(bl.bitlinear_forward_f32(up(x), packed, gamma)).view(np.int32),
                          down(y).view(np.int32))
    xg = make_acts(M, 2 * K, 8300 + M + K)
    gain, act = pro_args("gatednorm", K, 8400 + K)
    xqg, sg = bl.bitlinear_quantize_act(up(xg), up(gain), EPS, act)
    yg = bl.bitlinear_forward(xqg, sg, packed, gamma)
    ygf = bl.bitlinear_forward_f32(up(xg), packed, gamma, up(gain), EPS, act)
    assert np.array_equal(down(ygf).view(np.int32), down(yg).view(np.int32))


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
def test_gemm_parity(M, N, K):
    """Codes, accumulators and outputs bit-exact against the oracle; the call without the
    int32 copy (a different store path) gives the same output bits."""
    w = latents(N, K, 7000 + N + K)
    x = make_acts(M, K, 8000 + M + K, heavy=True)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xq, s = bl.bitlinear_quantize_act(up(x))
    y, acc = bl.bitlinear_forward(xq, s, packed, gamma, acc=True)
    y_plain = bl.bitlinear_forward(xq, s, packed, gamma)
    o = oracle.bitlinear(x, w)
    assert np.array_equal(down(xq), o["xq"])
    assert np.array_equal(down(acc), o["acc"])
    assert np.array_equal(down(y).view(np.int32), o["y"].view(np.int32))
    assert np.array_equal(down(y_plain).view(np.int32), o["y"].view(np.int32))


# ------------------------------------------------------------------------------ K split (10..32 tokens, long rows)

SPLIT_CASES = [
    # (M, N, K): 8 slices of 8 K steps; 8 slices on two feature tiles; 8 slices of 14 steps on
    # ragged token and feature tiles; 8 slices of 10 steps on a ragged feature tile; 8 slices
    # whose last one ends inside a K step (K % 256 = 64); 8 slices of 32 steps; the 100B down
    # projection at 32 tokens on a subset of its rows; 3 slices (many tiles)
    (16, 96, 16384), (32, 256, 16384), (20, 200, 28672), (32, 130, 20480), (17, 50, 16448),
    (16, 64, 65536), (32, 1024, 28672), (24, 40000, 16384),
    # from 10 tokens (and 8 on matrices of >= 64M weights): one token tile of few rows
    (10, 64, 16384), (13, 130, 20480), (8, 4100, 16384),
]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES)
def test_split_k_parity(M, N, K):
    """bitlinear_forward_ws (K split across blocks, int32 partials summed by a second
    kernel): y and acc bit for bit the unsplit call's and the oracle's, also with a
    workspace full of stale bytes reused twice; residual adds bit for bit as fp32."""
    need = bl.bitlinear_forward_workspace_bytes(M, N, K)
    assert need > 0, "shape must take the split path"
    w = latents(N, K, 9900 + N + K)
    x = make_acts(M, K, 9950 + M + K, heavy=True)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xq, s = bl.bitlinear_quantize_act(up(x))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    ys, accs = bl.bitlinear_forward(xq, s, packed, gamma, acc=True, workspace=ws)
    ys2 = bl.bitlinear_forward(xq, s, packed, gamma, workspace=ws)
    yu, accu = bl.bitlinear_forward(xq, s, packed, gamma, acc=True, split=False)
    o = oracle.bitlinear(x, w)
    assert np.array_equal(down(xq), o["xq"])
    assert np.array_equal(down(accs), o["acc"])
    assert np.array_equal(down(accu), o["acc"])
    for y in (ys, ys2, yu):
        assert np.array_equal(down(y).view(np.int32), o["y"].view(np.int32))
    y0 = datagen.outlier_acts(M, N, 9990 + M + N)
    yr = up(y0)
    bl.bitlinear_forward(xq, s, packed, gamma, y=yr, residual=True, workspace=ws)
    assert np.array_equal(down(yr).view(np.int32), oracle_residual(y0, o["y"]).view(np.int32))


# ------------------------------------------------------------------------------ few tokens on the matrix cores

MFMA_CASES = [
    # (M, N, K): 2..16 tokens through the matrix-core kernel with the activation codes in LDS:
    # ragged row groups (N % 16), K past the last full window of 256 codes (K % 256 = 64, 192),
    # one window, several row groups per block, the longest rows it takes (4 tokens at
    # K = 28672), 16 tokens (no zero slot), 2 tokens on a matrix of >= 128M weights
    (3, 33, 64), (4, 100, 320), (5, 257, 2560), (7, 1000, 448), (8, 130, 6912), (9, 64, 8192),
    (12, 8200, 256), (15, 77, 1088), (16, 129, 2560), (4, 50, 28672), (2, 16400, 8192),
    # rows longer than LDS holds, staged in phases: 2 phases (8 tokens at K = 28672, 12 at
    # 20480), 2 phases of 34 and 31 windows ending inside a window, 3 phases
    (8, 100, 28672), (12, 50, 20480), (15, 33, 16448), (5, 40, 65536),
    # 17..24 tokens: two tiles of 16 tokens per weight operand (zero slot for tokens past M)
    (17, 300, 2560), (24, 129, 6912), (20, 1000, 1088), (21, 64, 16448),
]


@pytest.mark.parametrize("M,N,K", MFMA_CASES)
def test_mfma_small_parity(M, N, K):
    """y and acc bit for bit the oracle's; the residual form adds in fp32 bit for bit; the
    fused call with a workspace (quantize, then the product) equals quantize + forward.
    The product is called without a workspace, so rows that the K split would take
    (10+ tokens, K >= 16384) also run on this kernel's LDS phases."""
    w = latents(N, K, 9500 + N + K)
    x = make_acts(M, K, 9550 + M + K, heavy=True)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xq, s = bl.bitlinear_quantize_act(up(x))
    y, acc = bl.bitlinear_forward(xq, s, packed, gamma, acc=True, split=False)
    o = oracle.bitlinear(x, w)
    assert np.array_equal(down(xq), o["xq"])
    assert np.array_equal(down(acc), o["acc"])
    assert np.array_equal(down(y).view(np.int32), o["y"].view(np.int32))
    y0 = datagen.outlier_acts(M, N, 9580 + M + N)
    yr = up(y0)
    bl.bitlinear_forward(xq, s, packed, gamma, y=yr, residual=True, split=False)
    assert np.array_equal(down(yr).view(np.int32), oracle_residual(y0, o["y"]).view(np.int32))
    gain, act = pro_args("relu2norm", K, 9590 + K)
    xg, gg = up(x), up(gain)
    need = bl.bitlinear_forward_f32_workspace_bytes(M, N, K)
    ws = torch.full((max(need, 16),), 0x3C, dtype=torch.uint8, device=DEV)
    yw = bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, act, workspace=ws)
    xq2, s2 = bl.bitlinear_quantize_act(xg, gg, EPS, act)
    y2 = bl.bitlinear_forward(xq2, s2, packed, gamma)
    assert np.array_equal(down(yw).view(np.int32), down(y2).view(np.int32))


# ------------------------------------------------------------------------------ residual forms

RESIDUAL_CASES = [
    # (M, N, K, mode): GEMV tiles of 1, 2 and 4 tokens incl. the large-K tiles, the
    # generic path (K % 64 != 0), the MFMA path (M >= 16), fused prologue modes
    (1, 2560, 2560, "norm"), (1, 2560, 6912, "relu2norm"), (1, 300, 6912, "gatednorm"), (2, 70, 2560, None),
    (4, 129, 8192, None), (3, 6912, 6912, None), (1, 37, 260, "norm"), (5, 33, 260, None), (64, 200, 2560, None),
    (16, 33, 64, None), (1, 1024, 28672, None),
    # one-token launch shapes of the decode stack and the 100B slice: two rows per lane
    # (2B up), three passes in flight (100B O: both the fused and the pre-quantized shape)
    (1, 6912, 2560, None), (1, 8192, 8192, "norm"),
    # the two-role kernel (fused rows of 257..448 chunks, one token; 32 lanes per row on
    # >= 128M weights)
    (1, 300, 28672, "relu2norm"), (1, 9000, 20480, "gatednorm"), (1, 16400, 8192, "relu2"),
]


WS_CASES = [
    # (M, N, K, mode): token counts that take the workspace path (quantize, then the MFMA
    # product), incl. ragged tiles, each input kind, and a K the matrix cores do not take
    (16, 96, 2560, None), (100, 130, 2560, "norm"), (300, 64, 6912, "relu2norm"), (64, 40, 2560, "gatednorm"),
    (33, 50, 260, "relu2"), (17, 8, 128, "gated"),
    # few tokens through the matrix-core product
    (4, 300, 2560, "norm"), (8, 77, 6912, "relu2norm"), (12, 130, 8192, None), (3, 50, 2560, "gatednorm"),
]


@pytest.mark.parametrize("M,N,K,mode", WS_CASES)
def test_forward_f32_workspace(M, N, K, mode):
    """bitlinear_forward_f32_ws: bit for bit quantize + forward, and the oracle's result
    (bit-exact on the plain path, within 1e-6 on the subln path); a reused workspace gives
    the same bits again."""
    w = latents(N, K, 9600 + N + K)
    x = make_acts(M, row_len(mode, K), 9700 + M + K, heavy=True)
    gain, act = pro_args(mode, K, 9800 + K)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xg, gg = up(x), None if gain is None else up(gain)
    need = bl.bitlinear_forward_f32_workspace_bytes(M, N, K)
    assert need >= M * K + 4 * M
    ws = torch.full((need + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    yw = bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, act, workspace=ws)
    yw2 = bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, act, workspace=ws)
    xq, s = bl.bitlinear_quantize_act(xg, gg, EPS, act)
    y = bl.bitlinear_forward(xq, s, packed, gamma)
    rw, rw2, r = down(yw), down(yw2), down(y)
    assert np.array_equal(rw.view(np.int32), r.view(np.int32))
    assert np.array_equal(rw2.view(np.int32), r.view(np.int32))
    o = oracle.bitlinear(x, w, gain=gain, eps=EPS, relu2=act) if mode else oracle.bitlinear(x, w)
    if gain is None:
        assert np.array_equal(rw.view(np.int32), o["y"].view(np.int32))
    else:
        yo = o["y"].astype(np.float64)
        assert (np.abs(rw.astype(np.float64) - yo) <= 1e-6 * np.abs(yo)).all()


def oracle_residual(y0, y_ora):
    return (y0.astype(np.float32) + y_ora.astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("M,N,K,mode", RESIDUAL_CASES)
def test_residual_parity(M, N, K, mode):
    """Y + product: bit for bit equal to adding the plain call's output in fp32, and
    against the oracle bit-exact on the plain path, within the 1e-6 output tolerance
    (plus the add's own rounding) on the RMSNorm path."""
    w = latents(N, K, 9100 + N + K)
    x = make_acts(M, row_len(mode, K), 9200 + M + K)
    gain, act = pro_args(mode, K, 9300 + K)
    y0 = datagen.outlier_acts(M, N, 9400 + M + N)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xg, gg = up(x), None if gain is None else up(gain)
    if mode is None:
        o = oracle.bitlinear(x, w)
        xq, s = bl.bitlinear_quantize_act(xg)
    else:
        o = oracle.bitlinear(x, w, gain=gain, eps=EPS, relu2=act)
        xq, s = bl.bitlinear_quantize_act(xg, gg, EPS, act)
    expect = oracle_residual(y0, o["y"])
    ya = up(y0)
    bl.bitlinear_forward(xq, s, packed, gamma, y=ya, residual=True)
    yb = up(y0)
    bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, act, y=yb, residual=True)
    yc = up(y0)
    bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, act, y=yc, residual=True, one_launch=True)
    plain = bl.bitlinear_forward(xq, s, packed, gamma)
    ra, rb, rc, rp = down(ya), down(yb), down(yc), down(plain)
    same = oracle_residual(y0, rp)
    assert np.array_equal(ra.view(np.int32), same.view(np.int32))
    assert np.array_equal(rb.view(np.int32), same.view(np.int32))
    assert np.array_equal(rc.view(np.int32), same.view(np.int32))
    if gain is None:
        assert np.array_equal(ra.view(np.int32), expect.view(np.int32))
    else:
        tol = 1e-6 * np.abs(o["y"].astype(np.float64)) + 2.0 ** -23 * np.abs(expect.astype(np.float64))
        assert (np.abs(ra.astype(np.float64) - expect.astype(np.float64)) <= tol).all()


def test_binding_rejects_short_buffers():
    """The library trusts the sizes it is given; the binding checks every buffer's shape."""
    w = latents(40, 256, 21)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    x = up(make_acts(3, 256, 22))
    xq, s = bl.bitlinear_quantize_act(x)
    with pytest.raises(ValueError):
        bl.bitlinear_forward(xq, s, packed, gamma, y=torch.empty((3, 39), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        bl.bitlinear_forward(xq, s[:2], packed, gamma)
    with pytest.raises(ValueError):
        bl.bitlinear_forward_f32(x, packed, gamma, torch.ones(255, device=DEV))
    with pytest.raises(ValueError):
        bl.bitlinear_quantize_act(x, xq=torch.empty((3, 255), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):
        bl.bitlinear_forward(xq, s, packed, gamma, y=torch.empty((3, 40), dtype=torch.float32, device=DEV),
                             residual=True, acc=True)


# ------------------------------------------------------------------------------ graph replay

@pytest.mark.parametrize("M,N,K,mode", [
    (1, 300, 2560, "relu2norm"),     # one-token fused product
    (8, 500, 2560, None),            # few tokens on the matrix cores
    (12, 200, 16384, None),          # K split across blocks (workspace, reduce kernel)
    (40, 300, 2560, None),           # tiled matrix-core product
])
def test_products_graph_replay(M, N, K, mode):
    """A captured graph of the product (with its workspace where it takes one) gives the
    eager result bit for bit on every replay, with eager work and synchronisations between
    the replays."""
    w = latents(N, K, 9700 + N + K)
    x = make_acts(M, row_len(mode, K), 9710 + M + K)
    gain, act = pro_args(mode, K, 9720 + K)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    xg, gg = up(x), None if gain is None else up(gain)
    if mode is None:
        xq, s = bl.bitlinear_quantize_act(xg)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = torch.empty((max(16, bl.bitlinear_forward_workspace_bytes(M, N, K)),), dtype=torch.uint8, device=DEV)

    def run(stream=None):
        if mode is None:
            bl.bitlinear_forward(xq, s, packed, gamma, y=y, workspace=ws, stream=stream)
        else:
            bl.bitlinear_forward_f32(xg, packed, gamma, gg, EPS, act, y=y, stream=stream)

    run()
    torch.cuda.synchronize()
    eager = down(y).copy()
    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            run(stream=st)
    for i in range(3):
        y.fill_(float("nan"))
        ws.fill_(0xA5 + i)
        other = torch.randn(64, 64, device=DEV) @ torch.randn(64, 64, device=DEV)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down(y).view(np.int32), eager.view(np.int32)), "replay %d" % i
        del other


def test_binding_scratch_survives_a_side_stream():
    """Scratch the binding allocates for a call on a side stream (here the workspace of the
    fused call at 32 tokens: codes and scales) must not be handed out again before that
    stream is done with it. The side stream is held back by a bounded spin kernel, the
    buffer is dropped when the call returns, and the current stream at once allocates the
    same number of bytes and fills them; the product must still equal the one computed on
    the current stream."""
    M, N, K = 32, 1024, 2560
    w = latents(N, K, 4242)
    x = make_acts(M, K, 4243)
    packed, gamma = bl.bitlinear_pack_weights(up(w))
    X = up(x)
    ref = bl.bitlinear_forward_f32(X, packed, gamma)
    torch.cuda.synchronize()
    need = bl.bitlinear_forward_f32_workspace_bytes(M, N, K)
    assert need > 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
    bl.bitlinear_forward_f32(X, packed, gamma, y=y, stream=side)
    junk = torch.empty((need,), dtype=torch.uint8, device=DEV)
    junk.fill_(0x7F)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
