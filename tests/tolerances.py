"""Output tolerances shared by the GPU parity tests, derived from the kernels' fp32
arithmetic (each function states its derivation)."""
import numpy as np

import oracle

U = 2.0 ** -24
D = 128
KAPPA = 1.4426950408889634 / np.sqrt(128.0)


def attention_bound(qkv, kc_after, vc_after, pos, H, KVH, theta=10000.0):
    """Per-output bound of decode attention (u = 2^-24; base-2 scores, query pre-scaled by
    kappa = log2(e)/sqrt(128)):
      * the rotated query is within 3u(|x_i| + |x_partner|) per dim, the scale adds 2u and
        the 128-term dot product (an 8-term FMA chain, then a 4-step tree) gamma_12, so
        |ds_j| <= 20 u E_j with E_j = kappa sum_i (|x_i| + |x_partner(i)|) |k_ji|;
      * exact softmax weights P_j move by at most 2 ln2 max_j |ds_j| relative; exp2 of
        s_j - m adds about 2u plus ln2 u |s_j - m| (weights with |s - m| > 94 are below
        2^-94 and drop out);
      * with n = pos / 64 + 1 sub-chunks of 64 positions, a lane sums at most 4 positions
        per sub-chunk and rescales its running sums (one product and one exp2, about 3u)
        at most once per sub-chunk; then 16 rows and at most n chunk partials are added.
    So |out_d - ref_d| <= u (28 max_j E_j + 8 n + 136) sum_j P_j |v_jd|; the bound returned
    is twice that. Rows of invalid positions are NaN."""
    M = qkv.shape[0]
    G = H // KVH
    tol = np.full((M, H * D), np.nan)
    for b in range(M):
        p = int(pos[b])
        if not 0 <= p < kc_after.shape[2]:
            continue
        n_sub = p // 64 + 1
        for h in range(H):
            g = h // G
            x = np.abs(qkv[b, h * D:(h + 1) * D].astype(np.float64))
            xx = x + np.roll(x, D // 2)                       # |x_i| + |x_partner(i)|
            keys = oracle.bf16_value(kc_after[b, g, :p + 1])
            E = KAPPA * np.abs(keys) @ xx
            qr = oracle.rope(qkv[b, h * D:(h + 1) * D], p, theta)
            s = keys @ qr / np.sqrt(D)
            w = np.exp(s - s.max())
            w /= w.sum()
            vals = np.abs(oracle.bf16_value(vc_after[b, g, :p + 1]))
            tol[b, h * D:(h + 1) * D] = 2 * U * (28 * E.max() + 8 * n_sub + 136) * (w @ vals) + 1e-30
    return tol
