"""P8: the chunkwise (UT/WY) form of the gated delta rule equals the token-by-token
recurrence, checked with an fp64 numpy mirror against the oracle.

The chunked form is what the HIP kernels compute (the pages' "chunkwise
algorithm built on a specialised variant of diagonal-plus-low-rank transition
matrices": architecture blog, "Kimi Delta Attention: the linear core"; bounded
log-decay making every causal tile a dense matrix product: technical-report
page, "Architecture at a glance").  Derivation, for one chunk of C tokens
starting from state S0, with G the chunk-local inclusive cumulative sum of g
and Gamma = exp(G):

    A[r,i] = beta_r * sum_c k_r[c] k_i[c] exp(G_r[c] - G_i[c])      (i < r; 0 otherwise)
    T      = (I + A)^{-1} diag(beta)
    W      = T (K * Gamma),   U~ = T V,   U = U~ - W S0
    P[r,i] = sum_c q_r[c] k_i[c] exp(G_r[c] - G_i[c])                (i <= r)
    O      = (Q * Gamma) S0 + P U
    S_C    = Diag(Gamma_last) S0 + (K * exp(G_last - G))^T U

The second mirror evaluates the exponent differences the way the kernels do:
per 16-row sub-tile of rows, against the cumulative sum just before that
sub-tile, so every factor stays finite in fp32 for g >= -5.
"""
import numpy as np
import pytest

import datagen
import oracle


def chunk_mirror(q, k, v, g, beta, S0, C, subtile=None):
    """One (sequence, head) in fp64: q, k, g [T, dk]; v [T, dv]; beta [T]; S0 [dk, dv]."""
    T = q.shape[0]
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, Gl, b = q[s:e], k[s:e], v[s:e], np.cumsum(g[s:e], axis=0), beta[s:e]
        n = e - s
        if subtile is None:
            D = Gl[:, None, :] - Gl[None, :, :]          # [r, i, c] = G_r - G_i
            Ekk = np.einsum("rc,ic,ric->ri", K, K, np.exp(np.where(D <= 0, D, 0)))
            Eqk = np.einsum("rc,ic,ric->ri", Q, K, np.exp(np.where(D <= 0, D, 0)))
        else:
            Ekk, Eqk = subtile_products(Q, K, Gl, subtile)
        A = np.tril(b[:, None] * Ekk, -1)
        Tm = np.linalg.solve(np.eye(n) + A, np.diag(b))
        Gam = np.exp(Gl)
        W = Tm @ (K * Gam)
        Ut = Tm @ V
        U = Ut - W @ S
        P = np.tril(Eqk)
        o[s:e] = (Q * Gam) @ S + P @ U
        S = np.exp(Gl[-1])[:, None] * S + (K * np.exp(Gl[-1] - Gl)).T @ U
    return o, S


def subtile_products(Q, K, G, L=16, dtype=np.float64):
    """Lower-triangular M_xk[r,i] = sum_c x_r[c] k_i[c] exp(G_r[c] - G_i[c]) for x in (k, q),
    factorised per L-row sub-tile b with reference R_b = G just before the sub-tile (0 for the first):
    rows scaled by exp(G_r - R_b) in [exp(-5L), 1], columns i <= end of b by exp(R_b - G_i)."""
    n, dk = K.shape
    Mkk = np.zeros((n, n))
    Mqk = np.zeros((n, n))
    for r0 in range(0, n, L):
        r1 = min(r0 + L, n)
        R = G[r0 - 1] if r0 > 0 else np.zeros(dk)
        row = np.exp((G[r0:r1] - R).astype(dtype))
        col = np.exp((R - G[:r1]).astype(dtype))
        assert np.all(np.isfinite(row)) and np.all(np.isfinite(col))
        Kc = (K[:r1] * col).astype(dtype)
        Mkk[r0:r1, :r1] = ((K[r0:r1] * row).astype(dtype) @ Kc.T)
        Mqk[r0:r1, :r1] = ((Q[r0:r1] * row).astype(dtype) @ Kc.T)
    return Mkk, Mqk


def rel(x, y):
    return np.abs(x - y).max() / np.abs(y).max()


@pytest.mark.parametrize("C", [1, 2, 16, 64, 100])
@pytest.mark.parametrize("subtile", [None, 16])
def test_p8_chunked_equals_recurrence(C, subtile):
    if subtile and C < 16:
        pytest.skip("sub-tiles apply to chunks of 16 or more")
    T, dk, dv = 256, 32, 16
    d = datagen.prefill_inputs(801, 1, T, 2, dk, dv, datagen.DT_F32, 0.02)
    o, hT = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    f = datagen.to_f64
    for h in range(2):
        om, Sm = chunk_mirror(f(d["q"][0, :, h]), f(d["k"][0, :, h]), f(d["v"][0, :, h]), f(d["g"][0, :, h]),
                              f(d["beta"][0, :, h]), f(d["h0"][0, h]), C, subtile)
        assert rel(om, o[0, :, h]) < 1e-12
        assert rel(Sm, hT[0, h]) < 1e-12


def test_subtile_factors_finite_in_fp32_at_the_decay_bound():
    """At g = -5 everywhere a 64-row tile spans 320 in log space: exp(G_r - G_i) over a whole chunk
    overflows fp32, the per-sub-tile factors do not."""
    n, dk = 64, 8
    rng = np.random.default_rng(0)
    K = rng.standard_normal((n, dk))
    G = np.cumsum(np.full((n, dk), -5.0), axis=0)
    with np.errstate(over="ignore"):
        assert not np.all(np.isfinite(np.exp((-G).astype(np.float32))))
    Mkk32, _ = subtile_products(K, K, G, 16, np.float32)
    Mkk64, _ = subtile_products(K, K, G, 16, np.float64)
    low = np.tril(np.ones((n, n), bool))
    assert np.all(np.isfinite(Mkk32[low]))
    D = G[:, None, :] - G[None, :, :]
    exact = np.einsum("rc,ic,ric->ri", K, K, np.exp(np.where(D <= 0, D, -np.inf)))
    assert np.abs(Mkk32[low] - exact[low]).max() < 1e-5 * np.abs(exact).max()
    assert np.abs(Mkk64[low] - exact[low]).max() < 1e-12 * np.abs(exact).max()
