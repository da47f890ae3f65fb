"""The chunkwise backward that the HIP kernels compute equals the oracle's reverse-mode
gradients (fp64 numpy mirror, no GPU).

The pages give no backward (training with KDA: technical-report page, "Training");
it is the chain rule through the chunkwise (UT/WY) form of the forward, for one chunk
of C tokens from state S0 (G the chunk-local inclusive cumulative sum of g, Gamma =
exp(G), gl = G of the last row):

  forward:   A = strictLower(beta_r Ekk),  L = (I + A)^{-1},  T = L diag(beta)
             W = T (K Gamma),  U~ = T V,  U = U~ - W S0,  P = lowerIncl(Eqk)
             O = (Q Gamma) S0 + P U,   S1 = Diag(exp(gl)) S0 + Kd^T U,  Kd = K exp(gl - G)
  adjoint chain (the only sequential part; it needs no forward state):
             dU = P^T dO + Kd dS1,   dS0 = (Q Gamma)^T dO + Diag(exp(gl)) dS1 - W^T dU
  per chunk, given S0 and dS1 (the adjoint of the state at the chunk's end):
    state products:  dP = lowerIncl(dO U^T),  dQG = dO S0^T,  dKd = U dS1^T,  dW = -dU S0^T,
                     dgl = exp(gl) rowsum(S0 . dS1)
    transform:       dT = dW (K Gamma)^T + dU V^T;  dKG = T^T dW;  dV = T^T dU
                     dL = dT diag(beta);  dbeta_i = sum_r dT[r,i] L[r,i]
                     dA = strictLower(-L^T dL L^T);  dbeta_r += sum_i dA[r,i] Ekk[r,i];  dEkk = beta_r dA
                     through Ekk, Eqk (one term exp(G_r - G_i) per (r, i, c)) into dQ, dK, dG;
                     elementwise through Q Gamma, K Gamma, Kd, exp(gl);  dg = reverse cumsum of dG.
"""
import numpy as np
import pytest

import oracle


def rnd(seed, T, dk, dv):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=r.standard_normal((T, dv)), g=-5.0 / (1.0 + np.exp(-r.standard_normal((T, dk)))),
                beta=1.0 / (1.0 + np.exp(-r.standard_normal(T))), h0=0.3 * r.standard_normal((dk, dv)),
                do=r.standard_normal((T, dv)), dhT=r.standard_normal((dk, dv)))


def chunk_parts(Q, K, V, g, b):
    n = Q.shape[0]
    G = np.cumsum(g, axis=0)
    D = G[:, None, :] - G[None, :, :]                     # [r, i, c] = G_r - G_i
    E = np.exp(np.where(D <= 0, D, 0.0)) * np.tril(np.ones((n, n)))[:, :, None]
    Ekk = np.einsum("rc,ic,ric->ri", K, K, E)
    Eqk = np.einsum("rc,ic,ric->ri", Q, K, E)
    A = np.tril(b[:, None] * Ekk, -1)
    L = np.linalg.inv(np.eye(n) + A)
    Gam = np.exp(G)
    gl = G[-1]
    return dict(G=G, E=E, Ekk=Ekk, Eqk=Eqk, L=L, T=L * b[None, :], Gam=Gam, gl=gl, KG=K * Gam,
                Kd=K * np.exp(gl - G), P=np.tril(Eqk))


def mirror_backward(d, C):
    q, k, v, g, beta = d["q"], d["k"], d["v"], d["g"], d["beta"]
    T = q.shape[0]
    starts = list(range(0, T, C))
    # forward: records and the state at every chunk start
    S = d["h0"].copy()
    S0s, parts = [], []
    for s in starts:
        e = min(s + C, T)
        p = chunk_parts(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e])
        W, Ut = p["T"] @ p["KG"], p["T"] @ v[s:e]
        S0s.append(S.copy())
        U = Ut - W @ S
        S = np.exp(p["gl"])[:, None] * S + p["Kd"].T @ U
        p.update(W=W, Ut=Ut)
        parts.append(p)
    # adjoint chain: the adjoint of the state at every chunk end
    dS = d["dhT"].copy()
    dS1s = [None] * len(starts)
    for n in range(len(starts) - 1, -1, -1):
        s, e = starts[n], min(starts[n] + C, T)
        p, dO = parts[n], d["do"][s:e]
        dS1s[n] = dS.copy()
        dU = p["P"].T @ dO + p["Kd"] @ dS
        dS = (q[s:e] * p["Gam"]).T @ dO + np.exp(p["gl"])[:, None] * dS - p["W"].T @ dU
    dh0 = dS
    # per chunk, independently
    out = {x: np.zeros_like(d[x]) for x in ("q", "k", "v", "g", "beta")}
    for n, s in enumerate(starts):
        e = min(s + C, T)
        p, S0, dS1, dO = parts[n], S0s[n], dS1s[n], d["do"][s:e]
        Q, K, V, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        U = p["Ut"] - p["W"] @ S0
        dU = p["P"].T @ dO + p["Kd"] @ dS1
        dP = np.tril(dO @ U.T)
        dQG, dKd, dW = dO @ S0.T, U @ dS1.T, -dU @ S0.T
        dgl = np.exp(p["gl"]) * (S0 * dS1).sum(axis=1)
        dT = np.tril(dW @ p["KG"].T + dU @ V.T)
        dKG, dV = p["T"].T @ dW, p["T"].T @ dU
        dL = dT * b[None, :]
        db = (dT * p["L"]).sum(axis=0)
        dA = np.tril(-p["L"].T @ dL @ p["L"].T, -1)
        db += (dA * p["Ekk"]).sum(axis=1)
        dEkk, dEqk = b[:, None] * dA, dP
        E = p["E"]
        dQ = np.einsum("ri,ic,ric->rc", dEqk, K, E)
        dK = np.einsum("ri,ic,ric->rc", dEkk, K, E) + np.einsum("ri,rc,ric->ic", dEqk, Q, E) \
            + np.einsum("ri,rc,ric->ic", dEkk, K, E)
        tq = np.einsum("ri,rc,ic,ric->ric", dEqk, Q, K, E) + np.einsum("ri,rc,ic,ric->ric", dEkk, K, K, E)
        dG = tq.sum(axis=1) - tq.sum(axis=0)
        dQ += dQG * p["Gam"]
        dG += dQG * Q * p["Gam"]
        dK += dKG * p["Gam"]
        dG += dKG * p["KG"]
        dK += dKd * np.exp(p["gl"] - p["G"])
        dG -= dKd * p["Kd"]
        dgl = dgl + (dKd * p["Kd"]).sum(axis=0)
        dG[-1] += dgl
        out["q"][s:e], out["k"][s:e], out["v"][s:e], out["beta"][s:e] = dQ, dK, dV, db
        out["g"][s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
    return out, dh0


@pytest.mark.parametrize("T,C", [(100, 16), (130, 64), (64, 64), (37, 32), (5, 64)])
def test_chunked_backward_equals_oracle(T, C):
    d = rnd(3000 + T + C, T, 12, 7)
    got, dh0 = mirror_backward(d, C)
    ref = oracle.backward(*(d[x][None, :, None] for x in ("q", "k", "v", "g")), d["beta"][None, :, None],
                          d["h0"][None, None], d["do"][None, :, None], d["dhT"][None, None])
    for name, r in zip(("q", "k", "v", "g", "beta"), ref[:5]):
        r = r[0, :, 0]
        err = np.abs(got[name] - r).max() / np.abs(r).max()
        assert err < 1e-11, (name, err)
    assert np.abs(dh0 - ref[5][0, 0]).max() < 1e-11 * np.abs(ref[5]).max()
