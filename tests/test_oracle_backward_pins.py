"""Pins of the oracle's backward (oracle.backward), the reverse-mode gradients of
L = <do, o> + <dhT, hT> through the plain recurrence.  The pages give no backward
(training with KDA: technical-report page, "Training"), so the gradients are
pinned to the forward oracle (already pinned) and to mathematics:

  P17  central finite differences of L, every element of every input, on a tiny case;
  P18  directional derivatives on a case long enough to cross the backward's
       checkpoint blocks (64 tokens), every input perturbed at once;
  P19  the adjoint identity: for fixed q, k, g, beta the map (h0, v) -> (o, hT) is
       linear, so L = <dh0, h0> + <dv, v> exactly;
  P20  beta = 0 closed forms: the state only decays, S_t = Diag(exp(G_t)) h0, so
       dq, dg, dbeta and dh0 are sums written out below and dk = dv = 0.

The last test plants slips in a copy of the backward's C source and checks a pin fails.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


def rnd(seed, B, T, H, dk, dv, h0=0.3):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=r.standard_normal((B, T, H, dv)), g=-5.0 / (1.0 + np.exp(-r.standard_normal((B, T, H, dk)))),
                beta=1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H)))),
                h0=h0 * r.standard_normal((B, H, dk, dv)), do=r.standard_normal((B, T, H, dv)),
                dhT=r.standard_normal((B, H, dk, dv)))


NAMES = ("q", "k", "v", "g", "beta", "h0")


def loss(d, **repl):
    x = dict(d, **repl)
    o, hT = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], nthreads=1)
    return float((o * x["do"]).sum() + (hT * x["dhT"]).sum())


def grads(d):
    dq, dk, dv, dg, db, dh0 = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["do"], d["dhT"])
    return dict(q=dq, k=dk, v=dv, g=dg, beta=db, h0=dh0)


def test_p17_finite_differences_every_element():
    d = rnd(1700, 1, 7, 2, 4, 3)
    gr = grads(d)
    eps = 1e-6
    for name in NAMES:
        fd = np.zeros_like(d[name])
        for idx in np.ndindex(d[name].shape):
            xp, xm = d[name].copy(), d[name].copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = (loss(d, **{name: xp}) - loss(d, **{name: xm})) / (2 * eps)
        err = np.abs(gr[name] - fd).max() / max(np.abs(fd).max(), 1e-30)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("T", [150, 64])
def test_p18_directional_derivatives(T):
    d = rnd(1800 + T, 2, T, 2, 16, 8)
    gr = grads(d)
    r = np.random.default_rng(T)
    dirs = {n: r.standard_normal(d[n].shape) for n in NAMES}
    dirs["g"] *= 0.1
    eps = 1e-5
    plus = loss(d, **{n: d[n] + eps * dirs[n] for n in NAMES})
    minus = loss(d, **{n: d[n] - eps * dirs[n] for n in NAMES})
    fd = (plus - minus) / (2 * eps)
    an = sum(float((gr[n] * dirs[n]).sum()) for n in NAMES)
    assert abs(fd - an) < 1e-6 * max(abs(an), 1.0), (fd, an)
    # each input's own directional derivative (a dropped term in one input's gradient cannot hide)
    for n in NAMES:
        p = loss(d, **{n: d[n] + eps * dirs[n]})
        m = loss(d, **{n: d[n] - eps * dirs[n]})
        fd_n, an_n = (p - m) / (2 * eps), float((gr[n] * dirs[n]).sum())
        assert abs(fd_n - an_n) < 1e-6 * max(abs(an_n), 1.0), (n, fd_n, an_n)


def test_p19_adjoint_identity_of_the_linear_part():
    d = rnd(1900, 2, 200, 3, 32, 16)
    gr = grads(d)
    lhs = loss(d)
    rhs = float((gr["h0"] * d["h0"]).sum() + (gr["v"] * d["v"]).sum())
    assert abs(lhs - rhs) < 1e-11 * max(abs(lhs), 1.0), (lhs, rhs)


def test_p20_beta_zero_closed_forms():
    d = rnd(2000, 1, 40, 2, 8, 5, h0=1.0)
    d["beta"] = np.zeros_like(d["beta"])
    gr = grads(d)
    q, k, v, G = d["q"][0], d["k"][0], d["v"][0], np.cumsum(d["g"][0], axis=0)  # [T, H, .]
    h0, do, dhT = d["h0"][0], d["do"][0], d["dhT"][0]
    T = q.shape[0]
    E = np.exp(G)                                                   # [T, H, dk]
    S = E[:, :, :, None] * h0[None]                                 # S_t [T, H, dk, dv]
    dq = np.einsum("thcj,thj->thc", S, do)
    h0do = np.einsum("hcj,thj->thc", h0, do)                        # (h0 do_t)[c]
    contrib = E * q * h0do                                          # d/dG_t of o_t . do_t
    final = E[-1] * np.einsum("hcj,hcj->hc", dhT, h0)               # d/dG_T of <dhT, S_T>
    dg = np.cumsum(contrib[::-1], axis=0)[::-1] + final[None]
    dh0 = np.einsum("thc,thj->hcj", E * q, do) + E[-1][:, :, None] * dhT
    # adjoint of S_t, and dbeta_t = <k_t, dS_t (v_t - S'_t^T k_t)> with S'_t = S_t when beta = 0
    db = np.zeros((T, q.shape[1]))
    for t in range(T):
        dS = q[t][:, :, None] * do[t][:, None, :]
        for s in range(t + 1, T):
            dS += np.exp(G[s] - G[t])[:, :, None] * q[s][:, :, None] * do[s][:, None, :]
        dS += np.exp(G[-1] - G[t])[:, :, None] * dhT
        resid = v[t] - np.einsum("hcj,hc->hj", S[t], k[t])
        db[t] = np.einsum("hc,hcj,hj->h", k[t], dS, resid)
    for name, ref in (("q", dq), ("g", dg), ("h0", dh0), ("beta", db)):
        got = gr[name][0] if name != "h0" else gr["h0"][0]
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err < 1e-12, (name, err)
    assert np.abs(gr["k"]).max() == 0.0 and np.abs(gr["v"]).max() == 0.0


def test_backward_inputs_in_every_storage_dtype():
    """bf16 bits, fp32 and fp64 inputs of the same values give the same gradients."""
    d = rnd(2100, 1, 30, 2, 8, 4)
    bits = {n: (d[n].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for n in ("q", "k", "v", "g", "beta")}
    dec = {n: (bits[n].astype(np.uint32) << 16).view(np.float32) for n in bits}
    a = oracle.backward(*(bits[n] for n in ("q", "k", "v", "g", "beta")), d["h0"], d["do"], d["dhT"])
    b = oracle.backward(*(dec[n] for n in ("q", "k", "v", "g", "beta")), d["h0"], d["do"], d["dhT"])
    c = oracle.backward(*(dec[n].astype(np.float64) for n in ("q", "k", "v", "g", "beta")), d["h0"], d["do"],
                        d["dhT"])
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_backward_without_dhT_and_empty():
    d = rnd(2200, 1, 20, 1, 4, 4)
    a = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["do"], None)
    b = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["do"], np.zeros_like(d["dhT"]))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    e = rnd(2201, 1, 0, 2, 4, 4)
    dq, dk, dv, dg, db, dh0 = oracle.backward(e["q"], e["k"], e["v"], e["g"], e["beta"], e["h0"], e["do"], e["dhT"])
    assert dq.shape == (1, 0, 2, 4) and np.array_equal(dh0, e["dhT"])


# slips planted in the backward only (anchors are unique to it)
MUTANTS = {
    "dq_from_state_before_write": ("acc += Snew[(size_t)c * dv + j] * dO[j];", "acc += Sd[(size_t)c * dv + j] * dO[j];"),
    "readout_adjoint_dropped": ("dS[(size_t)c * dv + j] += qc * dO[j];", "(void)qc;"),
    "dp_sign": ("du[j] = -b * du[j]; /* now dp */", "du[j] = b * du[j]; /* now dp */"),
    "erase_adjoint_dropped": ("dS[(size_t)c * dv + j] += kc * du[j];\n", "(void)kc;\n"),
    "dg_against_undecayed": ("acc += dS[(size_t)c * dv + j] * Sd[(size_t)c * dv + j];",
                             "acc += dS[(size_t)c * dv + j] * Sd[(size_t)c * dv + j] / a;"),
    "state_adjoint_not_decayed": ("dS[(size_t)c * dv + j] *= a;\n        }\n        dg[c] = acc;",
                                  "dS[(size_t)c * dv + j] *= 1.0;\n        }\n        dg[c] = acc;"),
    "dbeta_residual_sign": ("db += du[j] * (vj - p[j]);", "db += du[j] * (vj + p[j]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not unique: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", str(src), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "_SRC", str(src))
    monkeypatch.setattr(oracle, "_lib", None)
    failed = []
    for pin in (lambda: test_p18_directional_derivatives(150), test_p19_adjoint_identity_of_the_linear_part,
                test_p20_beta_zero_closed_forms):
        try:
            pin()
        except AssertionError:
            failed.append(pin)
    monkeypatch.setattr(oracle, "_lib", None)
    assert failed, "no pin caught the planted mistake %r" % name
