"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes a property the KDA recurrence must have (a hand-worked example,
a brute-force product form, closed forms of special cases, invariants), chosen
so that a plausible slip in the oracle -- a dropped term, a wrong sign, the
gate on the wrong axis, the read-out before the update, a transposed operand --
fails at least one of them.  The recurrence pinned here:

    S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t

(gated delta rule with a channel-wise forget gate: Kimi K3 technical-report
page, "Architecture at a glance" and FAQ; architecture blog, "Kimi Delta
Attention: the linear core").
"""
import json
import os

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = datagen.DT_F32


def rel_err(x, y):
    """max |x - y| / max |y| (0/0 = 0)."""
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    den = np.abs(y).max() if y.size else 0.0
    num = np.abs(x - y).max() if y.size else 0.0
    return 0.0 if num == 0 else num / (den if den > 0 else 1.0)


def f64(a):
    return datagen.to_f64(a)


def inputs(seed, B, T, H, dk, dv, h0_std=0.02):
    return datagen.prefill_inputs(seed, B, T, H, dk, dv, F32, h0_std)


def run(d, h0="same", **kw):
    return oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"] if h0 == "same" else h0, **kw)


# --------------------------------------------------------------------------------------------
# Worked example by hand (tests/golden/worked_example_3tok.json)


def test_golden_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_3tok.json")))
    f = lambda key, shape: np.asarray(ex[key], np.float32).reshape(shape)
    q, k, v, g = f("q", (1, 3, 1, 2)), f("k", (1, 3, 1, 2)), f("v", (1, 3, 1, 2)), f("g", (1, 3, 1, 2))
    beta = f("beta", (1, 3, 1))
    h0 = f("h0", (1, 1, 2, 2))
    o, hT = oracle.forward(q, k, v, g, beta, h0)
    tol = ex["tolerance"]
    assert np.abs(o[0, :, 0, :] - np.asarray(ex["expected_o"])).max() < tol
    assert np.abs(hT[0, 0] - np.asarray(ex["expected_hT"])).max() < tol


# --------------------------------------------------------------------------------------------
# P1: brute-force unrolled product form, T <= 16


def brute_force(q, k, v, g, beta, h0):
    """S_t = Phi(t,0) S_0 + sum_{j<=t} Phi(t,j) beta_j k_j v_j^T with
    Phi(t,j) = M_t ... M_{j+1}, M_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)); o_t = S_t^T q_t.
    One (sequence, head): q, k, g [T, dk]; v [T, dv]; beta [T]; h0 [dk, dv]."""
    T, dk = q.shape
    I = np.eye(dk)
    M = [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]

    def phi(t, j):  # product M_t ... M_{j+1}
        P = I.copy()
        for s in range(j + 1, t + 1):
            P = M[s] @ P
        return P

    o = np.zeros((T, v.shape[1]))
    S = None
    for t in range(T):
        S = phi(t, -1) @ h0
        for j in range(t + 1):
            S = S + phi(t, j) @ (beta[j] * np.outer(k[j], v[j]))
        o[t] = S.T @ q[t]
    return o, S


@pytest.mark.parametrize("T,dk,dv", [(1, 4, 3), (7, 8, 5), (16, 16, 16), (12, 5, 9)])
def test_p1_brute_force_product_form(T, dk, dv):
    d = inputs(11 + T, 2, T, 2, dk, dv)
    o, hT = run(d)
    for b in range(2):
        for h in range(2):
            ob, Sb = brute_force(f64(d["q"][b, :, h]), f64(d["k"][b, :, h]), f64(d["v"][b, :, h]),
                                 f64(d["g"][b, :, h]), f64(d["beta"][b, :, h]), f64(d["h0"][b, h]))
            assert rel_err(o[b, :, h], ob) < 1e-12
            assert rel_err(hT[b, h], Sb) < 1e-12


# --------------------------------------------------------------------------------------------
# P2: beta = 0, g = 0 -> nothing is written and nothing decays: S_t = h0, o_t = h0^T q_t


def test_p2_frozen_state():
    d = inputs(21, 1, 40, 3, 16, 12)
    d["beta"][:] = 0
    d["g"][:] = 0
    o, hT = run(d)
    h0 = f64(d["h0"])
    assert np.array_equal(hT, h0)
    exp = np.einsum("bhcj,bthc->bthj", h0, f64(d["q"]))
    assert rel_err(o, exp) < 1e-14


# --------------------------------------------------------------------------------------------
# P3: orthonormal keys, g = 0, h0 = 0 -> beta-weighted cumulative linear attention, exactly


def hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_p3_orthogonal_keys_linear_attention():
    dk, dv, T = 16, 10, 16
    rng = np.random.default_rng(3)
    Hd = hadamard(dk) / 4.0  # rows orthonormal, entries +-1/4 (exact in fp32)
    keys = (Hd[rng.permutation(dk)] * rng.choice([-1.0, 1.0], size=(dk, 1)))[:T]
    d = inputs(31, 1, T, 1, dk, dv, h0_std=None)
    d["k"][0, :, 0] = keys.astype(np.float32)
    d["g"][:] = 0
    o, hT = run(d)
    q, k, v, be = f64(d["q"][0, :, 0]), f64(d["k"][0, :, 0]), f64(d["v"][0, :, 0]), f64(d["beta"][0, :, 0])
    exp = np.array([sum(be[j] * (q[t] @ k[j]) * v[j] for j in range(t + 1)) for t in range(T)])
    assert rel_err(o[0, :, 0], exp) < 1e-14
    assert rel_err(hT[0, 0], sum(be[j] * np.outer(k[j], v[j]) for j in range(T))) < 1e-14


# --------------------------------------------------------------------------------------------
# P4: beta = eps * b, g = 0, h0 = 0 -> o / eps tends to sum_{j<=t} b_j (q_t . k_j) v_j, error O(eps)


def test_p4_small_beta_limit():
    dk, dv, T = 16, 8, 24
    d = inputs(41, 1, T, 1, dk, dv, h0_std=None)
    d["g"][:] = 0
    b = f64(d["beta"][0, :, 0])
    q, k, v = f64(d["q"][0, :, 0]), f64(d["k"][0, :, 0]), f64(d["v"][0, :, 0])
    lin = np.array([sum(b[j] * (q[t] @ k[j]) * v[j] for j in range(t + 1)) for t in range(T)])
    errs = []
    for eps in (1e-3, 1e-4, 1e-5):
        d2 = dict(d)
        d2["beta"] = (d["beta"].astype(np.float64) * eps).astype(np.float32)
        beps = f64(d2["beta"][0, :, 0])
        lin_eps = np.array([sum(beps[j] * (q[t] @ k[j]) * v[j] for j in range(t + 1)) for t in range(T)])
        o, _ = run(d2)
        errs.append(rel_err(o[0, :, 0], lin_eps))
    assert errs[0] < 1e-1 and errs[2] < 1e-4
    # first order: the error shrinks in proportion to eps
    assert 5 < errs[0] / errs[1] < 20 and 5 < errs[1] / errs[2] < 20
    assert rel_err(lin, lin) == 0


# --------------------------------------------------------------------------------------------
# P5: g = 0, beta = 1, one-hot keys (with repeats), q = k -> exact key overwrite


def test_p5_exact_key_overwrite():
    dk, dv, T = 8, 6, 30
    rng = np.random.default_rng(5)
    d = inputs(51, 1, T, 1, dk, dv)
    keys = rng.integers(0, dk - 2, size=T)  # the last two rows are never written
    d["k"][:] = 0
    d["k"][0, np.arange(T), 0, keys] = 1
    d["q"][:] = d["k"]
    d["g"][:] = 0
    d["beta"][:] = 1
    o, hT = run(d)
    v = f64(d["v"][0, :, 0])
    assert np.array_equal(o[0, :, 0], v)
    exp = f64(d["h0"][0, 0]).copy()
    for t in range(T):
        exp[keys[t]] = v[t]
    assert np.array_equal(hT[0, 0], exp)


# --------------------------------------------------------------------------------------------
# P6: fixed one-hot key e_c, constant gate, beta and v -> geometric sum on row c
#     x_t = r x_{t-1} + beta v, r = alpha_c (1 - beta); other rows decay as alpha^t


def test_p6_geometric_sum():
    dk, dv, T, c = 8, 5, 50, 3
    d = inputs(61, 1, T, 1, dk, dv)
    g_row = d["g"][0, 0, 0].copy()
    d["g"][:] = g_row
    d["k"][:] = 0
    d["k"][0, :, 0, c] = 1
    d["beta"][:] = d["beta"][0, 0, 0]
    d["v"][:] = d["v"][0, 0, 0]
    o, hT = run(d)
    alpha = np.exp(f64(g_row))
    be, v, S0 = float(f64(d["beta"][0, 0, 0])), f64(d["v"][0, 0, 0]), f64(d["h0"][0, 0])
    r = alpha[c] * (1 - be)
    q = f64(d["q"][0, :, 0])
    for t in range(1, T + 1):
        S = alpha[:, None] ** t * S0
        S[c] = r ** t * S0[c] + be * v * (1 - r ** t) / (1 - r)
        assert rel_err(o[0, t - 1, 0], S.T @ q[t - 1]) < 1e-13
    assert rel_err(hT[0, 0], S) < 1e-13


# --------------------------------------------------------------------------------------------
# P7: beta = 0 -> decay only: S_t = Diag(exp(G_t)) h0, G_t = sum_{s<=t} g_s; o_t = h0^T (exp(G_t) * q_t)


def test_p7_decay_only_product():
    d = inputs(71, 2, 64, 2, 16, 8)
    d["beta"][:] = 0
    o, hT = run(d)
    G = np.cumsum(f64(d["g"]), axis=1)
    h0 = f64(d["h0"])
    exp_o = np.einsum("bhcj,bthc->bthj", h0, np.exp(G) * f64(d["q"]))
    assert rel_err(o, exp_o) < 1e-13
    assert rel_err(hT, np.exp(G[:, -1])[..., None] * h0) < 1e-13


# --------------------------------------------------------------------------------------------
# P9: continuation -- two calls with hT -> h0 equal one call (exact in fp64)


def test_p9_continuation():
    d = inputs(91, 2, 96, 2, 16, 8)
    o, hT = run(d)
    first = {key: d[key][:, :40] for key in ("q", "k", "v", "g", "beta")}
    second = {key: d[key][:, 40:] for key in ("q", "k", "v", "g", "beta")}
    o1, h1 = oracle.forward(**first, h0=d["h0"])
    o2, h2 = oracle.forward(**second, h0=h1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(h2, hT)


# --------------------------------------------------------------------------------------------
# P10: the map (h0, V) -> (o, hT) is linear: out(h0, V) = out(h0, 0) + out(0, V)


def test_p10_linearity():
    d = inputs(101, 1, 80, 2, 16, 8)
    o, hT = run(d)
    dz = dict(d)
    dz["v"] = np.zeros_like(d["v"])
    oa, ha = run(dz)
    ob, hb = run(d, h0=None)
    assert rel_err(oa + ob, o) < 1e-13
    assert rel_err(ha + hb, hT) < 1e-13


# --------------------------------------------------------------------------------------------
# P11: value columns evolve independently: permuting columns of v and h0 permutes o and hT


def test_p11_column_independence():
    d = inputs(111, 1, 50, 2, 16, 12)
    o, hT = run(d)
    perm = np.random.default_rng(11).permutation(12)
    dp = dict(d)
    dp["v"] = np.ascontiguousarray(d["v"][..., perm])
    dp["h0"] = np.ascontiguousarray(d["h0"][..., perm])
    op, hp = run(dp)
    assert np.array_equal(op, o[..., perm])
    assert np.array_equal(hp, hT[..., perm])
    # and a slice of columns alone gives the same columns
    ds = dict(d)
    ds["v"] = np.ascontiguousarray(d["v"][..., 4:8])
    ds["h0"] = np.ascontiguousarray(d["h0"][..., 4:8])
    os_, hs = run(ds)
    assert np.array_equal(os_, o[..., 4:8]) and np.array_equal(hs, hT[..., 4:8])


# --------------------------------------------------------------------------------------------
# P15: a segment is an affine map of its initial state.  Run from the identity on d_k columns
# with zero values it gives M (and the per-token read-out of M); run from zero it gives b; then
# from any S: hT = M S + b and o = o(0) + o_M S.  The segment-parallel chain rests on this.


def test_p15_segment_affine_map():
    d = inputs(151, 1, 70, 2, 16, 8)
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    eye = np.broadcast_to(np.eye(dk), (B, H, dk, dk)).copy()
    di = dict(d)
    di["v"] = np.zeros((B, T, H, dk), d["v"].dtype)
    di["h0"] = eye
    o_M, M = run(di)
    o_0, b = run(d, h0=None)
    S = np.random.default_rng(15).standard_normal((B, H, dk, dv))
    dS = dict(d)
    dS["h0"] = S
    o_S, h_S = run(dS)
    assert rel_err(np.einsum("bhij,bhjk->bhik", M, S) + b, h_S) < 1e-12
    assert rel_err(o_0 + np.einsum("bthj,bhjk->bthk", o_M, S), o_S) < 1e-12


# --------------------------------------------------------------------------------------------
# P16: the fused forms (gate from its pre-activation, normalised q and k, output gate) reduce to
# the plain recurrence where their definitions fix the values exactly, and agree with the input
# generator's own transforms (independent code) up to the rounding of its stored inputs


def test_p16_fused_gate_special_values():
    d = inputs(161, 1, 60, 2, 16, 8)
    B, T, H, dk = d["q"].shape
    # sigmoid(0) = 1/2: g = -A/2 exactly
    x0 = np.zeros((B, T, H, dk), np.float32)
    o_f, h_f = oracle.forward_fused(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], x=x0, gate_scale=5.0)
    o_p, h_p = oracle.forward(d["q"], d["k"], d["v"], np.full((B, T, H, dk), -2.5, np.float32), d["beta"], d["h0"])
    assert rel_err(o_f, o_p) == 0.0 and rel_err(h_f, h_p) == 0.0
    # a very negative pre-activation: the decay is 1 in fp64
    xm = np.full((B, T, H, dk), -60.0, np.float32)
    o_f, _ = oracle.forward_fused(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], x=xm, gate_scale=5.0)
    o_p, _ = oracle.forward(d["q"], d["k"], d["v"], np.zeros((B, T, H, dk), np.float32), d["beta"], d["h0"])
    assert rel_err(o_f, o_p) == 0.0


def test_p16_fused_normalisation_and_output_gate():
    d = inputs(162, 1, 50, 2, 16, 8)
    raw = datagen.prefill_preactivations(162, 1, 50, 2, 16, 8, F32, 0.02)
    # normalisation is scale-free
    o1, h1 = oracle.forward_fused(raw["q"], raw["k"], d["v"], d["g"], d["beta"], d["h0"], normalize_qk=True)
    o4, h4 = oracle.forward_fused(4 * raw["q"], 4 * raw["k"], d["v"], d["g"], d["beta"], d["h0"], normalize_qk=True)
    assert rel_err(o4, o1) < 1e-12 and rel_err(h4, h1) < 1e-12
    # the output gate multiplies o only
    o_p, h_p = run(d)
    o_z, h_z = oracle.forward_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], z=2 * np.ones_like(d["v"]))
    assert rel_err(o_z, 2 * o_p) == 0.0 and rel_err(h_z, h_p) == 0.0
    o_z, _ = oracle.forward_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], z=raw["z"])
    assert rel_err(o_z, o_p * raw["z"].astype(np.float64)) == 0.0


def test_p16_fused_matches_the_generators_transforms():
    """prefill_inputs stores normalise(q), normalise(k) and -5 sigmoid(x) rounded to fp32; the fused
    oracle applies the same definitions to the unrounded draws."""
    raw = datagen.prefill_preactivations(163, 2, 40, 2, 16, 8, F32, 0.02)
    plain = datagen.prefill_inputs(163, 2, 40, 2, 16, 8, F32, 0.02)
    assert np.array_equal(raw["v"], plain["v"]) and np.array_equal(raw["beta"], plain["beta"])
    o_f, h_f = oracle.forward_fused(raw["q"], raw["k"], raw["v"], None, raw["beta"], raw["h0"], x=raw["x"],
                                    gate_scale=5.0, normalize_qk=True)
    o_p, h_p = run(plain)
    assert rel_err(o_f, o_p) < 1e-5 and rel_err(h_f, h_p) < 1e-5


def test_p16_fused_decode_is_one_token_prefill():
    raw = datagen.decode_preactivations(164, 0, 2, 3, 16, 8, F32)
    state = datagen.decode_state0(164, 2, 3, 16, 8).astype(np.float64)
    h0 = state.copy()
    o_d = oracle.decode_step_fused(raw["q"], raw["k"], raw["v"], None, raw["beta"], state, x=raw["x"],
                                   gate_scale=5.0, normalize_qk=True, z=raw["z"])
    one = {key: raw[key][:, None] for key in ("q", "k", "v", "x", "beta", "z")}
    o_p, h_p = oracle.forward_fused(one["q"], one["k"], one["v"], None, one["beta"], h0, x=one["x"], gate_scale=5.0,
                                    normalize_qk=True, z=one["z"])
    assert rel_err(o_d, o_p[:, 0]) < 1e-14 and rel_err(state, h_p) < 1e-14


def test_p16_fused_varlen_is_independent_fused_calls():
    lens = [5, 0, 13, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    raw = datagen.prefill_preactivations(165, 1, int(cu[-1]), 2, 16, 8, F32, None)
    h0 = datagen.fill(165, datagen.TID_H0, 0, 0, 0.02, F32, (len(lens), 2, 16, 8), 8)
    o, hT = oracle.forward_varlen_fused(raw["q"], raw["k"], raw["v"], None, raw["beta"], cu, h0, x=raw["x"],
                                        gate_scale=4.0, normalize_qk=True, z=raw["z"])
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        part = {key: np.ascontiguousarray(raw[key][:, s:e]) for key in ("q", "k", "v", "x", "beta", "z")}
        o_n, h_n = oracle.forward_fused(part["q"], part["k"], part["v"], None, part["beta"], h0[n:n + 1],
                                        x=part["x"], gate_scale=4.0, normalize_qk=True, z=part["z"])
        assert rel_err(o[s:e], o_n[0]) < 1e-14 and rel_err(hT[n:n + 1], h_n) < 1e-14


# --------------------------------------------------------------------------------------------
# P12: T single-token decode steps equal one prefill of T tokens


def test_p12_decode_equals_prefill():
    B, T, H, dk, dv = 2, 20, 3, 16, 8
    d = inputs(121, B, T, H, dk, dv)
    o, hT = run(d)
    state = f64(d["h0"]).copy()
    for t in range(T):
        ot = oracle.decode_step(d["q"][:, t], d["k"][:, t], d["v"][:, t], d["g"][:, t], d["beta"][:, t], state)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(state, hT)


# --------------------------------------------------------------------------------------------
# P13: packed varlen equals independent per-sequence calls; nothing crosses a boundary


def test_p13_varlen_independent_sequences():
    lens = [5, 0, 17, 64, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt, H, dk, dv = int(cu[-1]), 2, 16, 8
    d = inputs(131, 1, Tt, H, dk, dv, h0_std=None)
    h0 = datagen.fill(131, datagen.TID_H0, 0, 0, 0.02, F32, (len(lens), H, dk, dv), dv)
    o, hT = oracle.forward_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, h0)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, hn = oracle.forward(*(d[key][:, s:e] for key in ("q", "k", "v", "g", "beta")), h0=h0[n:n + 1])
        assert np.array_equal(o[s:e], on[0])
        assert np.array_equal(hT[n], hn[0])
    assert np.array_equal(hT[1], f64(h0[1]))  # empty sequence: hT = h0


# --------------------------------------------------------------------------------------------
# P14: contraction -- ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t|| when ||k|| = 1, beta in [0,1], alpha <= 1


def test_p14_norm_bound():
    B, T, H, dk, dv = 1, 300, 2, 32, 16
    d = inputs(141, B, T, H, dk, dv)
    state = f64(d["h0"]).copy()
    prev = np.linalg.norm(state, axis=(2, 3))
    for t in range(T):
        oracle.decode_step(d["q"][:, t], d["k"][:, t], d["v"][:, t], d["g"][:, t], d["beta"][:, t], state)
        now = np.linalg.norm(state, axis=(2, 3))
        bound = prev + f64(d["beta"][:, t]) * np.linalg.norm(f64(d["v"][:, t]), axis=-1)
        # keys are unit-norm only to fp32 rounding, hence the 1e-6 slack
        assert np.all(now <= bound * (1 + 1e-6))
        prev = now


# --------------------------------------------------------------------------------------------
# Edge cases: T = 0 (hT = h0), bf16 inputs decode exactly


def test_empty_sequence():
    d = inputs(151, 2, 0, 2, 8, 4)
    o, hT = run(d)
    assert o.shape == (2, 0, 2, 4)
    assert np.array_equal(hT, f64(d["h0"]))
    o, hT = run(d, h0=None)
    assert np.array_equal(hT, np.zeros_like(hT))


def test_bf16_inputs_decode_exactly():
    d32 = datagen.prefill_inputs(161, 1, 20, 2, 16, 8, datagen.DT_BF16, 0.02)
    dd = {key: (datagen.bf16_bits_to_f32(val) if key != "h0" else val) for key, val in d32.items()}
    o1, h1 = run(d32)
    o2, h2 = run(dd)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


# --------------------------------------------------------------------------------------------
# forward_units: the batched forward restricted to chosen (b, h) units, unit id = b * H + h.  Every
# unit runs the same token-by-token code as forward(), so a selected unit's o and hT must equal the
# batched call's slice bit for bit; a slip in the unit index (b and h swapped, id taken as h * B + b)
# or in the output stride fails this, because every unit sees different inputs and a different h0.


def test_forward_units_equals_batched_slices():
    B, T, H, dk, dv = 3, 37, 5, 16, 8
    d = inputs(171, B, T, H, dk, dv)
    o, hT = run(d)
    ids = [14, 0, 7, 7, 3, 11, 5]  # permuted, repeated, first and last unit, b and h both vary
    ou, hu = oracle.forward_units(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], ids)
    assert ou.shape == (len(ids), T, dv) and hu.shape == (len(ids), dk, dv)
    for i, uid in enumerate(ids):
        b, h = divmod(uid, H)
        assert np.array_equal(ou[i], o[b, :, h]), uid
        assert np.array_equal(hu[i], hT[b, h]), uid
    # without h0, and with only one of the outputs wanted
    o0, h00 = run(d, h0=None)
    _, hu0 = oracle.forward_units(d["q"], d["k"], d["v"], d["g"], d["beta"], None, ids, want_o=False)
    ou0, _ = oracle.forward_units(d["q"], d["k"], d["v"], d["g"], d["beta"], None, ids, want_hT=False)
    for i, uid in enumerate(ids):
        b, h = divmod(uid, H)
        assert np.array_equal(hu0[i], h00[b, h]) and np.array_equal(ou0[i], o0[b, :, h])
    with pytest.raises(RuntimeError):
        oracle.forward_units(d["q"], d["k"], d["v"], d["g"], d["beta"], None, [B * H])
