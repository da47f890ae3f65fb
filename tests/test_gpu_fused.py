"""Parity of the fused entry points (kda_chunked_forward_fused, kda_decode_step_fused) with the
oracle's fused forms: the log-decay formed from its gate pre-activation, q and k L2-normalised,
and an output gate on o, all inside the kernels."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, o_err, state_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

F32, BF16 = datagen.DT_F32, datagen.DT_BF16
OPTS = {"all": (True, True, True), "gate": (True, False, False), "norm": (False, True, False),
        "out_gate": (False, False, True)}


def fused_case(d, chunk, dt, gate, norm, zg, label, scale=5.0):
    # without in-kernel normalisation the inputs are the unit-norm q, k (raw N(0,1) rows of length
    # 128 would make the delta-rule write expand the state)
    d = dict(d)
    if not norm:
        d["q"], d["k"] = d["q_unit"], d["k_unit"]
    dv = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "x", "beta", "z")}
    g = None if gate else dev_tensor(d["g"])
    o, hT = kda.kda_chunked_forward_fused(dv["q"], dv["k"], dv["v"], g, dv["beta"], dev_tensor(d["h0"]),
                                          gate_x=dv["x"] if gate else None, gate_scale=scale, normalize_qk=norm,
                                          out_gate=dv["z"] if zg else None, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_fused(d["q"], d["k"], d["v"], None if gate else d["g"], d["beta"], d["h0"],
                                        x=d["x"] if gate else None, gate_scale=scale, normalize_qk=norm,
                                        z=d["z"] if zg else None)
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("%s: o %.2e hT %.2e" % (label, eo, eh))
    assert eo < TOL[dt] and eh < TOL[dt], (eo, eh)
    return o, hT


def raw_inputs(seed, B, T, H, dk, dv, dt, h0=0.02):
    d = datagen.prefill_preactivations(seed, B, T, H, dk, dv, dt, h0)
    # the generator's transformed inputs for the cases that keep g or q, k as given
    plain = datagen.prefill_inputs(seed, B, T, H, dk, dv, dt, h0)
    d["g"], d["q_unit"], d["k_unit"] = plain["g"], plain["q"], plain["k"]
    return d


@pytest.mark.parametrize("opt", list(OPTS))
def test_fused_prefill_bf16(opt):
    d = raw_inputs(700, 2, 333, 3, 128, 128, BF16)
    fused_case(d, 64, BF16, *OPTS[opt], "fused bf16 %s" % opt)


@pytest.mark.parametrize("opt", ["all", "gate"])
def test_fused_prefill_fp32(opt):
    d = raw_inputs(701, 2, 150, 2, 64, 64, F32)
    fused_case(d, 32, F32, *OPTS[opt], "fused fp32 %s" % opt)


@pytest.mark.parametrize("dv", [64, 128])
def test_fused_fp32_chunk64_gate_read_at_stores(dv):
    """fp32, d_k = 64, chunk 64: the chain kernel's two record buffers leave no LDS for the output
    gate, so its chain waves read the gate from global memory at the stores (the other instances
    stream it through LDS with the records)."""
    d = raw_inputs(703 + dv, 2, 200, 2, 64, dv, F32)
    fused_case(d, 64, F32, *OPTS["all"], "fused fp32 chunk 64 dv=%d" % dv)


@pytest.mark.parametrize("dv", [64, 128])
def test_fused_fp32_dk128_chunk64(dv):
    """fp32, d_k = 128, chunk 64: one LDS record buffer in the chain kernel, the output gate
    streamed with it."""
    d = raw_inputs(705 + dv, 2, 150, 2, 128, dv, F32)
    fused_case(d, 64, F32, *OPTS["all"], "fused fp32 d_k 128 chunk 64 dv=%d" % dv)


@pytest.mark.parametrize("T", [1, 17, 100])
def test_fused_gate_ragged_chunks(T):
    """Rows past a partial chunk's end must keep a decay of 1 (their pre-activation loads as 0, and
    -A sigmoid(0) is not 0): the final state checks the chunk's total decay."""
    d = raw_inputs(702 + T, 1, T, 2, 128, 128, BF16)
    fused_case(d, 64, BF16, True, False, False, "fused ragged T=%d" % T, scale=3.0)


def test_fused_with_whole_state_slices():
    """A plan with whole 128-column states per workgroup (32 segments): two buffers of the output
    gate do not fit beside the records, so the chain waves read the gate from global memory."""
    assert kda.chain_plan(1, 65601, 4, 128, 128) == (64, 32, 33)
    assert kda.chain_plan(2, 65601, 4, 128, 128) == (128, 32, 33)
    d = raw_inputs(711, 2, 65601, 4, 128, 128, BF16)
    fused_case(d, 64, BF16, True, True, True, "fused, whole-state slices")


def test_fused_with_segmented_chain():
    assert kda.chain_plan(1, 8229, 2, 128, 128)[1] == 4
    d = raw_inputs(710, 1, 8229, 2, 128, 128, BF16)
    fused_case(d, 64, BF16, True, True, True, "fused segmented")


def test_fused_reproduces_the_generators_inputs():
    """Pre-activations through the fused call give what the plain call gives on the generator's
    transformed inputs (the same draws, transformed in fp64 and rounded once)."""
    raw = datagen.prefill_preactivations(720, 2, 300, 4, 128, 128, BF16, 0.02)
    plain = datagen.prefill_inputs(720, 2, 300, 4, 128, 128, BF16, 0.02)
    r = {key: dev_tensor(raw[key]) for key in ("q", "k", "v", "x", "beta")}
    p = {key: dev_tensor(plain[key]) for key in ("q", "k", "v", "g", "beta")}
    h0 = dev_tensor(plain["h0"])
    o_f, h_f = kda.kda_chunked_forward_fused(r["q"], r["k"], r["v"], None, r["beta"], h0, gate_x=r["x"],
                                             gate_scale=5.0, normalize_qk=True)
    o_p, h_p = kda.kda_chunked_forward(p["q"], p["k"], p["v"], p["g"], p["beta"], h0)
    torch.cuda.synchronize()
    assert o_err(host64(o_f), host64(o_p)) < TOL[BF16]
    assert state_err(host64(h_f), host64(h_p)) < TOL[BF16]


@pytest.mark.parametrize("dt,dk,dv", [(BF16, 128, 128), (BF16, 64, 128), (F32, 64, 64)])
def test_fused_decode(dt, dk, dv):
    B, H, steps = 4, 8, 3
    state = dev_tensor(datagen.decode_state0(730, B, H, dk, dv))
    ref = datagen.decode_state0(730, B, H, dk, dv).astype(np.float64)
    for s in range(steps):
        d = datagen.decode_preactivations(730, s, B, H, dk, dv, dt)
        t = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "x", "beta", "z")}
        o = kda.kda_decode_step_fused(t["q"], t["k"], t["v"], None, t["beta"], state, gate_x=t["x"], gate_scale=5.0,
                                      normalize_qk=True, out_gate=t["z"])
        torch.cuda.synchronize()
        o_ref = oracle.decode_step_fused(d["q"], d["k"], d["v"], None, d["beta"], ref, x=d["x"], gate_scale=5.0,
                                         normalize_qk=True, z=d["z"])
        eo = o_err(host64(o)[:, None], o_ref[:, None])
        assert eo < TOL[dt], (s, eo)
    assert state_err(host64(state), ref) < TOL[dt]


def test_snapshots_and_fused_steps_together():
    """kda_chunked_forward_ex: the fused steps and state snapshots in one call; each snapshot is the
    oracle's final state of the fused forward on that prefix."""
    d = raw_inputs(740, 2, 700, 2, 128, 128, BF16)
    t = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "x", "beta", "z")}
    o, hT, states = kda.kda_chunked_forward_ex(t["q"], t["k"], t["v"], None, t["beta"], dev_tensor(d["h0"]),
                                               state_every=128, gate_x=t["x"], gate_scale=5.0, normalize_qk=True,
                                               out_gate=t["z"])
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_fused(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], x=d["x"], gate_scale=5.0,
                                        normalize_qk=True, z=d["z"])
    assert o_err(host64(o), o_ref) < TOL[BF16] and state_err(host64(hT), h_ref) < TOL[BF16]
    for j in range(700 // 128):
        n = (j + 1) * 128
        p = {key: np.ascontiguousarray(d[key][:, :n]) for key in ("q", "k", "v", "x", "beta")}
        _, h_j = oracle.forward_fused(p["q"], p["k"], p["v"], None, p["beta"], d["h0"], x=p["x"], gate_scale=5.0,
                                      normalize_qk=True, want_o=False)
        assert state_err(host64(states[:, :, j]), h_j) < TOL[BF16], j


def test_varlen_fused():
    lens = [300, 1, 257, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt, H = int(cu[-1]), 3
    d = datagen.prefill_preactivations(750, 1, Tt, H, 128, 128, BF16, None)
    h0 = datagen.fill(750, datagen.TID_H0, 0, 0, 0.02, F32, (len(lens), H, 128, 128), 128)
    t = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "x", "beta", "z")}
    o, hT, states = kda.kda_chunked_forward_varlen_ex(t["q"], t["k"], t["v"], None, t["beta"], dev_tensor(cu),
                                                      max(lens), dev_tensor(h0), state_every=64, gate_x=t["x"],
                                                      gate_scale=5.0, normalize_qk=True, out_gate=t["z"])
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_varlen_fused(d["q"], d["k"], d["v"], None, d["beta"], cu, h0, x=d["x"],
                                               gate_scale=5.0, normalize_qk=True, z=d["z"])
    from tests.kda_testlib import slice_err
    assert slice_err(host64(o)[0], o_ref, (1,)) < TOL[BF16]
    assert state_err(host64(hT), h_ref) < TOL[BF16]
    # one snapshot per sequence checked (the first full 64 tokens)
    for n, L in enumerate(lens):
        if L < 64:
            continue
        s = int(cu[n])
        p = {key: np.ascontiguousarray(d[key][:, s:s + 64]) for key in ("q", "k", "v", "x", "beta")}
        _, h_j = oracle.forward_fused(p["q"], p["k"], p["v"], None, p["beta"], h0[n:n + 1], x=p["x"], gate_scale=5.0,
                                      normalize_qk=True, want_o=False)
        assert state_err(host64(states[n:n + 1, :, 0]), h_j) < TOL[BF16], n
