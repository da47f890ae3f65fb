"""Parity of the HIP decode step (kda_decode_step through the C ABI) with the fp64 oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, slice_err, state_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")


def run_steps(seed, B, H, dk, dv, dt, steps, state0):
    """GPU and oracle side by side for `steps` decode steps; returns (max o err, final state err)."""
    st_gpu = dev_tensor(state0.copy())
    st_ref = state0.astype(np.float64)
    worst = 0.0
    for s in range(steps):
        d = datagen.decode_inputs(seed, s, B, H, dk, dv, dt)
        o = kda.kda_decode_step(*(dev_tensor(d[key]) for key in ("q", "k", "v", "g", "beta")), st_gpu)
        o_ref = oracle.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st_ref)
        worst = max(worst, slice_err(host64(o), o_ref, (0, 1)))
    torch.cuda.synchronize()
    return worst, state_err(host64(st_gpu), st_ref)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_decode_fp32(dk, dv):
    B, H = 3, 2
    s0 = datagen.decode_state0(1, B, H, dk, dv)
    eo, es = run_steps(11, B, H, dk, dv, datagen.DT_F32, 20, s0)
    print("decode fp32 dk=%d dv=%d: o %.2e state %.2e" % (dk, dv, eo, es))
    assert eo < 1e-4 and es < 1e-4


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_decode_bf16_shapes(dk, dv):
    B, H = 5, 3
    s0 = datagen.decode_state0(3, B, H, dk, dv)
    eo, es = run_steps(13, B, H, dk, dv, datagen.DT_BF16, 40, s0)
    print("decode bf16 dk=%d dv=%d: o %.2e state %.2e" % (dk, dv, eo, es))
    assert eo < TOL[datagen.DT_BF16] and es < TOL[datagen.DT_BF16]


def test_decode_bf16_many_steps():
    B, H, d = 4, 8, 128
    s0 = datagen.decode_state0(2, B, H, d, d)
    eo, es = run_steps(12, B, H, d, d, datagen.DT_BF16, 300, s0)
    print("decode bf16 300 steps: o %.2e state %.2e" % (eo, es))
    assert eo < TOL[datagen.DT_BF16] and es < TOL[datagen.DT_BF16]


def test_decode_full_size_1000_steps_sampled():
    """The 256-sequence x 32-head workload (512 MiB fp32 state) for all of its 1000 sequential
    steps: o of 48 sampled (sequence, head) units against the oracle at every step, and their
    states every 100 steps and at the end (the oracle carries only the sampled units' states)."""
    w = datagen.WORKLOADS["cfg3_decode_b256_h32_d128"]
    B, H, d = w.B, w.H, w.dk
    s0 = datagen.decode_state0(w.seed, B, H, d, d)
    st_gpu = dev_tensor(s0)
    units = np.random.default_rng(3).choice(B * H, size=48, replace=False)
    ub, uh = units // H, units % H
    ub_d, uh_d = torch.from_numpy(ub).cuda(), torch.from_numpy(uh).cuda()
    st_ref = s0[ub, uh].astype(np.float64)[:, None]  # [n, 1, dk, dv]
    worst_o = worst_s = 0.0
    for s in range(w.steps):
        dd = datagen.decode_inputs(w.seed, s, B, H, d, d, w.dtype)
        o = kda.kda_decode_step(*(dev_tensor(dd[key]) for key in ("q", "k", "v", "g", "beta")), st_gpu)
        sub = {key: np.ascontiguousarray(dd[key][ub, uh][:, None]) for key in ("q", "k", "v", "g", "beta")}
        o_ref = oracle.decode_step(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], st_ref)
        worst_o = max(worst_o, slice_err(host64(o[ub_d, uh_d])[:, None], o_ref, (0, 1)))
        if (s + 1) % 100 == 0:
            worst_s = max(worst_s, state_err(host64(st_gpu[ub_d, uh_d])[:, None], st_ref))
            print("decode step %d: o %.2e state %.2e" % (s + 1, worst_o, worst_s), flush=True)
    assert worst_o < TOL[w.dtype] and worst_s < TOL[w.dtype], (worst_o, worst_s)


def test_decode_steps_equal_prefill():
    """T decode steps equal one prefill of the same T tokens (both on the GPU)."""
    B, T, H, d = 2, 48, 4, 128
    inp = datagen.prefill_inputs(31, B, T, H, d, d, datagen.DT_BF16, 0.02)
    g = {key: dev_tensor(val) for key, val in inp.items()}
    o_pre, h_pre = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], chunk=16)
    st = g["h0"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.kda_decode_step(*(g[key][:, t].contiguous() for key in ("q", "k", "v", "g", "beta")), st))
    o_dec = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    assert slice_err(host64(o_dec), host64(o_pre), (0, 2)) < TOL[datagen.DT_BF16]
    assert state_err(host64(st), host64(h_pre)) < TOL[datagen.DT_BF16]


def test_decode_deterministic():
    B, H, d = 8, 4, 128
    s0 = datagen.decode_state0(4, B, H, d, d)
    dd = datagen.decode_inputs(14, 0, B, H, d, d, datagen.DT_BF16)
    args = [dev_tensor(dd[key]) for key in ("q", "k", "v", "g", "beta")]
    a, b = dev_tensor(s0), dev_tensor(s0)
    oa = kda.kda_decode_step(*args, a)
    ob = kda.kda_decode_step(*args, b)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(a, b)
