"""State snapshots every N tokens (kda_chunked_forward_with_states and the varlen form): entry j
must be the state after the first (j+1) N tokens, i.e. the oracle's hT on that prefix, and
resuming from it must reproduce the rest of the sequence.  o and hT are those of the plain call."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, o_err, state_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

F32, BF16 = datagen.DT_F32, datagen.DT_BF16
KEYS = ("q", "k", "v", "g", "beta")


def prefix(d, n):
    return {key: np.ascontiguousarray(d[key][:, :n]) for key in KEYS}


def check_states(d, chunk, every, dt, label):
    g = {key: dev_tensor(d[key]) for key in KEYS}
    h0 = dev_tensor(d["h0"])
    o, hT, states = kda.kda_chunked_forward_with_states(g["q"], g["k"], g["v"], g["g"], g["beta"], h0,
                                                        state_every=every, chunk=chunk)
    o_plain, h_plain = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], h0, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain) and torch.equal(hT, h_plain)
    T = d["q"].shape[1]
    assert states.shape[2] == T // every
    worst = 0.0
    for j in range(T // every):
        p = prefix(d, (j + 1) * every)
        _, h_ref = oracle.forward(p["q"], p["k"], p["v"], p["g"], p["beta"], d["h0"], want_o=False)
        e = state_err(host64(states[:, :, j]), h_ref)
        worst = max(worst, e)
        assert e < TOL[dt], (j, e)
    print("%s: %d states, worst %.2e" % (label, T // every, worst))
    return o, hT, states


@pytest.mark.parametrize("dt,B,T,H,dk,dv,chunk,every", [
    (BF16, 2, 1000, 3, 128, 128, 64, 128),
    (BF16, 1, 777, 2, 64, 128, 32, 96),
    (F32, 2, 300, 2, 64, 64, 32, 64),
    (F32, 1, 300, 2, 128, 128, 64, 128),  # one LDS record buffer in the chain
])
def test_states_are_prefix_states(dt, B, T, H, dk, dv, chunk, every):
    d = datagen.prefill_inputs(600 + T, B, T, H, dk, dv, dt, 0.02)
    check_states(d, chunk, every, dt, "states dt=%d T=%d every=%d" % (dt, T, every))


def test_states_with_segmented_chain():
    """Snapshots from every segment of a segmented chain (4 segments of 33 chunks)."""
    assert kda.chain_plan(1, 8229, 2, 128, 128)[1] == 4
    d = datagen.prefill_inputs(610, 1, 8229, 2, 128, 128, BF16, 0.02)
    check_states(d, 64, 1024, BF16, "segmented states")


def test_resume_from_a_state():
    """A prompt resumed from a cached state: states[j] as h0 of the remaining tokens gives the
    remaining outputs and the final state of the one-shot call."""
    d = datagen.prefill_inputs(620, 1, 900, 4, 128, 128, BF16, 0.02)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    o, hT, states = kda.kda_chunked_forward_with_states(g["q"], g["k"], g["v"], g["g"], g["beta"],
                                                        dev_tensor(d["h0"]), state_every=256)
    cut = 512
    rest = {key: dev_tensor(np.ascontiguousarray(d[key][:, cut:])) for key in KEYS}
    o2, h2 = kda.kda_chunked_forward(rest["q"], rest["k"], rest["v"], rest["g"], rest["beta"],
                                     states[:, :, cut // 256 - 1].contiguous())
    torch.cuda.synchronize()
    assert o_err(host64(o2), host64(o[:, cut:])) < TOL[BF16]
    assert state_err(host64(h2), host64(hT)) < TOL[BF16]


def test_varlen_states():
    lens = [300, 1, 640, 0, 129, 64]
    every = 64
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt, H, dk, dv = int(cu[-1]), 2, 128, 128
    d = datagen.prefill_inputs(630, 1, Tt, H, dk, dv, BF16, None)
    h0 = datagen.fill(630, datagen.TID_H0, 0, 0, 0.02, F32, (len(lens), H, dk, dv), dv)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    slots = max(lens) // every
    sentinel = torch.full((len(lens), H, slots, dk, dv), 7.0, dtype=torch.float32, device="cuda")
    o, hT, states = kda.kda_chunked_forward_varlen_with_states(g["q"], g["k"], g["v"], g["g"], g["beta"],
                                                               dev_tensor(cu), max(lens), dev_tensor(h0),
                                                               state_every=every, states=sentinel)
    o_plain, h_plain = kda.kda_chunked_forward_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(cu),
                                                      max(lens), dev_tensor(h0))
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain) and torch.equal(hT, h_plain)
    st = host64(states)
    for n, L in enumerate(lens):
        s = int(cu[n])
        for j in range(slots):
            if (j + 1) * every > L:
                assert np.all(st[n, :, j] == 7.0), (n, j)  # past the sequence: untouched
                continue
            e = s + (j + 1) * every
            seq = {key: np.ascontiguousarray(d[key][:, s:e]) for key in KEYS}
            _, h_ref = oracle.forward(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"], h0[n:n + 1],
                                      want_o=False)
            assert state_err(st[n:n + 1, :, j], h_ref) < TOL[BF16], (n, j)
