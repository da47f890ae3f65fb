"""Long single sequences on few heads: the segmented chain (segment summaries, the fp32 combine of
segment start states, the chain per segment) against the fp64 oracle.

* The plan shape of the 1,048,576-token workload (8 heads, d = 128, chunk 64: whole 128-column
  states per workgroup, 32 segments, summaries in two 128-column halves) at 65,601 tokens, and
  every other layout of the wide chain kernel, every element of o and hT against the oracle.
* The 1,048,576-token workload itself, in the launch configuration the benchmark times: hT against
  the oracle (the recurrence run over all tokens), o in a window starting mid-chunk 700,001 tokens
  in (segment 21 of 32; the oracle's state carried to the window start), o of the first 32,768
  tokens, and a call split in two.
* The packed 16-sequence workload (lengths in [1024, 131072]): every sequence's hT against the
  oracle and o in a window in the middle of every sequence (past 8,192 tokens for all but the
  shortest), the oracle's state carried to each window.

A fixed-size state is what lets the pages' model serve a 1M-token context at a constant cost per
token (how-K3-works page, "KDA: a fixed memory instead of a growing bill")."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, o_err, state_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

BF16 = datagen.DT_BF16
KEYS = ("q", "k", "v", "g", "beta")


def part(d, s, e):
    """Tokens [s, e) of batch-1 inputs (contiguous views)."""
    return {key: np.ascontiguousarray(d[key][:, s:e]) for key in KEYS}


def oracle_run(d, s, e, h0, want_o):
    """The oracle over tokens [s, e) of batch-1 inputs from state h0 (fp64 or None)."""
    p = part(d, s, e)
    return oracle.forward(p["q"], p["k"], p["v"], p["g"], p["beta"], h0, want_o=want_o)


@pytest.mark.parametrize("h0", [False, True])
def test_1m_plan_shape_against_oracle(h0):
    """8 heads, d = 128, chunk 64 and 1026 chunks give the 1M-token workload's plan: whole 128-column
    states per workgroup, 32 segments (of 33 chunks; the last is ragged), summaries of all 256
    columns (value and identity) in one workgroup."""
    B, T, H, d, chunk = 1, 65601, 8, 128, 64
    assert kda.chain_plan(B, T, H, d, d, chunk) == (128, 32, 33)
    assert kda.summary_slice(B, T, H, d, d, chunk) == 256
    w = datagen.WORKLOADS["cfg4_bf16_b1_h8_t1048576_d128"]
    assert kda.chain_plan(w.B, w.T, w.H, w.dk, w.dv, w.chunk) == (128, 32, 512)
    assert kda.summary_slice(w.B, w.T, w.H, w.dk, w.dv, w.chunk) == 256
    dd = datagen.prefill_inputs(911, B, T, H, d, d, BF16, 0.02 if h0 else None)
    g = {key: dev_tensor(dd[key]) for key in KEYS}
    o, hT = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(dd["h0"]), chunk=chunk)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"])
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("65601 tokens x 8 heads, 32 segments: o %.2e hT %.2e" % (eo, eh))
    assert eo < TOL[BF16] and eh < TOL[BF16]


@pytest.mark.parametrize("dk,dv,B,T,H,plan,summary", [
    (64, 64, 1, 4160, 1, (32, 2, 33), 128),
    (64, 128, 1, 4160, 1, (32, 2, 33), 192),
    (128, 64, 1, 4160, 1, (32, 2, 33), 192),
    (128, 128, 1, 4160, 1, (32, 2, 33), 256),
    (64, 64, 2, 65601, 4, (64, 32, 33), 128),
    (64, 128, 1, 65601, 4, (64, 32, 33), 192),
    (64, 128, 2, 65601, 4, (128, 32, 33), 192),
    (128, 64, 2, 65601, 4, (64, 32, 33), 192),
    (128, 128, 1, 65601, 4, (64, 32, 33), 256),
])
def test_wide_chain_layouts_against_oracle(dk, dv, B, T, H, plan, summary):
    """Every layout of the wide chain kernel (bf16, chunk 64) a segmented plan takes: value slices
    of 32, 64 and 128 columns, summaries of all d_v + d_k columns (128, 192, 256), every (d_k, d_v);
    every element of o and hT against the oracle."""
    assert kda.chain_plan(B, T, H, dk, dv, 64) == plan
    assert kda.summary_slice(B, T, H, dk, dv, 64) == summary
    dd = datagen.prefill_inputs(920 + dk + dv + B, B, T, H, dk, dv, BF16, 0.02)
    g = {key: dev_tensor(dd[key]) for key in KEYS}
    print("dk=%d dv=%d B=%d T=%d H=%d plan %s summary %d" % (dk, dv, B, T, H, plan, summary), flush=True)
    o, hT = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(dd["h0"]), chunk=64)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"])
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("  o %.2e hT %.2e" % (eo, eh))
    assert eo < TOL[BF16] and eh < TOL[BF16]


@pytest.fixture(scope="module")
def one_million():
    w = datagen.WORKLOADS["cfg4_bf16_b1_h8_t1048576_d128"]
    d = datagen.prefill_inputs(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.h0_std)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    print("1M-token workload: plan", kda.chain_plan(w.B, w.T, w.H, w.dk, w.dv, w.chunk), flush=True)
    o, hT = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], None, chunk=w.chunk)
    torch.cuda.synchronize()
    del g
    return w, d, o, hT


def test_1m_sequence_against_oracle(one_million):
    """hT after all 1,048,576 tokens, o in a 4096-token window starting mid-chunk 700,001 tokens in
    (segments are 512 chunks = 32,768 tokens) and o of the first 32,768 tokens (segment 0)."""
    w, d, o, hT = one_million
    cut, win = 700_001, 4096
    _, h_cut = oracle_run(d, 0, cut, None, want_o=False)
    o_win, h_win = oracle_run(d, cut, cut + win, h_cut, want_o=True)
    _, h_ref = oracle_run(d, cut + win, w.T, h_win, want_o=False)
    eo = o_err(host64(o[:, cut:cut + win]), o_win)
    eh = state_err(host64(hT), h_ref)
    print("1M tokens: o window [%d, %d) %.2e, hT %.2e" % (cut, cut + win, eo, eh))
    assert eo < TOL[w.dtype] and eh < TOL[w.dtype]
    P = 32768
    o_pre, _ = oracle_run(d, 0, P, None, want_o=True)
    ep = o_err(host64(o[:, :P]), o_pre)
    print("1M tokens: o prefix %.2e" % ep)
    assert ep < TOL[w.dtype]


def test_1m_sequence_split_call(one_million):
    """The call split in two (state handed over; each half plans its own segments) reproduces the
    second half's outputs and the final state."""
    w, d, o, hT = one_million
    cut = 600_000 + 17  # not a chunk multiple
    first, second = part(d, 0, cut), part(d, cut, w.T)
    g1 = {key: dev_tensor(first[key]) for key in KEYS}
    o1, h1 = kda.kda_chunked_forward(g1["q"], g1["k"], g1["v"], g1["g"], g1["beta"], None, chunk=w.chunk)
    del g1, o1
    g2 = {key: dev_tensor(second[key]) for key in KEYS}
    o2, h2 = kda.kda_chunked_forward(g2["q"], g2["k"], g2["v"], g2["g"], g2["beta"], h1, chunk=w.chunk)
    torch.cuda.synchronize()
    assert o_err(host64(o2), host64(o[:, cut:])) < TOL[w.dtype]
    assert state_err(host64(h2), host64(hT)) < TOL[w.dtype]
    assert np.isfinite(host64(hT)).all()


def test_varlen_16_sequences_against_oracle():
    """Every sequence's hT and o in a 2048-token window in the middle of every sequence."""
    w = datagen.WORKLOADS["cfg4v_varlen_n16_h8_d128"]
    lens = datagen.varlen_lengths(w.seed, w.num_seqs, w.len_lo, w.len_hi)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt = int(cu[-1])
    d = datagen.prefill_inputs(w.seed, 1, Tt, w.H, w.dk, w.dv, w.dtype, None)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    o, hT = kda.kda_chunked_forward_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(cu),
                                           int(lens.max()), None, chunk=w.chunk)
    torch.cuda.synchronize()
    del g
    win = 2048
    worst_o = worst_h = 0.0
    for n in range(w.num_seqs):
        s, e = int(cu[n]), int(cu[n + 1])
        a = s + max(0, (e - s) // 2 - win // 2)
        b = min(e, a + win)
        _, h_a = oracle_run(d, s, a, None, want_o=False)
        o_w, h_b = oracle_run(d, a, b, h_a, want_o=True)
        _, h_e = oracle_run(d, b, e, h_b, want_o=False)
        eo = o_err(host64(o[:, a:b]), o_w)
        eh = state_err(host64(hT[n:n + 1]), h_e)
        print("sequence %d (%d tokens): o [%d, %d) %.2e, hT %.2e" % (n, e - s, a - s, b - s, eo, eh), flush=True)
        worst_o, worst_h = max(worst_o, eo), max(worst_h, eh)
    assert worst_o < TOL[w.dtype] and worst_h < TOL[w.dtype], (worst_o, worst_h)
