"""Parity of kda_chunked_backward_varlen (gradients of <do, o> + <dhT, hT> through the packed
prefill) with the oracle's reverse-mode gradients, computed one sequence at a time on that
sequence's own inputs, h0 and dhT: no adjoint may cross a sequence boundary (the chunks restart at
every sequence, as the forward's do).  Element by element per (sequence, head) slice: 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs (fp32 state).

With bf16 inputs a sequence shorter than SHORT tokens is checked per head, pooled over all such
sequences of the call.  A one- or two-token slice of dbeta or dq is a single dot product over the
value columns (dbeta_t = dU_t . u_t; dq through dP = do . u), which can cancel to almost nothing;
the bf16 records the forward keeps (the same 2^-9 operand rounding as the forward's) then leave an
error that is small against the terms but unbounded against their sum.  Measured over 256 one-token
slices: dbeta up to 0.34 and dq up to 5.4e-2 of the slice's own value (13 and 7 slices over 2e-2),
every slice within 2e-2 from 16 tokens on.  The pooled slices hold at least 16 tokens per head."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, slice_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

F32, BF16 = datagen.DT_F32, datagen.DT_BF16
KEYS = ("q", "k", "v", "g", "beta")
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
SHORT = 16


def packed_case(seed, lens, H, dk, dv, dt, h0_std=0.02, dhT_std=0.5):
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, Tt = len(lens), int(cu[-1])
    d = datagen.prefill_inputs(seed, 1, Tt, H, dk, dv, dt, None)
    do, _ = datagen.backward_adjoints(seed, 1, Tt, H, dk, dv, dt, None)
    h0 = None if h0_std is None else datagen.prefill_inputs(seed + 1, N, 1, H, dk, dv, dt, h0_std)["h0"]
    dhT = None if dhT_std is None else datagen.backward_adjoints(seed + 1, N, 1, H, dk, dv, dt, dhT_std)[1]
    return d, do, h0, dhT, cu


def gpu_backward(d, do, h0, dhT, cu, chunk):
    t = {key: dev_tensor(d[key]) for key in KEYS}
    lens = np.diff(cu)
    got = kda.kda_chunked_backward_varlen(t["q"], t["k"], t["v"], t["g"], t["beta"], dev_tensor(cu),
                                          int(lens.max()) if len(lens) else 0, dev_tensor(h0), dev_tensor(do),
                                          dev_tensor(dhT), chunk=chunk)
    torch.cuda.synchronize()
    return got  # device tensors; checks copy the slices they need


def check_sequences(d, do, h0, dhT, cu, got, dt, seqs=None):
    """Every (or the given) sequence's gradients against the oracle on that sequence alone."""
    worst = {}
    pool = {}  # short bf16 sequences: per gradient, (got, ref) token rows concatenated
    H, dk, dv = d["q"].shape[2], d["q"].shape[3], d["v"].shape[3]
    for n in (range(len(cu) - 1) if seqs is None else seqs):
        s, e = int(cu[n]), int(cu[n + 1])
        h0n = None if h0 is None else h0[n:n + 1]
        dhTn = None if dhT is None else dhT[n:n + 1]
        if e == s:  # an empty sequence: no token gradients; the adjoint passes straight to h0
            want = np.zeros((1, H, dk, dv)) if dhTn is None else dhTn.astype(np.float64)
            assert np.array_equal(host64(got[5][n:n + 1]), want), n
            continue
        sl = {key: np.ascontiguousarray(d[key][:, s:e]) for key in KEYS}
        ref = oracle.backward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], h0n, np.ascontiguousarray(do[:, s:e]),
                              dhTn)
        for name, x, y in zip(NAMES, got, ref):
            if name == "dh0":
                err = slice_err(host64(x[n:n + 1]), y, (0, 1))
            elif dt == BF16 and e - s < SHORT:
                gx, gy = pool.get(name, ([], []))
                pool[name] = (gx + [host64(x[:, s:e])], gy + [y])
                continue
            else:
                err = slice_err(host64(x[:, s:e]), y, (0, 2))
            worst[name] = max(worst.get(name, 0.0), err)
    for name, (gx, gy) in pool.items():  # per head over the pooled tokens of the short sequences
        err = slice_err(np.concatenate(gx, axis=1), np.concatenate(gy, axis=1), (0, 2))
        worst[name] = max(worst.get(name, 0.0), err)
    print("  " + "  ".join("%s %.2e" % kv for kv in worst.items()), flush=True)
    for name, err in worst.items():
        assert err < TOL[dt], (name, err)


@pytest.mark.parametrize("dt,dk,dv,chunk", [(BF16, 128, 128, 64), (BF16, 128, 128, 16), (BF16, 64, 128, 32),
                                            (F32, 64, 64, 64), (F32, 64, 64, 16), (F32, 128, 128, 64),
                                            (F32, 128, 64, 32)])
def test_backward_varlen_against_oracle(dt, dk, dv, chunk):
    """Ten sequences: empty; 1, 2, 3, 5 and 8 tokens (19 pooled short tokens per head with bf16);
    one short of a chunk; one chunk; several chunks with a ragged tail; another empty one."""
    lens = [0, 1, 2, 3, 5, 8, chunk - 1, chunk, 3 * chunk + 7, 0]
    print("varlen backward dt=%d dk=%d dv=%d chunk=%d lengths %s" % (dt, dk, dv, chunk, lens), flush=True)
    d, do, h0, dhT, cu = packed_case(1200 + dk + dv + chunk + dt, lens, 3, dk, dv, dt)
    got = gpu_backward(d, do, h0, dhT, cu, chunk)
    check_sequences(d, do, h0, dhT, cu, got, dt)


def test_backward_varlen_without_h0_and_dhT():
    lens = [130, 0, 77]
    d, do, h0, dhT, cu = packed_case(1300, lens, 2, 128, 128, BF16, h0_std=None, dhT_std=None)
    got = gpu_backward(d, do, h0, dhT, cu, 64)
    check_sequences(d, do, h0, dhT, cu, got, BF16)


def test_backward_varlen_long_and_short():
    """Sequences of 1 to 90 chunks in one call (the adjoint chain takes them longest first)."""
    lens = [5000, 1, 2, 13, 3001, 64, 0, 777]
    d, do, h0, dhT, cu = packed_case(1400, lens, 2, 128, 128, BF16)
    got = gpu_backward(d, do, h0, dhT, cu, 64)
    check_sequences(d, do, h0, dhT, cu, got, BF16)


def test_backward_varlen_equals_batched():
    """Equal lengths packed: the same gradients as the batched backward, bitwise."""
    B, T, H, D = 3, 200, 2, 128
    d = datagen.prefill_inputs(1500, B, T, H, D, D, BF16, 0.02)
    do, dhT = datagen.backward_adjoints(1500, B, T, H, D, D, BF16, 0.5)
    t = {key: dev_tensor(d[key]) for key in KEYS}
    a = kda.kda_chunked_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], dev_tensor(d["h0"]), dev_tensor(do),
                                 dev_tensor(dhT))
    pk = {key: t[key].reshape((1, B * T) + tuple(t[key].shape[2:])) for key in KEYS}
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    b = kda.kda_chunked_backward_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], cu, T, dev_tensor(d["h0"]),
                                        dev_tensor(do).reshape(1, B * T, H, D), dev_tensor(dhT))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.reshape(y.shape), y)


def test_backward_varlen_empty_call():
    """T_total = 0: every sequence is empty, dh0 = dhT."""
    N, H, d = 3, 2, 64
    q = torch.empty((1, 0, H, d), dtype=torch.bfloat16, device="cuda")
    beta = torch.empty((1, 0, H), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    dhT = torch.randn((N, H, d, d), device="cuda")
    h0 = torch.randn((N, H, d, d), device="cuda")
    grads = kda.kda_chunked_backward_varlen(q, q, q, q, beta, cu, 0, h0, q, dhT)
    torch.cuda.synchronize()
    assert torch.equal(grads[5], dhT)


def test_backward_varlen_workload_sampled():
    """The 16 packed sequences of the varlen prefill workload (970,282 tokens x 8 heads): the whole
    backward call, its shortest sequence's gradients against the oracle (every head), and dh0 of
    every unit finite."""
    w = datagen.WORKLOADS["cfg4v_varlen_n16_h8_d128"]
    lens = datagen.varlen_lengths(w.seed, w.num_seqs, w.len_lo, w.len_hi)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt = int(cu[-1])
    d = datagen.prefill_inputs(w.seed, 1, Tt, w.H, w.dk, w.dv, w.dtype, None)
    do, _ = datagen.backward_adjoints(w.seed, 1, Tt, w.H, w.dk, w.dv, w.dtype, None)
    dhT = datagen.backward_adjoints(w.seed + 1, w.num_seqs, 1, w.H, w.dk, w.dv, w.dtype, 0.5)[1]
    print("varlen workload backward: %d tokens, %d sequences" % (Tt, w.num_seqs), flush=True)
    got = gpu_backward(d, do, None, dhT, cu, w.chunk)
    assert bool(torch.isfinite(got[5]).all())
    check_sequences(d, do, None, dhT, cu, got, w.dtype, seqs=[int(np.argmin(lens))])
