"""Parity of the HIP chunked prefill (kda_chunked_forward / _varlen through the C ABI) with the
fp64 oracle, on seeded inputs with the workloads' distributions: several chunks, ragged tails,
every chunk size, empty sequences, state hand-off and the full-size workloads."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, o_err, slice_err, state_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

F32, BF16 = datagen.DT_F32, datagen.DT_BF16
KEYS = ("q", "k", "v", "g", "beta")


def gpu_forward(d, chunk, h0="same", **kw):
    g = {key: dev_tensor(d[key]) for key in KEYS}
    h = dev_tensor(d["h0"]) if h0 == "same" else h0
    o, hT = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], h, chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, hT


def check(d, chunk, dt, label=""):
    o, hT = gpu_forward(d, chunk)
    o_ref, h_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("%s chunk=%d: o %.2e hT %.2e" % (label, chunk, eo, eh))
    assert eo < TOL[dt] and eh < TOL[dt], (eo, eh)
    return o, hT


def test_workload_fp32_b1_h2_t256_d64():
    w = datagen.WORKLOADS["cfg0_f32_b1_h2_t256_d64"]
    d = datagen.prefill_inputs(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.h0_std)
    check(d, w.chunk, w.dtype, w.name)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 257])
def test_fp32_ragged(chunk, T):
    d = datagen.prefill_inputs(100 + T, 2, T, 2, 64, 64, F32, 0.02)
    check(d, chunk, F32, "fp32 T=%d" % T)


@pytest.mark.parametrize("dk,dv,chunk", [(128, 64, 16), (128, 128, 32), (64, 128, 64), (128, 128, 64), (128, 64, 64)])
def test_fp32_shapes(dk, dv, chunk):
    d = datagen.prefill_inputs(7, 1, 150, 3, dk, dv, F32, 0.02)
    check(d, chunk, F32, "fp32 dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_bf16_shapes(chunk, dk, dv):
    d = datagen.prefill_inputs(200 + dk + dv, 2, 333, 3, dk, dv, BF16, 0.02)
    check(d, chunk, BF16, "bf16 dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("T", [1, 31, 64, 65, 1000])
def test_bf16_lengths(T):
    d = datagen.prefill_inputs(300 + T, 1, T, 4, 128, 128, BF16, 0.02)
    check(d, 64, BF16, "bf16 T=%d" % T)


def test_zero_initial_state_and_no_hT():
    d = datagen.prefill_inputs(41, 2, 130, 2, 128, 128, BF16, None)
    check(d, 64, BF16, "h0=None")
    o, hT = gpu_forward(d, 64, want_hT=False)
    assert hT is None
    o_ref, _ = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], None)
    assert o_err(host64(o), o_ref) < TOL[BF16]


def test_hT_aliases_h0():
    d = datagen.prefill_inputs(42, 2, 200, 2, 128, 128, BF16, 0.02)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    state = dev_tensor(d["h0"])
    o, hT = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], state, hT=state)
    torch.cuda.synchronize()
    assert hT.data_ptr() == state.data_ptr()
    o_ref, h_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    assert o_err(host64(o), o_ref) < TOL[BF16]
    assert state_err(host64(state), h_ref) < TOL[BF16]


def test_empty_sequences():
    d = datagen.prefill_inputs(43, 3, 0, 2, 128, 64, BF16, 0.02)
    o, hT = gpu_forward(d, 64)
    assert o.shape == (3, 0, 2, 64)
    assert torch.equal(hT.cpu(), torch.from_numpy(d["h0"]))
    o, hT = gpu_forward(d, 64, h0=None)
    assert torch.count_nonzero(hT).item() == 0


def test_chunk_size_invariance():
    """Different chunk sizes agree with each other within the same tolerance."""
    d = datagen.prefill_inputs(44, 2, 777, 4, 128, 128, BF16, 0.02)
    outs = {c: gpu_forward(d, c) for c in (16, 32, 64)}
    for a, b in ((16, 32), (16, 64), (32, 64)):
        assert o_err(host64(outs[a][0]), host64(outs[b][0])) < TOL[BF16]
        assert state_err(host64(outs[a][1]), host64(outs[b][1])) < TOL[BF16]
    d32 = datagen.prefill_inputs(45, 1, 300, 2, 64, 64, F32, 0.02)
    outs = {c: gpu_forward(d32, c) for c in (16, 32, 64)}
    for a, b in ((16, 32), (16, 64)):
        assert o_err(host64(outs[a][0]), host64(outs[b][0])) < TOL[F32]


def test_continuation_two_halves():
    """hT of one call is h0 of the next: two halves equal one call (state hand-off)."""
    d = datagen.prefill_inputs(46, 1, 4096, 8, 128, 128, BF16, 0.02)
    o, hT = gpu_forward(d, 64)
    first = {key: np.ascontiguousarray(d[key][:, :2048]) for key in KEYS}
    second = {key: np.ascontiguousarray(d[key][:, 2048:]) for key in KEYS}
    first["h0"] = d["h0"]
    o1, h1 = gpu_forward(first, 64)
    second["h0"] = None
    o2, h2 = gpu_forward(second, 64, h0=h1)
    assert o_err(host64(torch.cat([o1, o2], dim=1)), host64(o)) < TOL[BF16]
    assert state_err(host64(h2), host64(hT)) < TOL[BF16]
    o_ref, h_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    assert o_err(host64(o2), o_ref[:, 2048:]) < TOL[BF16]
    assert state_err(host64(h2), h_ref) < TOL[BF16]


@pytest.mark.parametrize("dt,B,T,H,dk,dv,chunk,h0", [
    (BF16, 1, 8229, 2, 128, 128, 64, True),   # 129 chunks: 4 segments, the last one shorter
    (BF16, 2, 4113, 2, 128, 128, 64, True),   # two sequences, 2 segments each, ragged tail
    (BF16, 1, 4480, 1, 128, 64, 64, True),    # the identity block is wider than the value columns
    (BF16, 1, 4480, 1, 64, 128, 64, False),
    (BF16, 1, 3000, 3, 64, 64, 32, True),     # 94 chunks of 32
    (F32, 1, 6400, 1, 64, 64, 64, True),
    (F32, 1, 2570, 1, 128, 128, 32, True),    # fp32 at d = 128 (16-column slices), ragged
    (F32, 1, 4480, 1, 128, 128, 64, True),    # fp32 records at d = 128, chunk 64: one LDS record buffer
])
def test_segmented_chain_against_oracle(dt, B, T, H, dk, dv, chunk, h0):
    """Long sequences on few heads run the chain per segment (summaries, start states, chain):
    o and hT still match the oracle element by element."""
    plan = kda.chain_plan(B, T, H, dk, dv, chunk, dtype=torch.float32 if dt == F32 else torch.bfloat16)
    assert plan[1] > 1, plan
    d = datagen.prefill_inputs(500 + T + dk, B, T, H, dk, dv, dt, 0.02 if h0 else None)
    check(d, chunk, dt, "segmented plan %s" % (plan,))


def test_segmented_wide_summary_against_oracle():
    """64 segments of one (sequence, head) pair: the summary launch (d_k more columns than the
    chain) would need more than one workgroup per CU at 32 columns, so it runs 64-column slices;
    o and hT still match the oracle element by element."""
    B, T, H, dk, dv, chunk = 1, 32805, 2, 64, 64, 16
    plan = kda.chain_plan(B, T, H, dk, dv, chunk)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert B * H * (plan[1] - 1) * (dk + dv) // 32 > cus, (plan, cus)
    d = datagen.prefill_inputs(733, B, T, H, dk, dv, BF16, 0.02)
    check(d, chunk, BF16, "segmented plan %s, wide summary" % (plan,))


def test_segmented_hT_aliases_h0():
    """In a segmented call h0 is read (by the start-state combine) before any segment writes hT."""
    assert kda.chain_plan(1, 4096, 8, 128, 128)[1] > 1
    d = datagen.prefill_inputs(47, 1, 4096, 8, 128, 128, BF16, 0.02)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    state = dev_tensor(d["h0"])
    o, hT = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], state, hT=state)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    assert o_err(host64(o), o_ref) < TOL[BF16]
    assert state_err(host64(state), h_ref) < TOL[BF16]


def varlen_case(lens, H, dk, dv, dt, seed, h0=True):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt = int(cu[-1])
    d = datagen.prefill_inputs(seed, 1, Tt, H, dk, dv, dt, None)
    d["h0"] = datagen.fill(seed, datagen.TID_H0, 0, 0, 0.02, F32, (len(lens), H, dk, dv), dv) if h0 else None
    return cu, d


@pytest.mark.parametrize("dt", [F32, BF16])
def test_varlen_against_oracle(dt):
    lens = [0, 1, 17, 64, 300, 129, 0, 65]
    dk = dv = 64 if dt == F32 else 128
    cu, d = varlen_case(lens, 3, dk, dv, dt, 47)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    o, hT = kda.kda_chunked_forward_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(cu), max(lens),
                                           dev_tensor(d["h0"]), chunk=32 if dt == F32 else 64)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["h0"])
    eo = slice_err(host64(o)[0], o_ref, (1,))
    eh = state_err(host64(hT), h_ref)
    print("varlen dt=%d: o %.2e hT %.2e" % (dt, eo, eh))
    assert eo < TOL[dt] and eh < TOL[dt]
    # a sequence's output depends on that sequence alone
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        if e == s:
            assert torch.equal(hT[n].cpu(), torch.from_numpy(d["h0"][n]))


@pytest.mark.parametrize("n", [300, 1100])
def test_varlen_many_sequences(n):
    """Many short packed sequences: the chain takes them longest first (ordered on the device up
    to 1024 sequences, in the given order beyond), with no effect on the results."""
    lens = list(datagen.uniform_ints(800 + n, datagen.TID_LEN, n, 0, 70))
    cu, d = varlen_case(lens, 1, 64, 64, BF16, 800 + n)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    o, hT = kda.kda_chunked_forward_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(cu), max(lens),
                                           dev_tensor(d["h0"]), chunk=32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["h0"])
    assert slice_err(host64(o)[0], o_ref, (1,)) < TOL[BF16]
    assert state_err(host64(hT), h_ref) < TOL[BF16]


def test_varlen_equals_batched():
    """Packed equal-length sequences give the same bits as the batched call."""
    B, T, H = 3, 200, 2
    d = datagen.prefill_inputs(48, B, T, H, 128, 128, BF16, 0.02)
    o_b, h_b = gpu_forward(d, 64)
    g = {key: dev_tensor(d[key]).reshape((1, B * T) + d[key].shape[2:]) for key in KEYS}
    cu = dev_tensor(np.arange(0, (B + 1) * T, T, dtype=np.int32))
    o_v, h_v = kda.kda_chunked_forward_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], cu, T,
                                              dev_tensor(d["h0"]), chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o_v.reshape(o_b.shape), o_b) and torch.equal(h_v, h_b)


def test_deterministic():
    d = datagen.prefill_inputs(49, 2, 500, 4, 128, 128, BF16, 0.02)
    a = gpu_forward(d, 64)
    b = gpu_forward(d, 64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_profiled_entry_matches():
    """kda_chunked_forward_profiled runs the same kernels: bitwise-equal results, positive timings."""
    d = datagen.prefill_inputs(50, 2, 300, 4, 128, 128, BF16, 0.02)
    a = gpu_forward(d, 64)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    o = torch.empty_like(a[0])
    hT = torch.empty_like(a[1])
    ms = kda.kda_chunked_forward_profiled(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(d["h0"]), o, hT,
                                          chunk=64)
    print("kernel ms", ms)
    assert torch.equal(o, a[0]) and torch.equal(hT, a[1])
    assert ms[0] > 0 and ms[1] > 0


def test_workload_b4_h16_t4096_full():
    """The 4 x 16-head x 4096-token bf16 workload, every output against the oracle."""
    w = datagen.WORKLOADS["cfg1_bf16_b4_h16_t4096_d128"]
    d = datagen.prefill_inputs(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.h0_std)
    check(d, w.chunk, w.dtype, w.name)


def test_workload_b1_h32_t65536_continuation():
    """The 32-head x 65536-token workload against the oracle, and against two half-length calls."""
    w = datagen.WORKLOADS["cfg2_bf16_b1_h32_t65536_d128"]
    d = datagen.prefill_inputs(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.h0_std)
    o, hT = gpu_forward(d, w.chunk)
    o_ref, h_ref = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("%s: o %.2e hT %.2e" % (w.name, eo, eh))
    assert eo < TOL[w.dtype] and eh < TOL[w.dtype]
    del o_ref
    half = w.T // 2
    first = {key: np.ascontiguousarray(d[key][:, :half]) for key in KEYS}
    second = {key: np.ascontiguousarray(d[key][:, half:]) for key in KEYS}
    first["h0"] = d["h0"]
    o1, h1 = gpu_forward(first, w.chunk)
    second["h0"] = None
    o2, h2 = gpu_forward(second, w.chunk, h0=h1)
    assert o_err(host64(torch.cat([o1, o2], dim=1)), host64(o)) < TOL[w.dtype]
    assert state_err(host64(h2), h_ref) < TOL[w.dtype]


def test_short_sequences_precision():
    """Sequences of 1-4 tokens from a zero state: the output is P U alone, so the intra-chunk products
    carry the whole result, including slices where q . k nearly cancels."""
    lens = [1 + (i % 4) for i in range(64)]
    cu, d = varlen_case(lens, 4, 128, 128, BF16, 50, h0=False)
    g = {key: dev_tensor(d[key]) for key in KEYS}
    o, hT = kda.kda_chunked_forward_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], dev_tensor(cu), max(lens),
                                           None, chunk=64)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, None)
    # per (sequence, head) slice
    worst = 0.0
    og = host64(o)[0]
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        worst = max(worst, slice_err(og[s:e], o_ref[s:e], (1,)))
    eh = state_err(host64(hT), h_ref)
    print("short sequences: o %.2e hT %.2e" % (worst, eh))
    assert worst < TOL[BF16] and eh < TOL[BF16]
