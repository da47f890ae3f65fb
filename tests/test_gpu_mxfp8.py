"""kda_chunked_forward_mxfp8 on the GPU: MXFP8 q, k, v (E4M3 codes, E8M0 scales of 32 channels)
against the fp64 oracle on the decoded inputs, and against the bf16 entry point on the same decoded
values (every decoded value here is a bf16 value, so the two calls give bitwise the same results)."""
import numpy as np
import pytest
import torch

import datagen
import gated_delta_rule_94_amd as kda
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, o_err, state_err

pytestmark = pytest.mark.gpu
BF16 = datagen.DT_BF16


def mx_call(d, chunk, want_hT=True):
    g = {key: dev_tensor(d[key]) for key in ("q8", "qs", "k8", "ks", "v8", "vs", "g", "beta")}
    o, hT = kda.kda_chunked_forward_mxfp8(g["q8"], g["qs"], g["k8"], g["ks"], g["v8"], g["vs"], g["g"], g["beta"],
                                          dev_tensor(d["h0"]), chunk=chunk, want_hT=want_hT)
    torch.cuda.synchronize()
    return o, hT


def bf16_bits(x64):
    """Exact bf16 bit patterns of fp64 values that are bf16 values."""
    b = np.asarray(x64, np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "not a bf16 value"
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("B,T,H,dk,dv,chunk", [
    (2, 200, 3, 128, 128, 64),   # three full chunks and a ragged tail
    (1, 257, 2, 64, 64, 16),
    (1, 100, 2, 64, 128, 32),
    (1, 130, 2, 128, 64, 64),
    (3, 1, 2, 128, 128, 64),     # one-token sequences
])
def test_mxfp8_against_oracle(B, T, H, dk, dv, chunk):
    d = datagen.mxfp8_prefill_inputs(900 + T + dk, B, T, H, dk, dv, 0.02)
    o, hT = mx_call(d, chunk)
    o_ref, h_ref = oracle.forward_mxfp8(d["q8"], d["qs"], d["k8"], d["ks"], d["v8"], d["vs"], d["g"], d["beta"],
                                        d["h0"])
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("mxfp8 B=%d T=%d H=%d d=%d/%d chunk=%d: o %.2e hT %.2e" % (B, T, H, dk, dv, chunk, eo, eh))
    assert eo < TOL[BF16] and eh < TOL[BF16]


@pytest.mark.parametrize("chunk", [16, 64])
def test_mxfp8_equals_bf16_call_on_decoded_inputs(chunk):
    d = datagen.mxfp8_prefill_inputs(77, 2, 300, 2, 128, 128, 0.02)
    o, hT = mx_call(d, chunk)
    dec = {n: dev_tensor(bf16_bits(oracle.mxfp8_decode(d[n + "8"], d[s]))) for n, s in (("q", "qs"), ("k", "ks"), ("v", "vs"))}
    o2, h2 = kda.kda_chunked_forward(dec["q"], dec["k"], dec["v"], dev_tensor(d["g"]), dev_tensor(d["beta"]),
                                     dev_tensor(d["h0"]), chunk=chunk)
    torch.cuda.synchronize()
    same_o = torch.equal(o, o2)
    same_h = torch.equal(hT, h2)
    print("chunk %d: o bitwise equal %s, hT bitwise equal %s" % (chunk, same_o, same_h))
    assert same_o and same_h  # same decoded values, same arithmetic after the loads


def test_mxfp8_empty_and_no_hT():
    d = datagen.mxfp8_prefill_inputs(5, 1, 0, 2, 64, 64, 0.02)
    o, hT = mx_call(d, 64)
    assert o.shape == (1, 0, 2, 64)
    assert np.array_equal(host64(hT), d["h0"].astype(np.float64))  # T = 0: hT = h0
    d = datagen.mxfp8_prefill_inputs(6, 1, 70, 2, 64, 64, None)
    o, hT = mx_call(d, 64, want_hT=False)
    assert hT is None
    o_ref, _ = oracle.forward_mxfp8(d["q8"], d["qs"], d["k8"], d["ks"], d["v8"], d["vs"], d["g"], d["beta"], None,
                                    want_hT=False)
    assert o_err(host64(o), o_ref) < TOL[BF16]


def test_mxfp8_workload_b4_h16_t4096_sampled():
    """The prefill workload's shape (4 x 4096 tokens x 16 heads, d = 128, chunk 64) with MXFP8
    q, k, v: two (sequence, head) units checked element by element against the oracle."""
    w = datagen.WORKLOADS["cfg1_bf16_b4_h16_t4096_d128"]
    d = datagen.mxfp8_prefill_inputs(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.h0_std)
    o, hT = mx_call(d, w.chunk)
    units = [(0, 3), (3, 15)]
    for b, h in units:
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, :, h:h + 1])
        o_ref, h_ref = oracle.forward_mxfp8(sl(d["q8"]), sl(d["qs"]), sl(d["k8"]), sl(d["ks"]), sl(d["v8"]),
                                            sl(d["vs"]), sl(d["g"]), sl(d["beta"]),
                                            np.ascontiguousarray(d["h0"][b:b + 1, h:h + 1]))
        eo = o_err(host64(o[b:b + 1, :, h:h + 1]), o_ref)
        eh = state_err(host64(hT[b:b + 1, h:h + 1]), h_ref)
        print("unit (%d, %d): o %.2e hT %.2e" % (b, h, eo, eh))
        assert eo < TOL[BF16] and eh < TOL[BF16]


def test_mxfp8_every_code():
    """Codes drawn over all 253 finite E4M3 values (subnormals, the largest magnitudes, -0) with
    scales that put each q / v block's largest magnitude at 448 * 2^-8 = 1.75, and k's at 448 * 2^-11
    (so that |k| stays in [0.5, 0.9] and the delta rule contracts): the decode in the kernel's loads
    matches the oracle's decoder through the whole recurrence, and the bf16 call on the decoded
    inputs."""
    B, T, H, dk, dv = 1, 160, 2, 128, 128
    rng = np.random.default_rng(2024)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    d = datagen.mxfp8_prefill_inputs(31, B, T, H, dk, dv, 0.02)
    for name, s, dd, shift in (("q", "qs", dk, 8), ("k", "ks", dk, 11), ("v", "vs", dv, 8)):
        codes = rng.choice(finite, size=(B, T, H, dd)).astype(np.uint8)
        codes[..., ::32] = 0x7E  # one 448 per block
        d[name + "8"] = codes
        d[s] = np.full((B, T, H, dd // 32), 127 - shift, np.uint8)
    o, hT = mx_call(d, 64)
    o_ref, h_ref = oracle.forward_mxfp8(d["q8"], d["qs"], d["k8"], d["ks"], d["v8"], d["vs"], d["g"], d["beta"],
                                        d["h0"])
    eo, eh = o_err(host64(o), o_ref), state_err(host64(hT), h_ref)
    print("every code: o %.2e hT %.2e" % (eo, eh))
    assert eo < TOL[BF16] and eh < TOL[BF16]
    dec = {n: dev_tensor(bf16_bits(oracle.mxfp8_decode(d[n + "8"], d[s]))) for n, s in (("q", "qs"), ("k", "ks"), ("v", "vs"))}
    o2, h2 = kda.kda_chunked_forward(dec["q"], dec["k"], dec["v"], dev_tensor(d["g"]), dev_tensor(d["beta"]),
                                     dev_tensor(d["h0"]), chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(hT, h2)
