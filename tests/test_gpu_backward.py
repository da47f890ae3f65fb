"""Parity of kda_chunked_backward (gradients of <do, o> + <dhT, hT> through the chunked prefill)
with the oracle's reverse-mode gradients of the plain recurrence, element by element per
(sequence, head) slice: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 state)."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, slice_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

F32, BF16 = datagen.DT_F32, datagen.DT_BF16
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def errors(got, ref):
    out = {}
    for name, x, y in zip(NAMES, got, ref):
        if x is None:
            continue
        axes = (0, 1) if name == "dh0" else (0, 2)
        out[name] = slice_err(host64(x), y, axes)
    return out


def run_case(seed, B, T, H, dk, dv, dt, chunk, h0_std=0.02, dhT_std=0.5, label=""):
    d = datagen.prefill_inputs(seed, B, T, H, dk, dv, dt, h0_std)
    do, dhT = datagen.backward_adjoints(seed, B, T, H, dk, dv, dt, dhT_std)
    t = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "g", "beta")}
    print("case %s: B=%d T=%d H=%d dk=%d dv=%d chunk=%d dt=%d" % (label, B, T, H, dk, dv, chunk, dt), flush=True)
    got = kda.kda_chunked_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], dev_tensor(d["h0"]), dev_tensor(do),
                                   dev_tensor(dhT), chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, dhT)
    e = errors(got, ref)
    print("  " + "  ".join("%s %.2e" % kv for kv in e.items()), flush=True)
    for name, err in e.items():
        assert err < TOL[dt], (name, err)
    return got, ref


@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_backward_bf16_d128(chunk):
    run_case(900 + chunk, 2, 333, 3, 128, 128, BF16, chunk, label="bf16 d128")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64)])
def test_backward_bf16_mixed_dims(dk, dv):
    run_case(910 + dk + dv, 1, 200, 2, dk, dv, BF16, 64, label="bf16 mixed")


@pytest.mark.parametrize("chunk,T", [(64, 256), (64, 150), (32, 97), (16, 40)])
def test_backward_fp32(chunk, T):
    run_case(920 + chunk + T, 1, T, 2, 64, 64, F32, chunk, label="fp32")


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_backward_fp32_d128(dk, dv, chunk):
    """fp32 with a 128-wide dimension: the state products take the value columns in passes (the
    LDS holds half or a quarter of them), and at d_k = 128, chunk 64, the transform reads q and v
    from global memory where it uses them."""
    run_case(985 + dk + dv + chunk, 2, 3 * chunk + 11, 2, dk, dv, F32, chunk, label="fp32 d128")


def test_backward_without_h0_and_dhT():
    run_case(930, 2, 130, 2, 128, 128, BF16, 64, h0_std=None, dhT_std=None, label="no h0/dhT")


@pytest.mark.parametrize("T", [1, 17, 64])
def test_backward_single_chunk(T):
    run_case(940 + T, 2, T, 2, 128, 128, BF16, 64, label="one chunk")


def test_backward_empty_sequence():
    """T = 0: no token gradients; dh0 = dhT."""
    B, H, d = 2, 3, 64
    q = torch.empty((B, 0, H, d), dtype=torch.bfloat16, device="cuda")
    beta = torch.empty((B, 0, H), dtype=torch.bfloat16, device="cuda")
    dhT = torch.randn((B, H, d, d), device="cuda")
    h0 = torch.randn((B, H, d, d), device="cuda")
    grads = kda.kda_chunked_backward(q, q, q, q, beta, h0, q, dhT)
    torch.cuda.synchronize()
    assert torch.equal(grads[5], dhT)


def test_backward_with_segmented_forward():
    """A long sequence on few heads: the forward recompute splits the chain into segments."""
    assert kda.chain_plan(1, 8229, 2, 128, 128)[1] == 4
    run_case(950, 1, 8229, 2, 128, 128, BF16, 64, label="segmented")


@pytest.mark.parametrize("dhT_std", [0.5, None])
def test_backward_segmented_adjoint_chain(dhT_std):
    """8 heads x 16,401 tokens (257 chunks of 64): (sequence, head, 32-column slice) would give 32
    workgroups, so the adjoint chain runs in 8 segments -- summaries of segments 1..7 over d_k extra
    identity columns, the combine of their end adjoints from dhT, then every segment -- and the
    forward recompute is segmented too.  Every gradient element against the oracle."""
    assert kda.chain_plan(1, 16401, 8, 128, 128)[1] > 1
    run_case(970, 1, 16401, 8, 128, 128, BF16, 64, dhT_std=dhT_std, label="segmented adjoint chain")


@pytest.mark.parametrize("chunk,T", [(64, 4160), (32, 2101)])
def test_backward_segmented_adjoint_chain_fp32(chunk, T):
    """One head, fp32, d = 64: 2 adjoint segments (ragged last chunk)."""
    run_case(975 + chunk, 1, T, 1, 64, 64, F32, chunk, label="segmented adjoint chain fp32")


def test_backward_is_deterministic():
    d = datagen.prefill_inputs(960, 2, 300, 4, 128, 128, BF16, 0.02)
    do, dhT = datagen.backward_adjoints(960, 2, 300, 4, 128, 128, BF16, 0.5)
    t = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "g", "beta")}
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], dev_tensor(d["h0"]), dev_tensor(do), dev_tensor(dhT))
    a = kda.kda_chunked_backward(*args)
    b = kda.kda_chunked_backward(*args)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_sampled_units():
    """The training-step shape of the prefill benchmark (4 x 4096 tokens, 16 heads, bf16, d = 128):
    two (sequence, head) units checked against the oracle on that unit's inputs alone."""
    B, T, H, D = 4, 4096, 16, 128
    d = datagen.prefill_inputs(9401, B, T, H, D, D, BF16, 0.02)
    do, dhT = datagen.backward_adjoints(9401, B, T, H, D, D, BF16, 0.5)
    t = {key: dev_tensor(d[key]) for key in ("q", "k", "v", "g", "beta")}
    got = kda.kda_chunked_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], dev_tensor(d["h0"]), dev_tensor(do),
                                   dev_tensor(dhT))
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 11)):
        sl = {key: np.ascontiguousarray(d[key][b:b + 1, :, h:h + 1]) for key in ("q", "k", "v", "g", "beta")}
        ref = oracle.backward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], d["h0"][b:b + 1, h:h + 1],
                              np.ascontiguousarray(do[b:b + 1, :, h:h + 1]), dhT[b:b + 1, h:h + 1])
        sub = [x[b:b + 1, :, h:h + 1] if x.dim() >= 3 and x.shape[1] == T else x[b:b + 1, h:h + 1] for x in got]
        e = errors(sub, ref)
        print("unit (%d, %d): " % (b, h) + "  ".join("%s %.2e" % kv for kv in e.items()), flush=True)
        for name, err in e.items():
            assert err < TOL[BF16], (b, h, name, err)
