"""A training step without the recompute: kda_chunked_forward_train gives o and hT bitwise equal to
kda_chunked_forward's and leaves the per-chunk records and chunk-start states in its saved buffer;
kda_chunked_backward_saved then gives gradients bitwise equal to kda_chunked_backward's (the same
kernels run on the same records and states, and the library is deterministic).  kda_chunked_backward
itself is checked against the oracle's gradients (test_gpu_backward.py), so the equality carries that
parity over.  Cases: bf16 and fp32, d = 64 and 128, chunks 16 / 32 / 64, ragged T, no h0 / dhT, the
segmented plan of a few long sequences, and one saved buffer used by two backward calls."""
import pytest
import torch

import datagen
from tests.kda_testlib import dev_tensor

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

KEYS = ("q", "k", "v", "g", "beta")


def case(seed, B, T, H, d, dt, h0_std=0.02, dhT_std=0.5):
    x = datagen.prefill_inputs(seed, B, T, H, d, d, dt, h0_std)
    t = {key: dev_tensor(x[key]) for key in KEYS}
    h0 = dev_tensor(x["h0"]) if h0_std is not None else None
    do, dhT = datagen.backward_adjoints(seed, B, T, H, d, d, dt, dhT_std if dhT_std is not None else 0.5)
    return t, h0, dev_tensor(do), (dev_tensor(dhT) if dhT_std is not None else None)


def check(t, h0, do, dhT, chunk):
    o_a, h_a = kda.kda_chunked_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, chunk=chunk)
    o_b, h_b, saved = kda.kda_chunked_forward_train(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, chunk=chunk)
    g_a = kda.kda_chunked_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, do, dhT, chunk=chunk)
    g_b = kda.kda_chunked_backward_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, do, dhT, saved, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(h_a, h_b)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), g_a, g_b):
        assert torch.equal(x, y), name
    return saved


@pytest.mark.parametrize("dt,B,T,H,d,chunk", [(datagen.DT_BF16, 2, 300, 3, 128, 64), (datagen.DT_BF16, 1, 257, 2, 64, 16),
                                              (datagen.DT_BF16, 2, 100, 2, 128, 32), (datagen.DT_F32, 2, 200, 2, 64, 32),
                                              (datagen.DT_F32, 1, 130, 2, 128, 64)])
def test_train_step_equals_recompute(dt, B, T, H, d, chunk):
    print("train step dt=%d B=%d T=%d H=%d d=%d chunk=%d" % (dt, B, T, H, d, chunk), flush=True)
    check(*case(3100 + T + d + dt, B, T, H, d, dt), chunk)


def test_train_step_without_h0_and_dhT():
    check(*case(3200, 2, 150, 2, 128, datagen.DT_BF16, h0_std=None, dhT_std=None), 64)


def test_train_step_segmented():
    """1 x 16,401 tokens x 8 heads: the forward chain and the adjoint chain both take 8 segments."""
    assert kda.chain_plan(1, 16401, 8, 128, 128, 64)[1] > 1
    print("train step segmented 1 x 16401 x 8", flush=True)
    check(*case(3300, 1, 16401, 8, 128, datagen.DT_BF16), 64)


def test_saved_buffer_serves_two_backward_calls():
    t, h0, do, dhT = case(3400, 2, 200, 2, 128, datagen.DT_BF16)
    saved = check(t, h0, do, dhT, 64)
    do2 = torch.flip(do, dims=[1]).contiguous()
    g_a = kda.kda_chunked_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, do2, None)
    g_b = kda.kda_chunked_backward_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, do2, None, saved)
    torch.cuda.synchronize()
    for x, y in zip(g_a, g_b):
        assert torch.equal(x, y)
