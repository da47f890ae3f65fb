"""kda_chunked_forward_noalloc (the prefill entry point for callers that cannot allocate: its scratch
is the library's fixed per-GPU device buffer) against kda_chunked_forward (scratch in a caller-owned
workspace), through the C ABI: two calls in a row, the second with a smaller input, each bitwise
equal to the workspace call (the same kernels run on the same inputs; the library is deterministic),
and the first also against the fp64 oracle.  The first call's plan splits its sequences into
segments, so the segment states share the scratch with the records."""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.kda_testlib import TOL, dev_tensor, host64, o_err, state_err

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

KEYS = ("q", "k", "v", "g", "beta")


def both(d, chunk):
    g = {key: dev_tensor(d[key]) for key in KEYS}
    h0 = dev_tensor(d["h0"])
    o_a, h_a = kda.kda_chunked_forward(g["q"], g["k"], g["v"], g["g"], g["beta"], h0, chunk=chunk)
    o_b = torch.empty_like(o_a)
    h_b = torch.empty_like(h_a)
    torch.cuda.synchronize()
    kda.kda_chunked_forward_noalloc(g["q"], g["k"], g["v"], g["g"], g["beta"], h0, chunk=chunk, o=o_b, hT=h_b)
    torch.cuda.synchronize()
    return (o_a, h_a), (o_b, h_b)


def test_noalloc_equals_workspace_call():
    # call 1: 2 heads x 20,001 tokens, bf16, d = 128: 626 records (46 MB) and 9 segments per head
    B, T, H, d, chunk = 1, 20001, 2, 128, 64
    assert kda.chain_plan(B, T, H, d, d, chunk)[1] > 1
    need = kda.workspace_bytes(B, T, H, d, d, chunk)
    assert 32 << 20 < need <= kda.NOALLOC_SCRATCH_BYTES, need
    d1 = datagen.prefill_inputs(8101, B, T, H, d, d, datagen.DT_BF16, 0.02)
    print("noalloc call 1: B=%d T=%d H=%d d=%d, scratch %d bytes" % (B, T, H, d, need), flush=True)
    (o_a, h_a), (o_b, h_b) = both(d1, chunk)
    assert torch.equal(o_a, o_b) and torch.equal(h_a, h_b)
    o_ref, h_ref = oracle.forward(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["h0"])
    assert o_err(host64(o_b), o_ref) < TOL[datagen.DT_BF16] and state_err(host64(h_b), h_ref) < TOL[datagen.DT_BF16]
    # call 2, smaller: 3 sequences x 4 heads x 333 tokens, fp32, d_k = 64, d_v = 128, chunk 32
    d2 = datagen.prefill_inputs(8102, 3, 333, 4, 64, 128, datagen.DT_F32, 0.02)
    print("noalloc call 2: B=3 T=333 H=4 dk=64 dv=128 fp32", flush=True)
    (o_a, h_a), (o_b, h_b) = both(d2, 32)
    assert torch.equal(o_a, o_b) and torch.equal(h_a, h_b)
    o_ref, h_ref = oracle.forward(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["h0"])
    assert o_err(host64(o_b), o_ref) < TOL[datagen.DT_F32] and state_err(host64(h_b), h_ref) < TOL[datagen.DT_F32]


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """A shape whose scratch exceeds the fixed buffer returns KDA_ERR_WORKSPACE before anything runs."""
    B, T, H, d, chunk = 4, 4096, 16, 128, 64
    assert kda.workspace_bytes(B, T, H, d, d, chunk) > kda.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros((B, T, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunked_forward_noalloc(x, x, x, x, beta, None, chunk=chunk)
    assert "KDA_ERR_WORKSPACE" in str(e.value)
    torch.cuda.synchronize()
