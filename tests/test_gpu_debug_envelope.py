"""The debug build (libkda_debug.so) against the release build, through the C ABI: inside the input
envelope (-5 <= g <= 0, 0 <= beta <= 1) every entry point returns KDA_OK with results bitwise
equal to the release build's (the same kernels run; the check only reads g and beta); one element
outside it (g below -5 or above 0, beta above 1, a NaN) returns KDA_ERR_ENVELOPE before anything
else is enqueued, so the outputs keep what they held.  A fused gate's pre-activation is not a
log-decay and is not checked (the fused gate keeps g in [-gate_scale, 0])."""
import ctypes

import pytest
import torch

import datagen
from tests.kda_testlib import dev_tensor

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

OK, ENVELOPE = 0, 5
SENTINEL = 7.0


def stream():
    return torch.cuda.current_stream().cuda_stream


def inputs(seed, B, T, H, d, dt):
    x = datagen.prefill_inputs(seed, B, T, H, d, d, dt, 0.02)
    return {key: dev_tensor(x[key]) for key in ("q", "k", "v", "g", "beta", "h0")}


def dtc(t):
    return kda.KDA_F32 if t.dtype == torch.float32 else kda.KDA_BF16


def forward(lib, t, chunk=64):
    """kda_chunked_forward of the library `lib`: (status, o, hT); o and hT start at SENTINEL."""
    B, T, H, d = t["q"].shape
    o = torch.full_like(t["v"], SENTINEL)
    hT = torch.full((B, H, d, d), SENTINEL, device="cuda")
    need = kda.workspace_bytes(B, T, H, d, d, chunk, t["q"].dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = lib.kda_chunked_forward(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["g"].data_ptr(),
                                 t["beta"].data_ptr(), t["h0"].data_ptr(), o.data_ptr(), hT.data_ptr(), B, T, H, d, d,
                                 chunk, dtc(t["q"]), ws.data_ptr(), need, stream())
    torch.cuda.synchronize()
    return st, o, hT


@pytest.mark.parametrize("dt", [datagen.DT_BF16, datagen.DT_F32])
def test_prefill_inside_envelope_equals_release(dt):
    t = inputs(9100 + dt, 2, 300, 2, 64, dt)
    t["g"][0, 5, 1, :] = -5.0  # the bound itself is inside
    t["beta"][1, 7, 0] = 1.0
    t["beta"][1, 8, 0] = 0.0
    print("debug build, prefill in envelope, dt=%d" % dt, flush=True)
    sa, oa, ha = forward(kda.lib(), t)
    sb, ob, hb = forward(kda.debug_lib(), t)
    assert sa == OK and sb == OK
    assert torch.equal(oa, ob) and torch.equal(ha, hb)


@pytest.mark.parametrize("where,value", [("g", -5.25), ("g", 0.125), ("g", float("nan")), ("beta", 1.25),
                                         ("beta", -0.25), ("beta", float("inf"))])
def test_prefill_outside_envelope_is_reported(where, value):
    t = inputs(9200, 2, 300, 2, 64, datagen.DT_BF16)
    if where == "g":
        t["g"][1, 299, 1, 63] = value  # the last element of the tensor
    else:
        t["beta"][0, 0, 0] = value     # the first
    print("debug build, prefill with %s = %r" % (where, value), flush=True)
    st, o, hT = forward(kda.debug_lib(), t)
    assert st == ENVELOPE
    assert bool((o == SENTINEL).all()) and bool((hT == SENTINEL).all())  # nothing was enqueued
    st_rel, _, _ = forward(kda.lib(), t)
    assert st_rel == OK  # the release build does not check


def test_fused_gate_preactivation_is_not_checked():
    t = inputs(9300, 1, 200, 2, 64, datagen.DT_BF16)
    x = torch.randn(t["g"].shape, device="cuda").to(torch.bfloat16) * 50  # far outside [-5, 0]: a pre-activation
    fu = kda.Fusion(gate_x=x.data_ptr(), gate_scale=5.0, normalize_qk=0, out_gate=None)
    outs = []
    for lib in (kda.lib(), kda.debug_lib()):
        o = torch.full_like(t["v"], SENTINEL)
        hT = torch.full((1, 2, 64, 64), SENTINEL, device="cuda")
        need = kda.workspace_bytes(1, 200, 2, 64, 64, 64, torch.bfloat16)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        st = lib.kda_chunked_forward_fused(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), None,
                                           t["beta"].data_ptr(), t["h0"].data_ptr(), o.data_ptr(), hT.data_ptr(),
                                           ctypes.byref(fu), 1, 200, 2, 64, 64, 64, kda.KDA_BF16, ws.data_ptr(), need,
                                           stream())
        torch.cuda.synchronize()
        assert st == OK
        outs.append((o, hT))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    t["beta"][0, 3, 1] = 2.0  # beta is still checked
    st = kda.debug_lib().kda_chunked_forward_fused(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), None,
                                                   t["beta"].data_ptr(), t["h0"].data_ptr(), o.data_ptr(),
                                                   hT.data_ptr(), ctypes.byref(fu), 1, 200, 2, 64, 64, 64,
                                                   kda.KDA_BF16, ws.data_ptr(), need, stream())
    torch.cuda.synchronize()
    assert st == ENVELOPE


def test_varlen_and_backward_report():
    t = inputs(9400, 1, 500, 2, 64, datagen.DT_BF16)
    t["g"][0, 250, 0, 10] = -6.0
    cu = torch.tensor([0, 100, 500], dtype=torch.int32, device="cuda")
    o = torch.full_like(t["v"], SENTINEL)
    hT = torch.zeros((2, 2, 64, 64), device="cuda")
    h0 = torch.zeros((2, 2, 64, 64), device="cuda")
    need = kda.varlen_workspace_bytes(2, 500, 400, 2, 64, 64, 64, torch.bfloat16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    dbg = kda.debug_lib()
    st = dbg.kda_chunked_forward_varlen(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["g"].data_ptr(),
                                        t["beta"].data_ptr(), h0.data_ptr(), o.data_ptr(), hT.data_ptr(),
                                        cu.data_ptr(), 2, 500, 400, 2, 64, 64, 64, kda.KDA_BF16, ws.data_ptr(), need,
                                        stream())
    torch.cuda.synchronize()
    assert st == ENVELOPE and bool((o == SENTINEL).all())
    grads = [torch.full_like(t[key], SENTINEL) for key in ("q", "k", "v", "g", "beta")]
    dh0 = torch.full((1, 2, 64, 64), SENTINEL, device="cuda")
    do = torch.randn_like(t["v"].float()).to(torch.bfloat16)
    need = kda.backward_workspace_bytes(1, 500, 2, 64, 64, 64, torch.bfloat16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = dbg.kda_chunked_backward(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["g"].data_ptr(),
                                  t["beta"].data_ptr(), t["h0"].data_ptr(), do.data_ptr(), None,
                                  *[x.data_ptr() for x in grads], dh0.data_ptr(), 1, 500, 2, 64, 64, 64,
                                  kda.KDA_BF16, ws.data_ptr(), need, stream())
    torch.cuda.synchronize()
    assert st == ENVELOPE and all(bool((x == SENTINEL).all()) for x in grads)


@pytest.mark.parametrize("dt", [datagen.DT_BF16, datagen.DT_F32])
def test_decode_step(dt):
    B, H, d = 4, 3, 64
    tdt = torch.float32 if dt == datagen.DT_F32 else torch.bfloat16
    q = torch.randn((B, H, d), device="cuda").to(tdt)
    k = torch.nn.functional.normalize(torch.randn((B, H, d), device="cuda"), dim=-1).to(tdt)
    v = torch.randn((B, H, d), device="cuda").to(tdt)
    g = (-5 * torch.rand((B, H, d), device="cuda")).to(tdt)
    beta = torch.rand((B, H), device="cuda").to(tdt)
    s0 = torch.randn((B, H, d, d), device="cuda") * 0.02
    res = []
    for lib in (kda.lib(), kda.debug_lib()):
        s = s0.clone()
        o = torch.full_like(v, SENTINEL)
        st = lib.kda_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), s.data_ptr(),
                                 o.data_ptr(), B, H, d, d, dtc(q), stream())
        torch.cuda.synchronize()
        assert st == OK
        res.append((s, o))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    g[2, 1, 0] = -7.0
    s = s0.clone()
    o = torch.full_like(v, SENTINEL)
    st = kda.debug_lib().kda_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                         s.data_ptr(), o.data_ptr(), B, H, d, d, dtc(q), stream())
    torch.cuda.synchronize()
    assert st == ENVELOPE and torch.equal(s, s0) and bool((o == SENTINEL).all())
