"""The C ABI without a GPU: libkda.so loads, exports every entry point include/kda.h declares,
and rejects invalid calls synchronously (before anything would be launched)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

kda = pytest.importorskip("gated_delta_rule_94_amd", reason="libkda.so not built")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 7
    lib = ctypes.CDLL(kda.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(kda.EXPORTS)


def test_debug_build_exports_and_flag():
    """libkda_debug.so (the debug build: envelope checks) exports the same entry points; only it
    reports debug checks."""
    dbg = ctypes.CDLL(kda.DEBUG_LIB_PATH)
    for name in declared_functions():
        assert hasattr(dbg, name), name
    assert kda.lib().kda_debug_checks() == 0
    assert kda.debug_lib().kda_debug_checks() == 1
    assert "envelope" in kda.kda_status_string(5)
    assert kda.STATUS[5] == "KDA_ERR_ENVELOPE"


def test_status_strings_and_version():
    assert kda.kda_status_string(0) == "ok"
    assert "invalid" in kda.kda_status_string(1)
    assert "unsupported" in kda.kda_status_string(2)
    assert kda.kda_status_string(99) == "unknown status"
    assert kda.kda_version() >= 200


def test_workspace_queries():
    lib = kda.lib()
    # one record per (chunk, head): -W, Q.Gamma, K'^T, P, U~ in bf16 plus e^{G_last} in fp32
    rec = 2 * (3 * 64 * 128 + 64 * 64 + 64 * 128) + 4 * 128
    rec = (rec + 255) // 256 * 256
    assert lib.kda_chunked_forward_workspace_bytes(4, 4096, 16, 128, 128, 64, 1) == 4 * 64 * 16 * rec
    assert lib.kda_chunked_forward_workspace_bytes(1, 100, 2, 128, 128, 64, 1) == 2 * 2 * rec  # ragged tail
    # packed: at most floor(T_total / C) + N chunks, plus the chunk map and the longest-first order
    n = lib.kda_chunked_forward_varlen_workspace_bytes(16, 1 << 20, 131072, 8, 128, 128, 64, 1)
    assert n == ((1 << 20) // 64 + 16) * 8 * rec + 256 + 256
    assert lib.kda_chunked_forward_workspace_bytes(0, 10, 2, 64, 64, 64, 1) == 0
    assert lib.kda_chunked_forward_workspace_bytes(1, 10, 2, 64, 64, 48, 1) == 0  # unsupported chunk


def test_chain_plan_and_segment_workspace():
    """The chain layout for 256 compute units (the count assumed without a device, and MI355X's):
    whole sequences in 16- or 32-column slices when (sequence, head, 32-column slice) fill the CUs
    or the sequences are too short to split; otherwise every sequence split into enough segments of
    at least 32 chunks to fill them -- for bf16 with 64-token chunks (the wide chain kernel) in the
    widest slice, up to d_v, that allows it.  The workspace grows by the segment start states and
    summaries."""
    f32 = torch.float32
    assert kda.chain_plan(4, 4096, 16, 128, 128) == (32, 1, 0)          # 256 workgroups already
    assert kda.chain_plan(1, 2048, 8, 128, 128) == (16, 1, 0)           # 32 chunks: too short to split
    assert kda.chain_plan(1, 1024, 8, 128, 128, chunk=32) == (16, 1, 0)
    assert kda.chain_plan(1, 4096, 8, 128, 128) == (32, 2, 32)
    assert kda.chain_plan(1, 65536, 32, 128, 128) == (128, 8, 128)      # 32 heads x 8 segments, whole states
    assert kda.chain_plan(1, 1 << 20, 8, 128, 128) == (128, 32, 512)    # 8 heads x 32 segments
    assert kda.summary_slice(1, 1 << 20, 8, 128, 128) == 256            # value and identity columns together
    assert kda.chain_plan(1, 8229, 2, 128, 128) == (32, 4, 33)          # ragged: 129 chunks, last segment 30
    assert kda.chain_plan(1, 8229, 2, 128, 128, chunk=32) == (32, 8, 33)
    assert kda.chain_plan(1, 6400, 1, 64, 64, dtype=f32) == (16, 3, 34)
    assert kda.chain_plan(1, 6400, 1, 128, 128, dtype=f32) == (16, 3, 34)  # fp32 records at d_k 128, chunk 64
    lib = kda.lib()
    rec = 2 * (3 * 64 * 128 + 64 * 64 + 64 * 128) + 4 * 128
    rec = (rec + 255) // 256 * 256
    al = lambda x: (x + 255) // 256 * 256
    units, nseg = 8, 32
    want = 16384 * 8 * rec + al(units * nseg * 128 * 128 * 4) + al(units * (nseg - 1) * 128 * 256 * 4)
    assert lib.kda_chunked_forward_workspace_bytes(1, 1 << 20, 8, 128, 128, 64, 1) == want


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced because validation fails first


def fwd(B=1, T=64, H=2, dk=64, dv=64, chunk=64, dt=1, ptr=FAKE, h0=None, hT=None, ws=FAKE, ws_bytes=1 << 40):
    return kda.lib().kda_chunked_forward(ptr, ptr, ptr, ptr, ptr, h0, ptr, hT, B, T, H, dk, dv, chunk, dt, ws, ws_bytes,
                                         None)


def test_prefill_validation():
    assert fwd(ptr=None) == INVALID
    assert fwd(ptr=FAKE + 4) == INVALID  # misaligned
    assert fwd(B=-1) == INVALID
    assert fwd(T=-1) == INVALID
    assert fwd(H=0) == INVALID
    assert fwd(dt=7) == INVALID
    assert fwd(dk=96) == UNSUPPORTED
    assert fwd(dv=32) == UNSUPPORTED
    assert fwd(chunk=48) == UNSUPPORTED
    assert fwd(chunk=128) == UNSUPPORTED
    assert fwd(h0=FAKE + 8) == INVALID
    # workspace missing, too small or misaligned
    need = kda.lib().kda_chunked_forward_workspace_bytes(1, 64, 2, 64, 64, 64, 1)
    assert fwd(ws=None) == 3
    assert fwd(ws_bytes=need - 1) == 3
    assert fwd(ws=FAKE + 16, ws_bytes=need) == 3
    # empty batch: nothing to do, null tensors allowed
    assert fwd(B=0, ptr=None, ws=None, ws_bytes=0) == OK


def fna(B=1, T=64, H=2, dk=64, dv=64, chunk=64, dt=1, ptr=FAKE, h0=None, hT=None):
    return kda.lib().kda_chunked_forward_noalloc(ptr, ptr, ptr, ptr, ptr, h0, ptr, hT, B, T, H, dk, dv, chunk, dt, None)


def test_noalloc_validation():
    """The no-allocation prefill checks its arguments as kda_chunked_forward does, and refuses, before
    anything runs, a shape whose scratch exceeds the library's fixed buffer."""
    assert fna(ptr=None) == INVALID
    assert fna(ptr=FAKE + 4) == INVALID
    assert fna(B=-1) == INVALID
    assert fna(dk=96) == UNSUPPORTED
    assert fna(chunk=48) == UNSUPPORTED
    assert fna(h0=FAKE + 8) == INVALID
    assert fna(B=0, ptr=None) == OK
    big = kda.lib().kda_chunked_forward_workspace_bytes(4, 4096, 16, 128, 128, 64, 1)
    assert big > kda.NOALLOC_SCRATCH_BYTES
    assert fna(B=4, T=4096, H=16, dk=128, dv=128) == 3
    header = open(os.path.join(ROOT, "include", "kda.h")).read()
    assert "#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in header
    assert kda.NOALLOC_SCRATCH_BYTES == 64 << 20


def fmx(B=1, T=64, H=2, dk=64, dv=64, chunk=64, ptr=FAKE, scale=FAKE + 1, h0=None, hT=None, ws=FAKE, ws_bytes=1 << 40):
    return kda.lib().kda_chunked_forward_mxfp8(ptr, scale, ptr, scale, ptr, scale, ptr, ptr, h0, ptr, hT, B, T, H, dk,
                                               dv, chunk, ws, ws_bytes, None)


def test_mxfp8_validation():
    """MXFP8 q, k, v: the bf16 shapes and checks, plus non-NULL scale pointers (any alignment)."""
    assert fmx(scale=None) == INVALID
    assert fmx(ptr=FAKE + 8) == INVALID  # misaligned codes
    assert fmx(ptr=None) == INVALID
    assert fmx(B=-1) == INVALID
    assert fmx(dk=96) == UNSUPPORTED
    assert fmx(chunk=128) == UNSUPPORTED
    need = kda.lib().kda_chunked_forward_workspace_bytes(1, 64, 2, 64, 64, 64, 1)
    assert fmx(ws=None) == 3
    assert fmx(ws_bytes=need - 1) == 3
    assert fmx(B=0, ptr=None, scale=None, ws=None, ws_bytes=0) == OK
    assert fmx(T=0, ptr=None, scale=None, ws=None, ws_bytes=0) == OK  # nothing to read and no hT


def test_states_validation():
    """Snapshot arguments are checked before anything would run: a 16-byte-aligned buffer and an
    interval that is a positive multiple of the chunk; a NULL buffer ignores the interval."""
    lib = kda.lib()

    def fs(states=FAKE, every=128, chunk=64, ws=FAKE):
        return lib.kda_chunked_forward_with_states(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, states, every,
                                                   1, 256, 2, 64, 64, chunk, 1, ws, 1 << 40, None)

    def fv(states=FAKE, every=128, chunk=64):
        return lib.kda_chunked_forward_varlen_with_states(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, states,
                                                          every, FAKE, 2, 256, 200, 2, 64, 64, chunk, 1, None, 0,
                                                          None)

    assert fs(every=96) == INVALID       # not a multiple of the chunk
    assert fs(every=0) == INVALID
    assert fs(every=-64) == INVALID
    assert fs(states=FAKE + 4) == INVALID  # misaligned
    assert fs(states=None, every=0, ws=None) == 3  # a NULL buffer ignores the interval (then: no workspace)
    assert fv(every=96) == INVALID
    assert fv(states=FAKE + 8) == INVALID


def test_fused_validation():
    """The fused steps are checked before anything would run: a gate scale in (0, 5] with a gate
    pre-activation (g itself may then be NULL), aligned pointers."""
    lib = kda.lib()

    def ff(gate_x=FAKE, scale=5.0, norm=1, out_gate=FAKE, g=None, ws=FAKE):
        fu = kda.Fusion(gate_x, scale, norm, out_gate)
        return lib.kda_chunked_forward_fused(FAKE, FAKE, FAKE, g, FAKE, None, FAKE, None, ctypes.byref(fu),
                                             1, 256, 2, 64, 64, 64, 1, ws, 1 << 40, None)

    def fd(gate_x=FAKE, scale=5.0, out_gate=FAKE, g=None):
        fu = kda.Fusion(gate_x, scale, 0, out_gate)
        return lib.kda_decode_step_fused(FAKE, FAKE, FAKE, g, FAKE, FAKE, FAKE, ctypes.byref(fu), 0, 2, 64, 64, 1,
                                         None)

    assert ff(scale=0.0) == INVALID
    assert ff(scale=5.5) == INVALID
    assert ff(scale=-1.0) == INVALID
    assert ff(gate_x=FAKE + 2) == INVALID
    assert ff(out_gate=FAKE + 4) == INVALID
    assert ff(gate_x=None, g=None) == INVALID      # no gate at all
    assert ff(ws=None) == 3                        # valid arguments (g NULL with gate_x): then no workspace
    assert ff(gate_x=None, g=FAKE, scale=0.0, ws=None) == 3  # no gate pre-activation: the scale is ignored
    assert fd(scale=6.0) == INVALID
    assert fd() == OK                              # B = 0: nothing to do
    nofu = lib.kda_chunked_forward_fused(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, 1, 256, 2, 64, 64,
                                         64, 1, None, 0, None)
    assert nofu == 3                               # a NULL fusion is the plain call


def test_varlen_validation():
    lib = kda.lib()
    call = lambda cu, N, Tt, ms, ptr=FAKE: lib.kda_chunked_forward_varlen(ptr, ptr, ptr, ptr, ptr, None, ptr, None,
                                                                         cu, N, Tt, ms, 2, 64, 64, 64, 1, FAKE,
                                                                         1 << 40, None)
    assert call(None, 2, 100, 60) == INVALID       # missing cu_seqlens
    assert call(FAKE, -1, 100, 60) == INVALID
    assert call(FAKE, 2, 100, 101) == INVALID      # max_seqlen beyond T_total
    assert call(FAKE, 2, 100, 60, ptr=None) == INVALID
    assert call(None, 0, 0, 0, ptr=None) == OK     # nothing to do
    assert lib.kda_chunked_forward_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 2, 100, 60, 2, 64, 64,
                                          64, 1, FAKE, 10, None) == 3  # workspace too small


def test_decode_validation():
    lib = kda.lib()
    call = lambda B=2, H=2, dk=64, dv=64, dt=1, ptr=FAKE: lib.kda_decode_step(ptr, ptr, ptr, ptr, ptr, ptr, ptr, B, H,
                                                                             dk, dv, dt, None)
    assert call(ptr=None) == INVALID
    assert call(ptr=FAKE + 2) == INVALID
    assert call(H=0) == INVALID
    assert call(dk=32) == UNSUPPORTED
    assert call(dt=3) == INVALID
    assert call(B=0, ptr=None) == OK


def test_backward_segment_workspace():
    """Long sequences on few heads segment the adjoint chain (as the forward chain): the backward
    workspace then also holds every segment's end adjoint and the segment summaries.  The per-chunk
    states and adjoints are kept in the operand type (bf16 here); the segment adjoints in fp32."""
    lib = kda.lib()
    al = lambda x: (x + 255) // 256 * 256
    B, T, H, d, C = 1, 16401, 8, 128, 64
    nch, units = (T + C - 1) // C, B * H
    fwd = al(lib.kda_chunked_forward_workspace_bytes(B, T, H, d, d, C, 1))
    grad = ((C * d + C * C + 3 * C * d + d + 63) // 64) * 64
    base = fwd + 2 * al(units * nch * d * d * 2) + al(units * nch * grad * 4) + al(B * T * H * d * 2)
    nseg = 8  # 8 heads x 4 slices of 32 columns: 32 workgroups, 257 chunks -> 8 segments of 33
    seg = al(units * nseg * d * d * 4) + al(units * (nseg - 1) * d * 2 * d * 4)
    assert lib.kda_chunked_backward_workspace_bytes(B, T, H, d, d, C, 1) == base + seg
    # 16 heads x 4 sequences fill the CUs: no segments
    B, T, H = 4, 4096, 16
    nch, units = T // C, B * H
    fwd = al(lib.kda_chunked_forward_workspace_bytes(B, T, H, d, d, C, 1))
    base = fwd + 2 * al(units * nch * d * d * 2) + al(units * nch * grad * 4) + al(B * T * H * d * 2)
    assert lib.kda_chunked_backward_workspace_bytes(B, T, H, d, d, C, 1) == base


def test_backward_workspace_and_validation():
    lib = kda.lib()
    rec = 2 * (3 * 64 * 128 + 64 * 64 + 64 * 128) + 4 * 128
    rec = (rec + 255) // 256 * 256
    al = lambda x: (x + 255) // 256 * 256
    B, T, H, D, C = 4, 4096, 16, 128, 64
    nch, units = T // C, B * H
    grad = (C * D + C * C + 3 * C * D + D + 63) // 64 * 64  # dU, dP, d(Q Gamma), dKd, dW, dgl (fp32)
    # records, the state after every chunk and the adjoint at every chunk end (both per (chunk, head)
    # record slot, in the operand type: bf16 here), the state products, an o scratch
    want = (al(B * nch * H * rec) + 2 * al(units * nch * D * D * 2) + al(units * nch * grad * 4)
            + al(B * T * H * D * 2))
    assert lib.kda_chunked_backward_workspace_bytes(B, T, H, D, D, C, 1) == want
    assert lib.kda_chunked_backward_workspace_bytes(1, 100, 2, 128, 128, 48, 1) == 0  # unsupported chunk
    assert lib.kda_chunked_backward_workspace_bytes(1, 100, 2, 128, 128, 64, 0) > 0  # fp32 at every d
    assert lib.kda_chunked_backward_workspace_bytes(1, 100, 2, 64, 64, 64, 0) > 0
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation
    a = [fake] * 5 + [None, fake, None] + [fake] * 5 + [None]

    def call(args, B=1, T=100, H=2, dk=128, dv=128, chunk=64, dt=1, ws=None, nbytes=0):
        return lib.kda_chunked_backward(*args, B, T, H, dk, dv, chunk, dt, ws, nbytes, None)

    assert call(a, chunk=48) == UNSUPPORTED
    assert call(a, dk=96) == UNSUPPORTED
    assert call(a, dt=0) == 3                               # fp32 with d = 128: supported, no workspace
    assert call(a, B=-1) == INVALID
    assert call(a, dt=5) == INVALID
    bad = list(a)
    bad[8] = None                                           # dq missing
    assert call(bad) == INVALID
    bad = list(a)
    bad[9] = ctypes.c_void_p((1 << 20) + 4)                 # dk misaligned
    assert call(bad) == INVALID
    bad = list(a)
    bad[6] = None                                           # d_o missing
    assert call(bad) == INVALID
    assert call(a) == 3                                     # no workspace: KDA_ERR_WORKSPACE
    assert call(a, B=0) == OK
    assert call(a, T=0) == OK                               # nothing to do without dh0


def test_backward_varlen_workspace_and_validation():
    """The packed backward: workspace for a bound on the chunks (T_total / C + num_seqs) after the
    varlen forward's own (records and chunk map), and the varlen forward's argument checks plus the
    gradient buffers'."""
    lib = kda.lib()
    al = lambda x: (x + 255) // 256 * 256
    N, Tt, maxlen, H, D, C = 3, 1000, 600, 4, 128, 64
    mc = Tt // C + N
    grad = (C * D + C * C + 3 * C * D + D + 63) // 64 * 64
    fwd = al(lib.kda_chunked_forward_varlen_workspace_bytes(N, Tt, maxlen, H, D, D, C, 1))
    want = fwd + 2 * al(mc * H * D * D * 2) + al(mc * H * grad * 4) + al(Tt * H * D * 2)
    assert lib.kda_chunked_backward_varlen_workspace_bytes(N, Tt, maxlen, H, D, D, C, 1) == want
    assert lib.kda_chunked_backward_varlen_workspace_bytes(N, Tt, maxlen, H, D, D, 48, 1) == 0
    assert lib.kda_chunked_backward_varlen_workspace_bytes(N, Tt, maxlen, H, D, D, C, 0) > 0
    assert lib.kda_chunked_backward_varlen_workspace_bytes(N, Tt, maxlen, H, 64, 64, C, 0) > 0
    assert lib.kda_chunked_backward_varlen_workspace_bytes(0, Tt, maxlen, H, D, D, C, 1) == 0
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation
    a = [fake] * 5 + [None, fake, None] + [fake] * 5 + [None, fake]

    def call(args, N=3, Tt=1000, maxlen=600, H=4, dk=128, dv=128, chunk=64, dt=1, ws=None, nbytes=0):
        return lib.kda_chunked_backward_varlen(*args, N, Tt, maxlen, H, dk, dv, chunk, dt, ws, nbytes, None)

    assert call(a, chunk=48) == UNSUPPORTED
    assert call(a, dk=96) == UNSUPPORTED
    assert call(a, dt=0) == 3                               # fp32 with d = 128: supported, no workspace
    assert call(a, N=-1) == INVALID
    assert call(a, maxlen=1001) == INVALID                  # longer than T_total
    assert call(a, dt=5) == INVALID
    bad = list(a)
    bad[14] = None                                          # cu_seqlens missing
    assert call(bad) == INVALID
    bad = list(a)
    bad[8] = None                                           # dq missing
    assert call(bad) == INVALID
    assert call(a) == 3                                     # no workspace: KDA_ERR_WORKSPACE
    assert call(a, N=0) == OK
    assert call(a, Tt=0, maxlen=0) == OK                    # nothing to do without dh0


def test_training_step_buffers_and_validation():
    """kda_chunked_forward_train's saved buffer plus kda_chunked_backward_saved's workspace hold what
    kda_chunked_backward's workspace holds, less its recomputed o; invalid calls fail before launch."""
    lib = kda.lib()
    al = lambda x: (x + 255) // 256 * 256
    for (B, T, H, d, C, dt) in [(4, 4096, 16, 128, 64, 1), (1, 16401, 8, 128, 64, 1), (2, 300, 2, 64, 32, 0)]:
        saved = lib.kda_chunked_forward_train_saved_bytes(B, T, H, d, d, C, dt)
        own = lib.kda_chunked_backward_saved_workspace_bytes(B, T, H, d, d, C, dt)
        full = lib.kda_chunked_backward_workspace_bytes(B, T, H, d, d, C, dt)
        assert saved > 0 and own > 0
        assert saved + own + al(B * T * H * d * (4 if dt == 0 else 2)) == full
    assert lib.kda_chunked_forward_train_saved_bytes(1, 100, 2, 128, 128, 48, 1) == 0
    assert lib.kda_chunked_backward_saved_workspace_bytes(1, 100, 2, 96, 128, 64, 1) == 0
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation
    fwd = [fake] * 5 + [None, fake, fake]

    def train(args=fwd, B=1, T=100, H=2, dk=128, chunk=64, dt=1, saved=None, nbytes=0):
        return lib.kda_chunked_forward_train(*args, B, T, H, dk, dk, chunk, dt, saved, nbytes, None)

    assert train() == 3                            # no saved buffer: KDA_ERR_WORKSPACE
    assert train(chunk=48) == UNSUPPORTED
    assert train(B=-1) == INVALID
    assert train(B=0) == OK
    bad = list(fwd)
    bad[6] = None                                  # o missing
    assert train(bad) == INVALID
    need = lib.kda_chunked_forward_train_saved_bytes(1, 100, 2, 128, 128, 64, 1)
    assert train(saved=ctypes.c_void_p((1 << 20) + 16), nbytes=need) == 3  # misaligned saved buffer
    bwd = [fake] * 5 + [None, fake, None] + [fake] * 5 + [None]

    def back(args=bwd, B=1, T=100, H=2, dk=128, chunk=64, dt=1, saved=None, sbytes=0, ws=None, wbytes=0):
        return lib.kda_chunked_backward_saved(*args, B, T, H, dk, dk, chunk, dt, saved, sbytes, ws, wbytes, None)

    own = lib.kda_chunked_backward_saved_workspace_bytes(1, 100, 2, 128, 128, 64, 1)
    assert back() == 3                                                  # neither buffer
    assert back(saved=fake, sbytes=need) == 3                           # no workspace
    assert back(ws=fake, wbytes=own) == 3                               # no saved buffer
    assert back(saved=fake, sbytes=need - 256, ws=fake, wbytes=own) == 3
    assert back(chunk=48) == UNSUPPORTED
    bad = list(bwd)
    bad[8] = None                                                       # dq missing
    assert back(bad, saved=fake, sbytes=need, ws=fake, wbytes=own) == INVALID
    assert back(B=0) == OK
