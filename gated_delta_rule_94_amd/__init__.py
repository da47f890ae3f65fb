"""Kimi Delta Attention (KDA) on AMD Instinct MI355X -- Python binding of libkda.so.

Thin ctypes marshalling over the C ABI declared in ``include/kda.h``: every
step of the computation runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  The functions carry the C
entry points' names:

* ``kda_chunked_forward``        -- chunked prefill, B equal-length sequences
* ``kda_chunked_forward_varlen`` -- chunked prefill, packed sequences (cu_seqlens)
* ``kda_chunked_forward_with_states`` / ``kda_chunked_forward_varlen_with_states`` -- the same,
  also keeping the state every N tokens (prefix states for a serving cache)
* ``kda_decode_step``            -- one token per sequence, state updated in place
* ``kda_chunked_forward_fused`` / ``kda_decode_step_fused`` -- with the gate formed from its
  pre-activation, q and k normalised, and an output gate, inside the kernels
* ``kda_chunked_forward_ex`` / ``kda_chunked_forward_varlen_ex`` -- snapshots and fused steps together
* ``kda_chunked_backward`` / ``kda_chunked_backward_varlen`` -- gradients of the chunked prefill
  (training), equal-length or packed sequences
* ``kda_chunked_forward_train`` / ``kda_chunked_backward_saved`` -- a training step whose backward
  uses what the forward saved instead of recomputing it

Importing this package fails loudly when ``libkda.so`` has not been built
(``python gated_delta_rule_94_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libkda_debug.so")  # the debug build: input envelope checked

KDA_F32, KDA_BF16 = 0, 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_HIP",
          5: "KDA_ERR_ENVELOPE"}

# exported symbols of libkda.so (the C ABI)
EXPORTS = (
    "kda_status_string", "kda_version", "kda_chunked_forward_workspace_bytes", "kda_chunked_forward_plan",
    "kda_chunked_forward", "kda_chunked_forward_with_states", "kda_chunked_forward_varlen_with_states",
    "kda_chunked_forward_fused", "kda_decode_step_fused", "kda_chunked_forward_ex", "kda_chunked_forward_varlen_ex",
    "kda_chunked_forward_profiled", "kda_chunked_forward_varlen", "kda_chunked_forward_varlen_workspace_bytes",
    "kda_decode_step", "kda_chunked_backward", "kda_chunked_backward_workspace_bytes", "kda_chunked_forward_mxfp8",
    "kda_chunked_forward_noalloc", "kda_chunked_backward_varlen", "kda_chunked_backward_varlen_workspace_bytes",
    "kda_debug_checks", "kda_chunked_forward_train", "kda_chunked_forward_train_saved_bytes",
    "kda_chunked_backward_saved", "kda_chunked_backward_saved_workspace_bytes",
)

# bytes of the library's fixed device scratch used by kda_chunked_forward_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

if not os.path.exists(LIB_PATH):
    raise ImportError("libkda.so is not built (%s): run `python gated_delta_rule_94_amd/build.py`" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


class Fusion(ctypes.Structure):
    """kda_fusion: gate pre-activation (g = -gate_scale * sigmoid(gate_x)), q/k normalisation, output gate."""
    _fields_ = [("gate_x", _vp), ("gate_scale", ctypes.c_float), ("normalize_qk", _i32), ("out_gate", _vp)]


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Argument and result types of every entry point (the same for the release and debug builds)."""
    lib.kda_status_string.argtypes = [_i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = _i32
    lib.kda_chunked_forward_workspace_bytes.argtypes = [_i32] * 7
    lib.kda_chunked_forward_workspace_bytes.restype = _sz
    lib.kda_chunked_forward_plan.argtypes = [_i32] * 7 + [_vp] * 4
    lib.kda_chunked_forward_plan.restype = _i32
    lib.kda_chunked_forward_varlen_workspace_bytes.argtypes = [_i32] * 8
    lib.kda_chunked_forward_varlen_workspace_bytes.restype = _sz
    lib.kda_chunked_forward.argtypes = [_vp] * 8 + [_i32] * 7 + [_vp, _sz, _vp]
    lib.kda_chunked_forward.restype = _i32
    lib.kda_chunked_forward_noalloc.argtypes = [_vp] * 8 + [_i32] * 7 + [_vp]
    lib.kda_chunked_forward_noalloc.restype = _i32
    lib.kda_chunked_forward_with_states.argtypes = [_vp] * 9 + [_i32] * 8 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_with_states.restype = _i32
    lib.kda_chunked_forward_varlen_with_states.argtypes = [_vp] * 9 + [_i32, _vp] + [_i32] * 8 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_varlen_with_states.restype = _i32
    lib.kda_chunked_forward_profiled.argtypes = [_vp] * 8 + [_i32] * 7 + [_vp, _sz, _vp, _vp]
    lib.kda_chunked_forward_profiled.restype = _i32
    lib.kda_chunked_forward_varlen.argtypes = [_vp] * 8 + [_vp] + [_i32] * 8 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_varlen.restype = _i32
    lib.kda_chunked_forward_mxfp8.argtypes = [_vp] * 11 + [_i32] * 6 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_mxfp8.restype = _i32
    lib.kda_decode_step.argtypes = [_vp] * 7 + [_i32] * 4 + [_i32, _vp]
    lib.kda_decode_step.restype = _i32
    lib.kda_chunked_forward_fused.argtypes = [_vp] * 8 + [ctypes.POINTER(Fusion)] + [_i32] * 7 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_fused.restype = _i32
    lib.kda_decode_step_fused.argtypes = [_vp] * 7 + [ctypes.POINTER(Fusion)] + [_i32] * 5 + [_vp]
    lib.kda_decode_step_fused.restype = _i32
    lib.kda_chunked_forward_ex.argtypes = [_vp] * 9 + [_i32, ctypes.POINTER(Fusion)] + [_i32] * 7 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_ex.restype = _i32
    lib.kda_chunked_forward_varlen_ex.argtypes = ([_vp] * 9 + [_i32, ctypes.POINTER(Fusion), _vp] + [_i32] * 8 +
                                                   [_vp, _sz, _vp])
    lib.kda_chunked_forward_varlen_ex.restype = _i32
    lib.kda_chunked_backward_workspace_bytes.argtypes = [_i32] * 7
    lib.kda_chunked_backward_workspace_bytes.restype = _sz
    lib.kda_chunked_backward.argtypes = [_vp] * 14 + [_i32] * 7 + [_vp, _sz, _vp]
    lib.kda_chunked_backward.restype = _i32
    lib.kda_chunked_backward_varlen_workspace_bytes.argtypes = [_i32] * 8
    lib.kda_chunked_backward_varlen_workspace_bytes.restype = _sz
    lib.kda_chunked_backward_varlen.argtypes = [_vp] * 15 + [_i32] * 8 + [_vp, _sz, _vp]
    lib.kda_chunked_backward_varlen.restype = _i32
    lib.kda_debug_checks.argtypes = []
    lib.kda_debug_checks.restype = _i32
    lib.kda_chunked_forward_train_saved_bytes.argtypes = [_i32] * 7
    lib.kda_chunked_forward_train_saved_bytes.restype = _sz
    lib.kda_chunked_forward_train.argtypes = [_vp] * 8 + [_i32] * 7 + [_vp, _sz, _vp]
    lib.kda_chunked_forward_train.restype = _i32
    lib.kda_chunked_backward_saved_workspace_bytes.argtypes = [_i32] * 7
    lib.kda_chunked_backward_saved_workspace_bytes.restype = _sz
    lib.kda_chunked_backward_saved.argtypes = [_vp] * 14 + [_i32] * 7 + [_vp, _sz, _vp, _sz, _vp]
    lib.kda_chunked_backward_saved.restype = _i32
    return lib


_declare(_lib)
_debug_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), kda_status_string(status)))
        self.status = status


def kda_status_string(status: int) -> str:
    return _lib.kda_status_string(int(status)).decode()


def kda_version() -> int:
    return int(_lib.kda_version())


def lib() -> ctypes.CDLL:
    """The loaded libkda.so (for callers that marshal arguments themselves)."""
    return _lib


def debug_lib() -> ctypes.CDLL:
    """The debug build, libkda_debug.so, loaded on first use: the same C ABI with every entry point
    first checking g and beta against the input envelope (KDA_ERR_ENVELOPE on a violation; one
    stream synchronisation per call).  Callers marshal arguments themselves, as with lib()."""
    global _debug_lib
    if _debug_lib is None:
        if not os.path.exists(DEBUG_LIB_PATH):
            raise ImportError("libkda_debug.so is not built (%s): run `python gated_delta_rule_94_amd/build.py`"
                              % DEBUG_LIB_PATH)
        _debug_lib = _declare(ctypes.CDLL(DEBUG_LIB_PATH))
    return _debug_lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError("KDA inputs must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _workspace(ws, nbytes, dev):
    if ws is not None:
        if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != dev:
            raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None


def _nbytes(ws):
    return 0 if ws is None else ws.numel()


def workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Device workspace kda_chunked_forward needs for this shape."""
    return int(_lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(torch.empty(0, dtype=dtype))))


def _plan(B, T, H, dk, dv, chunk, dtype):
    out = (ctypes.c_int * 4)()
    addr = ctypes.addressof(out)
    st = _lib.kda_chunked_forward_plan(B, T, H, dk, dv, chunk, _dtype_code(torch.empty(0, dtype=dtype)),
                                       addr, addr + 4, addr + 8, addr + 12)
    if st != 0:
        raise KDAError("kda_chunked_forward_plan", st)
    return tuple(int(x) for x in out)


def chain_plan(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16):
    """(value_slice, segments, segment_chunks): how kda_chunked_forward lays out its state chain on
    the current device for this shape."""
    return _plan(B, T, H, dk, dv, chunk, dtype)[:3]


def summary_slice(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16):
    """State columns per workgroup of the segment summary pass for this shape (0: no segments)."""
    return _plan(B, T, H, dk, dv, chunk, dtype)[3]


def varlen_workspace_bytes(num_seqs, T_total, max_seqlen, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Device workspace kda_chunked_forward_varlen needs for this shape."""
    return int(_lib.kda_chunked_forward_varlen_workspace_bytes(num_seqs, T_total, max_seqlen, H, dk, dv, chunk,
                                                                _dtype_code(torch.empty(0, dtype=dtype))))


def _check(name, t, shape, dtype=None, device=None):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))


def kda_chunked_forward(q, k, v, g, beta, h0=None, *, chunk: int = 64, o=None, hT=None, want_hT: bool = True,
                        workspace=None, stream=None):
    """Chunked prefill.  q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H] (one dtype, float32 or
    bfloat16); h0 [B,H,dk,dv] float32 or None.  Returns (o [B,T,H,dv], hT [B,H,dk,dv] float32 or None).
    o / hT may be passed preallocated; hT may be h0 (updated in place).  workspace: a uint8 device
    tensor of at least kda_chunked_forward_workspace_bytes(...) bytes, or None to allocate one."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    st = _lib.kda_chunked_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                  B, T, H, dk, dv, chunk, _dtype_code(q), _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward", st)
    return o, hT


def kda_chunked_forward_noalloc(q, k, v, g, beta, h0=None, *, chunk: int = 64, o=None, hT=None, want_hT: bool = True,
                                stream=None):
    """kda_chunked_forward with no workspace: the library's fixed device scratch (NOALLOC_SCRATCH_BYTES,
    one per GPU) holds the per-chunk records, and the C call allocates nothing.  Pass o (and hT) to
    make the whole call allocation-free; calls that overlap on one GPU race on the scratch."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    st = _lib.kda_chunked_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                          B, T, H, dk, dv, chunk, _dtype_code(q), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_noalloc", st)
    return o, hT


def kda_chunked_forward_mxfp8(q, q_scale, k, k_scale, v, v_scale, g, beta, h0=None, *, chunk: int = 64, o=None,
                              hT=None, want_hT: bool = True, workspace=None, stream=None):
    """Chunked prefill with MXFP8 q, k, v: q, k [B,T,H,dk] and v [B,T,H,dv] uint8 E4M3 codes;
    q_scale, k_scale [B,T,H,dk//32] and v_scale [B,T,H,dv//32] uint8 E8M0 scale codes (one per 32
    channels); g [B,T,H,dk] and beta [B,T,H] bfloat16; h0 [B,H,dk,dv] float32 or None.  Returns
    (o [B,T,H,dv] bfloat16, hT float32 or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    u8, bf = torch.uint8, torch.bfloat16
    for name, t, shp, dt in (("q", q, (B, T, H, dk), u8), ("k", k, (B, T, H, dk), u8), ("v", v, (B, T, H, dv), u8),
                             ("q_scale", q_scale, (B, T, H, dk // 32), u8), ("k_scale", k_scale, (B, T, H, dk // 32), u8),
                             ("v_scale", v_scale, (B, T, H, dv // 32), u8), ("g", g, (B, T, H, dk), bf),
                             ("beta", beta, (B, T, H), bf)):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=bf, device=dev)
    _check("o", o, (B, T, H, dv), bf, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, KDA_BF16)
    ws = _workspace(workspace, ws_bytes, dev)
    st = _lib.kda_chunked_forward_mxfp8(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale),
                                        _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), B, T, H, dk, dv, chunk,
                                        _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_mxfp8", st)
    return o, hT


def kda_chunked_forward_with_states(q, k, v, g, beta, h0=None, *, state_every: int, chunk: int = 64, o=None,
                                    hT=None, states=None, want_hT: bool = True, workspace=None, stream=None):
    """kda_chunked_forward that also returns the state after every state_every tokens (a positive
    multiple of chunk): states [B,H,T//state_every,dk,dv] float32, entry j = the state after the
    first (j+1)*state_every tokens.  Returns (o, hT, states)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    n_states = T // state_every if state_every > 0 else 0
    if states is None:
        states = torch.empty((B, H, n_states, dk, dv), dtype=torch.float32, device=dev)
    _check("states", states, (B, H, n_states, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    st = _lib.kda_chunked_forward_with_states(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                              _ptr(hT), _ptr(states), int(state_every), B, T, H, dk, dv, chunk,
                                              _dtype_code(q), _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_with_states", st)
    return o, hT, states


def _fusion(gate_x, gate_scale, normalize_qk, out_gate):
    return Fusion(_ptr(gate_x), float(gate_scale), 1 if normalize_qk else 0, _ptr(out_gate))


def kda_chunked_forward_fused(q, k, v, g, beta, h0=None, *, gate_x=None, gate_scale: float = 5.0,
                              normalize_qk: bool = False, out_gate=None, chunk: int = 64, o=None, hT=None,
                              want_hT: bool = True, workspace=None, stream=None):
    """kda_chunked_forward with the fused steps: gate_x (like g) gives g = -gate_scale * sigmoid(gate_x)
    and g is then not read (may be None); normalize_qk L2-normalises q and k over d_k; out_gate (like o)
    multiplies o elementwise.  Returns (o, hT)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("gate_x", gate_x, (B, T, H, dk)), ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)),
                         ("out_gate", out_gate, (B, T, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    fu = _fusion(gate_x, gate_scale, normalize_qk, out_gate)
    st = _lib.kda_chunked_forward_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                        ctypes.byref(fu), B, T, H, dk, dv, chunk, _dtype_code(q), _ptr(ws),
                                        _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_fused", st)
    return o, hT


def kda_chunked_forward_profiled(q, k, v, g, beta, h0, o, hT, *, chunk: int = 64, workspace=None, stream=None):
    """kda_chunked_forward into preallocated o / hT (hT may be None), returning the two kernels'
    durations in ms (intra-chunk, chain) from HIP events on the stream; synchronises the stream."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)), ("o", o, (B, T, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    ms = (ctypes.c_float * 2)()
    st = _lib.kda_chunked_forward_profiled(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                           _ptr(hT), B, T, H, dk, dv, chunk, _dtype_code(q), _ptr(ws), _nbytes(ws),
                                           _stream(stream), ctypes.cast(ms, _vp))
    if st:
        raise KDAError("kda_chunked_forward_profiled", st)
    return float(ms[0]), float(ms[1])


def kda_chunked_forward_varlen(q, k, v, g, beta, cu_seqlens, max_seqlen: int, h0=None, *, chunk: int = 64, o=None,
                               hT=None, want_hT: bool = True, workspace=None, stream=None):
    """Packed varlen prefill.  q, k, g [1,T_total,H,dk] (or [T_total,H,dk]); v [..,T_total,H,dv];
    beta [..,T_total,H]; cu_seqlens int32 [N+1] on the device; h0 [N,H,dk,dv] float32 or None.
    Returns (o shaped like v, hT [N,H,dk,dv] float32 or None)."""
    return _varlen_call(q, k, v, g, beta, cu_seqlens, max_seqlen, h0, chunk, o, hT, want_hT, workspace, stream, None, 0)


def _varlen_call(q, k, v, g, beta, cu_seqlens, max_seqlen, h0, chunk, o, hT, want_hT, workspace, stream, states,
                 state_every):
    Tt, H, dk = q.shape[-3:]
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt, dev = q.dtype, q.device
    lead = tuple(q.shape[:-3])
    if lead not in ((), (1,)):
        raise ValueError("varlen inputs are packed along one token axis (batch 1)")
    for name, t, shp in (("q", q, lead + (Tt, H, dk)), ("k", k, lead + (Tt, H, dk)), ("g", g, lead + (Tt, H, dk)),
                         ("v", v, lead + (Tt, H, dv)), ("beta", beta, lead + (Tt, H))):
        _check(name, t, shp, dt, dev)
    _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    _check("h0", h0, (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(lead + (Tt, H, dv), dtype=dt, device=dev)
    _check("o", o, lead + (Tt, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (N, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_varlen_workspace_bytes(N, Tt, max_seqlen, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    if states is None:
        st = _lib.kda_chunked_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                             _ptr(hT), _ptr(cu_seqlens), N, Tt, int(max_seqlen), H, dk, dv, chunk,
                                             _dtype_code(q), _ptr(ws), _nbytes(ws), _stream(stream))
        if st:
            raise KDAError("kda_chunked_forward_varlen", st)
    else:
        st = _lib.kda_chunked_forward_varlen_with_states(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _ptr(states), state_every,
            _ptr(cu_seqlens), N, Tt, int(max_seqlen), H, dk, dv, chunk, _dtype_code(q), _ptr(ws), _nbytes(ws),
            _stream(stream))
        if st:
            raise KDAError("kda_chunked_forward_varlen_with_states", st)
    return o, hT


def kda_chunked_forward_varlen_with_states(q, k, v, g, beta, cu_seqlens, max_seqlen: int, h0=None, *,
                                           state_every: int, chunk: int = 64, o=None, hT=None, states=None,
                                           want_hT: bool = True, workspace=None, stream=None):
    """kda_chunked_forward_varlen that also returns the state after every state_every tokens of each
    sequence: states [N,H,max_seqlen//state_every,dk,dv] float32 (entries past a sequence's length
    are left as allocated).  Returns (o, hT, states)."""
    Tt, H, dk = q.shape[-3:]
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dev = q.device
    n_states = int(max_seqlen) // state_every if state_every > 0 else 0
    if states is None:
        states = torch.zeros((N, H, n_states, dk, dv), dtype=torch.float32, device=dev)
    _check("states", states, (N, H, n_states, dk, dv), torch.float32, dev)
    o, hT = _varlen_call(q, k, v, g, beta, cu_seqlens, max_seqlen, h0, chunk, o, hT, want_hT, workspace, stream,
                         states, int(state_every))
    return o, hT, states


def kda_decode_step(q, k, v, g, beta, state, *, o=None, stream=None):
    """One decode step.  q, k, g [B,H,dk]; v [B,H,dv]; beta [B,H]; state [B,H,dk,dv] float32,
    updated in place.  Returns o [B,H,dv]."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("g", g, (B, H, dk)), ("v", v, (B, H, dv)),
                         ("beta", beta, (B, H))):
        _check(name, t, shp, dt, dev)
    _check("state", state, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, H, dv), dt, dev)
    st = _lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o), B, H, dk, dv,
                              _dtype_code(q), _stream(stream))
    if st:
        raise KDAError("kda_decode_step", st)
    return o


def kda_decode_step_fused(q, k, v, g, beta, state, *, gate_x=None, gate_scale: float = 5.0,
                          normalize_qk: bool = False, out_gate=None, o=None, stream=None):
    """kda_decode_step with the fused steps (see kda_chunked_forward_fused): gate_x [B,H,dk],
    out_gate [B,H,dv].  Returns o [B,H,dv]."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("g", g, (B, H, dk)),
                         ("gate_x", gate_x, (B, H, dk)), ("v", v, (B, H, dv)), ("beta", beta, (B, H)),
                         ("out_gate", out_gate, (B, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("state", state, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, H, dv), dt, dev)
    fu = _fusion(gate_x, gate_scale, normalize_qk, out_gate)
    st = _lib.kda_decode_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                                    ctypes.byref(fu), B, H, dk, dv, _dtype_code(q), _stream(stream))
    if st:
        raise KDAError("kda_decode_step_fused", st)
    return o


def kda_chunked_forward_ex(q, k, v, g, beta, h0=None, *, state_every: int = 0, states=None, gate_x=None,
                           gate_scale: float = 5.0, normalize_qk: bool = False, out_gate=None, chunk: int = 64,
                           o=None, hT=None, want_hT: bool = True, workspace=None, stream=None):
    """kda_chunked_forward with state snapshots (state_every > 0) and the fused steps together.
    Returns (o, hT, states or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("gate_x", gate_x, (B, T, H, dk)), ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)),
                         ("out_gate", out_gate, (B, T, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    if state_every > 0 and states is None:
        states = torch.empty((B, H, T // state_every, dk, dv), dtype=torch.float32, device=dev)
    if states is not None:
        _check("states", states, (B, H, T // state_every, dk, dv), torch.float32, dev)
    ws = _workspace(workspace, _lib.kda_chunked_forward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q)), dev)
    fu = _fusion(gate_x, gate_scale, normalize_qk, out_gate)
    st = _lib.kda_chunked_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                     _ptr(states), int(state_every), ctypes.byref(fu), B, T, H, dk, dv, chunk,
                                     _dtype_code(q), _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_ex", st)
    return o, hT, states


def kda_chunked_forward_varlen_ex(q, k, v, g, beta, cu_seqlens, max_seqlen: int, h0=None, *, state_every: int = 0,
                                  states=None, gate_x=None, gate_scale: float = 5.0, normalize_qk: bool = False,
                                  out_gate=None, chunk: int = 64, o=None, hT=None, want_hT: bool = True,
                                  workspace=None, stream=None):
    """kda_chunked_forward_varlen with state snapshots and the fused steps together (gate_x shaped like
    q, out_gate like v).  Returns (o, hT, states or None)."""
    Tt, H, dk = q.shape[-3:]
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt, dev = q.dtype, q.device
    lead = tuple(q.shape[:-3])
    if lead not in ((), (1,)):
        raise ValueError("varlen inputs are packed along one token axis (batch 1)")
    for name, t, shp in (("q", q, lead + (Tt, H, dk)), ("k", k, lead + (Tt, H, dk)), ("g", g, lead + (Tt, H, dk)),
                         ("gate_x", gate_x, lead + (Tt, H, dk)), ("v", v, lead + (Tt, H, dv)),
                         ("beta", beta, lead + (Tt, H)), ("out_gate", out_gate, lead + (Tt, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    _check("h0", h0, (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(lead + (Tt, H, dv), dtype=dt, device=dev)
    _check("o", o, lead + (Tt, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (N, H, dk, dv), torch.float32, dev)
    slots = int(max_seqlen) // state_every if state_every > 0 else 0
    if state_every > 0 and states is None:
        states = torch.zeros((N, H, slots, dk, dv), dtype=torch.float32, device=dev)
    if states is not None:
        _check("states", states, (N, H, slots, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_forward_varlen_workspace_bytes(N, Tt, max_seqlen, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    fu = _fusion(gate_x, gate_scale, normalize_qk, out_gate)
    st = _lib.kda_chunked_forward_varlen_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                            _ptr(hT), _ptr(states), int(state_every), ctypes.byref(fu),
                                            _ptr(cu_seqlens), N, Tt, int(max_seqlen), H, dk, dv, chunk,
                                            _dtype_code(q), _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_varlen_ex", st)
    return o, hT, states


def backward_workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Device workspace kda_chunked_backward needs for this shape (0: unsupported)."""
    return int(_lib.kda_chunked_backward_workspace_bytes(B, T, H, dk, dv, chunk,
                                                         _dtype_code(torch.empty(0, dtype=dtype))))


def kda_chunked_backward(q, k, v, g, beta, h0, do, dhT=None, *, chunk: int = 64, want_dh0: bool = True,
                         grads=None, workspace=None, stream=None):
    """Gradients of <do, o> + <dhT, hT> for (o, hT) = kda_chunked_forward(q, k, v, g, beta, h0).
    q, k, g [B,T,H,dk]; v, do [B,T,H,dv]; beta [B,T,H] (one dtype); h0, dhT [B,H,dk,dv] float32 or
    None.  Returns (dq, dk, dv, dg, dbeta, dh0): the first five like q, k, v, g, beta, dh0 float32
    [B,H,dk,dv] (None unless want_dh0).  grads: optional preallocated 6-tuple of outputs."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)), ("do", do, (B, T, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    _check("dhT", dhT, (B, H, dk, dv), torch.float32, dev)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
                 torch.empty_like(beta),
                 torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dh0 else None)
    dq, dkk, dvv, dg, db, dh0 = grads
    for name, t, ref in (("dq", dq, q), ("dk", dkk, k), ("dv", dvv, v), ("dg", dg, g), ("dbeta", db, beta)):
        _check(name, t, ref.shape, dt, dev)
    _check("dh0", dh0, (B, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_backward_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    st = _lib.kda_chunked_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dhT),
                                   _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dh0),
                                   B, T, H, dk, dv, chunk, _dtype_code(q), _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_backward", st)
    return dq, dkk, dvv, dg, db, dh0


def train_saved_bytes(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Bytes of the buffer kda_chunked_forward_train fills for kda_chunked_backward_saved (0: unsupported)."""
    return int(_lib.kda_chunked_forward_train_saved_bytes(B, T, H, dk, dv, chunk,
                                                          _dtype_code(torch.empty(0, dtype=dtype))))


def backward_saved_workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Device workspace kda_chunked_backward_saved needs besides the saved buffer (0: unsupported)."""
    return int(_lib.kda_chunked_backward_saved_workspace_bytes(B, T, H, dk, dv, chunk,
                                                               _dtype_code(torch.empty(0, dtype=dtype))))


def kda_chunked_forward_train(q, k, v, g, beta, h0=None, *, chunk: int = 64, o=None, hT=None, want_hT: bool = True,
                              saved=None, stream=None):
    """The forward of a training step: (o, hT) as kda_chunked_forward, plus `saved`, a uint8 device
    tensor holding what kda_chunked_backward_saved needs (the per-chunk records and chunk-start
    states).  Returns (o, hT, saved); keep saved and the inputs unchanged until the backward."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check("o", o, (B, T, H, dv), dt, dev)
    if hT is None and want_hT:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check("hT", hT, (B, H, dk, dv), torch.float32, dev)
    sv = _workspace(saved, _lib.kda_chunked_forward_train_saved_bytes(B, T, H, dk, dv, chunk, _dtype_code(q)), dev)
    st = _lib.kda_chunked_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                        B, T, H, dk, dv, chunk, _dtype_code(q), _ptr(sv), _nbytes(sv), _stream(stream))
    if st:
        raise KDAError("kda_chunked_forward_train", st)
    return o, hT, sv


def kda_chunked_backward_saved(q, k, v, g, beta, h0, do, dhT, saved, *, chunk: int = 64, want_dh0: bool = True,
                               grads=None, workspace=None, stream=None):
    """kda_chunked_backward for a forward run by kda_chunked_forward_train on the same inputs: the
    same gradients, from `saved` instead of a recomputed forward."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)), ("do", do, (B, T, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("h0", h0, (B, H, dk, dv), torch.float32, dev)
    _check("dhT", dhT, (B, H, dk, dv), torch.float32, dev)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
                 torch.empty_like(beta),
                 torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dh0 else None)
    dq, dkk, dvv, dg, db, dh0 = grads
    for name, t, ref in (("dq", dq, q), ("dk", dkk, k), ("dv", dvv, v), ("dg", dg, g), ("dbeta", db, beta)):
        _check(name, t, ref.shape, dt, dev)
    _check("dh0", dh0, (B, H, dk, dv), torch.float32, dev)
    sv = _workspace(saved, 0, dev)
    ws = _workspace(workspace, _lib.kda_chunked_backward_saved_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q)),
                    dev)
    st = _lib.kda_chunked_backward_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do),
                                         _ptr(dhT), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dh0),
                                         B, T, H, dk, dv, chunk, _dtype_code(q), _ptr(sv), _nbytes(sv), _ptr(ws),
                                         _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_backward_saved", st)
    return dq, dkk, dvv, dg, db, dh0


def backward_varlen_workspace_bytes(num_seqs, T_total, max_seqlen, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Device workspace kda_chunked_backward_varlen needs for this shape (0: unsupported)."""
    return int(_lib.kda_chunked_backward_varlen_workspace_bytes(num_seqs, T_total, max_seqlen, H, dk, dv, chunk,
                                                                _dtype_code(torch.empty(0, dtype=dtype))))


def kda_chunked_backward_varlen(q, k, v, g, beta, cu_seqlens, max_seqlen: int, h0, do, dhT=None, *, chunk: int = 64,
                                want_dh0: bool = True, grads=None, workspace=None, stream=None):
    """Gradients of <do, o> + <dhT, hT> for (o, hT) = kda_chunked_forward_varlen(q, k, v, g, beta, cu_seqlens,
    max_seqlen, h0): packed inputs as for the varlen forward ([1,T_total,...] or [T_total,...]), h0 and dhT
    [N,H,dk,dv] float32 or None.  Returns (dq, dk, dv, dg, dbeta, dh0) shaped like q, k, v, g, beta and
    [N,H,dk,dv] float32 (None unless want_dh0)."""
    Tt, H, dk = q.shape[-3:]
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt, dev = q.dtype, q.device
    lead = tuple(q.shape[:-3])
    if lead not in ((), (1,)):
        raise ValueError("varlen inputs are packed along one token axis (batch 1)")
    for name, t, shp in (("q", q, lead + (Tt, H, dk)), ("k", k, lead + (Tt, H, dk)), ("g", g, lead + (Tt, H, dk)),
                         ("v", v, lead + (Tt, H, dv)), ("beta", beta, lead + (Tt, H)), ("do", do, lead + (Tt, H, dv))):
        _check(name, t, shp, dt, dev)
    _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    _check("h0", h0, (N, H, dk, dv), torch.float32, dev)
    _check("dhT", dhT, (N, H, dk, dv), torch.float32, dev)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
                 torch.empty_like(beta),
                 torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dh0 else None)
    dq, dkk, dvv, dg, db, dh0 = grads
    for name, t, ref in (("dq", dq, q), ("dk", dkk, k), ("dv", dvv, v), ("dg", dg, g), ("dbeta", db, beta)):
        _check(name, t, ref.shape, dt, dev)
    _check("dh0", dh0, (N, H, dk, dv), torch.float32, dev)
    ws_bytes = _lib.kda_chunked_backward_varlen_workspace_bytes(N, Tt, int(max_seqlen), H, dk, dv, chunk,
                                                               _dtype_code(q))
    ws = _workspace(workspace, ws_bytes, dev)
    st = _lib.kda_chunked_backward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do),
                                          _ptr(dhT), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dh0),
                                          _ptr(cu_seqlens), N, Tt, int(max_seqlen), H, dk, dv, chunk, _dtype_code(q),
                                          _ptr(ws), _nbytes(ws), _stream(stream))
    if st:
        raise KDAError("kda_chunked_backward_varlen", st)
    return dq, dkk, dvv, dg, db, dh0
