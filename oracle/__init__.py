"""fp64 CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The KDA library (the HIP path) never
imports, links or calls it, and the two share no code.

The oracle is the plain definition of the KDA recurrence, evaluated token by
token in fp64 (``kda_oracle.c`` states the recurrence and the passages of the
Kimi K3 pages it follows).  This module compiles that C file with gcc on first
use and wraps it with ctypes.

Pins (tests/test_oracle_pins.py): a brute-force unrolled product form on short
sequences, closed forms (frozen state, cumulative linear attention with
orthogonal keys, first-order small-beta limit, exact key overwrite, geometric
sum of decay and erase, decay-only product), invariants (continuation,
linearity, column independence, varlen = independent calls, decode = prefill,
norm bound), a hand-computed worked example under tests/golden/, and an fp64
chunked mirror of the chunkwise (UT/WY) algebra.

MXFP8 inputs (``mxfp8_decode``, ``forward_mxfp8``) are decoded from the published OCP
Microscaling definition (E4M3 elements, E8M0 block scales of 32) and then run through the same
fp64 recurrence; the decoder is pinned in tests/test_oracle_mxfp8.py by the format's defining
values (largest normal 448, smallest subnormal 2^-9, the NaN codes, the scale range).

The backward (``backward``: reverse-mode gradients through the same recurrence) is
pinned in tests/test_oracle_backward_pins.py: finite differences of the forward,
directional derivatives across its checkpoint blocks, the adjoint identity of the
linear part, and closed forms at beta = 0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile libkda_oracle.so with gcc (plain -O2: no fast-math, fp64 as written)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
            lib.kda_oracle_forward.argtypes = [vp] * 5 + [i32, vp, vp, vp, i32, i64, i32, i32, i32, i32]
            lib.kda_oracle_forward.restype = i32
            lib.kda_oracle_forward_units.argtypes = [vp] * 5 + [i32, vp, vp, vp, i32, i64, i32, i32, i32, vp, i32, i32]
            lib.kda_oracle_forward_units.restype = i32
            lib.kda_oracle_forward_varlen.argtypes = [vp] * 5 + [i32, vp, i32, vp, vp, vp, i32, i32, i32, i32]
            lib.kda_oracle_forward_varlen.restype = i32
            lib.kda_oracle_decode_step.argtypes = [vp] * 5 + [i32, vp, vp, i32, i32, i32, i32, i32]
            lib.kda_oracle_decode_step.restype = i32
            lib.kda_oracle_backward.argtypes = [vp] * 5 + [i32] + [vp] * 9 + [i32, i64, i32, i32, i32, i32]
            lib.kda_oracle_backward.restype = i32
            _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _dtype_code(*arrs) -> int:
    dts = {a.dtype for a in arrs}
    if dts == {np.dtype(np.float32)}:
        return 0
    if dts == {np.dtype(np.uint16)}:
        return 1
    if dts == {np.dtype(np.float64)}:
        return 2
    raise TypeError("oracle inputs must all be float32, all bf16 bit patterns (uint16) or all float64, got %s" % dts)


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def _state64(h0):
    """Initial state as contiguous fp64 (fp32 converts exactly), or None."""
    if h0 is None:
        return None
    h0 = np.asarray(h0)
    assert h0.dtype in (np.float32, np.float64), h0.dtype
    return np.ascontiguousarray(h0, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def forward(q, k, v, g, beta, h0=None, want_o=True, want_hT=True, nthreads=None):
    """Batched forward.  q, k, g: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H];
    h0: [B,H,dk,dv] float32/float64 or None.  Returns (o [B,T,H,dv] fp64 or None,
    hT [B,H,dk,dv] fp64 or None)."""
    q, k, v, g, beta = map(_c, (q, k, v, g, beta))
    h0 = _state64(h0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    dt = _dtype_code(q, k, v, g, beta)
    if h0 is not None:
        assert h0.shape == (B, H, dk, dv)
    o = np.empty((B, T, H, dv), np.float64) if want_o else None
    hT = np.empty((B, H, dk, dv), np.float64) if want_hT else None
    rc = _load().kda_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), dt, _ptr(h0), _ptr(o), _ptr(hT),
                                    B, T, H, dk, dv, nthreads or default_threads())
    if rc:
        raise RuntimeError("kda_oracle_forward: invalid arguments")
    return o, hT


def forward_units(q, k, v, g, beta, h0, unit_ids, want_o=True, want_hT=True, nthreads=None):
    """Forward on a subset of (b, h) units (unit id = b * H + h), for sampled checks.
    Returns (o [n, T, dv] fp64 or None, hT [n, dk, dv] fp64 or None)."""
    q, k, v, g, beta = map(_c, (q, k, v, g, beta))
    h0 = _state64(h0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q, k, v, g, beta)
    if h0 is not None:
        assert h0.shape == (B, H, dk, dv)
    ids = np.ascontiguousarray(np.asarray(unit_ids, dtype=np.int32))
    n = ids.size
    o = np.empty((n, T, dv), np.float64) if want_o else None
    hT = np.empty((n, dk, dv), np.float64) if want_hT else None
    rc = _load().kda_oracle_forward_units(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), dt, _ptr(h0), _ptr(o),
                                          _ptr(hT), B, T, H, dk, dv, ids.ctypes.data, n,
                                          nthreads or default_threads())
    if rc:
        raise RuntimeError("kda_oracle_forward_units: invalid arguments")
    return o, hT


def forward_varlen(q, k, v, g, beta, cu_seqlens, h0=None, want_o=True, want_hT=True, nthreads=None):
    """Packed varlen forward.  q, k, g: [T_total,H,dk] (or [1,T_total,H,dk]); v: [..,T_total,H,dv];
    beta: [..,T_total,H]; cu_seqlens: int32 [N+1]; h0: [N,H,dk,dv] float32/float64 or None.
    Returns (o [T_total,H,dv] fp64, hT [N,H,dk,dv] fp64)."""
    q, k, v, g, beta = map(_c, (q, k, v, g, beta))
    h0 = _state64(h0)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = cu.size - 1
    dk, dv, H = q.shape[-1], v.shape[-1], q.shape[-2]
    Tt = int(cu[-1])
    assert q.size == Tt * H * dk and v.size == Tt * H * dv and beta.size == Tt * H
    dt = _dtype_code(q, k, v, g, beta)
    if h0 is not None:
        assert h0.shape == (N, H, dk, dv)
    o = np.empty((Tt, H, dv), np.float64) if want_o else None
    hT = np.empty((N, H, dk, dv), np.float64) if want_hT else None
    rc = _load().kda_oracle_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), dt, cu.ctypes.data, N,
                                           _ptr(h0), _ptr(o), _ptr(hT), H, dk, dv, nthreads or default_threads())
    if rc:
        raise RuntimeError("kda_oracle_forward_varlen: invalid arguments")
    return o, hT


def decode_step(q, k, v, g, beta, state, nthreads=None):
    """One decode step, in place on the fp64 state [B,H,dk,dv].  q, k, g: [B,H,dk];
    v: [B,H,dv]; beta: [B,H].  Returns o [B,H,dv] fp64."""
    q, k, v, g, beta = map(_c, (q, k, v, g, beta))
    assert state.dtype == np.float64 and state.flags["C_CONTIGUOUS"]
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q, k, v, g, beta)
    o = np.empty((B, H, dv), np.float64)
    rc = _load().kda_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), dt, state.ctypes.data,
                                        o.ctypes.data, B, H, dk, dv, nthreads or default_threads())
    if rc:
        raise RuntimeError("kda_oracle_decode_step: invalid arguments")
    return o


# --------------------------------------------------------------------------------------------
# Fused forms: the steps on either side of the recurrence, as plain fp64 definitions.
#  - the log-decay from its gate pre-activation x through a scaled sigmoid, g = -A sigmoid(x)
#    (technical-report page, "Architecture at a glance": the lower bound on the log-decay);
#  - q and k L2-normalised over d_k per (token, head): q / sqrt(sum q^2 + 1e-12);
#  - an output gate z multiplying o elementwise (same page: the input-dependent output gate; the
#    gate tensor is taken as given -- its projection needs trained weights).


def _dec(a):
    """Exact fp64 value of a stored fp32 / bf16-bits / fp64 array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return ((a.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    return a.astype(np.float64)


def _fused_inputs(q, k, g, x, gate_scale, normalize_qk):
    q, k = _dec(q), _dec(k)
    if normalize_qk:
        q = q / np.sqrt((q * q).sum(axis=-1, keepdims=True) + 1e-12)
        k = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + 1e-12)
    g = -float(gate_scale) / (1.0 + np.exp(-_dec(x))) if x is not None else _dec(g)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(g)


def forward_fused(q, k, v, g, beta, h0=None, *, x=None, gate_scale=5.0, normalize_qk=False, z=None,
                  want_o=True, want_hT=True, nthreads=None):
    """forward() with the fused steps: g = -gate_scale * sigmoid(x) when x is given (g unused),
    q and k normalised when normalize_qk, o multiplied by z when given.  Returns fp64 (o, hT)."""
    q64, k64, g64 = _fused_inputs(q, k, g, x, gate_scale, normalize_qk)
    o, hT = forward(q64, k64, np.ascontiguousarray(_dec(v)), g64, np.ascontiguousarray(_dec(beta)), h0,
                    want_o=want_o, want_hT=want_hT, nthreads=nthreads)
    if o is not None and z is not None:
        o = o * _dec(z)
    return o, hT


def decode_step_fused(q, k, v, g, beta, state, *, x=None, gate_scale=5.0, normalize_qk=False, z=None,
                      nthreads=None):
    """decode_step() with the fused steps (see forward_fused); state updated in place."""
    q64, k64, g64 = _fused_inputs(q, k, g, x, gate_scale, normalize_qk)
    o = decode_step(q64, k64, np.ascontiguousarray(_dec(v)), g64, np.ascontiguousarray(_dec(beta)), state,
                    nthreads=nthreads)
    return o * _dec(z) if z is not None else o


def forward_varlen_fused(q, k, v, g, beta, cu_seqlens, h0=None, *, x=None, gate_scale=5.0, normalize_qk=False,
                         z=None, want_o=True, want_hT=True, nthreads=None):
    """forward_varlen() with the fused steps (see forward_fused).  Returns fp64 (o, hT)."""
    q64, k64, g64 = _fused_inputs(q, k, g, x, gate_scale, normalize_qk)
    o, hT = forward_varlen(q64, k64, np.ascontiguousarray(_dec(v)), g64, np.ascontiguousarray(_dec(beta)),
                           cu_seqlens, h0, want_o=want_o, want_hT=want_hT, nthreads=nthreads)
    if o is not None and z is not None:
        o = o * _dec(z).reshape(o.shape)
    return o, hT


# --------------------------------------------------------------------------------------------
# Backward (reverse mode) of the plain recurrence, for training: the chain rule through the five
# steps of each token, in reverse order (kda_oracle.c states each step's adjoint).


def backward(q, k, v, g, beta, h0, do, dhT=None, nthreads=None):
    """Gradients of L = <do, o> + <dhT, hT> with o, hT = forward(q, k, v, g, beta, h0).
    q, k, g: [B,T,H,dk]; v, do: [B,T,H,dv]; beta: [B,T,H]; h0, dhT: [B,H,dk,dv] or None.
    do and dhT may be fp32, bf16 bits or fp64 (decoded exactly).  Returns fp64
    (dq, dk, dv, dg, dbeta, dh0) shaped like q, k, v, g, beta and [B,H,dk,dv]."""
    q, k, v, g, beta = map(_c, (q, k, v, g, beta))
    h0 = _state64(h0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    dt = _dtype_code(q, k, v, g, beta)
    do64 = np.ascontiguousarray(_dec(do))
    assert do64.shape == (B, T, H, dv)
    dhT64 = None if dhT is None else np.ascontiguousarray(_dec(dhT))
    if dhT64 is not None:
        assert dhT64.shape == (B, H, dk, dv)
    if h0 is not None:
        assert h0.shape == (B, H, dk, dv)
    dq, dkk, dg = (np.empty((B, T, H, dk)) for _ in range(3))
    dvv = np.empty((B, T, H, dv))
    db = np.empty((B, T, H))
    dh0 = np.empty((B, H, dk, dv))
    rc = _load().kda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), dt, _ptr(h0), _ptr(do64),
                                     _ptr(dhT64), _ptr(dq), _ptr(dkk), _ptr(dg), _ptr(dvv), _ptr(db), _ptr(dh0),
                                     B, T, H, dk, dv, nthreads or default_threads())
    if rc:
        raise RuntimeError("kda_oracle_backward: invalid arguments")
    return dq, dkk, dvv, dg, db, dh0


# ---------------------------------------------------------------------------------------------
# MXFP8 inputs.  The how-K3-works page ("The systems layer") says K3 trains with MXFP8
# activations; the format itself is the OCP Microscaling (MX) one:
#   - an element is FP8 E4M3: sign bit, 4 exponent bits e (bias 7), 3 mantissa bits m;
#     e = 0 is subnormal, m * 2^-9; otherwise (1 + m/8) * 2^(e-7); e = 15 with m = 7 is NaN
#     (no infinities), so the largest finite magnitude is 1.75 * 2^8 = 448;
#   - a block of 32 consecutive elements shares an E8M0 scale: an unsigned exponent s worth
#     2^(s-127), with s = 255 NaN;
#   - the value of an element is its E4M3 value times its block's scale.


def e4m3_value(codes):
    """fp64 value of FP8 E4M3 codes (uint8 array), per the OCP definition."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e8m0_value(codes):
    """fp64 value of E8M0 scale codes (uint8 array): 2^(s-127), NaN for 255."""
    s = np.asarray(codes).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2((s - 127).astype(np.float64)))


def mxfp8_decode(codes, scales, block=32):
    """fp64 values of an MXFP8 tensor: codes [..., d] uint8 (E4M3), scales [..., d/block] uint8
    (E8M0); element i of the last axis takes scale i // block."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    d = codes.shape[-1]
    assert d % block == 0 and scales.shape == codes.shape[:-1] + (d // block,)
    x = e4m3_value(codes).reshape(codes.shape[:-1] + (d // block, block))
    return np.ascontiguousarray((x * e8m0_value(scales)[..., None]).reshape(codes.shape))


def forward_mxfp8(q, q_scale, k, k_scale, v, v_scale, g, beta, h0=None, want_o=True, want_hT=True, nthreads=None):
    """forward() on MXFP8 q, k, v (codes and scales as above), bf16 / fp32 / fp64 g and beta:
    the inputs are decoded to their exact fp64 values first.  Returns fp64 (o, hT)."""
    return forward(mxfp8_decode(q, q_scale), mxfp8_decode(k, k_scale), mxfp8_decode(v, v_scale),
                   np.ascontiguousarray(_dec(g)), np.ascontiguousarray(_dec(beta)), h0,
                   want_o=want_o, want_hT=want_hT, nthreads=nthreads)
