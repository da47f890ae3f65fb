"""Seeded synthetic inputs for the KDA workloads (test and benchmark infrastructure).

Shared by the fp64 oracle and the HIP path; holds none of the delta-rule
arithmetic.  The C source (``datagen.c``) implements a counter-based
SplitMix64 stream per (seed, tensor id, sub-stream) and the Box-Muller
transform; this module compiles it with gcc on first use, wraps it with
ctypes and describes the workloads:

* q, k ~ N(0, 1) per element, then L2-normalised over d_k per (token, head)
  in fp64 before rounding;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1)) per (token, head);
* g (the log-decay, log alpha) = -5 * sigmoid(N(0, 1)) per (token, head, key
  channel) -- the scaled-sigmoid lower bound the Kimi K3 pages describe
  ("Architecture at a glance" and the FAQ of the technical-report page);
* h0 ~ 0.02 * N(0, 1) in fp32 where the workload starts from a random state.

Values are drawn in fp64 and rounded fp64 -> fp32 -> bf16 (both
round-to-nearest-even).  bf16 tensors are returned as ``numpy.uint16`` bit
patterns; ``bf16_bits_to_f64`` decodes them exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "datagen.c")
_LIB_PATH = os.path.join(_HERE, "libdatagen.so")
_lock = threading.Lock()
_lib = None

# tensor ids of the streams
TID_Q, TID_K, TID_V, TID_BETA, TID_G, TID_H0, TID_LEN, TID_Z, TID_DO, TID_DHT = 0, 1, 2, 3, 4, 5, 6, 7, 8, 9
_KIND_NORMAL, _KIND_UNIT_ROWS, _KIND_SIGMOID = 0, 1, 2
DT_F32, DT_BF16, DT_F64 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile libdatagen.so with gcc (always when ``force``)."""
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
            u64, i32 = ctypes.c_uint64, ctypes.c_int
            lib.dg_fill.argtypes = [u64, u64, u64, i32, ctypes.c_double, i32, u64, i32, ctypes.c_void_p, i32]
            lib.dg_fill.restype = i32
            lib.dg_uniform_ints.argtypes = [u64, u64, i32, i32, i32, ctypes.c_void_p]
            lib.dg_uniform_ints.restype = i32
            lib.dg_splitmix_out.argtypes = [u64, u64]
            lib.dg_splitmix_out.restype = u64
            lib.dg_normal_at.argtypes = [u64, u64, u64, u64]
            lib.dg_normal_at.restype = ctypes.c_double
            lib.dg_stream_base.argtypes = [u64, u64, u64]
            lib.dg_stream_base.restype = u64
            _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill(seed: int, tid: int, sub: int, kind: int, scale: float, dtype: int, shape, dim: int) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    assert n % dim == 0
    np_dt = {DT_F32: np.float32, DT_BF16: np.uint16, DT_F64: np.float64}[dtype]
    out = np.empty(shape, dtype=np_dt)
    if n:
        rc = _load().dg_fill(seed, tid, sub, kind, float(scale), dtype, n // dim, dim, out.ctypes.data, _threads())
        if rc:
            raise RuntimeError("dg_fill failed")
    return out


def uniform_ints(seed: int, tid: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if _load().dg_uniform_ints(seed, tid, n, lo, hi, out.ctypes.data):
        raise RuntimeError("dg_uniform_ints failed")
    return out


def splitmix_out(seed: int, i: int) -> int:
    return int(_load().dg_splitmix_out(seed, i))


def normal_at(seed: int, tid: int, sub: int, n: int) -> float:
    return float(_load().dg_normal_at(seed, tid, sub, n))


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of a stored fp32 array or bf16 bit-pattern array."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def prefill_inputs(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: int, h0_std=None, sub: int = 0):
    """Inputs of one prefill call: dict with q, k, g [B,T,H,dk], v [B,T,H,dv], beta [B,T,H],
    h0 [B,H,dk,dv] fp32 (or None)."""
    rows = (B, T, H)
    d = {
        "q": fill(seed, TID_Q, sub, _KIND_UNIT_ROWS, 1.0, dtype, rows + (dk,), dk),
        "k": fill(seed, TID_K, sub, _KIND_UNIT_ROWS, 1.0, dtype, rows + (dk,), dk),
        "v": fill(seed, TID_V, sub, _KIND_NORMAL, 1.0, dtype, rows + (dv,), dv),
        "g": fill(seed, TID_G, sub, _KIND_SIGMOID, -5.0, dtype, rows + (dk,), dk),
        "beta": fill(seed, TID_BETA, sub, _KIND_SIGMOID, 1.0, dtype, rows, 1),
    }
    d["h0"] = None if h0_std is None else fill(seed, TID_H0, 0, _KIND_NORMAL, h0_std, DT_F32, (B, H, dk, dv), dv)
    return d


def _e4m3_encode(y):
    """FP8 E4M3 codes of fp64 values y, rounded to the nearest representable value (ties to the
    even mantissa) and saturated to +-448.  Spacing of the E4M3 grid: 2^-9 below 2^-6
    (subnormals), 2^(E-3) in [2^E, 2^(E+1))."""
    y = np.asarray(y, np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), 448.0)
    E = np.clip(np.floor(np.log2(np.maximum(a, 2.0 ** -6))), -6, 8)
    step = np.exp2(E - 3)
    r = np.minimum(np.round(a / step) * step, 448.0)  # np.round: ties to even
    sub = r < 2.0 ** -6
    Er = np.floor(np.log2(np.maximum(r, 2.0 ** -6)))
    m = np.where(sub, r / 2.0 ** -9, r / np.exp2(Er) * 8.0 - 8.0)
    code = np.where(sub, m, (Er + 7) * 8 + m).astype(np.int64)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(x, block=32):
    """MXFP8 encoding of fp64 x [..., d]: per block of 32 channels the smallest shared scale 2^X
    that keeps every x / 2^X within the largest E4M3 magnitude, X = ceil(log2(max |x| / 448))
    (clamped to [-127, 127]; X = 0 for an all-zero block), then each x / 2^X as E4M3 (nearest).
    Returns (codes uint8 [..., d], scale codes uint8 [..., d/block])."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    xb = x.reshape(x.shape[:-1] + (d // block, block))
    amax = np.abs(xb).max(axis=-1)
    X = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0.0)
    X = np.clip(X, -127, 127)
    codes = _e4m3_encode(xb / np.exp2(X)[..., None]).reshape(x.shape)
    return np.ascontiguousarray(codes), np.ascontiguousarray((X + 127).astype(np.uint8))


def mxfp8_prefill_inputs(seed: int, B: int, T: int, H: int, dk: int, dv: int, h0_std=None, sub: int = 0):
    """prefill_inputs (bf16) with q, k and v also in MXFP8: keys q8, qs, k8, ks, v8, vs (codes,
    scale codes) quantised from the bf16 values; g and beta stay bf16."""
    d = prefill_inputs(seed, B, T, H, dk, dv, DT_BF16, h0_std, sub)
    for name in ("q", "k", "v"):
        d[name + "8"], d[name[0] + "s"] = mxfp8_quantize(to_f64(d[name]))
    return d


def backward_adjoints(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: int, dhT_std=None, sub: int = 0):
    """Adjoints for a backward call: do [B,T,H,dv] N(0,1) in the input dtype, dhT [B,H,dk,dv] fp32
    N(0, dhT_std) (or None)."""
    do = fill(seed, TID_DO, sub, _KIND_NORMAL, 1.0, dtype, (B, T, H, dv), dv)
    dhT = None if dhT_std is None else fill(seed, TID_DHT, 0, _KIND_NORMAL, dhT_std, DT_F32, (B, H, dk, dv), dv)
    return do, dhT


def prefill_preactivations(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: int, h0_std=None,
                           sub: int = 0):
    """The same draws as prefill_inputs before their last transform, for the fused entry points:
    q, k ~ N(0, 1) not normalised; x (the gate pre-activation, g = -5 sigmoid(x) in prefill_inputs)
    ~ N(0, 1); plus z = sigmoid(N(0, 1)) [B,T,H,dv], an output gate.  v, beta, h0 as prefill_inputs."""
    rows = (B, T, H)
    d = {
        "q": fill(seed, TID_Q, sub, _KIND_NORMAL, 1.0, dtype, rows + (dk,), dk),
        "k": fill(seed, TID_K, sub, _KIND_NORMAL, 1.0, dtype, rows + (dk,), dk),
        "v": fill(seed, TID_V, sub, _KIND_NORMAL, 1.0, dtype, rows + (dv,), dv),
        "x": fill(seed, TID_G, sub, _KIND_NORMAL, 1.0, dtype, rows + (dk,), dk),
        "beta": fill(seed, TID_BETA, sub, _KIND_SIGMOID, 1.0, dtype, rows, 1),
        "z": fill(seed, TID_Z, sub, _KIND_SIGMOID, 1.0, dtype, rows + (dv,), dv),
    }
    d["h0"] = None if h0_std is None else fill(seed, TID_H0, 0, _KIND_NORMAL, h0_std, DT_F32, (B, H, dk, dv), dv)
    return d


def decode_preactivations(seed: int, step: int, B: int, H: int, dk: int, dv: int, dtype: int):
    """decode_inputs before their last transform (see prefill_preactivations): q, k, x [B,H,dk],
    v, z [B,H,dv], beta [B,H]."""
    sub = step + 1
    rows = (B, H)
    return {
        "q": fill(seed, TID_Q, sub, _KIND_NORMAL, 1.0, dtype, rows + (dk,), dk),
        "k": fill(seed, TID_K, sub, _KIND_NORMAL, 1.0, dtype, rows + (dk,), dk),
        "v": fill(seed, TID_V, sub, _KIND_NORMAL, 1.0, dtype, rows + (dv,), dv),
        "x": fill(seed, TID_G, sub, _KIND_NORMAL, 1.0, dtype, rows + (dk,), dk),
        "beta": fill(seed, TID_BETA, sub, _KIND_SIGMOID, 1.0, dtype, rows, 1),
        "z": fill(seed, TID_Z, sub, _KIND_SIGMOID, 1.0, dtype, rows + (dv,), dv),
    }


def decode_inputs(seed: int, step: int, B: int, H: int, dk: int, dv: int, dtype: int):
    """Inputs of decode step `step` (0-based): q, k, g [B,H,dk], v [B,H,dv], beta [B,H]."""
    sub = step + 1
    rows = (B, H)
    return {
        "q": fill(seed, TID_Q, sub, _KIND_UNIT_ROWS, 1.0, dtype, rows + (dk,), dk),
        "k": fill(seed, TID_K, sub, _KIND_UNIT_ROWS, 1.0, dtype, rows + (dk,), dk),
        "v": fill(seed, TID_V, sub, _KIND_NORMAL, 1.0, dtype, rows + (dv,), dv),
        "g": fill(seed, TID_G, sub, _KIND_SIGMOID, -5.0, dtype, rows + (dk,), dk),
        "beta": fill(seed, TID_BETA, sub, _KIND_SIGMOID, 1.0, dtype, rows, 1),
    }


def decode_state0(seed: int, B: int, H: int, dk: int, dv: int, std: float = 0.02) -> np.ndarray:
    return fill(seed, TID_H0, 0, _KIND_NORMAL, std, DT_F32, (B, H, dk, dv), dv)


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    return uniform_ints(seed, TID_LEN, n, lo, hi)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode" | "varlen"
    seed: int
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: int           # DT_F32 | DT_BF16
    h0_std: float | None
    steps: int = 0       # decode steps
    num_seqs: int = 0    # varlen
    len_lo: int = 0
    len_hi: int = 0
    note: str = field(default="", compare=False)


# The five workloads the KDA measurements are quoted on (seed = 9400 + index).
WORKLOADS = {
    "cfg0_f32_b1_h2_t256_d64": Workload("cfg0_f32_b1_h2_t256_d64", "prefill", 9400, 1, 256, 2, 64, 64, 64, DT_F32, None),
    "cfg1_bf16_b4_h16_t4096_d128": Workload("cfg1_bf16_b4_h16_t4096_d128", "prefill", 9401, 4, 4096, 16, 128, 128, 64,
                                            DT_BF16, 0.02),
    "cfg2_bf16_b1_h32_t65536_d128": Workload("cfg2_bf16_b1_h32_t65536_d128", "prefill", 9402, 1, 65536, 32, 128, 128,
                                             64, DT_BF16, 0.02),
    "cfg3_decode_b256_h32_d128": Workload("cfg3_decode_b256_h32_d128", "decode", 9403, 256, 1, 32, 128, 128, 64,
                                          DT_BF16, 0.02, steps=1000),
    "cfg4_bf16_b1_h8_t1048576_d128": Workload("cfg4_bf16_b1_h8_t1048576_d128", "prefill", 9404, 1, 1 << 20, 8, 128,
                                              128, 64, DT_BF16, None),
    "cfg4v_varlen_n16_h8_d128": Workload("cfg4v_varlen_n16_h8_d128", "varlen", 94041, 1, 0, 8, 128, 128, 64, DT_BF16,
                                         None, num_seqs=16, len_lo=1024, len_hi=131072),
}
