"""Helpers shared by the GPU parity tests: seeded inputs on the device, the tolerance metric.

Tolerance metric (per output tensor, per (sequence, head) slice):
    err = max_i |x_i - y_i| / max_i |y_i|
and the gate is the maximum over slices; any NaN or Inf fails.  Bars: 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs with the fp32 state.
"""
import numpy as np
import torch

import datagen

TOL = {datagen.DT_F32: 1e-4, datagen.DT_BF16: 2e-2}


def dev_tensor(a, device="cuda"):
    """numpy fp32 array or bf16 bit-pattern array -> torch tensor on the device (same bits)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def slice_err(x, y, slice_axes):
    """Max over slices of max|x-y| / max|y|, where a slice fixes the axes in `slice_axes`."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if not np.all(np.isfinite(x)):
        return float("inf")
    if x.size == 0:
        return 0.0
    red = tuple(a for a in range(x.ndim) if a not in slice_axes)
    num = np.abs(x - y).max(axis=red)
    den = np.abs(y).max(axis=red)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def o_err(o_gpu, o_ref):
    """o [B,T,H,dv]: slices are (b, h)."""
    return slice_err(o_gpu, o_ref, (0, 2))


def state_err(s_gpu, s_ref):
    """states [B,H,dk,dv]: slices are (b, h)."""
    return slice_err(s_gpu, s_ref, (0, 1))


def gpu_inputs(d):
    return {key: dev_tensor(val) for key, val in d.items()}


def bf16_bits(x):
    """fp64 / fp32 values -> bf16 bit patterns (uint16), rounded fp64 -> fp32 -> bf16, both to nearest
    even, as the input generator rounds (finite values only)."""
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32)).view(np.uint32)
    return ((f + (((f >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def stored(x, dt):
    """fp64 values in the storage type of dtype code dt (fp32, or bf16 bit patterns)."""
    return bf16_bits(x) if dt == datagen.DT_BF16 else np.ascontiguousarray(np.asarray(x, np.float64), np.float32)
