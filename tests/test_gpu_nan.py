"""A NaN in one input element stays where the recurrence puts it (the header: NaN in an input
propagates to o and hT).  Value columns of the state evolve independently and no state crosses a
(sequence, head) unit, so:

* a NaN in v[b, t, h, j] makes column j of that unit's outputs non-finite from token t on and
  column j of its final state non-finite; every other column of that unit and every other unit is
  bitwise what the call gives without the NaN;
* a NaN in g[b, t, h, c] (the decay of key channel c) reaches every column through the chunk's
  products: that unit's outputs from token t on and its final state are non-finite, and every
  other unit is bitwise unchanged;
* the same for one decode step.

Tokens of the NaN's own chunk before t may also become NaN: the chunkwise form multiplies the
chunk's masked (zero) coefficients by the NaN.  Tokens of earlier chunks are bitwise unchanged."""
import numpy as np
import pytest
import torch

import datagen
from tests.kda_testlib import dev_tensor

pytestmark = pytest.mark.gpu
kda = pytest.importorskip("gated_delta_rule_94_amd")

KEYS = ("q", "k", "v", "g", "beta")
BF16_NAN = np.uint16(0x7FC0)


def run(d, chunk):
    t = {key: dev_tensor(d[key]) for key in KEYS}
    o, hT = kda.kda_chunked_forward(t["q"], t["k"], t["v"], t["g"], t["beta"], dev_tensor(d["h0"]), chunk=chunk)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), hT.cpu().numpy()


@pytest.mark.parametrize("B,T,H,chunk", [(2, 300, 3, 64), (2, 300, 3, 16), (1, 8229, 2, 64)])
@pytest.mark.parametrize("where", ["v", "g"])
def test_nan_stays_in_its_unit(where, B, T, H, chunk):
    d = datagen.prefill_inputs(990 + T + chunk, B, T, H, 128, 128, datagen.DT_BF16, 0.02)
    print("NaN in %s: B=%d T=%d H=%d chunk=%d plan %s" % (where, B, T, H, chunk, kda.chain_plan(B, T, H, 128, 128, chunk)),
          flush=True)
    o0, h0 = run(d, chunk)
    b, t, h, j = B - 1, T // 2 + 3, H - 1, 5
    bad = {key: val.copy() for key, val in d.items() if val is not None}
    bad["h0"] = d["h0"]
    bad[where][b, t, h, j] = BF16_NAN
    o1, h1 = run(bad, chunk)
    assert np.isfinite(o0).all() and np.isfinite(h0).all()
    first = (t // chunk) * chunk  # first token of the NaN's chunk
    for bb in range(B):
        for hh in range(H):
            if (bb, hh) != (b, h):
                assert np.array_equal(o1[bb, :, hh], o0[bb, :, hh]) and np.array_equal(h1[bb, hh], h0[bb, hh])
    assert np.array_equal(o1[b, :first, h], o0[b, :first, h])  # earlier chunks
    if where == "v":
        assert not np.isfinite(o1[b, t:, h, j]).any() and not np.isfinite(h1[b, h, :, j]).any()
        cols = [c for c in range(128) if c != j]
        assert np.array_equal(o1[b, :, h][:, cols], o0[b, :, h][:, cols])
        assert np.array_equal(h1[b, h][:, cols], h0[b, h][:, cols])
    else:
        assert not np.isfinite(o1[b, t:, h]).any() and not np.isfinite(h1[b, h]).any()


def test_nan_in_one_decode_unit():
    B, H, d = 4, 3, 128
    s0 = datagen.decode_state0(995, B, H, d, d)
    dd = datagen.decode_inputs(995, 0, B, H, d, d, datagen.DT_BF16)
    bad = {key: val.copy() for key, val in dd.items()}
    bad["v"][2, 1, 7] = BF16_NAN
    outs = []
    for inp in (dd, bad):
        st = dev_tensor(s0.copy())
        o = kda.kda_decode_step(*(dev_tensor(inp[key]) for key in KEYS), st)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), st.cpu().numpy()))
    (o0, s0_), (o1, s1) = outs
    assert np.isfinite(o0).all() and np.isfinite(s0_).all()
    assert np.isnan(o1[2, 1, 7]) and np.isnan(s1[2, 1, :, 7]).all()
    mask = np.ones((B, H, d), bool)
    mask[2, 1, 7] = False
    assert np.array_equal(o1[mask], o0[mask])
    smask = np.ones((B, H, d, d), bool)
    smask[2, 1, :, 7] = False
    assert np.array_equal(s1[smask], s0_[smask])
