"""The seeded input generator: SplitMix64 outputs, determinism, slice independence,
rounding, and the workload distributions."""
import numpy as np
import torch

import datagen

M64 = (1 << 64) - 1


def py_splitmix_out(seed, i):
    z = (seed + (i + 1) * 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix64_reference_outputs():
    # first outputs of SplitMix64 seeded with 0 (Vigna's reference splitmix64.c)
    assert [datagen.splitmix_out(0, i) for i in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                                              0x06C45D188009454F]
    for seed in (1, 9401, 2**63 + 5):
        for i in (0, 1, 77, 10**9):
            assert datagen.splitmix_out(seed, i) == py_splitmix_out(seed, i)


def test_deterministic_and_slice_independent():
    a = datagen.fill(7, 0, 0, 0, 1.0, datagen.DT_F64, (1000, 8), 8)
    b = datagen.fill(7, 0, 0, 0, 1.0, datagen.DT_F64, (1000, 8), 8)
    assert np.array_equal(a, b)
    # element n depends on n only: a longer fill starts with the same values
    c = datagen.fill(7, 0, 0, 0, 1.0, datagen.DT_F64, (3000, 8), 8)
    assert np.array_equal(c[:1000], a)
    assert datagen.normal_at(7, 0, 0, 8 * 500 + 3) == a[500, 3]
    # other tensor id / sub-stream / seed differ
    assert not np.array_equal(datagen.fill(7, 1, 0, 0, 1.0, datagen.DT_F64, (1000, 8), 8), a)
    assert not np.array_equal(datagen.fill(7, 0, 1, 0, 1.0, datagen.DT_F64, (1000, 8), 8), a)
    assert not np.array_equal(datagen.fill(8, 0, 0, 0, 1.0, datagen.DT_F64, (1000, 8), 8), a)


def test_normal_moments():
    x = datagen.fill(3, 2, 0, 0, 1.0, datagen.DT_F64, (200000,), 1)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_rounding_fp32_and_bf16_rne():
    x64 = datagen.fill(5, 2, 0, 0, 1.0, datagen.DT_F64, (4096, 16), 16)
    x32 = datagen.fill(5, 2, 0, 0, 1.0, datagen.DT_F32, (4096, 16), 16)
    xbf = datagen.fill(5, 2, 0, 0, 1.0, datagen.DT_BF16, (4096, 16), 16)
    assert np.array_equal(x32, x64.astype(np.float32))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(xbf, ref)


def test_workload_distributions():
    d = datagen.prefill_inputs(9401, 2, 64, 3, 128, 64, datagen.DT_BF16, 0.02)
    q = datagen.to_f64(d["q"])
    assert np.allclose(np.linalg.norm(q, axis=-1), 1, atol=1e-2)  # unit before bf16 rounding
    d32 = datagen.prefill_inputs(9401, 2, 64, 3, 128, 64, datagen.DT_F32, 0.02)
    assert np.allclose(np.linalg.norm(datagen.to_f64(d32["k"]), axis=-1), 1, atol=1e-6)
    g = datagen.to_f64(d["g"])
    assert g.max() <= 0 and g.min() >= -5
    assert 2.2 < -g.mean() < 2.8
    be = datagen.to_f64(d["beta"])
    assert be.min() > 0 and be.max() < 1 and abs(be.mean() - 0.5) < 0.05
    assert abs(d["h0"].std() - 0.02) < 0.002 and d["h0"].dtype == np.float32
    assert d["v"].shape == (2, 64, 3, 64) and d["beta"].shape == (2, 64, 3)


def test_varlen_lengths():
    n = datagen.varlen_lengths(94041, 16, 1024, 131072)
    assert n.min() >= 1024 and n.max() <= 131072 and len(set(n.tolist())) == 16
    big = datagen.uniform_ints(1, 6, 100000, 0, 9)
    assert set(np.unique(big).tolist()) == set(range(10))


def test_decode_steps_differ():
    a = datagen.decode_inputs(9403, 0, 4, 2, 16, 16, datagen.DT_BF16)
    b = datagen.decode_inputs(9403, 1, 4, 2, 16, 16, datagen.DT_BF16)
    assert not np.array_equal(a["q"], b["q"])
    assert np.array_equal(a["q"], datagen.decode_inputs(9403, 0, 4, 2, 16, 16, datagen.DT_BF16)["q"])
