"""The pins catch plausible mistakes: each test plants one slip in a copy of the
oracle's C source (on the CPU), builds it, and checks that some pin fails.

Mistakes planted: a sign flip in the delta correction, a dropped beta, a
dropped or inverted decay, the gate read from the wrong channel, the write
term subtracted, the read-out taken with the key instead of the query, the
decay applied after the write, and the decayed state not used for the erase.
For the sampled-unit forward (forward_units): b and h swapped in the unit id,
the initial state taken by output slot instead of unit, a wrong output stride.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "sign_of_correction": ("p[j] = b * (ld(in->v, in->dtype, row * dv + j) - p[j]);",
                           "p[j] = b * (ld(in->v, in->dtype, row * dv + j) + p[j]);"),
    "beta_dropped": ("p[j] = b * (ld(in->v, in->dtype, row * dv + j) - p[j]);",
                     "p[j] = (ld(in->v, in->dtype, row * dv + j) - p[j]);"),
    "decay_dropped": ("for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;\n    }\n    /* 2.",
                      "for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= 1.0;\n    }\n    /* 2."),
    "decay_inverted": ("double a = exp(ld(in->g, in->dtype, row * dk + c));\n      for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;\n    }\n    /* 2.",
                       "double a = exp(-ld(in->g, in->dtype, row * dk + c));\n      for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;\n    }\n    /* 2."),
    "gate_channel_reversed": ("double a = exp(ld(in->g, in->dtype, row * dk + c));\n      for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;\n    }\n    /* 2.",
                              "double a = exp(ld(in->g, in->dtype, row * dk + (dk - 1 - c)));\n      for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;\n    }\n    /* 2."),
    "write_subtracted": ("for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kk[c] * p[j];\n    /* 5.",
                         "for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] -= kk[c] * p[j];\n    /* 5."),
    "readout_with_key": ("for (int j = 0; j < dv; ++j) o[j] += S[(size_t)c * dv + j] * qq[c];\n    }\n  }\n  if (u->hT)",
                         "for (int j = 0; j < dv; ++j) o[j] += S[(size_t)c * dv + j] * kk[c];\n    }\n  }\n  if (u->hT)"),
    # erase measured against the state before its decay: compute p from S / a (undo the decay first)
    "erase_before_decay": ("for (int j = 0; j < dv; ++j) p[j] += S[(size_t)c * dv + j] * kk[c];\n    /* 3.-4.",
                           "for (int j = 0; j < dv; ++j) p[j] += S[(size_t)c * dv + j] / exp(ld(in->g, in->dtype, row * dk + c)) * kk[c];\n    /* 3.-4."),
}

PINS = [
    pins.test_golden_worked_example,
    lambda: pins.test_p1_brute_force_product_form(7, 8, 5),
    pins.test_p2_frozen_state,
    pins.test_p3_orthogonal_keys_linear_attention,
    pins.test_p4_small_beta_limit,
    pins.test_p5_exact_key_overwrite,
    pins.test_p6_geometric_sum,
    pins.test_p7_decay_only_product,
    pins.test_p12_decode_equals_prefill,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new, 1))  # the first occurrence is the prefill recurrence
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", str(src), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "_SRC", str(src))
    monkeypatch.setattr(oracle, "_lib", None)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
    monkeypatch.setattr(oracle, "_lib", None)
    print(name, "caught by", failed)
    # the decode-vs-prefill pin alone would not prove the recurrence wrong: require a pin of the math itself
    assert set(failed) - {"test_p12_decode_equals_prefill"}, "no pin caught the planted mistake %r" % name


# Slips in the unit selection of forward_units (the sampled-unit oracle): each must fail its pin.
UNIT_MUTANTS = {
    "unit_b_h_swapped": ("int b = id / H, h = id % H;", "int h = id / B, b = id % B;"),
    "unit_h0_of_slot": ("u->h0 = h0 ? h0 + (size_t)id * dk * dv : NULL;",
                        "u->h0 = h0 ? h0 + (size_t)i * dk * dv : NULL;"),
    "unit_o_stride": ("u->o = o ? o + (size_t)i * (size_t)T * dv : NULL;", "u->o = o ? o + (size_t)i * dv : NULL;"),
}


@pytest.mark.parametrize("name", sorted(UNIT_MUTANTS))
def test_unit_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = UNIT_MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not found: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", str(src), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "_SRC", str(src))
    monkeypatch.setattr(oracle, "_lib", None)
    with pytest.raises(AssertionError):
        pins.test_forward_units_equals_batched_slices()
    monkeypatch.setattr(oracle, "_lib", None)
