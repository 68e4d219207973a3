"""The oracle's pins are sharp: plant plausible mistakes in copies of the C
oracle (on the CPU, in a temporary directory) and check that the pin suite
fails for every one of them -- the forward's pins for mistakes in the forward,
the backward's pins for mistakes in the adjoint steps of the backward."""
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import test_oracle_backward as bpins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ckda_oracle.c")

# (name, [(regex on the source, replacement), ...]); the edits apply in order.
_DECAY = r"(?<!d)for \(int c = 0; c < dk; \+\+c\)\n\s*for \(int j = 0; j < dv; \+\+j\) S\[c \* dv \+ j\] \*= a\[c\];"
_DECAY_TEXT = ("for (int c = 0; c < dk; ++c)\n            "
               "for (int j = 0; j < dv; ++j) S[c * dv + j] *= a[c];")
_READOUT = (r"        /\* readout o = S\^T q \*/\n"
            r"        for \(int j = 0; j < dv; \+\+j\) o\[j\] = 0\.0;\n"
            r"        for \(int c = 0; c < dk; \+\+c\)\n"
            r"            for \(int j = 0; j < dv; \+\+j\) o\[j\] \+= q\[c\] \* S\[c \* dv \+ j\];\n")
_READOUT_TEXT = ("        for (int j = 0; j < dv; ++j) o[j] = 0.0;\n"
                 "        for (int c = 0; c < dk; ++c)\n"
                 "            for (int j = 0; j < dv; ++j) o[j] += q[c] * S[c * dv + j];\n")
MUTANTS = [
    ("decay dropped", [(r"(?<!d)S\[c \* dv \+ j\] \*= a\[c\];", ";")]),
    ("gate on value columns", [(r"(?<!d)S\[c \* dv \+ j\] \*= a\[c\];",
                                "S[c * dv + j] *= a[j % dk];")]),
    ("delta term sign", [(r"\+= b \* k\[c\] \* \(v\[j\] - u\[j\]\)",
                          "-= b * k[c] * (v[j] - u[j])")]),
    ("erase sign", [(r"\(v\[j\] - u\[j\]\)", "(v[j] + u[j])")]),
    ("readout of S, not S^T", [(r"o\[j\] \+= q\[c\] \* S\[c \* dv \+ j\];",
                                "o[j] += q[c] * S[(j % dk) * dv + (c % dv)];")]),
    ("beta squared", [(r"S\[c \* dv \+ j\] \+= b \* k", "S[c * dv + j] += b * b * k")]),
    ("beta dropped", [(r"S\[c \* dv \+ j\] \+= b \* k", "S[c * dv + j] += k")]),
    # decay applied after the erase and write instead of before them
    ("decay after the write", [(_DECAY, ";"),
                               (r"        /\* readout o = S\^T q \*/",
                                "        " + _DECAY_TEXT + "\n        /* readout */")]),
    # the readout taken from the state before token t's erase and write
    ("readout before the write", [(_READOUT, ""),
                                  (r"        /\* erase along k and write k v\^T",
                                   _READOUT_TEXT + "        /* erase along k and write k v^T")]),
]

# Mistakes in the backward's adjoint steps (each pattern occurs only there).
BWD_MUTANTS = [
    ("bwd readout term dropped", r"dS\[c \* dv \+ j\] \+= q\[c\] \* dO\[j\];", ";"),
    ("bwd erase term dropped", r"dS\[c \* dv \+ j\] \+= k\[c\] \* \(-b \* dd\[j\]\);", ";"),
    ("bwd gate gradient against S_t", r"acc \+= dS\[c \* dv \+ j\] \* P\[c \* dv \+ j\];",
     "acc += dS[c * dv + j] * S[c * dv + j];"),
    ("bwd state gradient not decayed", r"dS\[c \* dv \+ j\] \*= a\[c\];", ";"),
    ("bwd beta gradient without u", r"db \+= \(v\[j\] - u\[j\]\) \* dd\[j\];",
     "db += v[j] * dd[j];"),
    ("bwd key gradient against the old state",
     r"acc \+= Sp\[c \* dv \+ j\] \* \(-b \* dd\[j\]\);",
     "acc += P[c * dv + j] * (-b * dd[j]);"),
    ("bwd query gradient against S'", r"acc \+= S\[c \* dv \+ j\] \* dO\[j\];",
     "acc += Sp[c * dv + j] * dO[j];"),
]

BWD_PIN_TESTS = [
    bpins.test_backward_matches_finite_differences_uniform,
    bpins.test_backward_matches_finite_differences_packed,
    bpins.test_backward_beta_zero_unit_gate_closed_form,
    bpins.test_backward_first_token_from_zero_state_closed_form,
]

PIN_TESTS = [
    lambda: [pins.test_householder_dial(r) for r in pins._golden.load("householder_dial.txt")],
    pins.test_beta_zero_keeps_state_and_reads_it,
    pins.test_beta_zero_is_pure_gate_decay,
    pins.test_projection_erases_key_direction,
    pins.test_first_token_from_zero_state,
    pins.test_quarter_turn_golden,
    lambda: [pins.test_closed_form_2x2(r) for r in pins._golden.load("closed_form_rotation.txt")],
    lambda: [pins.test_sign_condition(r) for r in pins._golden.load("sign_condition.txt")],
    pins.test_orthogonal_and_non_expansive,
]


def _build_mutant(src, tmp):
    path = os.path.join(tmp, "mut.c")
    with open(path, "w") as f:
        f.write(src)
    so = os.path.join(tmp, "libmut.so")
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", "-pthread", path,
                           "-o", so])
    return so


def _pins_fail(tests=None):
    for t in (PIN_TESTS if tests is None else tests):
        try:
            with np.errstate(all="ignore"):
                t()
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            return True
    return False


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, edits, monkeypatch):
    mutated = open(SRC).read()
    for pat, rep in edits:
        mutated, n = re.subn(pat, lambda m, r=rep: r, mutated, count=1)
        assert n == 1, f"mutation pattern no longer matches the oracle source: {pat}"
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(mutated, tmp)
        monkeypatch.setattr(oracle, "_LIB_PATH", so)
        monkeypatch.setattr(oracle, "_lib", None)
        assert _pins_fail(), f"no pin caught the planted mistake: {name}"
    monkeypatch.setattr(oracle, "_lib", None)


@pytest.mark.parametrize("name,pat,rep", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_pins_catch_mutant(name, pat, rep, monkeypatch):
    src = open(SRC).read()
    mutated, n = re.subn(pat, rep, src)
    assert n == 1, "mutation pattern must match exactly one place in the backward"
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(mutated, tmp)
        monkeypatch.setattr(oracle, "_LIB_PATH", so)
        monkeypatch.setattr(oracle, "_lib", None)
        assert _pins_fail(BWD_PIN_TESTS), f"no backward pin caught the planted mistake: {name}"
    monkeypatch.setattr(oracle, "_lib", None)


def test_unmutated_oracle_passes_pins():
    assert not _pins_fail()
    assert not _pins_fail(BWD_PIN_TESTS)
