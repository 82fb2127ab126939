"""Mutation calibration of the oracle's pins (CPU only).

Each mutant is the oracle built with one planted mistake (ORACLE_MUTATION in
oracle/oracle.c).  Every mutant must fail at least one pin, so a plausible
slip anywhere in the oracle cannot pass unnoticed.  The QSA kernel page
("Validation", mutation calibration) uses the same idea on its own gate:
dropping the sigmoid's bf16 rounding must fail the exact check.
"""

import os
import tempfile

import pytest

import oracle
import oracle_pins

MUTANTS = {
    1: "sigmoid not rounded to bf16",
    2: "wrong sign in the second RoPE half",
    3: "interleaved RoPE pairs",
    4: "eps outside the square root",
    5: "w instead of (1+w)",
    6: "score scale dropped",
    7: "GQA map h % Hkv",
    8: "strict causality",
    10: "mask polarity inverted",
    11: "query position ignores q_base",
    12: "last visible key dropped from the context",
    13: "K read in place of V",
    14: "causal predicate kept in the bidirectional pass",
    15: "keys rotated at position 0 (key position ignored)",
    16: "every KV head's prepared keys taken from KV head 0",
}


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("m", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(mutant_dir, m):
    path = os.path.join(mutant_dir, f"liboracle_m{m}.so")
    oracle.build(out=path, mutation=m)
    o = oracle.Oracle(path)
    assert o.mutation == m
    failed = []
    for pin in oracle_pins.ALL_PINS:
        if pin is oracle_pins.pin_frozen_regression:
            continue          # a frozen copy of the oracle is not an outside pin
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {m} ({MUTANTS[m]}) passes every pin"
