"""Every planted oracle mistake is caught by at least one pin (CPU only).

The oracle source carries a compile-time switch that plants one plausible
mistake at a time (nibble order, a dropped offset or term, a flipped sign, a
wrong fp16 exponent bias, a transposed or scrambled operand). Each mutant is
built into a temporary directory and run against the pins.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    1: "Q4_0 sequential nibble order",
    2: "Q4_0 offset 8 dropped",
    3: "Q4_K high bits of sc dropped",
    4: "Q4_K min term sign flipped",
    5: "Q4_K low/high nibble halves swapped",
    6: "Q8_0 codes read unsigned",
    7: "fp16 subnormals decoded as normals",
    8: "fp16 exponent bias off by one",
    9: "fp32 GEMM reads B transposed",
    10: "quantized GEMM k index scrambled",
    11: "Q6_K high bits at the wrong shift",
    12: "Q6_K low-bit nibble halves swapped",
    13: "Q2_K scale and min nibbles swapped",
    14: "int4 codes not sign-extended",
    15: "int4 zero point added instead of subtracted",
    16: "int4 nibble order reversed within a word",
    17: "q1_0 code bits read most significant first",
    18: "q1_0 codes read as 0 / +d instead of -d / +d",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_mutant_is_caught(tmp_path, mutant):
    path = oracle.build(mutant=mutant, out=os.path.join(tmp_path, f"liboracle_m{mutant}.so"))
    o = oracle.Oracle(path)
    assert o.mutant == mutant
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"
