"""Planted mistakes in the oracle must each turn a pin red.

Every mutant is the oracle's own C source built with -DW4O_PLANT=<n>, which
compiles exactly one deliberate error in (see the list in the C file).  A
mutant that passes every pin would mean the pins cannot tell that mistake from
the definition.  Runs on the CPU only.
"""
import os

import pytest

import oracle
import pins

PLANTS = {
    1: "high nibble first",
    2: "bias dropped",
    3: "group of 32",
    4: "tie to the higher id",
    5: "no non-finite flag",
    6: "bias sign flipped",
    7: "scale/bias tables read as [G][N]",
    8: "-0.0 ordered below +0.0",
    9: "fp32 accumulation",
    10: "activation row stride taken from N",
    11: "last K group dropped",
    12: "runner-up tie to the higher id",
    13: "bf16 store ties away from zero",
    14: "high field first at other widths",
    15: "8-bit rows at the 4-bit pitch",
}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: f"{p}-{PLANTS[p].replace(' ', '_')}")
def test_plant_is_red(plant, tmp_path):
    path = oracle.build(plant=plant, out=os.path.join(str(tmp_path), f"liboracle_plant{plant}.so"))
    lib = oracle.load(path)
    assert lib.w4o_plant() == plant
    red = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            red.append(pin.__name__)
    assert red, f"planted mistake {plant} ({PLANTS[plant]}) passed every pin"
    print(f"plant {plant} ({PLANTS[plant]}): red on {', '.join(red)}")
