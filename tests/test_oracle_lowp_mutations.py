"""Mutation check of the low-precision oracle's pins: plausible mistakes
planted into a copy of oracle/lowp.py (in memory, on the CPU) must each make
at least one pin of tests/test_oracle_lowp.py fail."""
import os
import types

import pytest

import test_oracle_lowp as PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "lowp.py")

MUTANTS = {
    "ties away from zero": ("if r > 0.5 or (r == 0.5 and f % 2 == 1):",
                            "if r >= 0.5:"),
    "E4M3 bias 8": ("return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
                    "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    "subnormal step halved": ("return sign * (m / 8.0) * 2.0 ** -6",
                              "return sign * (m / 8.0) * 2.0 ** -7"),
    "row scale one binade loose": ("    return max(e, -126)\n",
                                   "    return max(e + 1, -126)\n"),
    "MX scale with emax 3": ("return int(min(254, max(0, 127 + e - 2)))",
                             "return int(min(254, max(0, 127 + e - 3)))"),
    "E2M1 saturating at 5": ("    if a >= 6.0:\n        return sign | 7",
                             "    if a >= 5.0:\n        return sign | 7"),
    "nibbles high first": ("return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)",
                           "return (codes[:, 1::2] | (codes[:, 0::2] << 4)).astype(np.uint8)"),
    "block scales tiled": ("return vals * np.repeat(sc, 32, axis=1)",
                           "return vals * np.tile(sc, (1, 32))"),
    "activation scale dropped": ("X = dequant_fp8(xc, 2.0 ** xe.astype(np.float64))",
                                 "X = dequant_fp8(xc, np.ones(len(xe)))"),
    "E2M1 3 and 4 swapped": ("E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)",
                             "E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 4.0, 3.0, 6.0)"),
}


def _run_pins(module):
    saved = PINS.L
    PINS.L = module
    try:
        for n in dir(PINS):
            if n.startswith("test_"):
                getattr(PINS, n)()
        return True
    except (AssertionError, ValueError, IndexError, KeyError):
        return False
    finally:
        PINS.L = saved


def test_pins_pass_on_the_oracle():
    from oracle import lowp
    assert _run_pins(lowp)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    mod = types.ModuleType("lowp_mutant")
    exec(compile(src.replace(old, new), "lowp_mutant", "exec"), mod.__dict__)
    assert not _run_pins(mod), "mutant '%s' survived every pin" % name
