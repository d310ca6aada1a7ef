"""Mutation check of the Q4_K oracle's pins: plausible mistakes planted into
a copy of oracle/q4k.py (in memory, on the CPU) must each make at least one
pin of tests/test_oracle_q4k.py fail."""
import os
import types

import pytest

import test_oracle_q4k as PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "q4k.py")

MUTANTS = {
    "nibble halves swapped": ("for half, j in ((0, 2 * p), (1, 2 * p + 1)):",
                              "for half, j in ((1, 2 * p), (0, 2 * p + 1)):"),
    "sub-blocks p and p+4 per run": (
        "for half, j in ((0, 2 * p), (1, 2 * p + 1)):",
        "for half, j in ((0, p), (1, p + 4)):"),
    "high scale bits from the min byte": ("((s[j - 4] >> 6) << 4)",
                                          "((s[j] >> 6) << 4)"),
    "scale and min nibbles swapped": (
        "sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4)\n"
        "            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)",
        "sc[j] = (s[j + 4] >> 4) | ((s[j - 4] >> 6) << 4)\n"
        "            mn[j] = (s[j + 4] & 15) | ((s[j] >> 6) << 4)"),
    "five-bit fields": ("sc[j] = s[j] & 63", "sc[j] = s[j] & 31"),
    "d and dmin swapped": ("d * sc[j] * q - dmin * mn[j]",
                           "dmin * sc[j] * q - d * mn[j]"),
    "min added": ("d * sc[j] * q - dmin * mn[j]", "d * sc[j] * q + dmin * mn[j]"),
    "quants read from the header": ("qs = blk[16:144]", "qs = blk[0:128]"),
    "weight not transposed": ("return x @ W.T", "return x @ W"),
    "row blocks interleaved": (
        "wq = _u8(wq).reshape(rows, cols // BLOCK_VALUES, BLOCK_BYTES)",
        "wq = _u8(wq).reshape(cols // BLOCK_VALUES, rows, BLOCK_BYTES)"
        ".transpose(1, 0, 2)"),
}


def _pins():
    return [getattr(PINS, n) for n in dir(PINS) if n.startswith("test_")]


def _run_pins(module):
    saved = PINS.Q
    PINS.Q = module
    try:
        for fn in _pins():
            fn()
        return True
    except (AssertionError, ValueError, IndexError):
        return False
    finally:
        PINS.Q = saved


def test_pins_pass_on_the_oracle():
    from oracle import q4k
    assert _run_pins(q4k)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    mod = types.ModuleType("q4k_mutant")
    exec(compile(src.replace(old, new), "q4k_mutant", "exec"), mod.__dict__)
    assert not _run_pins(mod), "mutant '%s' survived every pin" % name
