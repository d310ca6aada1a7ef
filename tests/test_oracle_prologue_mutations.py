"""Mutation check of the prologue oracle's pins: plausible mistakes planted
into a copy of oracle/prologue.py (in memory, on the CPU) must each make at
least one pin of tests/test_oracle_prologue.py fail."""
import importlib.util
import os
import sys
import types

import pytest

import test_oracle_prologue as PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "prologue.py")

MUTANTS = {
    "bias dropped": ("acc = np.zeros(C) if bias is None else bias.copy()",
                     "acc = np.zeros(C)"),
    "window shifted": ("acc = acc + w[:, j] * xe[t + j]",
                       "acc = acc + w[:, j] * xe[min(t + j + 1, xe.shape[0] - 1)]"),
    "taps reversed": ("acc = acc + w[:, j] * xe[t + j]",
                      "acc = acc + w[:, W - 1 - j] * xe[t + j]"),
    "sigmoid for SiLU": ("return x / (1.0 + np.exp(-x))",
                         "return 1.0 / (1.0 + np.exp(-x))"),
    "eps outside root": ("np.sqrt(np.sum(h * h, axis=-1, keepdims=True) + eps)",
                         "(np.sqrt(np.sum(h * h, axis=-1, keepdims=True)) + eps)"),
    "state order reversed": ("head = s0[n].T if s0 is not None",
                             "head = s0[n].T[::-1] if s0 is not None"),
    "state ignored": ("head = s0[n].T if s0 is not None",
                      "head = np.zeros((W - 1, C)) if True"),
    "final state first inputs": ("final[n] = xe[xe.shape[0] - (W - 1):].T",
                                 "final[n] = xe[:W - 1].T"),
    "q and k swapped": ("q = l2norm_heads(y[:, :cq], d_k, eps)",
                        "q = l2norm_heads(y[:, cq:2 * cq], d_k, eps)"),
    "v normalized": ("v = y[:, 2 * cq:].reshape(T, h_v, d_v)",
                     "v = l2norm_heads(y[:, 2 * cq:], d_v, eps).reshape(T, h_v, d_v)"),
}


def _pins():
    return [getattr(PINS, n) for n in dir(PINS) if n.startswith("test_")]


def _run_pins(module):
    """True if every pin passes with `module` standing in for the oracle."""
    saved = PINS.P
    PINS.P = module
    try:
        for fn in _pins():
            if fn.__name__ == "test_l2norm_eps_inside_root":
                for eps in (1e-6, 1.0):
                    fn(eps)
            else:
                fn()
        return True
    except AssertionError:
        return False
    finally:
        PINS.P = saved


def test_pins_pass_on_the_oracle():
    from oracle import prologue
    assert _run_pins(prologue)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    mod = types.ModuleType("prologue_mutant")
    exec(compile(src.replace(old, new), "prologue_mutant", "exec"), mod.__dict__)
    assert not _run_pins(mod), "mutant '%s' survived every pin" % name
