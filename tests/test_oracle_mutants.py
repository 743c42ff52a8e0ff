"""Planted mistakes in a copy of the oracle must each fail a pin (CPU only).

Each mutant is the oracle's own source with one plausible error edited in
(dropped term, wrong sign, wrong index, transposed operand, wrong alignment).
The battery below uses only checks that do not trust the oracle: brute force in
pure Python, torch's float64 SDPA on square shapes and closed forms.
"""
import math
import os
import types

import numpy as np
import pytest

import oracle.attention as ref_mod
from test_oracle_pins import _brute, _sdpa

SRC = open(ref_mod.__file__).read()

MUTANTS = {
    "dropped scale": ("scores = (qq @ kk.T) * float(scale)", "scores = (qq @ kk.T)"),
    "causal off by one": ("masked = keys[None, :] > (r[:, None] + off)",
                          "masked = keys[None, :] >= (r[:, None] + off)"),
    "top-left causal alignment": ("off = n - N_q", "off = 0"),
    "wrong GQA head map": ("g = h // G", "g = h % H_kv"),
    "V used for scores": ("scores = (qq @ kk.T)", "scores = (qq @ vv.T)"),
    "no max subtraction": ("p = np.exp(s - m[..., None])", "p = np.exp(s)"),
    "max over the wrong axis": ("m = s.max(axis=-1)", "m = s.max(axis=0)"),
    "unnormalised output": ("out = (p @ vv) / l[:, None]", "out = (p @ vv)"),
    "lse sign": ("row_lse = m + np.log(l)", "row_lse = m - np.log(l)"),
    "kv_lens ignored": ("n = N_kv if kv_lens is None else int(kv_lens[b])", "n = N_kv"),
    "empty rows not zeroed": ("out[empty] = 0.0", "pass"),
}


def _load(src):
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _battery(mod) -> bool:
    """True iff the module passes every independent check."""
    rng = np.random.default_rng(7)
    try:
        for (B, Hq, Hkv, Nq, Nkv, d, causal, lens) in [
            (1, 4, 2, 3, 5, 4, True, None), (2, 2, 1, 5, 3, 3, True, None),
            (2, 2, 2, 4, 4, 3, False, None), (3, 2, 1, 1, 6, 4, True, [6, 2, 0]),
        ]:
            q = rng.standard_normal((B, Hq, Nq, d))
            k = rng.standard_normal((B, Hkv, Nkv, d))
            v = rng.standard_normal((B, Hkv, Nkv, d))
            with np.errstate(all="ignore"):
                o, lse = mod.attention_ref(q, k, v, causal, 0.7, kv_lens=lens)
            ob, lb = _brute(q, k, v, causal, 0.7, kv_lens=lens)
            if not np.allclose(o, ob, atol=1e-10, rtol=0) or not np.array_equal(np.isinf(lse), np.isinf(lb)):
                return False
            fin = np.isfinite(lb)
            if not np.allclose(lse[fin], lb[fin], atol=1e-10):
                return False
        # large score offsets (torch SDPA float64 is the reference)
        q = rng.standard_normal((1, 2, 9, 8)) * 30
        k = rng.standard_normal((1, 2, 9, 8)) * 30
        v = rng.standard_normal((1, 2, 9, 8))
        for causal in (False, True):
            with np.errstate(all="ignore"):
                o, _ = mod.attention_ref(q, k, v, causal, 1 / math.sqrt(8))
            if not np.allclose(o, _sdpa(q, k, v, causal, 1 / math.sqrt(8)), atol=1e-10):
                return False
    except Exception:
        return False
    return True


def test_unmodified_oracle_passes_battery():
    assert _battery(_load(SRC))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name!r} not found"
    assert not _battery(_load(SRC.replace(old, new))), f"mutant {name!r} survived the pins"
