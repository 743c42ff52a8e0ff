"""Planted mistakes in a copy of the backward oracle must each fail a pin that
does not trust it: central finite differences of the (separately pinned)
forward oracle, on small causal and non-causal GQA shapes (CPU only)."""
import types

import numpy as np
import pytest

import oracle.backward as bwd_mod
from oracle import attention_ref

SRC = open(bwd_mod.__file__).read()

MUTANTS = {
    "dropped row term": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "dq without scale": ("dq = float(scale) * (ds @ k)", "dq = (ds @ k)"),
    "dk from dS not transposed": ("dk = float(scale) * (ds.T @ q)", "dk = float(scale) * (ds.T @ q) * 0 + float(scale) * (p.T @ q)"),
    "dv from P not transposed": ("dv = p.T @ do", "dv = p.T @ (do * 0 + q)"),
    "top-left causal": ("off = n - N_q", "off = 0"),
    "GQA grads not summed": ("dk[b, g] += bk", "dk[b, g] = bk"),
    "dp with K instead of V": ("dp = do @ v.T", "dp = do @ k.T"),
}


def _load(src):
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src, "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod


def _fd_ok(mod) -> bool:
    rng = np.random.default_rng(11)
    for (B, Hq, Hkv, Nq, Nkv, d, causal) in [(1, 4, 2, 3, 5, 3, True), (1, 2, 1, 4, 4, 3, False)]:
        q = rng.standard_normal((B, Hq, Nq, d))
        k = rng.standard_normal((B, Hkv, Nkv, d))
        v = rng.standard_normal((B, Hkv, Nkv, d))
        do = rng.standard_normal((B, Hq, Nq, d))
        with np.errstate(all="ignore"):
            grads = mod.attention_backward_ref(q, k, v, do, causal, 0.6)

        def loss():
            o, _ = attention_ref(q, k, v, causal, 0.6)
            return float((o * do).sum())
        for x, g in zip((q, k, v), grads):
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                i = it.multi_index
                old = x[i]
                x[i] = old + 1e-6
                lp = loss()
                x[i] = old - 1e-6
                lm = loss()
                x[i] = old
                if not abs((lp - lm) / 2e-6 - g[i]) <= 1e-6 * max(1.0, abs(g[i])):
                    return False
    return True


def test_unmutated_backward_oracle_passes():
    assert _fd_ok(_load(SRC))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name!r} not found"
    assert not _fd_ok(_load(SRC.replace(old, new)))
