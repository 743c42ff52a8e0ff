"""The online-softmax recurrence (m, l, u; rescale by exp(m - m')) reaches the
oracle's result in float64 for any block size, with lazy rescaling, and across
split-KV partitions merged by log-sum-exp (CPU only)."""
import numpy as np
import pytest

from blockwise_model import merge_partials, online_rows
from oracle import attention_ref

rng = np.random.default_rng(99)


def _vis(Nq, n, causal):
    i = np.arange(Nq)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i + (n - Nq)) if causal else np.ones((Nq, n), bool)


@pytest.mark.parametrize("block", [1, 3, 16, 64, 1000])
@pytest.mark.parametrize("lazy,lazy_sum", [(0.0, None), (8 * np.log(2), None), (0.0, 256.0)])
@pytest.mark.parametrize("causal,Nq,n", [(False, 37, 53), (True, 50, 50), (True, 20, 45), (True, 30, 10)])
def test_blockwise_equals_definition(block, lazy, lazy_sum, causal, Nq, n):
    d = 16
    q = rng.standard_normal((Nq, d)) * 2
    k = rng.standard_normal((n, d)) * 2
    v = rng.standard_normal((n, d))
    o, m, l = online_rows(q, k, v, 0.25, _vis(Nq, n, causal), block, lazy, lazy_sum)
    oref, lref = attention_ref(q[None, None], k[None, None], v[None, None], causal, 0.25)
    np.testing.assert_allclose(o, oref[0, 0], atol=1e-12)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, np.where(np.isfinite(m), m, 0) + np.log(np.where(l > 0, l, 1)), -np.inf)
    np.testing.assert_allclose(lse, lref[0, 0], atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 7, 64, 512])
def test_split_kv_merge_equals_definition(chunk):
    G, n, d = 8, 300, 32
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    ms, ls, us = [], [], []
    for s0 in range(0, max(n, 1), chunk):
        vis = np.ones((G, min(chunk, n - s0)), bool)
        _, m, l = online_rows(q, k[s0:s0 + chunk], v[s0:s0 + chunk], 0.2, vis, 16)
        o_s, _, _ = online_rows(q, k[s0:s0 + chunk], v[s0:s0 + chunk], 0.2, vis, 16)
        ms.append(m); ls.append(l); us.append(o_s * l[:, None])
    # an empty split (m = -inf, l = 0) must contribute nothing
    ms.append(np.full(G, -np.inf)); ls.append(np.zeros(G)); us.append(np.zeros((G, d)))
    o, lse = merge_partials(ms, ls, us)
    oref, lref = attention_ref(q[None, :, None, :], k[None, None], v[None, None], False, 0.2)
    np.testing.assert_allclose(o, oref[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(lse, lref[0, :, 0], atol=1e-12)
