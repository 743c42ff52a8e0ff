"""Pins of the backward oracle against facts outside it: central finite
differences of the forward oracle, torch autograd in float64, closed forms for
one visible key, and the invariants that a row softmax imposes (shifting every
key by one vector changes nothing, so sum_j dK_j = 0; sum_j dV_j = sum of dO over
rows that see a key)."""
import numpy as np
import pytest
import torch

import attn_inputs as A
from oracle import attention_backward_ref, attention_ref


def _loss(q, k, v, do, causal, scale):
    o, _ = attention_ref(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    B, Hq, Hkv, Nq, Nkv, d = 1, 2, 1, 3, 5, 4
    q = A.random_tensor((B, Hq, Nq, d), 601, "f32").astype(np.float64)
    k = A.random_tensor((B, Hkv, Nkv, d), 602, "f32").astype(np.float64)
    v = A.random_tensor((B, Hkv, Nkv, d), 603, "f32").astype(np.float64)
    do = A.random_tensor((B, Hq, Nq, d), 604, "f32").astype(np.float64)
    scale = 0.7
    dq, dk, dv = attention_backward_ref(q, k, v, do, causal, scale)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _loss(q, k, v, do, causal, scale)
            x[i] = old - eps
            lm = _loss(q, k, v, do, causal, scale)
            x[i] = old
            num[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_float64(causal):
    """torch's math attention in float64 with an explicit bottom-right mask and
    the KV heads repeated per query head; autograd sums the repeats."""
    B, Hq, Hkv, Nq, Nkv, d = 2, 4, 2, 6, 9, 8
    q = A.random_tensor((B, Hq, Nq, d), 611, "bf16")
    k = A.random_tensor((B, Hkv, Nkv, d), 612, "bf16")
    v = A.random_tensor((B, Hkv, Nkv, d), 613, "bf16")
    do = A.random_tensor((B, Hq, Nq, d), 614, "bf16")
    scale = 0.3
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    kk, vv = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
    mask = None
    if causal:
        mask = torch.arange(Nkv)[None, :] <= torch.arange(Nq)[:, None] + (Nkv - Nq)
    o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=mask, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    dq, dk, dv = attention_backward_ref(q, k, v, do, causal, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_one_visible_key_closed_form():
    # each row sees exactly one key (causal, N_q = N_kv = 1): P = 1, so O = v,
    # dV = dO, dS = 0, dQ = dK = 0
    q = A.random_tensor((1, 3, 1, 8), 621, "f32")
    k = A.random_tensor((1, 1, 1, 8), 622, "f32")
    v = A.random_tensor((1, 1, 1, 8), 623, "f32")
    do = A.random_tensor((1, 3, 1, 8), 624, "f32")
    dq, dk, dv = attention_backward_ref(q, k, v, do, True, 0.5)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0, 0], do[0, :, 0].astype(np.float64).sum(axis=0), rtol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_invariants(causal):
    B, Hq, Hkv, Nq, Nkv, d = 2, 4, 1, 7, 11, 16
    q = A.random_tensor((B, Hq, Nq, d), 631, "f16")
    k = A.random_tensor((B, Hkv, Nkv, d), 632, "f16")
    v = A.random_tensor((B, Hkv, Nkv, d), 633, "f16")
    do = A.random_tensor((B, Hq, Nq, d), 634, "f16")
    dq, dk, dv = attention_backward_ref(q, k, v, do, causal, 0.25)
    # a common shift of all keys does not move any row's softmax
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # probabilities of each row sum to one: sum_j dV_j = sum_i dO_i (all rows see keys here)
    np.testing.assert_allclose(dv.sum(axis=2)[:, 0], do.astype(np.float64).sum(axis=(1, 2)), rtol=1e-12,
                               atol=1e-12)


def test_rows_without_keys_contribute_nothing():
    # causal with N_q > N_kv: the first N_q - N_kv rows see no key
    B, Hq, Hkv, Nq, Nkv, d = 1, 2, 2, 6, 3, 8
    q = A.random_tensor((B, Hq, Nq, d), 641, "f32")
    k = A.random_tensor((B, Hkv, Nkv, d), 642, "f32")
    v = A.random_tensor((B, Hkv, Nkv, d), 643, "f32")
    do = A.random_tensor((B, Hq, Nq, d), 644, "f32")
    dq, dk, dv = attention_backward_ref(q, k, v, do, True, 0.5)
    assert np.all(dq[:, :, :3] == 0)
    do2 = do.copy()
    do2[:, :, :3] = 1e3           # gradients arriving at empty rows go nowhere
    _, dk2, dv2 = attention_backward_ref(q, k, v, do2, True, 0.5)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
