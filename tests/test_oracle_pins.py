"""Pins of the float64 oracle against facts fixed outside it (CPU only).

Each check compares the oracle with something it does not compute itself: values
the pages print, closed forms, textbook special cases, a library routine (torch's
CPU scaled_dot_product_attention in float64), or brute force in pure Python.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- printed values
def test_score_bytes_match_printed_table():
    rows = _rows("score_bytes_fp32.txt")
    assert len(rows) == 4
    for n, mib in rows:
        assert oracle.score_bytes(int(n), 4) == int(mib) * oracle.MiB


def test_score_and_cache_bytes_at_8192_tokens():
    for qty, tokens, heads, layers, bpe, gib in _rows("score_vs_cache_8192.txt"):
        tokens, heads, layers, bpe, gib = map(int, (tokens, heads, layers, bpe, gib))
        if qty == "scores":
            got = layers * heads * oracle.score_bytes(tokens, bpe)
        else:
            got = oracle.kv_cache_bytes(layers, tokens, heads, 128, bpe)
        assert got == gib * 2 ** 30


def test_visible_pair_counts_closed_forms():
    # non-causal: every pair; causal square: N(N+1)/2 ("about half the work")
    for n in (1, 2, 7, 512, 4096):
        assert oracle.visible_pairs(n, n, False) == n * n
        assert oracle.visible_pairs(n, n, True) == n * (n + 1) // 2
    # decode (one query) sees all n cached keys, causal or not
    assert oracle.visible_pairs(1, 32768, True) == 32768
    # more queries than keys under bottom-right alignment: the first N_q-n rows see nothing
    assert oracle.visible_pairs(5, 3, True) == 0 + 0 + 1 + 2 + 3
    # brute force
    for nq, n in itertools.product(range(0, 6), range(0, 6)):
        bf = sum(1 for i in range(nq) for j in range(n) if j <= i + n - nq)
        assert oracle.visible_pairs(nq, n, True) == bf


# ---------------------------------------------------------------- brute force
def _brute(q, k, v, causal, scale, kv_lens=None):
    """Pure-Python loops with math.exp / math.fsum over every (b, h, i, j)."""
    B, Hq, Nq, d = q.shape
    _, Hkv, Nkv, dv = v.shape
    G = Hq // Hkv
    o = np.zeros((B, Hq, Nq, dv))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        n = Nkv if kv_lens is None else int(kv_lens[b])
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                vis = [j for j in range(n) if (not causal) or j <= i + (n - Nq)]
                if not vis:
                    o[b, h, i] = 0.0
                    lse[b, h, i] = -math.inf
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, t]) * float(k[b, g, j, t]) for t in range(d))
                     for j in vis}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in vis}
                tot = math.fsum(w.values())
                for c in range(dv):
                    o[b, h, i, c] = math.fsum(w[j] * float(v[b, g, j, c]) for j in vis) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Nq, Nkv, d
    (1, 1, 1, 1, 1, 1), (1, 1, 1, 4, 4, 3), (2, 2, 1, 3, 5, 4), (1, 2, 2, 6, 6, 2),
    (2, 2, 1, 5, 3, 4), (1, 4, 2, 2, 6, 3),
])
def test_brute_force_tiny(shape, causal):
    B, Hq, Hkv, Nq, Nkv, d = shape
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nkv, d))
    v = rng.standard_normal((B, Hkv, Nkv, d))
    scale = 0.7
    o, lse = attention_ref(q, k, v, causal, scale)
    ob, lb = _brute(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def test_brute_force_kv_lens():
    q = rng.standard_normal((3, 2, 1, 4))
    k = rng.standard_normal((3, 1, 6, 4))
    v = rng.standard_normal((3, 1, 6, 4))
    lens = np.array([6, 1, 0])
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, causal, 0.5, kv_lens=lens)
        ob, lb = _brute(q, k, v, causal, 0.5, kv_lens=lens)
        np.testing.assert_allclose(o, ob, atol=1e-12)
        assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))
        np.testing.assert_allclose(lse[:2], lb[:2], atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_constant_scores_give_mean_of_values():
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 5
    q = np.zeros((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    o, lse = attention_ref(q, k, v, False, 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[:, h // 2].mean(axis=1, keepdims=True),
                                                            (B, N, d)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(N), atol=1e-14)
    # causal: prefix means v[0..i]
    o, lse = attention_ref(q, k, v, True, 0.3)
    counts = np.arange(1, N + 1)[:, None]
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h], np.cumsum(v[:, h // 2], axis=1) / counts, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-14)


def test_single_visible_key_returns_that_value_exactly():
    q = rng.standard_normal((1, 1, 7, 8))
    k = rng.standard_normal((1, 1, 7, 8))
    v = rng.standard_normal((1, 1, 7, 8))
    o, _ = attention_ref(q, k, v, True, 0.35)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    o, _ = attention_ref(q[:, :, :1], k, v, False, 0.35, kv_lens=[1])
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])


def test_two_keys_logistic_form():
    q = rng.standard_normal((1, 1, 3, 4))
    k = rng.standard_normal((1, 1, 2, 4))
    v = rng.standard_normal((1, 1, 2, 4))
    sc = 0.9
    o, lse = attention_ref(q, k, v, False, sc)
    for i in range(3):
        s0 = sc * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = sc * float(q[0, 0, i] @ k[0, 0, 1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(o[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1], atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))),
                                   atol=1e-13)


def test_max_shift_invariance_and_overflow_safety():
    """Adding c_i to every score of row i leaves the output unchanged and shifts lse by c_i.
    c_i up to 700 would overflow exp() without the max subtraction."""
    B, H, N, d = 1, 2, 6, 4
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    scale = 0.5
    c = rng.uniform(-700, 700, size=(B, H, N))
    # augment: q' = [q, c/scale], k' = [k, 1] gives s'_ij = s_ij + c_i
    q2 = np.concatenate([q, (c / scale)[..., None]], axis=-1)
    k2 = np.concatenate([k, np.ones((B, H, N, 1))], axis=-1)
    for causal in (False, True):
        o1, l1 = attention_ref(q, k, v, causal, scale)
        o2, l2 = attention_ref(q2, k2, v, causal, scale)
        assert np.all(np.isfinite(o2))
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        np.testing.assert_allclose(l2 - c, l1, atol=1e-9)


# ---------------------------------------------------------------- library routine
def _sdpa(q, k, v, causal, scale, gqa=False):
    t = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(
        *t, is_causal=causal, scale=scale, enable_gqa=gqa).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(2, 4, 4, 33, 16), (1, 8, 2, 70, 64), (1, 2, 1, 129, 128)])
def test_matches_torch_sdpa_float64(B, Hq, Hkv, N, d, causal):
    # square shapes only: torch's is_causal is top-left aligned, which equals
    # bottom-right alignment when N_q == N_kv
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    scale = 1 / math.sqrt(d)
    o, _ = attention_ref(q, k, v, causal, scale)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal, scale, gqa=Hq != Hkv), atol=1e-12)


# ---------------------------------------------------------------- structural
def test_gqa_equals_mha_with_repeated_kv_heads():
    B, Hq, Hkv, N, d = 2, 8, 2, 11, 6
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    G = Hq // Hkv
    for causal in (False, True):
        o1, l1 = attention_ref(q, k, v, causal, 0.4)
        o2, l2 = attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), causal, 0.4)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_equals_last_row_of_causal_prefill():
    B, Hq, Hkv, Nkv, d = 3, 4, 2, 10, 8
    k = rng.standard_normal((B, Hkv, Nkv, d))
    v = rng.standard_normal((B, Hkv, Nkv, d))
    lens = np.array([10, 4, 1])
    qd = rng.standard_normal((B, Hq, 1, d))
    od, ld = attention_ref(qd, k, v, True, 0.6, kv_lens=lens)
    for b, n in enumerate(lens):
        qp = np.concatenate([rng.standard_normal((1, Hq, n - 1, d)), qd[b:b + 1]], axis=2)
        op, lp = attention_ref(qp, k[b:b + 1, :, :n], v[b:b + 1, :, :n], True, 0.6)
        np.testing.assert_allclose(od[b, :, 0], op[0, :, -1], atol=1e-14)
        np.testing.assert_allclose(ld[b, :, 0], lp[0, :, -1], atol=1e-14)


def _softmax_python(row):
    """Softmax of one row in pure Python, written as w_i = 1 / sum_j exp(s_j - s_i)
    (no maximum taken; exact for rows whose entries differ by far less than 700)."""
    fin = [x for x in row if x != -math.inf]
    out = []
    for x in row:
        out.append(0.0 if x == -math.inf else 1.0 / math.fsum(math.exp(y - x) for y in fin))
    return out


def test_softmax_matches_pure_python_closed_form():
    s = rng.standard_normal((6, 11)) * 8
    s[2, 5:] = -np.inf
    s[4, :1] = -np.inf
    w = oracle.softmax_weights(s)
    for i in range(s.shape[0]):
        np.testing.assert_allclose(w[i], _softmax_python(list(s[i])), rtol=1e-13, atol=1e-300)
    # two entries: the logistic function of their difference
    a, b = 1.7, -0.4
    w2 = oracle.softmax_weights(np.array([[a, b]]))[0]
    assert abs(w2[0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
    assert abs(w2[1] - 1.0 / (1.0 + math.exp(a - b))) < 1e-15


def test_softmax_invariant_to_row_offsets_beyond_exp_range():
    """auturnal.com guide, section 8: subtracting the maximum changes only the
    representation. Offsets of +-800 put every exp(s) outside float64's range
    (exp(800) overflows, exp(-800) underflows to 0), so only a softmax that
    subtracts the row maximum returns the same weights."""
    s = rng.standard_normal((5, 9)) * 10
    s[1, 3:] = -np.inf
    w = oracle.softmax_weights(s)
    for c in (800.0, -800.0, 1e5):
        wc = oracle.softmax_weights(s + c)
        assert np.all(np.isfinite(wc))
        np.testing.assert_allclose(wc, w, rtol=0, atol=1e-10)
    p, m, l = oracle.softmax_stats(s + 800.0)
    np.testing.assert_allclose(m, s.max(axis=1) + 800.0, rtol=1e-15)
    assert np.all(p <= 1.0) and np.all(l >= 1.0)


def test_softmax_rows_without_visible_keys():
    s = np.full((2, 4), -np.inf)
    s[1, 2] = 3.0
    p, m, l = oracle.softmax_stats(s)
    assert np.all(p[0] == 0) and m[0] == 0 and l[0] == 0
    assert np.array_equal(oracle.softmax_weights(s), np.array([[0, 0, 0, 0], [0, 0, 1, 0]], float))


SOFTMAX_MUTANTS = {
    "no max subtraction": ("p = np.exp(s - m[..., None])", "p = np.exp(s)"),
    "max over the wrong axis": ("m = s.max(axis=-1)", "m = s.max(axis=0)"),
    "sum over the wrong axis": ("return p, m, p.sum(axis=-1)", "return p, m, p.sum(axis=0)"),
    "minimum instead of maximum": ("m = s.max(axis=-1)", "m = s.min(axis=-1)"),
}


@pytest.mark.parametrize("name", sorted(SOFTMAX_MUTANTS))
def test_softmax_pins_catch_planted_mistakes(name):
    import types
    src = open(oracle.attention.__file__).read()
    old, new = SOFTMAX_MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("softmax_mutant")
    exec(compile(src.replace(old, new), "softmax_mutant", "exec"), mod.__dict__)
    ok = True
    with np.errstate(all="ignore"):
        try:
            saved = oracle.softmax_weights, oracle.softmax_stats
            oracle.softmax_weights, oracle.softmax_stats = mod.softmax_weights, mod.softmax_stats
            try:
                test_softmax_matches_pure_python_closed_form()
                test_softmax_invariant_to_row_offsets_beyond_exp_range()
                test_softmax_rows_without_visible_keys()
            finally:
                oracle.softmax_weights, oracle.softmax_stats = saved
        except Exception:  # noqa: BLE001 (a failed assertion or a shape error)
            ok = False
    assert not ok, f"mutant {name!r} passed the softmax pins"


def test_invariants_weights_hull_permutation():
    s = rng.standard_normal((5, 9)) * 10
    s[1, 3:] = -np.inf
    w = oracle.softmax_weights(s)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-15)
    assert np.all(w[1, 3:] == 0)
    q = rng.standard_normal((1, 1, 12, 4))
    k = rng.standard_normal((1, 1, 12, 4))
    v = rng.standard_normal((1, 1, 12, 4))
    o, _ = attention_ref(q, k, v, True, 1.0)
    for i in range(12):   # each output coordinate is a convex combination of visible values
        assert np.all(o[0, 0, i] <= v[0, 0, :i + 1].max(axis=0) + 1e-12)
        assert np.all(o[0, 0, i] >= v[0, 0, :i + 1].min(axis=0) - 1e-12)
    perm = rng.permutation(12)
    o1, l1 = attention_ref(q, k, v, False, 1.0)
    o2, l2 = attention_ref(q, k[:, :, perm], v[:, :, perm], False, 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_empty_rows_are_zero_with_neg_inf_lse():
    q = rng.standard_normal((1, 1, 5, 3))
    k = rng.standard_normal((1, 1, 2, 3))
    v = rng.standard_normal((1, 1, 2, 3))
    o, lse = attention_ref(q, k, v, True, 1.0)   # 5 queries vs 2 keys: rows 0..2 see nothing
    assert np.all(o[0, 0, :3] == 0) and np.all(np.isneginf(lse[0, 0, :3]))
    assert np.all(np.isfinite(lse[0, 0, 3:]))
    o, lse = attention_ref(q[:, :, :1], k, v, False, 1.0, kv_lens=[0])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_row_sampled_entry_point_matches_full():
    q = rng.standard_normal((1, 2, 40, 8))
    k = rng.standard_normal((1, 1, 40, 8))
    v = rng.standard_normal((1, 1, 40, 8))
    o, lse = attention_ref(q, k, v, True, 0.3)
    rows = np.array([0, 7, 31, 39])
    os_, ls_ = oracle.attention_head_rows(q[0, 1, rows], rows, 40, k[0, 0], v[0, 0], True, 0.3)
    np.testing.assert_array_equal(os_, o[0, 1, rows])
    np.testing.assert_array_equal(ls_, lse[0, 1, rows])
