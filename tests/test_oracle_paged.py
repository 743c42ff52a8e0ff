"""Pins of the paged-cache oracle (gather by block table, then exact attention)
against facts that do not come from the oracle's own gather: a pool laid out
from a contiguous cache with the identity table, position-by-position brute
force, invariance under relabelling the pool's blocks, and blindness to
everything the block table does not point at below the request's length."""
import numpy as np

import attn_inputs as A
from oracle import attention_paged_ref, attention_ref, gather_paged


def _pool_from_cache(cache, bs):
    """Lay a contiguous cache [B, H, N, d] out as pool blocks, block (b, i) -> b*nb + i."""
    B, H, N, d = cache.shape
    nb = N // bs
    pool = cache.reshape(B, H, nb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nb, H, bs, d)
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    return pool, table


def test_identity_table_is_the_contiguous_cache():
    B, Hq, Hkv, N, d, bs = 3, 4, 2, 64, 16, 16
    q = A.random_tensor((B, Hq, 2, d), 501, "bf16")
    k = A.random_tensor((B, Hkv, N, d), 502, "bf16")
    v = A.random_tensor((B, Hkv, N, d), 503, "bf16")
    lens = np.array([64, 17, 1], np.int32)
    kp, table = _pool_from_cache(k, bs)
    vp, _ = _pool_from_cache(v, bs)
    for causal in (False, True):
        o1, l1 = attention_paged_ref(q, kp, vp, table, lens, bs, causal, 0.25)
        o2, l2 = attention_ref(q, k, v, causal, 0.25, kv_lens=lens)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_gather_brute_force_positions():
    B, H, d, bs, maxb = 2, 3, 4, 16, 5
    lens = np.array([70, 33], np.int32)
    table, nblocks = A.paged_layout(lens, bs, maxb, seed=7, spare=3)
    pool = A.random_tensor((nblocks, H, bs, d), 504, "f32")
    g = gather_paged(pool, table, lens, bs)
    for b in range(B):
        for p in range(int(lens[b])):
            blk = int(table[b][p // bs])
            for h in range(H):
                assert list(g[b, h, p]) == list(pool[blk, h, p % bs])


def test_relabelling_pool_blocks_changes_nothing():
    B, Hq, Hkv, d, bs, maxb = 2, 8, 1, 32, 16, 6
    lens = np.array([90, 41], np.int32)
    table, nblocks = A.paged_layout(lens, bs, maxb, seed=8, spare=2)
    kp = A.random_tensor((nblocks, Hkv, bs, d), 505, "f16")
    vp = A.random_tensor((nblocks, Hkv, bs, d), 506, "f16")
    q = A.random_tensor((B, Hq, 3, d), 507, "f16")
    o1, l1 = attention_paged_ref(q, kp, vp, table, lens, bs, True, 0.2)
    perm = np.random.default_rng(0).permutation(nblocks)      # new label of block p
    inv = np.argsort(perm)
    t2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    o2, l2 = attention_paged_ref(q, kp[inv], vp[inv], t2, lens, bs, True, 0.2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_unreferenced_blocks_and_entries_are_never_read():
    B, Hq, Hkv, d, bs, maxb = 2, 4, 2, 16, 32, 4
    lens = np.array([40, 64], np.int32)
    table, nblocks = A.paged_layout(lens, bs, maxb, seed=9, spare=2)
    kp = A.random_tensor((nblocks, Hkv, bs, d), 508, "bf16")
    vp = A.random_tensor((nblocks, Hkv, bs, d), 509, "bf16")
    q = A.random_tensor((B, Hq, 1, d), 510, "bf16")
    o1, _ = attention_paged_ref(q, kp, vp, table, lens, bs, False, 0.25)
    used = set(int(x) for x in table[table >= 0])
    kp2, vp2 = kp.copy(), vp.copy()
    for p in range(nblocks):
        if p not in used:
            kp2[p] = np.nan
            vp2[p] = np.nan
    t2 = table.copy()
    t2[table < 0] = 10 ** 6          # entries past the needed blocks are garbage
    o2, _ = attention_paged_ref(q, kp2, vp2, t2, lens, bs, False, 0.25)
    np.testing.assert_array_equal(o1, o2)


def test_paged_layout_allocates_distinct_blocks():
    lens = np.array([1, 16, 17, 0, 100], np.int32)
    table, nblocks = A.paged_layout(lens, 16, 8, seed=3, spare=5)
    need = [1, 1, 2, 0, 7]
    assert nblocks == sum(need) + 5
    got = table[table >= 0]
    assert len(got) == sum(need) and len(set(got.tolist())) == len(got)
    for b, n in enumerate(need):
        assert np.all(table[b, :n] >= 0) and np.all(table[b, n:] == -1)
