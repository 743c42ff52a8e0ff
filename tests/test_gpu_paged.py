"""GPU parity of attn_decode_paged_fwd (decode over a block-table KV cache)
against the float64 oracle, and against the contiguous decode path (MI355X only)."""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import TOL_LSE, TOL_O, check_lse, max_abs_err, to_device, to_host64
from oracle import attention_paged_ref

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _paged_case(B, Hq, Hkv, d, bs, maxb, lens, Nq, causal, dtype, seed, poison=False):
    _announce(f"paged B={B} Hq={Hq} Hkv={Hkv} d={d} bs={bs} maxb={maxb} Nq={Nq} causal={causal} "
              f"{dtype} lens={list(lens)[:6]}")
    lens = np.asarray(lens, np.int32)
    table, nblk = A.paged_layout(lens, bs, maxb, seed=seed, spare=3)
    q = A.random_tensor((B, Hq, Nq, d), seed * 3, dtype)
    kp = A.random_tensor((nblk, Hkv, bs, d), seed * 3 + 1, dtype)
    vp = A.random_tensor((nblk, Hkv, bs, d), seed * 3 + 2, dtype)
    kd, vd = to_device(kp, dtype), to_device(vp, dtype)
    tab = table.copy()
    if poison:
        # blocks no request uses, and table entries past each request's blocks,
        # must never be read
        used = set(int(x) for x in table[table >= 0])
        for p in range(nblk):
            if p not in used:
                kd[p] = float("nan")
                vd[p] = float("nan")
        tab[table < 0] = 123456789
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = E.attn_decode_paged_fwd(to_device(q, dtype), kd, vd, torch.from_numpy(tab).cuda(),
                                     kv_lens=torch.from_numpy(lens).cuda(), causal=causal,
                                     scale=scale, return_lse=True)
    torch.cuda.synchronize()
    oref, lref = attention_paged_ref(q, kp, vp, table, lens, bs, causal, scale)
    got = to_host64(o)
    assert np.all(np.isfinite(got))
    err = max_abs_err(got, oref)
    assert err <= TOL_O[dtype], f"max |err| {err}"
    check_lse(lse.cpu().numpy().astype(np.float64), lref, TOL_LSE[dtype])


PAGED = [
    # B, Hq, Hkv, d, block_size, max_blocks, lens, Nq
    (3, 8, 1, 128, 16, 200, [3200, 1, 1777], 1),
    (2, 32, 4, 128, 32, 80, [2560, 900], 1),
    (4, 16, 2, 64, 64, 40, [2560, 2500, 64, 65], 1),
    (2, 8, 2, 128, 256, 12, [3000, 257], 4),
    (2, 16, 2, 128, 16, 300, [4800, 2049], 6),
    (1, 4, 4, 64, 4096, 2, [5000], 2),
    (2, 8, 1, 128, 128, 3, [0, 300], 1),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", PAGED, ids=lambda c: f"bs{c[4]}x{c[3]}x{c[7]}")
def test_paged_decode_matches_oracle(case, dtype):
    B, Hq, Hkv, d, bs, maxb, lens, Nq = case
    seed = zlib.crc32(repr((case, dtype)).encode()) % 10000
    _paged_case(B, Hq, Hkv, d, bs, maxb, lens, Nq, Nq > 1, dtype, seed)


@pytest.mark.parametrize("bs", [16, 64])
def test_paged_decode_never_reads_unreferenced_memory(bs):
    _paged_case(3, 16, 2, 128, bs, 3000 // bs + 2, [2999, 5, 1500], 3, True, "bf16", seed=81,
                poison=True)


@pytest.mark.parametrize("bs", [16, 128])
def test_paged_equals_contiguous_bit_for_bit(bs, tune):
    """A contiguous cache laid out as pool blocks (in a shuffled order) gives the
    same bits through the paged path as through the contiguous path: the
    arithmetic is the same, only the addressing differs. (Both held to one split
    size: the two paths may otherwise choose different ones.)"""
    tune(decode_chunk=512)
    B, Hq, Hkv, d, N = 3, 16, 2, 128, 4096
    _announce(f"paged vs contiguous bs={bs}")
    q = to_device(A.random_tensor((B, Hq, 2, d), 61, "bf16"), "bf16")
    k = to_device(A.random_tensor((B, Hkv, N, d), 62, "bf16"), "bf16")
    v = to_device(A.random_tensor((B, Hkv, N, d), 63, "bf16"), "bf16")
    lens = torch.tensor([4096, 1000, 17], dtype=torch.int32, device="cuda")
    nb = N // bs
    perm = torch.from_numpy(np.random.default_rng(5).permutation(B * nb).astype(np.int64)).cuda()
    # logical block (b, i) lives in pool block perm[b * nb + i]
    kb = k.reshape(B, Hkv, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, d)
    vb = v.reshape(B, Hkv, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, d)
    kp = torch.empty_like(kb)
    vp = torch.empty_like(vb)
    kp[perm] = kb
    vp[perm] = vb
    table = perm.to(torch.int32).reshape(B, nb).contiguous()
    oc, lc = E.attn_decode_fwd(q, k, v, kv_lens=lens, causal=True, return_lse=True)
    op, lp = E.attn_decode_paged_fwd(q, kp, vp, table, kv_lens=lens, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(oc, op)
    assert torch.equal(lc, lp)


def test_paged_invalid_table_entry_reads_zeros_and_spares_other_requests():
    """An entry outside the pool reads as zero keys and values, touching nothing
    outside the pool; the other requests' results are unaffected."""
    _announce("paged invalid entry")
    B, Hq, Hkv, d, bs, maxb = 2, 8, 1, 128, 16, 8
    lens = np.array([128, 128], np.int32)
    table, nblk = A.paged_layout(lens, bs, maxb, seed=4)
    q = to_device(A.random_tensor((B, Hq, 1, d), 71, "bf16"), "bf16")
    kp = to_device(A.random_tensor((nblk, Hkv, bs, d), 72, "bf16"), "bf16")
    vp = to_device(A.random_tensor((nblk, Hkv, bs, d), 73, "bf16"), "bf16")
    lens_d = torch.from_numpy(lens).cuda()
    good = E.attn_decode_paged_fwd(q, kp, vp, torch.from_numpy(table).cuda(), kv_lens=lens_d)
    bad_table = table.copy()
    bad_table[1, 3] = nblk + 1000
    bad = E.attn_decode_paged_fwd(q, kp, vp, torch.from_numpy(bad_table).cuda(), kv_lens=lens_d)
    torch.cuda.synchronize()
    assert torch.equal(good[0], bad[0])
    assert torch.isfinite(bad[1].float()).all()
