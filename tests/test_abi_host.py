"""Host-side checks of the C-ABI library (CPU only: no kernel is launched).

The library must load, export every function include/attn.h declares, and turn
every invalid argument into its status code before touching a device."""
import ctypes
import os
import re

import pytest

import exact_attention_31_amd as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytest.importorskip("ctypes")
if not os.path.exists(E.LIB_PATH):
    pytest.skip("libattn.so not built", allow_module_level=True)

L = E.load()
P = ctypes.c_void_p
FAKE = [P(0x10000), P(0x20000000), P(0x40000000), P(0x60000000)]  # never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(attn_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"attn_prefill_fwd", "attn_decode_fwd", "attn_decode_workspace_size",
            "attn_status_string", "attn_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_status_strings():
    for code in range(10):
        assert E.attn_status_string(code) not in ("", "unknown status")
    assert E.attn_status_string(1234) == "unknown status"
    assert E.attn_version() == 100


def pf(q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], lse=None, B=1, Hq=2, Hkv=1, Nq=8, Nkv=8, d=64,
       causal=0, scale=0.125, dtype=E.ATTN_BF16):
    return L.attn_prefill_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, d, causal, scale, dtype, None)


def test_prefill_argument_errors():
    assert pf(q=None) == 1 and pf(o=None) == 1 and pf(k=None) == 1
    assert pf(Nq=-1) == 2 and pf(B=-3) == 2 and pf(B=70000) == 2
    assert pf(Hq=3, Hkv=2) == 3 and pf(Hkv=0) == 3
    assert pf(d=96) == 4 and pf(d=256) == 4 and pf(dtype=7) == 4
    assert pf(scale=float("nan")) == 9 and pf(scale=float("inf")) == 9 and pf(causal=2) == 9
    # the kernels take maxima of raw scores: the scale must be positive
    assert pf(scale=0.0) == 9 and pf(scale=-0.125) == 9
    assert pf(o=FAKE[0]) == 8                       # output aliases q
    assert pf(lse=ctypes.cast(FAKE[3], ctypes.c_void_p)) == 8
    # empty problems are accepted without touching a device
    assert pf(B=0, q=None, k=None, v=None, o=None) == 0
    assert pf(Nq=0) == 0
    # no keys needs no K/V pointer (goes on to the device check)
    assert pf(Nkv=0, k=None, v=None) in (0, 7)


def test_prefill_valid_arguments_reach_the_device_check():
    # this container has no GPU: a valid call must report "no device", not crash
    st = pf()
    assert st in (7,) or st == 0


def ws_size(B=2, Hq=8, Hkv=1, Nq=1, Nkv=1000, d=128, dtype=E.ATTN_BF16):
    return L.attn_decode_workspace_size(B, Hq, Hkv, Nq, Nkv, d, dtype)


def df(ws=P(0x7000000000), wsb=None, Nq=1, dtype=E.ATTN_BF16, lens=None, **kw):
    a = dict(B=2, Hq=8, Hkv=1, Nkv=1000, d=128)
    a.update(kw)
    if wsb is None:
        wsb = ws_size(a["B"], a["Hq"], a["Hkv"], Nq, a["Nkv"], a["d"], dtype)
    return L.attn_decode_fwd(FAKE[0], FAKE[1], FAKE[2], lens, FAKE[3], None, a["B"], a["Hq"],
                             a["Hkv"], Nq, a["Nkv"], a["d"], 0, 0.088, dtype, ws, wsb, None)


def test_decode_workspace_size():
    assert ws_size() > 0
    assert ws_size(Nq=65) == 0 and ws_size(Nq=0) == 0
    assert ws_size(d=80) == 0 and ws_size(Hq=7, Hkv=2) == 0
    # partials: (d + 2) floats per (request, query head, query row, split)
    s = ws_size()
    assert s % ((128 + 2) * 4 * 2 * 8) == 0
    assert ws_size(Nq=5) == 5 * s and ws_size(Nq=64) == 64 * s
    assert ws_size(B=64, Hq=32, Hkv=4, Nkv=32768) >= 64 * 32 * 130 * 4


def test_decode_argument_errors():
    assert df(Nq=65) == 4 and df(dtype=E.ATTN_F32) == 4 and df(d=32) == 4
    assert df(Nq=0, wsb=0) == 0      # nothing to do
    assert df(Nq=64) in (7,) and df(Nq=7) in (7,)
    assert df(Nq=4, wsb=ws_size(Nq=3)) == 5
    assert df(ws=None) == 5 and df(wsb=16) == 5
    assert df(Hq=12, Hkv=8) == 3
    assert df(ws=FAKE[1]) == 8       # workspace overlaps the K cache
    assert df() in (7,)              # valid: reaches the (absent) device


def pws(B=2, Hq=8, Hkv=1, Nq=1, maxb=64, bs=16, d=128, dtype=E.ATTN_BF16):
    return L.attn_decode_paged_workspace_size(B, Hq, Hkv, Nq, maxb, bs, d, dtype)


def pdf(ws=P(0x7000000000), wsb=None, table=P(0x7800000000), Nq=1, dtype=E.ATTN_BF16, **kw):
    a = dict(B=2, Hq=8, Hkv=1, maxb=64, bs=16, nblk=100, d=128)
    a.update(kw)
    if wsb is None:
        wsb = pws(a["B"], a["Hq"], a["Hkv"], Nq, a["maxb"], a["bs"], a["d"], dtype)
    return L.attn_decode_paged_fwd(FAKE[0], FAKE[1], FAKE[2], table, None, FAKE[3], None, a["B"],
                                   a["Hq"], a["Hkv"], Nq, a["maxb"], a["bs"], a["nblk"], a["d"], 0,
                                   0.088, dtype, ws, wsb, None)


def test_paged_decode_workspace_size_matches_contiguous_capacity():
    # a paged cache of max_blocks * block_size positions splits like a
    # contiguous cache of that capacity
    assert pws() == ws_size(Nkv=64 * 16) > 0
    assert pws(maxb=10, bs=256, Nq=3) == ws_size(Nkv=2560, Nq=3)
    assert pws(bs=24) == 0 and pws(bs=8) == 0 and pws(bs=8192) == 0 and pws(maxb=-1) == 0


def test_paged_decode_argument_errors():
    assert pdf(bs=48) == 4 and pdf(bs=8) == 4 and pdf(dtype=E.ATTN_F32) == 4 and pdf(Nq=65) == 4
    assert pdf(table=None) == 1
    assert pdf(maxb=-1) == 2 and pdf(nblk=-5) == 2
    assert pdf(ws=None) == 5 and pdf(wsb=8) == 5
    assert pdf(Hq=12, Hkv=8) == 3
    assert pdf(table=FAKE[3]) == 8   # block table overlaps the output
    assert pdf(B=0) == 0
    assert pdf() == 7 and pdf(bs=4096, maxb=3) == 7 and pdf(nblk=0) == 7


def f8(scale_k=0.02, scale_v=0.03, dtype=E.ATTN_BF16, Nq=1, ws=P(0x7000000000), wsb=None, **kw):
    a = dict(B=2, Hq=8, Hkv=1, Nkv=1000, d=128)
    a.update(kw)
    if wsb is None:
        wsb = ws_size(a["B"], a["Hq"], a["Hkv"], Nq, a["Nkv"], a["d"], E.ATTN_BF16)
    return L.attn_decode_fp8_fwd(FAKE[0], FAKE[1], FAKE[2], scale_k, scale_v, None, FAKE[3], None,
                                 a["B"], a["Hq"], a["Hkv"], Nq, a["Nkv"], a["d"], 0, 0.088, dtype,
                                 ws, wsb, None)


def test_fp8_decode_argument_errors():
    assert f8(dtype=E.ATTN_F16) == 4 and f8(dtype=E.ATTN_F32) == 4 and f8(d=96) == 4
    assert f8(scale_k=0.0) == 9 and f8(scale_v=-1.0) == 9 and f8(scale_k=float("inf")) == 9
    assert f8(ws=None) == 5
    assert f8(Hq=12, Hkv=8) == 3
    assert f8(B=0) == 0
    assert f8() == 7 and f8(Nq=5) == 7


def bw(dtype=E.ATTN_BF16, ws=P(0x7000000000), wsb=1 << 20, causal=0, **kw):
    a = dict(B=1, Hq=2, Hkv=1, Nq=8, Nkv=8, d=64)
    a.update(kw)
    return L.attn_backward(FAKE[0], FAKE[1], FAKE[2], P(0x3000000), P(0x3100000), P(0x3200000),
                           P(0x5000000), P(0x5100000), P(0x5200000), a["B"], a["Hq"], a["Hkv"],
                           a["Nq"], a["Nkv"], a["d"], causal, 0.125, dtype, ws, wsb, None)


def test_backward_argument_errors():
    assert L.attn_backward_workspace_size(2, 8, 2, 100, 50, 128, E.ATTN_BF16) == 2 * 2 * 8 * 100 * 4
    assert bw(dtype=E.ATTN_F32) == 4 and bw(d=96) == 4
    assert bw(Hq=3, Hkv=2) == 3 and bw(causal=3) == 9
    assert bw(ws=None) == 5 and bw(wsb=4) == 5
    assert bw(B=0) == 0
    assert bw() == 7 and bw(Nkv=0) == 7


def test_tuning_knobs_set_get_and_reject_invalid_values():
    for name, knob in E.TUNING_KNOBS.items():
        assert L.attn_get_tuning(knob) == 0, name      # automatic unless ATTN_TUNING says otherwise
    assert L.attn_get_tuning(99) == -1 and L.attn_set_tuning(99, 1) == 9
    bad = {"prefill_variant": [6, -1], "prefill_slots": [-2], "decode_chunk": [-5, 1 << 25],
           "decode_groups": [3, 8], "decode_rows_mode": [3, -1]}
    for name, values in bad.items():
        for v in values:
            assert L.attn_set_tuning(E.TUNING_KNOBS[name], v) == 9, (name, v)
            assert E.get_tuning(name) == 0
    with E.tuning(decode_chunk=700, decode_groups=2):
        assert E.get_tuning("decode_chunk") == 700 and E.get_tuning("decode_groups") == 2
    assert E.get_tuning("decode_chunk") == 0 and E.get_tuning("decode_groups") == 0


def test_tuning_defaults_come_from_the_environment_once():
    import subprocess
    import sys
    code = ("import exact_attention_31_amd as E; "
            "print(*[E.get_tuning(n) for n in ('prefill_variant', 'decode_chunk', 'decode_groups', "
            "'decode_rows_mode', 'prefill_slots')])")
    env = dict(os.environ, ATTN_TUNING="prefill_variant=4,decode_chunk=2048,decode_groups=3,bogus=1,"
                                       "decode_rows_mode=2x,prefill_slots=")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout.split()
    # decode_groups=3 is out of range, "2x" and "" do not parse: those stay automatic
    assert out == ["4", "2048", "0", "0", "0"]


def test_decode_workspace_follows_the_chunk_knob():
    base = L.attn_decode_workspace_size(2, 8, 2, 1, 16384, 128, E.ATTN_BF16)
    with E.tuning(decode_chunk=128):
        fine = L.attn_decode_workspace_size(2, 8, 2, 1, 16384, 128, E.ATTN_BF16)
    assert fine == 2 * 8 * 1 * (16384 // 128) * 130 * 4 and fine > base


def test_decode_plan_splits_finer_for_one_token():
    """The plan's finest split: about N_kv / 64 keys for one new token per
    request, N_kv / 16 for more (partials N_q times larger), within
    [128, 2048] keys."""
    per = lambda nq: 2 * 8 * nq * 130 * 4
    assert L.attn_decode_workspace_size(2, 8, 2, 1, 32768, 128, E.ATTN_BF16) == per(1) * 64
    assert L.attn_decode_workspace_size(2, 8, 2, 4, 32768, 128, E.ATTN_BF16) == per(4) * 16
    assert L.attn_decode_workspace_size(2, 8, 2, 1, 4096, 128, E.ATTN_BF16) == per(1) * 32
    assert L.attn_decode_workspace_size(2, 8, 2, 1, 262144, 128, E.ATTN_BF16) == per(1) * 128


def dfn(Nq=1, dtype=E.ATTN_BF16, lens=None, **kw):
    a = dict(B=2, Hq=8, Hkv=1, Nkv=1000, d=128)
    a.update(kw)
    return L.attn_decode_fwd_noalloc(FAKE[0], FAKE[1], FAKE[2], lens, FAKE[3], None, a["B"], a["Hq"],
                                     a["Hkv"], Nq, a["Nkv"], a["d"], 0, 0.088, dtype, None)


def test_noalloc_decode_argument_errors_and_scratch_limit():
    assert dfn(Nq=65) == 4 and dfn(dtype=E.ATTN_F32) == 4 and dfn(d=32) == 4
    assert dfn(Nq=0) == 0
    assert dfn(Hq=12, Hkv=8) == 3
    assert dfn() == 7                 # valid: reaches the (absent) device
    # one split of B*H_q*N_q rows of (d + 2) floats must fit the scratch
    rows_max = E.DECODE_SCRATCH_BYTES // ((128 + 2) * 4)
    assert dfn(B=64, Hq=(rows_max // 64) // 4 * 4, Hkv=4, Nkv=128) == 7
    assert dfn(B=64, Hq=(rows_max // 64 + 4) // 4 * 4, Hkv=4, Nkv=128) == 5
    # a finer split that would not fit is coarsened instead of rejected
    assert L.attn_decode_workspace_size(64, 64, 8, 2, 2048, 128, E.ATTN_BF16) > E.DECODE_SCRATCH_BYTES
    assert dfn(B=64, Hq=64, Hkv=8, Nq=2, Nkv=2048) == 7
