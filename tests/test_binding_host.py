"""Argument checks of the Python binding (CPU only).

The binding must reject malformed tensors before it calls into the library.
Here the library is replaced by an object that fails on any call, and the
device check is relaxed so that CPU tensors stand in for device tensors: every
case must raise ValueError without reaching the library."""
import pytest
import torch

import exact_attention_31_amd as E


class _NoCalls:
    def __getattr__(self, name):
        if name.startswith("attn_") and name.endswith("workspace_size"):
            return lambda *a: 1024
        raise AssertionError(f"library function {name} reached with invalid arguments")


@pytest.fixture
def no_lib(monkeypatch):
    def check(name, t, dtype, device, ndim=4):
        if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
            raise ValueError(name)
    monkeypatch.setattr(E, "load", lambda: _NoCalls())
    monkeypatch.setattr(E, "_check_tensor", check)


B, HQ, HKV, NQ, NKV, D = 2, 4, 2, 4, 64, 64


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


BAD_LSE = [(B, HQ, 1), (B, HQ, NQ + 1), (B, 1, NQ), (1, HQ, NQ)]


@pytest.mark.parametrize("shape", BAD_LSE)
def test_prefill_rejects_misshaped_lse(no_lib, shape):
    q, k = _t(B, HQ, NQ, D), _t(B, HKV, NKV, D)
    with pytest.raises(ValueError, match="lse"):
        E.attn_prefill_fwd(q, k, k.clone(), lse=_t(*shape, dtype=torch.float32))


@pytest.mark.parametrize("shape", BAD_LSE)
def test_decode_entry_points_reject_misshaped_lse(no_lib, shape):
    q = _t(B, HQ, NQ, D)
    k = _t(B, HKV, NKV, D)
    lens = torch.full((B,), NKV, dtype=torch.int32)
    lse = _t(*shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="lse"):
        E.attn_decode_fwd(q, k, k.clone(), kv_lens=lens, lse=lse)
    pool = _t(8, HKV, 16, D)
    table = torch.zeros((B, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="lse"):
        E.attn_decode_paged_fwd(q, pool, pool.clone(), table, kv_lens=lens, lse=lse)
    codes = _t(B, HKV, NKV, D, dtype=torch.uint8)
    with pytest.raises(ValueError, match="lse"):
        E.attn_decode_fp8_fwd(q, codes, codes.clone(), 1.0, 1.0, kv_lens=lens, lse=lse)
    pcodes = _t(8, HKV, 16, D, dtype=torch.uint8)
    with pytest.raises(ValueError, match="lse"):
        E.attn_decode_paged_fp8_fwd(q, pcodes, pcodes.clone(), 1.0, 1.0, table, kv_lens=lens, lse=lse)


@pytest.mark.parametrize("shape", BAD_LSE)
def test_backward_rejects_misshaped_lse(no_lib, shape):
    q, k = _t(B, HQ, NQ, D), _t(B, HKV, NKV, D)
    with pytest.raises(ValueError, match="lse"):
        E.attn_backward(q, k, k.clone(), q.clone(), q.clone(), _t(*shape, dtype=torch.float32))
