"""Exact scaled-dot-product attention for MI355X (gfx950): Python binding.

Argument marshalling only: every computation runs in the HIP kernels of the
C-ABI library libattn.so (declared in include/attn.h). PyTorch provides device
memory and the current stream. If the library is missing, importing works but
every call raises; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_GQA",
    4: "ATTN_ERR_UNSUPPORTED", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_LAUNCH",
    7: "ATTN_ERR_NO_DEVICE", 8: "ATTN_ERR_ALIAS", 9: "ATTN_ERR_VALUE",
}


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({attn_status_string(status)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libattn.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m exact_attention_31_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.attn_prefill_fwd.restype = i
    lib.attn_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.attn_decode_workspace_size.restype = sz
    lib.attn_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_decode_fwd.restype = i
    lib.attn_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.attn_decode_fwd_noalloc.restype = i
    lib.attn_decode_paged_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.attn_decode_paged_workspace_size.restype = sz
    lib.attn_decode_paged_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i,
                                          vp, sz, vp]
    lib.attn_decode_paged_fwd.restype = i
    lib.attn_decode_fp8_fwd.argtypes = [vp, vp, vp, f, f, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz,
                                        vp]
    lib.attn_decode_fp8_fwd.restype = i
    lib.attn_decode_paged_fp8_fwd.argtypes = [vp, vp, vp, f, f, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                              i, f, i, vp, sz, vp]
    lib.attn_decode_paged_fp8_fwd.restype = i
    lib.attn_backward_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.attn_backward_workspace_size.restype = sz
    lib.attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz,
                                  vp]
    lib.attn_backward.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i
    lib.attn_set_tuning.argtypes = [i, i]
    lib.attn_set_tuning.restype = i
    lib.attn_get_tuning.argtypes = [i]
    lib.attn_get_tuning.restype = i
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return load().attn_version()


TUNING_KNOBS = {"prefill_variant": 0, "prefill_slots": 1, "decode_chunk": 2, "decode_groups": 3,
                "decode_rows_mode": 4}


def set_tuning(name: str, value: int) -> int:
    """Set a process-wide tuning knob of the library (0 = automatic); returns the old value."""
    lib = load()
    knob = TUNING_KNOBS[name]
    old = lib.attn_get_tuning(knob)
    st = lib.attn_set_tuning(knob, int(value))
    if st != 0:
        raise AttnError(st, f"attn_set_tuning({name}={value})")
    return old


def get_tuning(name: str) -> int:
    return load().attn_get_tuning(TUNING_KNOBS[name])


class tuning:
    """Context manager that sets tuning knobs and restores them on exit:
    `with tuning(decode_chunk=2048): ...`."""

    def __init__(self, **knobs):
        self.knobs = knobs
        self.saved = {}

    def __enter__(self):
        for name, value in self.knobs.items():
            self.saved[name] = set_tuning(name, value)
        return self

    def __exit__(self, *exc):
        for name, value in self.saved.items():
            set_tuning(name, value)
        return False


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_tensor(name, t, dtype, device, ndim=4):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D tensor")


def _check_lse(lse, B, H_q, N_q, device):
    """lse: float32 [B, H_q, N_q] (the library writes B*H_q*N_q floats through it)."""
    _check_tensor("lse", lse, torch.float32, device, ndim=3)
    if tuple(lse.shape) != (B, H_q, N_q):
        raise ValueError(f"lse is {tuple(lse.shape)}, must be [B, H_q, N_q] = {(B, H_q, N_q)}")


def attn_prefill_fwd(q, k, v, o=None, lse=None, *, causal: bool = False, scale: float | None = None,
                     return_lse: bool = False, stream=None):
    """O = softmax(scale * Q K^T) V on the GPU (q [B,H_q,N_q,d], k/v [B,H_kv,N_kv,d]).

    Allocates o (and lse when return_lse) with torch if not given. Returns o, or (o, lse).
    """
    lib = load()
    if q.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k", k, q.dtype, dev)
    _check_tensor("v", v, q.dtype, dev)
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k.shape
    if tuple(k.shape) != (B, H_kv, N_kv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, q.dtype, dev)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_lse(lse, B, H_q, N_q, dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H_q, H_kv, N_q,
                                  N_kv, d, int(bool(causal)), float(scale), DTYPE_CODE[q.dtype],
                                  _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_prefill_fwd")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_decode_workspace_size(B, H_q, H_kv, N_q, N_kv, d, dtype) -> int:
    code = DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load().attn_decode_workspace_size(B, H_q, H_kv, N_q, N_kv, d, code))


def attn_decode_fwd(q, k_cache, v_cache, o=None, *, kv_lens=None, lse=None, causal: bool = False,
                    scale: float | None = None, workspace=None, return_lse: bool = False,
                    stream=None):
    """Split-KV GQA decode: q [B,H_q,N_q,d] (1 <= N_q <= 64 new tokens per request) against
    caches [B,H_kv,N_kv,d] whose first kv_lens[b] (int32 [B]) positions are valid."""
    lib = load()
    if q.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k_cache", k_cache, q.dtype, dev)
    _check_tensor("v_cache", v_cache, q.dtype, dev)
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, H_kv, N_kv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if kv_lens is not None:
        _check_tensor("kv_lens", kv_lens, torch.int32, dev, ndim=1)
        if kv_lens.shape[0] != B:
            raise ValueError("kv_lens must have B entries")
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, q.dtype, dev)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_lse(lse, B, H_q, N_q, dev)
    need = attn_decode_workspace_size(B, H_q, H_kv, N_q, N_kv, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_decode_fwd(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens), _ptr(o),
                                 _ptr(lse), B, H_q, H_kv, N_q, N_kv, d, int(bool(causal)),
                                 float(scale), DTYPE_CODE[q.dtype], _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fwd")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_decode_fwd_noalloc(q, k_cache, v_cache, o, *, kv_lens=None, lse=None, causal: bool = False,
                            scale: float | None = None, stream=None):
    """attn_decode_fwd with the split partials in the library's per-device scratch
    (ATTN_DECODE_SCRATCH_BYTES) instead of a workspace: the library allocates
    nothing, so o (and lse, if wanted) must be given. Calls that overlap on one
    device race on the shared scratch."""
    lib = load()
    if q.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k_cache", k_cache, q.dtype, dev)
    _check_tensor("v_cache", v_cache, q.dtype, dev)
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, H_kv, N_kv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if kv_lens is not None:
        _check_tensor("kv_lens", kv_lens, torch.int32, dev, ndim=1)
        if kv_lens.shape[0] != B:
            raise ValueError("kv_lens must have B entries")
    _check_tensor("o", o, q.dtype, dev)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is not None:
        _check_lse(lse, B, H_q, N_q, dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_decode_fwd_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens), _ptr(o),
                                         _ptr(lse), B, H_q, H_kv, N_q, N_kv, d, int(bool(causal)),
                                         float(scale), DTYPE_CODE[q.dtype], _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fwd_noalloc")
    return (o, lse) if lse is not None else o


def attn_decode_paged_workspace_size(B, H_q, H_kv, N_q, max_blocks, block_size, d, dtype) -> int:
    code = DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load().attn_decode_paged_workspace_size(B, H_q, H_kv, N_q, max_blocks, block_size, d,
                                                       code))


def attn_decode_paged_fwd(q, k_pool, v_pool, block_table, o=None, *, kv_lens=None, lse=None,
                          causal: bool = False, scale: float | None = None, workspace=None,
                          return_lse: bool = False, stream=None):
    """Decode over a paged KV cache: q [B,H_q,N_q,d]; pools [num_blocks,H_kv,block_size,d];
    block_table int32 [B,max_blocks] (pool block of each logical block); kv_lens int32 [B]."""
    lib = load()
    if q.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k_pool", k_pool, q.dtype, dev)
    _check_tensor("v_pool", v_pool, q.dtype, dev)
    _check_tensor("block_table", block_table, torch.int32, dev, ndim=2)
    B, H_q, N_q, d = q.shape
    num_blocks, H_kv, block_size, _ = k_pool.shape
    if tuple(k_pool.shape) != (num_blocks, H_kv, block_size, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pool shapes do not match q")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B rows")
    max_blocks = block_table.shape[1]
    if kv_lens is not None:
        _check_tensor("kv_lens", kv_lens, torch.int32, dev, ndim=1)
        if kv_lens.shape[0] != B:
            raise ValueError("kv_lens must have B entries")
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, q.dtype, dev)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_lse(lse, B, H_q, N_q, dev)
    need = attn_decode_paged_workspace_size(B, H_q, H_kv, N_q, max_blocks, block_size, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_decode_paged_fwd(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                       _ptr(kv_lens), _ptr(o), _ptr(lse), B, H_q, H_kv, N_q,
                                       max_blocks, block_size, num_blocks, d, int(bool(causal)),
                                       float(scale), DTYPE_CODE[q.dtype], _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_fwd")
    return (o, lse) if (return_lse or lse is not None) else o


_FP8 = getattr(torch, "float8_e4m3fn", None)


def _codes(name, t, dev, ndim=4):
    """FP8 E4M3 caches as uint8 codes (a float8_e4m3fn tensor is viewed as its bytes)."""
    if isinstance(t, torch.Tensor) and _FP8 is not None and t.dtype == _FP8:
        t = t.view(torch.uint8)
    _check_tensor(name, t, torch.uint8, dev, ndim=ndim)
    return t


def attn_decode_fp8_fwd(q, k_cache, v_cache, k_scale: float, v_scale: float, o=None, *,
                        kv_lens=None, lse=None, causal: bool = False, scale: float | None = None,
                        workspace=None, return_lse: bool = False, stream=None):
    """Decode over an FP8 E4M3 cache: q bf16 [B,H_q,N_q,d]; k/v_cache uint8 (or
    float8_e4m3fn) [B,H_kv,N_kv,d] holding codes; values = code * k_scale / v_scale."""
    lib = load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, dev)
    k_cache = _codes("k_cache", k_cache, dev)
    v_cache = _codes("v_cache", v_cache, dev)
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, H_kv, N_kv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if kv_lens is not None:
        _check_tensor("kv_lens", kv_lens, torch.int32, dev, ndim=1)
        if kv_lens.shape[0] != B:
            raise ValueError("kv_lens must have B entries")
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, q.dtype, dev)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_lse(lse, B, H_q, N_q, dev)
    need = attn_decode_workspace_size(B, H_q, H_kv, N_q, N_kv, d, ATTN_BF16)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_decode_fp8_fwd(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                     float(v_scale), _ptr(kv_lens), _ptr(o), _ptr(lse), B, H_q, H_kv,
                                     N_q, N_kv, d, int(bool(causal)), float(scale), ATTN_BF16,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fp8_fwd")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_decode_paged_fp8_fwd(q, k_pool, v_pool, k_scale: float, v_scale: float, block_table,
                              o=None, *, kv_lens=None, lse=None, causal: bool = False,
                              scale: float | None = None, workspace=None, return_lse: bool = False,
                              stream=None):
    """Paged decode over FP8 E4M3 pools [num_blocks,H_kv,block_size,d] (uint8 codes)."""
    lib = load()
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, dev)
    k_pool = _codes("k_pool", k_pool, dev)
    v_pool = _codes("v_pool", v_pool, dev)
    _check_tensor("block_table", block_table, torch.int32, dev, ndim=2)
    B, H_q, N_q, d = q.shape
    num_blocks, H_kv, block_size, _ = k_pool.shape
    if tuple(k_pool.shape) != (num_blocks, H_kv, block_size, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pool shapes do not match q")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B rows")
    max_blocks = block_table.shape[1]
    if kv_lens is not None:
        _check_tensor("kv_lens", kv_lens, torch.int32, dev, ndim=1)
        if kv_lens.shape[0] != B:
            raise ValueError("kv_lens must have B entries")
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, q.dtype, dev)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_lse(lse, B, H_q, N_q, dev)
    need = attn_decode_paged_workspace_size(B, H_q, H_kv, N_q, max_blocks, block_size, d, ATTN_BF16)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_decode_paged_fp8_fwd(_ptr(q), _ptr(k_pool), _ptr(v_pool), float(k_scale),
                                           float(v_scale), _ptr(block_table), _ptr(kv_lens), _ptr(o),
                                           _ptr(lse), B, H_q, H_kv, N_q, max_blocks, block_size,
                                           num_blocks, d, int(bool(causal)), float(scale), ATTN_BF16,
                                           _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_fp8_fwd")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_backward_workspace_size(B, H_q, H_kv, N_q, N_kv, d, dtype) -> int:
    code = DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load().attn_backward_workspace_size(B, H_q, H_kv, N_q, N_kv, d, code))


def attn_backward(q, k, v, o, d_o, lse, dq=None, dk=None, dv=None, *, causal: bool = False,
                  scale: float | None = None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attention given the forward's o and lse (float32
    [B,H_q,N_q], natural log) and the output gradient d_o."""
    lib = load()
    if q.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("d_o", d_o)):
        _check_tensor(name, t, q.dtype, dev)
    B, H_q, N_q, d = q.shape
    _check_lse(lse, B, H_q, N_q, dev)
    _, H_kv, N_kv, _ = k.shape
    if tuple(k.shape) != (B, H_kv, N_kv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v shapes do not match q")
    if tuple(o.shape) != tuple(q.shape) or tuple(d_o.shape) != tuple(q.shape):
        raise ValueError("o and d_o must have q's shape")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, q.dtype, dev)
    _check_tensor("dk", dk, q.dtype, dev)
    _check_tensor("dv", dv, q.dtype, dev)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shapes do not match their inputs")
    need = attn_backward_workspace_size(B, H_q, H_kv, N_q, N_kv, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(dev):
        st = lib.attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq),
                               _ptr(dk), _ptr(dv), B, H_q, H_kv, N_q, N_kv, d, int(bool(causal)),
                               float(scale), DTYPE_CODE[q.dtype], _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(dev, stream))
    if st != 0:
        raise AttnError(st, "attn_backward")
    return dq, dk, dv


DECODE_SCRATCH_BYTES = 64 << 20  # ATTN_DECODE_SCRATCH_BYTES in attn.h

__all__ = ["attn_prefill_fwd", "attn_decode_fwd", "attn_decode_fwd_noalloc", "attn_decode_workspace_size",
           "attn_decode_paged_fwd", "attn_decode_paged_workspace_size", "attn_decode_fp8_fwd",
           "attn_decode_paged_fp8_fwd", "attn_backward", "attn_backward_workspace_size", "attn_status_string",
           "attn_version", "set_tuning", "get_tuning", "tuning", "TUNING_KNOBS", "load", "AttnError", "LIB_PATH", "ATTN_F32", "ATTN_F16", "ATTN_BF16"]
