"""Float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the HIP library never
does, and it shares no code with it.

What it computes (the plain definition, written out):

* Attention is softmax(Q K^T / sqrt(d_k)) V: scores from Q and K, a row-wise
  softmax, then a weighted average of V (auturnal.com transformer-attention
  guide, section 2; marketmaker.cc "Flash Attention und die Frage nach der
  Sequenzlaenge", section "Warum Aufmerksamkeit gedaechtnisgebunden ist").
* It follows the standard (materialising) attention of the papanda925.com
  survey, "標準Attention計算の擬似コード": form the score matrix, set masked
  entries to -inf, apply softmax over the key axis, multiply by V. Heads are an
  independent batch axis; tensors are [batch, heads, seq, head_dim].
* The softmax subtracts the row maximum before exponentiating; the guide's
  section 8 notes that this changes only the representation, not the
  probabilities. Here it is the plain two-pass form (max, then exp and sum),
  never the blockwise online recurrence.
* Grouped-query attention: G = H_q / H_kv query heads share one KV head
  (code-journey.com attention co-design summary, "Group Size(G)"); query head
  h reads KV head h // G (contiguous groups).
* Causal masking hides keys "in the future" of a query (marketmaker.cc,
  section on causal masking). With N_q queries against n keys the last query
  is aligned with the last key: key j is visible to query i iff
  j <= i + (n - N_q). For N_q == n this is j <= i; for a single decode query it
  is every cached key.
* Decode reads a KV cache of capacity N_kv of which the first kv_lens[b]
  positions are valid (guide section 9; papanda925.com "KVキャッシュ管理の概念").
* A row with no visible key has output 0 and log-sum-exp -inf.
* lse = m + ln(l), the per-row statistics that the backward pass keeps
  (marketmaker.cc, "Rückwärtsdurchlauf").
* A paged (block-wise) KV cache stores fixed-size blocks in one shared pool
  and maps each request's logical blocks to pool blocks (papanda925.com survey,
  "Block-wise KV Cache" in its recent-trends and method sections). Attention
  over it is attention over the cache that the block table describes: gather
  the blocks into a contiguous cache, then apply the definition above.
* An FP8 KV cache (the pages' decode measurements assume one: code-journey.com
  attention co-design summary, arithmetic-intensity formulas) holds E4M3 codes
  and a per-tensor scale; attention over it is attention over the dequantised
  values code_value * scale. E4M3 here is the OCP 8-bit format: 1 sign bit,
  4 exponent bits (bias 7), 3 mantissa bits, subnormals at exponent 0, no
  infinities, and S.1111.111 the only NaN pattern.

All arithmetic is float64 on the exact (dtype-rounded) input values; numpy's
matmul (BLAS dgemm) forms the score rows and the weighted sum.
"""
from __future__ import annotations

import numpy as np

MiB = 2 ** 20


def score_bytes(n: int, bytes_per: int = 4) -> int:
    """Bytes to store one layer-head's n x n score matrix explicitly.

    The guide's section 4 gives n^2 x 4 bytes for float32 scores, and its
    section 6 tabulates 1, 4, 16, 64 MiB at n = 512, 1024, 2048, 4096.
    """
    return n * n * bytes_per


def kv_cache_bytes(layers: int, n: int, h_kv: int, d_h: int, bytes_per: int) -> int:
    """Approximate KV-cache size 2 * L * n * h_kv * d_h * b (keys and values of every
    past position in every layer; weights, workspace and fragmentation excluded),
    per the guide's section 9."""
    return 2 * layers * n * h_kv * d_h * bytes_per


def visible_pairs(N_q: int, n: int, causal: bool) -> int:
    """Number of (query, key) pairs that enter the softmax for one head.

    Counted by the definition above (bottom-right causal alignment). Each
    visible pair costs one exponential (code-journey.com, softmax op count,
    "Head Dimension(Hsz)"); causal skipping saves about half the work
    (marketmaker.cc, causal masking section).
    """
    if not causal:
        return N_q * n
    off = n - N_q
    total = 0
    for i in range(N_q):
        total += max(0, min(n, i + off + 1))
    return total


def softmax_stats(scores: np.ndarray):
    """The two-pass softmax of each score row (last axis), float64.

    Pass one takes the row maximum m over the finite entries; pass two forms
    p = exp(s - m) and their sum l. Subtracting m changes only the
    representation of the probabilities p / l, not their values (auturnal.com
    guide, section 8), and keeps exp from overflowing for large scores.
    Entries of -inf (masked keys) get p = 0. A row with no finite entry has
    m = 0 and l = 0. Returns (p, m, l).
    """
    s = np.asarray(scores, dtype=np.float64)
    m = s.max(axis=-1)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m[..., None])
    return p, m, p.sum(axis=-1)


def _head(q_rows: np.ndarray, rows: np.ndarray, N_q: int, k: np.ndarray, v: np.ndarray,
          causal: bool, scale: float, n: int, row_block: int = 512):
    """One head. q_rows [len(rows), d] are the queries at sequence positions `rows`
    (of N_q in all); k/v [>=n, d] with the first n rows valid. Returns (o, lse)."""
    rows = np.asarray(rows, dtype=np.int64)
    d_v = v.shape[1]
    o = np.zeros((len(rows), d_v), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    if n == 0 or len(rows) == 0:
        return o, lse
    kk = np.asarray(k[:n], dtype=np.float64)
    vv = np.asarray(v[:n], dtype=np.float64)
    off = n - N_q
    keys = np.arange(n)
    for s in range(0, len(rows), row_block):
        r = rows[s:s + row_block]
        qq = np.asarray(q_rows[s:s + row_block], dtype=np.float64)
        # 1. materialise the score rows
        scores = (qq @ kk.T) * float(scale)
        # 2. mask: keys after the aligned diagonal are -inf
        if causal:
            masked = keys[None, :] > (r[:, None] + off)
            scores = np.where(masked, -np.inf, scores)
        # 3. two-pass softmax over the key axis
        p, m, l = softmax_stats(scores)
        empty = l == 0.0                   # no visible key
        # 4. weighted sum of V, normalised
        with np.errstate(invalid="ignore", divide="ignore"):
            out = (p @ vv) / l[:, None]
            row_lse = m + np.log(l)
        out[empty] = 0.0
        row_lse[empty] = -np.inf
        o[s:s + row_block] = out
        lse[s:s + row_block] = row_lse
    return o, lse


def attention_ref(q, k, v, causal: bool, scale: float, kv_lens=None, row_block: int = 512):
    """Exact attention in float64.

    q: [B, H_q, N_q, d]; k, v: [B, H_kv, N_kv, d] (any float dtype; exact values).
    kv_lens: optional per-batch valid key counts (each in [0, N_kv]); default N_kv.
    Returns (o [B, H_q, N_q, d] float64, lse [B, H_q, N_q] float64, natural log).
    """
    B, H_q, N_q, d = q.shape
    Bk, H_kv, N_kv, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch")
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    o = np.zeros((B, H_q, N_q, v.shape[3]), dtype=np.float64)
    lse = np.zeros((B, H_q, N_q), dtype=np.float64)
    rows = np.arange(N_q)
    for b in range(B):
        n = N_kv if kv_lens is None else int(kv_lens[b])
        if not 0 <= n <= N_kv:
            raise ValueError("kv_lens out of range")
        for h in range(H_q):
            g = h // G
            o[b, h], lse[b, h] = _head(q[b, h], rows, N_q, k[b, g], v[b, g], causal, scale, n,
                                       row_block)
    return o, lse


def attention_head_rows(q_rows, rows, N_q: int, k_head, v_head, causal: bool, scale: float,
                        n: int | None = None):
    """Selected output rows of one head, for sampled checks of full-size runs.

    q_rows [len(rows), d] are the queries at positions `rows` of a sequence of N_q
    queries; k_head/v_head [N_kv, d] hold the head's keys/values, of which the
    first n (default all) are valid.
    """
    n = k_head.shape[0] if n is None else n
    return _head(q_rows, rows, N_q, k_head, v_head, causal, scale, n, 256)


def gather_paged(pool, block_table, lens, block_size: int):
    """The contiguous cache [B, H_kv, max_blocks * block_size, d] that a paged
    cache describes. pool: [num_blocks, H_kv, block_size, d]; block_table
    [B, max_blocks] maps logical block i of request b to a pool block; only
    the blocks holding positions below lens[b] are read (the rest stay 0)."""
    pool = np.asarray(pool)
    table = np.asarray(block_table)
    B, max_blocks = table.shape
    _, H_kv, bs, d = pool.shape
    if bs != block_size:
        raise ValueError("pool block size mismatch")
    out = np.zeros((B, H_kv, max_blocks * bs, d), dtype=pool.dtype)
    for b in range(B):
        n = int(lens[b])
        for i in range((n + bs - 1) // bs):
            out[b, :, i * bs:(i + 1) * bs] = pool[int(table[b, i])]
    return out


def attention_paged_ref(q, k_pool, v_pool, block_table, kv_lens, block_size: int, causal: bool,
                        scale: float):
    """Exact attention over a paged KV cache: attention_ref on the gathered cache."""
    k = gather_paged(k_pool, block_table, kv_lens, block_size)
    v = gather_paged(v_pool, block_table, kv_lens, block_size)
    return attention_ref(q, k, v, causal, scale, kv_lens=kv_lens)


def e4m3_value(code: int) -> float:
    """The value of one OCP FP8 E4M3 code, from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                      # subnormal: 0.man * 2^(1 - bias)
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequant_e4m3(codes, scale: float) -> np.ndarray:
    """float64 values code_value * scale of an array of E4M3 codes (uint8)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * float(scale)


def attention_fp8kv_ref(q, k_codes, v_codes, k_scale: float, v_scale: float, causal: bool,
                        scale: float, kv_lens=None):
    """Exact attention over an FP8 cache: attention_ref on the dequantised K and V."""
    return attention_ref(q, dequant_e4m3(k_codes, k_scale), dequant_e4m3(v_codes, v_scale), causal,
                         scale, kv_lens=kv_lens)


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Row softmax of a score matrix, float64: p / l from softmax_stats. -inf
    entries get weight 0; a row with no finite entry gets all zeros."""
    p, _, l = softmax_stats(scores)
    with np.errstate(invalid="ignore", divide="ignore"):
        w = p / l[..., None]
    return np.where(l[..., None] > 0.0, w, 0.0)


__all__ = ["score_bytes", "kv_cache_bytes", "visible_pairs", "attention_ref", "attention_head_rows",
           "gather_paged", "attention_paged_ref", "e4m3_value", "dequant_e4m3", "attention_fp8kv_ref",
           "softmax_stats", "softmax_weights", "MiB"]
