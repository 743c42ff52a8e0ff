"""Float64 model of the blockwise (online-softmax) evaluation, for tests only.

It restates the recurrence the GPU kernels use, so that the recurrence itself is
checked against the plain definition: per query row keep a running maximum m, a
denominator l and an un-normalised weighted sum u; when a block of keys arrives,
align to the new maximum m' and rescale l and u by exp(m - m'); the row's output
is u / l (auturnal.com transformer-attention guide, section 8; marketmaker.cc,
"Der Flash Attention-Algorithmus" and "Die Online-Softmax-Wiederholung", with
the FA2 change of dividing by l once at the end).

Options that mirror kernel choices:
* `lazy`: keep the old reference maximum unless the block's maximum exceeds it
  by more than `lazy` (natural-log units). The statistics stay exact: u and l
  share the same reference point, so only the representation changes.
* `lazy_sum`: the rule the prefill kernels apply: take the block's
  exponentials against the old reference first and keep them if they sum to
  at most `lazy_sum` (so each is at most that); otherwise, and while the
  reference is -inf, move it to the block's maximum if that is higher.
* split-KV: partial (m, l, u) over disjoint key ranges, merged with the same
  exp(m_s - m) weights (the recurrence applied across partitions).
"""
import numpy as np


def online_rows(q, k, v, scale, visible, block, lazy=0.0, lazy_sum=None):
    """q [R, d], k/v [n, d], visible [R, n] bool. Returns (o, m, l) in float64."""
    R = q.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    u = np.zeros((R, v.shape[1]))
    for j0 in range(0, k.shape[0], block):
        s = (q @ k[j0:j0 + block].T) * scale
        s = np.where(visible[:, j0:j0 + block], s, -np.inf)
        m_blk = s.max(axis=1)
        if lazy_sum is not None:
            with np.errstate(over="ignore", invalid="ignore"):
                first = np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None]).sum(axis=1)
            keep = np.isfinite(m) & (first <= lazy_sum)
            m_new = np.where(keep, m, np.maximum(m, m_blk))
        elif lazy:
            m_new = np.where(m_blk > m + lazy, m_blk, m)
        else:
            m_new = np.maximum(m, m_blk)
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        p = np.exp(s - m_ref[:, None])
        l = l * alpha + p.sum(axis=1)
        u = u * alpha[:, None] + p @ v[j0:j0 + block]
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(l[:, None] > 0, u / np.where(l > 0, l, 1)[:, None], 0.0)
    return o, m, l


def merge_partials(ms, ls, us):
    """Merge per-split (m_s, l_s, u_s): m = max m_s, w_s = exp(m_s - m) (0 for empty splits)."""
    ms = np.asarray(ms)
    m = ms.max(axis=0)
    m_ref = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - m_ref), 0.0)
    l = (w * np.asarray(ls)).sum(axis=0)
    u = (w[..., None] * np.asarray(us)).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(l[..., None] > 0, u / np.where(l > 0, l, 1)[..., None], 0.0)
        lse = np.where(l > 0, m_ref + np.log(np.where(l > 0, l, 1)), -np.inf)
    return o, lse
