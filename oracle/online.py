"""fp64 replicas of the single-pass online softmax and of the partition merge.

TEST INFRASTRUCTURE (see the package docstring).  These follow the steps of
"LLM 推理优化技术全景" (docs.ifdog.com), section "Flash Attention 深度剖析 >
在线 Softmax", in the page's notation: a running row maximum m, a running
exponential sum l and an output O, updated once per key/value block S_ij.
They exist to show, in exact-ish fp64, that the one-pass recurrence and the
split-then-merge schedule reproduce the three-pass result; the GPU kernels
implement the same algebra in fp32.
"""
import numpy as np


def online_softmax_rows(scores, values, block, normalise_each_block=True):
    """One pass over key blocks of width `block` for a single query row.

    scores: [N] fp64 (already scaled); values: [N, D] fp64.
    normalise_each_block=True keeps O normalised after every block, as the
    page's update O_new = O_old * l_old e^(m_old - m_new) / l_new
    + sum_j e^(S_j - m_new) V_j / l_new writes it.  False keeps an
    unnormalised accumulator and divides by l once at the end (the deferred
    rescale of the page's "Flash Attention v2 的改进").  Returns (O, m, l).
    With N = 0 returns zeros, -inf, 0.
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n, d = values.shape
    m = -np.inf
    l = 0.0
    o = np.zeros(d, dtype=np.float64)
    for j0 in range(0, n, block):
        s_blk = scores[j0:j0 + block]
        v_blk = values[j0:j0 + block]
        m_new = max(m, float(np.max(s_blk)))
        corr = np.exp(m - m_new) if np.isfinite(m) else 0.0
        e = np.exp(s_blk - m_new)
        l_new = l * corr + float(np.sum(e))
        if normalise_each_block:
            o = o * (l * corr / l_new) + (e @ v_blk) / l_new
        else:
            o = o * corr + e @ v_blk
        m, l = m_new, l_new
    if not normalise_each_block and l > 0.0:
        o = o / l
    return o, m, l


def partition_summary(scores, values):
    """Unnormalised summary (m, l, acc) of one key range: m = max s,
    l = sum e^(s - m), acc = sum e^(s - m) V.  An empty range gives
    (-inf, 0, 0).  The single-range case of the recurrence above."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if scores.size == 0:
        return -np.inf, 0.0, np.zeros(values.shape[1], dtype=np.float64)
    m = float(np.max(scores))
    e = np.exp(scores - m)
    return m, float(np.sum(e)), e @ values


def lse_merge(summaries):
    """Merge (m_k, l_k, acc_k) of disjoint key ranges into the normalised row.

    The page's rescale by e^(m_old - m_new), applied to whole-range summaries
    instead of single blocks: M = max_k m_k, L = sum_k l_k e^(m_k - M),
    out = sum_k acc_k e^(m_k - M) / L.  Ranges with l_k = 0 contribute
    nothing; if every range is empty the result is zeros.
    """
    ms = [m for (m, l, _) in summaries if l > 0.0]
    d = summaries[0][2].shape[0]
    if not ms:
        return np.zeros(d, dtype=np.float64)
    big_m = max(ms)
    big_l = 0.0
    acc = np.zeros(d, dtype=np.float64)
    for m, l, a in summaries:
        if l == 0.0:
            continue
        w = np.exp(m - big_m)
        big_l += l * w
        acc = acc + a * w
    return acc / big_l
