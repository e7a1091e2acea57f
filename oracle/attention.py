"""Exact decode attention, partials and their LSE merge in float64 (oracle; test only).

Definitions followed:
  - Decode attention for one query token is exact softmax attention over the whole context,
    with no compression or sparsification ([InplaceKVCache] §4.3 (iv), §7.1):
        s_t = scale * q . k_t,   o = sum_t softmax(s)_t v_t.
  - A partial over a token subset returns its own normalised output and its normaliser
    ([InplaceKVCache] §4.2: the CPU returns only its partial output and normalisers), kept
    here as the natural-log sum of exponentials of the scaled scores, lse = ln sum_t e^{s_t}.
  - Partials over disjoint token ranges merge exactly by LSE rescaling
    ([InplaceKVCache] §5.1): o = sum_p e^{lse_p - lse} o_p with lse = ln sum_p e^{lse_p}.
  - Grouped-query attention: consecutive query heads share one KV head, head h reading KV
    head h // (Hq / Hkv) ([CrossPool] §2.2 on grouped KV heads; the page does not fix the
    order, the consecutive grouping is the common convention).

An empty token set has no softmax; it is represented as o = 0, lse = -inf, which has zero
weight in a merge.  The max subtraction below is only for range safety of exp in float64;
it does not change the value.
"""

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Attention of Hq query heads over n tokens.

    q [Hq, Dk], k [n, Hkv, Dk], v [n, Hkv, Dv] (float64) -> o [Hq, Dv], lse [Hq].
    """
    q = np.asarray(q, np.float64)
    hq = q.shape[0]
    n, hkv, _ = k.shape
    dv = v.shape[2]
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    o = np.zeros((hq, dv), np.float64)
    lse = np.full(hq, -np.inf, np.float64)
    if n == 0:
        return o, lse
    for kvh in range(hkv):
        heads = slice(kvh * group, (kvh + 1) * group)
        s = scale * (q[heads] @ k[:, kvh, :].T)          # [group, n] scaled scores
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)                                  # e^{s_t - m}
        l = w.sum(axis=1, keepdims=True)                   # sum of the above
        o[heads] = (w @ v[:, kvh, :]) / l
        lse[heads] = (m + np.log(l))[:, 0]
    return o, lse


def merge(os_, lses):
    """Exact LSE merge of partials.

    os_  : sequence of arrays [..., Dv];  lses : sequence of arrays [...] (same leading
    shape).  Returns (o [..., Dv], lse [...]).  Partials with lse = -inf carry no weight;
    if every partial is empty the result is o = 0, lse = -inf.
    """
    o_stack = np.stack([np.asarray(o, np.float64) for o in os_])      # [P, ..., Dv]
    l_stack = np.stack([np.asarray(l, np.float64) for l in lses])     # [P, ...]
    big = l_stack.max(axis=0)
    finite = np.isfinite(big)
    safe_big = np.where(finite, big, 0.0)
    w = np.where(np.isfinite(l_stack), np.exp(l_stack - safe_big), 0.0)   # e^{lse_p - M}
    tot = w.sum(axis=0)
    lse = np.where(finite, safe_big + np.log(np.where(finite, tot, 1.0)), -np.inf)
    frac = np.where(finite, w / np.where(finite, tot, 1.0), 0.0)      # e^{lse_p - lse}
    o = (frac[..., None] * o_stack).sum(axis=0)
    return o, lse
