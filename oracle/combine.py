"""Log-sum-exp merge of partial attention results: TEST INFRASTRUCTURE ONLY.

Reading adopted (the pages never spell out split-KV; this is the plain identity
it rests on): if key set K is the disjoint union of K_1..K_S and, for one query
row, o_s / lse_s are the softmax-weighted value average and the natural-log
sum of exp(score) over K_s, then over K

    lse = log(sum_s exp(lse_s))
    out = sum_s exp(lse_s - lse) * o_s

A part with lse_s = -inf (no keys) has weight 0; if every part is empty the
result is out = 0, lse = -inf (the oracle's convention for a row with no keys).
float64 throughout.
"""
from __future__ import annotations

import numpy as np


def combine(o_parts, lse_parts):
    """o_parts: [S, rows, d_v], lse_parts: [S, rows] -> (out [rows, d_v], lse [rows])."""
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    assert o.ndim == 3 and l.shape == o.shape[:2]
    m = np.max(l, axis=0)                                   # [rows]
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(l - m_safe[None, :])                         # exp(-inf) = 0
    tot = np.sum(w, axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.einsum("sr,srd->rd", w, o) / tot[:, None]
        lse = m_safe + np.log(tot)
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse
