"""Pure-Python brute-force attention row: TEST INFRASTRUCTURE ONLY.

Shares nothing with `mla_oracle.c`: it takes a dense list of key rows (no pages,
no block table) and uses math.fsum for every sum, so its error is a few ulps.
It exists to pin the C oracle on tiny inputs.

For one query row q (length d_qk) and keys k_0..k_{n-1} (each length d_qk),
with values v_p = k_p[:d_v]:
    s_p   = scale * sum_d q[d] * k_p[d]
    lse   = log(sum_p exp(s_p))                (computed as m + log(sum exp(s_p - m)))
    out_d = sum_p exp(s_p - lse) * v_p[d]
With a sink logit sigma (attention-sink reading: one more term in the softmax, with a
zero value row) the score list gains sigma and the value sum does not.
"""
from __future__ import annotations

import math


def attend_row(q, keys, scale, d_v, sink=None):
    """Return (out list[d_v], lse float).  Empty `keys` and no sink -> zeros and -inf."""
    if not keys and sink is None:
        return [0.0] * d_v, -math.inf
    s = [scale * math.fsum(qd * kd for qd, kd in zip(q, k)) for k in keys]
    m = max(s + ([sink] if sink is not None else []))
    w = [math.exp(x - m) for x in s]
    tot = math.fsum(w + ([math.exp(sink - m)] if sink is not None else []))
    out = [math.fsum(wp * k[d] for wp, k in zip(w, keys)) / tot for d in range(d_v)]
    return out, m + math.log(tot)
