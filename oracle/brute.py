"""Pure-Python brute force for tiny MLA decode cases — oracle (test infrastructure).

Scalar loops with math.exp, no numpy arithmetic: the same definition as attention.py written out
element by element, so that the vectorised oracle can be checked against it on 1-4-row contexts.
See attention.py for the definition and the passages it follows.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence


def decode_token(q_heads: Sequence[Sequence[float]], rows: Sequence[Sequence[float]],
                 visible: Sequence[int], sm_scale: float, d_v: int,
                 sink: Optional[Sequence[float]] = None):
    """One query token: q_heads [H][d_qk], rows [L][d_qk], visible = list of row positions
    (repeats allowed). Returns (O [H][d_v], LSE [H])."""
    H = len(q_heads)
    outs: List[List[float]] = []
    lses: List[float] = []
    for h in range(H):
        scores = []
        for j in visible:
            acc = 0.0
            for d in range(len(q_heads[h])):
                acc += q_heads[h][d] * rows[j][d]
            scores.append(sm_scale * acc)
        terms = list(scores)
        if sink is not None:
            terms.append(sink[h])
        if not terms:
            outs.append([0.0] * d_v)
            lses.append(-math.inf)
            continue
        mx = max(terms)
        denom = sum(math.exp(x - mx) for x in terms)
        lse = mx + math.log(denom)
        o = [0.0] * d_v
        for s, j in zip(scores, visible):
            p = math.exp(s - lse)
            for d in range(d_v):
                o[d] += p * rows[j][d]
        outs.append(o)
        lses.append(lse)
    return outs, lses
