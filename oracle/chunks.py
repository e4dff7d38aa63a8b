"""Chunked-context plan — oracle (test infrastructure), integer arithmetic only.

This is the library's own chunk planner, not the page's. The vLLM mla_attention.py module
docstring ("The chunked prefill approach") only motivates it: the context rows a prefill gathers
are bounded by a workspace of W rows, so they are gathered in chunks. The planner the page prints
produces different plans (it has its own rules for empty contexts and for how much a split
request takes) and is neither followed nor reproduced here.

The library's rule:
- Requests with no context rows belong to no chunk.
- Walk the requests in order with a cursor (request r, first row s of what remains of it). A chunk
  takes whole remainders while they fit in W. When the next remainder does not fit, the chunk takes
  the longest prefix of it that fits and whose length is a multiple of the alignment A (a prefix of
  zero rows is not a span), then closes; the cursor moves past that prefix. A chunk is also closed
  when it is full. (The gather starts a split request's next span on an alignment boundary.)
- W must be at least A (else no row could ever be placed).

The result is a list of chunks, each a list of spans (request, first row, rows).

Pinned (tests/test_oracle_chunks.py) by hand-worked plans and by invariants: every context row is
covered once, in order; chunks hold at most W rows, a contiguous run of requests and no empty span;
split points are multiples of A; and a chunk closes only when its next aligned piece does not fit.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

Span = Tuple[int, int, int]


def plan_context_chunks(context_lens: Sequence[int], W: int, A: int) -> List[List[Span]]:
    if W < A or A < 1:
        raise ValueError("workspace rows must be at least the alignment")
    lens = [max(int(x), 0) for x in context_lens]
    chunks: List[List[Span]] = []
    cur: List[Span] = []
    rows = 0
    r, s = 0, 0
    while r < len(lens):
        remaining = lens[r] - s
        if remaining <= 0:
            r, s = r + 1, 0
            continue
        if rows + remaining <= W:
            cur.append((r, s, remaining))
            rows += remaining
            r, s = r + 1, 0
            if rows == W:
                chunks.append(cur)
                cur, rows = [], 0
            continue
        take = (W - rows) // A * A
        if take > 0:
            cur.append((r, s, take))
            s += take
        chunks.append(cur)  # non-empty: an empty chunk always has W >= A rows free
        cur, rows = [], 0
    if cur:
        chunks.append(cur)
    return chunks
