"""Split-KV work plan for MLA decode — oracle (test infrastructure), integer arithmetic only.

The pages say that a metadata step computes "tile scheduling metadata and split information" before
the decode (FlashMLA wrapper, get_mla_metadata) and that HALOps keeps a per-forward plan with a work
list (mla_attention_plan) shared by the layers of one kind, but neither page defines the algorithm.
The algorithm below is this library's own; the GPU plan must reproduce it bit for bit.

Definitions
- Query group: dense mode, one request b with R = Sq * H stacked query rows (row r = t * H + h);
  sparse mode (topk > 0), one (request, token) pair g = b * Sq + t with R = H rows.
- Effective rows n_g and first row j0_g (rows every query of the group may see):
    L <= 0                -> n = 0
    sparse                -> n = topk, or clamp(topk_lens[g], 0, topk) when lengths are given
    dense, window W > 0   -> n = min(L, W + Sq - 1), j0 = L - n   (union of the Sq windows)
    dense                 -> n = L, j0 = 0
- Blocks of 64 rows: nblk_g = ceil(n_g / 64).
- Kernel tile: M_TILE query rows per workgroup and FIXED (per-split overhead in block units) come
  from R: R <= 16 -> (16, 3); R <= 32 -> (32, 2); R <= 64 -> (64, 4); otherwise (128, 4).
  m_tiles = ceil(R / M_TILE).
- Work units: U = max(1, num_cus // m_tiles), num_cus being the compute units planned for.
- Cost: cost_g = nblk_g + FIXED if nblk_g > 0 else 0; P_g = exclusive prefix sum of cost;
  total = sum of cost; quota = max(1, ceil(total / U)).
- Block k of group g sits at position P_g + FIXED + k and belongs to unit
  min(U - 1, position // quota). A split is a maximal run of consecutive blocks of one group in one
  unit; splits are numbered in (group, block) order, so both their groups and units ascend.

Plan words (int32), in this order:
  header[16]   magic 0x4D4C4131, G, U, S, R, m_tiles, M_TILE, quota, FIXED, total, S_max, 0...
  grp_ptr[G+1] splits of group g are [grp_ptr[g], grp_ptr[g+1])
  unit_ptr[U+1] splits of unit u are [unit_ptr[u], unit_ptr[u+1])
  grp_rows[2G] (j0_g, n_g)
  splits[4 S]  (g, first block, end block, unit); S_max = G + U entries are reserved

Pinned by invariants (every block of every group covered once and in order, pointer monotonicity,
per-unit cost bound) and hand-worked plans in tests/golden/plan_cases.json.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

MAGIC = 0x4D4C4131
HEADER_WORDS = 16
BLOCK = 64


def tile_params(R: int):
    """(M_TILE, FIXED) for R stacked query rows per group."""
    if R <= 16:
        return 16, 3
    if R <= 32:
        return 32, 2
    if R <= 64:
        return 64, 4
    return 128, 4


def group_rows(seqlens: Sequence[int], q_len: int, topk: int, window: int,
               topk_lens: Optional[Sequence[int]] = None):
    """Per-group (j0, n) and the group count."""
    B = len(seqlens)
    out = []
    if topk > 0:
        for b in range(B):
            for t in range(q_len):
                g = b * q_len + t
                L = int(seqlens[b])
                if L <= 0:
                    n = 0
                elif topk_lens is not None:
                    n = min(max(int(topk_lens[g]), 0), topk)
                else:
                    n = topk
                out.append((0, n))
    else:
        for b in range(B):
            L = int(seqlens[b])
            if L <= 0:
                out.append((0, 0))
            elif window > 0:
                n = min(L, window + q_len - 1)
                out.append((L - n, n))
            else:
                out.append((0, L))
    return out


def build_plan(seqlens: Sequence[int], q_len: int, num_heads: int, num_cus: int, topk: int = 0,
               window: int = 0, topk_lens: Optional[Sequence[int]] = None) -> np.ndarray:
    """The plan's int32 words (header through the S used split records)."""
    rows = group_rows(seqlens, q_len, topk, window, topk_lens)
    G = len(rows)
    R = num_heads if topk > 0 else q_len * num_heads
    M_TILE, FIXED = tile_params(R)
    m_tiles = -(-R // M_TILE)
    U = max(1, int(num_cus) // m_tiles)
    nblk = [-(-n // BLOCK) for (_, n) in rows]
    cost = [(nb + FIXED) if nb > 0 else 0 for nb in nblk]
    total = sum(cost)
    quota = max(1, -(-total // U))

    splits = []            # (g, k_begin, k_end, unit)
    grp_ptr = [0]
    P = 0
    for g in range(G):
        if nblk[g] > 0:
            cur_unit = None
            for k in range(nblk[g]):
                u = min(U - 1, (P + FIXED + k) // quota)
                if u != cur_unit:
                    splits.append([g, k, k + 1, u])
                    cur_unit = u
                else:
                    splits[-1][2] = k + 1
        P += cost[g]
        grp_ptr.append(len(splits))
    S = len(splits)
    unit_ptr = [sum(1 for s in splits if s[3] < u) for u in range(U + 1)]

    header = [MAGIC, G, U, S, R, m_tiles, M_TILE, quota, FIXED, total, G + U, 0, 0, 0, 0, 0]
    words = list(header) + grp_ptr + unit_ptr
    for (j0, n) in rows:
        words += [j0, n]
    for s in splits:
        words += s
    return np.asarray(words, dtype=np.int64).astype(np.int32)


def unpack(words: np.ndarray) -> dict:
    """Named views of a plan's words."""
    w = np.asarray(words, dtype=np.int64)
    assert int(w[0]) == MAGIC, "not a plan"
    G, U, S = int(w[1]), int(w[2]), int(w[3])
    o = HEADER_WORDS
    grp_ptr = w[o:o + G + 1]
    o += G + 1
    unit_ptr = w[o:o + U + 1]
    o += U + 1
    grp_rows = w[o:o + 2 * G].reshape(G, 2)
    o += 2 * G
    splits = w[o:o + 4 * S].reshape(S, 4)
    return dict(G=G, U=U, S=S, R=int(w[4]), m_tiles=int(w[5]), M_TILE=int(w[6]),
                quota=int(w[7]), FIXED=int(w[8]), total=int(w[9]), S_max=int(w[10]),
                grp_ptr=grp_ptr, unit_ptr=unit_ptr, grp_rows=grp_rows, splits=splits,
                n_words=o + 4 * S)
