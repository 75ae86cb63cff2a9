"""Local routing permutation: the single-GPU "dispatch" plan (CPU oracle; test only).

P2, review comments: routing is prepared once (``ep_prepare``) and cached for
dispatch and combine; the grouped receive needs each expert's slot padded to an
alignment (128 there, 256 in P1's tests).  P1, later commit messages: the
NVFP4 paths take ``top_k``, ``alignment`` and the top-k index dtype.
"""

import numpy as np


def capacity(tokens, top_k, num_experts, alignment):
    """Upper bound on grouped rows: every slot used plus worst-case padding per expert."""
    return tokens * top_k + num_experts * (alignment - 1)


def route_plan(topk_idx, num_experts, alignment, r_cap=None):
    """R12: stable counting sort of (token, slot) entries by expert.

    * ``topk_idx`` [T, k]: entry -1 means "slot unused" and is skipped; any
      other value outside [0, E) is an error (reported, entry dropped).
    * count_e = number of entries naming expert e; P_e = roundup(count_e, A);
      off_0 = 0, off_{e+1} = off_e + P_e.
    * Grouped rows of expert e are [off_e, off_e + count_e) in ascending flat
      index t*k + j (token order, then slot); rows [off_e + count_e,
      off_e + P_e) are padding.
    * dst_row[t, j] = grouped row of entry (t, j), or -1 if skipped/dropped.
    * src_row[g] = token of grouped row g, or -1 for padding and for every
      row from off_E up to r_cap.

    Returns dict(counts int32 [E], offsets int32 [E+1], dst_row int32 [T, k],
    src_row int32 [r_cap], error bool).
    """
    topk_idx = np.asarray(topk_idx)
    t, k = topk_idx.shape
    if r_cap is None:
        r_cap = capacity(t, k, num_experts, alignment)
    flat = topk_idx.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < num_experts)
    error = bool(np.any(~valid & (flat != -1)))
    counts = np.bincount(flat[valid], minlength=num_experts).astype(np.int64)
    padded = (counts + alignment - 1) // alignment * alignment
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    key = np.where(valid, flat, num_experts)
    order = np.argsort(key, kind="stable")                 # entries grouped by expert, stable
    dst = np.full(t * k, -1, dtype=np.int64)
    src = np.full(r_cap, -1, dtype=np.int64)
    pos = 0
    for e in range(num_experts):
        ent = order[pos : pos + counts[e]]
        pos += counts[e]
        rows = offsets[e] + np.arange(counts[e])
        dst[ent] = rows
        src[rows] = ent // k
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                dst_row=dst.reshape(t, k).astype(np.int32), src_row=src.astype(np.int32),
                error=error)

