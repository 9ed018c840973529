"""Grouping of token rows by adapter (integer; the GPU path must match bit for bit).

Test infrastructure only.

The LLM-stack book (7.14.2, "The data layout") sorts the batch by adapter so
that rows of one adapter are contiguous and describes the segments with
``seg_start`` / ``seg_adapter``; LoRazor (3.1.1) calls the grouped row list
I_a with m_a = |I_a| and has blocks gather inputs and scatter results through
that adapter-grouped row-index array.

Outputs (all int64 numpy arrays here; the library uses int32):
  perm        [T]   live rows grouped by adapter, rows in increasing order
                    within a group; then the non-live rows in increasing order
  seg_start   [S+1] start of each group in ``perm`` plus an end sentinel
  seg_adapter [S]   adapter id of each group
  n_active, S, m_max

order = 0: groups by ascending adapter id (canonical).
order = 1: groups in order of each adapter's first appearance in the batch
           (reproduces the book's printed example).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np


def build_segments(ids, active: Optional[np.ndarray] = None, order: int = 0) -> Dict[str, object]:
    ids = [int(i) for i in np.asarray(ids).tolist()]
    T = len(ids)
    act = [1] * T if active is None else [int(a) for a in np.asarray(active).tolist()]
    live = [ids[i] >= 0 and act[i] != 0 for i in range(T)]

    groups: Dict[int, List[int]] = {}
    first_seen: List[int] = []
    for i in range(T):                    # one pass in row order keeps rows stable
        if live[i]:
            if ids[i] not in groups:
                groups[ids[i]] = []
                first_seen.append(ids[i])
            groups[ids[i]].append(i)

    keys = sorted(groups) if order == 0 else first_seen
    perm: List[int] = []
    seg_start = [0]
    for a in keys:
        perm.extend(groups[a])
        seg_start.append(len(perm))
    n_active = len(perm)
    perm.extend(i for i in range(T) if not live[i])
    lens = [len(groups[a]) for a in keys]
    return {
        "perm": np.array(perm, dtype=np.int64),
        "seg_start": np.array(seg_start, dtype=np.int64),
        "seg_adapter": np.array(keys, dtype=np.int64),
        "n_active": n_active,
        "S": len(keys),
        "m_max": max(lens) if lens else 0,
    }


def row_tiles(seg_start, bm: int) -> List[Tuple[int, int, int]]:
    """Row tiles of height ``bm`` inside each segment: (segment, first position
    in perm, row count), segment by segment, tiles in order."""
    out = []
    ss = [int(s) for s in np.asarray(seg_start).tolist()]
    for s in range(len(ss) - 1):
        p = ss[s]
        while p < ss[s + 1]:
            n = min(bm, ss[s + 1] - p)
            out.append((s, p, n))
            p += n
    return out
