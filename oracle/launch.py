"""Closed-form launch geometry of the row-tile grids (integer).

Test infrastructure only.  From "LoRazor: Trimming Adapter Execution for
Efficient Multi-LoRA Serving", 3.1:

* 3.1.1: the baseline launches ceil(M / B_M) row tiles for each of L adapter
  slots, although an adapter with m_a rows needs only ceil(m_a / B_M).
* 3.1.2 (Eq. 3): a common row bound R with m_max <= R <= M replaces M, giving
  L * ceil(R / B_M) row tiles (times the column tiles, slices and split-K
  partitions, which do not depend on the rows).
* 3.1.3 (Eqs. 4-6): two classes, small m_a <= 16 with row bound 16 over the L
  slots, large m_a > 16 with row bound R over a compact list of C = 16 slots:
  L * ceil(16 / B_M) + C * ceil(R / B_M) row tiles; enabled only when the
  small class has at least 8 adapters and the large class 1..C.
* 3.1.4 (Eqs. 7-8): the supported bounds for padded batch M are
  {16 * 2^k < M} U {M}; R is the smallest of them >= m_max.

The exact item count used by this library's host-sized grids is
sum_a ceil(m_a / B_M): the row tiles that hold work and nothing else.
"""
from __future__ import annotations

from typing import Iterable, List


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def row_bound_set(M: int) -> List[int]:
    out = []
    r = 16
    while r < M:
        out.append(r)
        r *= 2
    out.append(M)
    return out


def row_bound(M: int, m_max: int) -> int:
    return min(r for r in row_bound_set(M) if r >= m_max)


def tiles_full_batch(L: int, M: int, bm: int) -> int:
    return L * _ceil(M, bm)


def tiles_shared_bound(L: int, R: int, bm: int) -> int:
    return L * _ceil(R, bm)


def tiles_two_class(L: int, C: int, R: int, bm: int) -> int:
    return L * _ceil(16, bm) + C * _ceil(R, bm)


def class_separation_enabled(group_sizes: Iterable[int], C: int = 16) -> bool:
    sizes = [int(m) for m in group_sizes if m > 0]
    n_small = sum(1 for m in sizes if m <= 16)
    n_large = sum(1 for m in sizes if m > 16)
    return n_small >= 8 and 1 <= n_large <= C


def tiles_exact(group_sizes: Iterable[int], bm: int) -> int:
    return sum(_ceil(int(m), bm) for m in group_sizes if m > 0)
