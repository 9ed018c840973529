"""Pins for the integer parts of the oracle: adapter grouping and the
launch-geometry closed forms."""
import numpy as np
import pytest

import oracle
from golden_io import load


def test_book_printed_segment_example():
    g = load("segments_book_example.txt")
    ids = g["ids"].astype(int)
    seg = oracle.build_segments(ids, order=1)
    assert list(seg["seg_start"][:-1]) == list(g["printed_seg_start"].astype(int))
    assert seg["seg_start"][-1] == len(ids)
    assert list(seg["seg_adapter"]) == list(g["printed_seg_adapter"].astype(int))
    canon = oracle.build_segments(ids, order=0)
    assert list(canon["perm"]) == [5, 0, 1, 2, 3, 4]
    assert list(canon["seg_start"]) == [0, 1, 4, 6]
    assert list(canon["seg_adapter"]) == [0, 3, 7]


def _check_grouping(ids, act, seg, order):
    T = len(ids)
    live = [(ids[i] >= 0) and (act is None or act[i] != 0) for i in range(T)]
    perm = list(seg["perm"])
    assert sorted(perm) == list(range(T))                       # a permutation
    n = seg["n_active"]
    assert n == sum(live)
    assert all(live[i] for i in perm[:n]) and not any(live[i] for i in perm[n:])
    assert perm[n:] == sorted(perm[n:])                         # inactive rows ascending
    ss, sa = list(seg["seg_start"]), list(seg["seg_adapter"])
    assert ss[0] == 0 and ss[-1] == n and len(sa) == len(ss) - 1
    assert len(set(sa)) == len(sa)
    for s in range(len(sa)):
        rows = perm[ss[s]:ss[s + 1]]
        assert len(rows) > 0
        assert all(ids[i] == sa[s] for i in rows)
        assert rows == sorted(rows)                              # stable
    if order == 0:
        assert sa == sorted(sa)
    else:
        first = {}
        for i in range(T):
            if live[i] and ids[i] not in first:
                first[ids[i]] = i
        assert sa == sorted(sa, key=lambda a: first[a])
    lens = np.diff(ss)
    assert seg["m_max"] == (int(lens.max()) if len(lens) else 0)
    assert seg["S"] == len(sa)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("order", [0, 1])
def test_grouping_properties_random(seed, order):
    g = np.random.default_rng(seed)
    T = int(g.integers(0, 300))
    ids = g.integers(-1, 20, T)
    act = (g.uniform(size=T) > 0.3).astype(np.uint8) if seed % 2 else None
    _check_grouping(list(ids), None if act is None else list(act), oracle.build_segments(ids, act, order), order)


def test_grouping_brute_force_definition():
    # canonical order is a stable sort of the live rows by id: compare with
    # Python's sort (stable) on (id, row) keys
    g = np.random.default_rng(11)
    ids = g.integers(-1, 7, 200)
    act = (g.uniform(size=200) > 0.25).astype(np.uint8)
    seg = oracle.build_segments(ids, act)
    live = [i for i in range(200) if ids[i] >= 0 and act[i]]
    want = sorted(live, key=lambda i: ids[i]) + [i for i in range(200) if i not in set(live)]
    assert list(seg["perm"]) == want


def test_empty_and_all_inactive():
    seg = oracle.build_segments(np.zeros(0, int))
    assert seg["n_active"] == 0 and seg["S"] == 0 and list(seg["seg_start"]) == [0]
    seg = oracle.build_segments(np.full(5, -1))
    assert seg["n_active"] == 0 and list(seg["perm"]) == [0, 1, 2, 3, 4]
    seg = oracle.build_segments(np.arange(5), np.zeros(5, np.uint8))
    assert seg["S"] == 0 and seg["m_max"] == 0


def test_row_tiles():
    t = oracle.row_tiles([0, 3, 40, 41], 16)
    assert t == [(0, 0, 3), (1, 3, 16), (1, 19, 16), (1, 35, 5), (2, 40, 1)]


def test_lorazor_printed_launch_examples():
    g = load("launch_lorazor_examples.txt")
    M, BM, rows = int(g["M"]), int(g["BM"]), int(g["rows"])
    assert oracle.tiles_exact([rows], BM) == int(g["tiles_needed"])
    assert oracle.tiles_full_batch(1, M, BM) == int(g["tiles_full_batch_per_slot"])
    assert oracle.row_bound_set(M) == list(g["row_bound_set"].astype(int))
    # Eq. 3's row dimension under the shared bound, worked from the same page
    # numbers (a mistake that uses M, or m_max, for R fails here)
    for k in ("a", "b"):
        R = oracle.row_bound(M, int(g[f"m_max_{k}"]))
        assert R == int(g[f"R_{k}"])
        per_slot = int(g[f"shared_bound_tiles_per_slot_{k}"])
        assert oracle.tiles_shared_bound(1, R, BM) == per_slot
        assert oracle.tiles_shared_bound(7, R, BM) == 7 * per_slot


def test_row_bound_rules():
    assert oracle.row_bound_set(16) == [16]
    assert oracle.row_bound_set(100) == [16, 32, 64, 100]
    assert oracle.row_bound(256, 1) == 16
    assert oracle.row_bound(256, 17) == 32
    assert oracle.row_bound(256, 200) == 256
    assert oracle.row_bound(100, 65) == 100
    # ordering of the counts: exact <= shared bound <= full batch
    g = np.random.default_rng(1)
    for _ in range(50):
        M = int(g.integers(1, 600))
        sizes = np.bincount(g.integers(0, 40, M))
        sizes = sizes[sizes > 0]
        L = len(sizes)
        R = oracle.row_bound(M, int(sizes.max()))
        for bm in (1, 4, 16, 64):
            e = oracle.tiles_exact(sizes, bm)
            s = oracle.tiles_shared_bound(L, R, bm)
            f = oracle.tiles_full_batch(L, M, bm)
            assert e <= s <= f


def test_class_separation_rule():
    assert oracle.class_separation_enabled([1] * 8 + [40])
    assert not oracle.class_separation_enabled([1] * 7 + [40])
    assert not oracle.class_separation_enabled([1] * 20)
    assert not oracle.class_separation_enabled([1] * 8 + [40] * 17)
    assert oracle.tiles_two_class(L=32, C=16, R=256, bm=16) == 32 * 1 + 16 * 16


def test_lora_mac_fraction():
    g = load("lora_mac_fraction.txt")
    r, di, do = int(g["r"]), int(g["d_in"]), int(g["d_out"])
    frac = 100.0 * r * (di + do) / (di * do)
    assert abs(frac - float(g["percent_about"])) < 0.05
