"""Host-side tests of the C-ABI library: it loads, exports every declared
entry point, its host segment planner matches the oracle bit for bit, and
argument validation rejects bad calls before anything is enqueued.

No test here launches a kernel: every call with made-up device pointers is
built to fail validation (asserted), so it is safe with or without a GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from golden_io import load

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

agm = pytest.importorskip("adapter_gemm_amd", reason="liblora.so not built")


def _declared():
    src = open(os.path.join(ROOT, "include", "lora.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 10
    lib = ctypes.CDLL(agm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(agm.EXPORTED) == names


def test_status_strings():
    for s in range(8):
        assert agm.lib().lora_status_string(s)
    assert agm.lib().lora_last_error() == b""


def test_segment_words():
    assert agm.segment_words(0) == 17
    assert agm.segment_words(256) == 16 + 8 * 256 + 1


def _split(plan, T):
    h = agm.SEG_HEADER
    perm = plan[h:h + T]
    pos_seg = plan[h + T:h + 2 * T]
    seg_start = plan[h + 2 * T:h + 3 * T + 1]
    seg_adapter = plan[h + 3 * T + 1:h + 4 * T + 1]
    ts = plan[h + 4 * T + 1:h + 6 * T + 1].reshape(-1, 2) if T else np.zeros((0, 2), np.int32)
    tl = plan[h + 6 * T + 1:h + 8 * T + 1].reshape(-1, 2) if T else np.zeros((0, 2), np.int32)
    return perm, pos_seg, seg_start, seg_adapter, ts, tl


def _compare(ids, act, n_slots, order):
    T = len(ids)
    plan, s = agm.plan_segments(ids, act, n_slots, order)
    ref = oracle.build_segments(ids, act, order)
    perm, pos_seg, seg_start, seg_adapter, ts, tl = _split(plan, T)
    S = ref["S"]
    assert s["n_active"] == ref["n_active"] and s["n_segments"] == S and s["m_max"] == ref["m_max"]
    assert s["T"] == T and s["error"] == 0
    assert np.array_equal(perm, ref["perm"])
    assert np.array_equal(seg_start[:S + 1], ref["seg_start"])
    assert np.array_equal(seg_adapter[:S], ref["seg_adapter"])
    # segment index of every grouped position
    want_pos = np.full(T, -1)
    for k in range(S):
        want_pos[ref["seg_start"][k]:ref["seg_start"][k + 1]] = k
    assert np.array_equal(pos_seg, want_pos)
    for tile, lst, n in ((agm.TILE_SMALL, ts, s["n_tiles_small"]), (agm.TILE_LARGE, tl, s["n_tiles_large"])):
        want = oracle.row_tiles(ref["seg_start"], tile)
        assert n == len(want)
        assert [(int(b), int(a)) for a, b in lst[:n]] == [(w[0], w[1]) for w in want]
    want_R = oracle.row_bound(T, ref["m_max"]) if ref["n_active"] else 0
    assert s["row_bound"] == want_R


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("order", [0, 1])
def test_host_planner_matches_oracle(seed, order):
    g = np.random.default_rng(100 + seed)
    T = int(g.integers(0, 700))
    N = int(g.integers(1, 300))
    ids = g.integers(-1, N, T).astype(np.int32)
    act = (g.uniform(size=T) > 0.3).astype(np.uint8) if seed % 2 else None
    _compare(ids, act, N, order)


def test_host_planner_workloads():
    from lora_inputs import make_workload, CONFIG_NAMES
    for name in CONFIG_NAMES:
        w = make_workload(name)
        _compare(w.ids, w.active, w.projections[0].n_slots, 0)


def test_host_planner_book_example():
    g = load("segments_book_example.txt")
    ids = g["ids"].astype(np.int32)
    plan, s = agm.plan_segments(ids, None, 8, 1)
    _, _, seg_start, seg_adapter, _, _ = _split(plan, len(ids))
    assert list(seg_start[:3]) == list(g["printed_seg_start"].astype(int))
    assert list(seg_adapter[:3]) == list(g["printed_seg_adapter"].astype(int))


def test_planner_errors():
    with pytest.raises(agm.LoraError) as e:
        agm.plan_segments(np.array([0, 5], np.int32), None, 5, 0)
    assert e.value.status == agm.LORA_E_ID
    with pytest.raises(agm.LoraError) as e:
        agm.plan_segments(np.array([0, -2], np.int32), None, 5, 0)
    assert e.value.status == agm.LORA_E_ID
    with pytest.raises(agm.LoraError) as e:
        agm.plan_segments(np.array([0], np.int32), None, 5, 2)
    assert e.value.status == agm.LORA_E_ARG


# ---- validation with made-up device addresses (never reach a launch) ---------

FAKE = 1 << 40           # 16-byte aligned, never dereferenced


def _pool(**over):
    d = dict(A=FAKE, B=FAKE, slot_rank=FAKE, slot_scale=FAKE, dtype=agm.BF16, n_slots=4, r_cap=16,
             d_in=64, d_out=64)
    d.update(over)
    return agm.PoolDesc(**d)


def _shrink(pool, seg=FAKE, T=4, x=FAKE, ld_x=64, v=FAKE, ld_v=16, launch=agm.LAUNCH_PERSISTENT):
    return agm.lib().lora_shrink(None if pool is None else ctypes.byref(pool), seg, T, None, x, ld_x, v, ld_v,
                                 launch, None)


def test_shrink_validation():
    L = agm
    assert _shrink(None) == L.LORA_E_ARG
    assert _shrink(_pool(A=None)) == L.LORA_E_ARG
    assert _shrink(_pool(r_cap=0)) == L.LORA_E_RANK
    assert _shrink(_pool(r_cap=136)) == L.LORA_E_RANK
    assert _shrink(_pool(r_cap=12)) == L.LORA_E_ALIGN          # bf16 rank rows need 16-byte multiples
    assert _shrink(_pool(dtype=7)) == L.LORA_E_DTYPE
    assert _shrink(_pool(d_in=60)) == L.LORA_E_ALIGN
    assert _shrink(_pool(A=FAKE + 8)) == L.LORA_E_ALIGN
    assert _shrink(_pool(), seg=None) == L.LORA_E_ARG
    assert _shrink(_pool(), T=-1) == L.LORA_E_ARG
    assert _shrink(_pool(), ld_x=32) == L.LORA_E_ARG
    assert _shrink(_pool(), ld_v=8) == L.LORA_E_ARG
    assert _shrink(_pool(), x=FAKE + 4) == L.LORA_E_ALIGN
    assert _shrink(_pool(), launch=9) == L.LORA_E_ARG
    assert _shrink(_pool(), launch=agm.LAUNCH_EXACT) == L.LORA_E_ARG    # EXACT needs the host summary


def test_build_shrink_validation():
    """Every argument check of the combined build-and-shrink call runs before
    any launch (made-up device addresses are never dereferenced)."""
    L = agm

    def bs(pool=None, ids=FAKE, T=4, order=0, seg=FAKE, x=FAKE, ld_x=64, v=FAKE, ld_v=16):
        pool = _pool() if pool is None else pool
        return agm.lib().lora_build_shrink_dev(ids, None, T, order, ctypes.byref(pool), seg, x, ld_x, v, ld_v, None)

    assert agm.lib().lora_build_shrink_dev(FAKE, None, 4, 0, None, FAKE, FAKE, 64, FAKE, 16, None) == L.LORA_E_ARG
    assert bs(pool=_pool(r_cap=136)) == L.LORA_E_RANK
    assert bs(pool=_pool(dtype=7)) == L.LORA_E_DTYPE
    assert bs(pool=_pool(n_slots=L.DEV_MAX_SLOTS + 1)) == L.LORA_E_SIZE
    assert bs(ids=None) == L.LORA_E_ARG
    assert bs(seg=None) == L.LORA_E_ARG
    assert bs(T=-1) == L.LORA_E_ARG
    assert bs(order=2) == L.LORA_E_ARG
    assert bs(ld_x=32) == L.LORA_E_ARG
    assert bs(ld_v=8) == L.LORA_E_ARG
    assert bs(x=FAKE + 4) == L.LORA_E_ALIGN
    assert bs(v=FAKE + 8) == L.LORA_E_ALIGN


def test_expand_validation():
    lib = agm.lib()
    p = _pool()
    e = lambda **k: lib.lora_expand(ctypes.byref(k.get("pool", p)), k.get("seg", FAKE), 4, None,
                                    k.get("v", FAKE), 16, k.get("y", FAKE), k.get("yd", agm.BF16),
                                    k.get("ld_y", 64), agm.LAUNCH_PERSISTENT, None)
    assert e(yd=agm.FP8_E4M3) == agm.LORA_E_DTYPE
    assert e(ld_y=32) == agm.LORA_E_ARG
    assert e(y=FAKE + 2) == agm.LORA_E_ALIGN
    assert e(v=None) == agm.LORA_E_ARG
    assert e(pool=_pool(B=None)) == agm.LORA_E_ARG


def test_fused_validation():
    lib = agm.lib()
    base = agm.BaseDesc(FAKE, None, agm.BF16, 64)

    def f(base=base, pool=None, seg=None, v=None, flags=0, ws=None, ws_bytes=0, x=FAKE, y=FAKE + 4096,
          d_in=64, d_out=64):
        return lib.lora_fused_linear(ctypes.byref(base), None if pool is None else ctypes.byref(pool), seg, 4,
                                     x, 64, v, 16, y, 64, d_in, d_out, flags, ws, ws_bytes, None)

    assert f(flags=0x10) == agm.LORA_E_ARG
    assert f(flags=agm.FLAG_ACT_QUANT_E4M3) == agm.LORA_E_DTYPE          # W8A8 needs an fp8 base
    assert f(base=agm.BaseDesc(FAKE, None, agm.FP8_E4M3, 64)) == agm.LORA_E_ARG   # no w_scale
    assert f(base=agm.BaseDesc(FAKE, FAKE, agm.FP8_E4M3, 64), flags=agm.FLAG_ACT_QUANT_E4M3) == agm.LORA_E_SIZE
    assert f(base=agm.BaseDesc(FAKE, FAKE, agm.FP8_E4M3, 64), d_in=56) == agm.LORA_E_ALIGN
    assert f(pool=_pool(dtype=agm.F32), seg=FAKE, v=FAKE) == agm.LORA_E_DTYPE
    assert f(pool=_pool(), seg=None, v=FAKE) == agm.LORA_E_ARG
    assert f(pool=_pool(d_out=128), seg=FAKE, v=FAKE) == agm.LORA_E_ARG
    assert f(v=FAKE) == agm.LORA_E_ARG                                    # v without a pool
    assert f(x=FAKE, y=FAKE) == agm.LORA_E_ARG                            # y aliases x
    assert f(d_out=60) == agm.LORA_E_ALIGN
    assert f(base=agm.BaseDesc(None, None, agm.BF16, 64)) == agm.LORA_E_ARG


def test_quant_and_dev_builder_validation():
    lib = agm.lib()
    assert lib.lora_quantize_e4m3(FAKE, 4, 24, 32, FAKE, 32, FAKE, None) == agm.LORA_E_ALIGN
    assert lib.lora_quantize_e4m3(FAKE, 4, 32, 16, FAKE, 32, FAKE, None) == agm.LORA_E_ARG
    assert lib.lora_build_segments_dev(FAKE, None, 8, agm.DEV_MAX_SLOTS + 1, 0, FAKE, None) == agm.LORA_E_SIZE
    assert lib.lora_build_segments_dev(FAKE, None, 8, 4, 3, FAKE, None) == agm.LORA_E_ARG
    assert lib.lora_build_segments_dev(None, None, 8, 4, 0, FAKE, None) == agm.LORA_E_ARG
    # bf16 filling the GPU exactly once (256 tiles of 64 x 64): no workspace;
    # more 128-row tiles than CUs (3 x 96 of 128 x 128): 64 bytes of claim
    # counters, and with a pool the packed adapter records of the 3 row tiles
    # after them (256-byte aligned); 256-row tiles (16 x 128 of 256 x 256)
    # stay one-shot (records only) for small rank capacities, but pools of
    # capacity >= 96 leave no LDS for them and take persistent 128 x 128
    # tiles: the query covers every capacity; fp8 W8A8: codes + scales
    rcap = lib.lora_fused_workspace_bytes_rcap

    def rec(bm):                     # one packed adapter record: 320-byte header + bm rows of 256 bf16
        return -(-(320 + bm * 512) // 256) * 256
    assert lib.lora_fused_workspace_bytes(256, 64, 4096, agm.BF16, 0) == 0
    assert rcap(384, 64, 12288, agm.BF16, 0, 0) == 64
    assert rcap(384, 64, 12288, agm.BF16, 0, 8) == 256 + 3 * rec(128)
    assert rcap(4096, 64, 32768, agm.BF16, 0, 0) == 0
    assert rcap(4096, 64, 32768, agm.BF16, 0, 8) == 16 * rec(256)
    assert rcap(4096, 64, 32768, agm.BF16, 0, 128) == 256 + 32 * rec(128)
    assert lib.lora_fused_workspace_bytes(4096, 64, 32768, agm.BF16, 0) == 256 + 32 * rec(128)
    assert lib.lora_fused_workspace_bytes(4, 64, 64, agm.FP8_E4M3, agm.FLAG_ACT_QUANT_E4M3) >= 4 * 64 + 16
    # a small output (10 tiles of 64 x 64): 2 k splits + 1 adapter split per tile
    assert lib.lora_fused_workspace_bytes(100, 1024, 264, agm.BF16, 0) == 10 * 3 * 64 * 64 * 4 + 10 * 4
    assert lib.lora_fused_workspace_bytes(0, 64, 64, agm.BF16, 0) == 0


def test_fused_slices_host_checks():
    """Sizes and argument errors of the sliced fused call (no device work:
    every check runs before anything is enqueued)."""
    lib = agm.lib()
    d = (ctypes.c_int32 * 2)(264, 136)
    assert lib.lora_fused_slices_workspace_bytes(0, 100, 1024, d, agm.BF16, 0) == 0
    # slices whose merged plan would split k run one by one: the larger lone need
    lone = max(lib.lora_fused_workspace_bytes(100, 1024, 264, agm.BF16, 0),
               lib.lora_fused_workspace_bytes(100, 1024, 136, agm.BF16, 0))
    assert lib.lora_fused_slices_workspace_bytes(2, 100, 1024, d, agm.BF16, 0) == lone > 0
    # a merged launch needs no partial tiles, only the claim counters of a
    # persistent launch (64 bytes) and, 256-byte aligned, the packed adapter
    # records of every slice (at most 3 slices x 16 row tiles of 128 rows)
    big = (ctypes.c_int32 * 3)(4096, 1024, 1024)
    rec128 = -(-(320 + 128 * 512) // 256) * 256
    assert lib.lora_fused_slices_workspace_bytes(3, 2048, 4096, big, agm.BF16, 0) == 64 + 256 + 3 * 16 * rec128
    # errors: no slices; base dtypes that differ
    E_ARG, E_DTYPE = 1, 4
    assert lib.lora_fused_linear_slices(0, None, None, None, 0, None, 0, 0, None, None, None, None, None, 0,
                                        None, 0, None) == E_ARG
    fake = 1 << 20                                   # aligned, never dereferenced
    bases = (agm.BaseDesc * 2)(agm.BaseDesc(fake, None, agm.BF16, 64), agm.BaseDesc(fake, None, agm.F32, 64))
    ys = (ctypes.c_void_p * 2)(2 * fake, 3 * fake)
    ldy = (ctypes.c_int32 * 2)(8, 8)
    dd = (ctypes.c_int32 * 2)(8, 8)
    assert lib.lora_fused_linear_slices(2, bases, None, None, 8, fake, 64, 64, dd, None, None, ys, ldy, 0,
                                        None, 0, None) == E_DTYPE
    # two slices writing one output
    same = (agm.BaseDesc * 2)(agm.BaseDesc(fake, None, agm.BF16, 64), agm.BaseDesc(fake, None, agm.BF16, 64))
    ys2 = (ctypes.c_void_p * 2)(2 * fake, 2 * fake)
    assert lib.lora_fused_linear_slices(2, same, None, None, 8, fake, 64, 64, dd, None, None, ys2, ldy, 0,
                                        None, 0, None) == E_ARG


@pytest.mark.parametrize("policy", [0, 1])
def test_registry_matches_the_residency_rules(policy):
    """The library's registry and the oracle's residency rules take the same
    slot, install and eviction decisions over 3000 acquires and releases of a
    few hot adapters and a long tail, including refusals when every slot is in
    use."""
    rng = np.random.default_rng(11 + policy)
    n = 5
    reg = agm.Registry(n, policy)
    model = oracle.Residency(n, "lfu" if policy == 1 else "lru")
    held = []
    for step in range(3000):
        if held and rng.random() < 0.45:
            k = held.pop(int(rng.integers(len(held))))
            reg.release(k)
            assert model.release(k)
            continue
        k = int(min(rng.zipf(1.3), 12))              # a few hot adapters, a long tail
        want = model.acquire(k)
        if want is None:
            with pytest.raises(agm.LoraError):
                reg.acquire(k)
            continue
        assert reg.acquire(k) == want, (step, k)
        held.append(k)
        assert reg.lookup(k) == want[0]
    st = reg.stats()
    assert [st["hits"], st["misses"], st["evictions"]] == [model.hits, model.misses, model.evictions]
    assert st["resident"] == model.resident()
    with pytest.raises(agm.LoraError):
        reg.release(10**6)                           # never acquired


def test_registry_and_install_argument_errors():
    lib = agm.lib()
    h = ctypes.c_void_p()
    assert lib.lora_registry_create(0, 0, ctypes.byref(h)) == 1
    assert lib.lora_registry_create(4, 7, ctypes.byref(h)) == 1
    assert lib.lora_pool_install(None, 0, None, None, 0, 1.0, None) == 1


def test_descriptors_keep_their_tensors_alive():
    """A descriptor carries raw addresses into the library, so it must hold its
    tensors: a weight built inline (``base_desc(make())``) freed at once would
    hand its memory to the next allocation while the descriptor still points
    at it."""
    import gc
    import weakref
    import torch
    W = torch.zeros(8, 16, dtype=torch.bfloat16)
    ref = weakref.ref(W)
    d = agm.base_desc(W)
    del W
    gc.collect()
    assert ref() is not None and d.W == ref().data_ptr()
    A = torch.zeros(2, 4, 16, dtype=torch.bfloat16)
    refs = [weakref.ref(t) for t in (A,)]
    p = agm.pool_desc(A, torch.zeros(2, 8, 4, dtype=torch.bfloat16), torch.zeros(2, dtype=torch.int32),
                      torch.zeros(2))
    del A
    gc.collect()
    assert all(r() is not None for r in refs) and p.A == refs[0]().data_ptr()


def test_cu_masked_stream_argument_errors():
    """Bad arguments are refused before any HIP call (no GPU needed)."""
    lib = agm.lib()
    h = ctypes.c_void_p()
    mask = (ctypes.c_uint32 * 8)(*([0xffffffff] * 8))
    zero = (ctypes.c_uint32 * 8)()
    assert lib.lora_stream_create_cu_masked(None, 8, ctypes.byref(h)) == 1
    assert lib.lora_stream_create_cu_masked(mask, 0, ctypes.byref(h)) == 1
    assert lib.lora_stream_create_cu_masked(mask, 8, None) == 1
    assert lib.lora_stream_create_cu_masked(zero, 8, ctypes.byref(h)) == 1     # no CU at all
    assert lib.lora_stream_destroy(None) == 1
    assert lib.lora_device_cu_count(None) == 1
    assert agm.cu_mask_words([0, 31, 32, 255], 256) == [0x80000001, 1, 0, 0, 0, 0, 0, 0x80000000]
    with pytest.raises(ValueError):
        agm.cu_mask_words([256], 256)


@pytest.mark.parametrize("r_cap", [0, 8, 16, 64, 96, 128])
def test_fused_workspace_query_covers_every_rank_capacity(r_cap):
    """The size query takes no pool, so it must cover the schedule of any
    rank capacity.  The exact need of a capacity is checked against the call
    itself without launching anything: only shapes that need a workspace are
    called, one byte short (LORA_E_SIZE) and with enough bytes at a
    deliberately misaligned address (LORA_E_ALIGN, after the size check)."""
    lib = agm.lib()
    fake = 1 << 20
    for (T, d_in, d_out) in [(2048, 4096, 4096), (8192, 4096, 28672), (256, 4096, 4096), (100, 1024, 264),
                             (512, 8192, 28672)]:
        any_cap = lib.lora_fused_workspace_bytes(T, d_in, d_out, agm.BF16, 0)
        need = lib.lora_fused_workspace_bytes_rcap(T, d_in, d_out, agm.BF16, 0, r_cap)
        assert any_cap >= need
        if need == 0:
            continue                      # a complete call would launch: not made here
        pool = agm.PoolDesc(fake, fake, fake, fake, agm.BF16, 64, r_cap, d_in, d_out) if r_cap else None
        base = agm.BaseDesc(fake, None, agm.BF16, d_in)

        def call(ws, nbytes):
            return lib.lora_fused_linear(ctypes.byref(base), ctypes.byref(pool) if pool else None,
                                         fake if pool else None, T, 2 * fake, d_in, 3 * fake if pool else None,
                                         max(r_cap, 4), 4 * fake, d_out, d_in, d_out, 0, ws, nbytes, None)
        assert call(fake, need - 1) == agm.LORA_E_SIZE
        assert call(fake + 16, need) == agm.LORA_E_ALIGN
        assert call(fake + 16, any_cap) == agm.LORA_E_ALIGN
    # the 2048-row 4096 -> 4096 shape at capacity 128 runs persistent 128 x 128
    # tiles with 64 bytes of claim counters (and 16 packed records), which
    # capacity 8 (one-shot 256 x 128 tiles, 8 records) does not need
    rec = lambda bm: -(-(320 + bm * 512) // 256) * 256
    assert lib.lora_fused_workspace_bytes_rcap(2048, 4096, 4096, agm.BF16, 0, 128) == 256 + 16 * rec(128)
    assert lib.lora_fused_workspace_bytes_rcap(2048, 4096, 4096, agm.BF16, 0, 8) == 8 * rec(256)
    assert lib.lora_fused_workspace_bytes(2048, 4096, 4096, agm.BF16, 0) == 256 + 16 * rec(128)
