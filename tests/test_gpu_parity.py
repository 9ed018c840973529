"""GPU parity: every library call against the fp64 oracle on the same seeded
inputs, through the C-ABI.

Tolerances (relative L2 against the oracle):
  segments                 bit-exact
  fp32 outputs (v, fp32 y) 1e-4
  bf16 outputs             1e-2
  fp8-base outputs         3e-2 (oracle on the dequantised weights)
Each output is checked globally, per row (max over rows) and on the adapter
term alone (expand on a zero y, or the fused call on a zero base).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import adapter_gemm_amd as agm
import oracle
from lora_inputs import make_workload
from gpu_helpers import (DEV, DevProjection, segments, split_seg, rel_l2, row_rel_l2, row_rel_magnitude, to_f64,
                         bf16_dev)

TOL = {"fp32": 1e-4, "bf16": 1e-2, "fp8": 3e-2}

# small variants: several tiles in every dimension and ragged tails
# (T, d_in, d_out not multiples of the tile sizes)
SMALL = {
    "tiny_sgmv": dict(),
    "decode_bgmv": dict(T=300, d_in=1032, d_out=1048, n_slots=40),
    "prefill_sgmv": dict(T=1000, d_in=520, d_out=1176, n_slots=24, n_req=7),
    "fp8_fused": dict(T=200, d_in=1040, d_out=904, n_slots=32, r=64),
    "llama_layer": dict(n_slots=96, n_req=3, prefill_len=40, n_decode=70,
                        shapes=[("q", 520, 264), ("down", 264, 520)]),
}


# shapes that take the pipelined fused kernel (d_in a multiple of its k-step):
# split-k with a separate adapter workgroup (few output tiles), 64-, 128- and
# 256-row tiles, fp8 with and without splits, rank capacity 128 (the widened
# fp8 mode then takes the general kernel), many adapter groups per tile,
# persistent workgroups claiming tiles (64- and 128-row tiles, more tiles than
# CUs; bf16 and widened fp8), ragged T and d_out throughout
PIPE = {
    "decode_split": ("decode_bgmv", dict(T=100, d_in=1024, d_out=264, n_slots=40)),
    "decode_64tile": ("decode_bgmv", dict(T=300, d_in=1024, d_out=1048, n_slots=40)),
    "decode_many_groups": ("decode_bgmv", dict(T=250, d_in=2048, d_out=520, n_slots=200)),
    "prefill_256x256": ("prefill_sgmv", dict(T=4100, d_in=512, d_out=8200, n_slots=24, n_req=9)),
    "prefill_256x128": ("prefill_sgmv", dict(T=2000, d_in=512, d_out=4088, n_slots=24, n_req=9)),
    "prefill_256x256_part": ("prefill_sgmv", dict(T=2100, d_in=512, d_out=4104, n_slots=24, n_req=9)),
    "fp8_split": ("fp8_fused", dict(T=200, d_in=1024, d_out=904, n_slots=32, r=64)),
    "fp8_r128": ("fp8_fused", dict(T=130, d_in=512, d_out=392, n_slots=16, r=128)),
    "decode_persistent": ("decode_bgmv", dict(T=600, d_in=1024, d_out=3000, n_slots=40)),       # 64x64, 470 tiles
    "prefill_persistent128": ("prefill_sgmv", dict(T=1100, d_in=512, d_out=4104, n_slots=24, n_req=5)),  # 128x128, 297
    "fp8_persistent": ("fp8_fused", dict(T=520, d_in=512, d_out=4112, n_slots=32, r=64)),        # 64x64 W8A16, 585
    # persistent launches whose XCD ranges are whole columns: heaviest row tiles claimed first
    "fp8_row_order": ("fp8_fused", dict(T=512, d_in=512, d_out=9216, n_slots=200, r=64)),        # 128x128 W8A16, 288
    "prefill_row_order": ("prefill_sgmv", dict(T=1024, d_in=512, d_out=5120, n_slots=64, n_req=40)),  # 128x128, 320
    # W8A8 on 256 x 128 tiles (its largest), W8A16 on persistent 128 x 128 tiles
    "fp8_wide": ("fp8_fused", dict(T=600, d_in=256, d_out=16376, n_slots=32, r=64)),
    "llama_kv": ("llama_layer", dict(n_slots=96, n_req=3, prefill_len=40, n_decode=70,
                                     shapes=[("k", 1024, 264), ("down", 768, 1032)])),
}


def _tol(p):
    return TOL["fp8"] if p.base_dtype == "fp8" else TOL[p.data_dtype]


def _delta_magnitude(dp, w):
    """The adapter term's sums over absolute values, row by row
    (|s| |B| (|A| |x|)): per-row checks of the adapter term alone take their
    scale from it, since a rank-1 row whose v cancels to nearly zero is small
    while its rounding is set by the terms it sums."""
    x, ids, act, A, B, rank, scale = dp.oracle_args(w)
    return oracle.lora_delta(np.abs(x), ids, act, np.abs(A), np.abs(B), rank, np.abs(scale))


def _v_ref(dp, w, segd):
    """oracle v in grouped order [n_active, r_cap]"""
    v_rows = oracle.shrink_rows(dp.x_host, w.ids, w.active, dp.A_host, dp.p.slot_rank)
    n = int(segd["sum"][0])
    return v_rows[segd["perm"][:n]]


# ---- segments ------------------------------------------------------------------

@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("device_build", [False, True])
def test_segments_bit_exact(name, order, device_build):
    w = make_workload(name, **SMALL[name])
    N = w.projections[0].n_slots
    seg, s = segments(w, N, order, device_build)
    d = split_seg(seg, w.T)
    ref = oracle.build_segments(w.ids, w.active, order)
    S = ref["S"]
    assert s.error == 0 and s.n_active == ref["n_active"] and s.n_segments == S and s.m_max == ref["m_max"]
    assert np.array_equal(d["perm"], ref["perm"])
    assert np.array_equal(d["seg_start"][:S + 1], ref["seg_start"])
    assert np.array_equal(d["seg_adapter"][:S], ref["seg_adapter"])
    want_pos = np.full(w.T, -1)
    for k in range(S):
        want_pos[ref["seg_start"][k]:ref["seg_start"][k + 1]] = k
    assert np.array_equal(d["pos_seg"], want_pos)
    for key, tile, n in (("tiles_small", 16, s.n_tiles_small), ("tiles_large", 64, s.n_tiles_large)):
        want = oracle.row_tiles(ref["seg_start"], tile)
        assert n == len(want)
        assert [(int(b), int(a)) for a, b in d[key][:n]] == [(x[0], x[1]) for x in want]
    assert s.row_bound == (oracle.row_bound(w.T, ref["m_max"]) if ref["n_active"] else 0)


def _check_layout(ids, act, N, order):
    """Device segment buffer against the oracle's grouping, field by field."""
    T = len(ids)
    seg = torch.empty(agm.segment_words(T), dtype=torch.int32, device=DEV)
    agm.build_segments_dev(torch.from_numpy(ids).to(DEV), None if act is None else torch.from_numpy(act).to(DEV),
                           N, seg, order)
    torch.cuda.synchronize()
    s = agm.summary_from_words(seg[:agm.SEG_HEADER].cpu().numpy())
    w = type("W", (), {})()
    w.T = T
    d = split_seg(seg, T)
    ref = oracle.build_segments(ids, np.ones(T, np.uint8) if act is None else act, order)
    S = ref["S"]
    case = (T, N, order, act is None)
    assert s.error == 0 and s.n_active == ref["n_active"] and s.n_segments == S and s.m_max == ref["m_max"], case
    assert np.array_equal(d["perm"], ref["perm"]), case
    assert np.array_equal(d["seg_start"][:S + 1], ref["seg_start"]), case
    assert np.array_equal(d["seg_adapter"][:S], ref["seg_adapter"]), case
    want_pos = np.full(w.T, -1)
    for k in range(S):
        want_pos[ref["seg_start"][k]:ref["seg_start"][k + 1]] = k
    assert np.array_equal(d["pos_seg"], want_pos), case
    for key, tile, n in (("tiles_small", 16, s.n_tiles_small), ("tiles_large", 64, s.n_tiles_large)):
        want = oracle.row_tiles(ref["seg_start"], tile)
        assert n == len(want), case
        assert [(int(b), int(a)) for a, b in d[key][:n]] == [(x[0], x[1]) for x in want], case
    assert s.row_bound == (oracle.row_bound(w.T, ref["m_max"]) if ref["n_active"] else 0), case


@pytest.mark.parametrize("order", [0, 1])
def test_device_segments_small_batch_kernel(order):
    """Batches of at most 256 rows with pools of at most 1024 adapters take the
    lane-mask builder; the edges of that range and just past it (the general
    builder) must give the oracle's grouping."""
    g = np.random.default_rng(9 + order)
    cases = [
        (256, 1024, g.integers(-1, 1024, 256), None),               # largest pool of the small builder
        (256, 1025, g.integers(-1, 1025, 256), None),               # one past: the general builder
        (256, 64, np.minimum(g.zipf(1.1, 256) - 1, 63), (g.uniform(size=256) > 0.5)),
        (200, 3, np.full(200, 2), None),                            # one adapter for every row
        (130, 8, g.integers(-1, 8, 130), np.zeros(130, bool)),      # every row inactive
        (1, 5, np.array([4]), None),                                # a single row
        (64, 1, np.full(64, -1), None),                             # no adapter anywhere
        (255, 1000, np.repeat(g.permutation(1000)[:51], 5), None),  # runs spanning waves
    ]
    for T, N, ids, act in cases:
        ids = np.asarray(ids, np.int32)
        if act is not None:
            act = np.asarray(act, np.uint8)
        _check_layout(ids, act, N, order)
        _check_layout(ids, np.ones(T, np.uint8), N, order)     # flags given, all set


@pytest.mark.parametrize("order", [0, 1])
def test_device_segments_wave_range_builder(order):
    """Batches of 2049 .. 16384 rows over at most 1024 adapters take the
    builder whose 16 waves each own one contiguous row range: its edges (and
    just past them, the chunked builder), segments that cross wave ranges,
    ragged T, inactive rows, Zipf-skewed ids and every field of the layout
    against the oracle's grouping, in both segment orders."""
    g = np.random.default_rng(31 + order)
    cases = [
        (2049, 128, g.integers(-1, 128, 2049), None),                              # first size it takes
        (16384, 1024, g.integers(-1, 1024, 16384), g.uniform(size=16384) > 0.3),  # largest batch and pool
        (16385, 64, g.integers(-1, 64, 16385), None),                             # one past: chunked builder
        (5000, 1025, g.integers(-1, 1025, 5000), None),                           # pool one past: chunked
        (8192, 128, np.repeat(g.integers(-1, 128, 32), 256), None),               # request runs over waves
        (3001, 40, np.minimum(g.zipf(1.2, 3001) - 1, 39), g.uniform(size=3001) > 0.1),
        (4097, 7, np.full(4097, 6), None),                                        # one adapter everywhere
        (2500, 16, g.integers(0, 16, 2500), np.zeros(2500, bool)),                # every row inactive
        (6000, 300, np.full(6000, -1), None),                                     # no adapter anywhere
    ]
    for T, N, ids, act in cases:
        ids = np.asarray(ids, np.int32)
        if act is not None:
            act = np.asarray(act, np.uint8)
        _check_layout(ids, act, N, order)
    # an out-of-range id in this builder's range is reported, as elsewhere
    ids = g.integers(0, 50, 3000).astype(np.int32)
    ids[2999] = 50
    w = type("W", (), {})()
    w.ids, w.active, w.T = ids, np.ones(3000, np.uint8), 3000
    seg, s = segments(w, 50, order, True)
    assert s.error == agm.LORA_E_ID


def test_device_segments_large_and_bad_ids():
    g = np.random.default_rng(5)
    for T, N in [(1, 1), (1023, 7), (1025, 8192), (5000, 300), (20000, 1024)]:
        ids = g.integers(-1, N, T).astype(np.int32)
        act = (g.uniform(size=T) > 0.2).astype(np.uint8)
        w = type("W", (), {})()
        w.ids, w.active, w.T = ids, act, T
        seg, s = segments(w, N, 0, True)
        d = split_seg(seg, T)
        ref = oracle.build_segments(ids, act, 0)
        assert np.array_equal(d["perm"], ref["perm"]), (T, N)
        assert s.n_tiles_small == len(oracle.row_tiles(ref["seg_start"], 16))
    # an out-of-range id is reported on the device; kernels then see no rows
    w.ids = np.array([0, 3, 9], np.int32)
    w.active = np.ones(3, np.uint8)
    w.T = 3
    seg, s = segments(w, 4, 0, True)
    assert s.error == agm.LORA_E_ID


# ---- shrink, expand -----------------------------------------------------------------

@pytest.mark.parametrize("name", list(SMALL))
def test_shrink_expand_parity(name):
    w = make_workload(name, **SMALL[name])
    for p in w.projections:
        dp = DevProjection(w, p)
        seg, s = segments(w, p.n_slots)
        segd = split_seg(seg, w.T)
        v = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
        agm.shrink(dp.pool, seg, w.T, s, dp.x, v)
        # adapter term alone: expand on y = 0
        y = torch.zeros(w.T, p.d_out, dtype=dp.ydtype, device=DEV)
        agm.expand(dp.pool, seg, w.T, s, v, y)
        torch.cuda.synchronize()
        n = s.n_active
        vg = v.cpu().numpy().astype(np.float64)[:n]
        vr = _v_ref(dp, w, segd)
        mask = np.arange(p.r_cap)[None, :] < p.slot_rank[w.ids[segd["perm"][:n]]][:, None]
        assert rel_l2(np.where(mask, vg, 0), vr) <= TOL["fp32"], name
        d_ref = oracle.lora_delta(*dp.oracle_args(w))
        d_got = to_f64(y)
        live = oracle.live_rows(w.ids, w.active)
        tol = _tol(p)
        assert rel_l2(d_got, d_ref) <= tol
        assert row_rel_magnitude(d_got[live], d_ref[live], _delta_magnitude(dp, w)[live]) <= tol
        assert np.all(d_got[~live] == 0)                 # rows not live untouched


def _seg_meaningful(d, words):
    """the parts of a segment buffer that its summary declares written"""
    S, nts, ntl = int(words[1]), int(words[4]), int(words[5])
    return [d["sum"][:8], d["perm"], d["pos_seg"], d["seg_start"][:S + 1], d["seg_adapter"][:S],
            d["tiles_small"][:nts], d["tiles_large"][:ntl]]


BUILD_SHRINK = {
    # one launch (T <= 256, <= 1024 slots)
    "decode_200": ("decode_bgmv", dict(T=200, d_in=1024, d_out=264, n_slots=40), 0),
    "decode_256_order1": ("decode_bgmv", dict(T=256, d_in=512, d_out=264, n_slots=64), 1),
    "decode_1024_slots": ("decode_bgmv", dict(T=256, d_in=512, d_out=264, n_slots=1024), 0),
    "tiny_fp32": ("tiny_sgmv", dict(), 0),
    "fp8_r64": ("fp8_fused", dict(T=130, d_in=1024, d_out=264, n_slots=32, r=64), 0),
    # two launches (T > 256)
    "decode_300": ("decode_bgmv", dict(T=300, d_in=1032, d_out=264, n_slots=40), 0),
}


@pytest.mark.parametrize("case", list(BUILD_SHRINK))
def test_build_shrink_equals_build_then_shrink(case):
    """lora_build_shrink_dev gives the device builder's segment buffer bit for
    bit, and the persistent shrink's v up to fp32 rounding (the one-launch
    kernel's four waves add the k chunks in another order than the shrink's
    sixteen): within 1e-6 of it, and within the fp32 gate of the oracle."""
    name, kw, order = BUILD_SHRINK[case]
    w = make_workload(name, **kw)
    p = w.projections[0]
    dp = DevProjection(w, p)
    ids = torch.from_numpy(w.ids.astype(np.int32)).to(DEV)
    act = torch.from_numpy(w.active.astype(np.uint8)).to(DEV)
    seg_ref = torch.full((agm.segment_words(w.T),), -7, dtype=torch.int32, device=DEV)
    v_ref = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
    agm.build_segments_dev(ids, act, p.n_slots, seg_ref, order)
    agm.shrink(dp.pool, seg_ref, w.T, None, dp.x, v_ref, launch=agm.LAUNCH_PERSISTENT)
    seg = torch.full((agm.segment_words(w.T),), -9, dtype=torch.int32, device=DEV)
    v = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
    agm.build_shrink_dev(ids, act, dp.pool, seg, dp.x, v, order=order)
    torch.cuda.synchronize()
    d_ref, d = split_seg(seg_ref, w.T), split_seg(seg, w.T)
    words = d_ref["sum"]
    assert int(words[7]) == 0 and np.array_equal(d["sum"][:8], words[:8])
    for a, b in zip(_seg_meaningful(d, words), _seg_meaningful(d_ref, words)):
        assert np.array_equal(a, b), case
    n = int(words[0])
    mask = np.arange(p.r_cap)[None, :] < p.slot_rank[w.ids[d_ref["perm"][:n]]][:, None]
    vg, vr = v.cpu().numpy()[:n].astype(np.float64), v_ref.cpu().numpy()[:n].astype(np.float64)
    assert np.isfinite(vg[mask]).all()
    assert rel_l2(vg[mask], vr[mask]) <= 1e-6, case
    # deterministic: a second call gives the same bits
    v2 = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
    agm.build_shrink_dev(ids, act, dp.pool, seg, dp.x, v2, order=order)
    torch.cuda.synchronize()
    assert np.array_equal(v2.cpu().numpy()[:n][mask], v.cpu().numpy()[:n][mask])
    # and against the oracle
    ref = _v_ref(dp, w, d_ref)
    assert rel_l2(np.where(mask, vg.astype(np.float64), 0.0), ref) <= TOL["fp32"]


def test_build_shrink_bad_id_and_empty():
    """An id out of range is reported in the summary and v is not written; an
    empty batch writes the summary only."""
    w = make_workload("decode_bgmv", T=64, d_in=512, d_out=264, n_slots=16)
    p = w.projections[0]
    dp = DevProjection(w, p)
    bad = w.ids.astype(np.int32).copy()
    bad[5] = p.n_slots
    ids = torch.from_numpy(bad).to(DEV)
    seg = torch.zeros(agm.segment_words(w.T), dtype=torch.int32, device=DEV)
    v = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
    agm.build_shrink_dev(ids, None, dp.pool, seg, dp.x, v)
    torch.cuda.synchronize()
    words = seg[:agm.SEG_HEADER].cpu().numpy()
    assert int(words[7]) == agm.LORA_E_ID and int(words[6]) == w.T
    assert torch.isnan(v).all()
    seg0 = torch.full((agm.segment_words(0),), -1, dtype=torch.int32, device=DEV)
    agm.build_shrink_dev(torch.zeros(0, dtype=torch.int32, device=DEV), None, dp.pool, seg0, dp.x, v)
    torch.cuda.synchronize()
    w0 = seg0[:agm.SEG_HEADER].cpu().numpy()
    assert int(w0[0]) == 0 and int(w0[6]) == 0 and int(w0[7]) == 0


@pytest.mark.parametrize("launch", [agm.LAUNCH_EXACT, agm.LAUNCH_PERSISTENT, agm.LAUNCH_BUCKETED,
                                    agm.LAUNCH_FULL_BATCH])
def test_launch_modes_bitwise_identical(launch):
    w = make_workload("llama_layer", **SMALL["llama_layer"])
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    outs = []
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1)
    y0 = torch.randn(w.T, p.d_out, device=DEV, generator=gen).to(torch.bfloat16)
    for mode in (agm.LAUNCH_EXACT, launch):
        v = torch.zeros(w.T, p.r_cap, device=DEV)
        y = y0.clone()
        agm.shrink(dp.pool, seg, w.T, s, dp.x, v, launch=mode)
        agm.expand(dp.pool, seg, w.T, s, v, y, launch=mode)
        torch.cuda.synchronize()
        outs.append((v.cpu(), y.cpu()))
    n = s.n_active
    assert torch.equal(outs[0][0][:n], outs[1][0][:n])
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


@pytest.mark.parametrize("launch", [agm.LAUNCH_EXACT, agm.LAUNCH_BUCKETED])
def test_stale_host_summary_costs_no_rows(launch):
    """EXACT and BUCKETED size their grids from the host summary but take
    the work from the device buffer: a summary of another batch of the same
    T (one live row: one tile, row bound 16) still gives every row."""
    w = make_workload("llama_layer", **SMALL["llama_layer"])
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    assert s.n_tiles_small > 1 and s.row_bound > 16
    stale = agm.Summary(1, 1, 1, 16, 1, 1, w.T, 0)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2)
    y0 = torch.randn(w.T, p.d_out, device=DEV, generator=gen).to(torch.bfloat16)
    outs = []
    for summ in (s, stale):
        v = torch.zeros(w.T, p.r_cap, device=DEV)
        y = y0.clone()
        agm.shrink(dp.pool, seg, w.T, summ, dp.x, v, launch=launch)
        agm.expand(dp.pool, seg, w.T, summ, v, y, launch=launch)
        torch.cuda.synchronize()
        outs.append((v.cpu(), y.cpu()))
    n = s.n_active
    assert torch.equal(outs[0][0][:n], outs[1][0][:n])
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def test_expand_leaves_other_rows_bitwise_untouched():
    w = make_workload("decode_bgmv", **SMALL["decode_bgmv"])
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    v = torch.zeros(w.T, p.r_cap, device=DEV)
    agm.shrink(dp.pool, seg, w.T, s, dp.x, v)
    y0 = torch.randn(w.T, p.d_out, device=DEV).to(torch.bfloat16)
    y = y0.clone()
    agm.expand(dp.pool, seg, w.T, s, v, y)
    torch.cuda.synchronize()
    dead = torch.from_numpy(~oracle.live_rows(w.ids, w.active)).to(DEV)
    assert dead.sum() > 0
    assert torch.equal(y[dead].view(torch.int16), y0[dead].view(torch.int16))
    # and the live rows changed consistently with base + delta
    ref = y0.double().cpu().numpy() + oracle.lora_delta(*dp.oracle_args(w))
    assert rel_l2(to_f64(y), ref) <= TOL["bf16"]


# ---- fused linear -------------------------------------------------------------------

def _fused(dp, seg, s, w, flags=0, zero_base=False, with_pool=True):
    p = dp.p
    v = torch.zeros(w.T, p.r_cap, device=DEV)
    if with_pool:
        agm.shrink(dp.pool, seg, w.T, s, dp.x, v)
    base = dp.base
    if zero_base:
        Wz = torch.zeros_like(dp.W)
        base = agm.base_desc(Wz, dp.w_scale)
    y = torch.full((w.T, p.d_out), float("nan"), device=DEV).to(dp.ydtype)
    bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}[p.base_dtype]
    ws = agm.fused_workspace(w.T, p.d_in, p.d_out, bt, flags, device=DEV)
    agm.fused_linear(base, dp.pool if with_pool else None, seg if with_pool else None, dp.x,
                     v if with_pool else None, y, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    return to_f64(y)


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_parity(name):
    w = make_workload(name, **SMALL[name])
    for p in w.projections:
        dp = DevProjection(w, p)
        seg, s = segments(w, p.n_slots)
        y = _fused(dp, seg, s, w)
        ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
        tol = _tol(p)
        assert np.isfinite(y).all()
        assert rel_l2(y, ref) <= tol, (name, p.name, rel_l2(y, ref))
        assert row_rel_l2(y, ref) <= tol
        # adapter term alone (zero base)
        d = _fused(dp, seg, s, w, zero_base=True)
        d_ref = oracle.lora_delta(*dp.oracle_args(w))
        live = oracle.live_rows(w.ids, w.active)
        if live.any():
            assert rel_l2(d, d_ref) <= tol
            assert row_rel_l2(d[live], d_ref[live]) <= tol
        # inactive rows equal the base-only run bit for bit
        yb = _fused(dp, seg, s, w, with_pool=False)
        assert np.array_equal(y[~live], yb[~live])


@pytest.mark.parametrize("case", list(PIPE))
def test_fused_pipelined_parity(case):
    name, kw = PIPE[case]
    w = make_workload(name, **kw)
    for p in w.projections:
        assert p.d_in % 128 == 0
        dp = DevProjection(w, p)
        seg, s = segments(w, p.n_slots)
        y = _fused(dp, seg, s, w)
        ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
        tol = _tol(p)
        assert np.isfinite(y).all()
        assert rel_l2(y, ref) <= tol, (case, p.name, rel_l2(y, ref))
        assert row_rel_l2(y, ref) <= tol
        d = _fused(dp, seg, s, w, zero_base=True)
        d_ref = oracle.lora_delta(*dp.oracle_args(w))
        live = oracle.live_rows(w.ids, w.active)
        if live.any():
            assert rel_l2(d, d_ref) <= tol, (case, rel_l2(d, d_ref))
            assert row_rel_l2(d[live], d_ref[live]) <= tol
        yb = _fused(dp, seg, s, w, with_pool=False)
        assert np.array_equal(y[~live], yb[~live])
        # repeated calls (the split schedule re-arms its counters) are bitwise equal
        assert np.array_equal(_fused(dp, seg, s, w), y)
        if p.base_dtype == "fp8":
            # W8A8 adds the activation quantisation error on top (an option, not
            # the parity mode): the global gate against the fp64 oracle, and the
            # kernel checked row by row against the oracle's own W8A8 definition
            y8 = _fused(dp, seg, s, w, flags=agm.FLAG_ACT_QUANT_E4M3)
            assert rel_l2(y8, ref) <= TOL["fp8"]
            ref8 = oracle.linear_w8a8(dp.x_host, dp.w0_host[0], dp.w0_host[1], *dp.oracle_args(w)[1:])
            assert rel_l2(y8, ref8) <= TOL["bf16"] and row_rel_l2(y8, ref8) <= TOL["bf16"]


# ---- the shrink inside the fused launch (LORA_FLAG_SHRINK_IN_LAUNCH) ----------

# decode-sized tiles run the shrink in the same launch (64x64 bf16 one-shot and
# persistent, 128x128 bf16 persistent, W8A16 64x64 and 128x128 persistent);
# other plans (256-row tiles, W8A8) run it as a launch of its own first
INLAUNCH = {
    "decode_64": ("decode_bgmv", dict(T=300, d_in=1024, d_out=1048, n_slots=40)),
    "decode_small_split_shape": ("decode_bgmv", dict(T=100, d_in=1024, d_out=264, n_slots=40)),
    "decode_persistent": ("decode_bgmv", dict(T=600, d_in=1024, d_out=3000, n_slots=40)),
    "prefill_persistent128": ("prefill_sgmv", dict(T=1100, d_in=512, d_out=4104, n_slots=24, n_req=5)),
    "fp8_persistent64": ("fp8_fused", dict(T=520, d_in=512, d_out=4112, n_slots=32, r=64)),
    "fp8_wide128": ("fp8_fused", dict(T=600, d_in=256, d_out=16376, n_slots=32, r=64)),
    "prefill_256_fallback": ("prefill_sgmv", dict(T=2000, d_in=512, d_out=4088, n_slots=24, n_req=9)),
    "released_rows": ("llama_layer", dict(n_slots=96, n_req=3, prefill_len=40, n_decode=70,
                                          shapes=[("q", 1024, 1048)])),
}


def _fused_in_launch(dp, seg, w, flags=0):
    p = dp.p
    v = torch.full((w.T, p.r_cap), float("nan"), device=DEV)     # an output of the call
    y = torch.full((w.T, p.d_out), float("nan"), device=DEV).to(dp.ydtype)
    bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3}[p.base_dtype]
    f = flags | agm.FLAG_SHRINK_IN_LAUNCH
    ws = agm.fused_workspace(w.T, p.d_in, p.d_out, bt, f, device=DEV)
    agm.fused_linear(dp.base, dp.pool, seg, dp.x, v, y, flags=f, workspace=ws)
    torch.cuda.synchronize()
    return to_f64(y), v.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", list(INLAUNCH))
def test_fused_shrink_in_launch_parity(case):
    """EpiLoRA's decode path: the fused call computes v itself, in the same
    launch; v and y against the fp64 oracle, inactive rows against the base
    alone, and two calls bitwise equal."""
    name, kw = INLAUNCH[case]
    w = make_workload(name, **kw)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    print(f"case {case}: T={w.T} {p.d_in}->{p.d_out} r_cap={p.r_cap}", flush=True)
    y, v = _fused_in_launch(dp, seg, w)
    segd = split_seg(seg, w.T)
    n = s.n_active
    v_ref = _v_ref(dp, w, segd)
    rk = p.slot_rank[segd["seg_adapter"][segd["pos_seg"][:n]]] if n else np.zeros(0, int)
    mask = np.arange(p.r_cap)[None, :] < rk[:, None]
    assert rel_l2(v[:n][mask], v_ref[mask]) <= TOL["fp32"], (case, rel_l2(v[:n][mask], v_ref[mask]))
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    tol = _tol(p)
    assert np.isfinite(y).all()
    assert rel_l2(y, ref) <= tol, (case, rel_l2(y, ref))
    assert row_rel_l2(y, ref) <= tol
    # inactive rows get the base product only (the in-launch plan never splits
    # k, so its rounding can differ from a base-only call that does: compared
    # by value against the oracle's base rows)
    live = oracle.live_rows(w.ids, w.active)
    if (~live).any():
        base_ref = oracle.base_output(dp.x_host, dp.w0_host)
        assert row_rel_l2(y[~live], base_ref[~live]) <= tol
    y2, v2 = _fused_in_launch(dp, seg, w)
    assert np.array_equal(y2, y) and np.array_equal(v2[:n][mask], v[:n][mask])
    if p.base_dtype == "fp8":
        # W8A8: the shrink reads the unquantised x (a launch of its own first)
        y8, _ = _fused_in_launch(dp, seg, w, flags=agm.FLAG_ACT_QUANT_E4M3)
        ref8 = oracle.linear_w8a8(dp.x_host, dp.w0_host[0], dp.w0_host[1], *dp.oracle_args(w)[1:])
        assert rel_l2(y8, ref8) <= TOL["bf16"] and row_rel_l2(y8, ref8) <= TOL["bf16"]


# ---- several output slices of one x in one launch (q / k / v, gate / up) -------

# merged launches on 64- and 256-row tiles with ragged slice ends, a shape
# whose merged plan would split k (the slices then run one by one), and fp8
SLICES = {
    "qkv_64tile": ("llama_layer", dict(n_slots=96, n_req=3, prefill_len=40, n_decode=70,
                                       shapes=[("q", 1024, 1024), ("k", 1024, 264), ("v", 1024, 264)])),
    "qkv_split_fallback": ("llama_layer", dict(n_slots=40, n_req=2, prefill_len=20, n_decode=60,
                                               shapes=[("q", 512, 264), ("k", 512, 136), ("v", 512, 136)])),
    "gate_up_256": ("llama_layer", dict(n_slots=96, n_req=7, prefill_len=300, n_decode=4,
                                        shapes=[("gate", 512, 2056), ("up", 512, 2056)])),
    "fp8_two": ("fp8_fused", [904, 520]),
    # 640 tiles of 256 x 256 on 256 CUs (2.5 rounds): the last half round
    # runs as a second launch of 256 x 128 tiles over up's last 4080 columns
    "gate_up_tail_split": ("llama_layer", dict(n_slots=96, n_req=16, prefill_len=96, n_decode=512,
                                               shapes=[("gate", 128, 10240), ("up", 128, 10224)])),
}


def _slice_setup(case):
    name, kw = SLICES[case]
    if name == "fp8_fused":
        ws = [make_workload(name, T=200, d_in=1024, d_out=d, n_slots=32, r=64) for d in kw]
        assert all(np.array_equal(ws[0].ids, x.ids) for x in ws)
        return ws[0], [DevProjection(x, x.projections[0]) for x in ws], ws
    w = make_workload(name, **kw)
    return w, [DevProjection(w, p) for p in w.projections], [w] * len(w.projections)


def _random_slices(i):
    """Seeded random slice set: 2-4 projections of one input (own output
    width, rank capacity, ranks and scales each), bf16 or fp8 base."""
    g = np.random.default_rng(8100 + i)
    base = "fp8" if i % 2 else "bf16"
    T = int(g.integers(1, 1200))
    d_in = int(64 * g.integers(1, 20)) if i % 3 else int(16 * g.integers(1, 80))
    N = int(g.integers(1, 200))
    ids = np.minimum(g.zipf(1.2, T) - 1, N - 1) if g.uniform() < 0.5 else g.integers(0, N, T)
    ids = np.where(g.uniform(size=T) < 0.1, -1, ids).astype(np.int32)
    active = (g.uniform(size=T) > 0.1).astype(np.uint8)
    from lora_inputs import Projection, Workload
    projs = []
    for k in range(int(g.integers(2, 5))):
        r_cap = int(g.choice([8, 16, 32, 64]))
        ranks = np.where(g.uniform(size=N) < 0.3, r_cap, g.integers(1, r_cap + 1, N)).astype(np.int32)
        projs.append(Projection(f"s{k}", d_in, int(8 * g.integers(1, 700)), N, r_cap, ranks,
                                g.uniform(0.25, 2.0, N).astype(np.float32), 0.05, 0.05, 0.05, base, "bf16",
                                (i, 88, k)))
    return Workload("random_slices", i, T, projs, ids, active, "bf16")


@pytest.mark.parametrize("i", range(16))
def test_random_slices_parity(i):
    """Seeded random slice sets in one launch: every slice against the fp64
    oracle (W8A8 against its quantised definition) and the base products
    alone against the oracle without adapters."""
    w = _random_slices(i)
    dps = [DevProjection(w, p) for p in w.projections]
    p0 = dps[0].p
    print(f"case {i}: {p0.base_dtype} T={w.T} d_in={p0.d_in} slices {[(d.p.d_out, d.p.r_cap) for d in dps]} "
          f"N={p0.n_slots}", flush=True)
    seg, s = segments(w, p0.n_slots)
    x, x_host = dps[0].x, dps[0].x_host
    bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3}[p0.base_dtype]
    vs = []
    for dp in dps:
        v = torch.zeros(w.T, dp.p.r_cap, device=DEV)
        agm.shrink(dp.pool, seg, w.T, s, x, v)
        vs.append(v)
    d_outs = [dp.p.d_out for dp in dps]
    for flags in ([0, agm.FLAG_ACT_QUANT_E4M3] if p0.base_dtype == "fp8" else [0]):
        wsp = agm.fused_slices_workspace(w.T, p0.d_in, d_outs, bt, flags, device=DEV)
        ys = [torch.full((w.T, dp.p.d_out), float("nan"), device=DEV).to(dp.ydtype) for dp in dps]
        agm.fused_linear_slices([dp.base for dp in dps], [dp.pool for dp in dps], seg, x, vs, ys, flags=flags,
                                workspace=wsp)
        torch.cuda.synchronize()
        for dp, y in zip(dps, ys):
            got = to_f64(y)
            args = dp.oracle_args(w)[1:]
            if flags:
                ref, tol = oracle.linear_w8a8(x_host, dp.w0_host[0], dp.w0_host[1], *args), TOL["bf16"]
            else:
                ref, tol = oracle.linear(x_host, dp.w0_host, *args), _tol(dp.p)
            assert rel_l2(got, ref) <= tol and row_rel_l2(got, ref) <= tol, (i, dp.p.name, flags)
    ys = [torch.full((w.T, dp.p.d_out), float("nan"), device=DEV).to(dp.ydtype) for dp in dps]
    wsp = agm.fused_slices_workspace(w.T, p0.d_in, d_outs, bt, 0, device=DEV)
    agm.fused_linear_slices([dp.base for dp in dps], None, seg, x, None, ys, workspace=wsp)
    torch.cuda.synchronize()
    no_ids = np.full(w.T, -1, np.int32)
    for dp, y in zip(dps, ys):
        ref = oracle.linear(x_host, dp.w0_host, no_ids, w.active, dp.A_host, dp.B_host, dp.p.slot_rank,
                            dp.p.slot_scale)
        assert rel_l2(to_f64(y), ref) <= _tol(dp.p)


@pytest.mark.parametrize("case", list(SLICES))
def test_fused_slices_parity(case):
    w, dps, ws = _slice_setup(case)
    p0 = dps[0].p
    seg, s = segments(w, p0.n_slots)
    x, x_host = dps[0].x, dps[0].x_host          # one input for every slice
    bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}[p0.base_dtype]
    vs = []
    for dp in dps:
        v = torch.zeros(w.T, dp.p.r_cap, device=DEV)
        agm.shrink(dp.pool, seg, w.T, s, x, v)
        vs.append(v)
    d_outs = [dp.p.d_out for dp in dps]
    flag_sets = [0, agm.FLAG_ACT_QUANT_E4M3] if p0.base_dtype == "fp8" else [0]
    for flags in flag_sets:
        wsp = agm.fused_slices_workspace(w.T, p0.d_in, d_outs, bt, flags, device=DEV)
        ys = [torch.full((w.T, dp.p.d_out), float("nan"), device=DEV).to(dp.ydtype) for dp in dps]
        agm.fused_linear_slices([dp.base for dp in dps], [dp.pool for dp in dps], seg, x, vs, ys, flags=flags,
                                workspace=wsp)
        torch.cuda.synchronize()
        for dp, wk, y in zip(dps, ws, ys):
            got = to_f64(y)
            args = dp.oracle_args(wk)[1:]
            if flags:
                ref = oracle.linear_w8a8(x_host, dp.w0_host[0], dp.w0_host[1], *args)
                tol = TOL["bf16"]
            else:
                ref = oracle.linear(x_host, dp.w0_host, *args)
                tol = _tol(dp.p)
            assert np.isfinite(got).all(), (case, dp.p.name)
            assert rel_l2(got, ref) <= tol, (case, dp.p.name, flags, rel_l2(got, ref))
            assert row_rel_l2(got, ref) <= tol, (case, dp.p.name, flags)
            # the same product as a lone call on this slice, to the output's rounding
            y1 = torch.full_like(y, float("nan"))
            ws1 = agm.fused_workspace(w.T, dp.p.d_in, dp.p.d_out, bt, flags, device=DEV)
            agm.fused_linear(dp.base, dp.pool, seg, x, vs[dps.index(dp)], y1, flags=flags, workspace=ws1)
            torch.cuda.synchronize()
            assert rel_l2(got, to_f64(y1)) <= tol
    # base products alone: no pools, no v
    ys = [torch.full((w.T, dp.p.d_out), float("nan"), device=DEV).to(dp.ydtype) for dp in dps]
    wsp = agm.fused_slices_workspace(w.T, p0.d_in, d_outs, bt, 0, device=DEV)
    agm.fused_linear_slices([dp.base for dp in dps], None, seg, x, None, ys, workspace=wsp)
    torch.cuda.synchronize()
    live = np.zeros(w.T, bool)
    for dp, wk, y in zip(dps, ws, ys):
        args = list(dp.oracle_args(wk)[1:])
        args[0] = np.full(w.T, -1, np.int32)      # no adapter on any row: the base product
        ref = oracle.linear(x_host, dp.w0_host, *args)
        assert rel_l2(to_f64(y), ref) <= _tol(dp.p), (case, dp.p.name, "base only")


# ---- adapter residency: registry + slot installs ----------------------------------

def test_residency_install_and_evict():
    """Twelve adapters served through a five-slot pool: each batch acquires
    its adapters from the registry, the misses are installed from pinned host
    memory on a side stream, the compute stream waits for that copy, and the
    fused output matches the oracle on the adapters' own ids (the pool starts
    as NaN, so a slot read before its install would poison the output)."""
    from lora_inputs import bf16_round
    g = np.random.default_rng(21)
    n_ad, n_slots, r_cap, d_in, d_out, T = 12, 5, 16, 256, 136, 96
    ranks = g.integers(1, r_cap + 1, n_ad).astype(np.int32)
    scales = g.uniform(0.5, 2.0, n_ad).astype(np.float32)
    A_all = np.zeros((n_ad, r_cap, d_in), np.uint16)
    B_all = np.zeros((n_ad, d_out, r_cap), np.uint16)
    A_src, B_src = [], []
    for k in range(n_ad):
        a = bf16_round(g.standard_normal((ranks[k], d_in)).astype(np.float32) * 0.05)
        b = bf16_round(g.standard_normal((d_out, ranks[k])).astype(np.float32) * 0.05)
        A_all[k, :ranks[k]] = a
        B_all[k, :, :ranks[k]] = b
        A_src.append(torch.from_numpy(a.view(np.int16)).pin_memory())
        B_src.append(torch.from_numpy(b.view(np.int16)).pin_memory())
    W0 = bf16_round(g.standard_normal((d_out, d_in)).astype(np.float32) * 0.02)
    base = agm.base_desc(bf16_dev(W0))
    A_pool = torch.full((n_slots, r_cap, d_in), float("nan"), device=DEV).to(torch.bfloat16)
    B_pool = torch.full((n_slots, d_out, r_cap), float("nan"), device=DEV).to(torch.bfloat16)
    rank_d = torch.zeros(n_slots, dtype=torch.int32, device=DEV)
    scale_d = torch.zeros(n_slots, dtype=torch.float32, device=DEV)
    pool = agm.pool_desc(A_pool, B_pool, rank_d, scale_d)
    reg = agm.Registry(n_slots, agm.EVICT_LRU)
    copy = torch.cuda.Stream()
    ws = agm.fused_workspace(T, d_in, d_out, agm.BF16, device=DEV)
    for names in ([0, 1, 2], [3, 1, 4, 5, 6], [0, 7, 8], [9, 10, 11, 2, 3], [1, 0]):
        ids_ad = g.choice(names + [-1], size=T).astype(np.int32)
        slot_of = {}
        for k in sorted(set(ids_ad[ids_ad >= 0].tolist())):
            s_, need = reg.acquire(k)
            slot_of[k] = s_
            if need:
                agm.pool_install(pool, s_, A_src[k], B_src[k], int(ranks[k]), float(scales[k]), stream=copy)
        torch.cuda.current_stream().wait_event(copy.record_event())
        ids_slot = np.array([slot_of[k] if k >= 0 else -1 for k in ids_ad], np.int32)
        x_h = bf16_round(g.standard_normal((T, d_in)).astype(np.float32))
        x = bf16_dev(x_h)
        seg = torch.empty(agm.segment_words(T), dtype=torch.int32, device=DEV)
        agm.build_segments_dev(torch.from_numpy(ids_slot).to(DEV), None, n_slots, seg)
        v = torch.zeros(T, r_cap, device=DEV)
        agm.shrink(pool, seg, T, None, x, v, launch=agm.LAUNCH_PERSISTENT)
        y = torch.full((T, d_out), float("nan"), device=DEV).to(torch.bfloat16)
        agm.fused_linear(base, pool, seg, x, v, y, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.linear(x_h, W0, ids_ad, np.ones(T, np.uint8), A_all, B_all, ranks, scales)
        got = to_f64(y)
        assert np.isfinite(got).all(), names
        assert rel_l2(got, ref) <= TOL["bf16"] and row_rel_l2(got, ref) <= TOL["bf16"], names
        for k in slot_of:
            reg.release(k)
    st = reg.stats()
    assert st["evictions"] > 0 and st["hits"] > 0


def test_fused_w8a8_parity():
    w = make_workload("fp8_fused", **SMALL["fp8_fused"])
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    y = _fused(dp, seg, s, w, flags=agm.FLAG_ACT_QUANT_E4M3)
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    assert rel_l2(y, ref) <= TOL["fp8"]
    assert row_rel_l2(y, ref) <= TOL["fp8"]
    # same quantised activations as the oracle's W8A8 definition: much closer
    ref8 = oracle.linear_w8a8(dp.x_host, dp.w0_host[0], dp.w0_host[1], *dp.oracle_args(w)[1:])
    assert rel_l2(y, ref8) <= TOL["bf16"]


# every amax is a bf16 value: s_x = 3, 5, 1, inexact ones (312, 7.5, 0.1, 30720),
# a small one, 2^-90 and its neighbours on either side (1.5 and 1.75 x 2^-82,
# 2^-80), a huge one (2^103) and a subnormal one
_QUANT_AMAX = [1344.0, 2240.0, 448.0, 312.0, 7.5, 0.10009765625, 30720.0, 0.0478515625,
               1.5 * 2.0 ** -82, 1.75 * 2.0 ** -82, 2.0 ** -80, 2.0 ** 103, 1.1663108e-38]


@pytest.mark.parametrize("d", [5136, 17424])
@pytest.mark.parametrize("amax", _QUANT_AMAX)
def test_quantize_e4m3_every_bf16_value(amax, d):
    """Every finite bf16 value of magnitude <= amax, over rows of d values that
    each end in amax (so that every row's s_x = amax / 448 exactly as chosen),
    against the oracle's codes bit for bit: every quotient a row can produce,
    ties and near-ties to the e4m3 rounding boundaries included.  d: a row of
    up to 16384 values (held in registers between the two passes, here with a
    ragged last 2048-value chunk) and a longer one."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= np.float32(amax))]
    per = d - 1
    T = -(-len(vals) // per)
    flat = np.zeros(T * per, np.float32)    # (the padding is zeros)
    flat[:len(vals)] = vals
    x = np.empty((T, d), np.float32)
    x[:, :per] = flat.reshape(T, per)
    x[:, -1] = amax
    from lora_inputs import bf16_round
    assert np.array_equal(bf16_round(x).view(np.uint16).astype(np.uint32) << 16, x.view(np.uint32))
    xd = bf16_dev(bf16_round(x))
    q = torch.empty(T, d, dtype=torch.uint8, device=DEV)
    s = torch.empty(T, dtype=torch.float32, device=DEV)
    agm.quantize_e4m3(xd, q, s)
    torch.cuda.synchronize()
    codes, sx = oracle.act_quant_e4m3(x)
    assert np.array_equal(s.cpu().numpy(), sx)
    got = q.cpu().numpy()
    bad = np.argwhere(got != codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first (x, got, want): " + ", ".join(
        f"({x[i, k]!r}, {got[i, k]:#04x}, {codes[i, k]:#04x})" for i, k in bad[:12])


def test_quantize_e4m3_bit_exact():
    g = np.random.default_rng(0)
    from lora_inputs import bf16_round
    x = bf16_round((g.standard_normal((37, 1040)) * np.exp(g.uniform(-6, 6, (37, 1)))).astype(np.float32))
    x[5] = 0
    xd = bf16_dev(x)
    q = torch.empty(37, 1040, dtype=torch.uint8, device=DEV)
    s = torch.empty(37, dtype=torch.float32, device=DEV)
    agm.quantize_e4m3(xd, q, s)
    torch.cuda.synchronize()
    codes, sx = oracle.act_quant_e4m3(x)
    assert np.array_equal(s.cpu().numpy(), sx)
    assert np.array_equal(q.cpu().numpy(), codes)


def test_order_and_determinism():
    w = make_workload("decode_bgmv", **SMALL["decode_bgmv"])
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg0, s0 = segments(w, p.n_slots, 0)
    seg1, s1 = segments(w, p.n_slots, 1)
    ya = _fused(dp, seg0, s0, w)
    yb = _fused(dp, seg0, s0, w)
    yc = _fused(dp, seg1, s1, w)
    assert np.array_equal(ya, yb)                    # bitwise reproducible
    assert rel_l2(yc, ya) <= 1e-3                    # segment order does not matter


# ---- base and adapter work on disjoint CU sets --------------------------------------

@pytest.mark.parametrize("split", [("spread", 128), ("block", 64)])
def test_concurrent_cu_masked_streams(split):
    """The unfused design on CU-masked streams: the base product alone on one
    stream, builder -> shrink -> (after the base product) expand on another;
    y matches the oracle."""
    layout, k = split
    n = agm.cu_count()
    if layout == "spread":
        base_cus = [c for c in range(n) if c % 32 < k // max(1, n // 32)]
    else:
        base_cus = list(range(k))
    lora_cus = [c for c in range(n) if c not in set(base_cus)]
    sA, sB = agm.CUMaskedStream(base_cus, n), agm.CUMaskedStream(lora_cus, n)
    assert sA.cus == base_cus and sB.cus == lora_cus
    w = make_workload("decode_bgmv", **SMALL["decode_bgmv"])
    p = w.projections[0]
    dp = DevProjection(w, p)
    ids = torch.from_numpy(w.ids).to(DEV)
    act = torch.from_numpy(w.active).to(DEV)
    seg = torch.empty(agm.segment_words(w.T), dtype=torch.int32, device=DEV)
    v = torch.empty(w.T, p.r_cap, device=DEV)
    y = torch.full((w.T, p.d_out), float("nan"), device=DEV).to(torch.bfloat16)
    main = torch.cuda.current_stream()
    e0, e_base, e_lora = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()
    e0.record(main)
    sA.stream.wait_event(e0)
    sB.stream.wait_event(e0)
    agm.fused_linear(dp.base, None, None, dp.x, None, y, stream=sA.stream)
    e_base.record(sA.stream)
    agm.build_segments_dev(ids, act, p.n_slots, seg, stream=sB.stream)
    agm.shrink(dp.pool, seg, w.T, None, dp.x, v, launch=agm.LAUNCH_PERSISTENT, stream=sB.stream)
    sB.stream.wait_event(e_base)
    agm.expand(dp.pool, seg, w.T, None, v, y, launch=agm.LAUNCH_PERSISTENT, stream=sB.stream)
    e_lora.record(sB.stream)
    main.wait_event(e_lora)
    torch.cuda.synchronize()
    sA.close()
    sB.close()
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    got = to_f64(y)
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) <= TOL["bf16"] and row_rel_l2(got, ref) <= TOL["bf16"]


# ---- edge cases ------------------------------------------------------------------

def _custom(T, d_in, d_out, N, r_cap, ranks, ids, active=None, dtype="bf16", seed=0):
    """A workload built from explicit ids/ranks with the generator's draws."""
    from lora_inputs import Projection, Workload
    key = (seed, 99)
    p = Projection("p", d_in, d_out, N, r_cap, np.asarray(ranks, np.int32),
                   np.linspace(0.5, 2.0, N).astype(np.float32), 0.05, 0.05, 0.05, dtype, dtype, key)
    act = np.ones(T, np.uint8) if active is None else np.asarray(active, np.uint8)
    return Workload("custom", seed, T, [p], np.asarray(ids, np.int32), act, dtype)


@pytest.mark.parametrize("ranks,r_cap", [([1, 2, 4, 12], 16), ([16, 31, 32, 7], 32), ([64, 1, 33, 64], 64),
                                         ([128, 100, 5, 1], 128)])
def test_rank_edge_cases(ranks, r_cap):
    g = np.random.default_rng(len(ranks) + r_cap)
    T = 77
    ids = g.integers(-1, 4, T)
    w = _custom(T, 264, 200, 4, r_cap, ranks, ids)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, 4)
    y = _fused(dp, seg, s, w)
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    assert rel_l2(y, ref) <= TOL["bf16"] and row_rel_l2(y, ref) <= TOL["bf16"]
    v = torch.zeros(T, r_cap, device=DEV)
    agm.shrink(dp.pool, seg, T, s, dp.x, v)
    yz = torch.zeros(T, p.d_out, dtype=torch.bfloat16, device=DEV)
    agm.expand(dp.pool, seg, T, s, v, yz)
    torch.cuda.synchronize()
    d_ref = oracle.lora_delta(*dp.oracle_args(w))
    assert rel_l2(to_f64(yz), d_ref) <= TOL["bf16"]


@pytest.mark.parametrize("T,d_out,ranks,r_cap", [(1500, 2056, [5, 17, 33, 64], 64),      # 256 x 128 tiles
                                                  (4100, 8200, [1, 64, 9, 40], 64),       # 256 x 256 tiles
                                                  (1100, 4104, [128, 3, 72, 100], 128)])  # persistent 128 x 128
def test_packed_adapter_steps_ranks(T, d_out, ranks, r_cap):
    """Prefill-shaped batches (long groups over few slots) run the adapter
    term as pipelined steps from packed per-tile records: ranks that are not
    multiples of 8 leave part-filled chunks whose pool padding (NaN here) must
    never enter the product; requests of random lengths put 1 to 3 groups in
    a tile, and some rows carry no adapter."""
    g = np.random.default_rng(T + r_cap)
    lens = g.integers(40, 400, 64)
    ids = np.repeat(g.integers(-1, 4, 64), lens)[:T]
    ids = np.concatenate([ids, np.full(T - len(ids), 2)]).astype(np.int32)
    w = _custom(T, 512, d_out, 4, r_cap, ranks, ids)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, 4)
    y = _fused(dp, seg, s, w)
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    assert np.isfinite(y).all()
    assert rel_l2(y, ref) <= TOL["bf16"] and row_rel_l2(y, ref) <= TOL["bf16"]
    d = _fused(dp, seg, s, w, zero_base=True)
    d_ref = oracle.lora_delta(*dp.oracle_args(w))
    live = oracle.live_rows(w.ids, w.active)
    assert rel_l2(d, d_ref) <= TOL["bf16"] and row_rel_l2(d[live], d_ref[live]) <= TOL["bf16"]


@pytest.mark.parametrize("r_cap,ranks", [(16, [16, 9, 8, 1, 5, 12]), (8, [8, 1, 3, 7, 2, 5])])
def test_decode_tile_epilogue_ranks(r_cap, ranks):
    """64 x 64 bf16 tiles with rank capacity <= 16 take the per-output adapter
    epilogue: ranks below the capacity (a partly used second 8-rank chunk,
    rank 1, capacity 8 with no second chunk), NaN rank padding, a ragged last
    column tile, rows with id -1 and released rows."""
    g = np.random.default_rng(r_cap)
    T, N = 150, len(ranks)
    ids = g.integers(-1, N, T)
    act = (g.random(T) > 0.2).astype(np.uint8)
    w = _custom(T, 512, 328, N, r_cap, ranks, ids, act)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, N)
    y = _fused(dp, seg, s, w)
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    assert np.isfinite(y).all()
    assert rel_l2(y, ref) <= TOL["bf16"] and row_rel_l2(y, ref) <= TOL["bf16"]
    d = _fused(dp, seg, s, w, zero_base=True)
    d_ref = oracle.lora_delta(*dp.oracle_args(w))
    live = oracle.live_rows(w.ids, w.active)
    assert rel_l2(d, d_ref) <= TOL["bf16"] and row_rel_l2(d[live], d_ref[live]) <= TOL["bf16"]
    yb = _fused(dp, seg, s, w, with_pool=False)
    assert np.array_equal(y[~live], yb[~live])


@pytest.mark.parametrize("T,r_cap,ranks", [(2048, 64, [64, 1, 33, 17]), (4096, 64, [64, 40, 3, 16]),
                                           (4096, 128, [128, 100, 5, 33])])
def test_shrink_several_rank_blocks_per_item(T, r_cap, ranks):
    """Long batches over few adapters (mostly full 16-row tiles): each shrink
    item takes 2, 4 or 8 rank blocks that share the tile's x rows.  v matches
    the oracle on every rank (padding is NaN in the pool) and is bitwise the
    same in every launch mode."""
    g = np.random.default_rng(T + r_cap)
    ids = g.integers(-1, 4, T)
    w = _custom(T, 264, 200, 4, r_cap, ranks, ids)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, 4)
    segd = split_seg(seg, T)
    n = s.n_active
    vr = _v_ref(dp, w, segd)
    mask = np.arange(r_cap)[None, :] < p.slot_rank[w.ids[segd["perm"][:n]]][:, None]
    outs = []
    for mode in (agm.LAUNCH_EXACT, agm.LAUNCH_PERSISTENT, agm.LAUNCH_BUCKETED, agm.LAUNCH_FULL_BATCH):
        v = torch.full((T, r_cap), float("nan"), device=DEV)
        agm.shrink(dp.pool, seg, T, s, dp.x, v, launch=mode)
        torch.cuda.synchronize()
        vg = v.cpu().numpy().astype(np.float64)[:n]
        assert np.isfinite(vg[mask]).all(), mode
        got = np.where(mask, vg, 0.0)
        assert rel_l2(got, vr) <= TOL["fp32"] and row_rel_l2(got, vr) <= TOL["fp32"], mode
        outs.append(vg[mask])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("case", ["empty", "all_none", "all_inactive", "one_row", "one_adapter_big"])
def test_degenerate_batches(case):
    T = {"empty": 0, "one_row": 1}.get(case, 130)
    ids = np.zeros(T, np.int32)
    act = np.ones(T, np.uint8)
    if case == "all_none":
        ids[:] = -1
    if case == "all_inactive":
        act[:] = 0
    w = _custom(T, 136, 72, 3, 16, [16, 8, 4], ids, act)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, 3)
    y = _fused(dp, seg, s, w) if T else None
    if T:
        ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
        assert rel_l2(y, ref) <= TOL["bf16"]
    for mode in (agm.LAUNCH_EXACT, agm.LAUNCH_PERSISTENT, agm.LAUNCH_BUCKETED, agm.LAUNCH_FULL_BATCH):
        v = torch.zeros(max(T, 1), 16, device=DEV)
        yz = torch.zeros(max(T, 1), 72, dtype=torch.bfloat16, device=DEV)
        agm.shrink(dp.pool, seg, T, s, dp.x, v, launch=mode)
        agm.expand(dp.pool, seg, T, s, v, yz, launch=mode)
        torch.cuda.synchronize()
        if T:
            d_ref = oracle.lora_delta(*dp.oracle_args(w))
            assert rel_l2(to_f64(yz)[:T], d_ref) <= TOL["bf16"]
        else:
            assert torch.count_nonzero(yz.float()) == 0


def test_zero_B_gives_base_exactly():
    g = np.random.default_rng(3)
    T = 90
    w = _custom(T, 256, 136, 5, 16, [16] * 5, g.integers(-1, 5, T))
    p = w.projections[0]
    dp = DevProjection(w, p)
    dp.B.zero_()
    seg, s = segments(w, 5)
    y = _fused(dp, seg, s, w)
    yb = _fused(dp, seg, s, w, with_pool=False)
    assert np.array_equal(y, yb)


def _random_case(i):
    """Seeded random shape: base type, ragged sizes (16-byte aligned rows),
    rank capacity and per-slot ranks, Zipf or uniform ids with released and
    absent rows."""
    g = np.random.default_rng(7000 + i)
    kind = ["bf16", "fp8", "w8a8", "fp32"][i % 4]
    dtype = "fp32" if kind == "fp32" else "bf16"
    T = int(g.choice([1, 3, 64, 255, 256, 257, 700]) if i < 8 else g.integers(1, 900))
    d_in = int(16 * g.integers(1, 80))
    d_out = int(8 * g.integers(1, 300))
    N = int(g.integers(1, 300))
    r_cap = int(g.choice([8, 16, 32, 64, 128]))
    ranks = np.where(g.uniform(size=N) < 0.3, r_cap, g.integers(1, r_cap + 1, N))
    if g.uniform() < 0.5:
        ids = np.minimum(g.zipf(1.1, T) - 1, N - 1)
    else:
        ids = g.integers(0, N, T)
    ids = np.where(g.uniform(size=T) < 0.15, -1, ids)
    active = (g.uniform(size=T) > 0.1).astype(np.uint8)
    from lora_inputs import Projection, Workload
    base = "fp8" if kind in ("fp8", "w8a8") else dtype
    proj = Projection("p", d_in, d_out, N, r_cap, ranks.astype(np.int32),
                      g.uniform(0.25, 2.0, N).astype(np.float32), 0.05, 0.05, 0.05, base, dtype, (i, 77))
    w = Workload("random", i, T, [proj], ids.astype(np.int32), active, dtype)
    return kind, w


@pytest.mark.parametrize("i", range(48))
def test_random_shapes_fused_parity(i):
    """A seeded sweep of shapes no other case pins down: every base type,
    T from one row up, ragged d_in / d_out, 1-299 slots, rank capacities 8-128
    with mixed ranks, Zipf or uniform ids with absent and released rows; y
    against the fp64 oracle globally and per row, and the oracle's W8A8
    definition for the quantised mode."""
    kind, w = _random_case(i)
    p = w.projections[0]
    print(f"case {i}: {kind} T={w.T} {p.d_in}->{p.d_out} N={p.n_slots} r_cap={p.r_cap}", flush=True)
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    flags = agm.FLAG_ACT_QUANT_E4M3 if kind == "w8a8" else 0
    y = _fused(dp, seg, s, w, flags=flags)
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    tol = _tol(p)
    assert rel_l2(y, ref) <= tol
    if kind != "w8a8":
        assert row_rel_l2(y, ref) <= tol
    else:
        # per row, quantising a short row of x to e4m3 alone can move it past
        # 3e-2 from the unquantised product; against the W8A8 definition (the
        # same codes and scales) only accumulation and bf16 rounding remain
        ref8 = oracle.linear_w8a8(dp.x_host, dp.w0_host[0], dp.w0_host[1], *dp.oracle_args(w)[1:])
        assert rel_l2(y, ref8) <= TOL["bf16"] and row_rel_l2(y, ref8) <= TOL["bf16"]


@pytest.mark.parametrize("i", range(32))
def test_random_shapes_segments_shrink_expand(i):
    """The same seeded sweep through the other calls: the device builder's
    segment buffer bit-exact against the oracle's grouping (both orders), v of
    lora_shrink, and the adapter term of lora_expand on y = 0 (rows not live
    bitwise untouched)."""
    kind, w = _random_case(i)
    p = w.projections[0]
    print(f"case {i}: {kind} T={w.T} {p.d_in}->{p.d_out} N={p.n_slots} r_cap={p.r_cap}", flush=True)
    for order in (0, 1):
        _check_layout(w.ids, w.active, p.n_slots, order)
    if kind in ("fp8", "w8a8"):
        return                                   # same pools as bf16: nothing new for shrink / expand
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots, device_build=True)
    segd = split_seg(seg, w.T)
    v = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
    agm.shrink(dp.pool, seg, w.T, None, dp.x, v, launch=agm.LAUNCH_PERSISTENT)
    y = torch.zeros(w.T, p.d_out, dtype=dp.ydtype, device=DEV)
    agm.expand(dp.pool, seg, w.T, None, v, y, launch=agm.LAUNCH_PERSISTENT)
    torch.cuda.synchronize()
    n = s.n_active
    vg = v.cpu().numpy().astype(np.float64)[:n]
    vr = _v_ref(dp, w, segd)
    mask = np.arange(p.r_cap)[None, :] < p.slot_rank[w.ids[segd["perm"][:n]]][:, None]
    if n:
        assert rel_l2(np.where(mask, vg, 0), vr) <= TOL["fp32"]
    d_ref = oracle.lora_delta(*dp.oracle_args(w))
    d_got = to_f64(y)
    live = oracle.live_rows(w.ids, w.active)
    tol = _tol(p)
    if live.any():
        assert rel_l2(d_got, d_ref) <= tol
        assert row_rel_magnitude(d_got[live], d_ref[live], _delta_magnitude(dp, w)[live]) <= tol
    assert np.all(d_got[~live] == 0)


def _random_decode(i, kinds):
    """Seeded small-batch case (T <= 256, <= 1024 slots) for the one-launch
    build + shrink and the in-launch shrink."""
    g = np.random.default_rng(9100 + i)
    kind = kinds[i % len(kinds)]
    dtype = "fp32" if kind == "fp32" else "bf16"
    T = int(g.integers(1, 257))
    d_in = int(64 * g.integers(1, 40))
    d_out = int(8 * g.integers(1, 400))
    N = int(g.integers(1, 1025))
    r_cap = int(g.choice([8, 16, 32, 64]))
    ranks = np.where(g.uniform(size=N) < 0.3, r_cap, g.integers(1, r_cap + 1, N)).astype(np.int32)
    ids = np.minimum(g.zipf(1.1, T) - 1, N - 1) if g.uniform() < 0.5 else g.integers(0, N, T)
    ids = np.where(g.uniform(size=T) < 0.2, -1, ids).astype(np.int32)
    active = (g.uniform(size=T) > 0.25).astype(np.uint8)
    from lora_inputs import Projection, Workload
    base = "fp8" if kind == "fp8" else dtype
    proj = Projection("p", d_in, d_out, N, r_cap, ranks, g.uniform(0.25, 2.0, N).astype(np.float32),
                      0.05, 0.05, 0.05, base, dtype, (i, 99))
    return kind, Workload("random_decode", i, T, [proj], ids, active, dtype)


@pytest.mark.parametrize("i", range(16))
def test_random_build_shrink(i):
    """Seeded small batches through the one-launch build + shrink: its segment
    buffer equals the device builder's bit for bit, and its v the oracle's."""
    kind, w = _random_decode(i, ["bf16", "fp32"])
    p = w.projections[0]
    print(f"case {i}: {kind} T={w.T} d_in={p.d_in} N={p.n_slots} r_cap={p.r_cap}", flush=True)
    dp = DevProjection(w, p)
    ids = torch.from_numpy(w.ids).to(DEV)
    act = torch.from_numpy(w.active).to(DEV)
    order = i % 2
    seg_ref = torch.full((agm.segment_words(w.T),), -7, dtype=torch.int32, device=DEV)
    agm.build_segments_dev(ids, act, p.n_slots, seg_ref, order)
    seg = torch.full((agm.segment_words(w.T),), -9, dtype=torch.int32, device=DEV)
    v = torch.full((w.T, p.r_cap), float("nan"), device=DEV)
    agm.build_shrink_dev(ids, act, dp.pool, seg, dp.x, v, order=order)
    torch.cuda.synchronize()
    d_ref, d = split_seg(seg_ref, w.T), split_seg(seg, w.T)
    words = d_ref["sum"]
    assert int(words[7]) == 0 and np.array_equal(d["sum"][:8], words[:8])
    for a, b in zip(_seg_meaningful(d, words), _seg_meaningful(d_ref, words)):
        assert np.array_equal(a, b)
    n = int(words[0])
    if n:
        mask = np.arange(p.r_cap)[None, :] < p.slot_rank[w.ids[d_ref["perm"][:n]]][:, None]
        vg = v.cpu().numpy()[:n].astype(np.float64)
        assert rel_l2(np.where(mask, vg, 0.0), _v_ref(dp, w, d_ref)) <= TOL["fp32"]


@pytest.mark.parametrize("i", range(12))
def test_random_shrink_in_launch(i):
    """Seeded small batches through the fused call that computes its shrink in
    the same launch (bf16 and widened fp8): v and y against the oracle."""
    kind, w = _random_decode(i, ["bf16", "fp8"])
    p = w.projections[0]
    print(f"case {i}: {kind} T={w.T} {p.d_in}->{p.d_out} N={p.n_slots} r_cap={p.r_cap}", flush=True)
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    y, v = _fused_in_launch(dp, seg, w)
    segd = split_seg(seg, w.T)
    n = s.n_active
    if n:
        rk = p.slot_rank[segd["seg_adapter"][segd["pos_seg"][:n]]]
        mask = np.arange(p.r_cap)[None, :] < rk[:, None]
        assert rel_l2(v[:n][mask], _v_ref(dp, w, segd)[mask]) <= TOL["fp32"]
    ref = oracle.linear(dp.x_host, dp.w0_host, *dp.oracle_args(w)[1:])
    tol = _tol(p)
    assert np.isfinite(y).all()
    assert rel_l2(y, ref) <= tol and row_rel_l2(y, ref) <= tol


@pytest.mark.parametrize("T,d_out", [(512, 9216),    # persistent 128 x 128 W8A16 tiles
                                     (256, 264),     # 64 x 64 W8A16 tiles
                                     (528, 1000)])   # d_in % 64 != 0: the general kernel
def test_every_e4m3_code_widens_exactly(T, d_out):
    """Widened fp8 (W8A16) with x the identity (T = d_in): y[i, n] is the
    decoded code W0[n, i] times its channel scale, a power of two, so every
    finite e4m3 code (all 254, subnormals and signed zeros included) must come
    out as its exact value in bf16."""
    d_in = T
    n = np.arange(d_out)[:, None]
    k = np.arange(d_in)[None, :]
    codes = ((n * 37 + k) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00                     # the two NaN codes
    assert len(np.unique(codes[:, :256])) == 254
    scale = np.ldexp(1.0, (np.arange(d_out) % 5) - 2).astype(np.float32)
    expect = (oracle.decode_e4m3(codes) * scale.astype(np.float64)[:, None]).T   # [d_in = T, d_out]
    W = torch.from_numpy(codes).to(DEV)
    ws = torch.from_numpy(scale).to(DEV)
    x = torch.eye(T, dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device=DEV)
    wsp = agm.fused_workspace(T, d_in, d_out, agm.FP8_E4M3, 0, device=DEV)
    agm.fused_linear(agm.base_desc(W, ws), None, None, x, None, y, workspace=wsp)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("case", ["pool_over_2GiB", "over_65535_slots"])
def test_large_pools_take_the_general_kernel(case):
    """Pools the pipelined kernel cannot address (B over 2 GiB for its 32-bit
    buffer offsets; more than 65535 slots for the 16-bit slot field of its
    chunk records) go to the general kernel; rows whose adapter sits past
    those limits must still get the oracle's result.  Only the touched slots
    hold values (the rest stay zero); the oracle sees those slots alone."""
    if case == "pool_over_2GiB":
        kw = dict(T=96, d_in=256, d_out=4096, n_slots=2100, r=128)      # B: 2.2 GB
        far = [2099, 2050, 1200]
    else:
        kw = dict(T=64, d_in=128, d_out=264, n_slots=70000, r=8)
        far = [69999, 65536, 40000]
    w = make_workload("decode_bgmv", **kw)
    p = w.projections[0]
    ids = w.ids.copy()
    live_rows = np.flatnonzero(ids >= 0)
    for k, a in enumerate(far):                  # a few live rows on far slots
        ids[live_rows[3 * k:3 * k + 3]] = a
    w.ids = ids
    touched = w.touched_slots()
    assert max(touched) == far[0]
    A = torch.zeros((p.n_slots, p.r_cap, p.d_in), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((p.n_slots, p.d_out, p.r_cap), dtype=torch.bfloat16, device=DEV)
    A_c = np.zeros((len(touched), p.r_cap, p.d_in), np.uint16)
    B_c = np.zeros((len(touched), p.d_out, p.r_cap), np.uint16)
    for k, a in enumerate(touched):
        A_c[k], B_c[k] = p.slot(a)
        A[a] = bf16_dev(A_c[k])
        B[a] = bf16_dev(B_c[k])
    if case == "pool_over_2GiB":
        assert B.numel() * 2 > 0x7FFFFFFF
    rank = torch.from_numpy(p.slot_rank.astype(np.int32)).to(DEV)
    scale = torch.from_numpy(p.slot_scale.astype(np.float32)).to(DEV)
    pool = agm.pool_desc(A, B, rank, scale)
    w0 = p.w0()
    base = agm.base_desc(bf16_dev(w0), None)
    xh = w.x(p)
    x = bf16_dev(xh)
    seg, s = segments(w, p.n_slots)
    v = torch.zeros(w.T, p.r_cap, device=DEV)
    agm.shrink(pool, seg, w.T, s, x, v)
    y = torch.full((w.T, p.d_out), float("nan"), device=DEV).to(torch.bfloat16)
    ws = agm.fused_workspace(w.T, p.d_in, p.d_out, agm.BF16, 0, device=DEV)
    agm.fused_linear(base, pool, seg, x, v, y, workspace=ws)
    torch.cuda.synchronize()
    remap = {a: k for k, a in enumerate(touched)}
    ids_c = np.array([remap.get(int(a), -1) if a >= 0 else -1 for a in ids], np.int32)
    ref = oracle.linear(xh, w0, ids_c, w.active, A_c, B_c, p.slot_rank[touched], p.slot_scale[touched])
    got = to_f64(y)
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) <= TOL["bf16"] and row_rel_l2(got, ref) <= TOL["bf16"], case
    far_rows = np.isin(ids, far)
    assert row_rel_l2(got[far_rows], ref[far_rows]) <= TOL["bf16"], case
