"""HIP graph capture of the device path: the segment build, the shrink and the
fused linear are stream-ordered, allocate nothing and read nothing back to the
host, so one capture of a step replays it.  Every replay (outputs poisoned
with NaN first, unrelated eager work and a synchronisation between replays)
must equal the eager run bit for bit: the kernels are deterministic and take
the same launch shapes in both.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import adapter_gemm_amd as agm
from lora_inputs import make_workload
from gpu_helpers import DEV, DevProjection, split_seg

REPLAYS = 3


def _defined(seg, T):
    """The words of a segment buffer that the builder defines: summary, the
    permutation and row segments, S + 1 starts, S adapters, the listed tiles
    (the rest of each array is left as it was)."""
    d = split_seg(seg, T)
    S, n_small, n_large = int(d["sum"][1]), int(d["sum"][4]), int(d["sum"][5])
    return dict(sum=d["sum"][:8], perm=d["perm"], pos_seg=d["pos_seg"], seg_start=d["seg_start"][:S + 1],
                seg_adapter=d["seg_adapter"][:S], tiles_small=d["tiles_small"][:n_small],
                tiles_large=d["tiles_large"][:n_large])


def _step(w, dp, ids, act, seg, v, y, ws):
    """One pass of the path for the workload's first projection, as bench.py runs it."""
    if w.T <= 256 and dp.p.n_slots <= 1024:
        agm.build_shrink_dev(ids, act, dp.pool, seg, dp.x, v)
    else:
        agm.build_segments_dev(ids, act, dp.p.n_slots, seg)
        agm.shrink(dp.pool, seg, w.T, None, dp.x, v, launch=agm.LAUNCH_PERSISTENT)
    agm.fused_linear(dp.base, dp.pool, seg, dp.x, v, y, workspace=ws)


@pytest.mark.parametrize("name", ["decode_bgmv", "fp8_fused", "tiny_sgmv"])
def test_graph_replay_equals_eager(name):
    w = make_workload(name)
    p = w.projections[0]
    print(f"[graph] {name}: T={w.T}, {p.name} {p.d_in}->{p.d_out}", flush=True)
    dp = DevProjection(w, p, nan_fill=False)
    ids = torch.from_numpy(w.ids.astype(np.int32)).to(DEV)
    act = torch.from_numpy(w.active.astype(np.uint8)).to(DEV)
    seg = torch.empty(agm.segment_words(w.T), dtype=torch.int32, device=DEV)
    v = torch.empty((w.T, p.r_cap), dtype=torch.float32, device=DEV)
    y = torch.empty((w.T, p.d_out), dtype=dp.ydtype, device=DEV)
    bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}[p.base_dtype]
    ws = agm.fused_workspace(w.T, p.d_in, p.d_out, bt, 0, device=DEV)

    # eager reference (also the warm-up: first-call set-up happens outside the capture)
    _step(w, dp, ids, act, seg, v, y, ws)
    torch.cuda.synchronize()
    seg_ref, v_ref, y_ref = _defined(seg, w.T), v.clone(), y.clone()
    # v is defined for the live rows [0, n_act) and the directions below each row's rank
    n_act = int(seg_ref["sum"][0])
    rank = p.slot_rank[seg_ref["seg_adapter"][seg_ref["pos_seg"][:n_act]]]
    vmask = torch.from_numpy(np.arange(p.r_cap)[None, :] < rank[:, None]).to(DEV)
    v_ref = v_ref[:n_act][vmask]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, dp, ids, act, seg, v, y, ws)
    torch.cuda.synchronize()

    other = torch.randn(1024, 1024, device=DEV)
    for rep in range(REPLAYS):
        seg.fill_(-7)
        v.fill_(float("nan"))
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _defined(seg, w.T)
        for k, ref in seg_ref.items():
            assert np.array_equal(got[k], ref), (name, rep, k)
        assert torch.equal(v[:n_act][vmask], v_ref), (name, rep, "v")
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                           y_ref.view(torch.int16) if y.dtype == torch.bfloat16 else y_ref.view(torch.int32)), \
            (name, rep, "y")
        # unrelated eager work on the same device between replays
        other = torch.tanh(other @ other.T * 1e-3)
        torch.cuda.synchronize()
        print(f"[graph] {name}: replay {rep} bit-identical", flush=True)
    del g
    torch.cuda.empty_cache()


def test_graph_replay_sliced_launch():
    """q / k / v of the Llama layer set as one sliced launch on one input,
    after the device build and one shrink per projection."""
    w = make_workload("llama_layer")
    names = [p.name for p in w.projections]
    dps = [DevProjection(w, w.projections[names.index(n)], nan_fill=False) for n in ("q_proj", "k_proj", "v_proj")]
    print(f"[graph] llama_layer q/k/v: T={w.T}", flush=True)
    x = dps[0].x
    ids = torch.from_numpy(w.ids.astype(np.int32)).to(DEV)
    act = torch.from_numpy(w.active.astype(np.uint8)).to(DEV)
    seg = torch.empty(agm.segment_words(w.T), dtype=torch.int32, device=DEV)
    vs = [torch.empty((w.T, dp.p.r_cap), dtype=torch.float32, device=DEV) for dp in dps]
    ys = [torch.empty((w.T, dp.p.d_out), dtype=dp.ydtype, device=DEV) for dp in dps]
    ws = agm.fused_slices_workspace(w.T, dps[0].p.d_in, [dp.p.d_out for dp in dps], agm.BF16, device=DEV)

    def step():
        agm.build_segments_dev(ids, act, dps[0].p.n_slots, seg)
        for dp, v in zip(dps, vs):
            agm.shrink(dp.pool, seg, w.T, None, x, v, launch=agm.LAUNCH_PERSISTENT)
        agm.fused_linear_slices([dp.base for dp in dps], [dp.pool for dp in dps], seg, x, vs, ys, workspace=ws)

    step()
    torch.cuda.synchronize()
    y_ref = [y.view(torch.int16).clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.randn(1024, 1024, device=DEV)
    for rep in range(REPLAYS):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for dp, y, ref in zip(dps, ys, y_ref):
            assert torch.equal(y.view(torch.int16), ref), (dp.p.name, rep)
        other = torch.tanh(other @ other.T * 1e-3)
        torch.cuda.synchronize()
        print(f"[graph] llama_layer q/k/v: replay {rep} bit-identical", flush=True)
    del g
    torch.cuda.empty_cache()
