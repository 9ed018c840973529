"""The allocation-free fused call (lora_fused_linear_noalloc) against
lora_fused_linear with a caller workspace, through the C-ABI: the same kernels
and schedule, so the outputs must be equal bit for bit.  Two calls in a row on
one GPU share the static scratch; the second takes a smaller batch.  Shapes
chosen so that the scratch is really used: split-k partial tiles and their
counters (few output tiles), W8A8 activation codes, persistent claim
counters."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import adapter_gemm_amd as agm
from lora_inputs import make_workload
from gpu_helpers import DEV, DevProjection, segments

# (workload, sizes of the first call, T of the second, flags)
CASES = {
    "split_k": ("decode_bgmv", dict(T=100, d_in=1024, d_out=264, n_slots=40), 37, 0),
    "w8a8": ("fp8_fused", dict(T=200, d_in=1024, d_out=904, n_slots=32, r=64), 90, agm.FLAG_ACT_QUANT_E4M3),
    "persistent": ("decode_bgmv", dict(T=600, d_in=1024, d_out=3000, n_slots=40), 520, 0),
}


def _bt(p):
    return {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}[p.base_dtype]


def _run(name, sizes, flags):
    w = make_workload(name, **sizes)
    p = w.projections[0]
    dp = DevProjection(w, p)
    seg, s = segments(w, p.n_slots)
    v = torch.zeros(w.T, p.r_cap, device=DEV)
    agm.shrink(dp.pool, seg, w.T, s, dp.x, v)
    need = agm.lib().lora_fused_workspace_bytes_rcap(w.T, p.d_in, p.d_out, _bt(p), flags, p.r_cap)
    assert 0 < need <= agm.NOALLOC_SCRATCH_BYTES, need    # the scratch is really used
    ws = agm.fused_workspace(w.T, p.d_in, p.d_out, _bt(p), flags, device=DEV)
    y_ref = torch.full((w.T, p.d_out), float("nan"), dtype=dp.ydtype, device=DEV)
    y_new = torch.full((w.T, p.d_out), float("nan"), dtype=dp.ydtype, device=DEV)
    agm.fused_linear(dp.base, dp.pool, seg, dp.x, v, y_ref, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    print(f"case {name} {sizes} flags={flags}: noalloc call", flush=True)
    agm.fused_linear_noalloc(dp.base, dp.pool, seg, dp.x, v, y_new, flags=flags)
    torch.cuda.synchronize()
    return y_ref, y_new


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_equals_workspace_call_twice(case):
    name, sizes, t2, flags = CASES[case]
    for T in (sizes["T"], t2):                     # two calls in a row, the second smaller
        y_ref, y_new = _run(name, dict(sizes, T=T), flags)
        assert not torch.isnan(y_ref.float()).any()
        assert torch.equal(y_ref.view(torch.int16), y_new.view(torch.int16)), (case, T)


def test_noalloc_rejects_calls_beyond_the_scratch():
    # W8A8 codes of 8192 rows x 8192 need 64 MiB: refused before any work
    fake = 1 << 20
    base = agm.BaseDesc(fake, fake, agm.FP8_E4M3, 8192)
    st = agm.lib().lora_fused_linear_noalloc(ctypes.byref(base), None, None, 8192, 2 * fake, 8192, None, 0, 3 * fake, 8192,
                                             8192, 8192, agm.FLAG_ACT_QUANT_E4M3, None)
    assert st == agm.LORA_E_SIZE
    assert b"scratch" in agm.lib().lora_last_error()
