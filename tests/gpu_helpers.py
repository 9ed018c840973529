"""Shared helpers of the GPU parity tests: move a seeded workload to the
device, run the library's calls on it, and compare with the fp64 oracle.

Inputs come from lora_inputs only; expected values come from oracle only.
"""
from __future__ import annotations

import numpy as np
import torch

import adapter_gemm_amd as agm
import oracle
from lora_inputs import Projection, Workload

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.cpu().numpy().astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def row_rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if len(num) else 0.0


def row_rel_magnitude(got: np.ndarray, ref: np.ndarray, mag: np.ndarray) -> float:
    """Largest per-row error relative to the row's magnitude: `mag` holds the
    same sums taken over absolute values, the scale that fp32 rounding of the
    row's sums is relative to.  A row whose sums cancel to a small result is
    then held to the rounding its terms allow, not to its own size (mag is
    never smaller than the result)."""
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(mag, axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if len(num) else 0.0


class DevProjection:
    """One projection of a workload on the device.

    Pool slots that the batch does not touch, and rank padding of touched
    slots, are filled with NaN (bf16 / fp32): any read of them would poison
    the outputs."""

    def __init__(self, w: Workload, p: Projection, nan_fill: bool = True, all_slots: bool = False):
        self.p = p
        self.touched = list(range(p.n_slots)) if all_slots else w.touched_slots()
        A, B = p.pool(self.touched)
        if nan_fill:
            nan = np.float32(np.nan) if p.data_dtype == "fp32" else np.uint16(0x7FC0)
            untouched = np.setdiff1d(np.arange(p.n_slots), self.touched)
            A[untouched] = nan
            B[untouched] = nan
            for a in self.touched:
                r = int(p.slot_rank[a])
                A[a, r:] = nan
                B[a, :, r:] = nan
        self.A_host, self.B_host = A, B        # stored values (NaN where never read)
        mk = bf16_dev if p.data_dtype == "bf16" else f32_dev
        self.A = mk(A)
        self.B = mk(B)
        self.slot_rank = torch.from_numpy(p.slot_rank.astype(np.int32)).to(DEV)
        self.slot_scale = torch.from_numpy(p.slot_scale.astype(np.float32)).to(DEV)
        self.pool = agm.pool_desc(self.A, self.B, self.slot_rank, self.slot_scale)
        w0 = p.w0()
        self.w0_host = w0
        if p.base_dtype == "fp8":
            self.W = torch.from_numpy(w0[0]).to(DEV)
            self.w_scale = torch.from_numpy(w0[1]).to(DEV)
        elif p.base_dtype == "bf16":
            self.W = bf16_dev(w0)
            self.w_scale = None
        else:
            self.W = f32_dev(w0)
            self.w_scale = None
        self.base = agm.base_desc(self.W, self.w_scale)
        self.x_host = w.x(p)
        self.x = bf16_dev(self.x_host) if p.data_dtype == "bf16" else f32_dev(self.x_host)
        self.ydtype = torch.bfloat16 if p.data_dtype == "bf16" else torch.float32

    # oracle views (pools with NaN only where never read)
    def oracle_args(self, w: Workload):
        return (self.x_host, w.ids, w.active, self.A_host, self.B_host, self.p.slot_rank, self.p.slot_scale)


def segments(w: Workload, n_slots: int, order: int = 0, device_build: bool = False):
    """Segment buffer on the device + host summary (host builder), or the
    device builder's buffer with its summary read back (tests only)."""
    T = w.T
    seg = torch.empty(agm.segment_words(T), dtype=torch.int32, device=DEV)
    if device_build:
        ids = torch.from_numpy(w.ids.astype(np.int32)).to(DEV)
        act = torch.from_numpy(w.active.astype(np.uint8)).to(DEV)
        agm.build_segments_dev(ids, act, n_slots, seg, order)
        torch.cuda.synchronize()
        words = seg[:agm.SEG_HEADER].cpu().numpy()
        return seg, agm.summary_from_words(words)
    staging = torch.empty(agm.segment_words(T), dtype=torch.int32).pin_memory()
    ids = torch.from_numpy(w.ids.astype(np.int32))
    act = torch.from_numpy(w.active.astype(np.uint8))
    s = agm.build_segments(ids, act, n_slots, seg, staging, order)
    torch.cuda.synchronize()
    return seg, s


def split_seg(seg: torch.Tensor, T: int):
    plan = seg.cpu().numpy()
    h = agm.SEG_HEADER
    return dict(sum=plan[:h], perm=plan[h:h + T], pos_seg=plan[h + T:h + 2 * T],
                seg_start=plan[h + 2 * T:h + 3 * T + 1], seg_adapter=plan[h + 3 * T + 1:h + 4 * T + 1],
                tiles_small=plan[h + 4 * T + 1:h + 6 * T + 1].reshape(-1, 2) if T else plan[:0],
                tiles_large=plan[h + 6 * T + 1:h + 8 * T + 1].reshape(-1, 2) if T else plan[:0])
