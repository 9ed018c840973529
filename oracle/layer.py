"""fp64 definition of the batched heterogeneous-adapter linear layer.

Test infrastructure only.

For token row i with adapter a = ids[i] (LLM-stack book 7.14.1, "the
batched-heterogeneous problem"; LoRazor 3.1.1 Eqs. 1-2; LoRAForge 2
"Multi-LoRA Serving"):

    base_i = W0 x_i
    live_i = ids[i] >= 0 and active[i] != 0       (id -1 = no adapter, book
                                                   7.14.2 data layout; an
                                                   inactive row is a released
                                                   adapter, LoRazor 3.2)
    v_i    = A_a[:r_a] x_i                        (shrink, rank-r_a down-projection)
    y_i    = base_i + [live_i] s_a B_a[:, :r_a] v_i   (expand, scaled and added)

Storage convention used throughout (the stacked-pool layout of the book's
7.14.2 with one pool per projection): A_pool[a] is [R_cap, d_in] (row j is the
j-th down-projection direction) and B_pool[a] is [d_out, R_cap].  Rank entries
j >= r_a are padding and never read.

Inputs arrive as *stored* values (float32 arrays, bf16 bit patterns, or e4m3
codes with per-channel scales) and are decoded exactly to float64 here.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .numerics import decode_bf16, decode_e4m3, encode_e4m3, E4M3_MAX


def as_f64(a, kind: str = "auto") -> np.ndarray:
    """Stored array -> exact float64.  uint16 = bf16 bits; float32/64 as is."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return decode_bf16(a)
    if a.dtype == np.uint8:
        raise TypeError("fp8 codes need their scales: use dequant_e4m3_rows")
    return a.astype(np.float64)


def dequant_e4m3_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W0deq[n, k] = e4m3(codes[n, k]) * scale[n] (per-output-channel scale)."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def live_rows(ids: np.ndarray, active: Optional[np.ndarray] = None) -> np.ndarray:
    ids = np.asarray(ids)
    live = ids >= 0
    if active is not None:
        live = live & (np.asarray(active) != 0)
    return live


def base_output(x, w0) -> np.ndarray:
    """x W0^T in float64; w0 is a stored array or a (codes, scales) fp8 pair."""
    X = as_f64(x)
    W = dequant_e4m3_rows(*w0) if isinstance(w0, tuple) else as_f64(w0)
    return X @ W.T


def shrink_rows(x, ids, active, A_pool, slot_rank) -> np.ndarray:
    """v[i, j] = sum_k x[i, k] A_a[j, k] for live rows and j < r_a; 0 elsewhere.

    Indexed by token row (the GPU path stores it in segment order)."""
    X = as_f64(x)
    ids = np.asarray(ids)
    live = live_rows(ids, active)
    T = X.shape[0]
    R_cap = np.asarray(A_pool).shape[1]
    v = np.zeros((T, R_cap), np.float64)
    for a in sorted(set(int(i) for i in ids[live])):
        rows = np.nonzero(live & (ids == a))[0]
        r = int(slot_rank[a])
        A = as_f64(A_pool[a][:r])
        v[rows, :r] = X[rows] @ A.T
    return v


def lora_delta(x, ids, active, A_pool, B_pool, slot_rank, slot_scale, v_rows=None) -> np.ndarray:
    """The adapter term s_a B_a v_i per row, grouped by adapter.

    One down- and one up-projection per distinct live adapter, each adapter's
    weights loaded once (the book's 7.14.10 grouped formulation).  If
    ``v_rows`` is given it replaces the shrink result (used to check an
    expand in isolation)."""
    X = as_f64(x)
    ids = np.asarray(ids)
    live = live_rows(ids, active)
    T = X.shape[0]
    d_out = np.asarray(B_pool).shape[1]
    out = np.zeros((T, d_out), np.float64)
    for a in sorted(set(int(i) for i in ids[live])):
        rows = np.nonzero(live & (ids == a))[0]
        r = int(slot_rank[a])
        if v_rows is None:
            v = X[rows] @ as_f64(A_pool[a][:r]).T
        else:
            v = np.asarray(v_rows, np.float64)[rows, :r]
        out[rows] = float(slot_scale[a]) * (v @ as_f64(B_pool[a][:, :r]).T)
    return out


def lora_delta_per_row(x, ids, active, A_pool, B_pool, slot_rank, slot_scale,
                       rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Brute force, one row at a time: two matrix-vector products per row.

    Returns only the requested rows (all rows by default)."""
    X = as_f64(x)
    ids = np.asarray(ids)
    live = live_rows(ids, active)
    rows = range(X.shape[0]) if rows is None else rows
    d_out = np.asarray(B_pool).shape[1]
    out = np.zeros((len(rows), d_out), np.float64)
    for o, i in enumerate(rows):
        if not live[i]:
            continue
        a = int(ids[i])
        r = int(slot_rank[a])
        A = as_f64(A_pool[a][:r])          # [r, d_in]
        B = as_f64(B_pool[a][:, :r])       # [d_out, r]
        out[o] = float(slot_scale[a]) * (B @ (A @ X[i]))
    return out


def lora_delta_gathered(x, ids, active, A_pool, B_pool, slot_rank, slot_scale) -> np.ndarray:
    """Gather-per-row formulation: every row gathers its own A, B, scale and
    rank mask, then two batched products (the book's toy MultiLoRALinear
    forward, which indexes the stacked pools by the per-token index)."""
    X = as_f64(x)
    ids = np.asarray(ids)
    live = live_rows(ids, active)
    safe = np.where(live, ids, 0)
    R_cap = np.asarray(A_pool).shape[1]
    A = as_f64(np.asarray(A_pool)[safe])                 # [T, R_cap, d_in]
    B = as_f64(np.asarray(B_pool)[safe])                 # [T, d_out, R_cap]
    mask = (np.arange(R_cap)[None, :] < np.asarray(slot_rank)[safe][:, None]).astype(np.float64)
    s = np.asarray(slot_scale, np.float64)[safe] * live
    v = np.einsum("tk,tjk->tj", X, np.where(mask[:, :, None] > 0, A, 0.0)) * mask
    d = np.einsum("tj,tnj->tn", v, np.where(mask[:, None, :] > 0, B, 0.0))
    return d * s[:, None]


def linear(x, w0, ids, active, A_pool, B_pool, slot_rank, slot_scale) -> np.ndarray:
    """y = x W0^T + adapter term (fp64)."""
    return base_output(x, w0) + lora_delta(x, ids, active, A_pool, B_pool, slot_rank, slot_scale)


def merged_linear(x, w0, A, B, r: int, s: float) -> np.ndarray:
    """Single-adapter merged weight (W0 + s B A) applied to every row
    (the book's 7.14.1 "merging" paragraph): the multi-tenant result must equal
    this when every row carries the same adapter."""
    W = dequant_e4m3_rows(*w0) if isinstance(w0, tuple) else as_f64(w0)
    Af = as_f64(A)[:r]
    Bf = as_f64(B)[:, :r]
    return as_f64(x) @ (W + s * (Bf @ Af)).T


def act_quant_e4m3(x) -> tuple:
    """Per-token activation quantisation for the W8A8 base product.

    EpiLoRA 2 / Fig. 4: the activations are quantised once per token to FP8
    with a per-token scale s_x.  Reading adopted: s_x = amax_i / 448 computed in
    fp32, q = x / s_x in fp32, then round to nearest even e4m3 with
    saturation; an all-zero row gets s_x = 1.  The fp32 steps are the
    decision precision the kernel also uses, so the codes can be compared
    bit for bit.  Returns (codes uint8 [T, d], s_x float32 [T])."""
    X32 = as_f64(x).astype(np.float32)
    amax = np.abs(X32).max(axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[amax == 0] = np.float32(1.0)
    q = (X32 / s[:, None]).astype(np.float32)
    return encode_e4m3(q), s


def linear_w8a8(x, w0_codes, w0_scale, ids, active, A_pool, B_pool, slot_rank, slot_scale) -> np.ndarray:
    """W8A8 variant: the base product uses the quantised activations,
    y_i = (x_q,i . W_q) s_x,i s_w + adapter term on the unquantised x."""
    codes, s_x = act_quant_e4m3(x)
    xq = decode_e4m3(codes) * s_x.astype(np.float64)[:, None]
    base = xq @ dequant_e4m3_rows(w0_codes, w0_scale).T
    return base + lora_delta(x, ids, active, A_pool, B_pool, slot_rank, slot_scale)
