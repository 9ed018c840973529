"""Seeded synthetic workloads for the batched multi-adapter linear layer.

This module only *draws* inputs: it holds none of the layer's arithmetic.
Both the fp64 oracle (``oracle/``) and the GPU path (``adapter_gemm_amd``)
consume what it returns, and neither imports the other.

Every array is produced by numpy's PCG64 from a seed that is a tuple
``(seed, stream, ...)``, so that each component (base weight, each adapter
slot of each projection, activations, ids, masks) has its own independent
stream and can be regenerated on its own.  Stored values are the truth:
bf16 data is drawn in fp32 and rounded to bf16 (round to nearest even) here,
fp8 base weights are quantised here to OCP e4m3 codes plus per-output-channel
fp32 scales.  Both oracle and kernels read the stored values.

Shapes, distributions and id/mask/length recipes of the five workloads
(``CONFIG_NAMES``) are stated where each is built, in ``make_workload``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

# stream tags, fixed so that regenerating one component never shifts another
_S_W0, _S_SLOT, _S_X, _S_IDS, _S_MASK, _S_LEN, _S_RANK, _S_NEG = 1, 2, 3, 4, 5, 6, 7, 8


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_quantise_rows(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row fp8 (OCP e4m3fn) quantisation of an input weight matrix.

    scale[n] = amax(|w[n, :]|) / 448 in fp32 (1.0 for an all-zero row);
    codes = e4m3(w / scale) rounded to nearest even and clamped to +-448.
    The library conversion used here (torch's float8_e4m3fn cast) is an
    input-preparation step only; the oracle decodes codes with its own table.
    """
    import torch  # local: only this input-preparation step needs it

    w = np.ascontiguousarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    q = np.clip(w / scale[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


@dataclasses.dataclass
class Projection:
    """One linear layer: base weight plus an adapter pool of ``n_slots`` slots."""

    name: str
    d_in: int
    d_out: int
    n_slots: int
    r_cap: int
    slot_rank: np.ndarray          # int32 [N]
    slot_scale: np.ndarray         # float32 [N]
    w_std: float                   # std of W0 draws
    a_std: float                   # std of A draws
    b_std: float                   # std of B draws
    base_dtype: str                # "fp32" | "bf16" | "fp8"
    data_dtype: str                # "fp32" | "bf16" (x, A, B, y)
    _key: Tuple[int, ...] = ()

    # --- base weight -----------------------------------------------------
    def w0(self):
        """Stored base weight.

        fp32: float32 [d_out, d_in]; bf16: uint16 bits [d_out, d_in];
        fp8: (uint8 codes [d_out, d_in], float32 scales [d_out]).
        """
        g = _rng(*self._key, _S_W0)
        if self.base_dtype == "fp32":
            return (g.standard_normal((self.d_out, self.d_in)) * self.w_std).astype(np.float32)
        w = g.standard_normal((self.d_out, self.d_in), dtype=np.float32) * np.float32(self.w_std)
        if self.base_dtype == "bf16":
            return bf16_round(w)
        return e4m3_quantise_rows(w)

    # --- adapters --------------------------------------------------------
    def slot(self, a: int) -> Tuple[np.ndarray, np.ndarray]:
        """Stored (A [r_cap, d_in], B [d_out, r_cap]) of slot ``a``.

        Rank entries j >= slot_rank[a] (rows of A, columns of B) are zero.
        fp32 data -> float32 arrays, bf16 -> uint16 bits.  Draw order: A
        row-major [r, d_in], then B row-major [d_out, r].
        """
        r = int(self.slot_rank[a])
        g = _rng(*self._key, _S_SLOT, a)
        if self.data_dtype == "fp32":
            A = np.zeros((self.r_cap, self.d_in), np.float32)
            B = np.zeros((self.d_out, self.r_cap), np.float32)
            A[:r] = g.standard_normal((r, self.d_in)) * self.a_std
            B[:, :r] = g.standard_normal((self.d_out, r)) * self.b_std
            return A, B
        A = np.zeros((self.r_cap, self.d_in), np.uint16)
        B = np.zeros((self.d_out, self.r_cap), np.uint16)
        A[:r] = bf16_round(g.standard_normal((r, self.d_in), dtype=np.float32) * np.float32(self.a_std))
        B[:, :r] = bf16_round(g.standard_normal((self.d_out, r), dtype=np.float32) * np.float32(self.b_std))
        return A, B

    def pool(self, slots: Optional[List[int]] = None):
        """Stacked (A_pool [N, r_cap, d_in], B_pool [N, d_out, r_cap]).

        Slots not listed in ``slots`` are left zero (callers that only need
        the adapters a batch touches pass that list).
        """
        dt = np.float32 if self.data_dtype == "fp32" else np.uint16
        A = np.zeros((self.n_slots, self.r_cap, self.d_in), dt)
        B = np.zeros((self.n_slots, self.d_out, self.r_cap), dt)
        for a in (range(self.n_slots) if slots is None else slots):
            A[a], B[a] = self.slot(a)
        return A, B


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    T: int
    projections: List[Projection]
    ids: np.ndarray                # int32 [T], -1 = no adapter
    active: np.ndarray             # uint8 [T], 0 = released adapter
    data_dtype: str
    x_std: float = 1.0
    description: str = ""

    def x(self, proj: Projection) -> np.ndarray:
        """Activations [T, d_in] of one projection (float32 or bf16 bits)."""
        g = _rng(self.seed, 0, _S_X, proj.d_in, self.projections.index(proj))
        if self.data_dtype == "fp32":
            return (g.standard_normal((self.T, proj.d_in)) * self.x_std).astype(np.float32)
        return bf16_round(g.standard_normal((self.T, proj.d_in), dtype=np.float32) * np.float32(self.x_std))

    def live(self) -> np.ndarray:
        return (self.ids >= 0) & (self.active != 0)

    def touched_slots(self) -> List[int]:
        return sorted(set(int(i) for i in self.ids[self.live()]))


def zipf_ids(g: np.random.Generator, n_ids: int, s: float, size: int) -> np.ndarray:
    """Truncated Zipf: P(id = j) proportional to (j + 1)^-s for j in [0, n_ids)."""
    p = np.arange(1, n_ids + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return g.choice(n_ids, size=size, p=p).astype(np.int32)


def lognormal_lengths(g: np.random.Generator, n: int, mu: float, sigma: float, total: int) -> np.ndarray:
    """n lognormal(mu, sigma) request lengths rescaled to sum exactly ``total``.

    Scale by total/sum, take floor with a minimum of 1, then hand out the
    remainder +1 each by largest fractional part (ties to the lower index);
    if the minimum of 1 overshoots, take 1 back from the largest lengths.
    """
    raw = g.lognormal(mean=mu, sigma=sigma, size=n)
    scaled = raw * (total / raw.sum())
    base = np.maximum(np.floor(scaled).astype(np.int64), 1)
    rem = total - int(base.sum())
    frac = scaled - np.floor(scaled)
    if rem > 0:
        order = sorted(range(n), key=lambda i: (-frac[i], i))
        for i in order[:rem]:
            base[i] += 1
    while rem < 0:
        i = int(np.argmax(base))
        base[i] -= 1
        rem += 1
    assert int(base.sum()) == total and base.min() >= 1
    return base.astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = ("tiny_sgmv", "decode_bgmv", "prefill_sgmv", "fp8_fused", "llama_layer")


def _proj(key, name, d_in, d_out, n_slots, r_cap, ranks, scales, w_std, a_std, b_std, base, data):
    return Projection(name=name, d_in=d_in, d_out=d_out, n_slots=n_slots, r_cap=r_cap,
                      slot_rank=np.asarray(ranks, np.int32), slot_scale=np.asarray(scales, np.float32),
                      w_std=w_std, a_std=a_std, b_std=b_std, base_dtype=base, data_dtype=data, _key=key)


def make_workload(name: str, seed: Optional[int] = None, **over) -> Workload:
    """Build one of the five workloads.

    ``over`` may shrink sizes for fast tests (keys: T, d_in, d_out,
    n_slots, r, n_req); the recipe is otherwise unchanged.
    """
    idx = CONFIG_NAMES.index(name) + 1
    seed = idx if seed is None else seed
    key = (seed, idx)

    if name == "tiny_sgmv":
        # 512 -> 512 fp32; 4 adapters of rank 8; 64 tokens in 4 contiguous
        # segments of 16 with ids 0..3; W0, A ~ N(0, 1/d_in) (variance),
        # B ~ N(0, 1/r); x ~ N(0, 1); s = 2.
        d_in = over.get("d_in", 512)
        d_out = over.get("d_out", 512)
        r = over.get("r", 8)
        nseg = over.get("n_slots", 4)
        per = over.get("T", 64) // nseg
        T = per * nseg
        p = _proj(key, "proj", d_in, d_out, nseg, r, [r] * nseg, [2.0] * nseg,
                  1 / math.sqrt(d_in), 1 / math.sqrt(d_in), 1 / math.sqrt(r), "fp32", "fp32")
        ids = np.repeat(np.arange(nseg, dtype=np.int32), per)
        return Workload(name, seed, T, [p], ids, np.ones(T, np.uint8), "fp32",
                        description=f"{d_in}->{d_out} fp32, {nseg} adapters r{r}, {T} tokens")

    if name == "decode_bgmv":
        # q_proj 4096 -> 4096 bf16; 256 decode tokens; 64 slots of rank 16;
        # ids ~ Zipf(1.1); exactly 25% of rows set to -1; N(0, 0.02) weights.
        d_in = over.get("d_in", 4096)
        d_out = over.get("d_out", 4096)
        T = over.get("T", 256)
        N = over.get("n_slots", 64)
        r = over.get("r", 16)
        p = _proj(key, "q_proj", d_in, d_out, N, r, [r] * N, [2.0] * N, 0.02, 0.02, 0.02, "bf16", "bf16")
        ids = zipf_ids(_rng(*key, _S_IDS), N, 1.1, T)
        neg = _rng(*key, _S_NEG).choice(T, size=int(round(0.25 * T)), replace=False)
        ids[neg] = -1
        return Workload(name, seed, T, [p], ids, np.ones(T, np.uint8), "bf16",
                        description=f"{d_in}->{d_out} bf16, {T} decode tokens, {N} slots r{r}, Zipf(1.1), 25% id -1")

    if name == "prefill_sgmv":
        # fused gate+up 4096 -> 28672 bf16; 8192 tokens in 32 requests with
        # lognormal(5.5, 0.8) lengths; one adapter per request uniform over
        # 128; ranks uniform over {8,16,32,64}; s = 32 / r.
        d_in = over.get("d_in", 4096)
        d_out = over.get("d_out", 28672)
        T = over.get("T", 8192)
        n_req = over.get("n_req", 32)
        N = over.get("n_slots", 128)
        choices = np.array([8, 16, 32, 64], np.int32)
        ranks = choices[_rng(*key, _S_RANK).integers(0, 4, N)]
        r_cap = int(over.get("r", 64))
        ranks = np.minimum(ranks, r_cap)
        scales = (32.0 / ranks).astype(np.float32)
        p = _proj(key, "gate_up", d_in, d_out, N, r_cap, ranks, scales, 0.02, 0.02, 0.02, "bf16", "bf16")
        lens = lognormal_lengths(_rng(*key, _S_LEN), n_req, 5.5, 0.8, T)
        req_ids = _rng(*key, _S_IDS).integers(0, N, n_req).astype(np.int32)
        ids = np.repeat(req_ids, lens).astype(np.int32)
        w = Workload(name, seed, T, [p], ids, np.ones(T, np.uint8), "bf16",
                     description=f"{d_in}->{d_out} bf16, {T} tokens in {n_req} requests, {N} slots r{{8..64}}")
        w.request_lengths = lens
        return w

    if name == "fp8_fused":
        # 8192 -> 28672, W0 fp8 e4m3 + per-channel fp32 scales; bf16
        # activations; 512 decode tokens; 256 slots of rank 64; Zipf(1.1); s = 1.
        d_in = over.get("d_in", 8192)
        d_out = over.get("d_out", 28672)
        T = over.get("T", 512)
        N = over.get("n_slots", 256)
        r = over.get("r", 64)
        p = _proj(key, "proj", d_in, d_out, N, r, [r] * N, [1.0] * N, 0.02, 0.02, 0.02, "fp8", "bf16")
        ids = zipf_ids(_rng(*key, _S_IDS), N, 1.1, T)
        return Workload(name, seed, T, [p], ids, np.ones(T, np.uint8), "bf16",
                        description=f"{d_in}->{d_out} fp8 base, {T} decode tokens, {N} slots r{r}, Zipf(1.1)")

    if name == "llama_layer":
        # Llama-3-8B decoder-layer projections, bf16, 1024 slots of rank 16
        # per projection; 16 prefill requests of 96 tokens then 512 decode
        # rows; Zipf(1.05); half the decode rows masked inactive; s = 2.
        shapes = over.get("shapes", [("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
                                     ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336),
                                     ("up_proj", 4096, 14336), ("down_proj", 14336, 4096)])
        N = over.get("n_slots", 1024)
        r = over.get("r", 16)
        n_pre = over.get("n_req", 16)
        pre_len = over.get("prefill_len", 96)
        n_dec = over.get("n_decode", 512)
        T = n_pre * pre_len + n_dec
        projs = [_proj(key + (k,), nm, di, do, N, r, [r] * N, [2.0] * N, 0.02, 0.02, 0.02, "bf16", "bf16")
                 for k, (nm, di, do) in enumerate(shapes)]
        g = _rng(*key, _S_IDS)
        req = zipf_ids(g, N, 1.05, n_pre)
        dec = zipf_ids(g, N, 1.05, n_dec)
        ids = np.concatenate([np.repeat(req, pre_len), dec]).astype(np.int32)
        active = np.ones(T, np.uint8)
        off = _rng(*key, _S_MASK).choice(n_dec, size=n_dec // 2, replace=False)
        active[n_pre * pre_len + off] = 0
        return Workload(name, seed, T, projs, ids, active, "bf16",
                        description=f"Llama-3-8B layer set bf16, {N} slots r{r}, {n_pre}x{pre_len} prefill + {n_dec} decode")

    raise KeyError(name)
