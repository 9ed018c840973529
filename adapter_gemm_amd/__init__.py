"""Python binding of liblora (argument marshalling only).

Every step of the layer runs in the HIP kernels behind the C-ABI declared in
include/lora.h; this module turns torch tensors into pointers, sizes and the
current HIP stream, calls the library and raises on a non-zero status.  There
is no fallback: if liblora.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora.so")

# status codes / enums (mirror include/lora.h)
LORA_OK, LORA_E_ARG, LORA_E_ID, LORA_E_RANK, LORA_E_DTYPE, LORA_E_ALIGN, LORA_E_HIP, LORA_E_SIZE = range(8)
F32, BF16, FP8_E4M3 = 0, 1, 2
LAUNCH_EXACT, LAUNCH_PERSISTENT, LAUNCH_BUCKETED, LAUNCH_FULL_BATCH = 0, 1, 2, 3
FLAG_ACT_QUANT_E4M3 = 0x1
FLAG_SHRINK_IN_LAUNCH = 0x2
MAX_RANK = 128
DEV_MAX_SLOTS = 8192
TILE_SMALL, TILE_LARGE = 16, 64
SEG_HEADER = 16

EXPORTED = [
    "lora_segment_words", "lora_build_segments", "lora_plan_segments", "lora_build_segments_dev",
    "lora_shrink", "lora_build_shrink_dev", "lora_expand", "lora_fused_linear", "lora_fused_workspace_bytes",
    "lora_fused_workspace_bytes_rcap", "lora_fused_linear_noalloc",
    "lora_fused_linear_slices", "lora_fused_slices_workspace_bytes",
    "lora_registry_create", "lora_registry_destroy", "lora_registry_acquire", "lora_registry_release",
    "lora_registry_lookup", "lora_registry_stats", "lora_pool_install",
    "lora_device_cu_count", "lora_stream_create_cu_masked", "lora_stream_destroy",
    "lora_quantize_e4m3", "lora_status_string", "lora_last_error",
]


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.lora_status_string(status).decode()
        if status == LORA_E_HIP:
            msg += ": " + _lib.lora_last_error().decode()
        super().__init__(f"{where}: {msg} (status {status})")


class PoolDesc(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("slot_rank", ctypes.c_void_p),
                ("slot_scale", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("r_cap", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32)]


class BaseDesc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("w_scale", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ld_w", ctypes.c_int32)]


class Summary(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_active", "n_segments", "m_max", "row_bound", "n_tiles_small", "n_tiles_large", "T", "error")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


def _load():
    # torch ships its own HIP runtime (same soname as ROCm's); loading torch
    # first makes liblora bind to that one copy instead of opening a second
    # runtime in the same process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m adapter_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "lora_segment_words": (SZ, [I32]),
        "lora_plan_segments": (I32, [P, P, I32, I32, I32, P, P]),
        "lora_build_segments": (I32, [P, P, I32, I32, I32, P, P, P, P]),
        "lora_build_segments_dev": (I32, [P, P, I32, I32, I32, P, P]),
        "lora_shrink": (I32, [P, P, I32, P, P, I32, P, I32, I32, P]),
        "lora_build_shrink_dev": (I32, [P, P, I32, I32, P, P, P, I32, P, I32, P]),
        "lora_expand": (I32, [P, P, I32, P, P, I32, P, I32, I32, I32, P]),
        "lora_fused_linear": (I32, [P, P, P, I32, P, I32, P, I32, P, I32, I32, I32, I32, P, SZ, P]),
        "lora_fused_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
        "lora_fused_workspace_bytes_rcap": (SZ, [I32, I32, I32, I32, I32, I32]),
        "lora_fused_linear_noalloc": (I32, [P, P, P, I32, P, I32, P, I32, P, I32, I32, I32, I32, P]),
        "lora_fused_linear_slices": (I32, [I32, P, P, P, I32, P, I32, I32, P, P, P, P, P, I32, P, SZ, P]),
        "lora_fused_slices_workspace_bytes": (SZ, [I32, I32, I32, P, I32, I32]),
        "lora_registry_create": (I32, [I32, I32, P]),
        "lora_registry_destroy": (None, [P]),
        "lora_registry_acquire": (I32, [P, ctypes.c_int64, P, P]),
        "lora_registry_release": (I32, [P, ctypes.c_int64]),
        "lora_registry_lookup": (I32, [P, ctypes.c_int64, P]),
        "lora_registry_stats": (I32, [P, P]),
        "lora_pool_install": (I32, [P, I32, P, P, I32, ctypes.c_float, P]),
        "lora_device_cu_count": (I32, [P]),
        "lora_stream_create_cu_masked": (I32, [P, I32, P]),
        "lora_stream_destroy": (I32, [P]),
        "lora_quantize_e4m3": (I32, [P, I32, I32, I32, P, I32, P, P]),
        "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "lora_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def _check(status: int, where: str):
    if status != LORA_OK:
        raise LoraError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _ld(t) -> int:
    """Leading dimension of a row-major [rows, cols] tensor (rows <= 1: cols)."""
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1])


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8_E4M3,
            torch.float8_e4m3fn: FP8_E4M3}[t.dtype]


def pool_desc(A, B, slot_rank, slot_scale) -> PoolDesc:
    """A [N, r_cap, d_in], B [N, d_out, r_cap] (fp32 or bf16), slot_rank int32 [N],
    slot_scale fp32 [N], all on the device."""
    N, r_cap, d_in = A.shape
    d_out = B.shape[1]
    d = PoolDesc(A.data_ptr(), B.data_ptr(), slot_rank.data_ptr(), slot_scale.data_ptr(), _dtype_code(A),
                 N, r_cap, d_in, d_out)
    d._keep = (A, B, slot_rank, slot_scale)   # the descriptor holds raw addresses: keep their memory alive
    return d


def base_desc(W, w_scale=None) -> BaseDesc:
    """W [d_out, ld_w] fp32 / bf16 / uint8 e4m3 codes; w_scale fp32 [d_out] for fp8."""
    d = BaseDesc(W.data_ptr(), _ptr(w_scale), _dtype_code(W), W.stride(0))
    d._keep = (W, w_scale)
    return d


def segment_words(T: int) -> int:
    return int(_lib.lora_segment_words(T))


def plan_segments(ids, active, n_slots: int, order: int = 0):
    """Host-only grouping (numpy int32 ids / uint8 active) -> (plan int32 array, summary dict)."""
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = int(ids.shape[0])
    act = None if active is None else np.ascontiguousarray(active, dtype=np.uint8)
    plan = np.zeros(segment_words(T), dtype=np.int32)
    s = Summary()
    _check(_lib.lora_plan_segments(ids.ctypes.data, None if act is None else act.ctypes.data, T, n_slots, order,
                                   plan.ctypes.data, ctypes.byref(s)), "lora_plan_segments")
    return plan, s.as_dict()


def build_segments(ids, active, n_slots: int, seg, staging, order: int = 0, stream=None) -> Summary:
    """Host ids (CPU int32 tensor) -> device segment buffer `seg`; `staging` is a
    host int32 tensor of segment_words(T) words (pinned for an asynchronous copy)."""
    T = int(ids.shape[0])
    s = Summary()
    _check(_lib.lora_build_segments(_ptr(ids), _ptr(active), T, n_slots, order, staging.data_ptr(),
                                    seg.data_ptr(), ctypes.byref(s), _stream(stream)), "lora_build_segments")
    return s


def build_segments_dev(ids, active, n_slots: int, seg, order: int = 0, stream=None) -> None:
    T = int(ids.shape[0])
    _check(_lib.lora_build_segments_dev(_ptr(ids), _ptr(active), T, n_slots, order, seg.data_ptr(),
                                        _stream(stream)), "lora_build_segments_dev")


def shrink(pool: PoolDesc, seg, T: int, summary: Optional[Summary], x, v, launch: int = LAUNCH_EXACT,
           stream=None) -> None:
    _check(_lib.lora_shrink(ctypes.byref(pool), seg.data_ptr(), T,
                            None if summary is None else ctypes.byref(summary), x.data_ptr(), _ld(x),
                            v.data_ptr(), _ld(v), launch, _stream(stream)), "lora_shrink")


def build_shrink_dev(ids, active, pool: PoolDesc, seg, x, v, order: int = 0, stream=None) -> None:
    """Device segment build and persistent shrink of one batch (one launch for small batches)."""
    T = int(ids.shape[0])
    _check(_lib.lora_build_shrink_dev(_ptr(ids), _ptr(active), T, order, ctypes.byref(pool), seg.data_ptr(),
                                      x.data_ptr(), _ld(x), v.data_ptr(), _ld(v), _stream(stream)),
           "lora_build_shrink_dev")


def expand(pool: PoolDesc, seg, T: int, summary: Optional[Summary], v, y, launch: int = LAUNCH_EXACT,
           stream=None) -> None:
    _check(_lib.lora_expand(ctypes.byref(pool), seg.data_ptr(), T,
                            None if summary is None else ctypes.byref(summary), v.data_ptr(), _ld(v),
                            y.data_ptr(), _dtype_code(y), _ld(y), launch, _stream(stream)), "lora_expand")


def fused_workspace_bytes(T: int, d_in: int, d_out: int, base_dtype: int, flags: int = 0) -> int:
    """Workspace bytes of a fused call of this shape (base_dtype: F32, BF16 or FP8_E4M3)."""
    return int(_lib.lora_fused_workspace_bytes(T, d_in, d_out, base_dtype, flags))


def fused_workspace(T: int, d_in: int, d_out: int, base_dtype: int, flags: int = 0, device="cuda"):
    """A workspace tensor for a fused call of this shape (None when none is needed);
    torch's allocator hands out 256-byte aligned blocks."""
    import torch
    n = fused_workspace_bytes(T, d_in, d_out, base_dtype, flags)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


EVICT_LRU, EVICT_LFU = 0, 1


class Registry:
    """Adapter residency over the slots of a pool (host bookkeeping in the
    library): adapters are named by any hashable; acquire() returns the slot
    and whether it must be filled (pool_install) before kernels read it."""

    def __init__(self, n_slots: int, policy: int = EVICT_LRU):
        h = ctypes.c_void_p()
        _check(_lib.lora_registry_create(n_slots, policy, ctypes.byref(h)), "lora_registry_create")
        self._h = h
        self._destroy = _lib.lora_registry_destroy      # kept: module globals may be gone at exit
        self._keys = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    def _key(self, name) -> int:
        return self._keys.setdefault(name, len(self._keys))

    def acquire(self, name):
        """(slot, needs_install) for one use of `name`; raises LoraError with
        LORA_E_SIZE when every slot holds an adapter in use."""
        slot, need = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.lora_registry_acquire(self._h, self._key(name), ctypes.byref(slot), ctypes.byref(need)),
               "lora_registry_acquire")
        return int(slot.value), bool(need.value)

    def release(self, name) -> None:
        _check(_lib.lora_registry_release(self._h, self._key(name)), "lora_registry_release")

    def lookup(self, name) -> int:
        slot = ctypes.c_int32()
        _check(_lib.lora_registry_lookup(self._h, self._key(name), ctypes.byref(slot)), "lora_registry_lookup")
        return int(slot.value)

    def stats(self) -> dict:
        out = (ctypes.c_int64 * 4)()
        _check(_lib.lora_registry_stats(self._h, out), "lora_registry_stats")
        return {"hits": out[0], "misses": out[1], "evictions": out[2], "resident": out[3]}


def pool_install(pool: PoolDesc, slot: int, A, B, rank: int, scale: float, stream=None) -> None:
    """Fill one slot: A [rank, d_in], B [d_out, rank] (host, ideally pinned, or
    device tensors in the pool dtype), asynchronously on the stream."""
    _check(_lib.lora_pool_install(ctypes.byref(pool), slot, _ptr(A), _ptr(B), rank, scale, _stream(stream)),
           "lora_pool_install")


def cu_count() -> int:
    n = ctypes.c_int32()
    _check(_lib.lora_device_cu_count(ctypes.byref(n)), "lora_device_cu_count")
    return int(n.value)


def cu_mask_words(cus, n_cus: int):
    """32-bit mask words with the bits of the given logical CU indices set."""
    words = [0] * ((n_cus + 31) // 32)
    for c in cus:
        if not 0 <= c < n_cus:
            raise ValueError(f"CU {c} outside 0..{n_cus - 1}")
        words[c // 32] |= 1 << (c % 32)
    return words


class CUMaskedStream:
    """A stream whose kernels run only on the given CUs; `.stream` is a torch
    stream over it (pass it as `stream=` to the calls or to torch's events)."""

    def __init__(self, cus, n_cus: Optional[int] = None):
        import torch
        n = cu_count() if n_cus is None else n_cus
        words = cu_mask_words(cus, n)
        arr = (ctypes.c_uint32 * len(words))(*words)
        h = ctypes.c_void_p()
        _check(_lib.lora_stream_create_cu_masked(arr, len(words), ctypes.byref(h)), "lora_stream_create_cu_masked")
        self._h = h
        self._destroy = _lib.lora_stream_destroy
        self.cus = sorted(set(cus))
        self.stream = torch.cuda.ExternalStream(h.value)

    def close(self) -> None:
        # work still queued on the stream completes before its resources go
        if self._h is not None and self._h.value:
            self._destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fused_slices_workspace(T: int, d_in: int, d_outs, base_dtype: int, flags: int = 0, device="cuda"):
    """A workspace tensor for a sliced fused call (None when none is needed)."""
    import torch
    n = len(d_outs)
    arr = (ctypes.c_int32 * n)(*[int(d) for d in d_outs])
    nb = int(_lib.lora_fused_slices_workspace_bytes(n, T, d_in, arr, base_dtype, flags))
    return None if nb == 0 else torch.empty(nb, dtype=torch.uint8, device=device)


def fused_linear_slices(bases, pools, seg, x, vs, ys, flags: int = 0, workspace=None, stream=None) -> None:
    """Several projections of one x in one launch: slice s is fused_linear(bases[s],
    pools[s], seg, x, vs[s], ys[s]); pools / vs None for the base products alone."""
    n = len(bases)
    T, d_in = int(x.shape[0]), int(x.shape[1])
    b_arr = (BaseDesc * n)(*bases)
    p_arr = None if pools is None else (PoolDesc * n)(*pools)
    v_arr = None if vs is None else (ctypes.c_void_p * n)(*[v.data_ptr() for v in vs])
    ldv = None if vs is None else (ctypes.c_int32 * n)(*[_ld(v) for v in vs])
    y_arr = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    ldy = (ctypes.c_int32 * n)(*[_ld(y) for y in ys])
    d_out = (ctypes.c_int32 * n)(*[int(y.shape[1]) for y in ys])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lora_fused_linear_slices(n, b_arr, p_arr, _ptr(seg), T, x.data_ptr(), _ld(x), d_in, d_out,
                                         v_arr, ldv, y_arr, ldy, flags, _ptr(workspace), ws_bytes,
                                         _stream(stream)), "lora_fused_linear_slices")


def fused_linear(base: BaseDesc, pool: Optional[PoolDesc], seg, x, v, y, flags: int = 0, workspace=None,
                 stream=None) -> None:
    T, d_in = int(x.shape[0]), int(x.shape[1])
    d_out = int(y.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lora_fused_linear(ctypes.byref(base), None if pool is None else ctypes.byref(pool), _ptr(seg), T,
                                  x.data_ptr(), _ld(x), _ptr(v), 0 if v is None else _ld(v),
                                  y.data_ptr(), _ld(y), d_in, d_out, flags, _ptr(workspace), ws_bytes,
                                  _stream(stream)), "lora_fused_linear")


def fused_linear_noalloc(base: BaseDesc, pool: Optional[PoolDesc], seg, x, v, y, flags: int = 0,
                         stream=None) -> None:
    """fused_linear with the library's static per-GPU scratch instead of a
    workspace (the call allocates nothing; calls on one GPU must not overlap)."""
    T, d_in = int(x.shape[0]), int(x.shape[1])
    d_out = int(y.shape[1])
    _check(_lib.lora_fused_linear_noalloc(ctypes.byref(base), None if pool is None else ctypes.byref(pool),
                                          _ptr(seg), T, x.data_ptr(), _ld(x), _ptr(v), 0 if v is None else _ld(v),
                                          y.data_ptr(), _ld(y), d_in, d_out, flags, _stream(stream)),
           "lora_fused_linear_noalloc")


NOALLOC_SCRATCH_BYTES = 8 << 20


def quantize_e4m3(x, q, s_x, stream=None) -> None:
    T, d = int(x.shape[0]), int(x.shape[1])
    _check(_lib.lora_quantize_e4m3(x.data_ptr(), T, d, _ld(x), q.data_ptr(), _ld(q), s_x.data_ptr(),
                                   _stream(stream)), "lora_quantize_e4m3")


def summary_from_words(words) -> Summary:
    """Summary struct from the first words of a segment buffer (host copy)."""
    s = Summary()
    for k, (n, _) in enumerate(Summary._fields_):
        setattr(s, n, int(words[k]))
    return s
