"""Plain, slow, fp64 CPU oracle for the batched multi-adapter linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library
(``adapter_gemm_amd``): it has its own bf16/fp8 decoders, its own segment
grouping and its own launch-geometry formulas, written from the pages:

* "LLM-stack book 7.14 Multi-Tenant LoRA & Adapter Serving at Scale"
  (7.14.1 the LoRA forward and the batched-heterogeneous problem, 7.14.2 the
  SGMV/BGMV data layout and segment pointers, 7.14.10 the toy layer);
* "LoRazor: Trimming Adapter Execution for Efficient Multi-LoRA Serving"
  (3.1.1 Eqs. 1-2 shrink/expand, 3.1.2 Eq. 3, 3.1.3 Eqs. 4-6, 3.1.4 Eqs. 7-8
  and Algorithm 1, 3.2 adapter release);
* "EpiLoRA: Fusing Many LoRA Adapters into Low-Precision GEMMs" (2, Fig. 4:
  the per-token quantised FP8 projection y = (x_q W_q^T) s_x s_w; 3.1 K1/K2);
* the same book's 7.14.3-7.14.4 (hot-swapping, the adapter registry and its
  LRU / LFU eviction) for the slot residency rules;
* "LoRAForge" (2 Multi-LoRA Serving: Z = X A^T then the expand; 4.1 retained
  ranks below the pool capacity).

Each function is pinned in ``tests/test_oracle_*.py`` against something
other than itself (closed forms, invariants, a library routine, brute force,
the pages' printed segment example).
"""
from .numerics import decode_bf16, decode_e4m3, encode_e4m3, E4M3_MAX
from .layer import (live_rows, base_output, shrink_rows, lora_delta, lora_delta_per_row,
                     lora_delta_gathered, linear, merged_linear, act_quant_e4m3,
                     linear_w8a8)
from .segments import build_segments, row_tiles
from .launch import (row_bound_set, row_bound, tiles_full_batch, tiles_shared_bound,
                     tiles_two_class, tiles_exact, class_separation_enabled)
from .residency import Residency

__all__ = [
    "decode_bf16", "decode_e4m3", "encode_e4m3", "E4M3_MAX",
    "live_rows", "base_output", "shrink_rows", "lora_delta", "lora_delta_per_row",
    "lora_delta_gathered", "linear", "merged_linear", "act_quant_e4m3", "linear_w8a8",
    "build_segments", "row_tiles",
    "row_bound_set", "row_bound", "tiles_full_batch", "tiles_shared_bound", "tiles_two_class",
    "tiles_exact", "class_separation_enabled", "Residency",
]
