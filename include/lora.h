/*
 * liblora -- batched heterogeneous-adapter ("multi-LoRA") linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * For a batch of T token rows, row i carrying adapter id a = ids[i]:
 *
 *     y_i = W0 x_i + [live_i] * s_a * B_a (A_a x_i)
 *
 * ("LLM-stack book 7.14 Multi-Tenant LoRA & Adapter Serving at Scale",
 * 7.14.1: the parenthesised LoRA forward and the batched-heterogeneous
 * problem; 7.14.2: stacked adapter pools indexed by a per-token id with -1
 * meaning base only, segment pointers after grouping by adapter, SGMV/BGMV).
 * A row is live when its id is >= 0 and its active flag is set; an inactive
 * row stands for a released adapter and gets the base output only
 * ("LoRazor", 3.2: released rows continue on the backbone-only path).
 *
 * The layer is split the way the pages split it ("LoRazor" 3.1.1 Eqs. 1-2;
 * "LoRAForge" 2, Multi-LoRA Serving; "EpiLoRA" 3.1, kernels K1 and K2):
 *   lora_build_segments / _dev   group the live rows by adapter
 *   lora_shrink                  v = A_a x          (rank-r down-projection)
 *   lora_build_shrink_dev        the device grouping and the shrink of one
 *                                batch, in one launch for small batches
 *   lora_expand                  y += s_a B_a v     (unfused up-projection)
 *   lora_fused_linear            y = W0 x (+ s_a B_a v in the epilogue),
 *                                bf16 / fp32 / fp8-e4m3 base
 *   lora_fused_linear_slices     the same for several projections of one x
 *                                (q / k / v, gate / up) in one launch
 *   lora_quantize_e4m3           per-token fp8 activation quantisation used
 *                                by the fp8 W8A8 base product
 *   lora_registry_* / lora_pool_install
 *                                which adapter occupies which pool slot, and
 *                                filling a slot ("LLM-stack book" 7.14.3-4)
 *   lora_stream_create_cu_masked streams on disjoint CU sets, to run the base
 *                                product and the adapter term side by side
 *                                (HALO 4) instead of fused
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.  Every buffer is owned by the caller.  "device" pointers are HIP
 *   device memory of the current device; "host" pointers are ordinary host
 *   memory.  The library allocates no device memory and keeps no device
 *   state; a registry handle owns only host memory.
 * Streams.  Every call is asynchronous on the given hipStream_t (passed as
 *   void*; NULL = the null stream).  No call synchronises the stream or reads
 *   device memory back to the host.  The device-side calls
 *   (lora_build_segments_dev, lora_build_shrink_dev, lora_shrink, lora_expand,
 *   lora_fused_linear, lora_fused_linear_slices) enqueue kernels only (work
 *   counters are cleared by a kernel, never by hipMemsetAsync), so a HIP graph
 *   can capture a step and replay it.  lora_build_segments groups the rows on
 *   the host when it is called, so a captured copy of it would replay that
 *   one batch: use the device builder under capture.
 * Errors.  Every call returns an int status (LORA_OK = 0).  All argument
 *   checks run before any work is enqueued; a call that returns an error has
 *   modified no output.  Device-side id validation (lora_build_segments_dev)
 *   reports through the device summary instead (see there).
 * Layouts.  Row-major throughout; ld_* are leading dimensions in elements.
 *   Adapter pool of one projection:
 *     A: [n_slots, r_cap, d_in]   row j of A_a is the j-th down direction
 *     B: [n_slots, d_out, r_cap]  row n of B_a holds channel n's r_cap weights
 *   Rank entries j >= slot_rank[a] are padding: never read by any kernel.
 *   v (shrink output): fp32 [T, ld_v], row p = p-th row of the grouped order,
 *     columns j < rank of that row's adapter; other entries are not written.
 * Alignment.  x, A, B, W, y and v must be 16-byte aligned; d_in, d_out and
 *   every ld must be multiples of 8 elements (16 for fp8 codes, 4 for fp32
 *   v) so that rows can be moved in 128-bit loads.  Otherwise LORA_E_ALIGN.
 */
#ifndef LORA_H
#define LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  LORA_OK = 0,
  LORA_E_ARG = 1,    /* null pointer, negative size, ld < width, bad enum     */
  LORA_E_ID = 2,     /* an adapter id < -1 or >= n_slots                      */
  LORA_E_RANK = 3,   /* r_cap < 1 or r_cap > LORA_MAX_RANK                    */
  LORA_E_DTYPE = 4,  /* unsupported dtype combination                         */
  LORA_E_ALIGN = 5,  /* pointer or leading dimension not 16-byte aligned      */
  LORA_E_HIP = 6,    /* a HIP launch or copy failed (see lora_last_error)     */
  LORA_E_SIZE = 7    /* a size beyond a documented limit, or too small a
                        workspace / segment buffer                            */
};

/* ---- element types --------------------------------------------------- */
enum { LORA_F32 = 0, LORA_BF16 = 1, LORA_FP8_E4M3 = 2 };

/* ---- limits ---------------------------------------------------------- */
#define LORA_MAX_RANK 128          /* largest pool rank capacity r_cap        */
#define LORA_DEV_MAX_SLOTS 8192    /* n_slots limit of lora_build_segments_dev */
#define LORA_TILE_SMALL 16         /* row-tile height of the decode kernels   */
#define LORA_TILE_LARGE 64         /* row-tile height of the prefill kernels  */

/* ---- launch sizing (LoRazor 3.1) -------------------------------------- */
enum {
  /* grid = exactly the row tiles that hold live rows (sum_a ceil(m_a/BM))
     times the column blocks; needs the host summary.  In EXACT and
     BUCKETED the host summary sizes the grid only: the kernels take the
     work itself from the device segment buffer and stride over it, so a
     summary that does not match the buffer (another batch of the same T)
     costs time, never rows.                                               */
  LORA_LAUNCH_EXACT = 0,
  /* fixed grid that strides over the device-side tile count; needs no host
     summary, so the launch shape does not change from batch to batch.    */
  LORA_LAUNCH_PERSISTENT = 1,
  /* LoRazor's shared row bound (3.1.2, Eqs. 7-8): L = min(T, n_slots)
     adapter slots x ceil(R/BM) row tiles, R from the host summary; blocks
     without rows exit.                                                    */
  LORA_LAUNCH_BUCKETED = 2,
  /* the full-batch bound the pages start from (3.1.1): L x ceil(T/BM) row
     tiles per launch, blocks without rows exit.  For comparison only.     */
  LORA_LAUNCH_FULL_BATCH = 3
};

/* ---- fused-linear flags ---------------------------------------------- */
#define LORA_FLAG_ACT_QUANT_E4M3 0x1  /* fp8 base: quantise x per token
                                         (W8A8); default is W8A16           */
#define LORA_FLAG_SHRINK_IN_LAUNCH 0x2 /* lora_fused_linear computes v itself,
                                         in the same launch (see there)     */

/* Adapter pool of one projection (device pointers). */
typedef struct {
  const void* A;              /* [n_slots, r_cap, d_in], dtype               */
  const void* B;              /* [n_slots, d_out, r_cap], dtype              */
  const int32_t* slot_rank;   /* device int32 [n_slots], 0 <= rank <= r_cap  */
  const float* slot_scale;    /* device fp32 [n_slots]: s_a = alpha/r (or any
                                 caller-chosen scale; the kernels never see
                                 alpha or r separately)                      */
  int32_t dtype;              /* LORA_F32 or LORA_BF16                       */
  int32_t n_slots;
  int32_t r_cap;              /* 1 .. LORA_MAX_RANK                          */
  int32_t d_in;
  int32_t d_out;
} lora_pool_t;

/* Base weight of one projection (device pointers). */
typedef struct {
  const void* W;              /* [d_out, ld_w]: fp32 / bf16 values, or e4m3
                                 codes (one byte each)                        */
  const float* w_scale;       /* fp8 only: device fp32 [d_out], W0deq[n, k] =
                                 e4m3(W[n, k]) * w_scale[n]; else NULL       */
  int32_t dtype;              /* LORA_F32, LORA_BF16 or LORA_FP8_E4M3        */
  int32_t ld_w;
} lora_base_t;

/* Host copy of a segment build's summary. */
typedef struct {
  int32_t n_active;     /* live rows                                         */
  int32_t n_segments;   /* S = distinct adapters among live rows             */
  int32_t m_max;        /* largest group                                     */
  int32_t row_bound;    /* R = min{r in {16*2^k < T} U {T} : r >= m_max}
                           (LoRazor 3.1.4, Eqs. 7-8); 0 if no live row       */
  int32_t n_tiles_small;/* sum_a ceil(m_a / LORA_TILE_SMALL)                 */
  int32_t n_tiles_large;/* sum_a ceil(m_a / LORA_TILE_LARGE)                 */
  int32_t T;            /* rows the build covered                            */
  int32_t error;        /* device builder only: LORA_E_ID if an id was out of
                           range (outputs then undefined), else 0            */
} lora_summary_t;

/*
 * Segment buffer.  One caller-allocated device buffer of
 * lora_segment_words(T) int32 words (T = the row capacity), laid out as
 *   [0, 16)                       summary words (lora_summary_t order)
 *   perm        [T]               live rows grouped by adapter, then the
 *                                 non-live rows in increasing order
 *   pos_seg     [T]               segment index of each grouped position,
 *                                 -1 for positions >= n_active
 *   seg_start   [T + 1]           start of each segment in perm, plus the end
 *   seg_adapter [T]               adapter id of each segment
 *   tiles_small [2T]              (first position, segment) per 16-row tile
 *   tiles_large [2T]              (first position, segment) per 64-row tile
 * Only the first n_active / S / S+1 / n_tiles entries are meaningful.
 * There is no per-segment rank array: every kernel reads the rank of segment
 * s as slot_rank[seg_adapter[s]] from the pool's device metadata when it
 * runs, so one build stays valid when a slot is refilled with an adapter of
 * another rank ("LoRAForge" 4.1 and 5: each slot's retained rank lives in
 * device metadata at a fixed address).
 */
size_t lora_segment_words(int32_t T);

/*
 * Group token rows by adapter ("LLM-stack book" 7.14.2, the segment pointers
 * seg_start / seg_adapter of the sorted batch; "LoRazor" 3.1.1, the
 * adapter-grouped row-index array I_a with m_a = |I_a|).
 *
 *   ids      host int32 [T]: adapter id per row, -1 = no adapter
 *   active   host uint8 [T] or NULL (NULL = every row with id >= 0 is live)
 *   n_slots  the pool's slot count, the only part of a pool the grouping
 *            needs (ids are checked against it; ranks are not read here)
 *   order    0: segments by ascending adapter id (canonical);
 *            1: segments in order of first appearance in the batch
 *            (the book's printed example).  Rows keep batch order inside a
 *            segment in both cases.
 *   staging  host int32 buffer of lora_segment_words(T) words, written by the
 *            call and copied from asynchronously: it must stay untouched until
 *            the stream has passed this call (pinned memory lets the copy run
 *            asynchronously; pageable memory works but copies synchronously).
 *   seg      device segment buffer of lora_segment_words(T) words.
 *   summary  host: receives the summary immediately (before the copy lands),
 *            so the next launches can be sized exactly on the host.
 * Errors: LORA_E_ARG, LORA_E_ID (an id < -1 or >= n_slots; nothing copied).
 */
int lora_build_segments(const int32_t* ids, const uint8_t* active, int32_t T, int32_t n_slots,
                        int32_t order, int32_t* staging, int32_t* seg, lora_summary_t* summary,
                        void* stream);

/* The same grouping computed on the host only, into a host buffer of
 * lora_segment_words(T) words with the layout above; no HIP call. */
int lora_plan_segments(const int32_t* ids, const uint8_t* active, int32_t T, int32_t n_slots,
                       int32_t order, int32_t* plan, lora_summary_t* summary);

/*
 * Device variant: ids (device int32 [T]) and active (device uint8 [T] or
 * NULL) are read on the GPU by one workgroup; the summary is written to the
 * first words of `seg` only.  n_slots <= LORA_DEV_MAX_SLOTS.  An id out of
 * range sets summary.error = LORA_E_ID on the device and leaves the other
 * outputs undefined; kernels that consume such a segment buffer treat it as
 * having no live rows.
 */
int lora_build_segments_dev(const int32_t* ids, const uint8_t* active, int32_t T, int32_t n_slots,
                            int32_t order, int32_t* seg, void* stream);

/*
 * Shrink ("LoRazor" 3.1.1 Eq. 1; "LoRAForge" 5, rank-aware shrink):
 *   v[p, j] = sum_k x[perm[p], k] * A_a[j, k]   for p < n_active, j < r_a,
 * with a the adapter of p's segment, accumulated in fp32.
 *   x      device [T, ld_x], pool dtype (fp32 or bf16)
 *   v      device fp32 [T, ld_v], ld_v >= r_cap
 *   summary  host summary of the segment build, or NULL when `launch` is
 *            LORA_LAUNCH_PERSISTENT or LORA_LAUNCH_FULL_BATCH
 * Work items are (row tile of <= LORA_TILE_SMALL rows of one segment, one
 * or more blocks of up to 16 rank directions), each block a 16 x 16 MFMA
 * tile with operands streamed from global memory; long batches of mostly
 * full tiles put several blocks in one item so that they share the tile's x
 * rows; blocks past the adapter's rank do no work.
 * Deterministic: fixed-order reductions, no atomics.
 */
int lora_shrink(const lora_pool_t* pool, const int32_t* seg, int32_t T, const lora_summary_t* summary,
                const void* x, int32_t ld_x, float* v, int32_t ld_v, int32_t launch, void* stream);

/*
 * Device segment build followed by the shrink, for one batch: the segment
 * buffer of lora_build_segments_dev(ids, active, T, pool->n_slots, order,
 * seg), bit for bit, and the v of lora_shrink(pool, seg, T, NULL, x, ld_x, v,
 * ld_v, LORA_LAUNCH_PERSISTENT) up to fp32 rounding (the one-launch kernel
 * adds the k chunks in another fixed order; it is deterministic, and equal
 * to the two launches for larger batches) ("LLM-stack book" 7.14.2, the sorted
 * batch and its segment pointers; "LoRazor" 3.1.1 Eq. 1).  Batches of at most
 * 256 rows over pools of at most 1024 slots run as one launch in which every
 * workgroup groups the rows into its own LDS copy of the segment buffer and
 * takes its shrink items from it (workgroup 0 writes the buffer to `seg`);
 * larger ones run the two launches.
 *   ids, active, order, seg: as lora_build_segments_dev (device memory)
 *   pool, x, ld_x, v, ld_v:  as lora_shrink
 * Errors: LORA_E_ARG, LORA_E_SIZE (n_slots > LORA_DEV_MAX_SLOTS), LORA_E_RANK,
 * LORA_E_DTYPE, LORA_E_ALIGN, LORA_E_HIP; every check runs before any launch.
 * An id out of range is reported in the segment buffer's summary, as by the
 * device builder, and v is then not written.
 */
int lora_build_shrink_dev(const int32_t* ids, const uint8_t* active, int32_t T, int32_t order,
                          const lora_pool_t* pool, int32_t* seg, const void* x, int32_t ld_x, float* v, int32_t ld_v,
                          void* stream);

/*
 * Expand ("LoRazor" 3.1.1 Eq. 2; "LoRAForge" 5, RowExpand):
 *   y[perm[p], n] += s_a * sum_{j < r_a} v[p, j] * B_a[n, j]   for p < n_active
 * y is updated in place: fp32, or bf16 rounded once (nearest even) from
 * fp32(y) + the fp32 update.  Rows that are not live are not touched.
 */
int lora_expand(const lora_pool_t* pool, const int32_t* seg, int32_t T, const lora_summary_t* summary,
                const float* v, int32_t ld_v, void* y, int32_t y_dtype, int32_t ld_y, int32_t launch,
                void* stream);

/*
 * Fused linear ("EpiLoRA" 3.1 and Fig. 10, kernel K2: a GEMM over
 * adapter-sorted rows whose epilogue applies the base scales and adds each
 * adapter group's h B^T before writing the rows back in token order):
 *   y[i, n] = epi( sum_k x[i, k] * W0[n, k] )
 *   epi(acc) = acc * w_scale[n] [* s_x[i] for W8A8]
 *              + [live_i] * s_a * sum_{j < r_a} v[p(i), j] * B_a[n, j]
 * for every row i < T (p(i) = the grouped position of row i).
 *   base     fp32 base with fp32 pool/x/y; bf16 base with bf16 pool/x/y;
 *            fp8-e4m3 base with bf16 pool/x/y (W8A16: codes widened to bf16,
 *            bf16 MFMA; W8A8 with LORA_FLAG_ACT_QUANT_E4M3: x quantised per
 *            token into the workspace, fp8 MFMA).
 *   pool, v  NULL, NULL for the base product alone (seg may then be NULL:
 *            rows in batch order).
 *   workspace / workspace_bytes: device scratch, 256-byte aligned, of at
 *            least lora_fused_workspace_bytes(T, d_in, d_out, base->dtype,
 *            flags) bytes (NULL and 0 when that is 0).  It holds the W8A8
 *            codes and scales; for batches whose output has too few tiles
 *            to fill the GPU, the partial tiles of a split-k schedule with
 *            one counter per tile; for outputs of more tiles than the GPU
 *            has CUs, 64 bytes of counters from which one workgroup per CU
 *            claims tiles.  Counters are cleared on the stream before use.
 *            Calls that share a workspace must be ordered on one stream.
 *            LORA_E_SIZE if it is missing or too small.
 * y must not alias x.  Results do not depend on the schedule's timing: split
 * partial tiles are added in a fixed order.
 *
 * LORA_FLAG_SHRINK_IN_LAUNCH ("EpiLoRA" 3.1, the decode path and Fig. 1c: the
 * down-projection runs while the GEMM streams its weights, and only the
 * epilogue needs its result): v becomes an output, v = A_a x for the live
 * rows, computed in the same launch as the product.  The first workgroups of
 * the grid take shrink items (a row tile of one segment and a block of rank
 * directions, as lora_shrink's) from a counter in the workspace; a tile that
 * reaches its epilogue first runs any items still unclaimed, then waits until
 * every item is done and reads v, so progress never depends on which
 * workgroups the hardware schedules.  Needs a pool and a bf16 or fp8 base
 * (not fp32); the shrink reads the unquantised x (W8A8 included).  v equals
 * lora_shrink's up to fp32 rounding (the k chunks are added in another fixed
 * order) and is deterministic.  Shapes the pipelined kernel does not take run
 * lora_shrink and then the fused product, two launches, with the same result.
 */
int lora_fused_linear(const lora_base_t* base, const lora_pool_t* pool, const int32_t* seg, int32_t T,
                      const void* x, int32_t ld_x, const float* v, int32_t ld_v, void* y, int32_t ld_y,
                      int32_t d_in, int32_t d_out, int32_t flags, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace bytes lora_fused_linear needs for this call shape, whatever the
 * pool: the largest need over every rank capacity 1 .. LORA_MAX_RANK and over
 * the base product alone (the schedule depends on the pool's capacity, whose
 * rank-r v rows and B slices share the LDS with the main loop's ring).  This
 * stands in for a generic workspace query taking the call's descriptors: the
 * fused calls are the only ones that need a workspace. */
size_t lora_fused_workspace_bytes(int32_t T, int32_t d_in, int32_t d_out, int32_t base_dtype, int32_t flags);
/* The exact need of a call with a pool of rank capacity r_cap (0 = no pool). */
size_t lora_fused_workspace_bytes_rcap(int32_t T, int32_t d_in, int32_t d_out, int32_t base_dtype, int32_t flags,
                                       int32_t r_cap);

/*
 * lora_fused_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, the same kernels
 * and the same results as lora_fused_linear, with the scratch it needs (W8A8
 * codes and scales, split-k partial tiles, tile counters) taken from a
 * static device array of LORA_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends.  The call allocates and
 * frees nothing.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and give undefined
 * results; order them on one stream.  Whatever must start at zero is cleared
 * by a kernel on `stream` before use.  Errors: as lora_fused_linear, and
 * LORA_E_SIZE (text in lora_last_error) when the call needs more scratch
 * than the array holds (lora_fused_workspace_bytes_rcap gives the need).
 */
#define LORA_NOALLOC_SCRATCH_BYTES (8u << 20)
int lora_fused_linear_noalloc(const lora_base_t* base, const lora_pool_t* pool, const int32_t* seg, int32_t T,
                              const void* x, int32_t ld_x, const float* v, int32_t ld_v, void* y, int32_t ld_y,
                              int32_t d_in, int32_t d_out, int32_t flags, void* stream);

/*
 * Fused linear over several output slices of one input in one launch
 * ("LoRAForge" 4: the slices of a layer's fused projections, such as q / k /
 * v or gate / up, each with its own weights and adapters).  Slice s is
 * exactly lora_fused_linear with bases[s], pools[s], v[s], ld_v[s], y[s],
 * ld_y[s] and d_out[s]; x, ld_x, seg, T, d_in and flags are shared:
 *   y_s[i, n] = epi_s( sum_k x[i, k] * W0_s[n, k] )
 *               + [live_i] * s_a * sum_{j < r_a} v_s[p(i), j] * B_{s,a}[n, j]
 * The slices' column tiles share one grid, so narrow slices (k / v of a
 * grouped-query layer) still fill the GPU.
 *   bases    n_slices base descriptors of one dtype
 *   pools, v NULL, NULL for the base products alone; else n_slices pools over
 *            the same slot ids (seg is shared) and their v buffers
 *   y        n_slices distinct outputs
 *   workspace at least lora_fused_slices_workspace_bytes(n_slices, T, d_in,
 *            d_out, bases[0].dtype, flags) bytes, 256-byte aligned.
 * Up to 4 slices share a launch; more, or shapes the pipelined kernel does
 * not take, run slice by slice on the stream.  A slice's tile shape can
 * differ from a lone call's, so results agree with lora_fused_linear's to
 * the output's rounding, not bit for bit.  Errors: as lora_fused_linear,
 * for any slice; LORA_E_DTYPE if the base dtypes differ.
 */
int lora_fused_linear_slices(int32_t n_slices, const lora_base_t* bases, const lora_pool_t* pools,
                             const int32_t* seg, int32_t T, const void* x, int32_t ld_x, int32_t d_in,
                             const int32_t* d_out, const float* const* v, const int32_t* ld_v, void* const* y,
                             const int32_t* ld_y, int32_t flags, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes lora_fused_linear_slices needs for this call shape. */
size_t lora_fused_slices_workspace_bytes(int32_t n_slices, int32_t T, int32_t d_in, const int32_t* d_out,
                                         int32_t base_dtype, int32_t flags);

/* ---- adapter residency ------------------------------------------------ */
/*
 * A pool holds n_slots adapters at a time; an adapter registry decides which
 * adapter occupies which slot ("LLM-stack book" 7.14.4: a registry maps an
 * adapter to its slot, counts the batches in flight that use it, and when a
 * new adapter needs a slot evicts a resident one that no batch uses, by
 * least-recent use, or by fewest uses in the LFU variant).  The registry is
 * host bookkeeping (host memory owned by the handle, not thread-safe: one
 * host thread per registry); lora_pool_install moves the weights.
 */
#define LORA_EVICT_LRU 0
#define LORA_EVICT_LFU 1
typedef struct lora_registry lora_registry_t;

/* New registry over slots 0 .. n_slots-1, all free.  Errors: LORA_E_ARG. */
int lora_registry_create(int32_t n_slots, int32_t policy, lora_registry_t** out);
void lora_registry_destroy(lora_registry_t* registry);

/* One batch's use of adapter `key` (any id >= 0 the caller chooses).
 * Resident: *slot is its slot, *needs_install = 0.  Not resident: it takes
 * the lowest free slot, else evicts the policy's victim among slots whose
 * use count is zero; *needs_install = 1 and the caller must fill the slot
 * (lora_pool_install) before kernels read it.  Either way the slot's use
 * count goes up by one.  LORA_E_SIZE if every slot holds an adapter in use
 * (nothing changes).  LRU victim: oldest last acquire; LFU: fewest acquires
 * over the registry's life, ties by oldest last acquire. */
int lora_registry_acquire(lora_registry_t* registry, int64_t key, int32_t* slot, int32_t* needs_install);
/* End of one use (the batch's kernels are done with the slot).  LORA_E_ARG
 * if `key` is not resident or has no use to end. */
int lora_registry_release(lora_registry_t* registry, int64_t key);
/* *slot = the slot of `key`, or -1 if it is not resident. */
int lora_registry_lookup(const lora_registry_t* registry, int64_t key, int32_t* slot);
/* out4 = {hits, misses, evictions, resident adapters}. */
int lora_registry_stats(const lora_registry_t* registry, int64_t* out4);

/*
 * Fill pool slot `slot` with one adapter ("LLM-stack book" 7.14.3): A
 * [rank, d_in] and B [d_out, rank] in the pool dtype, host or device memory,
 * row-major and contiguous; rank 0 .. r_cap; scale = s_a.  Asynchronous on
 * `stream`: host sources should be pinned (hipHostMalloc) for the copy to be
 * asynchronous and must stay untouched until the stream has passed the call.
 * The slot's rank and scale are written by a kernel on the same stream, after
 * the weights, so a graph can capture the call.  Kernels that read the slot
 * must be ordered after it (same stream, or an event).  Entries past `rank`
 * are left as they were (kernels never read them).
 * Errors: as the pool checks of lora_shrink; LORA_E_ARG for a slot or rank
 * out of range or a NULL source with rank > 0.
 */
int lora_pool_install(const lora_pool_t* pool, int32_t slot, const void* A, const void* B, int32_t rank,
                      float scale, void* stream);

/* ---- concurrent base and adapter work ---------------------------------- */
/*
 * "From Overloaded to Guaranteed" (HALO), 4.1-4.2 and Fig. 6-7: the base layer
 * and the LoRA layer of a decode step run at the same time on disjoint sets of
 * compute units, the split chosen by measuring.  Here a split is two HIP
 * streams restricted to disjoint CU masks: the base product alone
 * (lora_fused_linear without a pool) on one, lora_shrink on the other, then
 * lora_expand adds the adapter term once the base product is in y.  The fused
 * call does the same work in one launch; these calls exist to measure that
 * alternative.
 */
/* *n_cus = compute units of the current device. */
int lora_device_cu_count(int32_t* n_cus);
/* New stream on the current device whose kernels run only on the CUs whose bit
 * is set: bit (i mod 32) of cu_mask[i / 32] is logical CU i, in the numbering of
 * the HIP runtime's CU masks; n_words 32-bit words are read.  Default priority.
 * The caller owns the stream (lora_stream_destroy).  Errors: LORA_E_ARG for a
 * NULL pointer, n_words <= 0 or an all-zero mask (checked before any HIP call);
 * LORA_E_HIP if the runtime refuses the mask or has no hardware queue left for
 * it (each CU-masked stream takes a queue of its own; a one-CU mask has been
 * refused on MI355X). */
int lora_stream_create_cu_masked(const uint32_t* cu_mask, int32_t n_words, void** stream);
/* Destroy a stream made by lora_stream_create_cu_masked.  LORA_E_ARG if NULL. */
int lora_stream_destroy(void* stream);

/*
 * Per-token activation quantisation for the W8A8 base product ("EpiLoRA" 2
 * and Fig. 4: x is quantised once per token, x -> (x_q, s_x)):
 *   s_x[i] = amax_k |x[i, k]| / 448 in fp32 (1 for an all-zero row)
 *   q[i, k] = e4m3( x[i, k] / s_x[i] ), fp32 division, round to nearest
 *             even, saturating to +-448
 *   x  device bf16 [T, ld_x]; q device uint8 [T, ld_q]; s_x device fp32 [T]
 * Rows must be finite: a NaN or an infinity leaves its row's codes and s_x
 * unspecified.  Errors (checked before any launch): LORA_E_ARG for negative
 * sizes, NULL pointers with T > 0, or ld_x / ld_q < d; LORA_E_ALIGN unless
 * d % 16 == 0, ld_x % 8 == 0, ld_q % 16 == 0 and x and q are 16-byte aligned.
 */
int lora_quantize_e4m3(const void* x, int32_t T, int32_t d, int32_t ld_x, uint8_t* q, int32_t ld_q,
                       float* s_x, void* stream);

/* Static description of a status code. */
const char* lora_status_string(int status);
/* Text of the last LORA_E_HIP error on the calling thread ("" if none). */
const char* lora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H */
