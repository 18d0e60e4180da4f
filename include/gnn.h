/*
 * gnn.h — C ABI of libgnn: GNN neighbourhood aggregation over a CSR adjacency
 * on one AMD Instinct MI355X (gfx950).
 *
 * Operations (Fomina et al., "On efficient scaling of GNNs via IO-aware layer
 * implementations"; section 2.2 names the three operator families, appendix D
 * gives the kernels):
 *   gnn_spmm         SpMM-based convolution Y = A_norm X      (section 2.2 (i), appendix D.4)
 *   gnn_spmm_block16 the same on 16x16 block-sparse tiles      (appendix D.3)
 *   gnn_reduce       segmented sum / mean / max / min          (section 2.2 (ii), appendix D.1)
 *   gnn_reduce_multi the four reductions in one pass           (section 2.2 (ii), appendix D.1)
 *   gnn_gatv2_fused  GATv2 attention, one pass, online softmax (section 2.2 (iii), appendix D.2)
 *   gnn_gt_fused     Graph Transformer attention, CSR or 16x16 block-sparse
 *                                                              (appendix D.2 and D.3)
 *   gnn_*_backward   gradients of SpMM, the reductions and both attention layers
 *                                                              (appendix D.1 and D.2, backward passes;
 *                                                               gnn_gt_backward_block16 on the tiles
 *                                                               of appendix D.3)
 *   gnn_reorder      degree-sort or RCM vertex reordering      (section 2.4; RCM as in
 *                    Tang et al., "A High-Throughput Solver for Marginalized Graph
 *                    Kernels on GPU", graph reordering section)
 *   gnn_dot_aggr     dot-aggr reordering micro-benchmark, feature- or
 *                    neighbour-parallel                        (Experiments, graph reordering,
 *                                                               Figure 1; appendix E.1)
 *
 * Conventions for every entry point:
 *   - Graph: CSR whose rows are DESTINATIONS: row i lists the sources j of the
 *     edges j -> i in col_idx[row_ptr[i] .. row_ptr[i+1]).  32-bit indices
 *     (appendix D.4 uses 32-bit CSR indices); nnz < 2^31.  Columns need not be
 *     sorted except where stated (gnn_reorder output is sorted; the WSB path
 *     needs no order either).  Duplicate entries count as separate edges.
 *   - All array pointers are DEVICE pointers, owned by the caller, unless a
 *     comment says otherwise.  The library never frees caller memory.
 *   - Dense features are row-major with a row stride (ld*, in elements).
 *   - Outputs are float32.  bf16 is an input format only; accumulation is
 *     float32.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) unless stated.  Validation happens on the host before any
 *     launch; on an error nothing is launched and no output is touched.
 *   - plan may be NULL in the calls that take one.  The call then builds a
 *     transient plan in stream order (stream-ordered allocations, degrees
 *     and one work item per row longer than 32 entries, 128 in the attention
 *     calls, rows longer than 1024 entries split into chunks of 1024, the
 *     counts kept on the device,
 *     released stream-ordered): no host synchronisation.  A plan built once
 *     by gnn_plan_create saves the per-call build and places the split
 *     threshold at a degree quantile.  Calls that need the 16x16 tiles
 *     (BLOCK16 modes, gnn_spmm_block16, gnn_gt_backward_block16) build a full
 *     transient plan instead, which synchronises `stream`.
 *   - Return value: a gnn_status.  gnn_last_error() gives a thread-local
 *     message for the last failing call on the calling thread.
 *   - Empty neighbourhoods: sum / mean / SpMM give 0; max / min give 0 with
 *     arg -1; attention gives out 0 and lse = -inf.
 *   - The CSR's contents are not read on the host.  With GNN_DEBUG_VALIDATE=1
 *     in the environment, gnn_plan_create (and so every call that builds a
 *     transient plan) and gnn_reorder first check them on the device:
 *     row_ptr[0] = 0, row_ptr[n_rows] = nnz, row_ptr never decreasing, every
 *     col_idx in [0, n_cols).  The check synchronises the stream and
 *     allocates; a violation returns INVALID_VALUE before any other kernel
 *     reads the CSR.  Without it, an invalid CSR is undefined behaviour.
 *     Calls given a plan then also run gnn_plan_verify.
 *   - Device memory: every allocation the library makes can fail with
 *     OUT_OF_MEMORY; the call then returns it with nothing left allocated
 *     (beyond the block cache below) and no output written beyond what
 *     finished kernels wrote.  Stream-ordered temporaries (those of calls
 *     without a plan, of plan builds and of reorders) are kept after the
 *     call in a per-device block cache of at most 8 GiB and reused by later
 *     calls, the reusing stream waiting on an event recorded where the block
 *     was last released; gnn_release_cached_memory gives them back.  Calls
 *     without a plan therefore allocate, record and wait on events: they are
 *     not for stream capture (gnn_reduce_multi_noalloc is).
 *     GNN_FAIL_ALLOC=k (or k:tag) in the environment makes the k-th allocation
 *     after the variable took that value fail that way, before any HIP call (a hook for
 *     testing the error paths).
 */
#ifndef GNN_H_
#define GNN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GNN_OK = 0,
  GNN_ERR_INVALID_VALUE = 1, /* null pointer, negative size, ld < width, bad enum */
  GNN_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head dim for a mode) */
  GNN_ERR_OUT_OF_MEMORY = 3, /* device allocation failed */
  GNN_ERR_DEVICE = 4,        /* a HIP call failed (launch error, earlier fault) */
  GNN_ERR_SIZE_OVERFLOW = 5, /* nnz >= 2^31, a size product overflows, or a
                                gathered row stride (ldx x element size) of
                                4 GB or more */
  GNN_ERR_PLAN_MISMATCH = 6  /* plan was built for another CSR */
} gnn_status;

typedef enum { GNN_F32 = 0, GNN_BF16 = 1 } gnn_dtype;

/* Edge weights of gnn_spmm (appendix D.4 names the modes none/left/right/both;
 * the GCN weight 1/sqrt(deg(i) deg(j)) is in section 2.2):
 *   NONE  w = 1                  LEFT  w = 1/deg_in(i)
 *   RIGHT w = 1/deg_out(j)       BOTH  w = 1/sqrt(deg_in(i) deg_out(j))
 * deg_in(i) = row length, deg_out(j) = number of entries equal to j, both
 * counting self loops present in the CSR; times edge_val[e] when given. */
typedef enum { GNN_NORM_NONE = 0, GNN_NORM_LEFT = 1, GNN_NORM_RIGHT = 2, GNN_NORM_BOTH = 3 } gnn_norm;

/* Segmented reductions (section 2.2 (ii), appendix D.1).  MEAN divides the
 * sum by deg_in.  MAX / MIN follow the IEEE total order on non-NaN values
 * (-0.0 < +0.0, the order of the order-preserving key of appendix D.1);
 * on equal values the smallest source index wins.  NaN inputs are not
 * supported. */
typedef enum { GNN_SUM = 0, GNN_MEAN = 1, GNN_MAX = 2, GNN_MIN = 3 } gnn_reduce_op;

/* Graph Transformer kernel choice: streaming CSR (appendix D.2) or the
 * 16x16 block-sparse matrix-core path on WSB tiles (appendix D.3), whose
 * sparse leftovers are processed by the CSR loop inside the same kernel.
 * AUTO picks from the plan's tiles (the pages' adaptive selection by local
 * density, appendix D.3): BLOCK16 when the plan has WSB tiles, the input
 * fits BLOCK16, at least half of the entries lie in dense tiles and those
 * average at least 32 entries per 16x16 tile (below that a tile's 32 gathered
 * K / V rows serve fewer entries than CSR's two rows per entry would); CSR
 * otherwise, and always without a plan with WSB tiles. */
typedef enum { GNN_GT_CSR = 0, GNN_GT_BLOCK16 = 1, GNN_GT_AUTO = 2 } gnn_gt_mode;

typedef enum { GNN_REORDER_DEGREE = 0, GNN_REORDER_RCM = 1 } gnn_reorder_kind;

/* dot-aggr mappings (Experiments, graph reordering): one wave per node, lanes
 * over features (sources walked one after another, coalesced row loads) or
 * lanes over sources (each lane walks its source's features: gathers). */
typedef enum { GNN_DOT_FEATURE = 0, GNN_DOT_NEIGHBOR = 1 } gnn_dot_map;
/* Per-lane load width of dot-aggr: 4-byte scalar or 16-byte vector loads. */
typedef enum { GNN_LOAD_SCALAR = 0, GNN_LOAD_VEC16 = 1 } gnn_dot_load;

typedef struct gnn_csr {
  int32_t n_rows;          /* destinations */
  int32_t n_cols;          /* sources (== n_rows for a square adjacency) */
  int64_t nnz;             /* == row_ptr[n_rows]; must be < 2^31 */
  const int32_t* row_ptr;  /* device [n_rows + 1], row_ptr[0] = 0, non-decreasing */
  const int32_t* col_idx;  /* device [nnz], each in [0, n_cols) */
  const float* edge_val;   /* device [nnz] or NULL (all ones); gnn_spmm only */
} gnn_csr;

/* Tuning knobs of a plan (appendix D.1 "degree threshold and autotuning
 * parameters"; appendix D.3 window and block sizes).  Zero-initialise and set
 * what you need; zero means the default. */
typedef struct gnn_plan_opts {
  float heavy_quantile;    /* gamma: rows above this degree quantile are split
                              into edge chunks (default 0.99; < 0 = never split) */
  int32_t light_max_deg;   /* rows up to this degree run one per 32-lane slot (default 32) */
  int32_t chunk_edges;     /* edges per chunk of a split row (default 1024) */
  int32_t build_wsb;       /* 1 = also build the 16x16 block-sparse tiles (GT BLOCK16) */
  int32_t wsb_min_nnz;     /* tau: tiles with fewer edges go to the CSR residual (default 8) */
  int32_t att_slot_max;    /* fused attention: rows of up to this many edges run one per slot,
                              longer ones one workgroup per row or chunk (default 128) */
  int32_t reserved[3];
} gnn_plan_opts;

/* Opaque plan: the per-graph cache of appendix D.4 made explicit.  It holds
 * the preprocessing products (degrees, normalisation scales, degree bins,
 * edge-chunk work items, WSB tiles) in library-owned device memory.  Bound to
 * one (n_rows, n_cols, nnz, row_ptr, col_idx); using it with another CSR is
 * GNN_ERR_PLAN_MISMATCH.  One call at a time per plan (its workspace is
 * shared). */
typedef struct gnn_plan gnn_plan;

/* Build a plan for `csr` (degree histogram, gamma-quantile threshold, bins,
 * chunk items; WSB tiles if opts->build_wsb).  opts may be NULL.  Launches on
 * `stream` and SYNCHRONISES it once (bin sizes are read back).  The CSR
 * arrays must stay alive and unchanged while the plan is used.
 * Errors: INVALID_VALUE, SIZE_OVERFLOW, OUT_OF_MEMORY, DEVICE. */
int gnn_plan_create(const gnn_csr* csr, const gnn_plan_opts* opts, void* stream, gnn_plan** out);

/* Free a plan and its device memory (the cache reset of appendix D.4).  Waits
 * for the plan's stream.  NULL is a no-op. */
int gnn_plan_destroy(gnn_plan* plan);

/* Check that a plan still matches its CSR's contents: the sizes and array
 * pointers must be those it was built for (as every call checks), and 64
 * evenly spaced entries of row_ptr (first and last included) and 64 of
 * col_idx, sampled on the device, must equal the samples taken when the
 * plan was built.  A cheap guard against a CSR rebuilt in place under a
 * cached plan (the failure mode of a pointer-keyed structure cache); an edit
 * of single entries between the samples goes unseen.  With
 * GNN_DEBUG_VALIDATE=1 every call that is given a plan runs this check
 * first (except gnn_reduce_multi_noalloc).  Synchronises `stream`;
 * allocates nothing.
 * Errors: INVALID_VALUE, PLAN_MISMATCH, DEVICE. */
int gnn_plan_verify(gnn_plan* plan, const gnn_csr* csr, void* stream);

/* Plan statistics for reports: counts[0] = light rows, [1] = medium rows,
 * [2] = heavy rows, [3] = chunk work items, [4] = degree threshold used,
 * [5] = WSB windows, [6] = WSB blocks (16x8), [7] = dense 16x16 tiles,
 * [8] = residual CSR edges.  Host memory, n >= 9. */
int gnn_plan_stats(const gnn_plan* plan, int64_t* counts, int32_t n);

/* Operation an autotuning run times. */
typedef enum { GNN_TUNE_SPMM = 0, GNN_TUNE_SUM = 1, GNN_TUNE_MULTI = 2 } gnn_tune_op;

/* Measured choice of a plan's degree-binning knobs for one aggregation
 * (appendix D.1 "degree threshold and autotuning parameters"): for every
 * candidate of heavy_quantile in {0.99, 0.999, -1 (no split)} x light_max_deg
 * in {16, 32} x chunk_edges in {256, 1024} (the defaults are one candidate),
 * build a plan, run the operation once untimed and `reps` times between HIP
 * events on `stream`, and keep the candidate of least mean time.  op:
 * GNN_TUNE_SPMM (gnn_spmm, norm NONE), GNN_TUNE_SUM (gnn_reduce SUM) or
 * GNN_TUNE_MULTI (gnn_reduce_multi with all six outputs).  X as in those
 * calls; reps in [1, 1000].  Outputs (host): *best receives the winning
 * options (other fields zero), *best_ms its mean time, *default_ms (nullable)
 * the defaults' mean time.  Allocates its output buffers and plans, frees
 * them, and synchronises `stream`.
 * Errors: INVALID_VALUE, SIZE_OVERFLOW, OUT_OF_MEMORY, DEVICE. */
int gnn_plan_autotune(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx, gnn_tune_op op,
                      int32_t reps, gnn_plan_opts* best, float* best_ms, float* default_ms, void* stream);

/* Operation an attention autotuning run times. */
typedef enum { GNN_TUNE_GATV2 = 0, GNN_TUNE_GT = 1 } gnn_tune_att_op;

/* Measured choice of the plan knobs of a fused attention layer on the
 * caller's graph and inputs (appendix D.1 autotuning parameters; appendix D.3
 * and section 5 pick CSR or block-sparse attention by local density).  The
 * CSR kernel is timed for heavy_quantile in {0.99, 0.999, -1 (no split)} x
 * chunk_edges in {256, 1024} x att_slot_max in {32, 128, 512}; for GT with
 * bf16 inputs, a square CSR and D in {32, 64, 128, 256} also the BLOCK16
 * kernel with wsb_min_nnz (tau) in {1, 8, 32}.  Each candidate: a plan, one
 * untimed call, `reps` timed calls between HIP events on `stream`; the one
 * of least mean time wins.  GATv2: q = xl, k = xr, att required, slope 0.2,
 * v unused; GT: q, k, v, scale 1/sqrt(D).  Shapes as gnn_gatv2_fused /
 * gnn_gt_fused.  Outputs (host): *best the winning options (pass them to
 * gnn_plan_create), *best_mode GNN_GT_CSR or GNN_GT_BLOCK16 (the mode to
 * call gnn_gt_fused with; CSR for GATv2), *best_ms its mean time,
 * *default_ms (nullable) the library defaults' (default plan, AUTO for GT).
 * Allocates its outputs and plans, frees them, synchronises `stream`.
 * Errors: INVALID_VALUE, UNSUPPORTED, SIZE_OVERFLOW, OUT_OF_MEMORY, DEVICE. */
int gnn_plan_autotune_attention(const gnn_csr* csr, gnn_tune_att_op op, const void* q, const void* k,
                                const void* v, gnn_dtype xtype, const float* att, int32_t H, int32_t D,
                                int32_t reps, gnn_plan_opts* best, gnn_gt_mode* best_mode, float* best_ms,
                                float* default_ms, void* stream);

/* Copy the plan's WSB layout (appendix D.3: windows of 16 rows, sorted
 * distinct source columns cut into blocks of 8 zero-padded columns, a 16x8
 * occupancy bitmap as two 64-bit words with bit r*8+c) into caller DEVICE
 * buffers: win_ptr [n_windows + 1], blk_col [n_blocks * 8],
 * blk_bits [n_blocks * 2].  Sizes from gnn_plan_stats.  Asynchronous.
 * Errors: INVALID_VALUE (null, or the plan has no WSB). */
int gnn_plan_wsb_export(const gnn_plan* plan, int32_t* win_ptr, int32_t* blk_col,
                        uint64_t* blk_bits, void* stream);

/* SpMM: Y[i, f] = sum_{e in row i} w_e * X[col_idx[e], f], f < F.
 * X: device [n_cols, ldx] of `xtype`; Y: device [n_rows, ldy] float32.
 * plan may be NULL (a transient one is built in stream order).
 * Errors: INVALID_VALUE (null, F <= 0, ldx < F, ldy < F, bad enum),
 * PLAN_MISMATCH, SIZE_OVERFLOW, OUT_OF_MEMORY, DEVICE. */
int gnn_spmm(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx, float* Y,
             int64_t ldy, gnn_norm norm, gnn_plan* plan, void* stream);

/* Block-sparse SpMM on the plan's WSB tiles (appendix D.3, the windowed
 * segmented bitmap format serving SpMM): the same product as gnn_spmm
 * (Y = A_norm X, norms as there), with each dense 16 x 16 tile of a 16-row
 * window multiplied by the 16 gathered feature rows of its columns on fp32
 * matrix cores (v_mfma_f32_16x16x4_f32: weights and features enter as fp32,
 * so products are fp32 products), and the plan's residual CSR added by a
 * plain loop.  For locally dense graphs, where a gathered row then serves
 * many entries of its window.  Needs a square CSR without edge values
 * (UNSUPPORTED otherwise) and a plan built with build_wsb = 1 (NULL builds a
 * transient one, WSB included); X device [n_cols, F] `xtype` with F and ldx
 * whole 16-byte chunks and X 16-byte aligned; Y device [n_rows, F] float32,
 * 16-byte aligned, ldy a multiple of 4.  Deterministic; the summation order
 * differs from gnn_spmm's.
 * Errors: INVALID_VALUE, UNSUPPORTED, PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_spmm_block16(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx, float* Y,
                     int64_t ldy, gnn_norm norm, gnn_plan* plan, void* stream);

/* Segmented reduction over each row's sources: Y[i, f] = op_j X[j, f].
 * arg: device [n_rows, lda = F] int32 or NULL; for MAX / MIN it receives the
 * winning source index (-1 for an empty row); it must be NULL for SUM / MEAN.
 * Light rows run one 32-lane slot per row, medium rows one workgroup per row,
 * heavy rows (above the gamma-quantile) are split into edge chunks merged by a
 * deterministic partials pass (SUM / MEAN) or by packed 64-bit (key, index)
 * atomics (MAX / MIN) followed by an unpack kernel (appendix D.1).
 * Errors as gnn_spmm. */
int gnn_reduce(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
               gnn_reduce_op op, float* Y, int64_t ldy, int32_t* arg, gnn_plan* plan, void* stream);

/* All four segmented reductions of section 2.2 (ii) in one pass: every
 * gathered neighbour row is read once and feeds the sum, mean, max and min
 * (with their source indices), the same IO-aware idea the fused attention
 * kernels apply (appendix D.2).  Definitions, tie rules and empty-row values
 * as gnn_reduce.  Y_sum, Y_mean, Y_max, Y_min: device [n_rows, ldy] float32,
 * each nullable (at least one required); arg_max / arg_min: device
 * [n_rows, F] int32 or NULL (each needs its value output).
 * Errors as gnn_reduce. */
int gnn_reduce_multi(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
                     float* Y_sum, float* Y_mean, float* Y_max, int32_t* arg_max, float* Y_min,
                     int32_t* arg_min, int64_t ldy, gnn_plan* plan, void* stream);

/* Bytes of device scratch memory that gnn_reduce_multi_noalloc may use. */
#define GNN_NOALLOC_SCRATCH_BYTES (32u << 20)

/* gnn_reduce_multi for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as gnn_reduce_multi, except:
 *   - plan is required (NULL is INVALID_VALUE): build it beforehand with
 *     gnn_plan_create, which does allocate;
 *   - the partial sums and packed (key, index) words of the plan's split rows
 *     live in a fixed library array of GNN_NOALLOC_SCRATCH_BYTES per GPU
 *     (held from the first call on that GPU until the process ends) instead
 *     of the plan's workspace; a plan and width F that need more
 *     (4 * F bytes per chunk of a split row, rounded up to 256, plus
 *     16 * F bytes per split row)
 *     return SIZE_OVERFLOW before any launch;
 *   - `stream` must belong to the calling thread's current device;
 *   - the call makes no device allocation, free or host synchronisation.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give wrong results;
 * calls ordered on one stream are safe.  The array keeps the last call's
 * contents; each call initialises what it reads. */
int gnn_reduce_multi_noalloc(const gnn_csr* csr, const void* X, gnn_dtype xtype, int32_t F, int64_t ldx,
                             float* Y_sum, float* Y_mean, float* Y_max, int32_t* arg_max, float* Y_min,
                             int32_t* arg_min, int64_t ldy, gnn_plan* plan, void* stream);

/* Fused GATv2 forward (section 2.2 (iii); appendix D.2 "fused CSR forward
 * (GATv2)"): for each destination i and head h,
 *   e_ij = sum_d att[h, d] * LeakyReLU(xl[i, h, d] + xr[j, h, d]),
 *   LeakyReLU(z) = z > 0 ? z : neg_slope * z,
 *   out[i, h, :] = sum_j softmax_j(e_ij) * xr[j, h, :],
 *   lse[i, h] = log sum_j exp(e_ij),
 * over the CSR row of i (add self loops to the CSR to include j = i).
 * xl: device [n_rows, H, D], xr: device [n_cols, H, D], both `xtype`, dense
 * (row stride H*D); att: device [H, D] float32; out: device [n_rows, H, D]
 * float32; lse: device [n_rows, H] float32 or NULL.  One pass with an online
 * softmax: no per-edge logits, weights or messages are written to memory.
 * Supported head shapes (appendix D.2 pairs head-dimension specialisations
 * with a fallback): xtype BF16 or F32, any H with H*D < 2^28, and a head of
 * D*sizeof(xtype) bytes that is either a multiple of 16 bytes up to 1 KB
 * (16-byte lane slices; lanes per head rounded up to a power of two; rows
 * wider than 64 lanes run as head groups) or at most 64 slices of the
 * widest of 8, 4 or 2 bytes dividing it (the generic mapping; every D <= 64
 * qualifies).  xl, xr, out 16-byte aligned.  plan may be NULL (a transient
 * one is built).
 * Errors: INVALID_VALUE, UNSUPPORTED, SIZE_OVERFLOW, PLAN_MISMATCH, DEVICE. */
int gnn_gatv2_fused(const gnn_csr* csr, const void* xl, const void* xr, gnn_dtype xtype,
                    const float* att, int32_t H, int32_t D, float neg_slope, float* out, float* lse,
                    gnn_plan* plan, void* stream);

/* Fused Graph Transformer forward (section 2.2 (iii): q_i = W_Q h_i,
 * k_j = W_K h_j, v_j = W_V h_j, e_ij = q_i . k_j / sqrt(D); appendix D.2 and
 * D.3): for each destination i and head h,
 *   out[i, h, :] = sum_j softmax_j(scale * <q[i,h,:], k[j,h,:]>) * v[j, h, :],
 *   lse[i, h] = log sum_j exp(scale * <q[i,h,:], k[j,h,:]>).
 * q: device [n_rows, H, D]; k, v: device [n_cols, H, D]; `xtype` BF16 (or F32
 * in CSR mode); scale <= 0 means 1/sqrt(D); out: device [n_rows, H, D]
 * float32; lse: device [n_rows, H] float32 or NULL.
 * GNN_GT_CSR: streaming online softmax; head shapes as for gnn_gatv2_fused
 * (a lane holds 32 bytes of rows of 1-2 KB whose heads fill a power of two
 * of such slices).
 * GNN_GT_BLOCK16: needs a plan built with build_wsb = 1, square CSR,
 * xtype BF16, D in {32, 64, 128, 256}, any H; dense 16x16 tiles run on bf16 MFMA with the
 * softmax weights rounded to bf16 for the P.V product; the residual edges of
 * sparse tiles run the CSR loop into the same per-row softmax state.
 * Errors: INVALID_VALUE, UNSUPPORTED, PLAN_MISMATCH, DEVICE. */
int gnn_gt_fused(const gnn_csr* csr, const void* q, const void* k, const void* v, gnn_dtype xtype,
                 int32_t H, int32_t D, float scale, gnn_gt_mode mode, float* out, float* lse,
                 gnn_plan* plan, void* stream);

/* Per-vertex projections that feed the attention layers (section 2.2 (iii):
 * GATv2 l_i = W_l h_i and r_j = W_r h_j; the Graph Transformer's q_i = W_Q h_i,
 * k_j = W_K h_j, v_j = W_V h_j; appendix D.2 consumes them precomputed per
 * vertex): for m < n_mat and every row i < n,
 *   Y[m][i, o] = sum_k X[i, k] * W[m][o, k],   o < f_out, k < f_in,
 * on bf16 matrix cores: bf16 inputs (products exact in float32), float32
 * accumulation, each output rounded to bf16 (round to nearest even).  One
 * pass over X serves all n_mat weights.
 * X: device bf16 [n, ldx], 16-byte aligned, ldx >= f_in a multiple of 8.
 * W: HOST array of n_mat (1 to 3) DEVICE pointers, each bf16 [f_out, f_in]
 * contiguous (one row per output feature, the nn.Linear layout), 16-byte
 * aligned.  Y: HOST array of n_mat DEVICE pointers, each bf16 [n, f_out]
 * contiguous, 16-byte aligned; as [n, H, D] with H * D = f_out they are the
 * dense per-vertex inputs of gnn_gatv2_fused and gnn_gt_fused.
 * Supported: f_in a multiple of 32 up to 512, f_out a multiple of 16.
 * Asynchronous on `stream`; no allocation.
 * Errors: INVALID_VALUE, UNSUPPORTED, SIZE_OVERFLOW, DEVICE. */
int gnn_project(const void* X, int32_t n, int32_t f_in, int64_t ldx, int32_t n_mat, const void* const* W,
                int32_t f_out, void* const* Y, void* stream);

/* ---------------------------------------------------------------------------
 * Backward passes.  Each takes the gradient of a forward output and returns
 * the gradients of its inputs, all float32, dense, owned by the caller and
 * fully overwritten.  They walk the transpose A^T, which the plan builds on
 * its first backward call (the entries of each transposed row keep their order
 * in A) and keeps; without a plan a transient one is built and freed.  A plan
 * serves one call at a time.
 * ------------------------------------------------------------------------- */

/* SpMM backward: dX = A_norm^T dY, i.e. dX[j, :] = sum over entries (i <- j)
 * of w_e dY[i, :], with the forward's weight w_e (norm and csr->edge_val as in
 * gnn_spmm).  dY: device [n_rows, F] float32, row stride ldy; dX: device
 * [n_cols, F] float32, row stride ldx (columns without entries get 0).
 * Deterministic.  Errors: INVALID_VALUE, PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_spmm_backward(const gnn_csr* csr, const float* dY, int32_t F, int64_t ldy, float* dX, int64_t ldx,
                      gnn_norm norm, gnn_plan* plan, void* stream);

/* Reduction backward (appendix D.1, backward pass).  SUM: dX = A^T dY;
 * MEAN: dX[j] = sum over entries (i <- j) of dY[i] / deg_in(i); MAX / MIN:
 * the gradient reaches only the source the forward selected,
 * dX[arg[i, f], f] += dY[i, f] (arg -1 passes nothing; values outside
 * [0, n_cols) are ignored), as a scatter with atomic adds, so when several
 * rows selected one source the order of its additions, and the last bits of
 * the sum, may differ between runs.  dY: device [n_rows, F] float32 (row
 * stride ldy); arg: device [n_rows, F] int32 as written by gnn_reduce /
 * gnn_reduce_multi (row stride F; required for MAX / MIN, ignored otherwise);
 * dX: device [n_cols, F] float32 (row stride ldx).
 * Errors: INVALID_VALUE, PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_reduce_backward(const gnn_csr* csr, gnn_reduce_op op, const float* dY, int32_t F, int64_t ldy,
                        const int32_t* arg, float* dX, int64_t ldx, gnn_plan* plan, void* stream);

/* GATv2 backward (appendix D.2, backward pass: weights recomputed as
 * alpha_ij = exp(e_ij - lse_i) from the forward's logsumexp; the per-(i, h)
 * statistic G = sum_j alpha_ij <dO_i, xr_j> = <dO_i, out_i>; a walk over A^T
 * for the right features; the attention-vector gradient reduced over nodes).
 * With z = xl_i + xr_j and de_ij = alpha_ij (<dO_i, xr_j> - G_i), per head:
 *   dxl[i] = sum_j de_ij att (.) LReLU'(z)
 *   dxr[j] = sum_i (alpha_ij dO_i + de_ij att (.) LReLU'(z))
 *   datt   = sum over entries of de_ij LReLU(z)
 * where LReLU'(z) = 1 for z > 0 and neg_slope otherwise.  Inputs as in
 * gnn_gatv2_fused, plus out [n_rows, H, D] and lse [n_rows, H] of the forward
 * (required) and dout [n_rows, H, D] float32.  Outputs (float32): dxl
 * [n_rows, H, D], dxr [n_cols, H, D], datt [H, D].  Two walks and an ordered
 * reduction; no atomics, deterministic.  The plan also keeps the per-(i, h)
 * statistic between the walks.  Shapes: any H with D * element size a
 * multiple of 16 bytes, at most 1 KB, and H * D < 2^28 (rows wider than 64
 * lane slices are cut into head groups; lanes per head are padded to a power
 * of two); all row tensors 16-byte aligned.
 * Errors: INVALID_VALUE, UNSUPPORTED (other head widths), SIZE_OVERFLOW,
 * PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_gatv2_backward(const gnn_csr* csr, const void* xl, const void* xr, gnn_dtype xtype, const float* att,
                       int32_t H, int32_t D, float neg_slope, const float* out, const float* lse,
                       const float* dout, float* dxl, float* dxr, float* datt, gnn_plan* plan, void* stream);

/* Graph Transformer backward (appendix D.2, backward pass: the cached
 * logsumexp and Delta[i, h] = <out[i, h, :], dout[i, h, :]>, weights
 * recomputed on the fly, a walk over A^T).  With e_ij = scale <q_i, k_j>,
 * alpha_ij = exp(e_ij - lse_i) and de_ij = alpha_ij (<dO_i, v_j> - Delta_i):
 *   dq[i] = scale sum_j de_ij k_j,  dk[j] = scale sum_i de_ij q_i,
 *   dv[j] = sum_i alpha_ij dO_i.
 * Inputs as in gnn_gt_fused (CSR layout; scale <= 0 means 1/sqrt(D)), plus
 * out [n_rows, H, D], lse [n_rows, H] of the forward (required) and dout
 * [n_rows, H, D] float32.  Outputs (float32): dq [n_rows, H, D], dk and dv
 * [n_cols, H, D].  Two walks, no atomics, deterministic.  Shapes as in
 * gnn_gatv2_backward; all row tensors 16-byte aligned.
 * Errors: INVALID_VALUE, UNSUPPORTED (other head widths), SIZE_OVERFLOW,
 * PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_gt_backward(const gnn_csr* csr, const void* q, const void* k, const void* v, gnn_dtype xtype, int32_t H,
                    int32_t D, float scale, const float* out, const float* lse, const float* dout, float* dq,
                    float* dk, float* dv, gnn_plan* plan, void* stream);

/* The same gradients as gnn_gt_backward computed on 16x16 block-sparse tiles
 * with bf16 matrix cores (appendix D.2 backward with cached statistics,
 * appendix D.3 block-sparse layout): a destination walk over the plan's
 * tiles of A gives dq (and Delta), a source walk over tiles of A^T gives dk
 * and dv; entries of sparse tiles run through the layouts' residual CSRs.
 * dO, alpha and dS are rounded to bf16 for the matrix cores, as alpha is in
 * the block-sparse forward: results are within the attention tolerance of
 * the exact gradients, not to fp32 rounding.  Square CSR, bf16 q, k, v only,
 * D in {32, 64, 128}, H*D*2 <= 2048; other arguments as in gnn_gt_backward.  The
 * plan must carry WSB tiles (NULL: a transient one is built); the tiles of
 * A^T are built on its first block-sparse backward call.  The plan keeps,
 * between the two walks, Delta [n_rows, H] float32 and dO rounded to bf16
 * [n_rows, H, D] (grown on demand, freed with the plan).
 * Errors: INVALID_VALUE, UNSUPPORTED, PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_gt_backward_block16(const gnn_csr* csr, const void* q, const void* k, const void* v, int32_t H,
                            int32_t D, float scale, const float* out, const float* lse, const float* dout,
                            float* dq, float* dk, float* dv, gnn_plan* plan, void* stream);

/* Vertex reordering of a square CSR (n_rows == n_cols).
 * DEGREE: perm sorts vertices by descending deg_in, ties by ascending id
 * (stable).  RCM: reverse Cuthill-McKee on the symmetrised pattern A u A^T
 * without self loops, each component started at its unvisited vertex of
 * smallest (degree, id), neighbours visited in increasing (degree, id).
 * perm: device [n_rows] int32, perm[new] = old (required).
 * row_ptr_out [n_rows + 1] and col_idx_out [nnz] (device, both or neither):
 * if given, receive the relabelled CSR P A P^T with each row's columns
 * sorted ascending.  Synchronises `stream` (RCM runs level by level) and
 * returns when the outputs are complete.  Temporaries: one stream-ordered
 * device allocation per call (RCM: about 64 bytes per CSR entry plus 40 per
 * vertex; degree sort with relabelling: about 16 per entry), freed before
 * return.
 * Errors: INVALID_VALUE (null, not square, one of the two outputs missing),
 * SIZE_OVERFLOW, OUT_OF_MEMORY, DEVICE. */
int gnn_reorder(const gnn_csr* csr, gnn_reorder_kind kind, int32_t* perm, int32_t* row_ptr_out,
                int32_t* col_idx_out, void* stream);

/* Gather rows: Xout[p, :] = X[perm[p], :] for p < n, F elements of `xtype`
 * per row, strides ldx / ldo (elements).  Used to carry features into a
 * reordered vertex numbering.  Errors: INVALID_VALUE, DEVICE. */
int gnn_permute_rows(const int32_t* perm, int32_t n, const void* X, gnn_dtype xtype, int32_t F,
                     int64_t ldx, void* Xout, int64_t ldo, void* stream);

/* dot-aggr, the cache-sensitive micro-benchmark with which the pages study
 * graph reordering (Experiments, graph reordering, Figure 1; appendix E.1,
 * Figure 2): for every node i of a square CSR,
 *   y[i] = sum over the sources j of row i of sum_d X[i, d] * X[j, d].
 * X: device float32 [n_rows, D], row stride ldx >= D (elements); y: device
 * float32 [n_rows].  map selects the wave-per-node mapping (gnn_dot_map),
 * load the per-lane load width (gnn_dot_load); every combination computes the
 * same sums, in a different order.  Rows longer than the plan's split
 * threshold run as the plan's edge chunks, one wave each, added in chunk order.
 * Supported: 1 <= D <= 1024; GNN_LOAD_VEC16 needs D and ldx multiples of 4
 * and X 16-byte aligned.  edge_val must be NULL (no weights).  plan may be
 * NULL (a transient plan is built in stream order).
 * Errors: INVALID_VALUE (null pointer, not square, bad D / ldx / enum, edge
 * values given, misaligned VEC16 input), UNSUPPORTED (D > 1024),
 * PLAN_MISMATCH, OUT_OF_MEMORY, DEVICE. */
int gnn_dot_aggr(const gnn_csr* csr, const float* X, int32_t D, int64_t ldx, gnn_dot_map map,
                 gnn_dot_load load, float* y, gnn_plan* plan, void* stream);

/* Plain streaming copy of n bytes (device to device), used to calibrate
 * bandwidth measurements and hardware counters.  Asynchronous. */
int gnn_copy_bytes(const void* src, void* dst, int64_t n, void* stream);

/* Gives the current device's cached stream-ordered blocks (see "Device
 * memory" above) back to the runtime.  Waits for the work that last used
 * each block; blocks that calls still in flight on the host hold are kept.
 * Errors: DEVICE. */
int gnn_release_cached_memory(void);

/* Text of a status code (static storage). */
const char* gnn_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
const char* gnn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GNN_H_ */
