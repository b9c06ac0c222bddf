/*
 * apmoe.h -- C ABI of libapmoe, the any-precision MoE expert layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer follows "PagedWeight: Efficient MoE LLM Serving with Dynamic
 * Quality-Aware Weight Quantization" (arXiv:2607.16184):
 *   - Section 3.1: a linear-block i = (layer, expert, u), u in {gate_up, down},
 *     is the unit of quantisation; its weight page table row holds the committed
 *     bitwidth q_i used by inference, the desired bitwidth d_i, and per-plane
 *     residency (GPU-resident, CPU-resident, in transfer).
 *   - Section 3 and the Figure 3 caption: weights are Any-Precision overlaid
 *     bit-planes (a b-bit weight uses a subset of the planes) plus a LUT of
 *     bitwidth-specific centroids.
 *   - Section 3.1 (offload/reload) and Section 3.3: q_i is lowered before pages
 *     leave the GPU and raised only after they are resident again, and changes
 *     are committed only at safe boundaries.
 *   - Section 3.3 ("Fused Mixed-Precision MoE Kernel"): routing, expert
 *     activation, down projection and output accumulation, each gate_up / down
 *     module at its own bitwidth.
 *
 * Format conventions (readings of the paper where it is silent):
 *   - 8 parent planes.  Plane p holds bit (7 - p) of the 8-bit parent code, so a
 *     q-bit block reads planes 0..q-1 and its code is the parent code >> (8 - q).
 *   - Canonical plane layout: plane p of an n x k block is uint32 [n][k/32]; bit j
 *     of word w is column 32*w + j.
 *   - Device plane layout read by the kernels ("tiled"): apmoe_tile_planes
 *     rearranges the canonical words of each plane into 32-row x 128-column tiles
 *     of 512 bytes, so one wave reads whole contiguous cache lines.
 *   - The LUT is per output row: level b is fp16 [n][2^b], entry [row][code].
 *   - gate_up is [2F x H] with rows [0, F) the gate and [F, 2F) the up
 *     projection; down is [H x F].  Activation is SiLU(gate) * up.
 *
 * Conventions of every call:
 *   - Every function returns an apmoe_status; no exception crosses the ABI and
 *     the library never aborts.  Arguments are validated on the host before
 *     anything is enqueued; a failed call enqueues nothing and changes nothing.
 *     apmoe_last_error() gives a thread-local message for the last failure.
 *   - Tensor arguments are device pointers owned by the caller, 16-byte
 *     aligned, row-major and dense.  The library allocates device memory only in
 *     apmoe_table_commit (the device table, once per table) and never on the
 *     compute calls.
 *   - Compute calls are asynchronous on the HIP stream passed as void*
 *     (NULL = the default stream) and never synchronise the host.
 *   - A context is bound to one device and is not thread-safe; use one per
 *     host thread.
 */
#ifndef APMOE_H
#define APMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t apmoe_status;

#define APMOE_OK 0
#define APMOE_INVALID_ARG 1   /* null pointer, bad shape, misalignment, index out of range */
#define APMOE_UNSUPPORTED 2   /* q outside 3..8, unsupported dtype, device not gfx950 */
#define APMOE_NOT_RESIDENT 3  /* commit would use a plane or LUT that is not resident */
#define APMOE_HIP_ERROR 4     /* the HIP runtime reported an error */
#define APMOE_OUT_OF_MEMORY 5 /* host or device allocation failed (create / first commit only) */

#define APMOE_GATE_UP 0
#define APMOE_DOWN 1

#define APMOE_F16 0
#define APMOE_F32 1

#define APMOE_MIN_BITS 3
#define APMOE_MAX_BITS 8
#define APMOE_PLANES 8
#define APMOE_MAX_EXPERTS 256
#define APMOE_MAX_TOPK 8
#define APMOE_MAX_SHARED 8 /* shared experts per layer */
#define APMOE_MAX_ASSIGN (APMOE_MAX_TOPK + APMOE_MAX_SHARED) /* assignments per token */

typedef struct apmoe_ctx apmoe_ctx;
typedef struct apmoe_table apmoe_table;

/*
 * One linear-block (Section 3.1 page table row, GPU part).
 *   n, k          : rows (outputs) and columns (inputs); k % 128 == 0, n >= 1.
 *   q             : committed bitwidth to publish, 3..8 (the paper's q_i).
 *   d             : desired bitwidth (the paper's d_i); stored, never read by kernels.
 *   resident_mask : bit p set when plane[p] holds valid device data.
 *   plane[p]      : device plane p (code bit 7 - p) in the tiled layout of
 *                   apmoe_tile_planes, apmoe_tiled_plane_words(n, k) words; may be
 *                   NULL when not resident.
 *   lut[b]        : device fp16 [n][2^b] for b = 3..8; lut[0..2] are ignored.
 * A commit of this block requires planes 0..q-1 resident and non-NULL and lut[q]
 * non-NULL.  Planes p >= q and other LUT levels are never read by the kernels.
 */
typedef struct apmoe_block_desc {
    int32_t n;
    int32_t k;
    int32_t q;
    int32_t d;
    uint32_t resident_mask;
    const uint32_t *plane[APMOE_PLANES];
    const uint16_t *lut[APMOE_MAX_BITS + 1];
} apmoe_block_desc;

/* Text of a status code (static storage). */
const char *apmoe_status_string(apmoe_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *apmoe_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t apmoe_version(void);

/* Bind a context to HIP device `device`.  Fails with APMOE_UNSUPPORTED on a
 * device that is not gfx950.  The context owns one stream of its own (default
 * priority), two events and about 200 KB of device memory for the completion counters of
 * the fused launches (zeroed here, on `device`), released by apmoe_destroy;
 * APMOE_HIP_ERROR if they cannot be created.  APMOE_UNFUSED=1 in the environment at
 * this call gives a context whose layer steps always run as separate launches. */
apmoe_status apmoe_create(apmoe_ctx **out, int device);
apmoe_status apmoe_destroy(apmoe_ctx *ctx);

/* Sticky fault flags of the context's fused launches, 0 when none was raised.
 * APMOE_FAULT_LAYER_WAIT: a work item of the one-launch decode layer (apmoe_moe_forward)
 * gave up waiting for the gate_up blocks of its expert after about a second -- a broken
 * completion count, which the design rules out; the bound only keeps such a bug from
 * hanging the GPU, and that launch's output is then not to be trusted.  The flag stays
 * set for the context's life.  Synchronises the device (a diagnostic, not for hot loops). */
#define APMOE_FAULT_LAYER_WAIT 1
apmoe_status apmoe_ctx_faults(apmoe_ctx *ctx, int32_t *flags);

/*
 * Eq. 3 (Section 3.1): M_i^b, the GPU bytes of an n x k block at b bits,
 * n * b * k / 8 plane bytes plus n * 2^b * 2 LUT bytes.  The memory released by
 * b -> b' is apmoe_block_bytes(n,k,b) - apmoe_block_bytes(n,k,b').  Host only;
 * returns -1 for invalid arguments.
 */
int64_t apmoe_block_bytes(int32_t n, int32_t k, int32_t b);

/* ---------------------------------------------------------------------------
 * Block table (Section 3.1 weight page table; Section 3.3 safe-boundary commit)
 *
 * The table has n_layers * n_experts * 2 entries.  set_* calls edit a host
 * staging copy only.  apmoe_table_commit validates the whole staging copy and
 * enqueues its publication on a stream: kernels enqueued on that stream before
 * the commit read the previous committed table, kernels enqueued after read the
 * new one.  Kernels enqueued on other streams are ordered only by the caller.
 * The caller keeps every plane and LUT referenced by a committed table alive
 * until a later commit no longer references it and the stream has passed that
 * commit.  Host-side calls below need no GPU except commit and destroy.
 * ------------------------------------------------------------------------ */
apmoe_status apmoe_table_create(int32_t n_layers, int32_t n_experts, apmoe_table **out);

/* Waits for this table's pending commits, then frees it. */
apmoe_status apmoe_table_destroy(apmoe_table *tbl);

/* Stage a whole block entry (copied; pointers are not dereferenced). */
apmoe_status apmoe_table_set_block(apmoe_table *tbl, int32_t layer, int32_t expert, int32_t kind,
                                   const apmoe_block_desc *desc);

/* Stage a new committed bitwidth q (3..8) for one block (offload lowers q before
 * pages leave; reload raises q after pages are resident). */
apmoe_status apmoe_table_set_bits(apmoe_table *tbl, int32_t layer, int32_t expert, int32_t kind, int32_t q);

/* Stage new residency for one block: mask bit p and plane[p] (NULL allowed). */
apmoe_status apmoe_table_set_plane(apmoe_table *tbl, int32_t layer, int32_t expert, int32_t kind, int32_t p,
                                   const uint32_t *plane, int32_t resident);

/* What apmoe_table_commit would return for the current staging copy (host only). */
apmoe_status apmoe_table_validate(const apmoe_table *tbl);

/* Committed (last published) bitwidth of a block, 0 if never committed. */
apmoe_status apmoe_table_committed_bits(const apmoe_table *tbl, int32_t layer, int32_t expert, int32_t kind,
                                        int32_t *q);

/* Validate the staging copy and publish it on `stream`.  On error the
 * committed table is unchanged.  The first commit allocates the device table. */
apmoe_status apmoe_table_commit(apmoe_ctx *ctx, apmoe_table *tbl, void *stream);

/* ---------------------------------------------------------------------------
 * Format tools
 * ------------------------------------------------------------------------ */

/* Child LUT levels from the parent level 8 (fp16 [n][256], device).  The paper's
 * Figure 3 caption gives every quantised tensor a LUT of bitwidth-specific
 * centroids over the shared bit-planes, a b-bit weight reading the top b planes;
 * it gives no rule that relates the levels.  The reading taken here: the b-bit code
 * c covers the (b+1)-bit codes 2c and 2c+1, and its centroid is their mean --
 * level b = fp16 round-to-nearest-even of the mean of entries 2c and 2c+1 of
 * level b+1.  levels is a host array of 9 device pointers; levels[b] (fp16
 * [n][2^b]) is written for each b in 3..7 that is non-NULL (ownership: caller).
 * Errors: INVALID_ARG for NULL or misaligned pointers or n < 0; nothing is
 * enqueued then. */
apmoe_status apmoe_lut_build(apmoe_ctx *ctx, const uint16_t *parent, int32_t n, uint16_t *const *levels,
                             void *stream);

/* Words of one plane of an n x k block in the tiled layout (-1 for bad shapes):
 * ceil(n/32) * (k/128) tiles of 128 words.  Host only. */
int64_t apmoe_tiled_plane_words(int32_t n, int32_t k);

/* Rearrange canonical planes (uint32 [8][n][k/32], device) into the tiled layout:
 * plane p occupies tiled[p * W .. (p+1) * W), W = apmoe_tiled_plane_words(n, k).
 * Tile (rt, kt) of a plane starts at word 128 * (rt * (k/128) + kt) and covers rows
 * 32rt..32rt+31 and columns 128kt..128kt+127; inside it, words 2L and 2L+1 with
 * L = 32g + i hold row 32rt+i, columns 128kt+64g .. +31 and +32 .. +63 (canonical
 * bit order).  Rows past n are zero.  k % 128 == 0. */
apmoe_status apmoe_tile_planes(apmoe_ctx *ctx, const uint32_t *canonical, int32_t n, int32_t k, uint32_t *tiled,
                               void *stream);

/* Pack parent codes (uint8 [n][k], device) into 8 canonical planes (uint32 [8][n][k/32]). */
apmoe_status apmoe_pack_planes(apmoe_ctx *ctx, const uint8_t *codes, int32_t n, int32_t k, uint32_t *planes,
                               void *stream);

/* ---------------------------------------------------------------------------
 * Page movement (Section 3.1: each bit-plane of a linear-block is a page, and
 * dropping the top planes lowers its bitwidth; Section 3.3 and Figure 4: pages
 * move asynchronously, a bitwidth is lowered before its pages are offloaded and
 * raised only after they are reloaded, and changes are committed only at safe
 * boundaries).  Both calls are asynchronous; copies run on copy_stream, the
 * commit on stream.  Plane buffers hold one tiled plane each
 * (apmoe_tiled_plane_words(n, k) * 4 bytes); host buffers should be pinned.
 * ------------------------------------------------------------------------ */

/*
 * Page-out: lower committed block (layer, expert, kind) from q_old to q_new and
 * copy its planes q_new .. q_old-1 to host_planes[p].  The bitwidth change is
 * committed on `stream` first, so launches enqueued after this call never read
 * those planes.  The copies start once `stream` has passed that commit (every
 * launch that may read the planes has finished) and overlap the launches enqueued
 * after it.  done_event (a caller-created hipEvent_t) completes after the copies;
 * then the device planes may be freed or reused.
 * The staged entry then lists those planes as not resident.  Errors (nothing
 * enqueued, nothing changed): INVALID_ARG unless 3 <= q_new < q_old, the block was
 * committed with no pending bitwidth change, and every needed pointer is set.
 */
apmoe_status apmoe_page_out(apmoe_ctx *ctx, apmoe_table *tbl, int32_t layer, int32_t expert, int32_t kind,
                            int32_t q_new, void *const *host_planes /*[8]*/, void *stream, void *copy_stream,
                            void *done_event);

/*
 * Page-in: copy host_planes[p] to dev_planes[p] (caller-allocated device memory)
 * for p = q_old .. q_new-1 on copy_stream, make `stream` wait for the copies
 * (copied_event, a caller-created hipEvent_t, is recorded after them), then stage
 * the planes and q_new and commit on `stream`: launches enqueued after this call
 * use q_new.  LUT level q_new must be in the block's descriptor.  Errors as for
 * page-out, with q_old < q_new <= 8 and 16-byte aligned device planes.
 */
apmoe_status apmoe_page_in(apmoe_ctx *ctx, apmoe_table *tbl, int32_t layer, int32_t expert, int32_t kind,
                           int32_t q_new, void *const *host_planes /*[8]*/, uint32_t *const *dev_planes /*[8]*/,
                           void *stream, void *copy_stream, void *copied_event);

/* ---------------------------------------------------------------------------
 * Layer steps
 * ------------------------------------------------------------------------ */

/*
 * Router (Section 2.1: the router weights E experts and keeps the top K).
 *   x [T][H] fp16, w_router [E][H] fp16 (E routed experts), bias [E] fp32 or NULL.
 *   logit z[t][e] = sum_h x*w in fp64 (exact fp16 products), then + bias[e].
 *   topk_ids [T][topk] : experts by descending logit, ties to the lower index.
 *   topk_w   [T][topk] : fp32; renormalize != 0: softmax over the selected
 *                        logits; else the full softmax over E, at the selected.
 *   Shared experts (Table 1 lists "+4" / "+1" experts visited by every token):
 *   experts E .. E+n_shared-1 have no router row; the pages give no gate for them,
 *   so they follow the topk routed experts in every token's row with weight 1.
 *   With kt = topk + n_shared and Et = E + n_shared:
 *   topk_ids, topk_w [T][kt]; counts [Et], offsets [Et+1] (offsets[Et] = T*kt),
 *   perm [T*kt]: assignment ids a = t*kt + j grouped by expert ascending,
 *   ascending a inside a group; inv_perm [T*kt]: inv_perm[perm[r]] = r.
 *   The later steps take kt as their topk and Et as the layer's expert count.
 * Limits: 1 <= E, E + n_shared <= 256, 1 <= topk <= min(E, 8), 0 <= n_shared <= 8,
 * T >= 0 (T = 0 writes counts and offsets only), H % 8 == 0.
 * Launches: with T * kt <= 256, one -- every token's selection, then the grouping by
 * the workgroup that finishes last, which it finds with a completion counter of the
 * context (zero between calls); above, two (selection, then grouping).  The outputs
 * are the same bits either way.  Calls on one context that may run at the same time
 * (different streams, host threads) share that counter and must be ordered by the
 * caller (or use a context each).  APMOE_UNFUSED=1 in the environment at apmoe_create
 * gives a context that always takes the two launches.
 */
apmoe_status apmoe_route(apmoe_ctx *ctx, const uint16_t *x, const uint16_t *w_router, const float *bias, int32_t T,
                         int32_t H, int32_t E, int32_t topk, int32_t n_shared, int32_t renormalize,
                         int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets, int32_t *perm,
                         int32_t *inv_perm, void *stream);

/* Device workspace of apmoe_route for these arguments: always 0 bytes.  The
 * per-token selection runs in one workgroup per token and the expert-grouping sort
 * in the LDS of one workgroup; besides its outputs the route touches only the
 * context's completion counter (allocated and zeroed by apmoe_create).  INVALID_ARG
 * for arguments apmoe_route would refuse. */
apmoe_status apmoe_route_workspace(apmoe_ctx *ctx, int32_t T, int32_t E, int32_t topk, int32_t n_shared,
                                   size_t *bytes);

/*
 * Online routing statistics (Section 2.1, Eq. 1: the routing mass of expert e is
 * the sum of the routing weights of its selections over the sum of all routing
 * weights; Section 3.2 "Routing statistics": collected during serving).  Adds this
 * batch's contribution to caller-owned device accumulators:
 *   mass[e]       += sum of topk_w[t][j] over assignments routed to e   (fp64)
 *   selections[e] += number of assignments routed to e                  (int64)
 *   total[0]      += sum of the topk_w[t][j] of experts 0 .. E-1         (fp64)
 * for e = 0 .. E-1.  topk_w, perm and offsets are the outputs of apmoe_route for
 * the same batch (perm groups the assignments by expert); topk is their row
 * stride.  With shared experts pass topk + n_shared as topk and the routed E:
 * the statistics then cover the routed choices only, as Eq. 1 does (shared
 * experts have no routing weight).  The caller zeroes the accumulators once and
 * reads mass[e] / total[0].  Sums are fp64 with a fixed reduction order:
 * repeated calls give identical bits.  Calls that overlap on the same
 * accumulators race.  Limits: 1 <= E <= 256, 1 <= topk <= 16; T = 0 adds nothing.
 */
apmoe_status apmoe_route_stats(apmoe_ctx *ctx, const float *topk_w, const int32_t *perm, const int32_t *offsets,
                               int32_t T, int32_t topk, int32_t E, double *mass, double *total, int64_t *selections,
                               void *stream);

/*
 * Any-precision expert product (Section 3.3 "Fused Mixed-Precision MoE Kernel": the
 * kernel reads the weight pages -- bit-planes and LUT -- directly and follows the
 * bitwidth the planner committed for each gate_up and down module; Figure 3
 * caption: a b-bit weight is the centroid its top-b-plane code selects in the
 * b-bit LUT).  Every expert of one (layer, kind) in one call: up to
 * three kernel launches, by the experts' row counts (up to 32 rows, 33..64, more),
 * each skipped when the batch has too few tokens for any expert to need it.  A short
 * launch for the largest experts (at most two tiles per CU) runs on the context's own
 * stream, forked from `stream` and joined back into it within the call: work
 * enqueued on `stream` after the call sees the whole product.
 * For expert e, rows r in [offsets[e], offsets[e+1]) of the output:
 *   out[r][n] = sum_c in_row(r)[c] * LUT_q[n][code_q(n, c)],   fp32 accumulation,
 * with q, planes and LUT of block (layer, e, kind) read from the committed
 * device table at execution time.  in_row(r) = in[perm[r] / topk] when
 * gather != 0 (gate_up reading token activations), else in[r].
 *   in  : fp16 [T][K] (gather) or [T*topk][K]
 *   out : [T*topk][N] of out_dtype (APMOE_F16 rounds to nearest even).
 * N and K are the block shape; every expert of (layer, kind) must be committed
 * with the same shape.  offsets is device memory written by apmoe_route; no
 * host synchronisation happens.  Errors (nothing enqueued): INVALID_ARG for NULL
 * or misaligned pointers, a bad layer or kind, topk outside 1..16, or a buffer of
 * 2 GiB or more; UNSUPPORTED for another out_dtype; NOT_RESIDENT if the table was
 * never committed or a block of (layer, kind) has no committed entry.
 */
apmoe_status apmoe_gemm(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, int32_t kind, const uint16_t *in,
                        int32_t gather, const int32_t *perm, const int32_t *offsets, int32_t T, int32_t topk,
                        void *out, int32_t out_dtype, void *stream);

/* Expert activation (Section 3.3: the fused kernel covers "expert activation"
 * between the two projections; the pages do not name the function -- the reading
 * taken is the SwiGLU of Mixtral-class experts):
 *   a[r][f] = SiLU(h[r][f]) * h[r][F + f],  SiLU(z) = z / (1 + e^-z),
 * in fp32, stored fp16 (round to nearest even).  h fp16 [R][2F] (gate columns
 * [0, F), up columns [F, 2F)), a fp16 [R][F], both device, caller-owned;
 * F % 8 == 0.  INVALID_ARG for NULL or misaligned pointers or a bad F. */
apmoe_status apmoe_act(apmoe_ctx *ctx, const uint16_t *h, int32_t R, int32_t F, uint16_t *a, void *stream);

/*
 * gate_up product with the expert activation in its epilogue (Section 3.3: the MoE
 * kernel covers the expert computation, activation included, in its launches):
 *   a[r][f] = SiLU(h16[r][f]) * h16[r][F + f],   h16 = fp16 (RNE) of the gate_up rows,
 * in fp32, stored fp16 -- bit for bit what apmoe_gemm(APMOE_GATE_UP, .., APMOE_F16)
 * followed by apmoe_act gives, without writing or reading h.
 *   x : fp16 [T][H] (gather != 0) or [T*topk][H];  a : fp16 [T*topk][F].
 * Each workgroup computes gate rows and the matching up rows together, so
 * F = N/2 must be a multiple of 64 (APMOE_INVALID_ARG otherwise); other arguments,
 * limits and errors as apmoe_gemm with kind = APMOE_GATE_UP.
 */
apmoe_status apmoe_gemm_act(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, const uint16_t *x,
                            int32_t gather, const int32_t *perm, const int32_t *offsets, int32_t T, int32_t topk,
                            uint16_t *a, void *stream);

/* Output accumulation (Section 3.3: the fused kernel ends with the "output
 * accumulation" of the selected experts' outputs, weighted by the routing weights
 * of Section 2.1):
 *   out[t][n] = sum_{j < topk} topk_w[t][j] * y[inv_perm[t*topk + j]][n],
 * fp32, summed in j order (a gather: no atomics, the same bits on every run), stored
 * fp16.  y is [T*topk][H] of y_dtype (expert-grouped rows, as the products write
 * them), topk_w [T][topk] fp32, inv_perm [T*topk], out fp16 [T][H]; all device,
 * caller-owned; H % 8 == 0.  INVALID_ARG for NULL or misaligned pointers or bad
 * sizes, UNSUPPORTED for another y_dtype. */
apmoe_status apmoe_combine(apmoe_ctx *ctx, const void *y, int32_t y_dtype, const float *topk_w,
                           const int32_t *inv_perm, int32_t T, int32_t topk, int32_t H, uint16_t *out, void *stream);

/* Device workspace bytes needed by apmoe_moe_forward for one layer of tbl. */
apmoe_status apmoe_moe_workspace(const apmoe_table *tbl, int32_t layer, int32_t T, int32_t topk, int32_t n_shared,
                                 size_t *bytes);

/*
 * Whole layer (Section 3.3 "Fused Mixed-Precision MoE Kernel": routing, expert
 * activation, down projection and output accumulation, each gate_up / down module
 * at its committed bitwidth) in four steps: route, gate_up with the activation
 * fused (apmoe_gemm_act, fp16 a), down (fp32 y), combine.  With at most 32 tokens
 * (every expert then takes the decode product) the output accumulation runs in the
 * down product's epilogue -- the workgroup that finishes a token's last contribution
 * to a 64-column block sums it, with the arithmetic of apmoe_combine -- so the
 * small-batch layer is three launches (with the one-launch route); the same bits as
 * the four steps.  A context created with APMOE_LAYER_KERNEL=1 runs gate_up and down
 * of such a batch as one launch, on layers of at most 16 experts whose gate_up has
 * more than 1024 and down at most 1024 64-row blocks in all (the Mixtral shapes): its
 * workgroups take the gate_up blocks first and start an expert's down blocks once its
 * gate_up blocks are stored (the same bits; measured slower than the two launches, so
 * not the default).  The completion counters of these fused launches belong to the
 * context: calls on one context that may run at the same time must be ordered by the
 * caller.  APMOE_UNFUSED=1 at apmoe_create: every step in its own launches.
 * The table's experts of the layer are the routed ones (w_router rows) followed by
 * n_shared shared experts.
 * ws is caller-owned device memory of at least apmoe_moe_workspace bytes, 256-byte
 * aligned; it holds ids, weights, counts, offsets, perm, inv_perm, a and y.
 * out fp16 [T][H].  Every argument and size limit of the four steps is checked
 * before the first launch: a refused call enqueues nothing.  The call enqueues only
 * kernel launches on `stream` (and an event fork and join with the context's side
 * stream): it can be captured in a HIP graph and replayed, the counters being reset
 * by the kernels.
 */
apmoe_status apmoe_moe_forward(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, const uint16_t *x,
                               const uint16_t *w_router, const float *bias, int32_t T, int32_t topk,
                               int32_t n_shared, int32_t renormalize, void *ws, size_t ws_bytes, uint16_t *out,
                               void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The same layer as
 * apmoe_moe_forward (the same launches and bits) with the workspace in a static
 * device array of APMOE_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends; this call allocates nothing.  Its
 * address is taken once per context at apmoe_create.  Inputs and out as for
 * apmoe_moe_forward.  INVALID_ARG (nothing enqueued) when the layer needs more
 * workspace than the array holds (apmoe_moe_workspace); other errors as for
 * apmoe_moe_forward.  Every call on one device shares that device's array and
 * leaves its contents behind (every byte a call reads is written by the same call
 * first, so nothing needs clearing): calls that overlap on one device -- on
 * different streams, or from different host threads -- race and must be ordered by
 * the caller.
 */
#define APMOE_NOALLOC_SCRATCH_BYTES (64u << 20)
apmoe_status apmoe_moe_forward_noalloc(apmoe_ctx *ctx, const apmoe_table *tbl, int32_t layer, const uint16_t *x,
                                       const uint16_t *w_router, const float *bias, int32_t T, int32_t topk,
                                       int32_t n_shared, int32_t renormalize, uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* APMOE_H */
