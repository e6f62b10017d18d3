/*
 * hetlora.h -- C ABI of the heterogeneous LoRA batching library for MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A batch of token rows, each either released (adapter id -1) or tied to one
 * LoRA adapter a of rank r_a, receives the low-rank delta
 *
 *     v_i    = x_i . A_a^T                  (shrink, d_in -> r_a)
 *     y_i   += s * v_i . B_a                (expand, r_a -> d_out)
 *
 * with no padding of ranks or rows (BEE-30060 "Multi-LoRA serving and adapter
 * management", Punica paragraph: every request adds its own x_i A_i B_i; SGMV
 * groups requests by adapter, BGMV serves one-token decode rows; S-LoRA
 * article, "Batching": adapters are computed without padding).  The mode
 * switch folds one adapter into a base weight and back out again,
 *
 *     W <- RNE_bf16(W + s * B_a^T . A_a)    (merge)
 *     W <- RNE_bf16(W - s * B_a^T . A_a)    (unmerge)
 *
 * (VaLoRA blog, section 4.4.1 "Swift Inference Mode Switch": Delta W = B x A is
 * computed at run time and added to / subtracted from the weights once).
 *
 * Layouts (all row-major, element strides "ld*" in elements)
 * ---------------------------------------------------------
 *   x  bf16 [n_rows][ldx]   token rows (input)
 *   y  fp32 [n_rows][ldy]   outputs, updated in place (y += ...)
 *   v  fp32 [v_slices][n_active][ldv]  rank-r intermediate (partial sums over
 *                           K slices); row p belongs to row_index[p]
 *   W  bf16 [d_out][ldw]    base weight (nn.Linear orientation, y = x W^T)
 *   A  r_a rows of d_in bf16 per adapter, B  r_a rows of d_out bf16 per adapter.
 * A and B are both stored as r "hidden-size vectors" (S-LoRA article, "Unified
 * Paging": a rank-R adapter weight occupies R pages of H-vectors), addressed
 * through a row-offset table, lora_rows_t, that covers both a dense packing
 * and a paged pool:
 *
 *   chunk c of row j of adapter a starts at
 *       pool + row_off[(a * max_rank + j) * chunks + c]      (bf16 elements)
 *   where chunks = ceil(row_len / chunk_len); the chunk holds chunk_len
 *   elements, the last one only up to row_len.
 *
 * bf16 values are passed as uint16_t bit patterns.
 *
 * Ownership, streams, errors
 * --------------------------
 * Every buffer belongs to the caller.  Pointers documented "device" must be
 * device memory of the current HIP device; "host" pointers are ordinary host
 * memory.  The library allocates no device memory, and apart from the pool
 * manager (lora_pool_create .. lora_pool_destroy: host state the caller owns
 * through its handle) it keeps no state or pointer after a call returns.
 * GPU work is enqueued on the given hipStream_t (passed as void*; NULL = the
 * null stream) and is asynchronous: no call synchronises.  All functions are
 * re-entrant (a pool manager serves one thread at a time); the only global
 * state is constant tables, a per-device occupancy cache and a small cache of
 * device-plan layouts already checked (lora_batch_build_device).
 * Arguments are validated before anything is launched; on error nothing is
 * launched and no output is written, except that the counts of
 * lora_build_segments / lora_plan are written on LORA_ECAPACITY so the caller
 * can resize.  Inputs that only the device sees (the row map and ranks of
 * lora_batch_build_device) are checked there, and an invalid batch becomes
 * an empty plan with an error status in the workspace header.  An empty batch (no active rows) is LORA_OK and launches nothing.
 * Device array contents (row_index, work, row_off) are trusted: they must be
 * what lora_build_segments / lora_plan / the caller's page table produced for
 * the host-side summary passed alongside.  x must not alias y; v must not
 * alias x or y.
 */
#ifndef HETLORA_H
#define HETLORA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 10
#define LORA_MAX_RANK 128   /* ranks are 1..128                              */
#define LORA_MAX_PROJ 8     /* projections per shrink/expand call            */
#define LORA_MAX_RANGES 48  /* kernel variants in one plan                   */
#define LORA_MAX_MERGE 8    /* weight matrices per merge/unmerge call        */
#define LORA_MAX_SLICES 16  /* K slices of one shrink segment                */
#define LORA_INLINE_ITEMS 64 /* fused items a plan may carry in its launch     */

/* Status codes (int32_t return value of every call except the two getters). */
#define LORA_OK         0  /* success                                                  */
#define LORA_EINVAL    -1  /* null pointer, negative count, ld < d, misaligned pointer */
#define LORA_EADAPTER  -2  /* adapter id outside [-1, n_adapters)                     */
#define LORA_ERANK     -3  /* rank outside [1, LORA_MAX_RANK]                          */
#define LORA_ESHAPE    -4  /* d_in / d_out / chunk_len not a positive multiple of 64   */
#define LORA_ECAPACITY -5  /* an output capacity is too small                          */
#define LORA_EHIP      -6  /* a HIP launch reported an error                           */

#define LORA_OP_SHRINK 0
#define LORA_OP_EXPAND 1
#define LORA_OP_APPLY 2   /* shrink + expand in one call, fused where chosen */

/* Adapter rows of one matrix kind (A or B of one projection).
 *   pool      device, bf16 elements; 16-byte aligned
 *   row_off   device, int64 [n_adapters * max_rank * chunks]; every offset a
 *             multiple of 8 (16 bytes); entries for j >= r_a are never read
 *   max_rank  row-slot stride of the table (>= every rank used with it)
 *   row_len   elements per row (d_in for A, d_out for B)
 *   chunk_len elements per chunk, a positive multiple of 64
 *   neg_from  device, int32 [n_adapters], or NULL.  Read on the A side only
 *             (by the calls that compute v): for adapter a, the rank rows
 *             j >= neg_from[a] enter with a minus sign, v_j = -(x . A_a[j]).
 *             This is how a deLoRA composite adapter (lora_mixture_rows)
 *             subtracts the merged adapter.  NULL: no row is negated.  The
 *             merge calls require NULL on both sides.                      */
typedef struct lora_rows {
    const uint16_t* pool;
    const int64_t* row_off;
    int32_t n_adapters;
    int32_t max_rank;
    int32_t row_len;
    int32_t chunk_len;
    const int32_t* neg_from;
} lora_rows_t;

/* One unit of kernel work: rows row_index[row0 .. row0+nrows) of one segment,
 * all on `adapter` of rank `rank`.  The shrink may split the reduction over
 * d_in into `nslices` K slices (64-wide blocks [s*nb/nslices,
 * (s+1)*nb/nslices), nb = d_in/64): a shrink item computes slice `kslice`
 * and writes it to v slice `kslice`; an expand item adds up the `nslices`
 * slices of its rows, in slice order. */
typedef struct lora_work {
    int32_t row0;
    int32_t nrows;
    int32_t adapter;
    int32_t rank;
    int32_t kslice;
    int32_t nslices;
    int32_t reserved[2];
} lora_work_t;

/* Work items [begin, begin+count) of the plan run kernel `variant`; no item
 * has more than rows_per_item rows. */
typedef struct lora_range {
    int32_t variant;
    int32_t begin;
    int32_t count;
    int32_t rows_per_item;
} lora_range_t;

/* Host-side summary of a plan, written by lora_plan. */
typedef struct lora_plan_info {
    int32_t op;           /* LORA_OP_SHRINK, LORA_OP_EXPAND or LORA_OP_APPLY */
    int32_t n_work;       /* work items written                          */
    int32_t n_active;     /* rows covered (= seg_start[n_seg])           */
    int32_t max_rank;     /* largest rank among the items                */
    int32_t max_adapter;  /* largest adapter id among the items (-1 if none) */
    int32_t v_slices;     /* v slices the shrink writes / the expand reads (>= 1) */
    int32_t d_in;         /* d_in and d_out the plan was made for: the calls  */
    int32_t d_out;        /* reject projections wider than these (LORA_ESHAPE) */
    int32_t n_ranges;
    lora_range_t ranges[LORA_MAX_RANGES];
} lora_plan_info_t;

/* What lora_shrink / lora_expand need to launch one plan.
 *   host_work, host_row_index  host copies of work and row_index (the
 *         staging buffer lora_batch_prepare wrote), or NULL.  lora_apply
 *         passes a small all-fused plan (one range of the fused variant, at
 *         most LORA_INLINE_ITEMS items) to its kernel in the launch
 *         arguments from these, and then reads neither device array; with
 *         LORA_PREPARE_INLINE, lora_batch_prepare copies nothing for such a
 *         plan and leaves row_index and work NULL.
 *   live  NULL for a plan built on the host.  For a plan built on the device
 *         (lora_batch_build_device): device int32 [info.n_ranges], the items
 *         range r really holds; info.ranges[r].count is then the range's
 *         capacity, every launch is sized for it, and items at or past
 *         live[r] are skipped on the device without being read. */
typedef struct lora_launch {
    const int32_t* row_index;   /* device int32 [info.n_active] (lora_build_segments) */
    const lora_work_t* work;    /* device [info.n_work] (lora_plan, same op)           */
    lora_plan_info_t info;      /* host copy of the plan summary                      */
    const int32_t* live;        /* see above                                          */
    const lora_work_t* host_work;      /* see above                                   */
    const int32_t* host_row_index;     /* see above                                   */
} lora_launch_t;

/* One projection of a shrink: v[p][j] = sum_k x[row_index[p]][k] * A_a[j][k],
 * as info.v_slices partial sums over K slices.
 *   x  device bf16 [*][ldx], 16-byte aligned, ldx % 8 == 0, ldx >= d_in
 *   v  device fp32 [info.v_slices][info.n_active][ldv], 16-byte aligned,
 *      ldv % 4 == 0, ldv >= info.max_rank; slice s of row p holds the part of
 *      the sum over slice s's K blocks; slices beyond a row's nslices and
 *      columns j >= r_a are not written                                     */
typedef struct lora_shrink_proj {
    const uint16_t* x;
    int64_t ldx;
    int32_t d_in;
    lora_rows_t A;
    float* v;
    int64_t ldv;
} lora_shrink_proj_t;

/* One projection of an expand: y[row_index[p]][n] += scale * sum_j v[p][j] * B_a[j][n],
 * with v[p][j] the sum of the row's K slices.
 *   v  device fp32 as written by lora_shrink with the matching plan (same
 *      v_slices, n_active and ldv)
 *   y  device fp32 [*][ldy], 16-byte aligned, ldy % 4 == 0, ldy >= d_out;
 *      rows not listed in row_index are not touched                         */
typedef struct lora_expand_proj {
    const float* v;
    int64_t ldv;
    lora_rows_t B;
    int32_t d_out;
    float* y;
    int64_t ldy;
    float scale;
} lora_expand_proj_t;

/* One weight matrix of a merge/unmerge.
 *   W  device bf16 [d_out][ldw], 16-byte aligned, ldw % 8 == 0, ldw >= d_in
 *   A  rows of d_in (A.row_len == d_in), B rows of d_out (B.row_len == d_out)
 *   adapter, rank: which adapter's rows 0..rank-1 to fold in            */
typedef struct lora_merge_mat {
    uint16_t* W;
    int64_t ldw;
    int32_t d_out;
    int32_t d_in;
    lora_rows_t A;
    lora_rows_t B;
    int32_t adapter;
    int32_t rank;
    float scale;
} lora_merge_mat_t;

/* One projection of lora_apply: the shrink's and the expand's arguments.
 *   x, ldx, d_in, A      as in lora_shrink_proj_t
 *   v, ldv               scratch for the segments that are not fused: device
 *                        fp32 [info.v_slices][info.n_active][ldv] as in
 *                        lora_shrink_proj_t; may be NULL when the plan has no
 *                        shrink or expand range (every segment fused); its
 *                        contents after the call are unspecified
 *   B, d_out, y, ldy, scale  as in lora_expand_proj_t                    */
typedef struct lora_apply_proj {
    const uint16_t* x;
    int64_t ldx;
    int32_t d_in;
    lora_rows_t A;
    float* v;
    int64_t ldv;
    lora_rows_t B;
    int32_t d_out;
    float* y;
    int64_t ldy;
    float scale;
} lora_apply_proj_t;

/* ABI version (LORA_ABI_VERSION of the built library). */
int32_t lora_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* lora_status_string(int32_t status);

/* Segment metadata of a batch (host only, deterministic).
 * Active rows are those with row_adapter[i] >= 0 (LoRazor article: a released
 * row gets no LoRA work); they are listed in row_index ordered by
 * (adapter id, row index), and grouped into one segment per distinct adapter,
 * in ascending adapter id (BEE-30060 page, Punica paragraph: requests are
 * grouped by adapter identity).
 *   row_adapter   host int32 [n_rows], each in [-1, n_adapters)
 *   adapter_rank  host int32 [n_adapters], each in [1, LORA_MAX_RANK]
 *   row_index     host int32 [n_rows] (capacity n_rows; n_active written)
 *   seg_start     host int32 [seg_capacity + 1]; seg_start[n_seg] == n_active
 *   seg_adapter, seg_rank  host int32 [seg_capacity]
 * Errors: LORA_EINVAL, LORA_EADAPTER, LORA_ERANK, LORA_ECAPACITY (n_seg and
 * n_active are written, nothing else). */
int32_t lora_build_segments(int32_t n_rows, const int32_t* row_adapter,
                            int32_t n_adapters, const int32_t* adapter_rank,
                            int32_t seg_capacity, int32_t* row_index,
                            int32_t* seg_start, int32_t* seg_adapter,
                            int32_t* seg_rank, int32_t* n_seg, int32_t* n_active);

/* Launch plan for one op (host only).  Every segment is cut into work items of
 * at most rows_per_item rows, where the kernel variant and rows_per_item come
 * from a compiled-in table keyed by (op, segment length, rank, d) buckets
 * (VaLoRA blog, section 4.3.2: the best tiling per input shape is found offline
 * and looked up at run time); the same table fixes into how many K slices
 * the shrink splits each segment, so the shrink and expand plans of one batch
 * (same seg_*, d_in, d_out) agree on v_slices.  Items cover only active rows
 * and are grouped by variant.  At most n_active * 16 items are written
 * (work_capacity >= 16 * n_active is always enough; 17 * n_active for
 * LORA_OP_APPLY, whose plan holds the shrink items, the expand items and the
 * fused items of its segments in one list).
 *   seg_*  as written by lora_build_segments
 *   d_in, d_out  positive multiples of 64 (the largest over the projections
 *                that will share this plan)
 * Errors: LORA_EINVAL, LORA_ERANK, LORA_ESHAPE, LORA_ECAPACITY (info->n_work
 * written). */
int32_t lora_plan(int32_t op, int32_t n_seg, const int32_t* seg_start,
                  const int32_t* seg_adapter, const int32_t* seg_rank,
                  int32_t d_in, int32_t d_out, int32_t work_capacity,
                  lora_work_t* work, lora_plan_info_t* info);

/* lora_plan with the caller's tile table, for the offline tiling search
 * (VaLoRA blog, section 4.3.2: input shapes are profiled offline and the
 * best tiling of each kept in a table looked up at run time), so candidate
 * tables can be timed with the library as built.  The tables have the
 * compiled-in table's layout (csrc/tile_table.inc), indexed [length bucket
 * 8][rank bucket 4][d bucket 4]:
 *   shrink_table  host int8 [8][4][4][2]: (shrink shape 0..2, K slices 1..16)
 *   expand_table  host int8 [8][4][4]: expand shape 0..4
 * A segment's K-slice count is min(slices, d_in / 64), as with the compiled
 * table.  Everything else as lora_plan.  Errors: as lora_plan; LORA_EINVAL
 * also for a null table or an entry outside those ranges. */
int32_t lora_plan_table(int32_t op, int32_t n_seg, const int32_t* seg_start,
                        const int32_t* seg_adapter, const int32_t* seg_rank,
                        int32_t d_in, int32_t d_out, const int8_t* shrink_table,
                        const int8_t* expand_table, int32_t work_capacity,
                        lora_work_t* work, lora_plan_info_t* info);

/* Everything the host does for one batch, in one call: the segment table
 * (lora_build_segments), the plans of the ops in op_mask (lora_plan), all
 * written into one caller buffer laid out for a single host-to-device copy,
 * and that copy, enqueued on hip_stream.  A serving loop then pays one call
 * per batch instead of one per step of the preparation.
 *   staging layout (int32 elements):  row_index [n_active], then the plan of
 *       each requested op in LORA_OP_* order (info.n_work lora_work_t each)
 *   op_mask      bit (1 << op) for each of LORA_OP_SHRINK / _EXPAND / _APPLY
 *                to plan; at least one.  With LORA_PREPARE_INLINE added and
 *                LORA_OP_APPLY the only op, a plan lora_apply can carry in
 *                its launch arguments (see lora_launch_t) is not copied: the
 *                launch's row_index and work stay NULL, its host_* pointers
 *                point into staging, and staging must then stay unchanged
 *                until the lora_apply calls that use it have been made
 *   seg_*        host int32 outputs as in lora_build_segments (seg_start
 *                [seg_capacity + 1], seg_adapter / seg_rank [seg_capacity])
 *   staging      host int32 [staging_capacity]; pinned memory makes the copy
 *                asynchronous, and then the caller must not rewrite it before
 *                the copy has run (record an event on hip_stream after the
 *                call and wait for it before the next call on this buffer)
 *   dev_staging  device int32 [staging_capacity]
 *   out          n_seg, n_active, n_staged (int32 elements used) and, per
 *                op, a ready lora_launch_t whose row_index and work point into
 *                dev_staging; ops not in op_mask get info.op = -1, which every
 *                call rejects
 * Errors: as lora_build_segments and lora_plan; LORA_ECAPACITY when
 * seg_capacity is too small (out->n_seg holds the count needed,
 * out->n_staged is 0) or staging_capacity is (out->n_staged holds the size
 * needed); nothing is copied then.  LORA_EHIP when the copy cannot be
 * enqueued. */
#define LORA_PREPARE_INLINE 0x100u

typedef struct lora_batch {
    int32_t n_seg;
    int32_t n_active;
    int64_t n_staged;
    lora_launch_t launch[3];    /* indexed by LORA_OP_SHRINK, _EXPAND, _APPLY */
} lora_batch_t;

int32_t lora_batch_prepare(int32_t n_rows, const int32_t* row_adapter,
                           int32_t n_adapters, const int32_t* adapter_rank,
                           int32_t d_in, int32_t d_out, uint32_t op_mask,
                           int32_t seg_capacity, int32_t* seg_start,
                           int32_t* seg_adapter, int32_t* seg_rank,
                           int32_t* staging, int64_t staging_capacity,
                           void* dev_staging, void* hip_stream, lora_batch_t* out);

/* Device-built batches: the segment table and the apply plan of a batch
 * whose row -> adapter map is already in device memory, built by one kernel
 * on the stream, with no host round trip and no host-to-device copy (the
 * grouping of rows by adapter identity of the BEE-30060 page, Punica
 * paragraph, and the run-time tile lookup of the VaLoRA blog, section 4.3.2,
 * done on the GPU).  The host fixes the launch shapes in advance from bounds
 * alone (rows, adapters, largest rank, d): lora_device_plan lists every
 * kernel variant a batch within those bounds can need, grouped into one
 * range per launch (variants one kernel runs share a range: the long-segment
 * shrink of ranks <= 64 per row shape, the MFMA expand per rank class), each
 * with room for the most items such a batch can put there.  The builder
 * fills a range with exactly the items lora_plan(LORA_OP_APPLY) gives its
 * variants for the same batch, variant after variant in ascending order, and
 * stores the count; lora_apply then walks each range's live items with a
 * grid of at most the resident workgroups.  Results are bit-identical to
 * lora_apply with the host-built plan of the same batch.
 *
 * lora_device_plan (host only): the layout for given bounds.
 *   n_rows      rows of row_adapter, 1 .. 65536
 *   n_adapters  adapter ids are in [0, n_adapters), 1 .. 4096
 *   max_rank    bound on every adapter's rank, 1 .. LORA_MAX_RANK
 *   d_in, d_out as in lora_plan (the largest over the projections)
 *   out         the layout: seg_capacity = min(n_rows, n_adapters);
 *               info (op LORA_OP_APPLY, n_active = n_rows, max_rank,
 *               max_adapter = n_adapters - 1, v_slices = the most K slices a
 *               segment can get, one range per launch group: variant = the
 *               group's smallest variant, begin, count = its capacity,
 *               rows_per_item = its largest); byte offsets of each part of
 *               the workspace and its size (256-byte aligned parts)
 * Errors: LORA_EINVAL (bounds out of range), LORA_ERANK, LORA_ESHAPE.
 *
 * lora_batch_build_device: enqueue the builder on hip_stream.
 *   plan          as written by lora_device_plan
 *   row_adapter   device int32 [plan->n_rows], each in [-1, n_adapters)
 *   adapter_rank  device int32 [plan->n_adapters], each in [1, max_rank]
 *   workspace     device, plan->workspace_bytes, 256-byte aligned; holds the
 *                 header (lora_device_header_t, offset 0), row_index, the
 *                 segment table (seg_start [seg_capacity + 1], seg_adapter,
 *                 seg_rank [seg_capacity], as lora_build_segments writes
 *                 them), a scratch part and the work items.  Only the
 *                 header's counts say which entries are current.
 *   out           host: a ready lora_launch_t (op LORA_OP_APPLY) whose
 *                 row_index, work and live point into the workspace; the
 *                 launches that use it must follow the builder on the device
 *                 (the same stream, or one ordered after it by an event), and
 *                 the next build into this workspace must follow them
 * The inputs are checked on the device: an adapter id outside [-1,
 * n_adapters) or a rank outside [1, max_rank] leaves status LORA_EADAPTER /
 * LORA_ERANK in the header and an empty plan (every live count 0), so the
 * launches that follow do nothing; the caller reads the header when it
 * wants to know.  Host-side errors: LORA_EINVAL (null or misaligned
 * pointer, a plan lora_device_plan did not write), LORA_EHIP. */
typedef struct lora_device_plan {
    int32_t n_rows;
    int32_t n_adapters;
    int32_t max_rank;
    int32_t d_in;
    int32_t d_out;
    int32_t seg_capacity;
    int32_t work_capacity;      /* items over all ranges                     */
    int32_t reserved;
    int64_t off_row_index;      /* byte offsets into the workspace           */
    int64_t off_seg_start;
    int64_t off_seg_adapter;
    int64_t off_seg_rank;
    int64_t off_scratch;
    int64_t off_work;
    int64_t workspace_bytes;
    lora_plan_info_t info;
} lora_device_plan_t;

typedef struct lora_device_header {
    int32_t status;             /* LORA_OK or the error found on the device  */
    int32_t n_seg;
    int32_t n_active;
    int32_t n_work;             /* items over all ranges                     */
    int32_t live[LORA_MAX_RANGES];
} lora_device_header_t;

int32_t lora_device_plan(int32_t n_rows, int32_t n_adapters, int32_t max_rank, int32_t d_in,
                         int32_t d_out, lora_device_plan_t* out);
int32_t lora_batch_build_device(const lora_device_plan_t* plan, const int32_t* row_adapter,
                                const int32_t* adapter_rank, void* workspace, void* hip_stream,
                                lora_launch_t* out);

/* Shrink for n_proj projections (1..LORA_MAX_PROJ) sharing one plan
 * (launch->info.op == LORA_OP_SHRINK): one kernel launch per variant range.
 * Errors: LORA_EINVAL (also: a range whose variant no kernel runs),
 * LORA_ESHAPE (also: a projection's d_in above the plan's info.d_in),
 * LORA_EADAPTER / LORA_ERANK (summary does not fit the row tables), LORA_EHIP. */
int32_t lora_shrink(const lora_launch_t* launch, int32_t n_proj,
                    const lora_shrink_proj_t* projs, void* hip_stream);

/* Expand for n_proj projections sharing one plan
 * (launch->info.op == LORA_OP_EXPAND).  Same errors as lora_shrink, with
 * d_out checked against info.d_out. */
int32_t lora_expand(const lora_launch_t* launch, int32_t n_proj,
                    const lora_expand_proj_t* projs, void* hip_stream);

/* Shrink and expand in one call, for a plan made with op = LORA_OP_APPLY:
 * y[row_index[p]] += scale * (x[row_index[p]] . A_a^T) . B_a for every active
 * row.  The plan fuses one-row segments (decode rows) of small enough d_in and
 * d_out into a single kernel that keeps v on chip; the other segments run the
 * shrink and expand kernels of lora_shrink / lora_expand through v.  The
 * result is the same delta within rounding (the fused kernel reduces over
 * d_in in another order).  Errors: as lora_shrink and lora_expand (d_in and
 * d_out both checked against the plan's). */
int32_t lora_apply(const lora_launch_t* launch, int32_t n_proj,
                   const lora_apply_proj_t* projs, void* hip_stream);

/* lora_apply without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid allocation.  The same as lora_apply, except that projs[i].v
 * and projs[i].ldv are ignored: v lives in an array the library holds on
 * each device it runs on (LORA_STATIC_SCRATCH_BYTES, kept until the process
 * ends), projection i in its own region of info.v_slices * max(1, n_active)
 * * ldv floats, ldv = info.max_rank rounded up to 4.  Nothing is allocated
 * and nothing needs to start at zero.  Every call on a device shares that
 * device's array, so calls that overlap in time on one device (other
 * streams, other threads) race and must not be made; the array keeps the
 * last call's contents.  Errors: as lora_apply; LORA_ECAPACITY when n_proj
 * regions do not fit the array (nothing is launched); LORA_EHIP when the
 * array's address on the current device cannot be found. */
#define LORA_STATIC_SCRATCH_BYTES (64u << 20)
int32_t lora_apply_static(const lora_launch_t* launch, int32_t n_proj,
                          const lora_apply_proj_t* projs, void* hip_stream);

/* Merge n_mats (1..LORA_MAX_MERGE) adapters into their weights in place, one
 * launch: W <- RNE_bf16(W + scale * B_a^T A_a), with Delta W accumulated in
 * fp32 and a single rounding to bf16.  Matrices must not overlap.
 * Errors: LORA_EINVAL, LORA_ESHAPE, LORA_EADAPTER, LORA_ERANK, LORA_EHIP. */
int32_t lora_merge(int32_t n_mats, const lora_merge_mat_t* mats, void* hip_stream);

/* Unmerge: identical to lora_merge with every scale negated. */
int32_t lora_unmerge(int32_t n_mats, const lora_merge_mat_t* mats, void* hip_stream);

/* Row-offset table of the packed dense layout (host only): adapters in id
 * order, rows j = 0..rank[a]-1 back to back, each row taking
 * ceil(row_len/8)*8 elements; chunk c of a row sits c*chunk_len elements after
 * the row start; slots j >= rank[a] are set to -1.
 *   rank      host int32 [n_adapters], each in [1, max_rank]
 *   row_off   host int64 [n_adapters * max_rank * ceil(row_len/chunk_len)]
 *   pool_elems  host, receives the pool size in elements the layout needs
 * Errors: LORA_EINVAL, LORA_ERANK, LORA_ESHAPE. */
int32_t lora_rows_dense_offsets(int32_t n_adapters, int32_t max_rank,
                                const int32_t* rank, int32_t row_len,
                                int32_t chunk_len, int64_t* row_off,
                                int64_t* pool_elems);

/* deLoRA mixture inference (VaLoRA blog, section 4.4.2 "Mixture Inference
 * Mode"): while adapter `merged` (m) is merged into the weights, a request
 * on adapter x != m is served with W_merge - Delta W_m + Delta W_x, i.e. on
 * the delta path y += s (x A_x^T) B_x - s (x A_m^T) B_m, and a request on m
 * needs no delta at all.  A request with no adapter (a released one, which
 * the LoRazor article's mechanism section serves on the backbone alone) is
 * the same formula with Delta W_x = 0: y += -s (x A_m^T) B_m, giving x W.
 * The two calls below express this as an ordinary heterogeneous batch over
 * "composite" adapters, so every call above (lora_apply, lora_shrink +
 * lora_expand) serves it in one pass:
 *
 * lora_mixture_row_adapter: host.  out_row_adapter[i] = -1 where
 *   row_adapter[i] == merged (no work: W_merge serves the row); `merged`
 *   where row_adapter[i] == -1 and base_rows != 0 (composite adapter m is
 *   "minus the merged adapter": the row gets the backbone output); -1 where
 *   row_adapter[i] == -1 and base_rows == 0 (a row whose output is not
 *   wanted, e.g. padding, stays untouched); else row_adapter[i].
 *   row_adapter, out_row_adapter: host int32 [n_rows] (may be the same
 *   array).  Errors: LORA_EINVAL (null pointer, n_rows < 0, merged < 0).
 *
 * lora_mixture_rows: host.  Builds the composite row-offset table of one
 *   matrix kind (call it once for A and once for B) from the table of the
 *   real adapters: composite adapter a (a != m) has rank r_a + r_m, rows
 *   j < r_a are adapter a's rows and rows r_a + i are the merged adapter's
 *   row i; composite adapter m has m's own r_m rows, all negated.
 *   rank        host int32 [n_adapters], ranks of the real adapters
 *   row_off     host int64 [n_adapters * max_rank * chunks], the real table
 *   out_row_off host int64 [n_adapters * out_max_rank * chunks]; slots past
 *               a composite rank are set to 0 (never read)
 *   out_rank    host int32 [n_adapters] (composite ranks; the adapter_rank
 *               argument of lora_build_segments for the mixture batch)
 *   out_neg_from host int32 [n_adapters]: r_a for a != m (the merged
 *               adapter's rows enter negated), 0 for m (every row negated);
 *               upload it and pass it as the A side's neg_from
 *   Outputs are written only on LORA_OK.  Errors: LORA_EINVAL (null
 *   pointer, n_adapters < 1, chunks < 1, merged outside [0, n_adapters)),
 *   LORA_ERANK (a rank outside [1, max_rank], or r_a + r_m > out_max_rank
 *   or > LORA_MAX_RANK).                                                    */
int32_t lora_mixture_row_adapter(int32_t n_rows, const int32_t* row_adapter,
                                 int32_t merged, int32_t base_rows, int32_t* out_row_adapter);
int32_t lora_mixture_rows(int32_t n_adapters, int32_t max_rank,
                          const int32_t* rank, int32_t merged, int32_t chunks,
                          const int64_t* row_off, int32_t out_max_rank,
                          int64_t* out_row_off, int32_t* out_rank,
                          int32_t* out_neg_from);

/* ---------------------------------------------------------------------------
 * Unified adapter pool (S-LoRA article, "Unified Paging": a rank-R adapter
 * weight occupies R pages of hidden-size vectors in one memory pool; adapters
 * are brought in on demand).  The pool is one caller-owned device array of
 * n_pages pages of page_elems bf16 elements.  A pool manager (host state
 * only, created and destroyed by the caller: the one library object that
 * outlives a call) assigns pages to adapters and keeps the row-offset tables
 * (lora_rows_t.row_off, chunk_len = page_elems) of n_tables row tables, e.g.
 * the A and B tables of every projection; table t has rows of row_len[t]
 * elements, each row taking ceil(row_len[t] / page_elems) pages.  An adapter
 * of rank r takes sum_t r * ceil(row_len[t] / page_elems) pages.
 * Pinned adapters (those of batches in flight) are never evicted; when the
 * pool is short, unpinned resident adapters are evicted least recently used
 * first.  Entries of adapters that are not resident are 0 (page 0, never read
 * by a valid batch).  Not thread-safe: one manager per caller thread.
 * ------------------------------------------------------------------------ */
typedef struct lora_pool lora_pool_t;

/* Errors: LORA_EINVAL (null out, non-positive sizes, n_tables outside
 * [1, 64]), LORA_ESHAPE (page_elems or a row_len not a positive multiple of
 * 64, or page_elems above 65536, the longest piece lora_pool_scatter copies),
 * LORA_ERANK (max_rank outside [1, LORA_MAX_RANK]). */
int32_t lora_pool_create(int64_t n_pages, int32_t page_elems, int32_t n_adapters,
                         int32_t max_rank, int32_t n_tables, const int32_t* row_len,
                         lora_pool_t** out);
int32_t lora_pool_destroy(lora_pool_t* pool);

/* Makes the n listed adapters (ranks[i] = rank of adapters[i]) resident and
 * pins each once (pins count; lora_pool_release drops one).  Adapters already
 * resident with that rank only get pinned and their use time refreshed; the
 * others get pages (evicting as above) and their ids are written to
 * load[0 .. *n_load), in the order given: their rows must be copied in before
 * a batch reads them (lora_pool_load_list, lora_pool_scatter).  A resident
 * adapter listed with another rank is reloaded.  Duplicates in the list are
 * allowed.  On LORA_ECAPACITY (the listed adapters do not fit beside the
 * pinned ones) nothing changes.  Errors: LORA_EINVAL, LORA_EADAPTER,
 * LORA_ERANK, LORA_ECAPACITY. */
int32_t lora_pool_acquire(lora_pool_t* pool, int32_t n, const int32_t* adapters,
                          const int32_t* ranks, int32_t* load, int32_t* n_load);

/* Drops one pin of each listed adapter (call once the batches that used them
 * have finished on the GPU).  Errors: LORA_EINVAL (an adapter not pinned). */
int32_t lora_pool_release(lora_pool_t* pool, int32_t n, const int32_t* adapters);

/* Host row-offset table of table t (n_adapters * max_rank * chunks int64,
 * element offsets into the pool), valid until the next acquire; *chunks =
 * ceil(row_len[t] / page_elems).  Adapter a's entries are the contiguous
 * block [a * max_rank * chunks, (a + 1) * max_rank * chunks). */
int32_t lora_pool_row_off(const lora_pool_t* pool, int32_t table, const int64_t** row_off,
                          int32_t* chunks);

/* Resident adapters, free pages and pinned adapters (any may be NULL). */
int32_t lora_pool_stats(const lora_pool_t* pool, int32_t* n_resident, int64_t* free_pages,
                        int32_t* n_pinned);

/* Copy list that places the rows of the n listed resident adapters: source
 * layout = the adapters in the order given, each as table 0's r rows of
 * row_len[0] elements, then table 1's, ... (packed, no gaps); one piece per
 * (adapter, table, rank row, chunk): src_off (elements into the packed
 * source), dst_off (elements into the pool), len (elements, <= page_elems).
 * Writes min(capacity, needed) pieces and *n_pieces = needed; *src_elems =
 * packed source size.  Errors: LORA_EINVAL (an adapter not resident),
 * LORA_ECAPACITY (capacity < needed). */
int32_t lora_pool_load_list(const lora_pool_t* pool, int32_t n, const int32_t* adapters,
                            int64_t capacity, int64_t* src_off, int64_t* dst_off, int32_t* len,
                            int64_t* n_pieces, int64_t* src_elems);

/* GPU: pool[dst_off[i] + e] = src[src_off[i] + e] for e < len[i], i < n
 * (bf16 bits; src, pool, src_off, dst_off, len device; offsets in elements,
 * multiples of 8, len a multiple of 8 and <= 65536; pieces must not
 * overlap in the pool).  One launch on hip_stream.  Errors: LORA_EINVAL,
 * LORA_EHIP. */
int32_t lora_pool_scatter(const uint16_t* src, uint16_t* pool, int64_t n,
                          const int64_t* src_off, const int64_t* dst_off, const int32_t* len,
                          void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HETLORA_H */
