// Host core of the library: segment metadata, launch planning, dense row
// offsets, status strings.  Plain C++17 with no HIP dependency, so every path
// here runs and is tested on a CPU-only machine.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/hetlora.h"
#include "variants.h"

#ifndef HETLORA_TILE_TABLE
#define HETLORA_TILE_TABLE "tile_table.inc"
#endif
namespace {
#include HETLORA_TILE_TABLE
}

extern "C" int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

extern "C" const char* lora_status_string(int32_t status) {
    switch (status) {
        case LORA_OK: return "ok";
        case LORA_EINVAL: return "invalid argument (null pointer, negative count, stride or alignment)";
        case LORA_EADAPTER: return "adapter id out of range";
        case LORA_ERANK: return "rank out of range [1, 128]";
        case LORA_ESHAPE: return "dimension or chunk length not a positive multiple of 64";
        case LORA_ECAPACITY: return "output capacity too small";
        case LORA_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

// Segment table: counting sort of the active rows by adapter id.  Rows keep
// their input order inside an adapter (stable), adapters come in ascending id,
// and one segment is emitted per adapter that has at least one row.
extern "C" int32_t lora_build_segments(int32_t n_rows, const int32_t* row_adapter,
                                       int32_t n_adapters, const int32_t* adapter_rank,
                                       int32_t seg_capacity, int32_t* row_index,
                                       int32_t* seg_start, int32_t* seg_adapter,
                                       int32_t* seg_rank, int32_t* n_seg, int32_t* n_active) {
    if (n_rows < 0 || n_adapters < 0 || seg_capacity < 0) return LORA_EINVAL;
    if ((n_rows > 0 && (row_adapter == nullptr || row_index == nullptr)) ||
        (n_adapters > 0 && adapter_rank == nullptr) || seg_start == nullptr ||
        (seg_capacity > 0 && (seg_adapter == nullptr || seg_rank == nullptr)) ||
        n_seg == nullptr || n_active == nullptr)
        return LORA_EINVAL;
    for (int32_t i = 0; i < n_rows; ++i)
        if (row_adapter[i] < -1 || row_adapter[i] >= n_adapters) return LORA_EADAPTER;
    for (int32_t a = 0; a < n_adapters; ++a)
        if (adapter_rank[a] < 1 || adapter_rank[a] > LORA_MAX_RANK) return LORA_ERANK;

    std::vector<int32_t> count((size_t)n_adapters + 1, 0);
    int32_t active = 0;
    for (int32_t i = 0; i < n_rows; ++i)
        if (row_adapter[i] >= 0) { ++count[(size_t)row_adapter[i] + 1]; ++active; }
    int32_t segs = 0;
    for (int32_t a = 0; a < n_adapters; ++a) segs += count[(size_t)a + 1] > 0;
    *n_seg = segs;
    *n_active = active;
    if (segs > seg_capacity) return LORA_ECAPACITY;

    for (int32_t a = 0; a < n_adapters; ++a) count[(size_t)a + 1] += count[(size_t)a];
    // count[a] is now the first slot of adapter a in row_index
    std::vector<int32_t> next(count.begin(), count.end() - 1);
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t a = row_adapter[i];
        if (a >= 0) row_index[next[(size_t)a]++] = i;
    }
    int32_t s = 0;
    for (int32_t a = 0; a < n_adapters; ++a) {
        if (count[(size_t)a + 1] == count[(size_t)a]) continue;
        seg_start[s] = count[(size_t)a];
        seg_adapter[s] = a;
        seg_rank[s] = adapter_rank[a];
        ++s;
    }
    seg_start[segs] = active;
    return LORA_OK;
}

namespace {

struct SegCfg {
    int shape;
    int32_t slices;
};

// Shape and K-slice count of a segment for one op.  The slice count always
// comes from the shrink table (with d_in), so the shrink and expand plans of
// one batch agree on it.
SegCfg pick(int32_t op, int32_t len, int32_t rank, int32_t d_in, int32_t d_out) {
    const int lb = lv_len_bucket(len), rb = lv_rank_bucket(rank);
    const ShrinkCfg sc = kShrinkCfg[lb][rb][lv_d_bucket(d_in)];
    int32_t slices = sc.slices < 1 ? 1 : sc.slices;
    if (slices > LORA_MAX_SLICES) slices = LORA_MAX_SLICES;
    if (slices > d_in / 64) slices = d_in / 64;
    if (op == LORA_OP_SHRINK) return SegCfg{sc.shape, slices};
    return SegCfg{kExpandShape[lb][rb][lv_d_bucket(d_out)], slices};
}

}  // namespace

namespace {

// One segment's share of a plan.
struct SegPlan {
    int variant;      // op-local variant id
    int32_t chunks;   // row chunks
    int32_t slices;   // K slices of the shrink (1 for expand-only / fused)
    int32_t mt;       // rows per item
    bool shrink;      // items carry K slices (one item per chunk x slice)
};

// Shrink and expand parts of a segment (the expand variant is op-local to an
// expand plan; an apply plan shifts it by LV_APPLY_EXPAND0).
SegPlan shrink_part(int32_t len, int32_t rank, int32_t d_in, int32_t d_out) {
    const SegCfg c = pick(LORA_OP_SHRINK, len, rank, d_in, d_out);
    const int32_t mt = lv_shrink_rows(c.shape);
    return SegPlan{c.shape * LV_RANK_CLASSES + lv_shrink_class(rank), (len + mt - 1) / mt, c.slices, mt, true};
}
SegPlan expand_part(int32_t len, int32_t rank, int32_t d_in, int32_t d_out) {
    const SegCfg c = pick(LORA_OP_EXPAND, len, rank, d_in, d_out);
    const int32_t mt = lv_expand_rows(c.shape);
    const int cls = c.shape == LV_E_BGMV ? 0 : lv_expand_class(rank);
    return SegPlan{c.shape * LV_RANK_CLASSES + cls, (len + mt - 1) / mt, c.slices, mt, false};
}
// Segments whose rows' whole reductions fit one workgroup each are fused in
// an apply plan (one item per row; the shrink result never leaves the chip):
// one-row segments always, and short segments while len * rank stays small.
// Each fused row re-reads the adapter's A and B rows (from L2 after the
// first), which beats the two-kernel path below that product: a 64-row
// rank-16 segment at d 4096 over q/k/v/o takes 11.1 us fused against 15.5 us
// as shrink + expand.
bool fused(int32_t len, int32_t rank, int32_t d_in, int32_t d_out) {
    return (len == 1 || (int64_t)len * rank <= LV_FUSED_MAX_ROWRANK) && d_in <= LV_FUSED_MAX_D &&
           d_out <= LV_FUSED_MAX_D;
}

}  // namespace

// Launch plan: every segment is cut into ceil(len / rows_per_item) row chunks
// whose sizes differ by at most one row; a shrink item is one row chunk x one
// K slice, an expand item one row chunk.  An apply plan holds, per segment,
// either one fused item or the segment's shrink and expand items.  Items are
// grouped by variant (in ascending variant id, segments in order inside a
// variant) so that each variant is one launch over a contiguous range.
extern "C" int32_t lora_plan(int32_t op, int32_t n_seg, const int32_t* seg_start,
                             const int32_t* seg_adapter, const int32_t* seg_rank,
                             int32_t d_in, int32_t d_out, int32_t work_capacity,
                             lora_work_t* work, lora_plan_info_t* info) {
    if ((op != LORA_OP_SHRINK && op != LORA_OP_EXPAND && op != LORA_OP_APPLY) || n_seg < 0 ||
        work_capacity < 0 || info == nullptr || seg_start == nullptr)
        return LORA_EINVAL;
    if (n_seg > 0 && (seg_adapter == nullptr || seg_rank == nullptr)) return LORA_EINVAL;
    if (d_in <= 0 || d_out <= 0 || d_in % 64 != 0 || d_out % 64 != 0) return LORA_ESHAPE;
    if (seg_start[0] != 0) return LORA_EINVAL;
    for (int32_t s = 0; s < n_seg; ++s) {
        if (seg_start[s + 1] <= seg_start[s]) return LORA_EINVAL;
        if (seg_adapter[s] < 0) return LORA_EADAPTER;
        if (seg_rank[s] < 1 || seg_rank[s] > LORA_MAX_RANK) return LORA_ERANK;
    }
    const int n_variants = op == LORA_OP_SHRINK ? LV_S_SHAPES * LV_RANK_CLASSES
                         : op == LORA_OP_EXPAND ? LV_E_SHAPES * LV_RANK_CLASSES
                                                : LV_APPLY_VARIANTS;

    // each segment contributes up to two parts (shrink + expand of an apply plan)
    std::vector<SegPlan> parts((size_t)n_seg * 2);
    std::vector<int32_t> per_variant((size_t)n_variants, 0);
    int64_t total = 0;
    int32_t v_slices = 1;
    for (int32_t s = 0; s < n_seg; ++s) {
        const int32_t len = seg_start[s + 1] - seg_start[s], r = seg_rank[s];
        SegPlan a{-1, 0, 1, 1, false}, b{-1, 0, 1, 1, false};
        if (op == LORA_OP_SHRINK) {
            a = shrink_part(len, r, d_in, d_out);
        } else if (op == LORA_OP_EXPAND) {
            a = expand_part(len, r, d_in, d_out);
        } else if (fused(len, r, d_in, d_out)) {
            a = SegPlan{LV_APPLY_FUSED, len, 1, 1, false};  // one item per row
        } else {
            a = shrink_part(len, r, d_in, d_out);
            b = expand_part(len, r, d_in, d_out);
            b.variant += LV_APPLY_EXPAND0;
        }
        for (SegPlan* q : {&a, &b}) {
            if (q->variant < 0) continue;
            const int32_t items = q->chunks * (q->shrink ? q->slices : 1);
            per_variant[(size_t)q->variant] += items;
            total += items;
            if (q->slices > v_slices) v_slices = q->slices;
        }
        parts[2 * (size_t)s] = a;
        parts[2 * (size_t)s + 1] = b;
    }
    info->n_work = (int32_t)total;
    if (total > work_capacity) return LORA_ECAPACITY;
    if (total > 0 && work == nullptr) return LORA_EINVAL;

    lora_plan_info_t out;
    memset(&out, 0, sizeof(out));
    out.op = op;
    out.n_work = (int32_t)total;
    out.n_active = seg_start[n_seg];
    out.max_rank = 0;
    out.max_adapter = -1;
    out.v_slices = v_slices;
    int32_t begin = 0;
    for (int v = 0; v < n_variants; ++v) {
        if (per_variant[(size_t)v] == 0) continue;
        lora_range_t& rg = out.ranges[out.n_ranges++];
        rg.variant = v;
        rg.begin = begin;
        rg.count = per_variant[(size_t)v];
        int32_t w = begin;
        for (int32_t s = 0; s < n_seg; ++s) {
            for (int h = 0; h < 2; ++h) {
                const SegPlan& q = parts[2 * (size_t)s + h];
                if (q.variant != v) continue;
                rg.rows_per_item = q.mt;
                const int32_t len = seg_start[s + 1] - seg_start[s];
                const int32_t base = len / q.chunks, extra = len % q.chunks;
                const int32_t ns = parts[2 * (size_t)s].slices;  // the segment's K slices
                int32_t row = seg_start[s];
                for (int32_t t = 0; t < q.chunks; ++t) {
                    const int32_t n = base + (t < extra ? 1 : 0);
                    if (q.shrink) {
                        for (int32_t sl = 0; sl < q.slices; ++sl)
                            work[w++] = lora_work_t{row, n, seg_adapter[s], seg_rank[s], sl, q.slices, {0, 0}};
                    } else {
                        work[w++] = lora_work_t{row, n, seg_adapter[s], seg_rank[s], 0,
                                                v == LV_APPLY_FUSED && op == LORA_OP_APPLY ? 1 : ns, {0, 0}};
                    }
                    row += n;
                }
                if (seg_rank[s] > out.max_rank) out.max_rank = seg_rank[s];
                if (seg_adapter[s] > out.max_adapter) out.max_adapter = seg_adapter[s];
            }
        }
        begin = w;
    }
    *info = out;
    return LORA_OK;
}

extern "C" int32_t lora_rows_dense_offsets(int32_t n_adapters, int32_t max_rank,
                                           const int32_t* rank, int32_t row_len,
                                           int32_t chunk_len, int64_t* row_off,
                                           int64_t* pool_elems) {
    if (n_adapters < 0 || pool_elems == nullptr || (n_adapters > 0 && (rank == nullptr || row_off == nullptr)))
        return LORA_EINVAL;
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERANK;
    if (row_len <= 0 || chunk_len <= 0 || chunk_len % 64 != 0) return LORA_ESHAPE;
    for (int32_t a = 0; a < n_adapters; ++a)
        if (rank[a] < 1 || rank[a] > max_rank) return LORA_ERANK;
    const int64_t chunks = (row_len + chunk_len - 1) / chunk_len;
    const int64_t stride = ((int64_t)row_len + 7) / 8 * 8;
    int64_t row = 0;
    for (int32_t a = 0; a < n_adapters; ++a) {
        for (int32_t j = 0; j < max_rank; ++j)
            for (int64_t c = 0; c < chunks; ++c) {
                const int64_t idx = ((int64_t)a * max_rank + j) * chunks + c;
                row_off[idx] = j < rank[a] ? (row + j) * stride + c * chunk_len : -1;
            }
        row += rank[a];
    }
    *pool_elems = row * stride;
    return LORA_OK;
}

// deLoRA mixture (VaLoRA blog, section 4.4.2): rows on the merged adapter
// get no delta; every other row keeps its adapter, which the composite
// tables below turn into "adapter a, minus the merged one".
extern "C" int32_t lora_mixture_row_adapter(int32_t n_rows, const int32_t* row_adapter, int32_t merged,
                                            int32_t* out_row_adapter) {
    if (n_rows < 0 || merged < 0 || (n_rows > 0 && (row_adapter == nullptr || out_row_adapter == nullptr)))
        return LORA_EINVAL;
    for (int32_t i = 0; i < n_rows; ++i) out_row_adapter[i] = row_adapter[i] == merged ? -1 : row_adapter[i];
    return LORA_OK;
}

// Composite row table: adapter a's rows, then the merged adapter's rows;
// the merged adapter's part is marked negative through neg_from.
extern "C" int32_t lora_mixture_rows(int32_t n_adapters, int32_t max_rank, const int32_t* rank, int32_t merged,
                                     int32_t chunks, const int64_t* row_off, int32_t out_max_rank,
                                     int64_t* out_row_off, int32_t* out_rank, int32_t* out_neg_from) {
    if (n_adapters < 1 || chunks < 1 || rank == nullptr || row_off == nullptr || out_row_off == nullptr ||
        out_rank == nullptr || out_neg_from == nullptr || merged < 0 || merged >= n_adapters)
        return LORA_EINVAL;
    if (max_rank < 1 || max_rank > LORA_MAX_RANK || out_max_rank < 1 || out_max_rank > LORA_MAX_RANK) return LORA_ERANK;
    const int32_t rm = rank[merged];
    for (int32_t a = 0; a < n_adapters; ++a) {
        if (rank[a] < 1 || rank[a] > max_rank) return LORA_ERANK;
        const int32_t r = a == merged ? rm : rank[a] + rm;
        if (r > out_max_rank || r > LORA_MAX_RANK) return LORA_ERANK;
    }
    for (int32_t a = 0; a < n_adapters; ++a) {
        const int32_t ra = rank[a];
        const int32_t r = a == merged ? rm : ra + rm;
        for (int32_t j = 0; j < out_max_rank; ++j) {
            int32_t src_a = a, src_j = j;
            if (a != merged && j >= ra) {
                src_a = merged;
                src_j = j - ra;
            }
            for (int32_t c = 0; c < chunks; ++c)
                out_row_off[((int64_t)a * out_max_rank + j) * chunks + c] =
                    j < r ? row_off[((int64_t)src_a * max_rank + src_j) * chunks + c] : 0;
        }
        out_rank[a] = r;
        out_neg_from[a] = a == merged ? rm : ra;
    }
    return LORA_OK;
}
