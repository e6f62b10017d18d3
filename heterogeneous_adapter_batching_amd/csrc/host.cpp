// Host core of the library: segment metadata, launch planning, dense row
// offsets, status strings.  Plain C++17 with no HIP dependency, so every path
// here runs and is tested on a CPU-only machine.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/hetlora.h"
#include "variants.h"

#ifndef HETLORA_TILE_TABLE
#define HETLORA_TILE_TABLE "tile_table.inc"
#endif
namespace {
#include HETLORA_TILE_TABLE
#include "plan_rules.h"
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

// Launch plan: every segment is cut into ceil(len / rows_per_item) row chunks
// whose sizes differ by at most one row; a shrink item is one row chunk x one
// K slice, an expand item one row chunk.  An apply plan holds, per segment,
// either one fused item or the segment's shrink and expand items.  Items are
// grouped by variant (in ascending variant id, segments in order inside a
// variant) so that each variant is one launch over a contiguous range.
namespace {
// Every segment's shape and K slices from the tile table st / et (the
// compiled-in one, or a caller's for the offline search).
int32_t plan_impl(int32_t op, int32_t n_seg, const int32_t* seg_start, const int32_t* seg_adapter,
                  const int32_t* seg_rank, int32_t d_in, int32_t d_out, int32_t work_capacity, lora_work_t* work,
                  lora_plan_info_t* info, ShrinkTab st, ExpandTab et) {
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
        if (op == LORA_OP_SHRINK)
            a = lv_shrink_part(len, r, d_in, d_out, st, et);
        else if (op == LORA_OP_EXPAND)
            a = lv_expand_part(len, r, d_in, d_out, st, et);
        else
            lv_apply_parts(len, r, d_in, d_out, a, b, st, et);
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
    out.d_in = d_in;
    out.d_out = d_out;
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
}  // namespace

extern "C" int32_t lora_plan(int32_t op, int32_t n_seg, const int32_t* seg_start,
                             const int32_t* seg_adapter, const int32_t* seg_rank,
                             int32_t d_in, int32_t d_out, int32_t work_capacity,
                             lora_work_t* work, lora_plan_info_t* info) {
    return plan_impl(op, n_seg, seg_start, seg_adapter, seg_rank, d_in, d_out, work_capacity, work, info,
                     kShrinkCfg, kExpandShape);
}

// The offline tile search's planner: lora_plan with the caller's table, so
// every candidate table can be timed with the library as built.
extern "C" int32_t lora_plan_table(int32_t op, int32_t n_seg, const int32_t* seg_start,
                                   const int32_t* seg_adapter, const int32_t* seg_rank, int32_t d_in,
                                   int32_t d_out, const int8_t* shrink_table, const int8_t* expand_table,
                                   int32_t work_capacity, lora_work_t* work, lora_plan_info_t* info) {
    static_assert(sizeof(ShrinkCfg) == 2, "a shrink entry is (shape, slices)");
    if (shrink_table == nullptr || expand_table == nullptr) return LORA_EINVAL;
    const int n = LV_LEN_BUCKETS * LV_RANK_BUCKETS * LV_D_BUCKETS;
    for (int i = 0; i < n; ++i) {
        if (shrink_table[2 * i] < 0 || shrink_table[2 * i] >= LV_S_SHAPES || shrink_table[2 * i + 1] < 1 ||
            shrink_table[2 * i + 1] > LORA_MAX_SLICES || expand_table[i] < 0 || expand_table[i] >= LV_E_SHAPES)
            return LORA_EINVAL;
    }
    return plan_impl(op, n_seg, seg_start, seg_adapter, seg_rank, d_in, d_out, work_capacity, work, info,
                     reinterpret_cast<ShrinkTab>(shrink_table), reinterpret_cast<ExpandTab>(expand_table));
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
// tables below turn into "adapter a, minus the merged one".  A released row
// (no adapter: served by the backbone, LoRazor article, mechanism section)
// becomes composite adapter `merged`, which the tables make "minus the
// merged adapter": the backbone output x W = x (W_merge - Delta W_m).
extern "C" int32_t lora_mixture_row_adapter(int32_t n_rows, const int32_t* row_adapter, int32_t merged,
                                            int32_t base_rows, int32_t* out_row_adapter) {
    if (n_rows < 0 || merged < 0 || (n_rows > 0 && (row_adapter == nullptr || out_row_adapter == nullptr)))
        return LORA_EINVAL;
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t a = row_adapter[i];
        out_row_adapter[i] = a == merged ? -1 : (a == -1 && base_rows) ? merged : a;
    }
    return LORA_OK;
}

// Composite row table: adapter a's rows, then the merged adapter's rows;
// the merged adapter's part is marked negative through neg_from.  The
// merged adapter's own composite holds its rows, all negated.
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
        out_neg_from[a] = a == merged ? 0 : ra;
    }
    return LORA_OK;
}

// Layout of a device-built apply plan.  A segment's parts depend only on its
// (length bucket, rank class) box, so the variants a batch can need follow
// from enumerating the boxes that the bounds allow.  A variant's capacity
// adds up, over the boxes that reach it, the most items the box's segments
// can produce: a non-fused segment in a box has at least `lnf` rows, so the
// box holds at most min(n_adapters, n_rows / lnf) of them, and their row
// chunks of mt rows number at most n_rows / mt plus one per segment (and at
// most ceil(len_max / mt) per segment).  Fused items are one per row, so at
// most n_rows in all.
namespace {
constexpr int32_t kLenLo[LV_LEN_BUCKETS] = {1, 2, 5, 9, 17, 33, 65, 257};
constexpr int32_t kLenHi[LV_LEN_BUCKETS] = {1, 4, 8, 16, 32, 64, 256, INT32_MAX};
int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }
int64_t chunk_bound(int64_t n_rows, int64_t nseg, int32_t len_max, int32_t mt) {
    const int64_t a = nseg * ((len_max + (int64_t)mt - 1) / mt), b = n_rows / mt + nseg;
    return a < b ? a : b;
}
}  // namespace

extern "C" int32_t lora_device_plan(int32_t n_rows, int32_t n_adapters, int32_t max_rank, int32_t d_in,
                                    int32_t d_out, lora_device_plan_t* out) {
    if (out == nullptr || n_rows < 1 || n_rows > 65536 || n_adapters < 1 || n_adapters > 4096) return LORA_EINVAL;
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERANK;
    if (d_in <= 0 || d_out <= 0 || d_in % 64 != 0 || d_out % 64 != 0) return LORA_ESHAPE;
    std::vector<int64_t> cap(LV_APPLY_VARIANTS, 0);
    std::vector<int32_t> rows_per(LV_APPLY_VARIANTS, 1);
    int32_t v_slices = 1;
    for (int c = 0; c <= lv_shrink_class(max_rank); ++c) {
        const int32_t rlo = c == 0 ? 1 : (8 << c) + 1, rhi = (16 << c) < max_rank ? (16 << c) : max_rank;
        for (int b = 0; b < LV_LEN_BUCKETS; ++b) {
            const int32_t llo = kLenLo[b], lhi = kLenHi[b] < n_rows ? kLenHi[b] : n_rows;
            if (llo > lhi) continue;
            // fusing is monotone: shorter segments and smaller ranks stay fused
            if (lv_fused(llo, rlo, d_in, d_out)) cap[LV_APPLY_FUSED] = n_rows;
            if (lv_fused(lhi, rhi, d_in, d_out)) continue;
            int32_t lnf = llo;  // shortest non-fused segment of the box
            while (lv_fused(lnf, rhi, d_in, d_out)) ++lnf;
            const int64_t nseg = std::min<int64_t>(n_adapters, n_rows / lnf);
            SegPlan sp, ep;
            lv_apply_parts(lhi, rhi, d_in, d_out, sp, ep);  // same variants for every member of the box
            cap[(size_t)sp.variant] += chunk_bound(n_rows, nseg, lhi, sp.mt) * sp.slices;
            cap[(size_t)ep.variant] += chunk_bound(n_rows, nseg, lhi, ep.mt);
            rows_per[(size_t)sp.variant] = sp.mt;
            rows_per[(size_t)ep.variant] = ep.mt;
            if (sp.slices > v_slices) v_slices = sp.slices;
        }
    }
    lora_device_plan_t p;
    memset(&p, 0, sizeof(p));
    p.n_rows = n_rows;
    p.n_adapters = n_adapters;
    p.max_rank = max_rank;
    p.d_in = d_in;
    p.d_out = d_out;
    p.seg_capacity = n_rows < n_adapters ? n_rows : n_adapters;
    lora_plan_info_t& I = p.info;
    I.op = LORA_OP_APPLY;
    I.n_active = n_rows;
    I.max_rank = max_rank;
    I.max_adapter = n_adapters - 1;
    I.v_slices = v_slices;
    I.d_in = d_in;
    I.d_out = d_out;
    // one range per launch group, keyed by its smallest variant
    std::vector<int64_t> gcap(LV_APPLY_VARIANTS, 0);
    std::vector<int32_t> grows(LV_APPLY_VARIANTS, 0);
    for (int v = 0; v < LV_APPLY_VARIANTS; ++v) {
        if (cap[(size_t)v] == 0) continue;
        const int g = lv_launch_group(v);
        gcap[(size_t)g] += cap[(size_t)v];
        grows[(size_t)g] = std::max(grows[(size_t)g], rows_per[(size_t)v]);
    }
    int64_t begin = 0;
    for (int g = 0; g < LV_APPLY_VARIANTS; ++g) {
        if (gcap[(size_t)g] == 0) continue;
        if (I.n_ranges == LORA_MAX_RANGES || begin + gcap[(size_t)g] > INT32_MAX / 2) return LORA_EINVAL;
        lora_range_t& R = I.ranges[I.n_ranges++];
        R.variant = g;
        R.begin = (int32_t)begin;
        R.count = (int32_t)gcap[(size_t)g];
        R.rows_per_item = grows[(size_t)g];
        begin += gcap[(size_t)g];
    }
    I.n_work = (int32_t)begin;
    p.work_capacity = (int32_t)begin;
    int64_t off = align256(sizeof(lora_device_header_t));
    p.off_row_index = off;
    off += align256(4 * (int64_t)n_rows);
    p.off_seg_start = off;
    off += align256(4 * ((int64_t)p.seg_capacity + 1));
    p.off_seg_adapter = off;
    off += align256(4 * (int64_t)p.seg_capacity);
    p.off_seg_rank = off;
    off += align256(4 * (int64_t)p.seg_capacity);
    p.off_scratch = off;
    off += align256(4 * (int64_t)n_rows);
    p.off_work = off;
    off += align256((int64_t)sizeof(lora_work_t) * begin);
    p.workspace_bytes = off;
    *out = p;
    return LORA_OK;
}
