// Per-segment plan rules, shared by the host planner (lora_plan) and the
// device plan builder (lora_batch_build_device), so that both cut a segment
// into the same work items.  Include after the tile-config table
// (kShrinkCfg, kExpandShape), inside the namespace that holds it.  Every rule
// takes the table's two parts by pointer (the device builder passes a copy
// in LDS); they default to the table itself.
#pragma once

typedef const ShrinkCfg (*ShrinkTab)[LV_RANK_BUCKETS][LV_D_BUCKETS];
typedef const int8_t (*ExpandTab)[LV_RANK_BUCKETS][LV_D_BUCKETS];

struct SegCfg {
    int shape;
    int32_t slices;
};

// Shape and K-slice count of a segment for one op.  The slice count always
// comes from the shrink table (with d_in), so the shrink and expand plans of
// one batch agree on it.
static inline LV_HD SegCfg lv_pick(int32_t op, int32_t len, int32_t rank, int32_t d_in, int32_t d_out,
                                   ShrinkTab st, ExpandTab et) {
    const int lb = lv_len_bucket(len), rb = lv_rank_bucket(rank);
    const ShrinkCfg sc = st[lb][rb][lv_d_bucket(d_in)];
    int32_t slices = sc.slices < 1 ? 1 : sc.slices;
    if (slices > LORA_MAX_SLICES) slices = LORA_MAX_SLICES;
    if (slices > d_in / 64) slices = d_in / 64;
    if (op == LORA_OP_SHRINK) return SegCfg{sc.shape, slices};
    return SegCfg{et[lb][rb][lv_d_bucket(d_out)], slices};
}

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
static inline LV_HD SegPlan lv_shrink_part(int32_t len, int32_t rank, int32_t d_in, int32_t d_out,
                                           ShrinkTab st = kShrinkCfg, ExpandTab et = kExpandShape) {
    const SegCfg c = lv_pick(LORA_OP_SHRINK, len, rank, d_in, d_out, st, et);
    const int32_t mt = lv_shrink_rows(c.shape);
    return SegPlan{c.shape * LV_RANK_CLASSES + lv_shrink_class(rank), (len + mt - 1) / mt, c.slices, mt, true};
}
static inline LV_HD SegPlan lv_expand_part(int32_t len, int32_t rank, int32_t d_in, int32_t d_out,
                                           ShrinkTab st = kShrinkCfg, ExpandTab et = kExpandShape) {
    const SegCfg c = lv_pick(LORA_OP_EXPAND, len, rank, d_in, d_out, st, et);
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
static inline LV_HD bool lv_fused(int32_t len, int32_t rank, int32_t d_in, int32_t d_out) {
    return (len == 1 || (int64_t)len * rank <= LV_FUSED_MAX_ROWRANK) && d_in <= LV_FUSED_MAX_D &&
           d_out <= LV_FUSED_MAX_D;
}

// The parts of one segment in an apply plan: a fused part (one item per
// row), or a shrink part and an expand part (variant shifted by
// LV_APPLY_EXPAND0).
static inline LV_HD void lv_apply_parts(int32_t len, int32_t rank, int32_t d_in, int32_t d_out, SegPlan& a,
                                        SegPlan& b, ShrinkTab st = kShrinkCfg, ExpandTab et = kExpandShape) {
    if (lv_fused(len, rank, d_in, d_out)) {
        a = SegPlan{LV_APPLY_FUSED, len, 1, 1, false};
        b = SegPlan{-1, 0, 1, 1, false};
    } else {
        a = lv_shrink_part(len, rank, d_in, d_out, st, et);
        b = lv_expand_part(len, rank, d_in, d_out, st, et);
        b.variant += LV_APPLY_EXPAND0;
    }
}
