// Kernel variants shared by the planner (host) and the launchers (HIP).
//
// A variant is (shape, rank class).  The shape fixes how many rows one work
// item may hold and how a workgroup splits the work; the rank class fixes how
// many 16-wide MFMA tiles the rank dimension needs, so registers are padded,
// never memory.  variant = shape * LV_RANK_CLASSES + rank_class.
#pragma once

#include <stdint.h>

// The helpers below serve the host planner and the device plan builder.
#ifdef __HIPCC__
#define LV_HD __host__ __device__
#else
#define LV_HD
#endif
// Address space of the tile-config table (constant memory where device code reads it).
#ifndef LV_TABLE_SPACE
#define LV_TABLE_SPACE
#endif

#define LV_RANK_CLASSES 4

// Shrink shapes (rows per work item): 4 waves split K over one 16-row tile,
// or 4 waves each own 16 / 32 rows over the full K.
#define LV_S_SPLITK16 0
#define LV_S_ROWS64 1
#define LV_S_ROWS128 2
#define LV_S_SHAPES 3

// Expand shapes: the MFMA kernel with work items of 16 / 64 / 128 / 32 rows
// (more rows reuse each B column strip more, fewer rows give more
// workgroups and a y stream of shorter columns), and the VALU kernel for
// decode items of at most 2 rows (BGMV), which has a single rank class.
#define LV_E_ROWS16 0
#define LV_E_ROWS64 1
#define LV_E_ROWS128 2
#define LV_E_ROWS32 3
#define LV_E_BGMV 4
#define LV_E_SHAPES 5

static inline LV_HD int32_t lv_shrink_rows(int shape) {
    return shape == LV_S_SPLITK16 ? 16 : shape == LV_S_ROWS64 ? 64 : 128;
}
static inline LV_HD int32_t lv_expand_rows(int shape) {
    return shape == LV_E_ROWS16 ? 16 : shape == LV_E_ROWS32 ? 32 : shape == LV_E_ROWS64 ? 64 : shape == LV_E_BGMV ? 2 : 128;
}
// Variant ids of an apply plan: the shrink variants, then the expand
// variants shifted by LV_APPLY_EXPAND0, then the fused one-row kernel.
#define LV_APPLY_EXPAND0 (LV_S_SHAPES * LV_RANK_CLASSES)
#define LV_APPLY_FUSED (LV_APPLY_EXPAND0 + LV_E_SHAPES * LV_RANK_CLASSES)
#define LV_APPLY_VARIANTS (LV_APPLY_FUSED + 1)
// The fused kernel covers d_in and d_out up to 8 x half its 1024 threads.
#define LV_FUSED_MAX_D 4096
#define LV_FUSED_MAX_ROWRANK 1024  // segments of more than one row are fused while len * rank <= this

// Launch group of an apply-plan variant in a device-built plan: variants one
// launch can run share a group (the shrink of one shape with ranks up to 64,
// whose kernels pick the rank tiles per item; the MFMA expand of one rank
// class, whose kernel takes items of any row count); every other variant is
// a group of its own.  The key is the group's smallest variant.
static inline LV_HD int lv_launch_group(int v) {
    if (v < LV_APPLY_EXPAND0) {
        const int shape = v / LV_RANK_CLASSES, cls = v % LV_RANK_CLASSES;
        return cls < LV_RANK_CLASSES - 1 ? shape * LV_RANK_CLASSES : v;
    }
    if (v < LV_APPLY_FUSED) {
        const int ev = v - LV_APPLY_EXPAND0, shape = ev / LV_RANK_CLASSES, cls = ev % LV_RANK_CLASSES;
        return shape == LV_E_BGMV ? v : LV_APPLY_EXPAND0 + cls;
    }
    return v;
}

// Member i (in ascending order) of the launch group keyed by `key`, or -1.
static inline LV_HD int lv_group_member(int key, int i) {
    if (key < LV_APPLY_EXPAND0) {
        const int n = key % LV_RANK_CLASSES == 0 ? LV_RANK_CLASSES - 1 : 1;
        return i < n ? key + i : -1;
    }
    if (key < LV_APPLY_EXPAND0 + LV_RANK_CLASSES)  // MFMA expand of one rank class: shapes 0 .. LV_E_ROWS32
        return i <= LV_E_ROWS32 ? key + i * LV_RANK_CLASSES : -1;
    return i == 0 ? key : -1;
}

// Columns per workgroup (a column group) of the expand kernels: 512 for both.
static inline LV_HD int32_t lv_expand_cols(int shape) { return shape >= 0 ? 512 : 0; }

// Shrink rank classes: N tiles of 16 ranks -> 1, 2, 4, 8 (rank <= 16, 32, 64, 128).
static inline LV_HD int lv_shrink_class(int32_t rank) {
    return rank <= 16 ? 0 : rank <= 32 ? 1 : rank <= 64 ? 2 : 3;
}
// Expand rank classes: K steps of 32 ranks -> 1, 2, 4 (rank <= 32, 64, 128);
// class 3 is unused.
static inline LV_HD int lv_expand_class(int32_t rank) {
    return rank <= 32 ? 0 : rank <= 64 ? 1 : 2;
}

// Bucket keys of the tile-config table.
#define LV_LEN_BUCKETS 8
#define LV_RANK_BUCKETS 4
#define LV_D_BUCKETS 4
static inline LV_HD int lv_len_bucket(int32_t len) {
    return len <= 1 ? 0 : len <= 4 ? 1 : len <= 8 ? 2 : len <= 16 ? 3 : len <= 32 ? 4 : len <= 64 ? 5
         : len <= 256 ? 6 : 7;
}
static inline LV_HD int lv_rank_bucket(int32_t r) { return r <= 16 ? 0 : r <= 32 ? 1 : r <= 64 ? 2 : 3; }
static inline LV_HD int lv_d_bucket(int32_t d) { return d <= 1024 ? 0 : d <= 4096 ? 1 : d <= 8192 ? 2 : 3; }
