// gfx950 kernels of the heterogeneous LoRA path and their C-ABI launchers.
//
//   shrink  v[p][j]  = sum_k x[row_index[p]][k] * A_a[j][k]       (j < r_a)
//   expand  y[row_index[p]][n] += s * sum_j v[p][j] * B_a[j][n]
//   merge   W[n][k]  = RNE_bf16(W[n][k] + s * sum_j B_a[j][n] * A_a[j][k])
//
// plus the adapter-pool scatter and the device-side plan builder (the
// segment table and the apply plan built on the GPU from a row -> adapter
// map, for lora_apply's grid-stride launches).
//
// (BEE-30060 "Multi-LoRA serving", Punica paragraph: per-request delta
// x_i A_i B_i, requests grouped by adapter; VaLoRA blog section 4.4.1:
// Delta W = B x A added once; S-LoRA article, Unified Paging: adapter rows are
// hidden-size vectors gathered from a pool.)
//
// All three use the bf16 MFMA v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  Operand convention relied upon: in the first operand lane l
// supplies row (l % 16), in the second operand column (l % 16); both take the
// same 8 reduction elements from lane group (l / 16); the fp32 result of lane l
// is column (l % 16), rows 4*(l / 16) + 0..3.  Because both operands use the
// same lane-group pairing, any fixed assignment of memory positions to the 32
// reduction slots gives the exact dot product; the kernels use that freedom to
// load 16 or 32 contiguous bytes per lane.
//
// Rows whose reduction index runs along memory (x and A in the shrink) load
// straight into operands.  Where the reduction index (the rank j) is the slow
// memory index (B in the expand, A and B in the merge), each lane loads 8
// rows x 8 consecutive columns and transposes that 8x8 bf16 block in
// registers; output column slot i of MFMA c then stands for memory column
// base + 8*i + c, so each lane still ends up owning 8 consecutive outputs.
//
// Row-offset loads are issued unconditionally, in one batch, at clamped valid
// indices; the data loads that depend on them follow in a second batch, each
// masked to the lanes whose row, rank slot and column are inside the work
// (masked-off lanes read nothing and use zero), except the merge's adapter
// rows, which are read at the clamped addresses and zeroed (L2 hits, cheaper
// than masking).  So the in-order memory counter never makes a load wait for
// another it does not depend on.  Stores are masked.
//
// No float atomics and a fixed reduction order everywhere: results do not
// depend on a row's position in a work item or on the launch order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/hetlora.h"
#define LV_TABLE_SPACE __constant__
#include "variants.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define WG 256

namespace {

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
// masked 16-byte load: lanes with ok == false read nothing and get zero
__device__ __forceinline__ u32x4_t ld16_if(bool ok, const void* p) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4_t*>(p);
    return v;
}
__device__ __forceinline__ u32x2_t ld8_if(bool ok, const void* p) {
    u32x2_t v = {0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x2_t*>(p);
    return v;
}
__device__ __forceinline__ f32x4_t ldf4_if(bool ok, const float* p) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (ok) v = *reinterpret_cast<const f32x4_t*>(p);
    return v;
}
__device__ __forceinline__ f32x4_t ldf4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Stores of y: a launch writes each y element once and does not read it back,
// so they go out as nontemporal (streaming) stores, which measured ~1% faster
// on the MFMA expand than plain stores
__device__ __forceinline__ void stf4(float* p, f32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void stf2(float* p, f32x2_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x2_t*>(p));
}
__device__ __forceinline__ u32x4_t sel(bool ok, u32x4_t v) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    return ok ? v : z;
}

// Compiler-only fence: keeps a batch of loads issued before the code that
// follows (stops the compiler from sinking a load into the branch that uses
// it, which would make that branch wait on the whole batch).  No instruction
// is emitted.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Wave-uniform read through the scalar data cache (row tables are read-only
// for the whole launch).  `i` must be the same in every lane of the wave.
__device__ __forceinline__ int64_t ld_uniform(const int64_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int64_t*)p)[i];
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value.  Branches on it are then scalar branches: an MFMA inside a branch the
// compiler takes for divergent runs under EXEC = 0 when no lane takes the
// branch, and MFMA does not honour EXEC, so it would still accumulate.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 bits, round to nearest, ties to even (the
// hardware convert, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// 8 rows (r[e] = 8 consecutive bf16 columns of row e) -> 8 columns
// (out[c] = the 8 rows' values in column c).
__device__ __forceinline__ void transpose8x8(const u32x4_t r[8], u32x4_t out[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int d = c >> 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a = r[2 * q][d], b = r[2 * q + 1][d];
            out[c][q] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
        }
    }
}

// Row table of one matrix kind (A or B of one projection).
struct Rows {
    const uint16_t* pool;
    const int64_t* row_off;
    int32_t n_adapters, max_rank, chunk_len, chunks;
    const int32_t* neg_from;  // A side: v_j negated for j >= neg_from[adapter] (NULL: none)
};
// First rank row of `adapter` whose v enters negated (a deLoRA composite
// adapter's merged part); `rank` when the table marks none.
__device__ __forceinline__ int32_t neg_start(const Rows& t, int32_t adapter, int32_t rank) {
    return t.neg_from ? t.neg_from[adapter] : rank;
}

// A work item is used only if it lies inside the launch's rows and fits the
// row tables and the kernel's rank capacity; anything else is skipped, so a
// corrupted work list cannot index outside the buffers.
__device__ __forceinline__ bool item_ok(const lora_work_t& it, int32_t n_active, int32_t v_slices, const Rows& t,
                                        int32_t rank_cap) {
    // bitwise, not short-circuit: every field is already loaded, and one
    // combined test lets the loads it needs issue together
    return (it.nrows > 0) & (it.row0 >= 0) & (it.row0 + it.nrows <= n_active) & (it.adapter >= 0) &
           (it.adapter < t.n_adapters) & (it.rank >= 1) & (it.rank <= rank_cap) & (it.rank <= t.max_rank) &
           (it.nslices >= 1) & (it.nslices <= v_slices) & (it.kslice >= 0) & (it.kslice < it.nslices);
}
// Item `i` of a launch is in use: every item of a host-built plan; for a
// device-built plan (live != NULL) only those below the range's live count.
// The item itself may be loaded before this is known: the launch never
// exceeds the range's capacity, so the load stays inside the work list.
__device__ __forceinline__ bool item_live(const int32_t* live, int i) { return !live || i < *live; }

// Index into row_off of chunk `c` of row j of adapter a.
__device__ __forceinline__ int64_t off_index(const Rows& t, int32_t a, int32_t j, int32_t c) {
    return ((int64_t)a * t.max_rank + j) * t.chunks + c;
}

// ------------------------------------------------------------------ shrink
struct ShrinkProj {
    const uint16_t* x;
    int64_t ldx;
    Rows A;
    int32_t d_in;
    float* v;
    int64_t ldv;
};
struct ShrinkArgs {
    const int32_t* row_index;
    const lora_work_t* work;
    const int32_t* live;  // device-built plan: items of the range (NULL: all `count`)
    int32_t begin;
    int32_t n_active;
    int32_t v_slices;
    int32_t count;   // work items of the launch (persistent kernel: tasks = count x n_proj)
    int32_t n_proj;
    // projections that share x, for the grouped long-segment kernel: group g
    // is gproj[gbeg[g]] .. gproj[gbeg[g+1] - 1]
    int32_t n_groups;
    int8_t gbeg[LORA_MAX_PROJ + 1];
    int8_t gproj[LORA_MAX_PROJ];
    ShrinkProj p[LORA_MAX_PROJ];
};

// One workgroup = one short-segment work item (at most 16 rows x one K
// slice) of one projection.  With KSPLIT = 4 (the configuration in use) the
// four waves share the item's 16 rows and take every 4th 64-wide K block;
// partial sums are added in LDS in wave order.  (KSPLIT = 1 would give wave w
// rows [16*MTW*w, 16*MTW*(w+1)); long segments use shrink_rows_kernel.)
// NT = number of 16-wide rank tiles; U = K blocks loaded ahead per step.
template <int KSPLIT, int MTW, int NT, int U>
__device__ __forceinline__ void shrink_item(const ShrinkArgs& args, const int bx, const int by) {
    const lora_work_t it = args.work[args.begin + bx];
    const ShrinkProj P = args.p[by];  // by value: its fields load in one batch
    if (!item_live(args.live, bx) || !item_ok(it, args.n_active, args.v_slices, P.A, 16 * NT) ||
        it.nrows > 16 * MTW * (KSPLIT > 1 ? 1 : 4))
        return;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int li = lane & 15, lg = lane >> 4;
    const int mbase = KSPLIT > 1 ? 0 : wave * 16 * MTW;
    if (KSPLIT == 1 && mbase >= it.nrows) return;  // no barrier in this configuration

    // x rows of this lane (rows past the item read its last row; their
    // results are not stored)
    const uint16_t* xrow[MTW];
#pragma unroll
    for (int t = 0; t < MTW; ++t) {
        const int m = mbase + 16 * t + li;
        xrow[t] = P.x + (int64_t)args.row_index[it.row0 + min(m, it.nrows - 1)] * P.ldx + 16 * lg;
    }
    issue_fence();
    f32x4_t acc[MTW][NT];
#pragma unroll
    for (int t = 0; t < MTW; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // 64-wide K blocks [kbeg, kend) of this item's slice
    const int kblocks = P.d_in / 64;
    const int kbeg = (int)((int64_t)it.kslice * kblocks / it.nslices);
    const int kend = (int)((int64_t)(it.kslice + 1) * kblocks / it.nslices);
    const int cblocks = P.A.chunk_len / 64;
    for (int c = kbeg / cblocks; c * cblocks < kend; ++c) {
        // A rows of this lane's rank slots (slots past the rank read row
        // rank-1; their results are not stored)
        const uint16_t* arow[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int j = 16 * n + li;
            arow[n] = P.A.pool + P.A.row_off[off_index(P.A, it.adapter, min(j, it.rank - 1), c)] + 16 * lg;
        }
        issue_fence();
        const int cbase = c * cblocks;
        const int kb0 = max(cbase, kbeg);
        const int kb1 = min(cbase + cblocks, kend);
        // first block owned by this wave (blocks are dealt round-robin by global index)
        const int first = KSPLIT > 1 ? kb0 + ((wave - kb0 % KSPLIT) + KSPLIT) % KSPLIT : kb0;
        if (first >= kb1) continue;  // wave-uniform
        // Two register stages of U blocks each: the loads of the next stage are
        // issued before the MFMAs of the current one, so a wave always has a
        // stage in flight.  Blocks past the slice are not loaded (a
        // wave-uniform branch; their MFMAs are skipped).  Rows past the item
        // and rank slots past the rank read clamped, real rows; their outputs
        // are never stored, so no load is masked.
        const int last = first + (kb1 - 1 - first) / KSPLIT * KSPLIT;
        u32x4_t xs[2][U][MTW][2], as[2][U][NT][2];
        auto load_stage = [&](int st, int k0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * KSPLIT;
                if (k > last) break;  // wave-uniform
                const int64_t kx = (int64_t)k * 64, ka = (int64_t)(k - cbase) * 64;
#pragma unroll
                for (int t = 0; t < MTW; ++t) {
                    xs[st][u][t][0] = ld16(xrow[t] + kx);
                    xs[st][u][t][1] = ld16(xrow[t] + kx + 8);
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    as[st][u][n][0] = ld16(arow[n] + ka);
                    as[st][u][n][1] = ld16(arow[n] + ka + 8);
                }
            }
        };
        auto mma_stage = [&](int st, int k0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u > 0 && k0 + u * KSPLIT > last) break;  // wave-uniform; k0 <= last
                // every rank tile, used or not: straight-line MFMAs (a tile
                // past the rank only adds to results that are not stored)
#pragma unroll
                for (int t = 0; t < MTW; ++t)
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        acc[t][n] = mfma_bf16(xs[st][u][t][0], as[st][u][n][0], acc[t][n]);
                        acc[t][n] = mfma_bf16(xs[st][u][t][1], as[st][u][n][1], acc[t][n]);
                    }
            }
        };
        // Empty asm that takes a stage's registers as in/out operands: placed
        // after the next stage's loads, it keeps those loads issued before
        // this stage's MFMAs (which consume its outputs), so the compiler can
        // neither sink the loads nor merge the two stages' registers.
        auto pin_stage = [&](int st) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int t = 0; t < MTW; ++t) {
                    asm volatile("" : "+v"(xs[st][u][t][0]));
                    asm volatile("" : "+v"(xs[st][u][t][1]));
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    asm volatile("" : "+v"(as[st][u][n][0]));
                    asm volatile("" : "+v"(as[st][u][n][1]));
                }
            }
        };
        constexpr int STEP = KSPLIT * U;
        int kb = first;
        load_stage(0, kb);
        for (;;) {
            load_stage(1, kb + STEP);
            pin_stage(0);
            mma_stage(0, kb);
            kb += STEP;
            if (kb > last) break;
            load_stage(0, kb + STEP);
            pin_stage(1);
            mma_stage(1, kb);
            kb += STEP;
            if (kb > last) break;
        }
    }

    if constexpr (KSPLIT > 1) {
        __shared__ f32x4_t red[KSPLIT - 1][NT][64];
        if (wave > 0)
#pragma unroll
            for (int n = 0; n < NT; ++n) red[wave - 1][n][lane] = acc[0][n];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[0][n] += red[w][n][lane];
    }
    // result lane layout: column j = 16n + li, rows 4*lg + e of tile t;
    // rank rows from neg_start on enter negated (deLoRA composite adapters)
    float* vout = P.v + (int64_t)it.kslice * args.n_active * P.ldv;
    const int jneg = neg_start(P.A, it.adapter, it.rank);
#pragma unroll
    for (int t = 0; t < MTW; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int j = 16 * n + li;
            if (j >= it.rank) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = mbase + 16 * t + 4 * lg + e;
                if (m < it.nrows) vout[(int64_t)(it.row0 + m) * P.ldv + j] = j >= jneg ? -acc[t][n][e] : acc[t][n][e];
            }
        }
}
template <int KSPLIT, int MTW, int NT, int U>
__global__ __launch_bounds__(WG) void shrink_kernel(ShrinkArgs args) {
    shrink_item<KSPLIT, MTW, NT, U>(args, blockIdx.x, blockIdx.y);
}
template <int KSPLIT, int MTW, int NT>
constexpr int unroll_for() {
    return KSPLIT > 1 ? (NT == 1 ? 4 : NT == 2 ? 2 : 1) : ((MTW + NT) <= 2 ? 2 : 1);
}
// The short-segment items of rank classes 0-2 (ranks up to 64) of a host
// plan in one launch: the item's rank picks the instance (a branch on a
// wave-uniform value), which computes exactly what that class's own launch
// computes.  The ranges lie back to back in the work list in class order; the
// grid takes them from the last (most rank tiles, most bytes per item) to the
// first, so the heaviest items are dispatched first and the launch does not
// end on a tail of them.  (One launch instead of three: 70B-mix shrink
// 192.8 -> 183.6 us.)
template <int KSPLIT, int MTW>
__global__ __launch_bounds__(WG) void shrink_classes_kernel(ShrinkArgs args) {
    const int bx = args.count - 1 - (int)blockIdx.x;
    const int rank = __builtin_amdgcn_readfirstlane(args.work[args.begin + bx].rank);
    if (rank <= 16)
        shrink_item<KSPLIT, MTW, 1, unroll_for<KSPLIT, MTW, 1>()>(args, bx, blockIdx.y);
    else if (rank <= 32)
        shrink_item<KSPLIT, MTW, 2, unroll_for<KSPLIT, MTW, 2>()>(args, bx, blockIdx.y);
    else
        shrink_item<KSPLIT, MTW, 4, unroll_for<KSPLIT, MTW, 4>()>(args, bx, blockIdx.y);
}
// The same for a device-built plan's launch group of those classes: a grid of
// at most the resident workgroups walks the group's live items, heaviest
// class first (the barrier after each item keeps the next item's LDS writes
// behind its reads).
template <int KSPLIT, int MTW>
__global__ __launch_bounds__(WG) void shrink_classes_loop_kernel(ShrinkArgs args) {
    const int live = *args.live;
    for (int i = blockIdx.x; i < live; i += gridDim.x) {
        const int bx = live - 1 - i;
        const int rank = __builtin_amdgcn_readfirstlane(args.work[args.begin + bx].rank);
        if (rank <= 16)
            shrink_item<KSPLIT, MTW, 1, unroll_for<KSPLIT, MTW, 1>()>(args, bx, blockIdx.y);
        else if (rank <= 32)
            shrink_item<KSPLIT, MTW, 2, unroll_for<KSPLIT, MTW, 2>()>(args, bx, blockIdx.y);
        else
            shrink_item<KSPLIT, MTW, 4, unroll_for<KSPLIT, MTW, 4>()>(args, bx, blockIdx.y);
        __syncthreads();
    }
}
// Device-built plans: a grid of at most the resident workgroups walks the
// range's live items (every wave reaches each barrier of an item, and the
// barrier after it keeps the next item's LDS writes behind its reads).
template <int KSPLIT, int MTW, int NT, int U>
__global__ __launch_bounds__(WG) void shrink_loop_kernel(ShrinkArgs args) {
    const int live = *args.live;
    for (int bx = blockIdx.x; bx < live; bx += gridDim.x) {
        shrink_item<KSPLIT, MTW, NT, U>(args, bx, blockIdx.y);
        __syncthreads();
    }
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global loads (a __syncthreads() fence would also drain the global loads
// that are in flight for the next K block).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Long segments (items of 64*MTW rows; wave w computes rows 16*MTW*w ..).
// Both operands of a 64-wide K step pass through LDS: the x tile (64*MTW rows
// x 128 B) and the A tile (16*NT rank rows x 128 B) are fetched with direct
// global-to-LDS loads (global_load_lds_dwordx4: lane l of a wave's load
// lands in LDS slot base + 16*l), eight lanes per row, so every load covers
// eight whole 128 B lines and A is read once per workgroup.  Fetching MFMA
// fragments straight from memory would touch 16 rows per load and use half
// of each line, and every wave would fetch A: the L1 request rate, not HBM,
// would bound the kernel.  A row's eight 16 B pieces are stored XOR-swizzled
// by (row mod 8), so the eight lanes of a fragment read that share a piece
// index hit eight different bank groups; with direct loads the swizzle is
// applied to the source address (lane l of a row fetches piece
// (l mod 8) ^ (row mod 8)).
// K order inside a step: lane group lg takes pieces lg and lg+4 (elements
// 8*lg .. +7 and 32 + 8*lg .. +7) for its two MFMAs; x and A use the same
// order.
// Pipeline: NBUF LDS buffers; the loads of step i+NBUF-1 are issued before
// the MFMAs of step i, and one barrier per step (after this wave's loads of
// step i+1 have landed) hands the buffers over.  Every wave issues the same
// number of loads per step (with one rank tile, waves 2 and 3 repeat the A
// loads of waves 0 and 1: the same bytes to the same LDS slots), and these
// are the only vector-memory loads during the steps, so the wait counts are
// exact.
// One direct global-to-LDS load of 16 B per lane: lane l's bytes land in
// LDS at dst + 16*l (dst is the same for the whole wave).  Issued as inline
// asm: the compiler's own wait insertion, which knows the builtin writes LDS,
// would wait for every load in flight before each LDS read, including the
// next step's prefetch.  The caller waits for these loads itself (vmcnt(0)
// before the step barrier); compiler-issued loads stay correct because the
// counter is in order (its waits can only over-wait for these).
__device__ __forceinline__ void dma16(const void* src, u32x4_t* dst) {
    const unsigned lds = (unsigned)(uintptr_t)((__attribute__((address_space(3))) u32x4_t*)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
// Barrier once this wave has at most N vector-memory operations in flight
// and no LDS operation.
template <int N>
__device__ __forceinline__ void step_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One task: item `it` for the G projections pj[0..G) that share x (the same
// x, ldx and d_in): each x tile is loaded once and multiplied by the G A
// tiles (a q/k/v group reads x once instead of three times).  G = 1 is the
// plain per-projection task.  The LDS holds GS A buffers per stage.
template <int MTW, int NT, int G, int GS, bool WHOLE_ROWS, int NBUF>
__device__ __forceinline__ void shrink_rows_task(const ShrinkArgs& args, const lora_work_t& it, const int (&pj)[4],
                                                 u32x4_t* sX, u32x4_t* sA) {
    constexpr int ROWS = 64 * MTW;           // rows of the item tile
    constexpr int XBUF = ROWS * 8;           // x pieces per LDS buffer
    constexpr int ABUF = 16 * NT * 8;        // A pieces per LDS buffer and projection (NT rank tiles)
    constexpr int ASTRIDE = GS * ABUF;       // A pieces per LDS stage
    constexpr int XW = XBUF / WG;            // x loads per lane (wave-loads per wave)
    constexpr int AWT = ABUF / 64;           // A wave-loads of the workgroup, per projection
    constexpr int AW = AWT >= 4 ? AWT / 4 : 1;  // A wave-loads per wave, per projection
    constexpr int DPW = XW + G * AW;         // loads per wave per step
    const int t = threadIdx.x, lane = t & 63, wave = wave_id();
    const int li = lane & 15, lg = lane >> 4;
    const int mbase = wave * 16 * MTW;
    const ShrinkProj& P0 = args.p[pj[0]];

    // x sources: wave-load j of this wave fills slots (XW*wave + j)*64 + lane
    const uint16_t* xsrc[XW];
#pragma unroll
    for (int j = 0; j < XW; ++j) {
        const int row = (XW * wave + j) * 8 + (lane >> 3);
        const int pc = (lane & 7) ^ (row & 7);
        // rows past the item read its last row (results not stored)
        xsrc[j] = P0.x + (int64_t)args.row_index[it.row0 + min(row, it.nrows - 1)] * P0.ldx + 8 * pc;
    }
    const int kblocks = P0.d_in / 64;
    const int kbeg = (int)((int64_t)it.kslice * kblocks / it.nslices);
    const int kend = (int)((int64_t)(it.kslice + 1) * kblocks / it.nslices);
    // A sources: wave-load j of this wave fills slots aw*64 + lane, aw =
    // (AW*wave + j) mod AWT (rank row aw*8 + lane/8, clamped to the rank);
    // with whole A rows in one chunk the row pointers are fixed, otherwise
    // each step looks its chunk up
    int arow[AW], apc[AW], cblocks[G];
    bool one_chunk = true;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        cblocks[g] = args.p[pj[g]].A.chunk_len / 64;
        one_chunk = one_chunk && (WHOLE_ROWS || kbeg / cblocks[g] == (kend - 1) / cblocks[g]);
    }
    const uint16_t* asrc[G][AW];
#pragma unroll
    for (int j = 0; j < AW; ++j) {
        const int row = ((AW * wave + j) % AWT) * 8 + (lane >> 3);
        arow[j] = min(row, it.rank - 1);
        apc[j] = (lane & 7) ^ (row & 7);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const Rows& A = args.p[pj[g]].A;
            const int c0 = kbeg / cblocks[g];
            // element offset of global K step 0 in this chunk's addressing
            // (the loads add k*64 for k inside the chunk, so every address
            // is in it)
            asrc[g][j] = A.pool + (A.row_off[off_index(A, it.adapter, arow[j], c0)] -
                                   (int64_t)c0 * cblocks[g] * 64 + 8 * apc[j]);
        }
    }
    f32x4_t acc[G][MTW][NT];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < MTW; ++q)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[g][q][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto fetch = [&](int k, int buf) {  // global K step k -> LDS buffer buf
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < AW; ++j) {
                const uint16_t* src;
                if (one_chunk) {
                    src = asrc[g][j] + (int64_t)k * 64;
                } else {
                    const Rows& A = args.p[pj[g]].A;
                    const int c = k / cblocks[g];
                    src = A.pool + A.row_off[off_index(A, it.adapter, arow[j], c)] +
                          (int64_t)(k - c * cblocks[g]) * 64 + 8 * apc[j];
                }
                dma16(src, sA + buf * ASTRIDE + g * ABUF + ((AW * wave + j) % AWT) * 64);
            }
#pragma unroll
        for (int j = 0; j < XW; ++j)
            dma16(xsrc[j] + (int64_t)k * 64, sX + buf * XBUF + (XW * wave + j) * 64);
    };
    auto mma = [&](int buf) {
        const u32x4_t* X = sX + buf * XBUF;
        u32x4_t xf[MTW][2];
#pragma unroll
        for (int q = 0; q < MTW; ++q) {
            const int row = mbase + 16 * q + li;
            xf[q][0] = X[row * 8 + (lg ^ (li & 7))];
            xf[q][1] = X[row * 8 + ((lg + 4) ^ (li & 7))];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const u32x4_t* A = sA + buf * ASTRIDE + g * ABUF;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int row = 16 * n + li;
                const u32x4_t a0 = A[row * 8 + (lg ^ (li & 7))];
                const u32x4_t a1 = A[row * 8 + ((lg + 4) ^ (li & 7))];
#pragma unroll
                for (int q = 0; q < MTW; ++q) {
                    acc[g][q][n] = mfma_bf16(xf[q][0], a0, acc[g][q][n]);
                    acc[g][q][n] = mfma_bf16(xf[q][1], a1, acc[g][q][n]);
                }
            }
        }
    };
    // Steps start at a point that depends on (adapter, first projection of
    // the group, K slice).  x rows and A rows lie a power-of-two distance
    // apart, so workgroups that read the same step in lock-step all hit the
    // same address bits; spreading the starting steps spreads the traffic.
    // The start is the same for every item of a segment and for every storage
    // layout, so a row's sum order (and hence its result, to the bit) depends
    // on neither which item holds it nor how A is paged.
    const int nb = kend - kbeg;
    const unsigned h = (unsigned)it.adapter * 2654435761u ^ ((unsigned)pj[0] * 40503u + (unsigned)it.kslice * 977u);
    const int rot = nb > 0 ? (int)((h >> 7) % (unsigned)nb) : 0;  // nb = 0: a slice past a narrow projection's d_in
    auto step = [&](int i) { return kbeg + (i + rot < nb ? i + rot : i + rot - nb); };
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b)
        if (b < nb) fetch(step(b), b);
    if (nb >= NBUF - 1)
        step_barrier<(NBUF - 2) * DPW>();  // step 0 has landed
    else
        step_barrier<0>();
    for (int i = 0; i < nb; ++i) {
        const int ahead = i + NBUF - 1;
        if (ahead < nb) fetch(step(ahead), ahead % NBUF);
        mma(i % NBUF);
        // step i+1 has landed and every wave is done with step i's buffer
        if (ahead < nb)
            step_barrier<(NBUF - 2) * DPW>();
        else
            step_barrier<0>();
    }
    if (mbase >= it.nrows) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const ShrinkProj& P = args.p[pj[g]];
        float* vout = P.v + (int64_t)it.kslice * args.n_active * P.ldv;
        const int jneg = neg_start(P.A, it.adapter, it.rank);  // deLoRA: negated rank rows
#pragma unroll
        for (int q = 0; q < MTW; ++q)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int j = 16 * n + li;
                if (j >= it.rank) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = mbase + 16 * q + 4 * lg + e;
                    if (m < it.nrows)
                        vout[(int64_t)(it.row0 + m) * P.ldv + j] = j >= jneg ? -acc[g][q][n][e] : acc[g][q][n][e];
                }
            }
    }
}

// Persistent: workgroup g takes tasks g, g + G, ... of the launch's tasks;
// the launcher sizes the grid so that every workgroup gets the same number of
// tasks and all are resident.  With GS = 1 a task is (item, projection); with
// GS > 1 it is (item, group of up to GS projections that share x).  The
// item's rank picks the number of rank tiles (1, 2 or 4 up to NTMAX = 4;
// NTMAX = 8 is its own kernel for ranks above 64, whose registers and LDS
// would lower the occupancy of the others).
template <int MTW, int NTMAX, bool WHOLE_ROWS, int GS>
__global__ __launch_bounds__(WG) void shrink_rows_kernel(ShrinkArgs args) {
    // LDS stages: three steps in flight (96 KiB with one projection per task
    // and rank <= 64: one workgroup per CU; measured against two and three
    // stages: prefill -11%, vision -1%, 70B mix +1%; 128 KiB above rank 64,
    // where one step in flight was 4% slower on the class heads; 160 KiB with
    // three A tiles per stage)
    constexpr int NBUF = 4;
    __shared__ u32x4_t sX[NBUF * 64 * MTW * 8];         // NBUF buffers x 64*MTW rows x 8 pieces of 16 B
    __shared__ u32x4_t sA[NBUF * GS * 16 * NTMAX * 8];  // NBUF x GS buffers x 16*NT rank rows x 8 pieces
    const int n_units = GS == 1 ? args.n_proj : args.n_groups;
    const int count = args.live ? min(args.count, *args.live) : args.count;
    const int ntasks = count * n_units;
    for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
        const int unit = task / count;
        const lora_work_t it = args.work[args.begin + task - unit * count];
        int pj[4] = {unit, unit, unit, unit};
        int ng = 1;
        if (GS > 1) {
            const int g0 = args.gbeg[unit];
            ng = args.gbeg[unit + 1] - g0;
#pragma unroll
            for (int g = 0; g < 4; ++g) pj[g] = args.gproj[g0 + (g < ng ? g : 0)];
        }
        // uniform over the workgroup: a skipped task skips no barrier
        bool ok = (it.nrows <= 64 * MTW) & (ng >= 1) & (ng <= GS);
#pragma unroll
        for (int g = 0; g < GS; ++g)
            if (g < ng) ok = ok & item_ok(it, args.n_active, args.v_slices, args.p[pj[g]].A, 16 * NTMAX);
        if (!ok) continue;
        if (NTMAX == 8) {
            shrink_rows_task<MTW, 8, 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
        } else if (ng == 1 || GS == 1) {
            if (it.rank > 32)
                shrink_rows_task<MTW, 4, 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
            else if (it.rank > 16)
                shrink_rows_task<MTW, 2, 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
            else
                shrink_rows_task<MTW, 1, 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
        } else if (ng == 2) {
            if (it.rank > 32)
                shrink_rows_task<MTW, 4, 2 <= GS ? 2 : 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
            else if (it.rank > 16)
                shrink_rows_task<MTW, 2, 2 <= GS ? 2 : 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
            else
                shrink_rows_task<MTW, 1, 2 <= GS ? 2 : 1, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
        } else {
            if (it.rank > 32)
                shrink_rows_task<MTW, 4, GS, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
            else if (it.rank > 16)
                shrink_rows_task<MTW, 2, GS, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
            else
                shrink_rows_task<MTW, 1, GS, GS, WHOLE_ROWS, NBUF>(args, it, pj, sX, sA);
        }
    }
}

// ------------------------------------------------------------------ expand
struct ExpandProj {
    const float* v;
    int64_t ldv;
    Rows B;
    int32_t d_out;
    float* y;
    int64_t ldy;
    float scale;
    int32_t cg_begin;  // first column group (grid.y) of this projection
};
struct ExpandArgs {
    const int32_t* row_index;
    const lora_work_t* work;
    const int32_t* live;  // device-built plan: items of the range (NULL: all `count`)
    int32_t begin;
    int32_t n_active;
    int32_t v_slices;
    int32_t n_proj;
    int32_t count;   // work items of the launch (MFMA expand: 1-D grid of count x groups)
    int32_t groups;  // column groups of all projections
    ExpandProj p[LORA_MAX_PROJ];
};

// The projection that column group `cg` belongs to: a count of the
// projections whose groups start at or before it, so that the launch's
// start columns are read in one batch rather than one after the other.
__device__ __forceinline__ int proj_of_group(const ExpandArgs& args, int cg) {
    int pi = 0;
#pragma unroll
    for (int i = 1; i < LORA_MAX_PROJ; ++i) pi += (i < args.n_proj) & (cg >= args.p[i].cg_begin);
    return pi;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  The MFMA expand's 1-D grid (a multiple of 8) is remapped so that XCD x
// takes the contiguous block x*G/8 .. (x+1)*G/8 - 1 of logical ids, ordered
// item-major: all column groups of an item (which share its v rows) and the
// neighbouring items of a segment (which share its B strips) then meet in
// one L2 instead of being fetched again by every XCD.
#define N_XCD 8
__device__ __forceinline__ int xcd_block(int wg, int n_wg) { return (wg % N_XCD) * (n_wg / N_XCD) + wg / N_XCD; }

// One workgroup = one work item (at most EXPAND_ROWS rows) x one 512-column
// group of one projection; wave w owns columns [128w, 128w+128) of the
// group.  v (the sum of the row's K slices, in slice order) is split as hi +
// lo bf16 (two MFMAs, so the product keeps ~16 mantissa bits of v) once per
// workgroup into LDS; the wave loads and transposes its B strip once (KS
// steps of 32 ranks), then walks the item's rows 16 at a time, loading the
// next tile's y while the current one is computed; y is read, updated and
// written in fp32.
#define EXPAND_ROWS 128
template <int KS>
__device__ __forceinline__ void expand_item(const ExpandArgs& args, const int lid) {
    constexpr int G = 4 * KS;  // groups of 8 ranks
    __shared__ int32_t s_rows[EXPAND_ROWS];          // the item's y row indices
    __shared__ u32x4_t s_v[EXPAND_ROWS * 2 * G];     // per row: (hi, lo) x G groups, XOR-swizzled
    if (lid >= args.count * args.groups) return;      // padding of the grid to a multiple of 8
    const int item = lid / args.groups, cg = lid - item * args.groups;
    const lora_work_t it = args.work[args.begin + item];
    // the projection by value: its fields are loaded in one batch, before
    // the checks branch on them
    const ExpandProj P = args.p[proj_of_group(args, cg)];
    // uniform over the workgroup, so returning here skips no barrier
    if (!(item_live(args.live, item) && item_ok(it, args.n_active, args.v_slices, P.B, 32 * KS) &
          (it.nrows <= EXPAND_ROWS)))
        return;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int li = lane & 15, lg = lane >> 4;
    // The wave's 128 columns are two halves of 64 (d_out is a multiple of
    // 64, so each half is wholly in or out of range, and lies in one chunk
    // of B).  Lane li owns columns 4*li .. +3 of each half: one 16 B y load
    // or store of the 16 lanes of a row group then covers 256 contiguous
    // bytes of the row (two whole lines).  MFMA c (c < 4) produces column
    // 4*li + c of the first half, MFMA c + 4 the same of the second half.
    const int col0 = (cg - P.cg_begin) * 512 + wave * 128;
    const bool wave_ok = col0 < P.d_out;  // wave-uniform; waves past d_out only help with the LDS tables
    const bool hi_ok = col0 + 64 < P.d_out;
    const int nlo = wave_ok ? col0 + 4 * li : 0;         // in-bounds columns for halves past d_out
    const int nhi = hi_ok ? col0 + 64 + 4 * li : nlo;
    const int clo = nlo / P.B.chunk_len, chi = nhi / P.B.chunk_len;
    const int inlo = nlo - clo * P.B.chunk_len, inhi = nhi - chi * P.B.chunk_len;

    // B strip: all row offsets, then all rows (masked to real ranks and
    // columns), then the register transpose
    int64_t blo[KS][8], bhi[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = min(32 * ks + 8 * lg + e, it.rank - 1);
            blo[ks][e] = P.B.row_off[off_index(P.B, it.adapter, j, clo)];
            bhi[ks][e] = P.B.row_off[off_index(P.B, it.adapter, j, chi)];
        }
    issue_fence();
    u32x4_t bop[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4_t rows[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool rk = 32 * ks + 8 * lg + e < it.rank;
            const u32x2_t lo = ld8_if(wave_ok && rk, P.B.pool + blo[ks][e] + inlo);
            const u32x2_t hi = ld8_if(hi_ok && rk, P.B.pool + bhi[ks][e] + inhi);
            rows[e] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
        transpose8x8(rows, bop[ks]);
    }

    // LDS tables: row indices, and v summed over its slices (in slice
    // order), zero past the rank, split into bf16 hi + lo.  Piece (g, h) of
    // row m (h = 0 hi, 1 lo) sits at slot m*2G + ((2g + h) ^ (m & 7)), so the
    // eight lanes of a fragment read that share g and h hit eight bank groups.
    const int64_t vslice = (int64_t)args.n_active * P.ldv;
    if ((int)threadIdx.x < it.nrows) s_rows[threadIdx.x] = args.row_index[it.row0 + threadIdx.x];
    for (int u = threadIdx.x; u < it.nrows * G; u += WG) {
        const int m = u / G, g = u - m * G, j0 = 8 * g;
        // columns j .. j+3 when they start below the rank, else column 0
        // (in the row: ldv is a multiple of 4 and at least the rank)
        const int ja = j0 < it.rank ? j0 : 0, jb = j0 + 4 < it.rank ? j0 + 4 : 0;
        const float* vrow = P.v + (int64_t)(it.row0 + m) * P.ldv;
        f32x4_t a = ldf4(vrow + ja), b = ldf4(vrow + jb);
        for (int sl = 1; sl < it.nslices; ++sl) {
            a += ldf4(vrow + sl * vslice + ja);
            b += ldf4(vrow + sl * vslice + jb);
        }
        float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        u32x4_t vh, vl;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (j0 + e >= it.rank) f[e] = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t h = pack_bf16(f[2 * q], f[2 * q + 1]);
            vh[q] = h;
            vl[q] = pack_bf16(f[2 * q] - bf16_lo(h), f[2 * q + 1] - bf16_hi(h));
        }
        s_v[m * 2 * G + ((2 * g) ^ (m & 7))] = vh;
        s_v[m * 2 * G + ((2 * g + 1) ^ (m & 7))] = vl;
    }

    // One 16-row tile = y rows 4*lg + e (this lane's outputs) and v row li
    // (this lane's MFMA operand).  Tile 0's y is loaded before the tables
    // are complete; the loads of tile mt+1 are issued before tile mt is
    // computed and stored.
    const int ntiles = (it.nrows + 15) / 16;
    f32x4_t ys[2][4][2];
    auto yrow_of = [&](int mt, int e) {
        const int mm = min(16 * mt + 4 * lg + e, it.nrows - 1);
        return P.y + (int64_t)args.row_index[it.row0 + mm] * P.ldy;
    };
    auto yrow_lds = [&](int mt, int e) {
        const int mm = min(16 * mt + 4 * lg + e, it.nrows - 1);
        return P.y + (int64_t)s_rows[mm] * P.ldy;
    };
    auto load_tile = [&](int st, const float* const (&yr)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ys[st][e][0] = ldf4(yr[e] + nlo);
            ys[st][e][1] = ldf4(yr[e] + nhi);
        }
    };
    {
        const float* yr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) yr[e] = yrow_of(0, e);
        if (wave_ok) load_tile(0, yr);
    }
    lds_barrier();
    if (!wave_ok) return;  // no barrier follows

    auto compute_tile = [&](int st, int mt) {
        const int m = min(16 * mt + li, it.nrows - 1);  // rows past the item: results not stored
        u32x4_t vhi[KS], vlo[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int g = 4 * ks + lg;
            vhi[ks] = s_v[m * 2 * G + ((2 * g) ^ (m & 7))];
            vlo[ks] = s_v[m * 2 * G + ((2 * g + 1) ^ (m & 7))];
        }
        f32x4_t acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc[c] = mfma_bf16(vhi[ks], bop[ks][c], acc[c]);
                acc[c] = mfma_bf16(vlo[ks], bop[ks][c], acc[c]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (16 * mt + 4 * lg + e >= it.nrows) continue;
            float* yr = yrow_lds(mt, e);
            f32x4_t o0, o1;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o0[c] = __builtin_fmaf(P.scale, acc[c][e], ys[st][e][0][c]);
                o1[c] = __builtin_fmaf(P.scale, acc[c + 4][e], ys[st][e][1][c]);
            }
            stf4(yr + nlo, o0);  // the wave's first half is in range (wave_ok)
            if (hi_ok) stf4(yr + nhi, o1);
        }
    };
    auto pin = [&](int st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            asm volatile("" : "+v"(ys[st][e][0]));
            asm volatile("" : "+v"(ys[st][e][1]));
        }
    };
    auto fetch = [&](int st, int mt) {
        const float* yr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) yr[e] = yrow_lds(mt, e);
        load_tile(st, yr);
    };
    for (int mt = 0;;) {
        // tile mt is in stage 0; fetch tile mt+1 (the last tile again at the
        // end: in bounds, never used)
        fetch(1, min(mt + 1, ntiles - 1));
        issue_fence();
        pin(0);
        compute_tile(0, mt);
        if (++mt >= ntiles) break;
        fetch(0, min(mt + 1, ntiles - 1));
        issue_fence();
        pin(1);
        compute_tile(1, mt);
        if (++mt >= ntiles) break;
    }
}
template <int KS>
__global__ __launch_bounds__(WG) void expand_kernel(ExpandArgs args) {
    expand_item<KS>(args, xcd_block((int)blockIdx.x, (int)gridDim.x));
}
// Device-built plans: the live (item, column group) pairs are split into 8
// contiguous shares, one per XCD (workgroup b runs on XCD b mod 8), and the
// XCD's workgroups walk its share; the grid is a multiple of 8 and need not
// match the live count.
template <int KS>
__global__ __launch_bounds__(WG) void expand_loop_kernel(ExpandArgs args) {
    const int total = *args.live * args.groups;
    const int x = (int)blockIdx.x % N_XCD, per_xcd = (int)gridDim.x / N_XCD;
    const int lo = (int)((int64_t)x * total / N_XCD), hi = (int)((int64_t)(x + 1) * total / N_XCD);
    for (int lid = lo + (int)blockIdx.x / N_XCD; lid < hi; lid += per_xcd) {
        expand_item<KS>(args, lid);
        __syncthreads();
    }
}

// One workgroup = one work item of at most BGMV_ROWS rows x one 512-column
// group of one projection (decode rows: BGMV).  Lane l of every wave owns
// columns 8l .. 8l+7 of the group; wave w takes the rank groups w and w + 4
// (16 ranks each: ranks 16w .. 16w+15, then 64+16w ..), so the B rows of up
// to 64 ranks are in flight at once, one round trip for their row offsets and
// one for the rows.  Each wave forms its partial sum_j v[row][j] * B[j][n]
// over its ranks with fp32 FMAs in rank order (v[row][j] loaded by one lane,
// its K slices summed in slice order, and broadcast with readlane); the
// partials of the four waves are added in wave order through LDS, and
// y[row][n] += s * that sum, each wave storing 128 of the columns.  With UNI
// (every chunk_len a multiple of 512, so that the group's 512 columns lie in
// one chunk of B) the row offsets are wave-uniform and come through the
// scalar cache.
#define BGMV_ROWS 2
#define BGMV_COLS 512
template <bool UNI>
__device__ __forceinline__ void bgmv_item(const ExpandArgs& args, const int bx, const int by) {
    __shared__ f32x4_t s_part[4][BGMV_ROWS][2][64];  // [wave][row][half][lane]: 16 KiB
    const lora_work_t it = args.work[args.begin + bx];
    const ExpandProj P = args.p[proj_of_group(args, by)];  // by value, as in expand_item
    // uniform over the workgroup, so returning here skips no barrier
    if (!item_live(args.live, bx) || !item_ok(it, args.n_active, args.v_slices, P.B, LORA_MAX_RANK) ||
        it.nrows > BGMV_ROWS)
        return;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g0 = (by - P.cg_begin) * BGMV_COLS;
    const int n0 = g0 + 8 * lane;
    const bool col_ok = n0 < P.d_out;
    const int nc = col_ok ? n0 : g0;  // g0 < d_out: the grid covers d_out
    const int cchunk = (UNI ? __builtin_amdgcn_readfirstlane(nc) : nc) / P.B.chunk_len;
    const int cin = nc - cchunk * P.B.chunk_len;
    const int64_t vslice = (int64_t)args.n_active * P.ldv;

    // this wave's rank groups: j0 = 16w (and 64 + 16w for ranks above 64)
    const int ja = 16 * wave, jb = 64 + 16 * wave;
    // lane l < 16 holds v[row][ja + l], lane 16 <= l < 32 v[row][jb + l - 16]
    float vsum[BGMV_ROWS];
    {
        const int j = lane < 16 ? ja + lane : jb + lane - 16;
        const bool jok = lane < 32 && j < it.rank;
#pragma unroll
        for (int p = 0; p < BGMV_ROWS; ++p) {
            const bool ok = jok && p < it.nrows;
            const float* vp = P.v + (int64_t)(it.row0 + min(p, it.nrows - 1)) * P.ldv + (ok ? j : 0);
            float t = 0.f;
            for (int sl = 0; sl < it.nslices; ++sl)
                if (ok) t += vp[sl * vslice];
            vsum[p] = t;
        }
    }
    f32x4_t acc0[BGMV_ROWS], acc1[BGMV_ROWS];
#pragma unroll
    for (int p = 0; p < BGMV_ROWS; ++p) acc0[p] = acc1[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // y of the columns this thread stores (see below), loaded with the first
    // group's B rows
    const int q = 16 * wave + (lane >> 2), part = lane & 3;
    const int nq = g0 + 8 * q + 2 * part;
    const bool q_ok = nq < P.d_out;
    int32_t yidx[BGMV_ROWS];
    float2 y0[BGMV_ROWS];
    // one rank group: row offsets, the 16 rows, then the FMAs in rank order
    auto group = [&](int j0, int vl0) {
        int64_t boff[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t i = off_index(P.B, it.adapter, min(j0 + e, it.rank - 1), cchunk);
            boff[e] = UNI ? ld_uniform(P.B.row_off, i) : P.B.row_off[i];
        }
        issue_fence();
        u32x4_t rows[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) rows[e] = ld16_if(col_ok && j0 + e < it.rank, P.B.pool + boff[e] + cin);
        if (vl0 == 0) {
#pragma unroll
            for (int p = 0; p < BGMV_ROWS; ++p) {
                const bool ok = q_ok && p < it.nrows;
                y0[p] = ok ? *reinterpret_cast<const float2*>(P.y + (int64_t)yidx[p] * P.ldy + nq) : float2{0.f, 0.f};
            }
        }
        issue_fence();
        // rank by rank: each row's 8 values are widened once and used for
        // both output rows (row-major would keep all 16 rows widened)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const u32x4_t r = rows[e];
            const float f[8] = {bf16_lo(r[0]), bf16_hi(r[0]), bf16_lo(r[1]), bf16_hi(r[1]),
                                bf16_lo(r[2]), bf16_hi(r[2]), bf16_lo(r[3]), bf16_hi(r[3])};
#pragma unroll
            for (int p = 0; p < BGMV_ROWS; ++p) {
                const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vsum[p]), vl0 + e));
                const float w = j0 + e < it.rank ? vj : 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc0[p][c] = __builtin_fmaf(w, f[c], acc0[p][c]);
                    acc1[p][c] = __builtin_fmaf(w, f[4 + c], acc1[p][c]);
                }
            }
        }
    };
#pragma unroll
    for (int p = 0; p < BGMV_ROWS; ++p) {
        yidx[p] = args.row_index[it.row0 + min(p, it.nrows - 1)];
        y0[p] = float2{0.f, 0.f};
    }
    // the wave's groups in turn (a loop, so that the second group's rows do
    // not take registers of their own)
    for (int j0 = ja, vl0 = 0; j0 < it.rank; j0 += 64, vl0 += 16) group(j0, vl0);
#pragma unroll
    for (int p = 0; p < BGMV_ROWS; ++p) {
        s_part[wave][p][0][lane] = acc0[p];
        s_part[wave][p][1][lane] = acc1[p];
    }
    // y: wave w stores the columns of lanes 16w .. 16w+15 (128 columns):
    // thread t = 64w + l handles lane q = 16w + l / 4, part (l & 3) of its
    // 8 columns (2 columns each)
    if (ja >= it.rank) {  // no group: load this thread's y here
#pragma unroll
        for (int p = 0; p < BGMV_ROWS; ++p) {
            const bool ok = q_ok && p < it.nrows;
            y0[p] = ok ? *reinterpret_cast<const float2*>(P.y + (int64_t)yidx[p] * P.ldy + nq) : float2{0.f, 0.f};
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < BGMV_ROWS; ++p) {
        if (p >= it.nrows || !q_ok) continue;
        float2 sum = {0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x4_t v = s_part[w][p][part >> 1][q];
            sum.x += (part & 1) ? v[2] : v[0];
            sum.y += (part & 1) ? v[3] : v[1];
        }
        stf2(P.y + (int64_t)yidx[p] * P.ldy + nq,
             f32x2_t{__builtin_fmaf(P.scale, sum.x, y0[p].x), __builtin_fmaf(P.scale, sum.y, y0[p].y)});
    }
}
template <bool UNI>
__global__ __launch_bounds__(WG) void bgmv_expand_kernel(ExpandArgs args) {
    bgmv_item<UNI>(args, blockIdx.x, blockIdx.y);
}
// Device-built plans: a grid of at most the resident workgroups walks the live items.
template <bool UNI>
__global__ __launch_bounds__(WG) void bgmv_expand_loop_kernel(ExpandArgs args) {
    const int live = *args.live;
    for (int bx = blockIdx.x; bx < live; bx += gridDim.x) {
        bgmv_item<UNI>(args, bx, blockIdx.y);
        __syncthreads();  // the next item's LDS writes wait for this one's reads
    }
}

// ------------------------------------------------------------------ fused (apply)
struct ApplyProj {
    const uint16_t* x;
    int64_t ldx;
    int32_t d_in;
    Rows A;
    Rows B;
    int32_t d_out;
    float* y;
    int64_t ldy;
    float scale;
};
struct FusedArgs {
    const int32_t* row_index;
    const lora_work_t* work;
    const int32_t* live;  // device-built plan: items of the range (NULL: every workgroup's)
    int32_t begin;
    int32_t n_active;
    ApplyProj p[LORA_MAX_PROJ];
    __device__ lora_work_t item(int i) const { return work[begin + i]; }
    __device__ int32_t row(int j) const { return row_index[j]; }
};
// The same for a small all-fused plan carried in the launch arguments: the
// items and the row index are read from the argument block (scalar loads),
// so the plan needs no device copy.
struct FusedInlineArgs {
    static constexpr const int32_t* live = nullptr;  // every item is in use
    int32_t begin;        // always 0
    int32_t n_active;
    ApplyProj p[LORA_MAX_PROJ];
    lora_work_t w[LORA_INLINE_ITEMS];
    int32_t rows[LORA_INLINE_ITEMS];
    __device__ lora_work_t item(int i) const { return w[i]; }
    __device__ int32_t row(int j) const { return rows[j]; }
};
static_assert(sizeof(FusedInlineArgs) <= 4096, "a kernel's arguments are at most 4 KiB");


// Sums of 8 values over the 64 lanes of a wave by reduce-scatter: at the
// steps 32, 16, 8 a lane keeps half of its remaining values and adds its
// partner's copy of them, then 4, 2, 1 are a plain butterfly on the one value
// left.  On return lane l holds the wave's sum of value 4*b5 + 2*b4 + b3
// (b_i = bit i of l); 10 cross-lane moves instead of 48.
__device__ __forceinline__ float wave_sum8(const float (&in)[8], int lane) {
    float a4[4], a2[2], a1;
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = b5 ? in[4 + i] : in[i], give = b5 ? in[i] : in[4 + i];
        a4[i] = keep + __shfl_xor(give, 32);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = b4 ? a4[2 + i] : a4[i], give = b4 ? a4[i] : a4[2 + i];
        a2[i] = keep + __shfl_xor(give, 16);
    }
    {
        const float keep = b3 ? a2[1] : a2[0], give = b3 ? a2[0] : a2[1];
        a1 = keep + __shfl_xor(give, 8);
    }
    a1 += __shfl_xor(a1, 4);
    a1 += __shfl_xor(a1, 2);
    a1 += __shfl_xor(a1, 1);
    return a1;
}

// One workgroup of FWG threads = one one-row work item of one projection:
// shrink, reduction and expand without v leaving the chip.  Thread t works on
// input elements and output columns 8c .. 8c+7 (c = t mod FWG/2; d_in, d_out
// <= 4*FWG) for ranks 8h .. 8h+7 of each group of 16 ranks (h = t / (FWG/2)).
// Per rank group: every thread forms its 8-element partial dot for each of its
// ranks, the partials are summed inside each wave (wave_sum8) and over the
// half's waves in wave order through LDS, and every thread then adds
// v[j] * B[j][n] for its ranks and columns; at the end the second half's
// column sums are added to the first half's through LDS (first half + second
// half, a fixed order) and the first half updates y.  Each thread loads its
// group's row offsets, then its 8 A rows and 8 B rows, so a decode row costs
// one round trip for metadata and one for data.  With UNI (every chunk_len a
// multiple of 512, so that a wave's 512 elements lie in one chunk) the row
// offsets are wave-uniform and come through the scalar cache.
#define FWG 1024
#define FHALF (FWG / 2)
template <bool UNI, typename Args>
__device__ __forceinline__ void fused_item(const Args& args, const int bx, const int by) {
    __shared__ float s_part[FWG / 64][8];
    __shared__ float s_v[16];
    __shared__ f32x4_t s_acc[FHALF][2];
    // the item and the projection by value: every field the workgroup needs
    // is loaded in one batch, before the checks branch on them
    const lora_work_t it = args.item(bx);
    const ApplyProj P = args.p[by];
    // uniform over the workgroup, so returning here skips no barrier
    if (!(item_live(args.live, bx) && item_ok(it, args.n_active, 1, P.A, LORA_MAX_RANK) & (it.nrows == 1) &
          (it.adapter < P.B.n_adapters) &
          (it.rank <= P.B.max_rank) & (P.d_in <= 8 * FHALF) & (P.d_out <= 8 * FHALF)))
        return;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int c = t & (FHALF - 1);
    const int h = __builtin_amdgcn_readfirstlane(t / FHALF);  // a wave lies in one half
    const int k0 = 8 * c, n0 = 8 * c;
    const bool k_ok = k0 < P.d_in, n_ok = n0 < P.d_out;
    const int kc = k_ok ? k0 : 0, nc = n_ok ? n0 : 0;  // in-bounds positions for idle threads
    // chunk of each lane's elements; with UNI the wave's first element decides
    const int kw = UNI ? __builtin_amdgcn_readfirstlane(kc) : kc;
    const int nw = UNI ? __builtin_amdgcn_readfirstlane(nc) : nc;
    const int ca = kw / P.A.chunk_len, cina = kc - ca * P.A.chunk_len;
    const int cb = nw / P.B.chunk_len, cinb = nc - cb * P.B.chunk_len;

    int32_t row = 0;
    int64_t aoff[8], boff[8];
    u32x4_t ar[8], br[8];
    // row offsets of this thread's 8 ranks of group g0 (and, for the first
    // group, the row index beside them), then (after a fence) their A and B
    // rows; rank slots past the rank read row rank-1 (zeroed)
    auto load_group = [&](int g0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = min(g0 + 8 * h + e, it.rank - 1);
            if (UNI) {
                aoff[e] = ld_uniform(P.A.row_off, off_index(P.A, it.adapter, j, ca));
                boff[e] = ld_uniform(P.B.row_off, off_index(P.B, it.adapter, j, cb));
            } else {
                aoff[e] = P.A.row_off[off_index(P.A, it.adapter, j, ca)];
                boff[e] = P.B.row_off[off_index(P.B, it.adapter, j, cb)];
            }
        }
        if (g0 == 0) row = args.row(it.row0);
        issue_fence();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ar[e] = ld16(P.A.pool + aoff[e] + cina);
            br[e] = ld16(P.B.pool + boff[e] + cinb);
        }
    };
    load_group(0);
    // y and x after the first group's rows (unconditional loads at clamped,
    // in-bounds positions; idle threads' values are zeroed or never stored),
    // so that waiting for x does not hold back the A and B loads
    float* const yp = P.y + (int64_t)row * P.ldy + nc;
    const f32x4_t y0 = ldf4(yp), y1 = ldf4(yp + 4);
    issue_fence();
    const u32x4_t xv = sel(k_ok, ld16(P.x + (int64_t)row * P.ldx + kc));
    float xf[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        xf[2 * q] = bf16_lo(xv[q]);
        xf[2 * q + 1] = bf16_hi(xv[q]);
    }
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int jneg = neg_start(P.A, it.adapter, it.rank);

    for (int g0 = 0; g0 < it.rank; g0 += 16) {
        if (g0 > 0) load_group(g0);
        const int jb = g0 + 8 * h;  // first rank of this thread's half
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ar[e] = sel(k_ok && jb + e < it.rank, ar[e]);
            br[e] = sel(n_ok && jb + e < it.rank, br[e]);
        }
        float part[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float d = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                d = __builtin_fmaf(xf[2 * q], bf16_lo(ar[e][q]), d);
                d = __builtin_fmaf(xf[2 * q + 1], bf16_hi(ar[e][q]), d);
            }
            part[e] = d;
        }
        const float ws = wave_sum8(part, lane);
        if ((lane & 7) == 0) s_part[wave][((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1)] = ws;
        __syncthreads();
        if (t < 16) {  // rank g0 + t: half t / 8, its waves in order
            const int hh = t >> 3, e = t & 7;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < FHALF / 64; ++w) v += s_part[hh * (FHALF / 64) + w][e];
            s_v[t] = g0 + t >= jneg ? -v : v;  // deLoRA: negated rank rows
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float vj = jb + e < it.rank ? s_v[8 * h + e] : 0.f;
            const u32x4_t r = br[e];
            acc0[0] = __builtin_fmaf(vj, bf16_lo(r[0]), acc0[0]);
            acc0[1] = __builtin_fmaf(vj, bf16_hi(r[0]), acc0[1]);
            acc0[2] = __builtin_fmaf(vj, bf16_lo(r[1]), acc0[2]);
            acc0[3] = __builtin_fmaf(vj, bf16_hi(r[1]), acc0[3]);
            acc1[0] = __builtin_fmaf(vj, bf16_lo(r[2]), acc1[0]);
            acc1[1] = __builtin_fmaf(vj, bf16_hi(r[2]), acc1[1]);
            acc1[2] = __builtin_fmaf(vj, bf16_lo(r[3]), acc1[2]);
            acc1[3] = __builtin_fmaf(vj, bf16_hi(r[3]), acc1[3]);
        }
        __syncthreads();  // s_part / s_v are reused by the next group
    }
    if (h == 1) {
        s_acc[c][0] = acc0;
        s_acc[c][1] = acc1;
    }
    __syncthreads();
    if (h == 0 && n_ok) {
        acc0 += s_acc[c][0];
        acc1 += s_acc[c][1];
        f32x4_t o0, o1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o0[q] = __builtin_fmaf(P.scale, acc0[q], y0[q]);
            o1[q] = __builtin_fmaf(P.scale, acc1[q], y1[q]);
        }
        stf4(yp, o0);
        stf4(yp + 4, o1);
    }
}
template <bool UNI>
__global__ __launch_bounds__(FWG) void fused_kernel(FusedArgs args) {
    fused_item<UNI>(args, blockIdx.x, blockIdx.y);
}
template <bool UNI>
__global__ __launch_bounds__(FWG) void fused_inline_kernel(FusedInlineArgs args) {
    fused_item<UNI>(args, blockIdx.x, blockIdx.y);
}
// Device-built plans: a grid of at most the resident workgroups walks the
// live rows (the barrier after each keeps the next row's LDS writes behind
// this one's reads).
template <bool UNI>
__global__ __launch_bounds__(FWG) void fused_loop_kernel(FusedArgs args) {
    const int live = *args.live;
    for (int bx = blockIdx.x; bx < live; bx += gridDim.x) {
        fused_item<UNI>(args, bx, blockIdx.y);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ merge
struct MergeMat {
    uint16_t* W;
    int64_t ldw;
    int32_t d_out, d_in;
    Rows A, B;
    int32_t adapter, rank;
    float scale;
    int32_t tiles_k;  // 512-column tiles along d_in
    int32_t tiles;    // total tiles of this matrix
};
struct MergeArgs {
    MergeMat m[LORA_MAX_MERGE];
};

// W passes the merge keeps in flight ahead of the one being computed.  The
// kernel runs two waves per SIMD at every rank: its A operands take 32 VGPRs
// per 32 ranks, 238 VGPRs in all at rank 128.
constexpr int MERGE_PREFETCH = 2;

// One workgroup = a 128 (rows n of W) x 512 (columns k) tile; wave w owns
// columns [128w, 128w+128).  First MFMA operand: B rows (rank x n) transposed
// so row slot i of MFMA c2 is n = nbase + 8*i + c2; second operand: A rows
// transposed so column slot i of MFMA c is k = kbase + 8*i + c.  Lane (li,lg)
// then owns W rows nbase + 8*(4*lg+e) + c2 at columns kbase + 8*li .. +7.
//
// Order of work: every wave first issues the W loads of its first passes (they
// need no adapter data), then the adapter row offsets and rows.  The B strip is
// the same for the four waves: wave w < KS loads and transposes rank group w
// of it into LDS (one 1-KiB operand block per (group, c2)); each wave keeps
// its own A operands in registers.  After the one barrier the wave walks its
// tile in 8 passes (one c2 each, 4 rows x 16 bytes per lane), issuing the W
// loads of a later pass before it computes and stores the current one.
//
// Rows past d_out: d_out - nbase is a multiple of 64, so row 8*(4*lg+e) + c2
// of the tile is inside the matrix exactly when 8*(4*lg+e) is; such rows read
// row c2 of the tile instead and are never stored.
template <int KS>
__global__ __launch_bounds__(WG, 2) void merge_kernel(MergeArgs args) {
    constexpr int PF = MERGE_PREFETCH;
    __shared__ u32x4_t s_bstrip[KS][8][64];
    const MergeMat& M = args.m[blockIdx.y];
    if ((int)blockIdx.x >= M.tiles) return;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int li = lane & 15, lg = lane >> 4;
    const int tn = blockIdx.x / M.tiles_k, tk = blockIdx.x % M.tiles_k;
    const int nbase = tn * 128, kbase = tk * 512 + wave * 128;
    const bool live = kbase < M.d_in;                  // wave-uniform
    const int k0 = kbase + 8 * li;
    const bool k_ok = k0 < M.d_in;
    const int kc = k_ok ? k0 : 0;                       // in-bounds column
    const int nn = nbase + 8 * li;
    const bool n_ok = nn < M.d_out;
    const int ncol = n_ok ? nn : nbase;                 // in-bounds column of B

    // W rows of this lane: pass c2 reads wrow[e] + c2 * ldw
    bool row_ok[4];
    uint16_t* wrow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int n = nbase + 8 * (4 * lg + e);
        row_ok[e] = n < M.d_out;
        wrow[e] = M.W + kc + (int64_t)(row_ok[e] ? n : nbase) * M.ldw;
    }
    u32x4_t wv[PF + 1][4];
    if (live) {
#pragma unroll
        for (int c2 = 0; c2 < PF; ++c2)
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[c2][e] = ld16(wrow[e] + (int64_t)c2 * M.ldw);
    }
    issue_fence();

    // adapter rows (no masked loads: rank slots past the rank and columns past
    // the matrix read clamped addresses and are zeroed after the transpose)
    const bool b_wave = wave < KS && 32 * wave < M.rank;   // wave-uniform
    u32x4_t astrip[KS][8];
    if (b_wave) {
        const int cb = ncol / M.B.chunk_len;
        int64_t ob[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ob[e] = M.B.row_off[off_index(M.B, M.adapter, min(32 * wave + 8 * lg + e, M.rank - 1), cb)];
        issue_fence();
        u32x4_t rb[8], tb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rb[e] = ld16(M.B.pool + ob[e] + (ncol - cb * M.B.chunk_len));
#pragma unroll
        for (int e = 0; e < 8; ++e) rb[e] = sel(32 * wave + 8 * lg + e < M.rank && n_ok, rb[e]);
        transpose8x8(rb, tb);
#pragma unroll
        for (int c2 = 0; c2 < 8; ++c2) s_bstrip[wave][c2][lane] = tb[c2];
    }
    if (live) {
        const int ca = kc / M.A.chunk_len;
        int64_t oa[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                oa[ks][e] = M.A.row_off[off_index(M.A, M.adapter, min(32 * ks + 8 * lg + e, M.rank - 1), ca)];
        issue_fence();
        u32x4_t ra[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) ra[ks][e] = ld16(M.A.pool + oa[ks][e] + (kc - ca * M.A.chunk_len));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ra[ks][e] = sel(32 * ks + 8 * lg + e < M.rank && k_ok, ra[ks][e]);
            transpose8x8(ra[ks], astrip[ks]);
        }
    }
    __syncthreads();
    if (!live) return;

#pragma unroll
    for (int c2 = 0; c2 < 8; ++c2) {
        if (c2 + PF < 8)
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[(c2 + PF) % (PF + 1)][e] = ld16(wrow[e] + (int64_t)(c2 + PF) * M.ldw);
        f32x4_t acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (32 * ks >= M.rank) break;
            const u32x4_t b = s_bstrip[ks][c2][lane];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = mfma_bf16(b, astrip[ks][c], acc[c]);
        }
        const u32x4_t* cur = wv[c2 % (PF + 1)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (!(k_ok && row_ok[e])) continue;
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w = cur[e][q];
                const float lo = __builtin_fmaf(M.scale, acc[2 * q][e], bf16_lo(w));
                const float hi = __builtin_fmaf(M.scale, acc[2 * q + 1][e], bf16_hi(w));
                o[q] = pack_bf16(lo, hi);
            }
            *reinterpret_cast<u32x4_t*>(wrow[e] + (int64_t)c2 * M.ldw) = o;
        }
    }
}

// ------------------------------------------------------------------ host side
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t check_rows(const lora_rows_t& r, int32_t d, int32_t max_rank, int32_t max_adapter) {
    if (!r.pool || !r.row_off || !aligned16(r.pool)) return LORA_EINVAL;
    if (r.row_len != d) return LORA_ESHAPE;
    if (r.chunk_len <= 0 || r.chunk_len % 64 != 0) return LORA_ESHAPE;
    if (r.max_rank < 1 || r.max_rank > LORA_MAX_RANK || max_rank > r.max_rank) return LORA_ERANK;
    if (max_adapter >= r.n_adapters) return LORA_EADAPTER;
    return LORA_OK;
}

Rows to_rows(const lora_rows_t& r) {
    return Rows{r.pool, r.row_off, r.n_adapters, r.max_rank, r.chunk_len, (r.row_len + r.chunk_len - 1) / r.chunk_len,
                r.neg_from};
}

// A plan lora_apply carries in its launch arguments: one range of the fused
// variant, at most LORA_INLINE_ITEMS items (one row each).
bool plan_inlines(const lora_plan_info_t& I) {
    return I.op == LORA_OP_APPLY && I.n_ranges == 1 && I.ranges[0].variant == LV_APPLY_FUSED &&
           I.ranges[0].begin == 0 && I.ranges[0].count == I.n_work && I.n_work <= LORA_INLINE_ITEMS &&
           I.n_active <= LORA_INLINE_ITEMS;
}
bool launch_inlines(const lora_launch_t* L) {
    return !L->live && L->host_work && L->host_row_index && plan_inlines(L->info);
}

// An expand variant (op-local id) that a kernel runs: the MFMA shapes in
// rank classes 0..2 (rank <= 32, 64, 128), the VALU decode shape in class 0.
bool expand_variant_ok(int ev) {
    if (ev < 0 || ev >= LV_E_SHAPES * LV_RANK_CLASSES) return false;
    const int shape = ev / LV_RANK_CLASSES, cls = ev % LV_RANK_CLASSES;
    return shape == LV_E_BGMV ? cls == 0 : cls < LV_RANK_CLASSES - 1;
}
bool variant_ok(int32_t op, int v) {
    if (op == LORA_OP_SHRINK) return v >= 0 && v < LV_S_SHAPES * LV_RANK_CLASSES;
    if (op == LORA_OP_EXPAND) return expand_variant_ok(v);
    if (v >= 0 && v < LV_APPLY_EXPAND0) return true;
    return v == LV_APPLY_FUSED || expand_variant_ok(v - LV_APPLY_EXPAND0);
}

int32_t check_launch(const lora_launch_t* L, int32_t op, int32_t n_proj) {
    if (!L || n_proj < 1 || n_proj > LORA_MAX_PROJ) return LORA_EINVAL;
    const lora_plan_info_t& I = L->info;
    if (I.op != op || I.n_work < 0 || I.n_ranges < 0 || I.n_ranges > LORA_MAX_RANGES) return LORA_EINVAL;
    if (I.v_slices < 1 || I.v_slices > LORA_MAX_SLICES || I.n_active < 0) return LORA_EINVAL;
    if (I.n_work > 0 && (!L->row_index || !L->work) && !(op == LORA_OP_APPLY && launch_inlines(L))) return LORA_EINVAL;
    if (I.max_rank > LORA_MAX_RANK) return LORA_ERANK;
    if (I.d_in <= 0 || I.d_out <= 0 || I.d_in % 64 != 0 || I.d_out % 64 != 0) return LORA_ESHAPE;
    for (int r = 0; r < I.n_ranges; ++r) {
        const lora_range_t& R = I.ranges[r];
        if (!variant_ok(op, R.variant) || R.begin < 0 || R.count < 0 || R.begin + R.count > I.n_work)
            return LORA_EINVAL;
    }
    return LORA_OK;
}

typedef void (*shrink_fn)(ShrinkArgs);
template <int KSPLIT, int MTW, int NT>
shrink_fn shrink_inst(bool loop) {
    return loop ? shrink_loop_kernel<KSPLIT, MTW, NT, unroll_for<KSPLIT, MTW, NT>()>
                : shrink_kernel<KSPLIT, MTW, NT, unroll_for<KSPLIT, MTW, NT>()>;
}
// Short-segment (SPLITK16) shrink kernels by rank class (loop: the
// grid-stride form for device-built plans).
shrink_fn shrink_table(int variant, bool loop) {
    static const shrink_fn t[2][LV_RANK_CLASSES] = {
        {shrink_inst<4, 1, 1>(false), shrink_inst<4, 1, 2>(false), shrink_inst<4, 1, 4>(false),
         shrink_inst<4, 1, 8>(false)},
        {shrink_inst<4, 1, 1>(true), shrink_inst<4, 1, 2>(true), shrink_inst<4, 1, 4>(true),
         shrink_inst<4, 1, 8>(true)}};
    return t[loop][variant % LV_RANK_CLASSES];
}

typedef void (*expand_fn)(ExpandArgs);
expand_fn expand_table(int rank_class, bool loop) {
    static const expand_fn t[2][3] = {{expand_kernel<1>, expand_kernel<2>, expand_kernel<4>},
                                      {expand_loop_kernel<1>, expand_loop_kernel<2>, expand_loop_kernel<4>}};
    return t[loop][rank_class];
}

// Launches `fn` and returns the status of this launch alone
// (hipLaunchKernel's own result: an error left behind by an earlier,
// unrelated runtime call is neither reported here nor cleared).
template <typename A>
hipError_t launch(void (*fn)(A), dim3 grid, dim3 block, hipStream_t s, A& args) {
    void* p[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, p, 0, s);
}
// The first failure of a sequence of launches.
inline hipError_t first_error(hipError_t acc, hipError_t e) { return acc != hipSuccess ? acc : e; }

// Workgroups of `fn` (`block` threads) that the current device holds at
// once: CUs x resident workgroups per CU, cached per (device, kernel).
int resident_slots(const void* fn, int block = WG) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    static std::mutex mu;
    static struct Entry { int dev; const void* fn; int slots; } cache[64];
    static int n_cache = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i)
        if (cache[i].dev == dev && cache[i].fn == fn) return cache[i].slots;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    const int slots = cus * per_cu;
    if (n_cache < 64) cache[n_cache++] = Entry{dev, fn, slots};
    return slots;
}

// Grid of a persistent launch over `tasks` equal tasks: as few rounds as
// the resident slots allow, and the tasks spread evenly over the workgroups
// (every workgroup gets the same number, give or take one, and no partly
// filled last round).
unsigned persistent_grid(const void* fn, int64_t tasks) {
    const int64_t slots = resident_slots(fn);
    const int64_t rounds = (tasks + slots - 1) / slots;
    return (unsigned)((tasks + rounds - 1) / rounds);
}

// grid.x of a grid-stride launch (device-built plans) over `count` items
// with grid.y = ny: at most one round of resident workgroups, at least one.
unsigned loop_grid_x(const void* fn, int64_t count, int ny, int block = WG) {
    int64_t gx = resident_slots(fn, block) / ny;
    if (gx > count) gx = count;
    return (unsigned)(gx > 0 ? gx : 1);
}

// Groups of up to SHRINK_GROUP projections with the same x (pointer, ldx
// and d_in), in first-appearance order; returns true when some group has more
// than one projection.
constexpr int SHRINK_GROUP = 3;
bool group_shared_x(ShrinkArgs& args, int32_t n_proj) {
    bool taken[LORA_MAX_PROJ] = {};
    int n = 0, ng = 0;
    bool shared = false;
    for (int i = 0; i < n_proj; ++i) {
        if (taken[i]) continue;
        args.gbeg[ng++] = (int8_t)n;
        args.gproj[n++] = (int8_t)i;
        taken[i] = true;
        int size = 1;
        for (int j = i + 1; j < n_proj && size < SHRINK_GROUP; ++j) {
            const ShrinkProj &a = args.p[i], &b = args.p[j];
            if (taken[j] || a.x != b.x || a.ldx != b.ldx || a.d_in != b.d_in) continue;
            args.gproj[n++] = (int8_t)j;
            taken[j] = true;
            ++size;
            shared = true;
        }
    }
    args.gbeg[ng] = (int8_t)n;
    args.n_groups = ng;
    return shared;
}

// Shrink launches for the plan's ranges [r0, r1) (shrink variants only).
// In a host plan the short-segment ranges of ranks up to 64, and the
// long-segment ranges of one shape with ranks up to 64, are consecutive in the
// work list and share one launch each (the kernel picks the rank tiles per
// item); ranks above 64 get their own.  A device-built plan (live != NULL)
// already has one range per launch group: each range is one launch, bounded
// by its live count.
hipError_t launch_shrink_ranges(const lora_plan_info_t& info, const int32_t* live, int r0, int r1, int32_t n_proj,
                                hipStream_t s, ShrinkArgs& args) {
    hipError_t err = hipSuccess;
    args.n_proj = n_proj;
    bool whole = true;  // every projection keeps each A row in one chunk
    for (int i = 0; i < n_proj; ++i) whole = whole && args.p[i].A.chunk_len >= args.p[i].d_in;
    const bool grouped = group_shared_x(args, n_proj);
    for (int r = r0; r < r1;) {
        const lora_range_t& R = info.ranges[r];
        const int shape = R.variant / LV_RANK_CLASSES, cls = R.variant % LV_RANK_CLASSES;
        args.live = live ? live + r : nullptr;
        if (shape == LV_S_SPLITK16 && !live && cls < LV_RANK_CLASSES - 1) {
            int e = r, count = 0;
            while (e < r1 && info.ranges[e].variant / LV_RANK_CLASSES == LV_S_SPLITK16 &&
                   info.ranges[e].variant % LV_RANK_CLASSES < LV_RANK_CLASSES - 1 &&
                   info.ranges[e].begin == R.begin + count) {
                count += info.ranges[e].count;
                ++e;
            }
            if (count > 0) {
                args.begin = R.begin;
                args.count = count;
                err = first_error(err, launch(shrink_classes_kernel<4, 1>, dim3((unsigned)count, (unsigned)n_proj),
                                              dim3(WG), s, args));
            }
            r = e;
            continue;
        }
        if (shape == LV_S_SPLITK16 || cls == LV_RANK_CLASSES - 1) {
            if (R.count > 0) {
                args.begin = R.begin;
                args.count = R.count;
                if (shape == LV_S_SPLITK16) {
                    // a device-built plan's range of classes 0-2 is one launch group
                    const shrink_fn fn = live && cls < LV_RANK_CLASSES - 1 ? shrink_classes_loop_kernel<4, 1>
                                                                         : shrink_table(R.variant, live != nullptr);
                    const unsigned gx =
                        live ? loop_grid_x(reinterpret_cast<const void*>(fn), R.count, n_proj) : (unsigned)R.count;
                    err = first_error(err, launch(fn, dim3(gx, (unsigned)n_proj), dim3(WG), s, args));
                } else {
                    shrink_fn fn = shape == LV_S_ROWS64
                                       ? (whole ? shrink_rows_kernel<1, 8, true, 1> : shrink_rows_kernel<1, 8, false, 1>)
                                       : (whole ? shrink_rows_kernel<2, 8, true, 1> : shrink_rows_kernel<2, 8, false, 1>);
                    const unsigned g = persistent_grid(reinterpret_cast<const void*>(fn), (int64_t)R.count * n_proj);
                    err = first_error(err, launch(fn, dim3(g), dim3(WG), s, args));
                }
            }
            ++r;
            continue;
        }
        // ranges r .. e-1: same shape, rank classes below the last one (a
        // device-built plan's ranges have their own live counts: one each)
        int e = r, count = 0;
        while (e < r1 && (e == r || !live) && info.ranges[e].variant / LV_RANK_CLASSES == shape &&
               info.ranges[e].variant % LV_RANK_CLASSES < LV_RANK_CLASSES - 1 &&
               info.ranges[e].begin == R.begin + count) {
            count += info.ranges[e].count;
            ++e;
        }
        if (count > 0) {
            args.begin = R.begin;
            args.count = count;
            shrink_fn fn;
            if (grouped)  // tasks are (item, group of projections that share x)
                fn = shape == LV_S_ROWS64
                         ? (whole ? shrink_rows_kernel<1, 4, true, SHRINK_GROUP>
                                  : shrink_rows_kernel<1, 4, false, SHRINK_GROUP>)
                         : (whole ? shrink_rows_kernel<2, 4, true, SHRINK_GROUP>
                                  : shrink_rows_kernel<2, 4, false, SHRINK_GROUP>);
            else
                fn = shape == LV_S_ROWS64
                         ? (whole ? shrink_rows_kernel<1, 4, true, 1> : shrink_rows_kernel<1, 4, false, 1>)
                         : (whole ? shrink_rows_kernel<2, 4, true, 1> : shrink_rows_kernel<2, 4, false, 1>);
            const unsigned g = persistent_grid(reinterpret_cast<const void*>(fn),
                                               (int64_t)count * (grouped ? args.n_groups : n_proj));
            err = first_error(err, launch(fn, dim3(g), dim3(WG), s, args));
        }
        r = e;
    }
    return err;
}

#ifndef EXPAND_LOOP_ROUNDS
#define EXPAND_LOOP_ROUNDS 8
#endif
// Expand launch of one range: op-local variant `ev` (shape x rank class),
// items [begin, begin + count); live != NULL for a device-built plan.
hipError_t launch_expand_range(int ev, int32_t begin, int32_t count, const int32_t* live, int32_t n_proj,
                               hipStream_t s, ExpandArgs& args) {
    const int shape = ev / LV_RANK_CLASSES;
    const int32_t width = lv_expand_cols(shape);
    int32_t groups = 0;  // column groups of every projection, back to back on grid.y
    for (int i = 0; i < n_proj; ++i) {
        args.p[i].cg_begin = groups;
        groups += (args.p[i].d_out + width - 1) / width;
    }
    args.begin = begin;
    args.count = count;
    args.groups = groups;
    args.live = live;
    if (shape == LV_E_BGMV) {
        bool uni = true;  // every wave's row offsets are uniform
        for (int i = 0; i < n_proj; ++i) uni = uni && args.p[i].B.chunk_len % 512 == 0;
        const auto fn = live ? (uni ? bgmv_expand_loop_kernel<true> : bgmv_expand_loop_kernel<false>)
                             : (uni ? bgmv_expand_kernel<true> : bgmv_expand_kernel<false>);
        const unsigned gx =
            live ? loop_grid_x(reinterpret_cast<const void*>(fn), count, groups) : (unsigned)count;
        return launch(fn, dim3(gx, (unsigned)groups), dim3(WG), s, args);
    }
    const expand_fn fn = expand_table(ev % LV_RANK_CLASSES, live != nullptr);
    int64_t n1 = (int64_t)count * groups;
    if (live) {
        // a launch group mixes items of 16 to 128 rows: several rounds of
        // workgroups let the dispatcher even out the load
        const int64_t cap = EXPAND_LOOP_ROUNDS * (int64_t)resident_slots(reinterpret_cast<const void*>(fn));
        if (n1 > cap) n1 = cap;
    }
    n1 = (n1 + N_XCD - 1) / N_XCD * N_XCD;  // xcd_block needs a multiple of 8
    return launch(fn, dim3((unsigned)n1), dim3(WG), s, args);
}

}  // namespace

extern "C" int32_t lora_shrink(const lora_launch_t* L, int32_t n_proj, const lora_shrink_proj_t* projs,
                               void* hip_stream) {
    int32_t st = check_launch(L, LORA_OP_SHRINK, n_proj);
    if (st != LORA_OK) return st;
    if (!projs) return LORA_EINVAL;
    ShrinkArgs args;
    args.row_index = L->row_index;
    args.work = L->work;
    args.n_active = L->info.n_active;
    args.v_slices = L->info.v_slices;
    for (int i = 0; i < n_proj; ++i) {
        const lora_shrink_proj_t& p = projs[i];
        if (!p.x || !p.v || !aligned16(p.x) || !aligned16(p.v)) return LORA_EINVAL;
        if (p.d_in <= 0 || p.d_in % 64 != 0 || p.d_in > L->info.d_in) return LORA_ESHAPE;
        if (p.ldx < p.d_in || p.ldx % 8 != 0 || p.ldv % 4 != 0 || p.ldv < L->info.max_rank) return LORA_EINVAL;
        if ((st = check_rows(p.A, p.d_in, L->info.max_rank, L->info.max_adapter)) != LORA_OK) return st;
        args.p[i] = ShrinkProj{p.x, p.ldx, to_rows(p.A), p.d_in, p.v, p.ldv};
    }
    if (L->info.n_work == 0) return LORA_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t err = hipSuccess;
    err = launch_shrink_ranges(L->info, L->live, 0, L->info.n_ranges, n_proj, s, args);
    return err == hipSuccess ? LORA_OK : LORA_EHIP;
}

extern "C" int32_t lora_expand(const lora_launch_t* L, int32_t n_proj, const lora_expand_proj_t* projs,
                               void* hip_stream) {
    int32_t st = check_launch(L, LORA_OP_EXPAND, n_proj);
    if (st != LORA_OK) return st;
    if (!projs) return LORA_EINVAL;
    ExpandArgs args;
    args.row_index = L->row_index;
    args.work = L->work;
    args.n_active = L->info.n_active;
    args.v_slices = L->info.v_slices;
    args.n_proj = n_proj;
    for (int i = 0; i < n_proj; ++i) {
        const lora_expand_proj_t& p = projs[i];
        if (!p.v || !p.y || !aligned16(p.v) || !aligned16(p.y)) return LORA_EINVAL;
        if (p.d_out <= 0 || p.d_out % 64 != 0 || p.d_out > L->info.d_out) return LORA_ESHAPE;
        if (p.ldy < p.d_out || p.ldy % 4 != 0 || p.ldv % 4 != 0 || p.ldv < L->info.max_rank) return LORA_EINVAL;
        if ((st = check_rows(p.B, p.d_out, L->info.max_rank, L->info.max_adapter)) != LORA_OK) return st;
        args.p[i] = ExpandProj{p.v, p.ldv, to_rows(p.B), p.d_out, p.y, p.ldy, p.scale, 0};
    }
    if (L->info.n_work == 0) return LORA_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t err = hipSuccess;
    for (int r = 0; r < L->info.n_ranges; ++r) {
        const lora_range_t& R = L->info.ranges[r];
        if (R.count == 0) continue;
        err = first_error(err, launch_expand_range(R.variant, R.begin, R.count, L->live ? L->live + r : nullptr,
                                                   n_proj, s, args));
    }
    return err == hipSuccess ? LORA_OK : LORA_EHIP;
}

namespace {
int32_t apply_impl(const lora_launch_t* L, int32_t n_proj, const lora_apply_proj_t* projs, void* hip_stream) {
    int32_t st = check_launch(L, LORA_OP_APPLY, n_proj);
    if (st != LORA_OK) return st;
    if (!projs) return LORA_EINVAL;
    bool need_v = false;  // any shrink or expand range (segments that are not fused)
    bool fused = false;   // any fused range
    for (int r = 0; r < L->info.n_ranges; ++r) {
        if (L->info.ranges[r].count == 0) continue;
        if (L->info.ranges[r].variant != LV_APPLY_FUSED) need_v = true;
        else fused = true;
    }
    ShrinkArgs sa;
    ExpandArgs ea;
    FusedArgs fa;
    sa.row_index = ea.row_index = fa.row_index = L->row_index;
    sa.work = ea.work = fa.work = L->work;
    sa.n_active = ea.n_active = fa.n_active = L->info.n_active;
    sa.v_slices = ea.v_slices = L->info.v_slices;
    ea.n_proj = n_proj;
    const int32_t mr = L->info.max_rank, ma = L->info.max_adapter;
    for (int i = 0; i < n_proj; ++i) {
        const lora_apply_proj_t& p = projs[i];
        if (!p.x || !p.y || !aligned16(p.x) || !aligned16(p.y)) return LORA_EINVAL;
        if (need_v && (!p.v || !aligned16(p.v) || p.ldv % 4 != 0 || p.ldv < mr)) return LORA_EINVAL;
        if (p.d_in <= 0 || p.d_in % 64 != 0 || p.d_out <= 0 || p.d_out % 64 != 0) return LORA_ESHAPE;
        if (p.d_in > L->info.d_in || p.d_out > L->info.d_out) return LORA_ESHAPE;
        // the fused kernel covers d_in and d_out up to LV_FUSED_MAX_D (a plan
        // lora_plan made never fuses past it; a hand-made one is refused)
        if (fused && (p.d_in > LV_FUSED_MAX_D || p.d_out > LV_FUSED_MAX_D)) return LORA_ESHAPE;
        if (p.ldx < p.d_in || p.ldx % 8 != 0 || p.ldy < p.d_out || p.ldy % 4 != 0) return LORA_EINVAL;
        if ((st = check_rows(p.A, p.d_in, mr, ma)) != LORA_OK) return st;
        if ((st = check_rows(p.B, p.d_out, mr, ma)) != LORA_OK) return st;
        sa.p[i] = ShrinkProj{p.x, p.ldx, to_rows(p.A), p.d_in, p.v, p.ldv};
        ea.p[i] = ExpandProj{p.v, p.ldv, to_rows(p.B), p.d_out, p.y, p.ldy, p.scale, 0};
        fa.p[i] = ApplyProj{p.x, p.ldx, p.d_in, to_rows(p.A), to_rows(p.B), p.d_out, p.y, p.ldy, p.scale};
    }
    if (L->info.n_work == 0) return LORA_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    bool uni = true;  // every wave's row offsets are uniform
    for (int i = 0; i < n_proj; ++i) uni = uni && fa.p[i].A.chunk_len % 512 == 0 && fa.p[i].B.chunk_len % 512 == 0;
    if (launch_inlines(L)) {  // the plan goes in the launch arguments
        FusedInlineArgs ia{};
        ia.begin = 0;
        ia.n_active = L->info.n_active;
        for (int i = 0; i < n_proj; ++i) ia.p[i] = fa.p[i];
        memcpy(ia.w, L->host_work, sizeof(lora_work_t) * (size_t)L->info.n_work);
        memcpy(ia.rows, L->host_row_index, sizeof(int32_t) * (size_t)L->info.n_active);
        const hipError_t e = launch(uni ? fused_inline_kernel<true> : fused_inline_kernel<false>,
                                    dim3((unsigned)L->info.n_work, (unsigned)n_proj), dim3(FWG), s, ia);
        return e == hipSuccess ? LORA_OK : LORA_EHIP;
    }
    hipError_t err = hipSuccess;
    // ranges come in variant order: shrink, expand, fused; the expand ranges
    // follow every shrink range on the stream
    int r_shrink = 0;
    while (r_shrink < L->info.n_ranges && L->info.ranges[r_shrink].variant < LV_APPLY_EXPAND0) ++r_shrink;
    err = launch_shrink_ranges(L->info, L->live, 0, r_shrink, n_proj, s, sa);
    for (int r = r_shrink; r < L->info.n_ranges; ++r) {
        const lora_range_t& R = L->info.ranges[r];
        if (R.count == 0) continue;
        if (R.variant < LV_APPLY_FUSED) {
            err = first_error(err, launch_expand_range(R.variant - LV_APPLY_EXPAND0, R.begin, R.count,
                                                       L->live ? L->live + r : nullptr, n_proj, s, ea));
        } else {
            fa.begin = R.begin;
            fa.live = L->live ? L->live + r : nullptr;
            const auto fn = fa.live ? (uni ? fused_loop_kernel<true> : fused_loop_kernel<false>)
                                    : (uni ? fused_kernel<true> : fused_kernel<false>);
            const unsigned gx = fa.live ? loop_grid_x(reinterpret_cast<const void*>(fn), R.count, n_proj, FWG)
                                        : (unsigned)R.count;
            err = first_error(err, launch(fn, dim3(gx, (unsigned)n_proj), dim3(FWG), s, fa));
        }
    }
    return err == hipSuccess ? LORA_OK : LORA_EHIP;
}
}  // namespace

extern "C" int32_t lora_apply(const lora_launch_t* L, int32_t n_proj, const lora_apply_proj_t* projs,
                              void* hip_stream) {
    return apply_impl(L, n_proj, projs, hip_stream);
}

// ------------------------------------------------------------------ lora_apply without a workspace
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation): lora_apply with v taken
// from this file-scope array instead of the caller's buffers.  Each device
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is not a device address: its address on the current
// device comes from hipGetSymbolAddress (once per device, kept below) and
// is the only form of it the host ever passes on.
static __device__ __align__(256) float scratch[LORA_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace {
// Address of `scratch` on the current device (nullptr if the lookup fails).
float* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    static std::mutex mu;
    static void* addr[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return static_cast<float*>(addr[dev]);
}
}  // namespace

extern "C" int32_t lora_apply_static(const lora_launch_t* L, int32_t n_proj, const lora_apply_proj_t* projs,
                                     void* hip_stream) {
    if (!L || !projs || n_proj < 1 || n_proj > LORA_MAX_PROJ) return LORA_EINVAL;
    // each projection's v: [v_slices][n_active][ldv] floats, ldv the plan's
    // largest rank rounded up to 4, back to back in the array
    const int64_t ldv = L->info.max_rank < 1 ? 4 : ((int64_t)L->info.max_rank + 3) / 4 * 4;
    const int64_t rows = L->info.n_active < 1 ? 1 : L->info.n_active;
    const int64_t per = (int64_t)(L->info.v_slices < 1 ? 1 : L->info.v_slices) * rows * ldv;
    const int64_t region = (per + 63) / 64 * 64;  // 256-byte aligned regions
    if (L->info.n_active < 0 || L->info.v_slices > LORA_MAX_SLICES || L->info.max_rank > LORA_MAX_RANK ||
        region * n_proj > (int64_t)(LORA_STATIC_SCRATCH_BYTES / sizeof(float)))
        return LORA_ECAPACITY;
    float* base = scratch_on_current_device();
    if (!base) return LORA_EHIP;
    lora_apply_proj_t p[LORA_MAX_PROJ];
    for (int i = 0; i < n_proj; ++i) {
        p[i] = projs[i];
        p[i].v = base + region * i;
        p[i].ldv = ldv;
    }
    return apply_impl(L, n_proj, p, hip_stream);
}

// ------------------------------------------------------------------ device plan builder
// The tile-config table and the per-segment rules of the host planner, in
// constant memory, so the device cuts every segment exactly as lora_plan does.
#ifndef HETLORA_TILE_TABLE
#define HETLORA_TILE_TABLE "tile_table.inc"
#endif
namespace devplan {
#include HETLORA_TILE_TABLE
#include "plan_rules.h"
}  // namespace devplan

namespace {

#define BWG 1024                 // one workgroup builds the whole plan
#define BWAVES (BWG / 64)
#define B_MAX_ADAPTERS 4096
#define B_ERR_ADAPTER 1
#define B_ERR_RANK 2
#define B_ERR_CAPACITY 4

struct BuildArgs {
    const int32_t* row_adapter;
    const int32_t* adapter_rank;
    int32_t n_rows, n_adapters, max_rank, d_in, d_out, n_ranges;
    lora_device_header_t* hdr;
    int32_t* row_index;
    int32_t* seg_start;
    int32_t* seg_adapter;
    int32_t* seg_rank;
    int32_t* scratch;
    lora_work_t* work;
    int32_t range_variant[LORA_MAX_RANGES];
    int32_t range_begin[LORA_MAX_RANGES];
    int32_t range_cap[LORA_MAX_RANGES];
};

// Exclusive prefix sum of v over the workgroup's threads in thread order;
// `total` gets the sum of all.  Every thread must call it.
__device__ int block_scan(int v, int* s_tmp, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < BWAVES; ++i) {
        const int t = s_tmp[i];
        before += i < w ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}


// Stable counting sort of the rows by adapter id, the segment table, and the
// apply plan.  Thread t owns adapters 4t .. 4t+3 and so the segments of those
// adapters (segments come in adapter order); wave w owns rows [w*B, (w+1)*B).
// Before A, every thread loads its share of the ids and its adapters' ranks
// (the only global reads), and the tile table is copied to LDS.
//  A  each wave counts its rows per adapter in its own LDS column: lanes with
//     equal ids are found by ballot, one id at a time, and the id's first
//     lane adds the count; each row keeps (id, rank among the equal ids before
//     it in the block), in LDS when it fits, else in the scratch part
//  B  per owned adapter, the exclusive prefix over the waves; one prefix sum
//     over the adapters gives each adapter's first row_index slot and each
//     segment's id (the segment table is written here); each owned segment is
//     cut into its plan parts (lv_apply_parts, as lora_plan cuts it)
//  C  row i goes to slot first[a] + (rows of a in earlier waves) + its rank
//  then the segment records go to LDS (it is free once C is done)
//  D  wave w takes ranges w, w+16, ...: over the range's variants in order,
//     an exclusive prefix of the item counts over the segments in order gives
//     each part its first item in the range
//  E  the items: small parts one thread each, larger ones a wave each
// Invalid ids or ranks, or a range over its capacity, leave an error status
// and every live count 0.
__global__ __launch_bounds__(BWG) void build_plan_kernel(BuildArgs a) {
    // A-C: per wave and adapter a row count, then the exclusive prefix over
    // the waves (16 x NA uint16), then per row (id << 16 | rank in block) when
    // it fits; E: 8 ints per segment
    __shared__ uint32_t s_mem[BWAVES * B_MAX_ADAPTERS / 2];
    __shared__ int32_t s_first[B_MAX_ADAPTERS];
    __shared__ int32_t s_tmp[BWAVES];
    __shared__ int32_t s_live[LORA_MAX_RANGES];
    __shared__ int32_t s_rvar[LORA_MAX_RANGES], s_rbeg[LORA_MAX_RANGES], s_rcap[LORA_MAX_RANGES];
    __shared__ int32_t s_vrange[LV_APPLY_VARIANTS];  // the range (launch group) of each variant (-1: none)
    __shared__ devplan::ShrinkCfg s_stab[LV_LEN_BUCKETS][LV_RANK_BUCKETS][LV_D_BUCKETS];
    __shared__ int8_t s_etab[LV_LEN_BUCKETS][LV_RANK_BUCKETS][LV_D_BUCKETS];
    __shared__ int32_t s_err, s_n_active, s_n_seg;
    uint16_t* s_h = reinterpret_cast<uint16_t*>(s_mem);
    int32_t* s_rec = reinterpret_cast<int32_t*>(s_mem);

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int NA = a.n_adapters, n_rows = a.n_rows;
    const int B = ((n_rows + BWAVES - 1) / BWAVES + 63) / 64 * 64;  // rows per wave
    // per-row data: after the counters in LDS if it fits, else the scratch part
    const bool rows_in_lds = n_rows <= BWAVES * B_MAX_ADAPTERS / 2 - BWAVES * NA / 2;
    uint32_t* rowdat = rows_in_lds ? s_mem + BWAVES * NA / 2 : reinterpret_cast<uint32_t*>(a.scratch);

    constexpr int APT = B_MAX_ADAPTERS / BWG;  // adapters (and segments) per thread
    int rk[APT];
#pragma unroll
    for (int j = 0; j < APT; ++j) rk[j] = APT * t + j < NA ? a.adapter_rank[APT * t + j] : 1;
    for (int i = t; i < BWAVES * NA / 2; i += BWG) s_mem[i] = 0;
    if (t == 0) {
        s_err = 0;
        // the range table, copied with constant indices (the argument
        // block is never indexed at run time)
#pragma unroll
        for (int r = 0; r < LORA_MAX_RANGES; ++r) {
            s_rvar[r] = a.range_variant[r];
            s_rbeg[r] = a.range_begin[r];
            s_rcap[r] = a.range_cap[r];
        }
#pragma unroll
        for (int v = 0; v < LV_APPLY_VARIANTS; ++v) s_vrange[v] = -1;
        // ranges are keyed by their group's smallest variant (in [0, LV_APPLY_VARIANTS))
        for (int r = 0; r < a.n_ranges; ++r) s_vrange[s_rvar[r]] = r;
#pragma unroll
        for (int v = 0; v < LV_APPLY_VARIANTS; ++v) s_vrange[v] = s_vrange[lv_launch_group(v)];  // key <= v
    }
    {  // the tile table, copied to LDS byte by byte (phase B looks it up per segment)
        constexpr int NS = (int)sizeof(s_stab), NE = (int)sizeof(s_etab);
        if (t < NS)
            reinterpret_cast<uint8_t*>(&s_stab[0][0][0])[t] = reinterpret_cast<const uint8_t*>(devplan::kShrinkCfg)[t];
        else if (t < NS + NE)
            reinterpret_cast<uint8_t*>(&s_etab[0][0][0])[t - NS] =
                reinterpret_cast<const uint8_t*>(devplan::kExpandShape)[t - NS];
    }
    // the ids, loaded by all threads at once (each wave's walk below then
    // reads them from LDS or L2 instead of waiting on HBM chunk by chunk)
    for (int i = t; i < n_rows; i += BWG) rowdat[i] = (uint32_t)a.row_adapter[i];
    __syncthreads();

    // A
    {
        const int r0 = w * B, r1 = min(n_rows, r0 + B);
        for (int base = r0; base < r1; base += 64) {
            const int i = base + lane;
            int key = -1;
            if (i < r1) {
                key = (int)rowdat[i];
                if (key < -1 || key >= NA) {
                    atomicOr(&s_err, B_ERR_ADAPTER);
                    key = -1;
                }
            }
            uint64_t pending = __ballot(key >= 0);
            int below = 0, leader = lane, cnt = 0;
            while (pending) {
                const int l = __ffsll((unsigned long long)pending) - 1;
                const int k = __builtin_amdgcn_readlane(key, l);
                const uint64_t m = __ballot(key == k);
                if (key == k) {
                    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                    leader = l;
                    cnt = __popcll(m);
                }
                pending &= ~m;
            }
            int before = 0;
            if (key >= 0 && lane == leader) {  // one lane per id: distinct addresses
                before = s_h[w * NA + key];
                s_h[w * NA + key] = (uint16_t)(before + cnt);
            }
            before = __shfl(before, leader);
            if (i < r1) rowdat[i] = key >= 0 ? ((uint32_t)key << 16) | (uint32_t)(before + below) : 0xFFFFFFFFu;
        }
    }
    __syncthreads();

    // B
    int cnt[APT], rows = 0, segs = 0;
#pragma unroll
    for (int j = 0; j < APT; ++j) {
        const int ad = APT * t + j;
        int sum = 0;
        if (ad < NA) {
            int c[BWAVES];  // all loads first, then the prefix
#pragma unroll
            for (int ww = 0; ww < BWAVES; ++ww) c[ww] = s_h[ww * NA + ad];
#pragma unroll
            for (int ww = 0; ww < BWAVES; ++ww) {
                s_h[ww * NA + ad] = (uint16_t)sum;
                sum += c[ww];
            }
            if (rk[j] < 1 || rk[j] > a.max_rank) atomicOr(&s_err, B_ERR_RANK);
        }
        cnt[j] = sum;
        rows += sum;
        segs += sum > 0;
    }
    // one scan for both: rows (<= 65536, 17 bits) and segments above them
    int tot;
    const int pre = block_scan(rows | (segs << 17), s_tmp, tot);
    const int n_active = tot & 0x1FFFF, n_seg = tot >> 17;
    int st[APT], sid[APT], va[APT], vb[APT], ia[APT], ib[APT], sl[APT];
    {
        int r = pre & 0x1FFFF, sg = pre >> 17;
#pragma unroll
        for (int j = 0; j < APT; ++j) {
            const int ad = APT * t + j;
            st[j] = r;
            sid[j] = cnt[j] > 0 ? sg : -1;
            va[j] = vb[j] = -1;
            ia[j] = ib[j] = 0;
            sl[j] = 1;
            if (ad < NA) s_first[ad] = r;
            if (cnt[j] > 0) {
                a.seg_start[sg] = r;
                a.seg_adapter[sg] = ad;
                a.seg_rank[sg] = rk[j];
                ++sg;
                // the segment's plan parts (as lora_plan cuts them)
                devplan::SegPlan pa, pb;
                devplan::lv_apply_parts(cnt[j], rk[j], a.d_in, a.d_out, pa, pb, s_stab, s_etab);
                sl[j] = pa.slices;
                va[j] = pa.variant;
                vb[j] = pb.variant;
                ia[j] = pa.chunks * (pa.shrink ? pa.slices : 1);
                ib[j] = pb.variant >= 0 ? pb.chunks : 0;
                if (s_vrange[pa.variant] < 0 || (pb.variant >= 0 && s_vrange[pb.variant] < 0))
                    atomicOr(&s_err, B_ERR_CAPACITY);
            }
            r += cnt[j];
        }
    }
    if (t == 0) {
        a.seg_start[n_seg] = n_active;
        s_n_active = n_active;
        s_n_seg = n_seg;
    }
    __syncthreads();  // s_first and the wave prefixes are complete

    // C
    for (int i = t; i < n_rows; i += BWG) {
        const uint32_t d = rowdat[i];
        const int key = (int)(d >> 16);
        if (key >= NA) continue;  // released (or an invalid id)
        const int pos = s_first[key] + s_h[(i / B) * NA + key] + (int)(d & 0xFFFFu);
        if (pos >= 0 && pos < n_rows) a.row_index[pos] = i;
    }
    __syncthreads();  // LDS is free for the segment records

    // segment records: start, len, adapter, rank | K slices << 16,
    // variant of part a | variant of part b << 8 (0xFF: none), then the
    // parts' item counts (replaced by their first item in the range below)
#pragma unroll
    for (int j = 0; j < APT; ++j) {
        if (sid[j] < 0) continue;
        int32_t* rec = s_rec + 8 * sid[j];
        rec[0] = st[j];
        rec[1] = cnt[j];
        rec[2] = APT * t + j;
        rec[3] = (rk[j] & 0xFFFF) | (sl[j] << 16);
        rec[4] = (va[j] & 0xFF) | ((vb[j] & 0xFF) << 8);
        rec[5] = ia[j];
        rec[6] = ib[j];
    }
    __syncthreads();

    // D: wave w takes ranges w, w+16, ...: the range's variants in order,
    // each an exclusive prefix of the item counts over the segments in order
    // (64 at a time), continuing from the variant before
    for (int r = w; r < a.n_ranges; r += BWAVES) {
        int run = 0;
        for (int m = 0; m < LV_RANK_CLASSES; ++m) {
            const int v = lv_group_member(s_rvar[r], m);
            if (v < 0) break;
            for (int base = 0; base < n_seg; base += 64) {
                const int sg = base + lane;
                int c = 0, slot = -1;
                if (sg < n_seg) {
                    const int32_t* rec = s_rec + 8 * sg;
                    const int vv = rec[4];
                    if ((int8_t)(vv & 0xFF) == v) slot = 5;
                    else if ((int8_t)((vv >> 8) & 0xFF) == v) slot = 6;
                    if (slot >= 0) c = rec[slot];
                }
                int x = c;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(x, o);
                    if (lane >= o) x += y;
                }
                if (slot >= 0) s_rec[8 * sg + slot] = run + x - c;
                run += __shfl(x, 63);
            }
        }
        if (lane == 0) {
            s_live[r] = run;
            if (run > s_rcap[r]) atomicOr(&s_err, B_ERR_CAPACITY);
        }
    }
    __syncthreads();

    // E: small parts one thread each, larger ones a wave each (lanes over items)
    for (int pass = 0; pass < 2; ++pass) {
        const int first = pass == 0 ? t : w, stride = pass == 0 ? BWG : BWAVES;
        for (int sg = first; sg < n_seg; sg += stride) {
            const int32_t* rec = s_rec + 8 * sg;
            const int start = rec[0], len = rec[1], adapter = rec[2], rank = (int16_t)(rec[3] & 0xFFFF);
            const int slices = rec[3] >> 16;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int v = (int8_t)((rec[4] >> (8 * h)) & 0xFF), o = rec[5 + h];
                if (v < 0) continue;
                const int r = s_vrange[v];
                if (r < 0) continue;
                // the part's shape follows from its variant
                const bool fused = v == LV_APPLY_FUSED, shrink = v < LV_APPLY_EXPAND0;
                const int mt = fused ? 1 : shrink ? lv_shrink_rows(v / LV_RANK_CLASSES)
                                                  : lv_expand_rows((v - LV_APPLY_EXPAND0) / LV_RANK_CLASSES);
                const int lg = __builtin_ctz(mt);  // rows per item are powers of two
                const int chunks = (len + mt - 1) >> lg;
                const int per = shrink ? slices : 1;  // items per row chunk
                const int n = chunks * per;
                if (o + n > s_rcap[r] || (n <= 4) != (pass == 0)) continue;
                const int nslices = shrink ? slices : (fused ? 1 : slices);
                const int base = len / chunks, extra = len - base * chunks;
                for (int i = pass == 0 ? 0 : lane; i < n; i += pass == 0 ? 1 : 64) {
                    const int c = per == 1 ? i : i / per, ks = i - c * per;
                    const lora_work_t it{start + c * base + min(c, extra), base + (c < extra ? 1 : 0), adapter, rank,
                                         ks, nslices, {0, 0}};
                    a.work[s_rbeg[r] + o + i] = it;
                }
            }
        }
    }
    __syncthreads();

    if (t < LORA_MAX_RANGES) a.hdr->live[t] = (s_err == 0 && t < a.n_ranges) ? s_live[t] : 0;
    if (t == 0) {
        const int e = s_err;
        a.hdr->status = (e & B_ERR_ADAPTER) ? LORA_EADAPTER : (e & B_ERR_RANK) ? LORA_ERANK
                      : (e & B_ERR_CAPACITY) ? LORA_ECAPACITY : LORA_OK;
        int n_work = 0;
        for (int r = 0; r < a.n_ranges; ++r) n_work += s_live[r];
        a.hdr->n_seg = e ? 0 : s_n_seg;
        a.hdr->n_active = e ? 0 : s_n_active;
        a.hdr->n_work = e ? 0 : n_work;
    }
}

// The plan lora_device_plan writes for the same bounds (so the builder's
// capacities, which bound every write it makes, can be trusted).
bool same_plan(const lora_device_plan_t& p, const lora_device_plan_t& q) {
    if (p.n_rows != q.n_rows || p.n_adapters != q.n_adapters || p.max_rank != q.max_rank || p.d_in != q.d_in ||
        p.d_out != q.d_out || p.seg_capacity != q.seg_capacity || p.work_capacity != q.work_capacity ||
        p.off_row_index != q.off_row_index || p.off_seg_start != q.off_seg_start ||
        p.off_seg_adapter != q.off_seg_adapter || p.off_seg_rank != q.off_seg_rank ||
        p.off_scratch != q.off_scratch || p.off_work != q.off_work || p.workspace_bytes != q.workspace_bytes)
        return false;
    const lora_plan_info_t &a = p.info, &b = q.info;
    if (a.op != b.op || a.n_work != b.n_work || a.n_active != b.n_active || a.max_rank != b.max_rank ||
        a.max_adapter != b.max_adapter || a.v_slices != b.v_slices || a.d_in != b.d_in || a.d_out != b.d_out ||
        a.n_ranges != b.n_ranges)
        return false;
    for (int r = 0; r < a.n_ranges; ++r)
        if (a.ranges[r].variant != b.ranges[r].variant || a.ranges[r].begin != b.ranges[r].begin ||
            a.ranges[r].count != b.ranges[r].count || a.ranges[r].rows_per_item != b.ranges[r].rows_per_item)
            return false;
    return true;
}

}  // namespace

extern "C" int32_t lora_batch_build_device(const lora_device_plan_t* plan, const int32_t* row_adapter,
                                           const int32_t* adapter_rank, void* workspace, void* hip_stream,
                                           lora_launch_t* out) {
    if (!plan || !row_adapter || !adapter_rank || !workspace || !out || ((uintptr_t)workspace & 255u) != 0)
        return LORA_EINVAL;
    // the capacities bound every write of the builder, so the plan must be
    // one lora_device_plan wrote; plans verified before are remembered (the
    // layout costs a few microseconds to recompute, a serving loop calls this
    // every step)
    static std::mutex mu;
    static lora_device_plan_t verified[8];
    static int n_verified = 0, next_slot = 0;
    bool known = false;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < n_verified && !known; ++i) known = same_plan(verified[i], *plan);
    }
    lora_device_plan_t chk;
    if (!known) {
        if (lora_device_plan(plan->n_rows, plan->n_adapters, plan->max_rank, plan->d_in, plan->d_out, &chk) !=
                LORA_OK ||
            !same_plan(chk, *plan))
            return LORA_EINVAL;
        std::lock_guard<std::mutex> lock(mu);
        verified[next_slot] = chk;
        next_slot = (next_slot + 1) % 8;
        if (n_verified < 8) ++n_verified;
    } else {
        chk = *plan;
    }
    char* ws = static_cast<char*>(workspace);
    BuildArgs args;
    memset(&args, 0, sizeof(args));
    args.row_adapter = row_adapter;
    args.adapter_rank = adapter_rank;
    args.n_rows = chk.n_rows;
    args.n_adapters = chk.n_adapters;
    args.max_rank = chk.max_rank;
    args.d_in = chk.d_in;
    args.d_out = chk.d_out;
    args.n_ranges = chk.info.n_ranges;
    args.hdr = reinterpret_cast<lora_device_header_t*>(ws);
    args.row_index = reinterpret_cast<int32_t*>(ws + chk.off_row_index);
    args.seg_start = reinterpret_cast<int32_t*>(ws + chk.off_seg_start);
    args.seg_adapter = reinterpret_cast<int32_t*>(ws + chk.off_seg_adapter);
    args.seg_rank = reinterpret_cast<int32_t*>(ws + chk.off_seg_rank);
    args.scratch = reinterpret_cast<int32_t*>(ws + chk.off_scratch);
    args.work = reinterpret_cast<lora_work_t*>(ws + chk.off_work);
    for (int r = 0; r < chk.info.n_ranges; ++r) {
        args.range_variant[r] = chk.info.ranges[r].variant;
        args.range_begin[r] = chk.info.ranges[r].begin;
        args.range_cap[r] = chk.info.ranges[r].count;
    }
    const hipError_t e = launch(build_plan_kernel, dim3(1), dim3(BWG), reinterpret_cast<hipStream_t>(hip_stream), args);
    if (e != hipSuccess) return LORA_EHIP;
    memset(out, 0, sizeof(*out));
    out->row_index = args.row_index;
    out->work = args.work;
    out->info = chk.info;
    out->live = args.hdr->live;
    return LORA_OK;
}

// ------------------------------------------------------------------ pool scatter
struct ScatterArgs {
    const uint16_t* src;
    uint16_t* pool;
    int64_t n;
    const int64_t* src_off;
    const int64_t* dst_off;
    const int32_t* len;
};
// One workgroup per piece (grid-stride over pieces): 16 bytes per lane and
// step, so a 8192-element page is four steps of the workgroup.
__global__ __launch_bounds__(WG) void pool_scatter_kernel(ScatterArgs a) {
    for (int64_t i = blockIdx.x; i < a.n; i += gridDim.x) {
        const int64_t so = a.src_off[i], d = a.dst_off[i];
        const int32_t l = a.len[i];
        if (so < 0 || d < 0 || l <= 0 || l > 65536 || ((so | d | (int64_t)l) & 7)) continue;  // cheap to refuse
        for (int32_t e = 8 * (int32_t)threadIdx.x; e < l; e += 8 * WG)
            *reinterpret_cast<u32x4_t*>(a.pool + d + e) = *reinterpret_cast<const u32x4_t*>(a.src + so + e);
    }
}

extern "C" int32_t lora_pool_scatter(const uint16_t* src, uint16_t* pool, int64_t n, const int64_t* src_off,
                                     const int64_t* dst_off, const int32_t* len, void* hip_stream) {
    if (n < 0) return LORA_EINVAL;
    if (n == 0) return LORA_OK;
    if (!src || !pool || !src_off || !dst_off || !len || !aligned16(src) || !aligned16(pool)) return LORA_EINVAL;
    ScatterArgs a{src, pool, n, src_off, dst_off, len};
    const unsigned grid = (unsigned)(n < 65536 ? n : 65536);
    const hipError_t e = launch(pool_scatter_kernel, dim3(grid), dim3(WG), reinterpret_cast<hipStream_t>(hip_stream), a);
    return e == hipSuccess ? LORA_OK : LORA_EHIP;
}

extern "C" int32_t lora_batch_prepare(int32_t n_rows, const int32_t* row_adapter, int32_t n_adapters,
                                      const int32_t* adapter_rank, int32_t d_in, int32_t d_out, uint32_t op_mask,
                                      int32_t seg_capacity, int32_t* seg_start, int32_t* seg_adapter,
                                      int32_t* seg_rank, int32_t* staging, int64_t staging_capacity,
                                      void* dev_staging, void* hip_stream, lora_batch_t* out) {
    constexpr int64_t wi = sizeof(lora_work_t) / sizeof(int32_t);
    const bool want_inline = (op_mask & LORA_PREPARE_INLINE) != 0;
    op_mask &= ~LORA_PREPARE_INLINE;
    if (!out || !staging || !dev_staging || op_mask == 0 || (op_mask & ~7u) || staging_capacity < 0 || n_rows < 0)
        return LORA_EINVAL;
    if (staging_capacity < n_rows) {  // row_index goes first
        out->n_staged = n_rows;
        return LORA_ECAPACITY;
    }
    int32_t n_seg = 0, n_active = 0;
    int32_t st = lora_build_segments(n_rows, row_adapter, n_adapters, adapter_rank, seg_capacity, staging, seg_start,
                                     seg_adapter, seg_rank, &n_seg, &n_active);
    out->n_seg = n_seg;
    out->n_active = n_active;
    out->n_staged = 0;
    if (st != LORA_OK) return st;
    lora_plan_info_t info[3];
    int64_t off[3] = {-1, -1, -1}, used = n_active;
    bool fits = true;
    for (int op = 0; op < 3; ++op) {
        if (!(op_mask & (1u << op))) continue;
        const int64_t room = fits ? (staging_capacity - used) / wi : 0;
        st = lora_plan(op, n_seg, seg_start, seg_adapter, seg_rank, d_in, d_out,
                       (int32_t)(room < INT32_MAX ? room : INT32_MAX),
                       reinterpret_cast<lora_work_t*>(staging + used), &info[op]);
        if (st == LORA_ECAPACITY) fits = false;
        else if (st != LORA_OK) return st;
        off[op] = used;
        used += wi * info[op].n_work;
    }
    out->n_staged = used;
    if (!fits) return LORA_ECAPACITY;
    // a small all-fused apply plan travels in the launch arguments: no copy
    const bool inline_only = want_inline && op_mask == (1u << LORA_OP_APPLY) && plan_inlines(info[LORA_OP_APPLY]);
    int32_t* dev = static_cast<int32_t*>(dev_staging);
    for (int op = 0; op < 3; ++op) {
        lora_launch_t& L = out->launch[op];
        if (off[op] < 0) {
            memset(&L, 0, sizeof(L));
            L.info.op = -1;
            continue;
        }
        L.row_index = inline_only ? nullptr : dev;
        L.work = inline_only ? nullptr : reinterpret_cast<const lora_work_t*>(dev + off[op]);
        L.info = info[op];
        L.live = nullptr;
        L.host_row_index = staging;
        L.host_work = reinterpret_cast<const lora_work_t*>(staging + off[op]);
    }
    if (used == 0 || inline_only) return LORA_OK;
    const hipError_t e = hipMemcpyAsync(dev_staging, staging, (size_t)used * sizeof(int32_t), hipMemcpyHostToDevice,
                                        reinterpret_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? LORA_OK : LORA_EHIP;
}

namespace {
int32_t merge_impl(int32_t n_mats, const lora_merge_mat_t* mats, float sign, void* hip_stream) {
    if (n_mats < 1 || n_mats > LORA_MAX_MERGE || !mats) return LORA_EINVAL;
    MergeArgs args;
    int32_t max_tiles = 0, max_rank = 0;
    for (int i = 0; i < n_mats; ++i) {
        const lora_merge_mat_t& m = mats[i];
        if (!m.W || !aligned16(m.W)) return LORA_EINVAL;
        if (m.d_out <= 0 || m.d_in <= 0 || m.d_out % 64 != 0 || m.d_in % 64 != 0) return LORA_ESHAPE;
        if (m.ldw < m.d_in || m.ldw % 8 != 0) return LORA_EINVAL;
        if (m.rank < 1 || m.rank > LORA_MAX_RANK) return LORA_ERANK;
        if (m.adapter < 0) return LORA_EADAPTER;
        int32_t st;
        if ((st = check_rows(m.A, m.d_in, m.rank, m.adapter)) != LORA_OK) return st;
        if ((st = check_rows(m.B, m.d_out, m.rank, m.adapter)) != LORA_OK) return st;
        if (m.A.neg_from || m.B.neg_from) return LORA_EINVAL;  // the merge takes plain adapters
        const int32_t tk = (m.d_in + 511) / 512, tn = (m.d_out + 127) / 128;
        args.m[i] = MergeMat{m.W, m.ldw, m.d_out, m.d_in, to_rows(m.A), to_rows(m.B), m.adapter, m.rank,
                             sign * m.scale, tk, tk * tn};
        if (tk * tn > max_tiles) max_tiles = tk * tn;
        if (m.rank > max_rank) max_rank = m.rank;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t err = hipSuccess;
    const dim3 grid((unsigned)max_tiles, (unsigned)n_mats);
    err = launch(max_rank <= 32 ? merge_kernel<1> : max_rank <= 64 ? merge_kernel<2> : merge_kernel<4>, grid, dim3(WG),
                 s, args);
    return err == hipSuccess ? LORA_OK : LORA_EHIP;
}
}  // namespace

extern "C" int32_t lora_merge(int32_t n_mats, const lora_merge_mat_t* mats, void* hip_stream) {
    return merge_impl(n_mats, mats, 1.0f, hip_stream);
}

extern "C" int32_t lora_unmerge(int32_t n_mats, const lora_merge_mat_t* mats, void* hip_stream) {
    return merge_impl(n_mats, mats, -1.0f, hip_stream);
}
