// Host core of the library under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_host_sanitizers.py with g++ from csrc/host.cpp and
// csrc/pool.cpp (no HIP): drives every host entry point with seeded random
// and edge-case inputs, including every error path, through buffers
// allocated at exactly the documented sizes, so any read or write past them
// stops the run.  Light checks of the outputs ride along; bit-exact parity
// with the oracle is the Python tests' job.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "hetlora.h"

#define CHECK(c)                                                                         \
    do {                                                                                 \
        if (!(c)) {                                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);              \
            exit(1);                                                                     \
        }                                                                                \
    } while (0)

static std::mt19937_64 rng(20261202);
static int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

// heap copies of exactly n elements (a std::vector of size 0 has no storage)
template <typename T>
struct Exact {
    T* p;
    explicit Exact(size_t n) : p(n ? static_cast<T*>(malloc(n * sizeof(T))) : nullptr) {}
    ~Exact() { free(p); }
};

static void segments_and_plans() {
    for (int iter = 0; iter < 400; ++iter) {
        const int n_ad = uni(1, 40), n_rows = uni(0, 300);
        std::vector<int32_t> ra(n_rows), rk(n_ad);
        for (auto& r : rk) r = uni(1, LORA_MAX_RANK);
        const int mode = uni(0, 3);
        for (int i = 0; i < n_rows; ++i)
            ra[i] = mode == 0 ? uni(-1, n_ad - 1) : mode == 1 ? uni(0, std::min(1, n_ad - 1)) : mode == 2 ? (i * 7) % n_ad : -1;
        const int cap = std::min(n_rows, n_ad);
        Exact<int32_t> row_index(n_rows), seg_start(cap + 1), seg_adapter(cap), seg_rank(cap);
        int32_t n_seg = -1, n_active = -1;
        const int32_t st = lora_build_segments(n_rows, ra.data(), n_ad, rk.data(), cap, row_index.p, seg_start.p,
                                               seg_adapter.p, seg_rank.p, &n_seg, &n_active);
        CHECK(st == LORA_OK && n_seg <= cap && n_active <= n_rows);
        for (int s = 0; s < n_seg; ++s) CHECK(seg_start.p[s] < seg_start.p[s + 1]);
        if (n_seg > 0) {  // one slot short
            Exact<int32_t> sa(n_seg - 1), sr(n_seg - 1), ss(n_seg);
            int32_t ns2, na2;
            CHECK(lora_build_segments(n_rows, ra.data(), n_ad, rk.data(), n_seg - 1, row_index.p, ss.p, sa.p, sr.p,
                                      &ns2, &na2) == LORA_ECAPACITY);
        }
        for (int op = LORA_OP_SHRINK; op <= LORA_OP_APPLY; ++op) {
            const int d_in = 64 * uni(1, 160), d_out = 64 * uni(1, 500);
            lora_plan_info_t info;
            // size query with capacity 0, then the exact capacity, then one short
            int32_t q = lora_plan(op, n_seg, seg_start.p, seg_adapter.p, seg_rank.p, d_in, d_out, 0, nullptr, &info);
            CHECK(q == LORA_OK || q == LORA_ECAPACITY);
            const int32_t need = info.n_work;
            Exact<lora_work_t> work(need);
            CHECK(lora_plan(op, n_seg, seg_start.p, seg_adapter.p, seg_rank.p, d_in, d_out, need, work.p, &info) ==
                  LORA_OK);
            for (int w = 0; w < info.n_work; ++w) CHECK(work.p[w].nrows >= 1 && work.p[w].row0 < n_active);
            if (need > 0) {
                Exact<lora_work_t> short_work(need - 1);
                CHECK(lora_plan(op, n_seg, seg_start.p, seg_adapter.p, seg_rank.p, d_in, d_out, need - 1,
                                short_work.p, &info) == LORA_ECAPACITY);
            }
        }
    }
    // error paths
    int32_t ns, na, ri[4], ss[3], sa[2], sr[2];
    const int32_t rk2[2] = {4, 8};
    const int32_t bad_id[2] = {0, 2}, bad_lo[2] = {0, -2};
    CHECK(lora_build_segments(2, bad_id, 2, rk2, 2, ri, ss, sa, sr, &ns, &na) == LORA_EADAPTER);
    CHECK(lora_build_segments(2, bad_lo, 2, rk2, 2, ri, ss, sa, sr, &ns, &na) == LORA_EADAPTER);
    const int32_t bad_rank[2] = {0, 129}, ok_id[2] = {0, 1};
    CHECK(lora_build_segments(2, ok_id, 2, bad_rank, 2, ri, ss, sa, sr, &ns, &na) == LORA_ERANK);
    CHECK(lora_build_segments(2, nullptr, 2, rk2, 2, ri, ss, sa, sr, &ns, &na) == LORA_EINVAL);
    lora_plan_info_t info;
    CHECK(lora_plan(7, 0, ss, sa, sr, 64, 64, 0, nullptr, &info) == LORA_EINVAL);
    CHECK(lora_plan(LORA_OP_SHRINK, 0, ss, sa, sr, 100, 64, 0, nullptr, &info) == LORA_ESHAPE);
}

static void device_plans() {
    for (int iter = 0; iter < 300; ++iter) {
        const int n_rows = uni(1, 70000), n_ad = uni(0, 4200), mr = uni(0, 130);
        const int d_in = 64 * uni(0, 300), d_out = 64 * uni(0, 500);
        lora_device_plan_t p;
        const int32_t st = lora_device_plan(n_rows, n_ad, mr, d_in, d_out, &p);
        const bool ok = n_rows <= 65536 && n_ad >= 1 && n_ad <= 4096 && mr >= 1 && mr <= LORA_MAX_RANK && d_in > 0 &&
                        d_out > 0;
        CHECK((st == LORA_OK) == ok);
        if (!ok) continue;
        int64_t sum = 0;
        for (int r = 0; r < p.info.n_ranges; ++r) {
            CHECK(p.info.ranges[r].begin == sum && p.info.ranges[r].count > 0);
            sum += p.info.ranges[r].count;
        }
        CHECK(sum == p.work_capacity && p.off_work + 32 * sum <= p.workspace_bytes);
    }
    CHECK(lora_device_plan(64, 16, 16, 4096, 4096, nullptr) == LORA_EINVAL);
}

static void offsets_and_mixture() {
    for (int iter = 0; iter < 200; ++iter) {
        const int n_ad = uni(1, 12), mr = uni(1, 128), row_len = uni(1, 5000), chunk = 64 * uni(1, 40);
        std::vector<int32_t> rk(n_ad);
        for (auto& r : rk) r = uni(1, mr);
        const int chunks = (row_len + chunk - 1) / chunk;
        Exact<int64_t> off((size_t)n_ad * mr * chunks);
        int64_t pe = 0;
        CHECK(lora_rows_dense_offsets(n_ad, mr, rk.data(), row_len, chunk, off.p, &pe) == LORA_OK);
        const int merged = uni(0, n_ad - 1);
        int out_mr = 0;
        for (int a = 0; a < n_ad; ++a) out_mr = std::max(out_mr, a == merged ? rk[a] : rk[a] + rk[merged]);
        if (out_mr > LORA_MAX_RANK) {
            Exact<int64_t> o2((size_t)n_ad * LORA_MAX_RANK * chunks);
            Exact<int32_t> r2(n_ad), n2(n_ad);
            CHECK(lora_mixture_rows(n_ad, mr, rk.data(), merged, chunks, off.p, LORA_MAX_RANK, o2.p, r2.p, n2.p) ==
                  LORA_ERANK);
            continue;
        }
        Exact<int64_t> o2((size_t)n_ad * out_mr * chunks);
        Exact<int32_t> r2(n_ad), n2(n_ad);
        CHECK(lora_mixture_rows(n_ad, mr, rk.data(), merged, chunks, off.p, out_mr, o2.p, r2.p, n2.p) == LORA_OK);
        std::vector<int32_t> ra(uni(0, 50)), ra2(ra.size());
        for (auto& v : ra) v = uni(-1, n_ad - 1);
        CHECK(lora_mixture_row_adapter((int32_t)ra.size(), ra.data(), merged, (int32_t)(iter & 1), ra2.data()) == LORA_OK);
    }
    int64_t pe;
    const int32_t rk[1] = {4};
    CHECK(lora_rows_dense_offsets(1, 4, rk, 100, 100, nullptr, &pe) == LORA_EINVAL);
}

static void pool() {
    for (int iter = 0; iter < 60; ++iter) {
        const int n_tables = uni(1, 4), page = 64 * uni(1, 64), n_ad = uni(1, 30), mr = uni(1, 64);
        std::vector<int32_t> row_len(n_tables);
        for (auto& r : row_len) r = 64 * uni(1, 200);
        const int64_t n_pages = uni(1, 400);
        lora_pool_t* pl = nullptr;
        CHECK(lora_pool_create(n_pages, page, n_ad, mr, n_tables, row_len.data(), &pl) == LORA_OK);
        std::vector<int32_t> pinned, rank_of(n_ad);
        for (auto& r : rank_of) r = uni(1, mr);  // an adapter keeps its rank while pinned
        for (int step = 0; step < 40; ++step) {
            const int n = uni(0, 6);
            std::vector<int32_t> ads(n), rks(n);
            for (int i = 0; i < n; ++i) {
                ads[i] = uni(0, n_ad - 1);
                rks[i] = rank_of[ads[i]];
            }
            Exact<int32_t> load(n);
            int32_t n_load = -1;
            const int32_t st = lora_pool_acquire(pl, n, ads.data(), rks.data(), load.p, &n_load);
            CHECK(st == LORA_OK || st == LORA_ECAPACITY);
            if (st == LORA_OK) {
                CHECK(n_load >= 0 && n_load <= n);
                // the copy list of the resident listed adapters: size query, then exact
                int64_t need = 0, src = 0;
                lora_pool_load_list(pl, n, ads.data(), 0, nullptr, nullptr, nullptr, &need, &src);
                Exact<int64_t> so(need), dof(need);
                Exact<int32_t> len(need);
                int64_t got = 0;
                CHECK(lora_pool_load_list(pl, n, ads.data(), need, so.p, dof.p, len.p, &got, &src) == LORA_OK);
                CHECK(got == need);
                for (int t = 0; t < n_tables; ++t) {
                    const int64_t* off = nullptr;
                    int32_t chunks = 0;
                    CHECK(lora_pool_row_off(pl, t, &off, &chunks) == LORA_OK && off != nullptr);
                    volatile int64_t sink = 0;
                    for (int64_t e = 0; e < (int64_t)n_ad * mr * chunks; ++e) sink = sink + off[e];
                }
                pinned.insert(pinned.end(), ads.begin(), ads.end());
            }
            if (!pinned.empty() && uni(0, 1)) {  // release a random prefix of the pins
                const int k = uni(1, (int)pinned.size());
                CHECK(lora_pool_release(pl, k, pinned.data()) == LORA_OK);
                pinned.erase(pinned.begin(), pinned.begin() + k);
            }
            int32_t nr, np;
            int64_t fp;
            CHECK(lora_pool_stats(pl, &nr, &fp, &np) == LORA_OK && fp >= 0 && fp <= n_pages);
        }
        const int32_t bad = n_ad;
        const int32_t one = 1;
        int32_t ld[1], nl;
        CHECK(lora_pool_acquire(pl, 1, &bad, &one, ld, &nl) == LORA_EADAPTER);
        if (pinned.empty()) {
            const int32_t a0 = 0;
            CHECK(lora_pool_release(pl, 1, &a0) == LORA_EINVAL);
        }
        CHECK(lora_pool_destroy(pl) == LORA_OK);
    }
    lora_pool_t* pl = nullptr;
    const int32_t rl[1] = {100};
    CHECK(lora_pool_create(10, 64, 4, 8, 1, rl, &pl) == LORA_ESHAPE);
    CHECK(lora_pool_create(10, 64, 4, 0, 1, rl, &pl) == LORA_ERANK);
}

int main() {
    CHECK(lora_abi_version() == LORA_ABI_VERSION);
    for (int s = 1; s >= -7; --s) CHECK(lora_status_string(s) != nullptr);
    segments_and_plans();
    device_plans();
    offsets_and_mixture();
    pool();
    printf("host core ok\n");
    return 0;
}
