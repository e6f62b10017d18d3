// Unified adapter pool manager (host state only): pages of a caller-owned
// device pool are assigned to adapters on demand, least recently used unpinned
// adapters are evicted when the pool is short, and the row-offset tables the
// kernels read are kept up to date.  S-LoRA article, "Unified Paging": a
// rank-R adapter weight occupies R pages of hidden-size vectors in one pool.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "../../include/hetlora.h"

struct lora_pool {
    int64_t n_pages = 0;
    int32_t page_elems = 0, n_adapters = 0, max_rank = 0, n_tables = 0;
    std::vector<int32_t> row_len, chunks;
    int64_t pages_per_rank = 0;      // pages one rank row takes over all tables
    std::vector<int64_t> free_pages;  // stack of free page ids
    struct Adapter {
        int32_t rank = 0;             // resident rank (0: not resident)
        int32_t pins = 0;
        uint64_t used = 0;            // last acquire that listed it
        std::vector<int64_t> pages;   // table-major, then rank row, then chunk
    };
    std::vector<Adapter> ad;
    std::vector<std::vector<int64_t>> row_off;  // per table: n_adapters * max_rank * chunks
    uint64_t tick = 0;

    int64_t pages_of(int32_t rank) const { return pages_per_rank * rank; }

    void place(int32_t a, int32_t rank) {  // assign pages (free list must hold enough)
        Adapter& A = ad[(size_t)a];
        A.rank = rank;
        A.pages.resize((size_t)pages_of(rank));
        size_t k = 0;
        for (int32_t t = 0; t < n_tables; ++t) {
            const int32_t ch = chunks[(size_t)t];
            int64_t* tab = row_off[(size_t)t].data() + (int64_t)a * max_rank * ch;
            for (int32_t j = 0; j < rank; ++j)
                for (int32_t c = 0; c < ch; ++c) {
                    const int64_t p = free_pages.back();
                    free_pages.pop_back();
                    A.pages[k++] = p;
                    tab[(int64_t)j * ch + c] = p * page_elems;
                }
        }
    }
    void evict(int32_t a) {
        Adapter& A = ad[(size_t)a];
        for (int64_t p : A.pages) free_pages.push_back(p);
        A.pages.clear();
        A.rank = 0;
        for (int32_t t = 0; t < n_tables; ++t) {
            const int32_t ch = chunks[(size_t)t];
            int64_t* tab = row_off[(size_t)t].data() + (int64_t)a * max_rank * ch;
            std::fill(tab, tab + (int64_t)max_rank * ch, (int64_t)0);
        }
    }
};

extern "C" int32_t lora_pool_create(int64_t n_pages, int32_t page_elems, int32_t n_adapters, int32_t max_rank,
                                    int32_t n_tables, const int32_t* row_len, lora_pool_t** out) {
    if (!out || !row_len || n_pages <= 0 || n_adapters <= 0 || n_tables < 1 || n_tables > 64) return LORA_EINVAL;
    // pages up to 65536 elements: the scatter kernel's piece limit
    if (page_elems <= 0 || page_elems % 64 != 0 || page_elems > 65536) return LORA_ESHAPE;
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERANK;
    for (int32_t t = 0; t < n_tables; ++t)
        if (row_len[t] <= 0 || row_len[t] % 64 != 0) return LORA_ESHAPE;
    lora_pool* P = new (std::nothrow) lora_pool;
    if (!P) return LORA_EINVAL;
    P->n_pages = n_pages;
    P->page_elems = page_elems;
    P->n_adapters = n_adapters;
    P->max_rank = max_rank;
    P->n_tables = n_tables;
    P->row_len.assign(row_len, row_len + n_tables);
    for (int32_t t = 0; t < n_tables; ++t) {
        const int32_t ch = (row_len[t] + page_elems - 1) / page_elems;
        P->chunks.push_back(ch);
        P->pages_per_rank += ch;
        P->row_off.emplace_back((size_t)n_adapters * max_rank * ch, (int64_t)0);
    }
    P->ad.resize((size_t)n_adapters);
    P->free_pages.resize((size_t)n_pages);
    for (int64_t i = 0; i < n_pages; ++i) P->free_pages[(size_t)i] = n_pages - 1 - i;  // page 0 handed out first
    *out = P;
    return LORA_OK;
}

extern "C" int32_t lora_pool_destroy(lora_pool_t* pool) {
    delete pool;
    return LORA_OK;
}

extern "C" int32_t lora_pool_acquire(lora_pool_t* P, int32_t n, const int32_t* adapters, const int32_t* ranks,
                                     int32_t* load, int32_t* n_load) {
    if (!P || n < 0 || !n_load || (n > 0 && (!adapters || !ranks || !load))) return LORA_EINVAL;
    // validate, and find each listed adapter's rank (conflicting ranks: invalid)
    std::vector<int32_t> want((size_t)P->n_adapters, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i], r = ranks[i];
        if (a < 0 || a >= P->n_adapters) return LORA_EADAPTER;
        if (r < 1 || r > P->max_rank) return LORA_ERANK;
        if (want[(size_t)a] != 0 && want[(size_t)a] != r) return LORA_EINVAL;
        const lora_pool::Adapter& A = P->ad[(size_t)a];
        if (A.pins > 0 && A.rank != r) return LORA_EINVAL;  // a rank cannot change while in use
        want[(size_t)a] = r;
    }
    // pages needed by the listed adapters that are not resident at their rank,
    // and pages that can be had: free, listed adapters reloaded at another
    // rank, and unpinned residents that are not listed
    int64_t need = 0, avail = (int64_t)P->free_pages.size();
    for (int32_t a = 0; a < P->n_adapters; ++a) {
        const lora_pool::Adapter& A = P->ad[(size_t)a];
        const int32_t w = want[(size_t)a];
        if (w != 0 && A.rank != w) need += P->pages_of(w);
        if (A.rank != 0 && A.pins == 0 && (w == 0 || A.rank != w)) avail += P->pages_of(A.rank);
    }
    if (need > avail) return LORA_ECAPACITY;

    // listed adapters resident at another rank give their pages back first
    for (int32_t a = 0; a < P->n_adapters; ++a) {
        const int32_t w = want[(size_t)a];
        if (w != 0 && P->ad[(size_t)a].rank != 0 && P->ad[(size_t)a].rank != w) P->evict(a);
    }
    const uint64_t now = ++P->tick;
    int32_t nl = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i], r = ranks[i];
        lora_pool::Adapter& A = P->ad[(size_t)a];
        if (A.rank != r) {
            while ((int64_t)P->free_pages.size() < P->pages_of(r)) {
                // least recently used resident that is neither pinned nor listed
                int32_t victim = -1;
                for (int32_t b = 0; b < P->n_adapters; ++b) {
                    const lora_pool::Adapter& B = P->ad[(size_t)b];
                    if (B.rank == 0 || B.pins > 0 || want[(size_t)b] != 0) continue;
                    if (victim < 0 || B.used < P->ad[(size_t)victim].used) victim = b;
                }
                P->evict(victim);  // exists: checked above
            }
            P->place(a, r);
            load[nl++] = a;
        }
        A.used = now;
        ++A.pins;
    }
    *n_load = nl;
    return LORA_OK;
}

extern "C" int32_t lora_pool_release(lora_pool_t* P, int32_t n, const int32_t* adapters) {
    if (!P || n < 0 || (n > 0 && !adapters)) return LORA_EINVAL;
    std::vector<int32_t> drop((size_t)P->n_adapters, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i];
        if (a < 0 || a >= P->n_adapters) return LORA_EADAPTER;
        if (++drop[(size_t)a] > P->ad[(size_t)a].pins) return LORA_EINVAL;
    }
    for (int32_t a = 0; a < P->n_adapters; ++a) P->ad[(size_t)a].pins -= drop[(size_t)a];
    return LORA_OK;
}

extern "C" int32_t lora_pool_row_off(const lora_pool_t* P, int32_t table, const int64_t** row_off, int32_t* chunks) {
    if (!P || !row_off || !chunks || table < 0 || table >= P->n_tables) return LORA_EINVAL;
    *row_off = P->row_off[(size_t)table].data();
    *chunks = P->chunks[(size_t)table];
    return LORA_OK;
}

extern "C" int32_t lora_pool_stats(const lora_pool_t* P, int32_t* n_resident, int64_t* free_pages, int32_t* n_pinned) {
    if (!P) return LORA_EINVAL;
    int32_t res = 0, pin = 0;
    for (const lora_pool::Adapter& A : P->ad) {
        res += A.rank != 0;
        pin += A.pins > 0;
    }
    if (n_resident) *n_resident = res;
    if (free_pages) *free_pages = (int64_t)P->free_pages.size();
    if (n_pinned) *n_pinned = pin;
    return LORA_OK;
}

extern "C" int32_t lora_pool_load_list(const lora_pool_t* P, int32_t n, const int32_t* adapters, int64_t capacity,
                                       int64_t* src_off, int64_t* dst_off, int32_t* len, int64_t* n_pieces,
                                       int64_t* src_elems) {
    if (!P || n < 0 || capacity < 0 || !n_pieces || !src_elems || (n > 0 && !adapters)) return LORA_EINVAL;
    if (capacity > 0 && (!src_off || !dst_off || !len)) return LORA_EINVAL;
    int64_t needed = 0, src = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i];
        if (a < 0 || a >= P->n_adapters || P->ad[(size_t)a].rank == 0) return LORA_EINVAL;
        needed += P->pages_of(P->ad[(size_t)a].rank);
    }
    *n_pieces = needed;
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        const lora_pool::Adapter& A = P->ad[(size_t)adapters[i]];
        size_t q = 0;
        for (int32_t t = 0; t < P->n_tables; ++t) {
            const int32_t rl = P->row_len[(size_t)t], ch = P->chunks[(size_t)t];
            for (int32_t j = 0; j < A.rank; ++j)
                for (int32_t c = 0; c < ch; ++c, ++q) {
                    if (k < capacity) {
                        src_off[k] = src + (int64_t)j * rl + (int64_t)c * P->page_elems;
                        dst_off[k] = A.pages[q] * P->page_elems;
                        len[k] = std::min(P->page_elems, rl - c * P->page_elems);
                    }
                    ++k;
                }
            src += (int64_t)A.rank * rl;
        }
    }
    *src_elems = src;
    return needed > capacity ? LORA_ECAPACITY : LORA_OK;
}
