// tq4_pages.cpp -- host page allocator for the TQ4 page pools (the ownership side of the paged
// cache; "Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory", section "StateTrans: Request
// Transitions at Safe Boundaries").  Plain host C++: no HIP calls.
//
//   - admission reserves ceil((prompt + min(output budget, 8192)) / page_size) page equivalents;
//     a request is admitted only while the reservations of all live requests fit the pool;
//   - shared prefix pages are reference counted;
//   - a departing request is filtered at the step boundary, and only then are its page
//     references dropped; a page returns to the free list when its count reaches zero.
// The free list is first in, first out: pages are handed out from its head, returned pages join
// its tail (in the departing requests' finish order, each request's pages in table order).
#include <cstdint>
#include <deque>
#include <new>
#include <vector>

#include "tq4.h"

struct tq4_page_pool {
    int32_t num_pages = 0;
    int32_t page_size = 0;
    std::vector<int32_t> refcount;
    std::deque<int32_t> free_list;
    int64_t reserved = 0;
    struct Request {
        int64_t reservation = 0;
        std::vector<int32_t> pages;
        bool live = false;
        bool departing = false;
    };
    std::vector<Request> requests;
    std::vector<int32_t> departing;  // finish order
};

namespace {

constexpr int64_t kGuaranteedOutput = 8192;

bool request_ok(const tq4_page_pool *pool, int32_t request) {
    return pool != nullptr && request >= 0 && request < static_cast<int32_t>(pool->requests.size()) &&
           pool->requests[request].live;
}

}  // namespace

extern "C" {

tq4_status tq4_pages_create(int32_t num_pages, int32_t page_size, tq4_page_pool **out) {
    if (out == nullptr) return TQ4_ERR_NULL;
    *out = nullptr;
    if (num_pages < 1 || page_size < 1) return TQ4_ERR_SHAPE;
    tq4_page_pool *pool = new (std::nothrow) tq4_page_pool;
    if (pool == nullptr) return TQ4_ERR_CAPACITY;
    pool->num_pages = num_pages;
    pool->page_size = page_size;
    pool->refcount.assign(num_pages, 0);
    for (int32_t i = 0; i < num_pages; ++i) pool->free_list.push_back(i);
    *out = pool;
    return TQ4_OK;
}

void tq4_pages_destroy(tq4_page_pool *pool) { delete pool; }

int64_t tq4_pages_admission_need(int64_t prompt_len, int64_t output_budget, int32_t page_size) {
    if (prompt_len < 0 || output_budget < 0 || page_size < 1) return -1;
    const int64_t tokens = prompt_len + (output_budget < kGuaranteedOutput ? output_budget : kGuaranteedOutput);
    return (tokens + page_size - 1) / page_size;
}

tq4_status tq4_pages_admit(tq4_page_pool *pool, int64_t prompt_len, int64_t output_budget,
                           const int32_t *prefix_pages, int32_t n_prefix, int32_t *request_out) {
    if (pool == nullptr || request_out == nullptr) return TQ4_ERR_NULL;
    if (n_prefix < 0 || (n_prefix > 0 && prefix_pages == nullptr)) return TQ4_ERR_SHAPE;
    const int64_t need = tq4_pages_admission_need(prompt_len, output_budget, pool->page_size);
    if (need < 0) return TQ4_ERR_SHAPE;
    if (static_cast<int64_t>(n_prefix) * pool->page_size > prompt_len) return TQ4_ERR_SHAPE;
    for (int32_t i = 0; i < n_prefix; ++i) {  // shared pages must be live
        const int32_t pg = prefix_pages[i];
        if (pg < 0 || pg >= pool->num_pages || pool->refcount[pg] < 1) return TQ4_ERR_SHAPE;
    }
    if (pool->reserved + need > pool->num_pages) return TQ4_ERR_CAPACITY;
    tq4_page_pool::Request r;
    r.reservation = need;
    r.live = true;
    r.pages.assign(prefix_pages, prefix_pages + n_prefix);
    for (int32_t pg : r.pages) ++pool->refcount[pg];
    pool->reserved += need;
    pool->requests.push_back(std::move(r));
    *request_out = static_cast<int32_t>(pool->requests.size() - 1);
    return TQ4_OK;
}

tq4_status tq4_pages_extend(tq4_page_pool *pool, int32_t request, int64_t length) {
    if (!request_ok(pool, request)) return TQ4_ERR_SHAPE;
    tq4_page_pool::Request &r = pool->requests[request];
    if (r.departing || length < 0) return TQ4_ERR_SHAPE;
    const int64_t pages = (length + pool->page_size - 1) / pool->page_size;
    const int64_t more = pages - static_cast<int64_t>(r.pages.size());
    if (more <= 0) return TQ4_OK;
    if (more > static_cast<int64_t>(pool->free_list.size())) return TQ4_ERR_CAPACITY;
    for (int64_t i = 0; i < more; ++i) {
        const int32_t pg = pool->free_list.front();
        pool->free_list.pop_front();
        pool->refcount[pg] = 1;
        r.pages.push_back(pg);
    }
    return TQ4_OK;
}

int32_t tq4_pages_table(const tq4_page_pool *pool, int32_t request, int32_t *table, int32_t capacity) {
    if (!request_ok(pool, request)) return -1;
    const std::vector<int32_t> &pg = pool->requests[request].pages;
    const int32_t n = static_cast<int32_t>(pg.size());
    if (table != nullptr)
        for (int32_t i = 0; i < n && i < capacity; ++i) table[i] = pg[i];
    return n;
}

tq4_status tq4_pages_finish(tq4_page_pool *pool, int32_t request) {
    if (!request_ok(pool, request)) return TQ4_ERR_SHAPE;
    tq4_page_pool::Request &r = pool->requests[request];
    if (r.departing) return TQ4_ERR_SHAPE;
    r.departing = true;
    pool->departing.push_back(request);
    return TQ4_OK;
}

tq4_status tq4_pages_boundary(tq4_page_pool *pool) {
    if (pool == nullptr) return TQ4_ERR_NULL;
    for (int32_t id : pool->departing) {
        tq4_page_pool::Request &r = pool->requests[id];
        for (int32_t pg : r.pages)
            if (--pool->refcount[pg] == 0) pool->free_list.push_back(pg);
        pool->reserved -= r.reservation;
        r.pages.clear();
        r.live = false;
    }
    pool->departing.clear();
    return TQ4_OK;
}

int32_t tq4_pages_free_count(const tq4_page_pool *pool) {
    return pool == nullptr ? -1 : static_cast<int32_t>(pool->free_list.size());
}

int32_t tq4_pages_free_list(const tq4_page_pool *pool, int32_t *pages, int32_t capacity) {
    if (pool == nullptr) return -1;
    const int32_t n = static_cast<int32_t>(pool->free_list.size());
    if (pages != nullptr)
        for (int32_t i = 0; i < n && i < capacity; ++i) pages[i] = pool->free_list[i];
    return n;
}

int32_t tq4_pages_refcount(const tq4_page_pool *pool, int32_t page) {
    if (pool == nullptr || page < 0 || page >= pool->num_pages) return -1;
    return pool->refcount[page];
}

int64_t tq4_pages_reserved(const tq4_page_pool *pool) { return pool == nullptr ? -1 : pool->reserved; }

}  // extern "C"
