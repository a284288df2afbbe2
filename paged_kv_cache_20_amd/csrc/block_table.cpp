// block_table.cpp -- host-side block-table builder.
//
// The pages fix what a block table is ("kern manifest v7" schema,
// $defs.Domain: an index into a paged state with `stride` token slots per
// entry; $defs.HostTensor: the page count is the host's choice) but no
// dealing rule.  This one gives every sequence distinct pages scattered over
// a shared pool: the pool's ids are shuffled (Durstenfeld's Fisher-Yates,
// driven by Vigna's splitmix64), then dealt to the sequences in order.
#include <cstdint>
#include <vector>

#include "../../include/pagedattn.h"

namespace pa {
// Sets the calling thread's attn_last_error() message; returns `code`
// (api.cpp).
int set_error(int code, const char* fmt, ...);
int clear_error();
}  // namespace pa

namespace {

struct SplitMix64 {
    uint64_t state;
    uint64_t next()
    {
        uint64_t z = (state += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

}  // namespace

extern "C" int attn_block_table_build(int32_t n_seq, const int32_t* ctx_lens_host,
                                      int32_t page_size, int64_t pool_pages, uint64_t seed,
                                      int32_t max_pages_per_seq, int32_t* block_table_host,
                                      int32_t* slot_mapping_host)
{
    const char* fn = "attn_block_table_build";
    if (!ctx_lens_host || !block_table_host)
        return pa::set_error(ATTN_E_ARG, "%s: ctx_lens_host/block_table_host is NULL", fn);
    if (n_seq <= 0 || page_size <= 0 || max_pages_per_seq <= 0)
        return pa::set_error(ATTN_E_ARG,
                             "%s: n_seq %d, page_size %d and max_pages_per_seq %d must be positive",
                             fn, n_seq, page_size, max_pages_per_seq);
    if (pool_pages <= 0 || pool_pages > (int64_t)INT32_MAX)
        return pa::set_error(ATTN_E_ARG, "%s: pool_pages %lld outside 1 .. 2^31 - 1", fn,
                             (long long)pool_pages);
    int64_t total = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        if (ctx_lens_host[s] < 0)
            return pa::set_error(ATTN_E_RANGE, "%s: ctx_lens_host[%d] = %d is negative", fn, s,
                                 ctx_lens_host[s]);
        const int64_t need = ((int64_t)ctx_lens_host[s] + page_size - 1) / page_size;
        if (need > max_pages_per_seq)
            return pa::set_error(ATTN_E_RANGE,
                                 "%s: sequence %d needs %lld pages, rows hold %d", fn, s,
                                 (long long)need, max_pages_per_seq);
        total += need;
    }
    if (total > pool_pages)
        return pa::set_error(ATTN_E_RANGE, "%s: the sequences need %lld pages, the pool has %lld",
                             fn, (long long)total, (long long)pool_pages);

    std::vector<int32_t> perm((size_t)pool_pages);
    for (int64_t i = 0; i < pool_pages; ++i)
        perm[(size_t)i] = (int32_t)i;
    SplitMix64 rng{seed};
    for (int64_t i = pool_pages - 1; i >= 1; --i) {
        const int64_t j = (int64_t)(rng.next() % (uint64_t)(i + 1));
        const int32_t tmp = perm[(size_t)i];
        perm[(size_t)i] = perm[(size_t)j];
        perm[(size_t)j] = tmp;
    }
    int64_t pos = 0, slot_pos = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        const int64_t need = ((int64_t)ctx_lens_host[s] + page_size - 1) / page_size;
        int32_t* row = block_table_host + (int64_t)s * max_pages_per_seq;
        for (int64_t i = 0; i < max_pages_per_seq; ++i)
            row[i] = i < need ? perm[(size_t)(pos + i)] : -1;
        pos += need;
        if (slot_mapping_host) {
            for (int64_t t = 0; t < ctx_lens_host[s]; ++t)
                slot_mapping_host[slot_pos++] =
                    (int32_t)((int64_t)row[t / page_size] * page_size + t % page_size);
        }
    }
    return pa::clear_error();
}
