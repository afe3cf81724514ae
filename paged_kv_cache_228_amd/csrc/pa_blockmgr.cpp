// Host-side KV block manager and the block copy that copy-on-write needs.
//
// paged-attention-runtime summary, "CORE CAPABILITIES" 1 (Block Manager: fixed
// 16-token blocks, a free-list allocator, reference counting, prefix sharing,
// copy-on-write, fragmentation metrics); PagedAttention & KV-Cache Memory
// Management, glossary page (the prefix-sharing allocator: per physical block
// a reference count and an optional prefix hash; a cached hash hands out the
// same block with one more reference; free blocks go out lowest id first).
// Declarations and the contract of each call are in include/pa.h.
#include <cstdint>
#include <functional>
#include <mutex>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_manager {
    int block_size = 16;
    std::vector<int32_t> ref;                 // references per block
    std::vector<uint64_t> hash;               // prefix hash per block
    std::vector<uint8_t> hashed;              // whether the block holds one
    std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free;  // lowest id first
    std::unordered_map<uint64_t, int32_t> cache;  // prefix hash -> live block
    std::mutex mu;                            // one call at a time per manager

    bool live(int32_t b) const { return b >= 0 && (size_t)b < ref.size() && ref[b] > 0; }

    int32_t take(const uint64_t* h)  // a free block with one reference
    {
        const int32_t b = free.top();
        free.pop();
        ref[b] = 1;
        hashed[b] = h != nullptr;
        hash[b] = h ? *h : 0;
        if (h) cache[*h] = b;
        return b;
    }

    void drop(int32_t b)  // one reference fewer; the block goes free at zero
    {
        if (--ref[b] > 0) return;
        if (hashed[b]) {
            auto it = cache.find(hash[b]);
            if (it != cache.end() && it->second == b) cache.erase(it);
        }
        hashed[b] = 0;
        free.push(b);
    }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int block_size)
{
    if (num_blocks <= 0 || num_blocks > 0x7fffffffLL || block_size <= 0) return nullptr;
    pa_block_manager* m = new (std::nothrow) pa_block_manager;
    if (!m) return nullptr;
    try {
        m->block_size = block_size;
        m->ref.assign((size_t)num_blocks, 0);
        m->hash.assign((size_t)num_blocks, 0);
        m->hashed.assign((size_t)num_blocks, 0);
        std::vector<int32_t> ids((size_t)num_blocks);
        for (int64_t i = 0; i < num_blocks; ++i) ids[(size_t)i] = (int32_t)i;
        m->free = decltype(m->free)(std::greater<int32_t>(), std::move(ids));
    } catch (...) {
        delete m;
        return nullptr;
    }
    return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int pa_bm_allocate(pa_block_manager* m, const uint64_t* prefix_hash, int32_t* block, int* cache_hit)
{
    if (!m || !block) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    if (prefix_hash) {
        auto it = m->cache.find(*prefix_hash);
        if (it != m->cache.end()) {
            ++m->ref[it->second];
            *block = it->second;
            if (cache_hit) *cache_hit = 1;
            return PA_OK;
        }
    }
    if (m->free.empty()) return PA_ERR_FULL;
    try {
        *block = m->take(prefix_hash);
    } catch (...) {
        return PA_ERR_FULL;
    }
    if (cache_hit) *cache_hit = 0;
    return PA_OK;
}

int pa_bm_share(pa_block_manager* m, int32_t block)
{
    if (!m) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    if (!m->live(block)) return PA_ERR_STATE;
    if (m->ref[block] == 0x7fffffff) return PA_ERR_FULL;
    ++m->ref[block];
    return PA_OK;
}

int pa_bm_release(pa_block_manager* m, int32_t block)
{
    if (!m) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    if (!m->live(block)) return PA_ERR_STATE;
    m->drop(block);
    return PA_OK;
}

int pa_bm_copy_on_write(pa_block_manager* m, int32_t block, int32_t* out_block, int* must_copy)
{
    if (!m || !out_block || !must_copy) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    if (!m->live(block)) return PA_ERR_STATE;
    if (m->ref[block] == 1) {
        *out_block = block;
        *must_copy = 0;
        return PA_OK;
    }
    if (m->free.empty()) return PA_ERR_FULL;
    *out_block = m->take(nullptr);
    --m->ref[block];  // still referenced by the others
    *must_copy = 1;
    return PA_OK;
}

int64_t pa_bm_num_free(pa_block_manager* m)
{
    if (!m) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    return (int64_t)m->free.size();
}

int pa_bm_refcounts(pa_block_manager* m, int32_t* out, int64_t n)
{
    if (!m || !out) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lock(m->mu);
    if (n != (int64_t)m->ref.size()) return PA_ERR_SHAPE;
    for (int64_t i = 0; i < n; ++i) out[i] = m->ref[(size_t)i];
    return PA_OK;
}

double pa_internal_fragmentation(const int32_t* context_lens, int num_seqs, int block_size)
{
    if (!context_lens || num_seqs <= 0 || block_size <= 0) return 0.0;
    long double used = 0, slots = 0;
    for (int s = 0; s < num_seqs; ++s) {
        const int64_t n = context_lens[s];
        if (n <= 0) continue;
        used += (long double)n;
        slots += (long double)((n + block_size - 1) / block_size) * block_size;
    }
    return slots > 0 ? (double)(1.0L - used / slots) : 0.0;
}

}  // extern "C"
