// Host-side block manager with a prefix cache: the C ABI of
// include/pa_block_manager.h (see there for the behaviour and its sources
// in the pages).  Host code only.
#include "pa_block_manager.h"

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;
constexpr uint64_t kChainStart = kFnvOffset;     // "previous hash" of a sequence's first block

uint64_t fnv_bytes(uint64_t h, uint64_t v, int nbytes) {
    for (int i = 0; i < nbytes; ++i) {
        h ^= (v >> (8 * i)) & 0xFFu;
        h *= kFnvPrime;
    }
    return h;
}

// H(previous block's hash, the block's token ids, extra key)
uint64_t block_hash(uint64_t prev, const int32_t* tokens, int n, uint64_t extra) {
    uint64_t h = fnv_bytes(kFnvOffset, prev, 8);
    for (int i = 0; i < n; ++i) h = fnv_bytes(h, (uint32_t)tokens[i], 4);
    return fnv_bytes(h, extra, 8);
}

struct Block {
    int32_t ref = 0;
    bool in_free = false;
    int32_t prev = -1, next = -1;          // free-queue links
    bool cached = false;                   // holds a prefix-cache entry
    uint64_t hash = 0, prev_hash = 0;
    std::vector<int32_t> tokens;           // the block's tokens while cached
};

struct Sequence {
    std::vector<int32_t> tokens;
    std::vector<int32_t> table;
    std::vector<uint64_t> hashes;          // chained hash of every full block
};

}  // namespace

struct pa_bm {
    int32_t num_blocks = 0, block_size = 0;
    uint64_t extra = 0;
    std::vector<Block> blocks;
    int32_t head = -1, tail = -1, free_count = 0;   // free queue: head = least recently used
    std::unordered_map<uint64_t, int32_t> cache;
    std::unordered_map<int64_t, Sequence> seqs;
    std::vector<std::pair<int32_t, int32_t>> copies;
    int64_t lookups = 0, hits = 0, evictions = 0;

    void push_mru(int32_t b) {
        Block& k = blocks[b];
        k.in_free = true;
        k.prev = tail;
        k.next = -1;
        if (tail >= 0) blocks[tail].next = b;
        else head = b;
        tail = b;
        ++free_count;
    }
    void unlink(int32_t b) {
        Block& k = blocks[b];
        if (k.prev >= 0) blocks[k.prev].next = k.next;
        else head = k.next;
        if (k.next >= 0) blocks[k.next].prev = k.prev;
        else tail = k.prev;
        k.prev = k.next = -1;
        k.in_free = false;
        --free_count;
    }
    void drop_cache_entry(int32_t b) {
        Block& k = blocks[b];
        if (!k.cached) return;
        auto it = cache.find(k.hash);
        if (it != cache.end() && it->second == b) cache.erase(it);
        k.cached = false;
        k.tokens.clear();
    }
    // Least recently used free block; its cache entry is evicted.  The caller
    // has checked that one exists.
    int32_t allocate() {
        const int32_t b = head;
        unlink(b);
        if (blocks[b].cached) {
            drop_cache_entry(b);
            ++evictions;
        }
        blocks[b].ref = 1;
        return b;
    }
    void release(int32_t b) {
        if (--blocks[b].ref == 0) push_mru(b);
    }
    // The cached block for `hash`, if its predecessor and tokens match too.
    int32_t lookup(uint64_t hash, uint64_t prev, const int32_t* toks) const {
        auto it = cache.find(hash);
        if (it == cache.end()) return -1;
        const Block& k = blocks[it->second];
        if (k.prev_hash != prev || memcmp(k.tokens.data(), toks, sizeof(int32_t) * block_size) != 0) return -1;
        return it->second;
    }
    void register_full(int32_t b, uint64_t hash, uint64_t prev, const int32_t* toks) {
        if (cache.count(hash)) return;                 // an equal prefix is already findable
        Block& k = blocks[b];
        k.cached = true;
        k.hash = hash;
        k.prev_hash = prev;
        k.tokens.assign(toks, toks + block_size);
        cache.emplace(hash, b);
    }
};

extern "C" {

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, uint64_t extra_key, const int32_t* initial_order) {
    if (num_blocks <= 0 || block_size <= 0) return nullptr;
    pa_bm* bm = new (std::nothrow) pa_bm;
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->extra = extra_key;
        bm->blocks.resize(num_blocks);
        if (initial_order) {
            std::vector<char> seen(num_blocks, 0);
            for (int32_t i = 0; i < num_blocks; ++i) {
                const int32_t b = initial_order[i];
                if (b < 0 || b >= num_blocks || seen[b]) {
                    delete bm;
                    return nullptr;
                }
                seen[b] = 1;
            }
        }
        for (int32_t i = 0; i < num_blocks; ++i) bm->push_mru(initial_order ? initial_order[i] : i);
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                             int32_t* cached_tokens) {
    if (!bm || (num_tokens > 0 && !tokens)) return PA_ERR_NULL_POINTER;
    if (num_tokens < 0 || bm->seqs.count(seq_id)) return PA_ERR_BAD_SHAPE;
    const int32_t bs = bm->block_size;
    const int32_t full = num_tokens / bs;
    const int32_t total = (num_tokens + bs - 1) / bs;
    try {
        // walk the cache up to the first miss
        std::vector<uint64_t> hashes;
        std::vector<int32_t> hit_blocks;
        uint64_t prev = kChainStart;
        for (int32_t i = 0; i < full; ++i) {
            const uint64_t h = block_hash(prev, tokens + (int64_t)i * bs, bs, bm->extra);
            const int32_t b = (int32_t)hit_blocks.size() == i ? bm->lookup(h, prev, tokens + (int64_t)i * bs) : -1;
            if (b >= 0) hit_blocks.push_back(b);
            hashes.push_back(h);
            prev = h;
        }
        const int32_t n_hit = (int32_t)hit_blocks.size();
        int32_t revived = 0;
        for (int32_t b : hit_blocks) revived += bm->blocks[b].ref == 0;
        if (bm->free_count - revived < total - n_hit) return PA_ERR_POOL_EXHAUSTED;

        Sequence seq;
        seq.tokens.assign(tokens, tokens + num_tokens);
        seq.hashes = hashes;
        seq.table.reserve(total);
        for (int32_t b : hit_blocks) {
            if (bm->blocks[b].ref == 0) bm->unlink(b);
            ++bm->blocks[b].ref;
            seq.table.push_back(b);
        }
        for (int32_t i = n_hit; i < total; ++i) {
            const int32_t b = bm->allocate();
            seq.table.push_back(b);
            if (i < full) bm->register_full(b, hashes[i], i ? hashes[i - 1] : kChainStart, tokens + (int64_t)i * bs);
        }
        bm->lookups += n_hit < full ? n_hit + 1 : full;   // the walk stops at the first miss
        bm->hits += n_hit;
        bm->seqs.emplace(seq_id, std::move(seq));
        if (cached_tokens) *cached_tokens = n_hit * bs;
    } catch (...) {
        return PA_ERR_POOL_EXHAUSTED;              // host allocation failure
    }
    return PA_OK;
}

pa_status pa_bm_append_token(pa_bm* bm, int64_t seq_id, int32_t token) {
    if (!bm) return PA_ERR_NULL_POINTER;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQUENCE;
    Sequence& seq = it->second;
    const int32_t bs = bm->block_size;
    const int32_t n = (int32_t)seq.tokens.size();
    try {
        seq.tokens.reserve(n + 1);
        seq.table.reserve(seq.table.size() + 1);
        bm->copies.reserve(bm->copies.size() + 1);
        if (n % bs == 0) {                         // the tail block is full (or there is none)
            if (bm->free_count == 0) return PA_ERR_POOL_EXHAUSTED;
            seq.table.push_back(bm->allocate());
        } else {
            const int32_t tail = seq.table.back();
            if (bm->blocks[tail].ref > 1) {        // shared: copy before writing
                if (bm->free_count == 0) return PA_ERR_POOL_EXHAUSTED;
                const int32_t b = bm->allocate();
                bm->copies.emplace_back(tail, b);
                bm->release(tail);
                seq.table.back() = b;
            }
        }
        seq.tokens.push_back(token);
        if ((n + 1) % bs == 0) {                   // the block just filled up: make it findable
            const uint64_t prev = seq.hashes.empty() ? kChainStart : seq.hashes.back();
            const int32_t* toks = seq.tokens.data() + (n + 1 - bs);
            const uint64_t h = block_hash(prev, toks, bs, bm->extra);
            seq.hashes.push_back(h);
            bm->register_full(seq.table.back(), h, prev, toks);
        }
    } catch (...) {
        return PA_ERR_POOL_EXHAUSTED;
    }
    return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
    if (!bm) return PA_ERR_NULL_POINTER;
    auto it = bm->seqs.find(parent_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQUENCE;
    if (bm->seqs.count(child_id)) return PA_ERR_BAD_SHAPE;
    try {
        Sequence child = it->second;
        for (int32_t b : child.table) ++bm->blocks[b].ref;
        bm->seqs.emplace(child_id, std::move(child));
    } catch (...) {
        return PA_ERR_POOL_EXHAUSTED;
    }
    return PA_OK;
}

pa_status pa_bm_free_sequence(pa_bm* bm, int64_t seq_id) {
    if (!bm) return PA_ERR_NULL_POINTER;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_UNKNOWN_SEQUENCE;
    const std::vector<int32_t>& table = it->second.table;
    for (auto b = table.rbegin(); b != table.rend(); ++b) bm->release(*b);
    bm->seqs.erase(it);
    return PA_OK;
}

int32_t pa_bm_take_copies(pa_bm* bm, int32_t* pairs, int32_t max_pairs) {
    if (!bm) return -1;
    if (!pairs || max_pairs <= 0) return 0;
    const int32_t n = (int32_t)std::min<size_t>(bm->copies.size(), (size_t)max_pairs);
    for (int32_t i = 0; i < n; ++i) {
        pairs[2 * i] = bm->copies[i].first;
        pairs[2 * i + 1] = bm->copies[i].second;
    }
    bm->copies.erase(bm->copies.begin(), bm->copies.begin() + n);
    return n;
}

int32_t pa_bm_sequence_length(const pa_bm* bm, int64_t seq_id) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : (int32_t)it->second.tokens.size();
}

int32_t pa_bm_block_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t max_blocks) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return -1;
    const std::vector<int32_t>& t = it->second.table;
    if (out)
        for (int32_t i = 0; i < (int32_t)t.size() && i < max_blocks; ++i) out[i] = t[i];
    return (int32_t)t.size();
}

int32_t pa_bm_ref_count(const pa_bm* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->blocks[block].ref;
}

pa_status pa_bm_stats_get(const pa_bm* bm, pa_bm_stats* out) {
    if (!bm || !out) return PA_ERR_NULL_POINTER;
    int32_t cached_free = 0;
    for (int32_t b = bm->head; b >= 0; b = bm->blocks[b].next) cached_free += bm->blocks[b].cached;
    out->num_blocks = bm->num_blocks;
    out->free_blocks = bm->free_count;
    out->cached_free_blocks = cached_free;
    out->cached_blocks = (int32_t)bm->cache.size();
    out->num_sequences = (int32_t)bm->seqs.size();
    out->lookups = bm->lookups;
    out->hits = bm->hits;
    out->evictions = bm->evictions;
    return PA_OK;
}

}  // extern "C"
