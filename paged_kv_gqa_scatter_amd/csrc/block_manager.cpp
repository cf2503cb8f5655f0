// Host-side block manager and prefix cache of the paged KV pools (the C ABI
// of include/pkv_blocks.h).
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.3.1: fixed 256-token blocks
// (any power of two in [16, 256] here) taken from a free pool in O(1), one
// block list per sequence, a new block when the last one is full.  Section
// 4.4.4: a prefix's KV found by a hash of its token ids, the longest cached
// prefix first.  Here a cached prefix is a chain of entries, one per block:
// entry i holds the token ids stored in block i and points to entry i - 1, so
// a lookup walks the chain block by block (each step one hash probe plus an
// exact comparison of at most block_size token ids) and stops at the first
// block that is not cached; only the last block of a chain may be partial.
// Blocks carry a reference count (sequences and cache entries holding them)
// and a fill level; a sequence writes a block in place only at its frontier,
// else it first gets a private copy (copy-on-write).  The count of blocks
// only the cache holds is kept up to date, so available() is O(1), and the
// cache entries that may be evicted are kept ordered by last use, so the
// least recently used one is found in O(log n).
#include <algorithm>
#include <cstdint>
#include <deque>
#include <memory>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/pkv.h"
#include "../../include/pkv_blocks.h"

namespace {

struct Entry {
    Entry* parent;
    int32_t block;
    std::vector<int32_t> tokens;  // token ids held by this block (block_size, or fewer at a chain's end)
    uint64_t key;
    int32_t children = 0;  // entries whose parent this is
    uint64_t last_use = 0;
    bool in_lru = false;   // listed among the evictable entries, under lru_key
    uint64_t lru_key = 0;
};

struct Block {
    int32_t ref = 0;     // sequences + cache entries holding the block
    int32_t cached = 0;  // cache entries among them
    int32_t fill = 0;    // slots [0, fill) hold K/V
    std::vector<Entry*> owners;  // the cache entries holding the block
};

struct Sequence {
    std::vector<int32_t> blocks;
    int32_t len = 0;
};

// FNV-1a over the parent's key and the token ids: the content key of a block.
uint64_t chain_key(uint64_t parent_key, const int32_t* t, int32_t n) {
    uint64_t h = parent_key ^ 0xcbf29ce484222325ull;
    for (int32_t i = 0; i < n; ++i) {
        uint32_t v = (uint32_t)t[i];
        for (int b = 0; b < 4; ++b) {
            h ^= (v >> (8 * b)) & 0xffu;
            h *= 0x100000001b3ull;
        }
    }
    return h;
}

constexpr uint64_t kRootKey = 0x9e3779b97f4a7c15ull;

}  // namespace

struct pkv_block_manager {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<Block> blocks;
    std::deque<int32_t> free_pool;
    std::unordered_map<int64_t, Sequence> seqs;
    std::unordered_multimap<uint64_t, Entry*> table;
    std::unordered_map<Entry*, std::unique_ptr<Entry>> entries;
    uint64_t clock = 0;

    Entry* find(const Entry* parent, const int32_t* t, int32_t n) const {
        const uint64_t key = chain_key(parent ? parent->key : kRootKey, t, n);
        auto range = table.equal_range(key);
        for (auto it = range.first; it != range.second; ++it) {
            Entry* e = it->second;
            if (e->parent != parent || (int32_t)e->tokens.size() != n) continue;
            bool same = true;
            for (int32_t i = 0; i < n && same; ++i) same = e->tokens[i] == t[i];
            if (same) return e;
        }
        return nullptr;
    }

    // evictable entries (no child entry, no sequence holding the block) by last use
    std::set<std::pair<uint64_t, Entry*>> lru;
    int32_t cache_only = 0;  // blocks held by cache entries alone (ref > 0, ref == cached)

    bool evictable(const Entry* e) const {
        const Block& b = blocks[e->block];
        return e->children == 0 && b.ref == b.cached;
    }

    // Put e in or out of the eviction order (and re-key it) after a change of
    // its last use, its children or its block's holders.
    void refresh(Entry* e) {
        if (e->in_lru) {
            lru.erase({e->lru_key, e});
            e->in_lru = false;
        }
        if (evictable(e)) {
            e->lru_key = e->last_use;
            lru.insert({e->lru_key, e});
            e->in_lru = true;
        }
    }

    // Change a block's holders (sequences via dref, cache entries via dcached
    // as well), keeping the cache-only count and the eviction order current.
    void hold(int32_t b, int32_t dref, int32_t dcached) {
        Block& bl = blocks[b];
        const bool was = bl.ref > 0 && bl.ref == bl.cached;
        bl.ref += dref;
        bl.cached += dcached;
        const bool now = bl.ref > 0 && bl.ref == bl.cached;
        cache_only += (int32_t)now - (int32_t)was;
        if (was != now)
            for (Entry* e : bl.owners) refresh(e);
    }

    int32_t available() const { return (int32_t)free_pool.size() + cache_only; }

    // One holder less (a cache entry's too when dcached = -1); the block goes
    // back to the free pool when nothing holds it.
    void release(int32_t b, int32_t dcached = 0) {
        hold(b, -1, dcached);
        if (blocks[b].ref == 0) {
            blocks[b].fill = 0;
            free_pool.push_back(b);
        }
    }

    void add_entry(Entry* e) {
        blocks[e->block].owners.push_back(e);
        hold(e->block, 1, 1);
        if (e->parent) {
            ++e->parent->children;
            refresh(e->parent);
        }
        refresh(e);
    }

    void evict(Entry* e) {
        auto range = table.equal_range(e->key);
        for (auto it = range.first; it != range.second; ++it)
            if (it->second == e) {
                table.erase(it);
                break;
            }
        if (e->in_lru) lru.erase({e->lru_key, e});
        e->in_lru = false;
        if (e->parent) {
            --e->parent->children;
            refresh(e->parent);
        }
        std::vector<Entry*>& own = blocks[e->block].owners;
        own.erase(std::find(own.begin(), own.end(), e));
        release(e->block, -1);
        entries.erase(e);
    }

    // A block from the free pool, evicting least recently used cached chain
    // ends no sequence holds while the pool is empty.  The caller has checked
    // available(), so this succeeds: a cache-only block's entries are evicted
    // chain end first, and each eviction frees a block or makes its parent
    // evictable.
    int32_t alloc() {
        while (free_pool.empty() && !lru.empty()) evict(lru.begin()->second);
        if (free_pool.empty()) return -1;  // unreachable when available() was checked
        const int32_t b = free_pool.front();
        free_pool.pop_front();
        hold(b, 1, 0);
        blocks[b].fill = 0;
        return b;
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size) {
    if (num_blocks <= 0 || block_size < 16 || block_size > 256 || (block_size & (block_size - 1))) return nullptr;
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->blocks.resize(num_blocks);
        for (int32_t b = 0; b < num_blocks; ++b) bm->free_pool.push_back(b);
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_available(const pkv_block_manager* bm) { return bm ? bm->available() : 0; }

int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int32_t n_tokens, int32_t* cow_src,
                      int32_t* cow_dst) {
    if (!bm || !cow_src || !cow_dst) return PKV_ERR_NULL_POINTER;
    if (n_tokens < 0) return PKV_ERR_BAD_SHAPE;
    *cow_src = *cow_dst = -1;
    const int32_t B = bm->block_size;
    auto it = bm->seqs.find(seq_id);
    const int32_t len = it == bm->seqs.end() ? 0 : it->second.len;
    const int32_t nblk = it == bm->seqs.end() ? 0 : (int32_t)it->second.blocks.size();
    if ((int64_t)len + n_tokens > INT32_MAX) return PKV_ERR_BAD_SHAPE;
    if (n_tokens == 0) {
        if (it == bm->seqs.end()) bm->seqs.emplace(seq_id, Sequence());
        return PKV_OK;
    }
    const int32_t off = len % B;
    const bool cow = off != 0 && bm->blocks[it->second.blocks.back()].fill != off;
    const int32_t need = (int32_t)(((int64_t)len + n_tokens - 1) / B + 1) - nblk + (cow ? 1 : 0);
    if (need > bm->available()) return PKV_ERR_NO_BLOCKS;
    Sequence& s = bm->seqs[seq_id];
    if (cow) {
        const int32_t src = s.blocks.back();
        const int32_t dst = bm->alloc();
        bm->blocks[dst].fill = off;
        s.blocks.back() = dst;
        bm->release(src);
        *cow_src = src;
        *cow_dst = dst;
    }
    const int32_t end = len + n_tokens;
    while ((int64_t)s.blocks.size() * B < end) s.blocks.push_back(bm->alloc());
    for (int32_t i = len / B; i < (int32_t)s.blocks.size(); ++i) {
        const int32_t f = end - i * B < B ? end - i * B : B;
        Block& b = bm->blocks[s.blocks[i]];
        if (f > b.fill) b.fill = f;
    }
    s.len = end;
    return PKV_OK;
}

int32_t pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_NULL_POINTER;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    for (int32_t b : it->second.blocks) bm->release(b);
    bm->seqs.erase(it);
    return PKV_OK;
}

int32_t pkv_bm_block_table(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                           int32_t max_blocks_per_seq, int32_t* table) {
    if (!bm || (n > 0 && (!seq_ids || !table))) return PKV_ERR_NULL_POINTER;
    if (n < 0 || max_blocks_per_seq < 0) return PKV_ERR_BAD_SHAPE;
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
        if ((int32_t)it->second.blocks.size() > max_blocks_per_seq) return PKV_ERR_BAD_SHAPE;
    }
    for (int32_t i = 0; i < n; ++i) {
        const std::vector<int32_t>& bl = bm->seqs.find(seq_ids[i])->second.blocks;
        int32_t* row = table + (int64_t)i * max_blocks_per_seq;
        for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < (int32_t)bl.size() ? bl[j] : -1;
    }
    return PKV_OK;
}

int32_t pkv_bm_cache_prefix(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n_tokens) {
    if (!bm || (n_tokens > 0 && !tokens)) return PKV_ERR_NULL_POINTER;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (n_tokens < 0 || n_tokens > it->second.len) return PKV_ERR_BAD_SHAPE;
    const int32_t B = bm->block_size;
    Entry* parent = nullptr;
    const uint64_t now = ++bm->clock;
    for (int32_t i = 0; (int64_t)i * B < n_tokens; ++i) {
        const int32_t n = n_tokens - i * B < B ? n_tokens - i * B : B;
        const int32_t* t = tokens + (int64_t)i * B;
        Entry* e = bm->find(parent, t, n);
        if (!e) {
            std::unique_ptr<Entry> ne(new Entry());
            ne->parent = parent;
            ne->block = it->second.blocks[i];
            ne->tokens.assign(t, t + n);
            ne->key = chain_key(parent ? parent->key : kRootKey, t, n);
            e = ne.get();
            e->last_use = now;
            bm->entries.emplace(e, std::move(ne));
            bm->table.emplace(e->key, e);
            bm->add_entry(e);
        }
        e->last_use = now;
        bm->refresh(e);
        parent = e;
    }
    return PKV_OK;
}

int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t new_seq_id, const int32_t* tokens, int32_t n_tokens,
                    int32_t* matched) {
    if (!bm || !matched || (n_tokens > 0 && !tokens)) return PKV_ERR_NULL_POINTER;
    if (n_tokens < 0) return PKV_ERR_BAD_SHAPE;
    if (bm->seqs.count(new_seq_id)) return PKV_ERR_BAD_SHAPE;
    const int32_t B = bm->block_size;
    const uint64_t now = ++bm->clock;
    Sequence s;
    Entry* parent = nullptr;
    int32_t m = 0;
    while (m + B <= n_tokens) {  // whole blocks first
        Entry* e = bm->find(parent, tokens + m, B);
        if (!e) break;
        e->last_use = now;
        bm->refresh(e);
        s.blocks.push_back(e->block);
        parent = e;
        m += B;
    }
    const int32_t rest = n_tokens - m < B - 1 ? n_tokens - m : B - 1;
    for (int32_t r = rest; r > 0; --r) {  // then the longest partial block
        Entry* e = bm->find(parent, tokens + m, r);
        if (e) {
            e->last_use = now;
            bm->refresh(e);
            s.blocks.push_back(e->block);
            m += r;
            break;
        }
    }
    for (int32_t b : s.blocks) bm->hold(b, 1, 0);
    s.len = m;
    bm->seqs.emplace(new_seq_id, std::move(s));
    *matched = m;
    return PKV_OK;
}

}  // extern "C"
