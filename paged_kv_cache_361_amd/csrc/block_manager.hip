// block_manager.hip - host-side bookkeeping of the paged KV pool: which
// physical blocks each sequence's block table holds, reference counts for
// shared blocks, copy-on-write, and block-level prefix caching.  No device
// code: it produces the block tables, slot numbers and copy pairs that the
// kernels consume.
//
// What it follows ("vLLM 推理引擎源码级拆解"):
//   §2.1-2.2  fixed-size blocks handed out on demand from one pool; a
//             per-sequence table maps logical to physical blocks; a new
//             token fills the last block's free slot or a fresh block;
//             several tables may point at one physical block, kept alive by
//             a reference count, and a write into a shared block copies it
//             first (copy on write);
//   §3.3      the manager keeps the books (owners, reference counts, free
//             blocks) and never touches the data;
//   §4.2      prefix caching: a full block's hash covers its own tokens and
//             the hash of the block before it, so equal hashes mean equal
//             prefixes; a new sequence whose leading blocks hash to cached
//             blocks points its table at them (reference count + 1) and
//             skips their prefill; cached blocks nobody references stay
//             reusable and are reclaimed least recently used first.
// Policies the pages leave open, fixed here so results are reproducible:
// the lowest-numbered free block is handed out first; when none is free,
// the cached block released longest ago is evicted; a sequence's partial
// last block is never cached; a hash match is confirmed by comparing the
// stored token ids and the previous block (no false sharing on a hash
// collision).
#include "pagedkv.h"

#include <cstdint>
#include <list>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

struct pkv_block_manager {
    struct Cached {                    // a full block registered in the prefix cache
        uint64_t hash;
        int32_t prev_block;            // block before it in the sequence it came from (-1: first)
        std::vector<int32_t> tokens;
    };
    struct Seq {
        std::vector<int32_t> table;    // physical blocks, logical order
        std::vector<int32_t> tokens;   // token ids of the whole sequence
        std::vector<uint64_t> hashes;  // hash of each full block
    };

    int32_t NB, bs;
    bool prefix_cache;
    std::vector<int32_t> ref;          // reference count per block
    std::set<int32_t> free_blocks;     // refcount 0, not cached
    std::list<int32_t> lru;            // refcount 0, cached: front = released longest ago
    std::vector<std::list<int32_t>::iterator> lru_at;
    std::vector<char> in_lru;
    std::vector<char> cached;          // block holds a registered full block
    std::vector<Cached> info;
    std::unordered_multimap<uint64_t, int32_t> by_hash;
    std::unordered_map<int64_t, Seq> seqs;

    pkv_block_manager(int32_t nb, int32_t b, bool pc)
        : NB(nb), bs(b), prefix_cache(pc), ref(nb, 0), lru_at(nb), in_lru(nb, 0), cached(nb, 0),
          info(nb) {
        for (int32_t i = 0; i < nb; i++) free_blocks.insert(free_blocks.end(), i);
    }

    int32_t available() const { return (int32_t)free_blocks.size() + (int32_t)lru.size(); }

    void uncache(int32_t b) {
        if (!cached[b]) return;
        auto range = by_hash.equal_range(info[b].hash);
        for (auto it = range.first; it != range.second; ++it)
            if (it->second == b) {
                by_hash.erase(it);
                break;
            }
        cached[b] = 0;
        info[b].tokens.clear();
    }

    // A block for new data: lowest free block, else evict the LRU cached one.
    int32_t take() {
        int32_t b;
        if (!free_blocks.empty()) {
            b = *free_blocks.begin();
            free_blocks.erase(free_blocks.begin());
        } else {
            b = lru.front();
            lru.pop_front();
            in_lru[b] = 0;
            uncache(b);
        }
        ref[b] = 1;
        return b;
    }

    void retain(int32_t b) {
        if (ref[b] == 0 && in_lru[b]) {
            lru.erase(lru_at[b]);
            in_lru[b] = 0;
        }
        ref[b]++;
    }

    void release(int32_t b) {
        if (--ref[b] > 0) return;
        if (cached[b]) {
            lru_at[b] = lru.insert(lru.end(), b);
            in_lru[b] = 1;
        } else {
            free_blocks.insert(b);
        }
    }

    // 64-bit hash of (previous block's hash, token ids), splitmix64 steps.
    static uint64_t mix(uint64_t x) {
        x += 0x9E3779B97F4A7C15ull;
        x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
        x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
        return x ^ (x >> 31);
    }
    uint64_t block_hash(uint64_t prev, const int32_t* t) const {
        uint64_t h = mix(prev ^ 0x50414745444B56ull);
        for (int32_t i = 0; i < bs; i++) h = mix(h ^ (uint32_t)t[i]);
        return h;
    }

    // Cached block holding exactly these tokens after `prev_block`, or -1.
    int32_t lookup(uint64_t h, int32_t prev_block, const int32_t* t) const {
        auto range = by_hash.equal_range(h);
        for (auto it = range.first; it != range.second; ++it) {
            const Cached& c = info[it->second];
            if (c.prev_block != prev_block) continue;
            bool same = true;
            for (int32_t i = 0; i < bs && same; i++) same = c.tokens[i] == t[i];
            if (same) return it->second;
        }
        return -1;
    }

    void register_full(Seq& s, int32_t j) {
        // block j of s just became full: record its hash; cache it unless an
        // equal block is cached already
        const uint64_t prev = j > 0 ? s.hashes[j - 1] : 0;
        const uint64_t h = block_hash(prev, s.tokens.data() + (size_t)j * bs);
        s.hashes.push_back(h);
        if (!prefix_cache) return;
        const int32_t b = s.table[j];
        const int32_t pb = j > 0 ? s.table[j - 1] : -1;
        if (cached[b] || lookup(h, pb, s.tokens.data() + (size_t)j * bs) >= 0) return;
        cached[b] = 1;
        info[b].hash = h;
        info[b].prev_block = pb;
        info[b].tokens.assign(s.tokens.begin() + (size_t)j * bs,
                              s.tokens.begin() + (size_t)(j + 1) * bs);
        by_hash.emplace(h, b);
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t enable_prefix_cache) {
    if (num_blocks <= 0 || block_size <= 0) return nullptr;
    return new (std::nothrow) pkv_block_manager(num_blocks, block_size, enable_prefix_cache != 0);
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                        int32_t num_tokens, int64_t* slots, int32_t* num_cached) {
    if (!bm || (!token_ids && num_tokens > 0) || !num_cached || (!slots && num_tokens > 0))
        return PKV_ERR_NULL;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (bm->seqs.count(seq_id)) return PKV_ERR_SHAPE;
    const int32_t bs = bm->bs;
    const int32_t nfull = num_tokens / bs;
    const int32_t nblk = (num_tokens + bs - 1) / bs;
    // leading full blocks found in the prefix cache
    std::vector<int32_t> hit;
    std::vector<uint64_t> hashes;
    uint64_t prev = 0;
    int32_t prev_block = -1;
    for (int32_t j = 0; j < nfull; j++) {
        const uint64_t h = bm->block_hash(prev, token_ids + (size_t)j * bs);
        hashes.push_back(h);
        prev = h;
        if (!bm->prefix_cache || (int32_t)hit.size() != j) continue;
        const int32_t b = bm->lookup(h, prev_block, token_ids + (size_t)j * bs);
        if (b < 0) continue;
        hit.push_back(b);
        prev_block = b;
    }
    // blocks to take: all but the hits (a hit in the LRU list is not free)
    int32_t lru_hits = 0;
    for (int32_t b : hit) lru_hits += bm->in_lru[b] ? 1 : 0;
    if (nblk - (int32_t)hit.size() > bm->available() - lru_hits) return PKV_ERR_NO_BLOCKS;

    pkv_block_manager::Seq s;
    for (int32_t b : hit) {
        bm->retain(b);
        s.table.push_back(b);
    }
    s.tokens.assign(token_ids, token_ids + num_tokens);
    s.hashes.assign(hashes.begin(), hashes.begin() + hit.size());
    for (int32_t j = (int32_t)hit.size(); j < nblk; j++) {
        s.table.push_back(bm->take());
        if (j < nfull) bm->register_full(s, j);
    }
    for (int32_t t = 0; t < num_tokens; t++)
        slots[t] = (int64_t)s.table[t / bs] * bs + t % bs;
    *num_cached = (int32_t)hit.size() * bs;
    bm->seqs.emplace(seq_id, std::move(s));
    return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int32_t token_id, int64_t* slot,
                  int32_t* copy_src, int32_t* copy_dst) {
    if (!bm || !slot || !copy_src || !copy_dst) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
    pkv_block_manager::Seq& s = it->second;
    const int32_t bs = bm->bs;
    const int32_t n = (int32_t)s.tokens.size();
    *copy_src = *copy_dst = -1;
    if (n % bs == 0) {                              // last block full (or none): a fresh one
        if (bm->available() < 1) return PKV_ERR_NO_BLOCKS;
        s.table.push_back(bm->take());
    } else {
        const int32_t last = s.table.back();
        if (bm->ref[last] > 1) {                    // shared: copy on write
            if (bm->available() < 1) return PKV_ERR_NO_BLOCKS;
            const int32_t b = bm->take();
            bm->release(last);
            s.table.back() = b;
            *copy_src = last;
            *copy_dst = b;
        }
    }
    s.tokens.push_back(token_id);
    *slot = (int64_t)s.table.back() * bs + n % bs;
    if ((n + 1) % bs == 0) bm->register_full(s, (n + 1) / bs - 1);
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PKV_ERR_SHAPE;
    pkv_block_manager::Seq s = it->second;
    for (int32_t b : s.table) bm->retain(b);
    bm->seqs.emplace(child, std::move(s));
    return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
    // the last block first, so a sequence's leading (more shareable) blocks
    // are released last and evicted last
    for (auto b = it->second.table.rbegin(); b != it->second.table.rend(); ++b) bm->release(*b);
    bm->seqs.erase(it);
    return PKV_OK;
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) {
    return bm ? bm->available() : PKV_ERR_NULL;
}

int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? PKV_ERR_SHAPE : (int32_t)it->second.tokens.size();
}

int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                           int32_t max_entries) {
    if (!bm || (!out && max_entries > 0)) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
    const std::vector<int32_t>& t = it->second.table;
    for (int32_t i = 0; i < max_entries && i < (int32_t)t.size(); i++) out[i] = t[i];
    return (int32_t)t.size();
}

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
    if (!bm) return PKV_ERR_NULL;
    if (block < 0 || block >= bm->NB) return PKV_ERR_SHAPE;
    return bm->ref[block];
}

}  // extern "C"
