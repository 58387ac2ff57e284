// block_manager.cpp -- host-side pool of physical KV blocks: the bookkeeping
// that produces the block tables and slot mappings the attention calls read.
//
// What it implements:
//   * "LLM 推理引擎深度解析：vLLM、SGLang 与 TensorRT-LLM 的核心优化原理",
//     section 2.1 "PagedAttention": a pool of num_blocks fixed-size blocks
//     with a free list; a sequence of n tokens holds ceil(n / block_size)
//     blocks, which need not be contiguous; allocation fails (no memory)
//     when too few are free; freeing returns a sequence's blocks, and
//     freeing an unknown id does nothing;
//   * "让 Agent 跑得快：LLM 推理服务", section 五: blocks are taken on
//     demand, one more each time the last one is full, so at most
//     block_size - 1 slots per sequence are unused; block tables may share
//     physical blocks under a reference count;
//   * same page, section 二, "Copy-on-Write": writing a new token into a
//     shared, partly filled last block first copies that block to a fresh
//     one and repoints the table entry (the caller performs the returned
//     copies on the device with pkv_copy_blocks before writing); a block
//     whose count drops to zero returns to the pool.
//   * same page, section 七 (automatic prefix caching): a full block is
//     identified by its parent block's identity, its tokens and an optional
//     cache salt; allocating a prompt looks its full blocks up in order,
//     takes every hit (reference count + 1) and stops at the first miss,
//     from where the prompt must be prefilled; released blocks stay
//     matchable in the free queue until it hands them out again.
// Blocks leave the front of the free list and come back at its end; a hit
// on a free cached block takes it out of the middle, so the list is doubly
// linked over block ids.  Taking a block for new contents drops its cache
// registration (the longest-freed cached block is evicted first).  The
// cache is an open-addressing table of 64-bit chain hashes; every entry
// keeps its block's parent hash, salt and tokens, which a lookup compares,
// so a hash collision is a miss, never a wrong hit.  Both structures have
// a fixed capacity (the table is sized at the first cached allocation), so
// giving blocks back and undoing a failed batch never allocate.  A call
// that would run out of blocks part-way changes nothing.
//
// Radix-tree prefix sharing ("LLM 推理优化技术全景", section "Prefix Caching 与
// RadixAttention"; "让 Agent 跑得快", section 七): cached prompts live in a
// compressed trie over their tokens (each edge a run of tokens, children
// told apart by their first token), so the longest prefix a new prompt
// shares with any of them is one walk down the trie, token by token.  An
// entry is a prompt's tokens up to its last full block with those blocks,
// on each of which it holds a reference; the partly filled last block
// stays out, since the sequence keeps writing into it.  A new prompt
// shares the donor's blocks that the match covers whole, and when the
// match ends inside a block it gets a fresh block plus a copy of the
// donor's (prefill then starts at the match's end).  The donor is the most
// recently used entry below the match point.  When blocks run short,
// entries are dropped least recently used first (never the donor), each
// releasing its references; a call that cannot be met that way changes
// nothing.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr uint64_t kRootHash = 0x6a09e667f3bcc908ull;  // parent of a prompt's first block

uint64_t mix64(uint64_t x) {  // the splitmix64 finaliser
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ull;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebull;
    return x ^ (x >> 31);
}

uint64_t chain_hash(uint64_t parent, int64_t salt, const int32_t* tokens, int n) {
    uint64_t h = mix64(parent ^ mix64((uint64_t)salt + 0x9e3779b97f4a7c15ull));
    for (int i = 0; i < n; ++i) h = mix64(h ^ (uint32_t)tokens[i]) + (uint64_t)i;
    return h;
}

}  // namespace

struct pkv_block_manager {
    struct Seq {
        std::vector<int64_t> blocks;
        int64_t length = 0;
    };
    int64_t num_blocks = 0;
    int block_size = 16;
    // free list, doubly linked through prev / next (-1 ends it)
    std::vector<int64_t> prev, next;
    int64_t head = -1, tail = -1, num_free = 0;
    std::vector<int32_t> refcount;
    std::unordered_map<int64_t, Seq> seqs;
    // prefix cache: per block, its registration (valid while has_key);
    // `evicted` remembers whether the last take() dropped a live entry
    std::vector<uint8_t> has_key, evicted;
    std::vector<uint64_t> key_hash, key_parent;
    std::vector<int64_t> key_salt;
    std::vector<int32_t> key_tokens;  // [num_blocks][block_size], sized with the table
    std::vector<uint64_t> slot_hash;  // open addressing, linear probing
    std::vector<int64_t> slot_block;  // -1: empty
    int64_t cached = 0;

    // radix tree: node 0 is the root (empty label); dead nodes and entries
    // are recycled through their free lists
    struct RNode {
        std::vector<int32_t> label;  // tokens on the edge from the parent
        int parent = -1;
        std::vector<int> kids;       // children, first tokens all different
        std::vector<int> entries;    // entries whose tokens end here
    };
    struct REntry {
        std::vector<int64_t> blocks;  // one per block_size tokens
        int64_t stamp = 0;            // last registration or hit
        int node = -1;                // where its tokens end; -1: dead
    };
    std::vector<RNode> rnodes;
    std::vector<int> rnode_free;
    std::vector<REntry> rentries;
    std::vector<int> rentry_free;
    int64_t rclock = 0, rlive = 0;
    std::vector<int> rscratch;                        // trie walks
    std::vector<std::pair<int64_t, int>> rorder;      // eviction order
    std::unordered_map<int64_t, int32_t> rdrop;       // simulated releases

    int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }

    // ---- free list
    void link_back(int64_t b) {
        prev[(size_t)b] = tail;
        next[(size_t)b] = -1;
        if (tail >= 0) next[(size_t)tail] = b; else head = b;
        tail = b;
        ++num_free;
    }
    void link_front(int64_t b) {
        next[(size_t)b] = head;
        prev[(size_t)b] = -1;
        if (head >= 0) prev[(size_t)head] = b; else tail = b;
        head = b;
        ++num_free;
    }
    void unlink(int64_t b) {
        const int64_t p = prev[(size_t)b], n = next[(size_t)b];
        if (p >= 0) next[(size_t)p] = n; else head = n;
        if (n >= 0) prev[(size_t)n] = p; else tail = p;
        --num_free;
    }

    // ---- cache table
    size_t slot_of(uint64_t h) const { return (size_t)(mix64(h) & (slot_hash.size() - 1)); }
    int64_t find(uint64_t h) const {
        if (slot_hash.empty()) return -1;
        for (size_t i = slot_of(h);; i = (i + 1) & (slot_hash.size() - 1)) {
            if (slot_block[i] < 0) return -1;
            if (slot_hash[i] == h) return slot_block[i];
        }
    }
    void put(uint64_t h, int64_t b) {  // insert or replace; the table never fills
        size_t i = slot_of(h);
        while (slot_block[i] >= 0 && slot_hash[i] != h) i = (i + 1) & (slot_hash.size() - 1);
        if (slot_block[i] < 0) ++cached;
        slot_hash[i] = h;
        slot_block[i] = b;
    }
    void erase(uint64_t h) {  // backward-shift deletion keeps probe runs unbroken
        const size_t mask = slot_hash.size() - 1;
        size_t i = slot_of(h);
        while (slot_block[i] >= 0 && slot_hash[i] != h) i = (i + 1) & mask;
        if (slot_block[i] < 0) return;
        --cached;
        for (size_t j = (i + 1) & mask;; j = (j + 1) & mask) {
            if (slot_block[j] < 0) break;
            const size_t home = slot_of(slot_hash[j]);
            // move j back into the hole at i unless its home lies in (i, j]
            if (((j - home) & mask) >= ((j - i) & mask)) {
                slot_hash[i] = slot_hash[j];
                slot_block[i] = slot_block[j];
                i = j;
            }
        }
        slot_block[i] = -1;
    }
    bool ensure_cache() {  // sized once, at the first cached allocation
        if (!slot_hash.empty()) return true;
        try {
            size_t cap = 16;
            while (cap < 2 * (size_t)num_blocks) cap <<= 1;
            key_tokens.resize((size_t)num_blocks * (size_t)block_size);
            slot_hash.assign(cap, 0);
            slot_block.assign(cap, -1);
        } catch (...) {
            key_tokens.clear();
            slot_hash.clear();
            slot_block.clear();
            return false;
        }
        return true;
    }

    // ---- taking and returning blocks
    int64_t take() {
        const int64_t b = head;
        unlink(b);
        refcount[(size_t)b] = 1;
        evicted[(size_t)b] = 0;
        if (has_key[(size_t)b]) {  // new contents: the registration goes
            if (find(key_hash[(size_t)b]) == b) {
                erase(key_hash[(size_t)b]);
                evicted[(size_t)b] = 1;
            }
            has_key[(size_t)b] = 0;
        }
        return b;
    }
    void release(int64_t b) {
        if (--refcount[(size_t)b] == 0) link_back(b);
    }
    // Undo of take(): b goes back to the FRONT of the free list with its
    // registration, so undoing takes in reverse order restores everything.
    void untake(int64_t b) {
        refcount[(size_t)b] = 0;
        link_front(b);
        if (evicted[(size_t)b]) {
            has_key[(size_t)b] = 1;
            put(key_hash[(size_t)b], b);
            evicted[(size_t)b] = 0;
        }
    }

    // What one append changed, enough to put it back.
    struct Undo {
        Seq* seq;
        int64_t old_length;
        size_t old_blocks;
        int64_t cow_old;  // -1: no copy
    };

    // Room for n more tokens of s: slots written, at most one copy (src, dst)
    // written to copy_pair when room_for_copy.  Changes nothing on failure.
    int append(Seq& s, int64_t n, int64_t* slots, int64_t* copy_pair, bool room_for_copy,
               Undo* undo) {
        const int bs = block_size;
        undo->seq = &s;
        undo->old_length = s.length;
        undo->old_blocks = s.blocks.size();
        undo->cow_old = -1;
        if (n == 0) return PKV_OK;
        // what the pool must supply: a copy of a shared partly filled last
        // block, and one block per boundary crossed
        const bool last_shared = s.length % bs != 0 && refcount[(size_t)s.blocks.back()] > 1;
        const int64_t new_blocks = blocks_for(s.length + n) - (int64_t)s.blocks.size();
        if ((last_shared ? 1 : 0) + new_blocks > num_free) return PKV_ERR_NO_MEMORY;
        if (last_shared && !room_for_copy) return PKV_ERR_SHAPE;
        try {
            s.blocks.reserve(s.blocks.size() + (size_t)new_blocks);
        } catch (...) {
            return PKV_ERR_HOST_ALLOC;
        }
        if (last_shared) {
            const int64_t old = s.blocks.back();
            const int64_t dst = take();
            copy_pair[0] = old;
            copy_pair[1] = dst;
            undo->cow_old = old;
            release(old);  // stays above zero: it was shared
            s.blocks.back() = dst;
        }
        for (int64_t i = 0; i < n; ++i) {
            const int64_t pos = s.length + i;
            if (pos / bs == (int64_t)s.blocks.size()) s.blocks.push_back(take());
            slots[i] = s.blocks[(size_t)(pos / bs)] * bs + pos % bs;
        }
        s.length += n;
        return PKV_OK;
    }

    // ---- radix tree
    int kid_with(int node, int32_t tok) const {
        for (int c : rnodes[(size_t)node].kids)
            if (rnodes[(size_t)c].label[0] == tok) return c;
        return -1;
    }
    // Longest prefix of tokens[0, n) in the trie: its length, and the node
    // below which every entry reaches it (the child whose edge it stops in,
    // or the node it ends at).
    int64_t radix_match(const int32_t* tokens, int64_t n, int* below) const {
        int node = 0;
        int64_t d = 0;
        while (d < n) {
            const int c = kid_with(node, tokens[d]);
            if (c < 0) break;
            const std::vector<int32_t>& lab = rnodes[(size_t)c].label;
            size_t m = 0;
            while (m < lab.size() && d + (int64_t)m < n && lab[m] == tokens[d + (int64_t)m]) ++m;
            d += (int64_t)m;
            node = c;
            if (m < lab.size()) break;
        }
        *below = node;
        return d;
    }
    // The most recently used live entry in the subtree of `node`.
    int radix_newest(int node) {
        int best = -1;
        rscratch.clear();
        rscratch.push_back(node);
        while (!rscratch.empty()) {
            const int x = rscratch.back();
            rscratch.pop_back();
            for (int e : rnodes[(size_t)x].entries)
                if (best < 0 || rentries[(size_t)e].stamp > rentries[(size_t)best].stamp) best = e;
            for (int c : rnodes[(size_t)x].kids) rscratch.push_back(c);
        }
        return best;
    }
    // Adding an entry for tokens[0, n) creates at most two nodes: the
    // middle of an edge the tokens leave part-way (split after m tokens) and
    // a leaf for the rest.  prepare() does everything that allocates, into
    // this plan; commit() then changes the trie without allocating.
    struct InsertPlan {
        int at = 0;          // node the walk stopped at
        int split = -1;      // child whose edge is split, or -1
        size_t m = 0;        // tokens of that edge kept in the middle node
        bool leaf = false;   // a leaf for tokens[d, n) hangs below
        RNode mid, lf;
    };
    void radix_prepare(const int32_t* tokens, int64_t n, InsertPlan& pl) {
        int node = 0;
        int64_t d = 0;
        while (d < n) {
            const int c = kid_with(node, tokens[d]);
            if (c < 0) break;
            const std::vector<int32_t>& lab = rnodes[(size_t)c].label;
            size_t m = 0;
            while (m < lab.size() && d + (int64_t)m < n && lab[m] == tokens[d + (int64_t)m]) ++m;
            if (m < lab.size()) {
                pl.split = c;
                pl.m = m;
                pl.mid.label.assign(lab.begin(), lab.begin() + (long)m);
                pl.mid.kids.reserve(2);
                pl.mid.entries.reserve(1);
                d += (int64_t)m;
                break;
            }
            node = c;
            d += (int64_t)m;
        }
        pl.at = node;
        if (d < n) {
            pl.leaf = true;
            pl.lf.label.assign(tokens + d, tokens + n);
            pl.lf.entries.reserve(1);
            if (pl.split < 0) rnodes[(size_t)node].kids.reserve(rnodes[(size_t)node].kids.size() + 1);
        } else if (pl.split < 0) {
            rnodes[(size_t)node].entries.reserve(rnodes[(size_t)node].entries.size() + 1);
        }
        rnodes.reserve(rnodes.size() + 2);
        rnode_free.reserve(rnodes.capacity());
    }
    int place_rnode(RNode&& x) {  // capacity reserved: no allocation
        if (!rnode_free.empty()) {
            const int i = rnode_free.back();
            rnode_free.pop_back();
            rnodes[(size_t)i] = std::move(x);
            return i;
        }
        rnodes.push_back(std::move(x));
        return (int)rnodes.size() - 1;
    }
    void radix_commit(InsertPlan& pl, int e) {
        int node = pl.at;
        if (pl.split >= 0) {
            const int c = pl.split;
            pl.mid.parent = node;
            pl.mid.kids.push_back(c);
            const int mid = place_rnode(std::move(pl.mid));
            RNode& cn = rnodes[(size_t)c];
            cn.label.erase(cn.label.begin(), cn.label.begin() + (long)pl.m);
            cn.parent = mid;
            for (int& k : rnodes[(size_t)node].kids)
                if (k == c) k = mid;
            node = mid;
        }
        if (pl.leaf) {
            pl.lf.parent = node;
            const int leaf = place_rnode(std::move(pl.lf));
            rnodes[(size_t)node].kids.push_back(leaf);
            node = leaf;
        }
        rnodes[(size_t)node].entries.push_back(e);
        rentries[(size_t)e].node = node;
    }
    // Drops entry e: its references go back, and nodes left with neither
    // entries nor children leave the trie.
    void radix_remove(int e) {
        REntry& en = rentries[(size_t)e];
        int node = en.node;
        std::vector<int>& es = rnodes[(size_t)node].entries;
        es.erase(std::find(es.begin(), es.end(), e));
        while (node != 0 && rnodes[(size_t)node].entries.empty() && rnodes[(size_t)node].kids.empty()) {
            const int p = rnodes[(size_t)node].parent;
            std::vector<int>& ks = rnodes[(size_t)p].kids;
            ks.erase(std::find(ks.begin(), ks.end(), node));
            rnodes[(size_t)node].label.clear();
            rnode_free.push_back(node);
            node = p;
        }
        for (int64_t b : en.blocks) release(b);
        en.blocks.clear();
        en.node = -1;
        rentry_free.push_back(e);
        --rlive;
    }

    void rollback(const Undo& u) {
        Seq& s = *u.seq;
        while (s.blocks.size() > u.old_blocks) {
            untake(s.blocks.back());
            s.blocks.pop_back();
        }
        if (u.cow_old >= 0) {
            untake(s.blocks.back());
            ++refcount[(size_t)u.cow_old];
            s.blocks.back() = u.cow_old;
        }
        s.length = u.old_length;
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int64_t num_blocks, int block_size) {
    if (num_blocks < 0 || num_blocks > INT32_MAX || block_size <= 0) return nullptr;
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
    if (bm == nullptr) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        const size_t n = (size_t)num_blocks;
        bm->refcount.assign(n, 0);
        bm->prev.assign(n, -1);
        bm->next.assign(n, -1);
        bm->has_key.assign(n, 0);
        bm->evicted.assign(n, 0);
        bm->key_hash.assign(n, 0);
        bm->key_parent.assign(n, 0);
        bm->key_salt.assign(n, 0);
        for (int64_t b = 0; b < num_blocks; ++b) bm->link_back(b);
        bm->rnodes.emplace_back();  // the radix tree's root
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int64_t pkv_bm_num_free(const pkv_block_manager* bm) {
    return bm == nullptr ? -1 : bm->num_free;
}

int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens) {
    if (bm == nullptr) return PKV_ERR_NULL;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (bm->seqs.count(seq_id)) return PKV_ERR_STATE;
    const int64_t need = bm->blocks_for(num_tokens);
    if (need > bm->num_free) return PKV_ERR_NO_MEMORY;
    try {
        pkv_block_manager::Seq s;
        s.blocks.reserve((size_t)need);
        s.length = num_tokens;
        auto& slot = bm->seqs[seq_id];  // may throw before anything is taken
        for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
        slot = std::move(s);
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    return PKV_OK;
}

int pkv_bm_allocate_cached(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                           int64_t num_tokens, int64_t salt, int64_t* num_cached_tokens) {
    if (bm == nullptr || num_cached_tokens == nullptr || (num_tokens > 0 && tokens == nullptr))
        return PKV_ERR_NULL;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (bm->seqs.count(seq_id)) return PKV_ERR_STATE;
    const int bs = bm->block_size;
    const int64_t nfull = num_tokens / bs;
    const int64_t nblk = bm->blocks_for(num_tokens);
    if (nfull > 0 && !bm->ensure_cache()) return PKV_ERR_HOST_ALLOC;
    std::vector<uint64_t> h;
    pkv_block_manager::Seq s;
    try {
        h.resize((size_t)nfull);
        s.blocks.reserve((size_t)nblk);
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    uint64_t parent = kRootHash;
    for (int64_t i = 0; i < nfull; ++i) {
        h[(size_t)i] = chain_hash(parent, salt, tokens + i * bs, bs);
        parent = h[(size_t)i];
    }
    // hits: the leading full blocks whose whole key matches
    int64_t hits = 0, free_hits = 0;
    for (; hits < nfull; ++hits) {
        const int64_t b = bm->find(h[(size_t)hits]);
        if (b < 0 || !bm->has_key[(size_t)b]) break;
        const size_t k = (size_t)b;
        const uint64_t want_parent = hits == 0 ? kRootHash : h[(size_t)hits - 1];
        if (bm->key_parent[k] != want_parent || bm->key_salt[k] != salt ||
            std::memcmp(&bm->key_tokens[k * bs], tokens + hits * bs, sizeof(int32_t) * bs) != 0)
            break;
        if (bm->refcount[k] == 0) ++free_hits;
        s.blocks.push_back(b);
    }
    if (nblk - hits > bm->num_free - free_hits) return PKV_ERR_NO_MEMORY;
    try {
        bm->seqs.emplace(seq_id, pkv_block_manager::Seq{});  // before any change
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    for (int64_t b : s.blocks) {
        if (bm->refcount[(size_t)b] == 0) bm->unlink(b);
        ++bm->refcount[(size_t)b];
    }
    for (int64_t i = hits; i < nblk; ++i) s.blocks.push_back(bm->take());
    for (int64_t i = hits; i < nfull; ++i) {  // register the new full blocks
        const size_t k = (size_t)s.blocks[(size_t)i];
        bm->key_hash[k] = h[(size_t)i];
        bm->key_parent[k] = i == 0 ? kRootHash : h[(size_t)i - 1];
        bm->key_salt[k] = salt;
        std::memcpy(&bm->key_tokens[k * bs], tokens + i * bs, sizeof(int32_t) * bs);
        bm->has_key[k] = 1;
        bm->put(h[(size_t)i], (int64_t)k);
    }
    s.length = num_tokens;
    bm->seqs[seq_id] = std::move(s);
    *num_cached_tokens = hits * bs;
    return PKV_OK;
}

int64_t pkv_bm_num_cached(const pkv_block_manager* bm) { return bm == nullptr ? -1 : bm->cached; }

int pkv_bm_allocate_radix(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                          int64_t num_tokens, int64_t* num_cached_tokens, int64_t* copy_pair) {
    if (bm == nullptr || num_cached_tokens == nullptr || copy_pair == nullptr ||
        (num_tokens > 0 && tokens == nullptr))
        return PKV_ERR_NULL;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (bm->seqs.count(seq_id)) return PKV_ERR_STATE;
    const int bs = bm->block_size;
    const int64_t n = num_tokens;
    const int64_t nblk = bm->blocks_for(n);
    const int64_t nfull = n / bs;
    int64_t L = 0, shared = 0, fresh = nblk;
    int donor = -1, e = -1;
    bool reg = false;
    size_t ndrop = 0;
    pkv_block_manager::Seq s;
    pkv_block_manager::InsertPlan plan;
    try {
        // the longest cached prefix and its donor
        int below = 0;
        L = bm->radix_match(tokens, n, &below);
        donor = L > 0 ? bm->radix_newest(below) : -1;
        if (donor < 0) L = 0;
        shared = L / bs;
        fresh = nblk - shared;
        reg = nfull > 0 && L < nfull * bs;  // else a prefix of the donor's tokens
        // what dropping entries least recently used first (never the donor)
        // would give back; nothing changes until the whole call is known to fit
        int64_t free = bm->num_free;
        if (free < fresh) {
            bm->rorder.clear();
            for (size_t k = 0; k < bm->rentries.size(); ++k)
                if (bm->rentries[k].node >= 0 && (int)k != donor)
                    bm->rorder.emplace_back(bm->rentries[k].stamp, (int)k);
            std::sort(bm->rorder.begin(), bm->rorder.end());
            bm->rdrop.clear();
            while (free < fresh && ndrop < bm->rorder.size()) {
                for (int64_t b : bm->rentries[(size_t)bm->rorder[ndrop].second].blocks)
                    if (bm->refcount[(size_t)b] - ++bm->rdrop[b] == 0) ++free;
                ++ndrop;
            }
            if (free < fresh) return PKV_ERR_NO_MEMORY;
        }
        // everything the call adds, allocated before anything changes
        s.blocks.reserve((size_t)nblk);
        if (reg) {
            bm->radix_prepare(tokens, nfull * bs, plan);
            if (bm->rentry_free.empty()) {
                bm->rentries.emplace_back();
                e = (int)bm->rentries.size() - 1;
            } else {
                e = bm->rentry_free.back();
            }
            bm->rentries[(size_t)e].blocks.reserve((size_t)nfull);
        }
        // dropped nodes and entries go to their free lists without allocating
        bm->rnode_free.reserve(bm->rnodes.capacity());
        bm->rentry_free.reserve(bm->rentries.capacity());
        bm->seqs.emplace(seq_id, pkv_block_manager::Seq{});
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    if (reg && !bm->rentry_free.empty() && bm->rentry_free.back() == e) bm->rentry_free.pop_back();
    // the new sequence's references on the shared blocks, then the drops
    for (int64_t i = 0; i < shared; ++i) {
        const int64_t b = bm->rentries[(size_t)donor].blocks[(size_t)i];
        ++bm->refcount[(size_t)b];  // held by the donor as well: never free here
        s.blocks.push_back(b);
    }
    for (size_t k = 0; k < ndrop; ++k) bm->radix_remove(bm->rorder[k].second);
    for (int64_t i = shared; i < nblk; ++i) s.blocks.push_back(bm->take());
    copy_pair[0] = copy_pair[1] = -1;
    if (L % bs != 0) {  // the match ends inside block `shared`: the donor's copy
        copy_pair[0] = bm->rentries[(size_t)donor].blocks[(size_t)shared];
        copy_pair[1] = s.blocks[(size_t)shared];
    }
    if (donor >= 0) bm->rentries[(size_t)donor].stamp = ++bm->rclock;
    if (reg) {
        pkv_block_manager::REntry& en = bm->rentries[(size_t)e];
        en.blocks.assign(s.blocks.begin(), s.blocks.begin() + (long)nfull);  // capacity reserved
        for (int64_t b : en.blocks) ++bm->refcount[(size_t)b];
        en.stamp = ++bm->rclock;
        bm->radix_commit(plan, e);
        ++bm->rlive;
    }
    s.length = n;
    bm->seqs[seq_id] = std::move(s);
    *num_cached_tokens = L;
    return PKV_OK;
}

int64_t pkv_bm_radix_num_entries(const pkv_block_manager* bm) {
    return bm == nullptr ? -1 : bm->rlive;
}

int pkv_bm_radix_clear(pkv_block_manager* bm) {
    if (bm == nullptr) return PKV_ERR_NULL;
    // least recently used first, as the drops of an allocation go
    try {
        bm->rorder.clear();
        for (size_t e = 0; e < bm->rentries.size(); ++e)
            if (bm->rentries[e].node >= 0) bm->rorder.emplace_back(bm->rentries[e].stamp, (int)e);
        bm->rnode_free.reserve(bm->rnodes.capacity());
        bm->rentry_free.reserve(bm->rentries.capacity());
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    std::sort(bm->rorder.begin(), bm->rorder.end());
    for (const auto& o : bm->rorder) bm->radix_remove(o.second);
    return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id) {
    if (bm == nullptr) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_OK;
    for (int64_t b : it->second.blocks) bm->release(b);
    bm->seqs.erase(it);
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
    if (bm == nullptr) return PKV_ERR_NULL;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PKV_ERR_STATE;
    try {
        pkv_block_manager::Seq s = it->second;  // copy before inserting (rehash)
        bm->seqs.emplace(child, std::move(s));
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    for (int64_t b : bm->seqs.at(child).blocks) ++bm->refcount[b];
    return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens, int64_t* slots,
                  int64_t* copies, int64_t max_copies, int64_t* num_copies) {
    if (bm == nullptr || num_copies == nullptr || (num_tokens > 0 && slots == nullptr))
        return PKV_ERR_NULL;
    if (num_tokens < 0 || max_copies < 0) return PKV_ERR_SHAPE;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_STATE;
    *num_copies = 0;
    pkv_block_manager::Undo undo;
    const int st = bm->append(it->second, num_tokens, slots, copies,
                              copies != nullptr && max_copies >= 1, &undo);
    if (st == PKV_OK && undo.cow_old >= 0) *num_copies = 1;
    return st;
}

int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, const int64_t* num_tokens,
                        int num_seqs, int64_t* slots, int64_t* copies, int64_t max_copies,
                        int64_t* num_copies) {
    if (bm == nullptr || num_copies == nullptr) return PKV_ERR_NULL;
    if (num_seqs < 0 || max_copies < 0) return PKV_ERR_SHAPE;
    *num_copies = 0;
    if (num_seqs == 0) return PKV_OK;
    if (seq_ids == nullptr || num_tokens == nullptr) return PKV_ERR_NULL;
    int64_t total = 0;
    for (int i = 0; i < num_seqs; ++i) {
        if (num_tokens[i] < 0) return PKV_ERR_SHAPE;
        total += num_tokens[i];
    }
    if (total > 0 && slots == nullptr) return PKV_ERR_NULL;
    std::vector<pkv_block_manager::Undo> log;
    try {
        log.reserve((size_t)num_seqs);
    } catch (...) {
        return PKV_ERR_HOST_ALLOC;
    }
    int64_t done_tokens = 0, done_copies = 0;
    int st = PKV_OK;
    for (int i = 0; i < num_seqs && st == PKV_OK; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) {
            st = PKV_ERR_STATE;
            break;
        }
        pkv_block_manager::Undo undo;
        st = bm->append(it->second, num_tokens[i], slots + done_tokens,
                        copies == nullptr ? nullptr : copies + 2 * done_copies,
                        copies != nullptr && done_copies < max_copies, &undo);
        if (st != PKV_OK) break;
        log.push_back(undo);
        done_tokens += num_tokens[i];
        if (undo.cow_old >= 0) ++done_copies;
    }
    if (st != PKV_OK) {
        for (auto u = log.rbegin(); u != log.rend(); ++u) bm->rollback(*u);
        return st;
    }
    *num_copies = done_copies;
    return PKV_OK;
}

int pkv_bm_seq_info(const pkv_block_manager* bm, int64_t seq_id, int64_t* num_tokens,
                    int64_t* num_blocks) {
    if (bm == nullptr || num_tokens == nullptr || num_blocks == nullptr) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_STATE;
    *num_tokens = it->second.length;
    *num_blocks = (int64_t)it->second.blocks.size();
    return PKV_OK;
}

int pkv_bm_refcount(const pkv_block_manager* bm, int64_t block, int32_t* count) {
    if (bm == nullptr || count == nullptr) return PKV_ERR_NULL;
    if (block < 0 || block >= bm->num_blocks) return PKV_ERR_SHAPE;
    *count = bm->refcount[(size_t)block];
    return PKV_OK;
}

int pkv_bm_block_table(const pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                       int32_t* table, int max_blocks_per_seq, int32_t* context_lens) {
    if (bm == nullptr) return PKV_ERR_NULL;
    if (num_seqs < 0 || max_blocks_per_seq < 0) return PKV_ERR_SHAPE;
    if (num_seqs == 0) return PKV_OK;
    if (seq_ids == nullptr || table == nullptr || context_lens == nullptr) return PKV_ERR_NULL;
    for (int i = 0; i < num_seqs; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return PKV_ERR_STATE;
        if ((int64_t)it->second.blocks.size() > max_blocks_per_seq ||
            it->second.length > INT32_MAX)
            return PKV_ERR_SHAPE;
    }
    for (int i = 0; i < num_seqs; ++i) {
        const auto& s = bm->seqs.at(seq_ids[i]);
        int32_t* row = table + (size_t)i * max_blocks_per_seq;
        std::fill(row, row + max_blocks_per_seq, -1);
        for (size_t j = 0; j < s.blocks.size(); ++j) row[j] = (int32_t)s.blocks[j];
        context_lens[i] = (int32_t)s.length;
    }
    return PKV_OK;
}

}  // extern "C"
