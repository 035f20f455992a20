// block_manager.cpp -- host-side bookkeeping of refcounted KV blocks with
// copy-on-write (declared in include/paged_gqa.h, pgqa_bm_*).
//
// What it follows: a sequence's KV cache is a list of fixed-size blocks taken
// from a pool only when a token needs one and given back when the request ends
// ("The Ultimate Guide to LLM Inference Optimization- Part 2", section "Paged
// Attention"); blocks carry a reference counter so that sequences can point at
// the same prefix blocks, and when they diverge only the block being modified
// is copied ("Modern LLM Inference", section 8.2, "Prefix Sharing
// (Copy-on-Write)").
//
// Policy (the pages leave it open): new blocks are the lowest-numbered free
// ones, new sequences get the lowest unused id, a fork shares the parent's whole
// table, and an append copies the last block first exactly when that block is
// partly filled (so the append writes into it) and shared.  Full blocks are
// never written again, so they stay shared.  An append that cannot get all the
// blocks it needs fails with PGQA_ENOSPC and changes nothing.
//
// Costs: every operation is O(pages touched + log(pool)); the free list is an
// ordered set.  Not thread-safe: one caller at a time per manager.
#include "paged_gqa.h"

#include <stdint.h>

#include <map>
#include <new>
#include <set>
#include <vector>

struct pgqa_block_manager {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> ref;
    std::set<int32_t> free_blocks;
    struct Seq {
        std::vector<int32_t> table;
        int64_t length = 0;
    };
    std::map<int32_t, Seq> seqs;

    int32_t lowest_free_id() const {
        int32_t id = 0;
        for (const auto& kv : seqs) {   // ordered by id
            if (kv.first != id) break;
            ++id;
        }
        return id;
    }
    int32_t take_block() {
        const int32_t b = *free_blocks.begin();
        free_blocks.erase(free_blocks.begin());
        ref[b] = 1;
        return b;
    }
    void drop_ref(int32_t b) {
        if (--ref[b] == 0) free_blocks.insert(b);
    }
};

namespace {

int64_t pages_for(int64_t length, int32_t bs) { return (length + bs - 1) / bs; }

}  // namespace

extern "C" {

pgqa_block_manager* pgqa_bm_create(int32_t num_blocks, int32_t block_size) {
    if (num_blocks <= 0 || block_size <= 0) return nullptr;
    pgqa_block_manager* bm = new (std::nothrow) pgqa_block_manager;
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->ref.assign((size_t)num_blocks, 0);
        for (int32_t b = 0; b < num_blocks; ++b) bm->free_blocks.insert(bm->free_blocks.end(), b);
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pgqa_bm_destroy(pgqa_block_manager* bm) { delete bm; }

int pgqa_bm_new_sequence(pgqa_block_manager* bm, int32_t* seq) {
    if (!bm || !seq) return PGQA_EINVAL;
    try {
        const int32_t id = bm->lowest_free_id();
        bm->seqs[id];
        *seq = id;
    } catch (...) {
        return PGQA_ENOSPC;
    }
    return PGQA_OK;
}

int pgqa_bm_fork(pgqa_block_manager* bm, int32_t parent, int32_t* child) {
    if (!bm || !child) return PGQA_EINVAL;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end()) return PGQA_EINVAL;
    try {
        const int32_t id = bm->lowest_free_id();
        pgqa_block_manager::Seq s = it->second;   // copy before inserting (may rebalance)
        bm->seqs[id] = std::move(s);
        for (int32_t b : bm->seqs[id].table) ++bm->ref[b];
        *child = id;
    } catch (...) {
        return PGQA_ENOSPC;
    }
    return PGQA_OK;
}

int pgqa_bm_append(pgqa_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* copy_src,
                   int32_t* copy_dst) {
    if (!bm || !copy_src || !copy_dst || num_tokens < 0) return PGQA_EINVAL;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PGQA_EINVAL;
    pgqa_block_manager::Seq& s = it->second;
    *copy_src = -1;
    *copy_dst = -1;
    if (num_tokens == 0) return PGQA_OK;
    if (s.length + num_tokens > INT32_MAX) return PGQA_EINVAL;
    const bool cow = (s.length % bm->block_size) != 0 && bm->ref[s.table.back()] > 1;
    const int64_t fresh = pages_for(s.length + num_tokens, bm->block_size) - (int64_t)s.table.size();
    if ((int64_t)bm->free_blocks.size() < fresh + (cow ? 1 : 0)) return PGQA_ENOSPC;
    try {
        s.table.reserve((size_t)(s.table.size() + fresh));
    } catch (...) {
        return PGQA_ENOSPC;
    }
    if (cow) {
        const int32_t old = s.table.back();
        const int32_t nb = bm->take_block();
        bm->drop_ref(old);
        s.table.back() = nb;
        *copy_src = old;
        *copy_dst = nb;
    }
    for (int64_t i = 0; i < fresh; ++i) s.table.push_back(bm->take_block());
    s.length += num_tokens;
    return PGQA_OK;
}

int pgqa_bm_free_sequence(pgqa_block_manager* bm, int32_t seq) {
    if (!bm) return PGQA_EINVAL;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PGQA_EINVAL;
    for (int32_t b : it->second.table) bm->drop_ref(b);
    bm->seqs.erase(it);
    return PGQA_OK;
}

int32_t pgqa_bm_sequence_length(const pgqa_block_manager* bm, int32_t seq) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? -1 : (int32_t)it->second.length;
}

int32_t pgqa_bm_block_table(const pgqa_block_manager* bm, int32_t seq, int32_t* pages, int32_t capacity) {
    if (!bm || capacity < 0 || (capacity > 0 && !pages)) return -1;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return -1;
    const std::vector<int32_t>& t = it->second.table;
    for (int32_t i = 0; i < capacity && i < (int32_t)t.size(); ++i) pages[i] = t[(size_t)i];
    return (int32_t)t.size();
}

int32_t pgqa_bm_refcount(const pgqa_block_manager* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->ref[(size_t)block];
}

int32_t pgqa_bm_num_free_blocks(const pgqa_block_manager* bm) {
    return bm ? (int32_t)bm->free_blocks.size() : -1;
}

}  // extern "C"
