// Host-side block manager for the paged KV cache (declared in
// include/pkv_block_manager.h): on-demand block allocation from a free
// stack, per-block reference counts for shared blocks, copy-on-write of a
// shared, partly filled last block when a sequence appends to it, and
// swapping of whole sequences to a pool of host blocks and back.

#include "pkv_block_manager.h"

#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

struct pkv_block_manager {
    int num_blocks;
    int num_host_blocks;
    int block_size;
    std::vector<int32_t> free_stack;          // top = back()
    std::vector<int32_t> refcount;            // per physical block
    std::vector<int32_t> host_free;           // the same for the host pool
    std::vector<int32_t> host_refcount;
    struct Seq {
        std::vector<int32_t> table;           // logical -> physical (host blocks if swapped)
        int len = 0;
        bool swapped = false;
    };
    std::unordered_map<int64_t, Seq> seqs;
    std::vector<std::pair<int32_t, int32_t>> copies;   // queued (src, dst)
};

namespace {

int32_t pop_free(pkv_block_manager* bm) {
    const int32_t b = bm->free_stack.back();
    bm->free_stack.pop_back();
    bm->refcount[b] = 1;
    return b;
}

void release(pkv_block_manager* bm, int32_t b) {
    if (--bm->refcount[b] == 0) bm->free_stack.push_back(b);
}

// Give every distinct block held by the sequences ids[0..n) a block of the
// other pool (device -> host if to_host, else host -> device), in order of
// first use, and move the sequences' references there; the blocks of the
// pool they leave are released as by pkv_bm_free_sequence. Writes the
// (old, new) pairs and returns their number; all or nothing.
int move_sequences(pkv_block_manager* bm, const int64_t* ids, int n, int32_t* pairs,
                   int max_pairs, bool to_host) {
    if (!bm || n < 0 || max_pairs < 0) return PKV_ERR_INVALID;
    if (n == 0) return 0;
    if (!ids || !bm->copies.empty()) return PKV_ERR_INVALID;
    std::vector<pkv_block_manager::Seq*> seqs;
    std::unordered_map<int32_t, int32_t> where;
    std::vector<int32_t> order;
    try {
        std::unordered_map<int64_t, int> seen;
        for (int i = 0; i < n; ++i) {
            auto it = bm->seqs.find(ids[i]);
            if (it == bm->seqs.end() || seen[ids[i]]++ || it->second.swapped == to_host)
                return PKV_ERR_INVALID;
            seqs.push_back(&it->second);
        }
        for (auto* s : seqs)
            for (int32_t b : s->table)
                if (where.emplace(b, -1).second) order.push_back(b);
    } catch (...) {
        return PKV_ERR_INVALID;
    }
    std::vector<int32_t>& src_ref = to_host ? bm->refcount : bm->host_refcount;
    std::vector<int32_t>& src_free = to_host ? bm->free_stack : bm->host_free;
    std::vector<int32_t>& dst_ref = to_host ? bm->host_refcount : bm->refcount;
    std::vector<int32_t>& dst_free = to_host ? bm->host_free : bm->free_stack;
    if (order.size() > dst_free.size()) return PKV_ERR_NO_BLOCKS;
    if ((int)order.size() > max_pairs) return PKV_ERR_WORKSPACE;
    if (!order.empty() && !pairs) return PKV_ERR_INVALID;
    // From here on nothing allocates: the free stacks have their full
    // capacity reserved.
    for (size_t k = 0; k < order.size(); ++k) {
        const int32_t fresh = dst_free.back();
        dst_free.pop_back();
        dst_ref[fresh] = 0;
        where[order[k]] = fresh;
        pairs[2 * k] = order[k];
        pairs[2 * k + 1] = fresh;
    }
    for (auto* s : seqs) {
        for (int32_t& b : s->table) {
            const int32_t fresh = where[b];
            ++dst_ref[fresh];
            if (--src_ref[b] == 0) src_free.push_back(b);
            b = fresh;
        }
        s->swapped = to_host;
    }
    return (int)order.size();
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create_swappable(int num_blocks, int num_host_blocks, int block_size) {
    if (num_blocks <= 0 || num_host_blocks < 0 || block_size <= 0) return nullptr;
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->num_host_blocks = num_host_blocks;
        bm->block_size = block_size;
        bm->free_stack.reserve(num_blocks);
        for (int b = num_blocks - 1; b >= 0; --b) bm->free_stack.push_back(b);
        bm->refcount.assign(num_blocks, 0);
        bm->host_free.reserve(num_host_blocks);
        for (int b = num_host_blocks - 1; b >= 0; --b) bm->host_free.push_back(b);
        bm->host_refcount.assign(num_host_blocks, 0);
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

pkv_block_manager* pkv_bm_create(int num_blocks, int block_size) {
    return pkv_bm_create_swappable(num_blocks, 0, block_size);
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm || bm->seqs.count(seq_id)) return PKV_ERR_INVALID;
    try {
        bm->seqs.emplace(seq_id, pkv_block_manager::Seq{});
    } catch (...) {
        return PKV_ERR_INVALID;
    }
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm || parent == child || bm->seqs.count(child)) return PKV_ERR_INVALID;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || it->second.swapped) return PKV_ERR_INVALID;
    try {
        pkv_block_manager::Seq s = it->second;
        bm->seqs.emplace(child, std::move(s));
    } catch (...) {
        return PKV_ERR_INVALID;
    }
    for (int32_t b : bm->seqs[child].table) ++bm->refcount[b];
    return PKV_OK;
}

int pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t* block, int32_t* offset) {
    if (!bm) return PKV_ERR_INVALID;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end() || it->second.swapped) return PKV_ERR_INVALID;
    pkv_block_manager::Seq& s = it->second;
    const int slot = s.len % bm->block_size;
    if (slot == 0) {
        // the last block is full (or there is none): a fresh block
        if (bm->free_stack.empty()) return PKV_ERR_NO_BLOCKS;
        s.table.push_back(pop_free(bm));
    } else {
        const int32_t last = s.table.back();
        if (bm->refcount[last] > 1) {
            // shared and partly filled: this sequence gets its own copy
            if (bm->free_stack.empty()) return PKV_ERR_NO_BLOCKS;
            const int32_t fresh = pop_free(bm);
            bm->copies.emplace_back(last, fresh);
            --bm->refcount[last];
            s.table.back() = fresh;
        }
    }
    ++s.len;
    if (block) *block = s.table.back();
    if (offset) *offset = slot;
    return PKV_OK;
}

int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int n, int32_t* blocks,
                        int32_t* offsets) {
    if (!bm || n < 0) return PKV_ERR_INVALID;
    if (n == 0) return PKV_OK;
    if (!seq_ids) return PKV_ERR_INVALID;
    // Dry run: the blocks the step needs, replaying the reference counts of
    // shared last blocks in order (the last holder of a shared block writes
    // in place, so only the holders before it need a copy).
    std::unordered_map<int32_t, int32_t> ref;
    std::unordered_map<int64_t, int> seen;
    size_t need = 0;
    for (int i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end() || it->second.swapped || seen[seq_ids[i]]++)
            return PKV_ERR_INVALID;
        const pkv_block_manager::Seq& s = it->second;
        if (s.len % bm->block_size == 0) {
            ++need;
        } else {
            const int32_t last = s.table.back();
            auto r = ref.find(last);
            int32_t& cnt = r == ref.end() ? (ref[last] = bm->refcount[last]) : r->second;
            if (cnt > 1) {
                ++need;
                --cnt;
            }
        }
    }
    if (need > bm->free_stack.size()) return PKV_ERR_NO_BLOCKS;
    for (int i = 0; i < n; ++i) {
        int32_t b, o;
        pkv_bm_append_token(bm, seq_ids[i], &b, &o);
        if (blocks) blocks[i] = b;
        if (offsets) offsets[i] = o;
    }
    return PKV_OK;
}

int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_INVALID;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_INVALID;
    // A queued copy's destination or source could return to the free stack
    // here and be handed out again before the copy runs: as a second copy's
    // destination (two pairs writing one block) or as a destination while
    // still a source (pairs of one copy_blocks call run concurrently).
    if (!bm->copies.empty()) return PKV_ERR_INVALID;
    if (it->second.swapped) {
        for (int32_t b : it->second.table)
            if (--bm->host_refcount[b] == 0) bm->host_free.push_back(b);
    } else {
        for (int32_t b : it->second.table) release(bm, b);
    }
    bm->seqs.erase(it);
    return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* bm, const int64_t* seq_ids, int n, int32_t* pairs,
                    int max_pairs) {
    return move_sequences(bm, seq_ids, n, pairs, max_pairs, true);
}

int pkv_bm_swap_in(pkv_block_manager* bm, const int64_t* seq_ids, int n, int32_t* pairs,
                   int max_pairs) {
    return move_sequences(bm, seq_ids, n, pairs, max_pairs, false);
}

int pkv_bm_is_swapped(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_INVALID;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? PKV_ERR_INVALID : (it->second.swapped ? 1 : 0);
}

int pkv_bm_num_free_host_blocks(const pkv_block_manager* bm) {
    return bm ? (int)bm->host_free.size() : PKV_ERR_INVALID;
}

int pkv_bm_host_refcount(const pkv_block_manager* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->num_host_blocks) return PKV_ERR_INVALID;
    return bm->host_refcount[block];
}

int pkv_bm_num_free_blocks(const pkv_block_manager* bm) {
    return bm ? (int)bm->free_stack.size() : PKV_ERR_INVALID;
}

int pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_INVALID;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? PKV_ERR_INVALID : it->second.len;
}

int pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return PKV_ERR_INVALID;
    return bm->refcount[block];
}

int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                       int max_blocks) {
    if (!bm) return PKV_ERR_INVALID;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_INVALID;
    const std::vector<int32_t>& t = it->second.table;
    if ((int)t.size() > max_blocks) return PKV_ERR_WORKSPACE;
    if (!t.empty() && !out) return PKV_ERR_INVALID;
    for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
    return (int)t.size();
}

int pkv_bm_take_copies(pkv_block_manager* bm, int32_t* pairs, int max_pairs) {
    if (!bm || max_pairs < 0 || (max_pairs > 0 && !pairs)) return PKV_ERR_INVALID;
    const int n = (int)bm->copies.size() < max_pairs ? (int)bm->copies.size() : max_pairs;
    for (int i = 0; i < n; ++i) {
        pairs[2 * i] = bm->copies[i].first;
        pairs[2 * i + 1] = bm->copies[i].second;
    }
    bm->copies.erase(bm->copies.begin(), bm->copies.begin() + n);
    return n;
}

int pkv_bm_shared_prefix(const pkv_block_manager* bm, const int64_t* seq_ids, int n,
                         int group_size, int32_t* shared_tokens) {
    if (!bm || n < 0 || group_size <= 0 || n % group_size != 0) return PKV_ERR_INVALID;
    if (n == 0) return PKV_OK;
    if (!seq_ids || !shared_tokens) return PKV_ERR_INVALID;
    std::vector<const pkv_block_manager::Seq*> seqs;
    try {
        seqs.reserve(n);
    } catch (...) {
        return PKV_ERR_INVALID;
    }
    for (int i = 0; i < n; ++i) {             // validate everything before writing
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end() || it->second.swapped) return PKV_ERR_INVALID;
        seqs.push_back(&it->second);
    }
    for (int k = 0; k < n / group_size; ++k) {
        const pkv_block_manager::Seq* first = seqs[(size_t)k * group_size];
        size_t blocks = first->table.size();
        for (int j = 1; j < group_size; ++j) {
            const std::vector<int32_t>& t = seqs[(size_t)k * group_size + j]->table;
            size_t b = 0;
            while (b < blocks && b < t.size() && t[b] == first->table[b]) ++b;
            blocks = b;
        }
        shared_tokens[k] = (int32_t)(blocks * (size_t)bm->block_size);
    }
    return PKV_OK;
}

int pkv_bm_build_batch(const pkv_block_manager* bm, const int64_t* seq_ids, int n,
                       int32_t* tables, int max_blocks, int32_t* seq_lens) {
    if (!bm || n < 0 || max_blocks <= 0) return PKV_ERR_INVALID;
    if (n == 0) return PKV_OK;
    if (!seq_ids || !tables || !seq_lens) return PKV_ERR_INVALID;
    for (int i = 0; i < n; ++i) {            // validate everything before writing
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end() || it->second.swapped) return PKV_ERR_INVALID;
        if ((int)it->second.table.size() > max_blocks) return PKV_ERR_WORKSPACE;
    }
    for (int i = 0; i < n; ++i) {
        const pkv_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
        int32_t* row = tables + (size_t)i * max_blocks;
        for (int j = 0; j < max_blocks; ++j) row[j] = j < (int)s.table.size() ? s.table[j] : -1;
        seq_lens[i] = s.len;
    }
    return PKV_OK;
}

}  // extern "C"
