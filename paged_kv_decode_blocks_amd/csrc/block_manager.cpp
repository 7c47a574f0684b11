// block_manager.cpp -- host-side paging lifecycle of the KV pool (C ABI in include/pkv.h).
//
// Physical blocks are handed out when a sequence's next token needs one and
// return to one global free pool when no sequence maps them any more
// ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2, the third
// step).  Blocks may be mapped by several sequences (a shared prompt prefix,
// same page, section 2.3), so each carries a reference count; a sequence that
// is about to write into a partly filled block it shares gets a private copy
// first (copy-on-write), which the caller performs on the device.
//
// Free blocks sit in a binary min-heap keyed by their rank in the allocation
// order, so every allocation and release is O(log n_blocks).  Each call checks
// everything that can fail before it changes anything, so a failed call leaves
// the manager as it was.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"
#include "pkv_host.h"

using pkv::fail;

namespace {

// Output mix of the SplitMix64 generator (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014).
uint64_t splitmix64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

struct Sequence {
    int32_t len = 0;
    std::vector<int32_t> blocks;   // logical block j -> physical block id
};

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

}  // namespace

struct pkv_block_manager {
    int32_t n_blocks;
    int32_t bs;
    std::vector<int32_t> refcount;   // per physical block; 0 = free
    std::vector<int32_t> order;      // order[r] = block handed out r-th when all are free
    std::vector<int32_t> rank;       // inverse of order
    std::vector<int32_t> free_heap;  // ranks of the free blocks, min-heap
    std::unordered_map<int64_t, Sequence> seqs;

    int32_t num_free() const { return (int32_t)free_heap.size(); }

    int32_t alloc() {
        std::pop_heap(free_heap.begin(), free_heap.end(), std::greater<int32_t>());
        const int32_t b = order[free_heap.back()];
        free_heap.pop_back();
        refcount[b] = 1;
        return b;
    }

    void release(int32_t b) {
        if (--refcount[b] == 0) {
            free_heap.push_back(rank[b]);
            std::push_heap(free_heap.begin(), free_heap.end(), std::greater<int32_t>());
        }
    }

    // Does appending one token to s need a fresh block (a new block, or a copy)?
    bool append_needs_block(const Sequence& s, int32_t shared_refs) const {
        if (s.len % bs == 0) return true;
        return shared_refs > 1;
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t n_blocks, int32_t block_size, uint64_t shuffle_seed) {
    if (n_blocks <= 0 || block_size <= 0) {
        fail(PKV_ERR_INVALID_ARG, "n_blocks = %d and block_size = %d must be positive", n_blocks, block_size);
        return nullptr;
    }
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
    if (!bm) {
        fail(PKV_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    bm->n_blocks = n_blocks;
    bm->bs = block_size;
    bm->refcount.assign(n_blocks, 0);
    bm->order.resize(n_blocks);
    for (int32_t i = 0; i < n_blocks; ++i) bm->order[i] = i;
    if (shuffle_seed != 0) {
        std::vector<uint64_t> key(n_blocks);
        for (int32_t i = 0; i < n_blocks; ++i)
            key[i] = splitmix64_mix(shuffle_seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull);
        std::sort(bm->order.begin(), bm->order.end(),
                  [&](int32_t a, int32_t b) { return key[a] != key[b] ? key[a] < key[b] : a < b; });
    }
    bm->rank.resize(n_blocks);
    for (int32_t r = 0; r < n_blocks; ++r) bm->rank[bm->order[r]] = r;
    bm->free_heap.resize(n_blocks);
    for (int32_t r = 0; r < n_blocks; ++r) bm->free_heap[r] = r;   // ascending = already a min-heap
    pkv::clear_error();
    return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens = %d is negative", num_tokens);
    if (bm->seqs.count(seq_id)) return fail(PKV_ERR_SEQUENCE, "sequence %lld already exists", (long long)seq_id);
    const int32_t need = ceil_div(num_tokens, bm->bs);
    if (need > bm->num_free())
        return fail(PKV_ERR_OUT_OF_BLOCKS, "sequence %lld needs %d blocks, %d free", (long long)seq_id, need,
                    bm->num_free());
    Sequence s;
    s.len = num_tokens;
    s.blocks.reserve(need);
    for (int32_t j = 0; j < need; ++j) s.blocks.push_back(bm->alloc());
    bm->seqs.emplace(seq_id, std::move(s));
    pkv::clear_error();
    return PKV_OK;
}

int pkv_bm_add_sequence_shared(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens, int64_t prefix_id,
                               int32_t prefix_tokens, int32_t* shared_tokens) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    auto it = bm->seqs.find(prefix_id);
    if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "prefix sequence %lld does not exist", (long long)prefix_id);
    if (bm->seqs.count(seq_id)) return fail(PKV_ERR_SEQUENCE, "sequence %lld already exists", (long long)seq_id);
    const Sequence& pre = it->second;
    if (prefix_tokens < 0 || prefix_tokens > num_tokens || prefix_tokens > pre.len)
        return fail(PKV_ERR_INVALID_ARG, "prefix_tokens = %d must lie in [0, min(num_tokens = %d, prefix length = %d)]",
                    prefix_tokens, num_tokens, pre.len);
    const int32_t k = prefix_tokens / bm->bs;
    const int32_t need = ceil_div(num_tokens, bm->bs) - k;
    if (need > bm->num_free())
        return fail(PKV_ERR_OUT_OF_BLOCKS, "sequence %lld needs %d blocks, %d free", (long long)seq_id, need,
                    bm->num_free());
    Sequence s;
    s.len = num_tokens;
    s.blocks.reserve(k + need);
    for (int32_t j = 0; j < k; ++j) {
        s.blocks.push_back(pre.blocks[j]);
        ++bm->refcount[pre.blocks[j]];
    }
    for (int32_t j = 0; j < need; ++j) s.blocks.push_back(bm->alloc());
    bm->seqs.emplace(seq_id, std::move(s));
    if (shared_tokens) *shared_tokens = k * bm->bs;
    pkv::clear_error();
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    auto it = bm->seqs.find(parent_id);
    if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "sequence %lld does not exist", (long long)parent_id);
    if (bm->seqs.count(child_id)) return fail(PKV_ERR_SEQUENCE, "sequence %lld already exists", (long long)child_id);
    Sequence c = it->second;
    for (int32_t b : c.blocks) ++bm->refcount[b];
    bm->seqs.emplace(child_id, std::move(c));
    pkv::clear_error();
    return PKV_OK;
}

int pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t* position, int32_t* cow_src,
                        int32_t* cow_dst) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "sequence %lld does not exist", (long long)seq_id);
    Sequence& s = it->second;
    if (s.len == INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "sequence %lld is at the int32 length limit", (long long)seq_id);
    const int32_t last_refs = s.len % bm->bs ? bm->refcount[s.blocks.back()] : 0;
    if (bm->append_needs_block(s, last_refs) && bm->num_free() == 0)
        return fail(PKV_ERR_OUT_OF_BLOCKS, "sequence %lld needs a block, none free", (long long)seq_id);
    int32_t src = -1, dst = -1;
    if (s.len % bm->bs == 0) {
        s.blocks.push_back(bm->alloc());
    } else if (last_refs > 1) {
        src = s.blocks.back();
        dst = bm->alloc();
        s.blocks.back() = dst;
        bm->release(src);
    }
    if (position) *position = s.len;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
    ++s.len;
    pkv::clear_error();
    return PKV_OK;
}

int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int32_t B, int32_t* tables,
                        int32_t bt_stride, int32_t* positions, int32_t* cow_src, int32_t* cow_dst,
                        int32_t* n_cow) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B = %d is negative", B);
    if (n_cow) *n_cow = 0;
    if (B == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!seq_ids || !tables || !positions) return fail(PKV_ERR_NULL, "seq_ids, tables and positions must not be NULL");
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride = %d must be positive", bt_stride);
    // Dry run: every id known and distinct, tables fit, and enough free blocks
    // for the whole batch.  Copy-on-write of a block two batch members share
    // frees the later one from copying, so shared counts are tracked as we go.
    std::vector<Sequence*> seq(B);
    std::unordered_set<int64_t> seen;
    seen.reserve(B * 2);
    std::unordered_map<int32_t, int32_t> refs;   // block -> reference count after earlier batch members
    int32_t need = 0, copies = 0;
    for (int32_t b = 0; b < B; ++b) {
        auto it = bm->seqs.find(seq_ids[b]);
        if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "sequence %lld does not exist", (long long)seq_ids[b]);
        if (!seen.insert(seq_ids[b]).second)
            return fail(PKV_ERR_INVALID_ARG, "sequence %lld appears twice in the batch", (long long)seq_ids[b]);
        Sequence& s = it->second;
        seq[b] = &s;
        if (s.len == INT32_MAX)
            return fail(PKV_ERR_INVALID_ARG, "sequence %lld is at the int32 length limit", (long long)seq_ids[b]);
        if (ceil_div(s.len + 1, bm->bs) > bt_stride)
            return fail(PKV_ERR_INVALID_ARG, "sequence %lld needs %d table entries, bt_stride = %d",
                        (long long)seq_ids[b], ceil_div(s.len + 1, bm->bs), bt_stride);
        if (s.len % bm->bs == 0) {
            ++need;
        } else {
            const int32_t last = s.blocks.back();
            auto r = refs.find(last);
            const int32_t cnt = r == refs.end() ? bm->refcount[last] : r->second;
            if (cnt > 1) {
                ++need;
                ++copies;
                refs[last] = cnt - 1;
            }
        }
    }
    if (copies && (!cow_src || !cow_dst))
        return fail(PKV_ERR_INVALID_ARG, "the batch needs %d block copies but cow_src/cow_dst are NULL", copies);
    if (need > bm->num_free())
        return fail(PKV_ERR_OUT_OF_BLOCKS, "the batch needs %d blocks, %d free", need, bm->num_free());
    int32_t nc = 0;
    for (int32_t b = 0; b < B; ++b) {
        Sequence& s = *seq[b];
        if (s.len % bm->bs == 0) {
            s.blocks.push_back(bm->alloc());
        } else if (bm->refcount[s.blocks.back()] > 1) {
            const int32_t src = s.blocks.back();
            const int32_t dst = bm->alloc();
            s.blocks.back() = dst;
            bm->release(src);
            cow_src[nc] = src;
            cow_dst[nc] = dst;
            ++nc;
        }
        positions[b] = s.len++;
        int32_t* row = tables + (int64_t)b * bt_stride;
        const int32_t nb = (int32_t)s.blocks.size();
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        std::fill(row + nb, row + bt_stride, -1);
    }
    if (n_cow) *n_cow = nc;
    pkv::clear_error();
    return PKV_OK;
}

int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "sequence %lld does not exist", (long long)seq_id);
    for (int32_t b : it->second.blocks) bm->release(b);
    bm->seqs.erase(it);
    pkv::clear_error();
    return PKV_OK;
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? bm->num_free() : -1; }

int32_t pkv_bm_num_sequences(const pkv_block_manager* bm) { return bm ? (int32_t)bm->seqs.size() : -1; }

int32_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_block_refcount(const pkv_block_manager* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->n_blocks) return -1;
    return bm->refcount[block];
}

int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table, int32_t capacity,
                       int32_t* n_blocks) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    if (capacity < 0) return fail(PKV_ERR_INVALID_ARG, "capacity = %d is negative", capacity);
    if (capacity > 0 && !table) return fail(PKV_ERR_NULL, "table is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "sequence %lld does not exist", (long long)seq_id);
    const std::vector<int32_t>& blk = it->second.blocks;
    const int32_t n = (int32_t)blk.size();
    std::copy(blk.begin(), blk.begin() + std::min(n, capacity), table);
    if (n_blocks) *n_blocks = n;
    pkv::clear_error();
    return PKV_OK;
}

int pkv_bm_batch_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t B, int32_t* tables,
                        int32_t bt_stride, int32_t* context_lens) {
    if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B = %d is negative", B);
    if (B == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!seq_ids || !tables || !context_lens) return fail(PKV_ERR_NULL, "seq_ids, tables and context_lens must not be NULL");
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride = %d must be positive", bt_stride);
    std::vector<const Sequence*> seq(B);
    for (int32_t b = 0; b < B; ++b) {
        auto it = bm->seqs.find(seq_ids[b]);
        if (it == bm->seqs.end()) return fail(PKV_ERR_SEQUENCE, "sequence %lld does not exist", (long long)seq_ids[b]);
        if ((int32_t)it->second.blocks.size() > bt_stride)
            return fail(PKV_ERR_INVALID_ARG, "sequence %lld has %zu blocks, bt_stride = %d", (long long)seq_ids[b],
                        it->second.blocks.size(), bt_stride);
        seq[b] = &it->second;
    }
    for (int32_t b = 0; b < B; ++b) {
        int32_t* row = tables + (int64_t)b * bt_stride;
        const int32_t nb = (int32_t)seq[b]->blocks.size();
        std::copy(seq[b]->blocks.begin(), seq[b]->blocks.end(), row);
        std::fill(row + nb, row + bt_stride, -1);
        context_lens[b] = seq[b]->len;
    }
    pkv::clear_error();
    return PKV_OK;
}

}  // extern "C"
