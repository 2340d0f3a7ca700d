// Block manager: host-side bookkeeping of the paged KV cache ("vLLM" page,
// section "가상 메모리 방식의 해결": fixed-size blocks handed out as tokens
// arrive, a per-sequence table from logical to physical blocks, blocks shared
// between requests of the same prompt and copied only when a branch writes
// into a shared block).
//
// State per manager: a stack of free block numbers, a reference count per
// block, and per sequence its token count and block table.  The first blocks
// handed out are 0, 1, 2, ...; a freed block is reused first.  Everything is
// plain host memory owned by the manager object; nothing touches the GPU.
#include "../../include/tv.h"

#include <cstdint>
#include <new>
#include <vector>

struct tv_block_manager {
    int32_t block_size = 0;
    int32_t max_blocks_per_seq = 0;
    std::vector<int32_t> free_stack;          // top = back()
    std::vector<int32_t> refcount;            // per physical block
    std::vector<int32_t> length;              // per sequence; -1 = not in use
    std::vector<std::vector<int32_t>> table;  // per sequence
};

namespace {

bool valid_seq(const tv_block_manager *bm, int32_t seq)
{
    return bm && seq >= 0 && seq < (int32_t)bm->length.size();
}

bool live_seq(const tv_block_manager *bm, int32_t seq)
{
    return valid_seq(bm, seq) && bm->length[seq] >= 0;
}

int32_t blocks_for(const tv_block_manager *bm, int64_t tokens)
{
    return (int32_t)((tokens + bm->block_size - 1) / bm->block_size);
}

int32_t take_block(tv_block_manager *bm)
{
    const int32_t b = bm->free_stack.back();
    bm->free_stack.pop_back();
    bm->refcount[b] = 1;
    return b;
}

void release_block(tv_block_manager *bm, int32_t b)
{
    if (--bm->refcount[b] == 0)
        bm->free_stack.push_back(b);
}

}  // namespace

extern "C" {

tv_status tv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                       int32_t max_blocks_per_seq, tv_block_manager **out)
{
    if (!out)
        return TV_ERR_NULL;
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0)
        return TV_ERR_SHAPE;
    tv_block_manager *bm = new (std::nothrow) tv_block_manager;
    if (!bm)
        return TV_ERR_NO_BLOCKS;
    try {
        bm->block_size = block_size;
        bm->max_blocks_per_seq = max_blocks_per_seq;
        bm->free_stack.resize(num_blocks);
        for (int32_t i = 0; i < num_blocks; ++i)
            bm->free_stack[i] = num_blocks - 1 - i;          // block 0 on top
        bm->refcount.assign(num_blocks, 0);
        bm->length.assign(max_seqs, -1);
        bm->table.resize(max_seqs);
    } catch (...) {
        delete bm;
        return TV_ERR_NO_BLOCKS;
    }
    *out = bm;
    return TV_OK;
}

void tv_bm_destroy(tv_block_manager *bm)
{
    delete bm;
}

int32_t tv_bm_num_free(const tv_block_manager *bm)
{
    return bm ? (int32_t)bm->free_stack.size() : -1;
}

int32_t tv_bm_refcount(const tv_block_manager *bm, int32_t block)
{
    if (!bm || block < 0 || block >= (int32_t)bm->refcount.size())
        return -1;
    return bm->refcount[block];
}

int32_t tv_bm_length(const tv_block_manager *bm, int32_t seq)
{
    return valid_seq(bm, seq) ? bm->length[seq] : -1;
}

tv_status tv_bm_add_sequence(tv_block_manager *bm, int32_t seq, int32_t num_tokens)
{
    if (!bm)
        return TV_ERR_NULL;
    if (!valid_seq(bm, seq) || bm->length[seq] >= 0 || num_tokens < 0)
        return TV_ERR_SHAPE;
    const int32_t need = blocks_for(bm, num_tokens);
    if (need > bm->max_blocks_per_seq)
        return TV_ERR_SHAPE;
    if (need > (int32_t)bm->free_stack.size())
        return TV_ERR_NO_BLOCKS;
    std::vector<int32_t> &t = bm->table[seq];
    t.clear();
    for (int32_t i = 0; i < need; ++i)
        t.push_back(take_block(bm));
    bm->length[seq] = num_tokens;
    return TV_OK;
}

tv_status tv_bm_fork(tv_block_manager *bm, int32_t parent, int32_t child)
{
    if (!bm)
        return TV_ERR_NULL;
    if (!live_seq(bm, parent) || !valid_seq(bm, child) || bm->length[child] >= 0)
        return TV_ERR_SHAPE;
    bm->table[child] = bm->table[parent];
    for (int32_t b : bm->table[child])
        ++bm->refcount[b];
    bm->length[child] = bm->length[parent];
    return TV_OK;
}

tv_status tv_bm_append_slot(tv_block_manager *bm, int32_t seq, int64_t *slot,
                            int64_t *copy_src, int64_t *copy_dst)
{
    if (!bm || !slot || !copy_src || !copy_dst)
        return TV_ERR_NULL;
    if (!live_seq(bm, seq))
        return TV_ERR_SHAPE;
    std::vector<int32_t> &t = bm->table[seq];
    const int32_t n = bm->length[seq];
    const int32_t off = n % bm->block_size;
    *copy_src = -1;
    *copy_dst = -1;
    if (off == 0) {                               // the position opens a new block
        if ((int32_t)t.size() + 1 > bm->max_blocks_per_seq)
            return TV_ERR_SHAPE;
        if (bm->free_stack.empty())
            return TV_ERR_NO_BLOCKS;
        t.push_back(take_block(bm));
    } else {
        int32_t &last = t[n / bm->block_size];
        if (bm->refcount[last] > 1) {             // shared: copy on write
            if (bm->free_stack.empty())
                return TV_ERR_NO_BLOCKS;
            const int32_t fresh = take_block(bm);
            *copy_src = last;
            *copy_dst = fresh;
            --bm->refcount[last];
            last = fresh;
        }
    }
    *slot = (int64_t)t[n / bm->block_size] * bm->block_size + off;
    bm->length[seq] = n + 1;
    return TV_OK;
}

tv_status tv_bm_free_sequence(tv_block_manager *bm, int32_t seq)
{
    if (!bm)
        return TV_ERR_NULL;
    if (!live_seq(bm, seq))
        return TV_ERR_SHAPE;
    std::vector<int32_t> &t = bm->table[seq];
    for (auto it = t.rbegin(); it != t.rend(); ++it)   // the first block ends on top
        release_block(bm, *it);
    t.clear();
    bm->length[seq] = -1;
    return TV_OK;
}

tv_status tv_bm_block_table(const tv_block_manager *bm, int32_t seq, int32_t *row,
                            int32_t width, int32_t *num_blocks)
{
    if (!bm || !row || !num_blocks)
        return TV_ERR_NULL;
    if (!live_seq(bm, seq))
        return TV_ERR_SHAPE;
    const std::vector<int32_t> &t = bm->table[seq];
    if ((int32_t)t.size() > width)
        return TV_ERR_SHAPE;
    for (size_t i = 0; i < t.size(); ++i)
        row[i] = t[i];
    *num_blocks = (int32_t)t.size();
    return TV_OK;
}

tv_status tv_bm_slots(const tv_block_manager *bm, int32_t seq, int32_t start, int32_t count,
                      int64_t *slots)
{
    if (!bm || (count > 0 && !slots))
        return TV_ERR_NULL;
    if (!live_seq(bm, seq) || start < 0 || count < 0 ||
        (int64_t)start + count > bm->length[seq])
        return TV_ERR_SHAPE;
    const std::vector<int32_t> &t = bm->table[seq];
    for (int32_t i = 0; i < count; ++i) {
        const int32_t pos = start + i;
        slots[i] = (int64_t)t[pos / bm->block_size] * bm->block_size + pos % bm->block_size;
    }
    return TV_OK;
}

}  // extern "C"
