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

#include <algorithm>
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
    std::vector<uint8_t> seen;                // prepare_decode scratch, per sequence
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

// One reserved position, with what it did to the books so that it can be
// taken back.
struct Append {
    enum Kind { kInPlace, kNewBlock, kCopy } kind = kInPlace;
    int32_t seq = -1;
    int32_t index = 0;        // table index of the block holding the position
    int32_t old_block = -1;   // kCopy: the shared block it replaced
    int32_t new_block = -1;   // kNewBlock / kCopy: the block taken from the free list
    int64_t slot = -1;
};

// Reserve position n = length[seq] of a live sequence (see tv_bm_append_slot).
// On TV_ERR_SHAPE / TV_ERR_NO_BLOCKS nothing has changed.
tv_status append(tv_block_manager *bm, int32_t seq, Append *out)
{
    std::vector<int32_t> &t = bm->table[seq];
    const int32_t n = bm->length[seq];
    const int32_t off = n % bm->block_size;
    Append a;
    a.seq = seq;
    a.index = n / bm->block_size;
    if (off == 0) {                               // the position opens a new block
        if ((int32_t)t.size() + 1 > bm->max_blocks_per_seq)
            return TV_ERR_SHAPE;
        if (bm->free_stack.empty())
            return TV_ERR_NO_BLOCKS;
        try {
            t.reserve(t.size() + 1);
        } catch (...) {
            return TV_ERR_NO_BLOCKS;
        }
        a.kind = Append::kNewBlock;
        a.new_block = take_block(bm);
        t.push_back(a.new_block);
    } else if (bm->refcount[t[a.index]] > 1) {    // shared: copy on write
        if (bm->free_stack.empty())
            return TV_ERR_NO_BLOCKS;
        a.kind = Append::kCopy;
        a.old_block = t[a.index];
        a.new_block = take_block(bm);
        --bm->refcount[a.old_block];
        t[a.index] = a.new_block;
    }
    a.slot = (int64_t)t[a.index] * bm->block_size + off;
    bm->length[seq] = n + 1;
    *out = a;
    return TV_OK;
}

// Take back the most recent append still standing.  Undoing appends in the
// reverse of their order restores the free list's order too.
void undo(tv_block_manager *bm, const Append &a)
{
    std::vector<int32_t> &t = bm->table[a.seq];
    --bm->length[a.seq];
    if (a.kind == Append::kNewBlock) {
        t.pop_back();
        release_block(bm, a.new_block);
    } else if (a.kind == Append::kCopy) {
        t[a.index] = a.old_block;
        ++bm->refcount[a.old_block];
        release_block(bm, a.new_block);
    }
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
        bm->seen.assign(max_seqs, 0);
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
    try {
        t.reserve((size_t)need);
    } catch (...) {
        return TV_ERR_NO_BLOCKS;
    }
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
    try {
        bm->table[child] = bm->table[parent];
    } catch (...) {
        return TV_ERR_NO_BLOCKS;
    }
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
    Append r;
    const tv_status st = append(bm, seq, &r);
    if (st != TV_OK)
        return st;
    *slot = r.slot;
    *copy_src = r.kind == Append::kCopy ? r.old_block : -1;
    *copy_dst = r.kind == Append::kCopy ? r.new_block : -1;
    return TV_OK;
}

tv_status tv_bm_prepare_decode(tv_block_manager *bm, const int32_t *seqs, int32_t num_seqs,
                               int32_t width, int32_t *block_tables, int32_t *context_lens,
                               int64_t *slot_mapping, int64_t *copy_pairs, int32_t *num_copies)
{
    if (!bm || !num_copies)
        return TV_ERR_NULL;
    if (num_seqs < 0 || width < 0)
        return TV_ERR_SHAPE;
    if (num_seqs > 0 && (!seqs || !block_tables || !context_lens || !slot_mapping || !copy_pairs))
        return TV_ERR_NULL;
    // Every check that does not depend on the free list comes first, so that
    // only a shortage of blocks can stop the loop below.
    std::vector<Append> done;
    try {
        done.reserve((size_t)num_seqs);
    } catch (...) {
        return TV_ERR_NO_BLOCKS;
    }
    std::vector<uint8_t> &seen = bm->seen;    // all zero between calls
    tv_status bad = TV_OK;
    int32_t checked = 0;
    for (; checked < num_seqs; ++checked) {
        const int32_t seq = seqs[checked];
        if (!live_seq(bm, seq) || seen[seq]) {
            bad = TV_ERR_SHAPE;
            break;
        }
        seen[seq] = 1;
        const int32_t need = blocks_for(bm, (int64_t)bm->length[seq] + 1);
        if (need > width || need > bm->max_blocks_per_seq) {
            ++checked;
            bad = TV_ERR_SHAPE;
            break;
        }
    }
    for (int32_t r = 0; r < checked; ++r)
        seen[seqs[r]] = 0;
    if (bad != TV_OK)
        return bad;
    for (int32_t r = 0; r < num_seqs; ++r) {
        Append a;
        const tv_status st = append(bm, seqs[r], &a);
        if (st != TV_OK) {
            for (auto it = done.rbegin(); it != done.rend(); ++it)
                undo(bm, *it);
            return st;
        }
        done.push_back(a);
    }
    int32_t copies = 0;
    for (int32_t r = 0; r < num_seqs; ++r) {
        const int32_t seq = seqs[r];
        const std::vector<int32_t> &t = bm->table[seq];
        int32_t *row = block_tables + (int64_t)r * width;
        std::copy(t.begin(), t.end(), row);
        std::fill(row + t.size(), row + width, 0);
        context_lens[r] = bm->length[seq];
        slot_mapping[r] = done[r].slot;
        if (done[r].kind == Append::kCopy) {
            copy_pairs[2 * copies] = done[r].old_block;
            copy_pairs[2 * copies + 1] = done[r].new_block;
            ++copies;
        }
    }
    *num_copies = copies;
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
