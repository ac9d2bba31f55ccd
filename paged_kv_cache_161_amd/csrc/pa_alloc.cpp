// pa_alloc.cpp -- host block allocator: free pool, reference counts, copy-on-write and
// rollback bookkeeping for paged KV blocks.
//
// The free pool is first-in first-out: acquire takes from the front, release appends to
// the back, and a request the pool cannot fill takes nothing (LLM-101-CN "推理优化",
// section "物理块与逻辑块", PageAllocator).  Blocks carry reference counts so sequences
// can share them (a beam-search prefix); a shared block that a sequence is about to
// write is replaced by a private copy first (same page, section "Copy-on-Write 优化").
// Every entry point validates all of its input before changing anything, so a failed
// call leaves the allocator and the caller's arrays as they were.
#include <limits.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "../../include/paged_attention.h"

struct pa_block_allocator {
    std::vector<int32_t> ring;    // free block ids, circular: [head, head + nfree)
    std::vector<int32_t> ref;     // reference count per block, 0 = free
    int32_t head = 0;
    int32_t nfree = 0;

    int32_t n() const { return (int32_t)ref.size(); }
    bool valid(int32_t b) const { return b >= 0 && b < n(); }
    int32_t take()
    {
        const int32_t b = ring[head];
        head = (head + 1) % n();
        --nfree;
        ref[b] = 1;
        return b;
    }
    void give_back(int32_t b)
    {
        ring[(head + nfree) % n()] = b;
        ++nfree;
    }
    void unref(int32_t b)
    {
        if (--ref[b] == 0)
            give_back(b);
    }
};

namespace {

constexpr int32_t kBlock = PA_BLOCK_SIZE;

int32_t blocks_for(int64_t tokens) { return (int32_t)((tokens + kBlock - 1) / kBlock); }

// The first `used` entries of a row must be blocks in use.
bool row_ok(const pa_block_allocator *a, const int32_t *row, int32_t used)
{
    for (int32_t i = 0; i < used; ++i)
        if (!a->valid(row[i]) || a->ref[row[i]] <= 0)
            return false;
    return true;
}

// Each listed block holds at least as many references as times it is listed, so
// dropping one reference per listing never goes below zero.
bool refs_cover(const pa_block_allocator *a, const int32_t *ids, int32_t count)
{
    std::vector<int32_t> need;
    try {
        need.assign(a->n(), 0);
    } catch (...) {
        return false;
    }
    for (int32_t i = 0; i < count; ++i)
        if (!a->valid(ids[i]) || ++need[ids[i]] > a->ref[ids[i]])
            return false;
    return true;
}

}  // namespace

extern "C" {

pa_block_allocator *pa_allocator_create(int32_t num_blocks)
{
    if (num_blocks <= 0 || (int64_t)num_blocks * kBlock > INT32_MAX)   // slots are int32
        return nullptr;
    pa_block_allocator *a = new (std::nothrow) pa_block_allocator;
    if (!a)
        return nullptr;
    try {
        a->ring.resize(num_blocks);
        a->ref.assign(num_blocks, 0);
    } catch (...) {
        delete a;
        return nullptr;
    }
    for (int32_t i = 0; i < num_blocks; ++i)
        a->ring[i] = i;
    a->nfree = num_blocks;
    return a;
}

void pa_allocator_destroy(pa_block_allocator *alloc) { delete alloc; }

int32_t pa_allocator_num_free(const pa_block_allocator *alloc)
{
    return alloc ? alloc->nfree : -1;
}

int32_t pa_allocator_ref_count(const pa_block_allocator *alloc, int32_t block)
{
    return (alloc && alloc->valid(block)) ? alloc->ref[block] : -1;
}

pa_status pa_allocator_acquire(pa_block_allocator *alloc, int32_t count, int32_t *ids_out)
{
    if (!alloc || count < 0 || (count > 0 && !ids_out))
        return PA_ERR_INVALID_ARG;
    if (count > alloc->nfree)
        return PA_ERR_OUT_OF_BLOCKS;
    for (int32_t i = 0; i < count; ++i)
        ids_out[i] = alloc->take();
    return PA_OK;
}

pa_status pa_allocator_share(pa_block_allocator *alloc, const int32_t *ids, int32_t count)
{
    if (!alloc || count < 0 || (count > 0 && !ids) || !row_ok(alloc, ids, count))
        return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < count; ++i)
        ++alloc->ref[ids[i]];
    return PA_OK;
}

pa_status pa_allocator_release(pa_block_allocator *alloc, const int32_t *ids, int32_t count)
{
    if (!alloc || count < 0 || (count > 0 && !ids) || !refs_cover(alloc, ids, count))
        return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < count; ++i)
        alloc->unref(ids[i]);
    return PA_OK;
}

pa_status pa_seq_reserve(pa_block_allocator *alloc, int32_t *table_row, int32_t max_blocks,
                         int32_t context_len, int32_t num_new, int32_t *slots_out,
                         int32_t *copy_pairs_out, int32_t *num_copies_out)
{
    if (!alloc || !table_row || max_blocks <= 0 || context_len < 0 || num_new < 0 ||
        !num_copies_out || (num_new > 0 && (!slots_out || !copy_pairs_out)))
        return PA_ERR_INVALID_ARG;
    const int64_t new_len = (int64_t)context_len + num_new;
    if (new_len > (int64_t)max_blocks * kBlock)
        return PA_ERR_INVALID_ARG;
    const int32_t have = blocks_for(context_len);
    if (!row_ok(alloc, table_row, have))
        return PA_ERR_INVALID_ARG;
    *num_copies_out = 0;
    if (num_new == 0)
        return PA_OK;
    // the partly filled last block gets written; a shared one is copied first
    const bool cow = (context_len % kBlock) != 0 && alloc->ref[table_row[have - 1]] > 1;
    const int32_t fresh = blocks_for(new_len) - have;
    if (fresh + (cow ? 1 : 0) > alloc->nfree)
        return PA_ERR_OUT_OF_BLOCKS;
    if (cow) {
        const int32_t old = table_row[have - 1];
        const int32_t dst = alloc->take();
        alloc->unref(old);                 // still > 0: other sharers keep it
        table_row[have - 1] = dst;
        copy_pairs_out[0] = old;
        copy_pairs_out[1] = dst;
        *num_copies_out = 1;
    }
    for (int32_t i = 0; i < fresh; ++i)
        table_row[have + i] = alloc->take();
    for (int32_t i = 0; i < num_new; ++i) {
        const int64_t pos = (int64_t)context_len + i;
        slots_out[i] = table_row[pos / kBlock] * kBlock + (int32_t)(pos % kBlock);
    }
    return PA_OK;
}

pa_status pa_seq_fork(pa_block_allocator *alloc, const int32_t *src_row, int32_t *dst_row,
                      int32_t max_blocks, int32_t context_len)
{
    if (!alloc || !src_row || !dst_row || max_blocks <= 0 || context_len < 0 ||
        (int64_t)context_len > (int64_t)max_blocks * kBlock)
        return PA_ERR_INVALID_ARG;
    const int32_t used = blocks_for(context_len);
    if (!row_ok(alloc, src_row, used))
        return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < used; ++i) {
        dst_row[i] = src_row[i];
        ++alloc->ref[src_row[i]];
    }
    for (int32_t i = used; i < max_blocks; ++i)
        dst_row[i] = -1;
    return PA_OK;
}

pa_status pa_seq_truncate(pa_block_allocator *alloc, int32_t *table_row, int32_t max_blocks,
                          int32_t context_len, int32_t new_len)
{
    if (!alloc || !table_row || max_blocks <= 0 || context_len < 0 || new_len < 0 ||
        new_len > context_len || (int64_t)context_len > (int64_t)max_blocks * kBlock)
        return PA_ERR_INVALID_ARG;
    const int32_t used = blocks_for(context_len);
    const int32_t keep = blocks_for(new_len);
    if (!row_ok(alloc, table_row, used) || !refs_cover(alloc, table_row + keep, used - keep))
        return PA_ERR_INVALID_ARG;
    for (int32_t i = keep; i < used; ++i) {
        alloc->unref(table_row[i]);
        table_row[i] = -1;
    }
    return PA_OK;
}

}  // extern "C"
