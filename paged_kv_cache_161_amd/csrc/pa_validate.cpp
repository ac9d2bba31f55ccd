// pa_validate.cpp -- host checks of a batch's index arrays against the contract the
// kernels assume, for callers that build block tables and slot mappings themselves.
//
// The kernels never read outside the pool whatever these arrays hold (a bad entry
// turns into NaN rows or a skipped row); these checks name the first offending
// sequence or row on the host instead, before anything is launched.  The rules are
// those of the block table (LLM-101-CN "推理优化", section "物理块与逻辑块": logical
// block i of a request lives in physical block table[i]; token t in block t / 16 at
// offset t % 16) and of the slot numbering slot = block * 16 + offset of the append.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/paged_attention.h"

namespace {

constexpr int64_t kBlock = PA_BLOCK_SIZE;

void set_bad(int32_t *out, int32_t v)
{
    if (out)
        *out = v;
}

// Sequence b's context length and the table entries it reads.
bool seq_ok(int32_t b, const int32_t *block_tables, int32_t max_blocks,
            const int32_t *context_lens, int32_t max_context_len, int32_t num_blocks)
{
    const int32_t ctx = context_lens[b];
    if (ctx < 0 || ctx > max_context_len || (int64_t)ctx > (int64_t)max_blocks * kBlock)
        return false;
    const int64_t nblk = (ctx + kBlock - 1) / kBlock;
    const int32_t *row = block_tables + (int64_t)b * max_blocks;
    for (int64_t i = 0; i < nblk; ++i)
        if (row[i] < 0 || row[i] >= num_blocks)
            return false;
    return true;
}

}  // namespace

extern "C" {

pa_status pa_validate_decode_tables(int32_t num_seqs, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t max_context_len, int32_t num_blocks,
                                    int32_t *bad_seq_out)
{
    set_bad(bad_seq_out, -1);
    if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!block_tables || !context_lens))
        return PA_ERR_INVALID_ARG;
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (!seq_ok(b, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                    num_blocks)) {
            set_bad(bad_seq_out, b);
            return PA_ERR_INVALID_ARG;
        }
    }
    return PA_OK;
}

pa_status pa_validate_prefill_batch(int32_t num_seqs, const int32_t *query_start,
                                    int32_t num_query_tokens, int32_t max_query_len,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t max_context_len,
                                    int32_t num_blocks, int32_t *bad_seq_out)
{
    set_bad(bad_seq_out, -1);
    if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || max_blocks_per_seq < 0 ||
        max_context_len < 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!query_start || !block_tables || !context_lens))
        return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && query_start[0] != 0) {
        set_bad(bad_seq_out, 0);
        return PA_ERR_INVALID_ARG;
    }
    for (int32_t b = 0; b < num_seqs; ++b) {
        const int64_t lo = query_start[b], hi = query_start[b + 1];
        const bool range_ok = lo <= hi && hi <= num_query_tokens && hi - lo <= max_query_len;
        if (!range_ok || !seq_ok(b, block_tables, max_blocks_per_seq, context_lens,
                                 max_context_len, num_blocks)) {
            set_bad(bad_seq_out, b);
            return PA_ERR_INVALID_ARG;
        }
    }
    if (num_seqs > 0 && query_start[num_seqs] != num_query_tokens) {
        set_bad(bad_seq_out, num_seqs - 1);
        return PA_ERR_INVALID_ARG;
    }
    return PA_OK;
}

pa_status pa_validate_slots(const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                            int32_t *bad_token_out)
{
    set_bad(bad_token_out, -1);
    if (num_tokens < 0 || num_blocks <= 0 || (num_tokens > 0 && !slot_mapping))
        return PA_ERR_INVALID_ARG;
    const int64_t slots = (int64_t)num_blocks * kBlock;
    std::vector<uint8_t> seen;
    try {
        seen.assign((size_t)slots, 0);
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s < 0)
            continue;                       // padding row
        if (s >= slots || seen[(size_t)s]) {
            set_bad(bad_token_out, i);
            return PA_ERR_INVALID_ARG;
        }
        seen[(size_t)s] = 1;
    }
    return PA_OK;
}

int32_t pa_tables_share_blocks(int32_t num_seqs, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens)
{
    if (num_seqs < 0 || max_blocks_per_seq < 0)
        return -1;
    if (num_seqs > 0 && (!block_tables || !context_lens))
        return -1;
    std::vector<int32_t> live;
    try {
        for (int32_t b = 0; b < num_seqs; ++b) {
            const int32_t ctx = context_lens[b];
            if (ctx < 0 || (int64_t)ctx > (int64_t)max_blocks_per_seq * kBlock)
                return -1;
            const int32_t *row = block_tables + (int64_t)b * max_blocks_per_seq;
            for (int64_t i = 0; i < (ctx + kBlock - 1) / kBlock; ++i)
                if (row[i] >= 0)            // a negative id names no block
                    live.push_back(row[i]);
        }
    } catch (...) {
        return -1;
    }
    std::sort(live.begin(), live.end());
    return std::adjacent_find(live.begin(), live.end()) != live.end() ? 1 : 0;
}

}  // extern "C"
