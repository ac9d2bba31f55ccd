// pa_prefill.h -- prefill kernel arguments, launch shape and launcher.
#pragma once

#include "pa_common.h"

namespace pa {

// Arguments of the prefill kernel.
struct PrefillArgs {
    const void *k_pool;               // [num_blocks][hkv][16][D]
    const void *v_pool;               // [num_blocks][hkv][D][16]
    const void *q;                    // [T][hq][D]
    void *out;                        // [T][hq][D]
    const int32_t *query_start;       // [B+1]: q rows of sequence b
    const int32_t *block_tables;      // [B][max_blocks]
    const int32_t *context_lens;      // [B], chunk included
    int32_t num_seqs;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t group;                    // hq / hkv
    int32_t max_blocks;
    int32_t max_context_len;
    int32_t num_tokens;               // T
    int32_t max_query_len;
    int32_t q_tile;                   // query positions per workgroup
    int32_t num_qtiles;               // ceil(max_query_len / q_tile)
    float scale_log2;                 // scale * log2(e) (* k_scale for fp8 pools), > 0
    float v_scale;
    int32_t longest_first;            // 1: sequences taken in order of estimated tile cost
    // fp8 pools: per-kv-head scales ([hkv], device) or null; a non-null k_head_scales
    // multiplies scale_log2 for its head, a non-null v_head_scales replaces v_scale.
    const float *k_head_scales;
    const float *v_head_scales;
    // key splits (launch grid y): each (sequence, kv-head, query tile) is cut into this
    // many contiguous ranges of its key steps; above 1 the workgroups write partials
    // (slot = (q-row * hq + head) * splits + split) that pa_prefill_reduce merges
    int32_t splits;
    float *ws_o;                      // [T * hq * splits][D] unnormalised outputs
    float *ws_m;                      // [T * hq * splits] reference max (log2 domain)
    float *ws_l;                      // [T * hq * splits] normaliser
};

// Most key splits one prefill launch takes.
constexpr int kPrefillMaxSplits = 8;

// Prefill workgroup shape: waves and 16-row MFMA column blocks per wave.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
#ifndef PA_PREFILL_COLS
#define PA_PREFILL_COLS 2
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
constexpr int kPrefillCols = PA_PREFILL_COLS;

// Column blocks per wave at head_dim d, so that C * d = 256 at every size (the same
// registers for O accumulators, q fragments and K/V fragments): four at d = 64, where
// more rows per wave halve the LDS fragment bytes per product; kPrefillCols at
// d = 128; one at d = 256.
constexpr int prefill_cols(int head_dim)
{
    return head_dim > 128 ? 1 : (head_dim <= 64 ? 2 * kPrefillCols : kPrefillCols);
}

// Query rows ((position, q-head) pairs) one prefill workgroup holds at head_dim d.
int prefill_rows_per_group(int head_dim);

hipError_t launch_prefill(int dtype, int act_dtype, int head_dim, const PrefillArgs &a,
                          hipStream_t stream);

// Token rows one reduce workgroup merges, all q-heads of one kv-head for each: 256
// threads x 4 items of 4 elements, at least one row.
constexpr int prefill_reduce_rows(int group, int head_dim)
{
    return group * head_dim / 4 >= 1024 ? 1 : 1024 / (group * head_dim / 4);
}

}  // namespace pa
