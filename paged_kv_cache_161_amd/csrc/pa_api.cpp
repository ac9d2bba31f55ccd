// pa_api.cpp -- the library's C ABI: argument checks, partition choice, launches.
// Every check here runs on the host before anything is enqueued, so an error return
// means nothing was written.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>


#include "../../include/paged_attention.h"
#include "pa_common.h"
#include "pa_prefill.h"

namespace {

using pa::kBlock;

bool dtype_ok(int32_t dtype)
{
    return dtype == PA_F32 || dtype == PA_F16 || dtype == PA_BF16 || dtype == PA_FP8_E4M3;
}

bool head_dim_ok(int32_t dtype, int32_t head_dim)
{
    if (head_dim == 64 || head_dim == 128)
        return true;
    return head_dim == 256 && dtype != PA_F32;
}

size_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_FP8_E4M3 ? 1 : 2); }

// Most blocks one partition may hold: the kernels keep the block ids a wave (or block
// lane) walks one per lane of a single register, 64 per lane.
int32_t max_part_blocks(int32_t dtype, int32_t head_dim, int32_t group)
{
    return pa::decode_lanes(dtype, head_dim, group) * pa::kWave;
}

// Partition workgroups per (sequence, kv-head, partition): one per
// decode_chunks(dtype, head_dim, group) x 16 q-heads of the group.
int64_t wg_chunks(int32_t dtype, int32_t head_dim, int32_t group)
{
    const int64_t hs = 16 * pa::decode_chunks(dtype, head_dim, group);
    return (group + hs - 1) / hs;
}

// The kernels move pool tiles, q, out, new rows and workspace partials in 16-byte
// vectors, and index arrays as 32-bit words.
bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

// The per-head scale arrays the kernels see: only fp8 pools use them.
const float *k_heads(const pa_kv_pool *pool)
{
    return pool->dtype == PA_FP8_E4M3 ? pool->k_head_scales : nullptr;
}
const float *v_heads(const pa_kv_pool *pool)
{
    return pool->dtype == PA_FP8_E4M3 ? pool->v_head_scales : nullptr;
}

pa_status check_pool(const pa_kv_pool *pool)
{
    if (!pool || !pool->k_pool || !pool->v_pool)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(pool->k_pool) || !aligned16(pool->v_pool))
        return PA_ERR_INVALID_ARG;
    if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0)
        return PA_ERR_INVALID_ARG;
    if (!dtype_ok(pool->dtype))
        return PA_ERR_UNSUPPORTED;
    if (pool->block_size != PA_BLOCK_SIZE || !head_dim_ok(pool->dtype, pool->head_dim))
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)pool->num_blocks * kBlock > INT32_MAX)   // slots are int32
        return PA_ERR_UNSUPPORTED;
    if ((pool->flags & ~PA_POOL_SHARED_BLOCKS) != 0)
        return PA_ERR_INVALID_ARG;
    if (pool->dtype == PA_FP8_E4M3) {
        if (pool->act_dtype != PA_F16 && pool->act_dtype != PA_BF16)
            return PA_ERR_UNSUPPORTED;
        // a pool-wide scale must be valid where no per-head array replaces it; per-head
        // values live on the device and are checked there (a bad one poisons its head)
        if (!pool->k_head_scales && (!(pool->k_scale > 0.f) || !isfinite(pool->k_scale)))
            return PA_ERR_INVALID_ARG;
        if (!pool->v_head_scales && (!(pool->v_scale > 0.f) || !isfinite(pool->v_scale)))
            return PA_ERR_INVALID_ARG;
        if (!aligned4(pool->k_head_scales) || !aligned4(pool->v_head_scales))
            return PA_ERR_INVALID_ARG;
    } else if (pool->act_dtype != pool->dtype) {
        return PA_ERR_UNSUPPORTED;
    }
    return PA_OK;
}

// Partition length in blocks for a (validated) decode call; 0 on invalid input.
int32_t choose_part_blocks(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t dtype, int32_t max_context_len,
                           int32_t partition_tokens)
{
    const int32_t max_blocks = (max_context_len + kBlock - 1) / kBlock;
    if (max_blocks == 0)
        return 1;
    if (partition_tokens > 0)
        return partition_tokens / kBlock;
    // Auto: as few partitions as fit (a partition is at most 64 blocks per wave), so
    // each workgroup streams long runs and no merge pass is needed when a sequence fits
    // one; cut finer only when that leaves fewer workgroups than the GPU has CUs, but
    // not below ~2 blocks per wave.
    const int32_t group = num_q_heads / num_kv_heads;
    const int32_t nw = pa::decode_lanes(dtype, head_dim, group);
    const int64_t units = (int64_t)num_seqs * num_kv_heads * wg_chunks(dtype, head_dim, group);
    const int64_t max_pb = max_part_blocks(dtype, head_dim, group);
    int64_t parts = (max_blocks + max_pb - 1) / max_pb;
    if (units * parts < pa::kTargetGroups) {
        const int64_t fill = (pa::kTargetGroups + units - 1) / units;
        const int64_t cap = (max_blocks + 2 * nw - 1) / (2 * nw);
        const int64_t want = fill < cap ? fill : cap;
        if (want > parts)
            parts = want;
    }
    if (parts < 1)
        parts = 1;
    int32_t pb = (int32_t)((max_blocks + parts - 1) / parts);
    if (pb > max_pb)
        pb = (int32_t)max_pb;
    return pb;
}

// Host-side validation of pa_decode's scalar arguments (dtype: the pools' element type).
pa_status check_decode_scalars(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype, int32_t max_context_len,
                               int32_t partition_tokens)
{
    if (!dtype_ok(dtype) || head_dim <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0)
        return PA_ERR_INVALID_ARG;
    if (max_context_len > INT32_MAX - kBlock)         // block counts stay in int32
        return PA_ERR_UNSUPPORTED;
    if (num_q_heads % num_kv_heads != 0)
        return PA_ERR_INVALID_ARG;
    if (partition_tokens < 0 || partition_tokens % kBlock != 0)
        return PA_ERR_INVALID_ARG;
    const int32_t group = num_q_heads / num_kv_heads;
    if (partition_tokens > 0 &&
        partition_tokens / kBlock > max_part_blocks(dtype, head_dim, group))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535)
        return PA_ERR_UNSUPPORTED;
    // grid y of the partition kernel and of the reduce
    if ((int64_t)num_kv_heads * wg_chunks(dtype, head_dim, group) > 65535 ||
        (int64_t)num_kv_heads * ((group + 15) / 16) > 65535)
        return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t dtype)
{
    if (num_blocks <= 0 || num_kv_heads <= 0 || !dtype_ok(dtype) || !head_dim_ok(dtype, head_dim))
        return 0;
    return (size_t)num_blocks * num_kv_heads * kBlock * head_dim * elem_bytes(dtype);
}

const char *pa_status_string(int32_t status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
    case PA_ERR_SCRATCH: return "needs more than pa_decode_noalloc's static scratch buffer";
    default: return "unknown status";
    }
}

pa_status pa_cache_append(const pa_kv_pool *pool, const void *k_new, const void *v_new,
                          const int32_t *slot_mapping, int32_t num_tokens, void *stream)
{
    pa_status st = check_pool(pool);
    if (st != PA_OK)
        return st;
    if (num_tokens < 0)
        return PA_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return PA_OK;
    if ((int64_t)num_tokens * pool->num_kv_heads > (int64_t(1) << 34))   // launch size
        return PA_ERR_UNSUPPORTED;
    if (!k_new || !v_new || !slot_mapping)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned4(slot_mapping))
        return PA_ERR_INVALID_ARG;
    pa::AppendArgs a;
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_blocks = pool->num_blocks;
    a.num_kv_heads = pool->num_kv_heads;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.bf16 = pool->act_dtype == PA_BF16 ? 1 : 0;
    a.k_head_scales = k_heads(pool);
    a.v_head_scales = v_heads(pool);
    hipError_t e = pa::launch_append(pool->dtype, pool->act_dtype, pool->head_dim, a,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks(const pa_kv_pool *pool, const int32_t *pairs, int32_t num_pairs,
                         void *stream)
{
    pa_status st = check_pool(pool);
    if (st != PA_OK)
        return st;
    if (num_pairs < 0)
        return PA_ERR_INVALID_ARG;
    if (num_pairs == 0)
        return PA_OK;
    if (!pairs || num_pairs > 65535)
        return num_pairs > 65535 ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG;
    if (!aligned4(pairs))
        return PA_ERR_INVALID_ARG;
    const size_t block_bytes =
        (size_t)pool->num_kv_heads * kBlock * pool->head_dim * elem_bytes(pool->dtype);
    hipError_t e = pa::launch_copy_blocks(pool->k_pool, pool->v_pool, pairs, num_pairs,
                                          pool->num_blocks, block_bytes,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t dtype, int32_t max_context_len)
{
    if (check_decode_scalars(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                             max_context_len, 0) != PA_OK)
        return -1;
    return choose_part_blocks(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                              max_context_len, 0) *
           kBlock;
}

int32_t pa_decode_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t dtype, const int32_t *context_lens_host)
{
    if (num_seqs < 0 || (num_seqs > 0 && !context_lens_host) || head_dim <= 0)
        return -1;
    int32_t max_ctx = 0;
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (context_lens_host[b] < 0)
            return -1;
        if (context_lens_host[b] > max_ctx)
            max_ctx = context_lens_host[b];
    }
    if (check_decode_scalars(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype, max_ctx, 0) !=
        PA_OK)
        return -1;
    const int32_t auto_pb =
        choose_part_blocks(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype, max_ctx, 0);
    const int32_t max_blocks = (max_ctx + kBlock - 1) / kBlock;
    if (max_blocks == 0)
        return auto_pb * kBlock;
    bool equal = true;
    for (int32_t b = 1; b < num_seqs && equal; ++b)
        equal = context_lens_host[b] == context_lens_host[0];
    if (equal)                  // every sequence cut alike: the automatic, even split
        return auto_pb * kBlock;
    // Workgroups that stream at least one block, for partitions of pb blocks (empty
    // partitions exit at once).  Non-increasing in pb.
    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t per_seq = (int64_t)num_kv_heads * wg_chunks(dtype, head_dim, group);
    auto busy_groups = [&](int64_t pb) {
        int64_t w = 0;
        for (int32_t b = 0; b < num_seqs; ++b)
            w += ((context_lens_host[b] + kBlock - 1) / kBlock + pb - 1) / pb;
        return w * per_seq;
    };
    // The longest sequence is cut into the most partitions that still keep every busy
    // workgroup in one round of the GPU's CUs, and those partitions are made as long as
    // that count allows (the last one short): measured on the long + shared-prefix
    // decode, 6 partitions of 408 blocks run 7 % faster than 6 of 344.  When no
    // partition allows one round, the automatic rule.
    const int64_t nw = pa::decode_lanes(dtype, head_dim, group);
    const int64_t max_pb = max_part_blocks(dtype, head_dim, group);
    int64_t lo = 2 * nw, hi = max_pb < max_blocks ? max_pb : max_blocks;
    if (lo > hi)
        lo = hi;
    if (busy_groups(hi) > pa::kTargetGroups)
        return auto_pb * kBlock;
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (busy_groups(mid) <= pa::kTargetGroups)
            hi = mid;
        else
            lo = mid + 1;
    }
    const int64_t parts = (max_blocks + lo - 1) / lo;  // of the longest sequence
    if (parts <= 1)                                    // one partition per sequence
        return auto_pb * kBlock;
    // Two partitions are cut evenly instead: a short second one would leave half the
    // longest sequences' workgroups nearly empty while the other half streams almost
    // the whole context, one workgroup's streaming rate then setting the time
    // (4,096-token contexts at G = 16: 248 + 8 blocks 67 us, 128 + 128 blocks 56 us).
    int64_t pb = parts == 2 ? (max_blocks + 1) / 2 + nw - 1   // even halves,
                            : (max_blocks - 1) / (parts - 1); // else longest with that count,
    pb = pb / nw * nw;
    const int64_t pb_min = (lo + nw - 1) / nw * nw;           // whole blocks per wave
    if (pb < pb_min)
        pb = pb_min;
    if (pb > max_pb)
        pb = max_pb;
    return (int32_t)(pb * kBlock);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, int32_t max_context_len,
                                 int32_t partition_tokens)
{
    if (check_decode_scalars(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                             max_context_len, partition_tokens) != PA_OK)
        return SIZE_MAX;
    const int32_t pb = choose_part_blocks(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                                          max_context_len, partition_tokens);
    const int32_t max_blocks = (max_context_len + kBlock - 1) / kBlock;
    const int64_t parts = max_blocks == 0 ? 1 : (max_blocks + pb - 1) / pb;
    if (parts <= 1)
        return 0;
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)parts;
    return rows * (size_t)head_dim * sizeof(float) + 2 * rows * sizeof(float);
}

}  // extern "C"

namespace {

// Fewest keys of the longest context one prefill key split covers: below that the
// partials' write and merge outweigh the CUs the split brings in.
constexpr int64_t kPrefillMinSplitKeys = 1024;

// Scalar checks shared by pa_prefill and its planners; PA_OK when the shapes are ones
// the prefill kernels take.
pa_status check_prefill_scalars(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, int32_t num_query_tokens,
                                int32_t max_query_len, int32_t max_context_len,
                                int32_t key_splits)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || num_query_tokens < 0 || max_query_len < 0 ||
        max_context_len < 0 || key_splits < 0)
        return PA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype) || !head_dim_ok(dtype, head_dim))
        return PA_ERR_UNSUPPORTED;
    // 16-bit MFMA kernels only (fp8 pools convert to their 16-bit activation type)
    if (dtype == PA_F32)
        return PA_ERR_UNSUPPORTED;
    if (key_splits > pa::kPrefillMaxSplits)
        return PA_ERR_UNSUPPORTED;
    const int32_t group = num_q_heads / num_kv_heads;
    if (group > pa::prefill_rows_per_group(head_dim))
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_query_tokens * num_q_heads > INT32_MAX)
        return PA_ERR_UNSUPPORTED;
    if (max_context_len > INT32_MAX - kBlock)         // block counts stay in int32
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_kv_heads * kBlock * head_dim > UINT32_MAX)
        return PA_ERR_UNSUPPORTED;                    // block stride in 32 bits
    return PA_OK;
}

// Key splits of a prefill launch: key_splits when given; otherwise as many as bring the
// launch's (sequence, kv-head, query tile) units up to one per CU, at most
// kPrefillMaxSplits and at least kPrefillMinSplitKeys keys of the longest context per
// split.  Units are estimated from host bounds only: per kv-head the tiles of T query
// rows in chunks of at most max_query_len, i.e. at most T / q_tile + B and B x
// ceil(max_query_len / q_tile) -- ragged batches are overestimated, so they split less.
int32_t choose_prefill_splits(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_query_tokens, int32_t max_query_len,
                              int32_t max_context_len, int32_t key_splits)
{
    if (key_splits > 0)
        return key_splits;
    const int64_t q_tile = pa::prefill_rows_per_group(head_dim) / (num_q_heads / num_kv_heads);
    const int64_t qtiles = ((int64_t)max_query_len + q_tile - 1) / q_tile;
    const int64_t tiles = std::min<int64_t>((num_query_tokens + q_tile - 1) / q_tile + num_seqs,
                                            (int64_t)num_seqs * qtiles);
    const int64_t units = (int64_t)num_kv_heads * tiles;
    if (units <= 0 || units * 2 > pa::kTargetGroups)
        return 1;
    int64_t sp = pa::kTargetGroups / units;
    sp = std::min<int64_t>(sp, pa::kPrefillMaxSplits);
    sp = std::min<int64_t>(sp, max_context_len / kPrefillMinSplitKeys);
    return (int32_t)std::max<int64_t>(sp, 1);
}

// pa_decode, and pa_decode_append when k_new / v_new are given.
pa_status decode_impl(const pa_kv_pool *pool, const void *q, const void *k_new,
                      const void *v_new, void *out, int32_t num_seqs, int32_t num_q_heads,
                      float scale, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t max_context_len,
                      int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    pa_status st = check_pool(pool);
    if (st != PA_OK)
        return st;
    st = check_decode_scalars(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim,
                              pool->dtype, max_context_len, partition_tokens);
    if (st != PA_OK)
        return st;
    if (max_blocks_per_seq < 0 || !isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_seqs == 0)
        return PA_OK;
    if (!q || !out || !block_tables || !context_lens || max_blocks_per_seq == 0)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned4(block_tables) || !aligned4(context_lens))
        return PA_ERR_INVALID_ARG;
    if ((k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
        return PA_ERR_INVALID_ARG;

    const int32_t pb = choose_part_blocks(num_seqs, num_q_heads, pool->num_kv_heads,
                                          pool->head_dim, pool->dtype, max_context_len,
                                          partition_tokens);
    const int32_t max_blocks = (max_context_len + kBlock - 1) / kBlock;
    const int32_t parts = max_blocks == 0 ? 1 : (max_blocks + pb - 1) / pb;
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, pool->num_kv_heads,
                                                  pool->head_dim, pool->dtype, max_context_len,
                                                  partition_tokens);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return PA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace))
        return PA_ERR_INVALID_ARG;
    if (pb > max_part_blocks(pool->dtype, pool->head_dim, num_q_heads / pool->num_kv_heads))
        return PA_ERR_UNSUPPORTED;

    pa::DecodeArgs a;
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.q = q;
    a.out = out;
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)parts;
    a.ws_o = parts > 1 ? static_cast<float *>(workspace) : nullptr;
    a.ws_m = parts > 1 ? a.ws_o + rows * pool->head_dim : nullptr;
    a.ws_l = parts > 1 ? a.ws_m + rows : nullptr;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_blocks = pool->num_blocks;
    a.num_kv_heads = pool->num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.group = num_q_heads / pool->num_kv_heads;
    a.head_chunks = (a.group + 15) / 16;
    a.wg_heads = 16 * pa::decode_chunks(pool->dtype, pool->head_dim, a.group);
    a.wg_chunks = (a.group + a.wg_heads - 1) / a.wg_heads;
    a.max_blocks = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.part_blocks = pb;
    a.num_parts = parts;
    const bool fp8 = pool->dtype == PA_FP8_E4M3;
    // a per-head K scale multiplies scale * log2(e) on the device, in this same order
    a.scale_log2 = scale * 1.4426950408889634f * (fp8 && !k_heads(pool) ? pool->k_scale : 1.0f);
    a.v_scale = fp8 ? pool->v_scale : 1.0f;
    a.k_head_scales = k_heads(pool);
    a.v_head_scales = v_heads(pool);
    a.split = parts > 1 ? 1 : 0;
    a.longest_first = (num_seqs > 1 && num_seqs <= pa::kLongestFirstMax) ? 1 : 0;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_quant = pool->k_scale;
    a.v_quant = pool->v_scale;
    a.act_bf16 = pool->act_dtype == PA_BF16 ? 1 : 0;
    a.stream_kv = (pool->flags & PA_POOL_SHARED_BLOCKS) ? 0 : 1;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = pa::launch_decode(pool->dtype, pool->act_dtype, pool->head_dim, a, num_seqs, s);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ---------------------------------------------------- allocation-free decode's buffer
// pa_decode_noalloc keeps its split partials here instead of in a caller's workspace.
// Each GPU the library runs on holds its own copy of the array until the process ends.
// On the host, `scratch` names only a host-side stand-in: its device address on each
// GPU comes from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This thread's current device's address of `scratch` (looked up on its first use).
pa_status current_device_scratch(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return PA_ERR_HIP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return PA_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(const pa_kv_pool *pool, const void *q, void *out, int32_t num_seqs,
                            int32_t num_q_heads, float scale, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, int32_t partition_tokens, void *stream)
{
    void *ws = nullptr;
    pa_status st = current_device_scratch(&ws);
    if (st != PA_OK)
        return st;
    // pa_decode's checks and launches, the static array as the workspace; the only
    // workspace error left is a need beyond the array's size
    st = decode_impl(pool, q, nullptr, nullptr, out, num_seqs, num_q_heads, scale, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, partition_tokens, ws,
                     PA_NOALLOC_SCRATCH_BYTES, stream);
    return st == PA_ERR_WORKSPACE ? PA_ERR_SCRATCH : st;
}

pa_status pa_decode(const pa_kv_pool *pool, const void *q, void *out, int32_t num_seqs,
                    int32_t num_q_heads, float scale, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                    int32_t max_context_len, int32_t partition_tokens, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    return decode_impl(pool, q, nullptr, nullptr, out, num_seqs, num_q_heads, scale,
                       block_tables, max_blocks_per_seq, context_lens, max_context_len,
                       partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_append(const pa_kv_pool *pool, const void *q, const void *k_new,
                           const void *v_new, void *out, int32_t num_seqs, int32_t num_q_heads,
                           float scale, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t max_context_len,
                           int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    if (num_seqs > 0 && (!k_new || !v_new))
        return PA_ERR_INVALID_ARG;
    return decode_impl(pool, q, k_new, v_new, out, num_seqs, num_q_heads, scale, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, partition_tokens,
                       workspace, workspace_bytes, stream);
}

int32_t pa_prefill_key_splits(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t dtype, int32_t num_query_tokens,
                              int32_t max_query_len, int32_t max_context_len)
{
    if (check_prefill_scalars(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                              num_query_tokens, max_query_len, max_context_len, 0) != PA_OK)
        return -1;
    return choose_prefill_splits(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 num_query_tokens, max_query_len, max_context_len, 0);
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t dtype, int32_t num_query_tokens,
                                  int32_t max_query_len, int32_t max_context_len,
                                  int32_t key_splits)
{
    if (check_prefill_scalars(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                              num_query_tokens, max_query_len, max_context_len,
                              key_splits) != PA_OK)
        return SIZE_MAX;
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0)
        return 0;
    const int32_t sp = choose_prefill_splits(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             num_query_tokens, max_query_len, max_context_len,
                                             key_splits);
    if (sp <= 1)
        return 0;
    return (size_t)num_query_tokens * num_q_heads * sp * (head_dim + 2) * sizeof(float);
}

pa_status pa_prefill(const pa_kv_pool *pool, const void *q, void *out, int32_t num_seqs,
                     int32_t num_q_heads, float scale, const int32_t *query_start,
                     int32_t num_query_tokens, int32_t max_query_len,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t max_context_len,
                     int32_t key_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    pa_status st = check_pool(pool);
    if (st != PA_OK)
        return st;
    if (max_blocks_per_seq < 0 || !isfinite(scale) || !(scale > 0.f))
        return PA_ERR_INVALID_ARG;
    st = check_prefill_scalars(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim,
                               pool->dtype, num_query_tokens, max_query_len, max_context_len,
                               key_splits);
    if (st != PA_OK)
        return st;
    const int32_t group = num_q_heads / pool->num_kv_heads;
    const int32_t rows = pa::prefill_rows_per_group(pool->head_dim);
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0)
        return PA_OK;
    if (!q || !out || !query_start || !block_tables || !context_lens || max_blocks_per_seq == 0)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned4(query_start) || !aligned4(block_tables) ||
        !aligned4(context_lens))
        return PA_ERR_INVALID_ARG;
    const int32_t q_tile = rows / group;
    const int64_t qtiles = ((int64_t)max_query_len + q_tile - 1) / q_tile;
    const int64_t pairs = (int64_t)num_seqs * pool->num_kv_heads;
    if (pairs > INT32_MAX || ((pairs + 7) / 8) * 8 * qtiles > INT32_MAX)
        return PA_ERR_UNSUPPORTED;
    const int32_t splits = choose_prefill_splits(num_seqs, num_q_heads, pool->num_kv_heads,
                                                 pool->head_dim, num_query_tokens,
                                                 max_query_len, max_context_len, key_splits);
    const size_t need = splits > 1 ? pa_prefill_workspace_bytes(
                                         num_seqs, num_q_heads, pool->num_kv_heads,
                                         pool->head_dim, pool->dtype, num_query_tokens,
                                         max_query_len, max_context_len, key_splits)
                                   : 0;
    // the reduce of a split launch runs one workgroup column per sequence and kv-head
    if (splits > 1 && (num_seqs > 65535 || pool->num_kv_heads > 65535))
        return PA_ERR_UNSUPPORTED;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return PA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace))
        return PA_ERR_INVALID_ARG;

    pa::PrefillArgs a;
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.q = q;
    a.out = out;
    a.query_start = query_start;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_blocks = pool->num_blocks;
    a.num_kv_heads = pool->num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.group = group;
    a.max_blocks = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.num_tokens = num_query_tokens;
    a.max_query_len = max_query_len;
    a.q_tile = q_tile;
    a.num_qtiles = (int32_t)qtiles;
    const bool fp8 = pool->dtype == PA_FP8_E4M3;
    a.scale_log2 = scale * 1.4426950408889634f * (fp8 && !k_heads(pool) ? pool->k_scale : 1.0f);
    a.v_scale = fp8 ? pool->v_scale : 1.0f;
    a.k_head_scales = k_heads(pool);
    a.v_head_scales = v_heads(pool);
    a.longest_first = (num_seqs > 1 && num_seqs <= pa::kLongestFirstMax) ? 1 : 0;
    a.splits = splits;
    const size_t partials = (size_t)num_query_tokens * num_q_heads * splits;
    a.ws_o = splits > 1 ? static_cast<float *>(workspace) : nullptr;
    a.ws_m = splits > 1 ? a.ws_o + partials * pool->head_dim : nullptr;
    a.ws_l = splits > 1 ? a.ws_m + partials : nullptr;
    hipError_t e = pa::launch_prefill(pool->dtype, pool->act_dtype, pool->head_dim, a,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
