/*
 * paged_attention.h -- C ABI of the MI355X (gfx950) decode-phase PagedAttention library.
 *
 * Two operations, as the web pages on paged KV caches state the problem:
 *
 *   pa_cache_append  writes the K/V rows a decode step produces into a pool of fixed
 *                    16-token physical blocks, through a slot mapping.
 *                    (LLM-101-CN "推理优化", section "vLLM 架构深度解析",
 *                    KVCachePool.write_tokens: new rows go to a page and an offset
 *                    inside it; "LLM应用 12 推理优化", PagedKVCache.update: page =
 *                    position // page_size, offset = position % page_size.)
 *
 *   pa_decode        for every sequence and q-head, softmax(q . K^T * scale) . V over
 *                    the sequence's context, reading K/V through the sequence's block
 *                    table (logical block -> physical block), with GQA head groups.
 *                    (LLM-101-CN "推理优化", sections "物理块与逻辑块" and
 *                    "PagedAttention 内核实现" (decode: per-page local attention merged
 *                    with the max/normaliser combine); "大模型推理的三维本质原理解析与
 *                    工程实践", section 6 GQA; "Deep dive into vLLM 06", section on
 *                    Flash-Decoding: split the KV axis and merge partials with the same
 *                    m, l rescaling rule.)
 *
 * Around them: pa_decode_append (both in one launch), pa_decode_noalloc (pa_decode with
 * no workspace argument), pa_prefill (prompt chunks over the same pool), pa_copy_blocks
 * and the host block allocator (copy-on-write and rollback), the partition planners and
 * host checks of the index arrays.
 *
 * Conventions shared by every entry point
 *   - Pointers named *_pool, q, out, k_new, v_new, slot_mapping, block_tables,
 *     context_lens and workspace are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors).  pa_kv_pool itself lives in host memory and is read during the call.
 *   - Alignment: pools (k_pool, v_pool), q, out, k_new, v_new and workspace start on a
 *     16-byte boundary (every hipMalloc and torch allocation does; a view that starts
 *     inside one may not); the int32 arrays on a 4-byte boundary.  A misaligned pointer
 *     is PA_ERR_INVALID_ARG.
 *   - The caller owns every buffer.  The library allocates no device memory at run time
 *     and never frees caller memory; the only state it keeps across calls is cached
 *     device attributes and pa_decode_noalloc's static per-GPU buffer (a 16 MiB device
 *     array in the library's image).  The host allocator's state lives in the handle
 *     the caller creates and destroys.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream): they return once the kernels are enqueued.
 *   - Argument errors are detected on the host before anything is enqueued; nothing is
 *     written then.  A launch failure returns PA_ERR_HIP.  Nothing throws across the ABI.
 *   - Element types: PA_F32 (4 bytes), PA_F16 (IEEE half), PA_BF16 (bfloat16),
 *     PA_FP8_E4M3 (OCP 8-bit float, 4 exponent bits, 3 fraction bits, max 448, no
 *     infinities).  q, out and the new rows use the pool's act_dtype; for f32/f16/bf16
 *     pools that is the pool's own type.  An fp8 pool holds codes c with K = c * k_scale
 *     and V = c * v_scale, q/out/new rows being f16 or bf16 (the pages' FP8 E4M3
 *     inference format with a scale per tensor, "Deep dive into vLLM 06", FP8 section).
 *     The scale is either one per pool or one per kv-head (each head's slice of the
 *     cache treated as its own tensor; see pa_kv_pool).  Arithmetic is fp32.
 *   - Calls on different streams touching disjoint buffers may run concurrently.
 *
 * Pool layout (one layer; K and V are two separate buffers of equal size):
 *   k_pool [num_blocks][num_kv_heads][16][head_dim]   token-major inside a block
 *   v_pool [num_blocks][num_kv_heads][head_dim][16]   token-minor inside a block
 * so one (block, kv-head) tile of K or of V is a single contiguous run of
 * 16 * head_dim elements (4 KiB for head_dim 128 in 16-bit types, 2 KiB in fp8).
 * Token t of a sequence is row t % 16 of physical block block_tables[seq][t / 16]; its
 * slot number is physical_block * 16 + t % 16.
 */
#ifndef PAGED_ATTENTION_H
#define PAGED_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* null or misaligned pointer, negative size, bad shapes */
    PA_ERR_UNSUPPORTED = 2,   /* valid but not built: dtype, head_dim, block size     */
    PA_ERR_WORKSPACE = 3,     /* workspace pointer null or smaller than required      */
    PA_ERR_HIP = 4,           /* the HIP runtime reported an error at launch          */
    PA_ERR_OUT_OF_BLOCKS = 5, /* the block allocator has too few free blocks           */
    PA_ERR_SCRATCH = 6        /* pa_decode_noalloc: more than its static buffer holds  */
} pa_status;

typedef enum pa_dtype {
    PA_F32 = 0,
    PA_F16 = 1,
    PA_BF16 = 2,
    PA_FP8_E4M3 = 3
} pa_dtype;

/* One layer's paged KV pool.  block_size must be PA_BLOCK_SIZE; head_dim must be one
 * of 64, 128, 256 (64 or 128 for PA_F32).  dtype is the pools' element type;
 * act_dtype the type of q, out and the new rows: equal to dtype for f32/f16/bf16
 * pools, PA_F16 or PA_BF16 for fp8 pools.
 * Scales (fp8 pools only; ignored for other pools) turn stored codes into values:
 *   k_head_scales, v_head_scales  NULL, or DEVICE arrays of num_kv_heads fp32 values
 *                  (4-byte aligned): K of kv-head h = code * k_head_scales[h], and V
 *                  likewise.  Read on the device by every call that uses the pool, so
 *                  they may change between calls (and between replays of a captured
 *                  graph) without touching the host.  A head whose scale is not finite
 *                  and > 0 gets NaN codes on append and NaN outputs from decode and
 *                  prefill; no other head is affected.
 *   k_scale, v_scale  one scale for the whole pool (finite, > 0), used where the
 *                  corresponding per-head array is NULL.
 * flags: 0, or PA_POOL_SHARED_BLOCKS when one call's block tables may name the same
 *   physical block for several sequences (forked beams, a shared prompt prefix: the
 *   blocks whose reference count, pa_allocator_ref_count, is above 1; LLM-101-CN
 *   "推理优化", copy-on-write between sequences).  A performance hint for the decode
 *   calls, never a correctness one: results are bit for bit the same either way.
 *   Without it the decode kernels stream K/V with non-temporal loads, which read once
 *   from HBM at the rate of a plain read but leave nothing in the caches for another
 *   workgroup; with it they use ordinary loads, so the repeats of a shared block are
 *   served by the L2 and the last-level cache.  Other bits are invalid. */
#define PA_POOL_SHARED_BLOCKS 1

typedef struct pa_kv_pool {
    void *k_pool;
    void *v_pool;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
    int32_t act_dtype;
    float k_scale;
    float v_scale;
    const float *k_head_scales;
    const float *v_head_scales;
    int32_t flags;
} pa_kv_pool;

/* Bytes of ONE of the two pools (K or V) for these dimensions; 0 if any argument is
 * invalid or unsupported.  Host-only, no device access.  This is one layer's K (or
 * V) share of the pages' KV-cache size, 2 * L * H * d_h * S * B * dtype_size
 * (LLM-101-CN "推理优化", section "KV Cache 的显存计算"), taken at L = 1 and for one of
 * K and V, with num_blocks * 16 token slots in place of S * B. */
size_t pa_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                     int32_t dtype);
/* (dtype is the pools' element type: 4, 2, 2 or 1 bytes per element.) */

/* Scatter num_tokens new rows into the pool (LLM-101-CN "推理优化",
 * KVCachePool.write_tokens; "LLM应用 12 推理优化", PagedKVCache.update).
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim], the pool's act_dtype, device
 *   slot_mapping   [num_tokens] int32, device: row i goes to physical block
 *                  slot_mapping[i] / 16, row slot_mapping[i] % 16, for every kv-head.
 * Bytes are copied unchanged; an fp8 pool instead stores the E4M3 code of
 * x / s, s being the row's kv-head scale for K (for V), the quotient taken in IEEE
 * fp32 and rounded to the nearest code (ties to even), magnitudes >= 448 saturating
 * to +-448 and NaN kept NaN ("Deep dive into vLLM 06", kernel fusion: KV-cache write
 * fused with quantisation).  A negative slot means "no row" (padding) and is skipped.  A slot
 * >= num_blocks * 16 is also skipped (never written), so a bad slot cannot corrupt
 * memory outside the pool.  Two rows with the same slot race (caller
 * error).  num_tokens == 0 is a valid no-op; num_tokens * num_kv_heads above 2^34
 * returns PA_ERR_UNSUPPORTED. */
pa_status pa_cache_append(const pa_kv_pool *pool, const void *k_new, const void *v_new,
                          const int32_t *slot_mapping, int32_t num_tokens, void *stream);

/* The partition length, in tokens, pa_decode uses when partition_tokens == 0 (auto)
 * for a pool of this head_dim and element type dtype (the pools' pa_dtype: the kernel,
 * its waves per workgroup and so the longest partition depend on both).  A return value
 * >= max_context_len means a single pass (no partials, no workspace).  Host-only; the
 * same inputs always give the same answer.  Returns -1 on bad input. */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                   int32_t max_context_len);

/* A partition length for pa_decode / pa_decode_append planned from the batch's context
 * lengths as the host knows them (a serving scheduler tracks each request's KV length:
 * LLM-101-CN "推理优化", Chunked Prefill scheduler, kv_len per request).  The split
 * cuts the KV axis so that the GPU's CUs all work ("Deep dive into vLLM 06",
 * Flash-Decoding): the longest sequence is cut into the most partitions that still
 * keep every workgroup with work in one round of the MI355X's 256 CUs, each as long as
 * that count allows (two partitions are cut evenly instead); when no partition allows
 * one round, it returns the automatic choice.  A batch of equal lengths gets the
 * automatic choice.  The lengths must be those passed on the
 * device to the call that uses the result (anything else is still correct, only
 * planned for other lengths).  dtype is the pools' pa_dtype.  Host-only; returns a
 * positive multiple of 16, or -1 on bad input. */
int32_t pa_decode_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t dtype, const int32_t *context_lens_host);

/* Workspace bytes pa_decode needs for these arguments (partition_tokens as passed to
 * pa_decode, 0 = auto): the Flash-Decoding partials of a split KV axis, one
 * unnormalised output row and its running max and normaliser per (sequence, q-head,
 * partition), all fp32 ("Deep dive into vLLM 06", Flash-Decoding section: each split
 * yields a partial result with its own max and sum, merged afterwards), i.e.
 * num_seqs * num_q_heads * partitions * (head_dim + 2) * 4 bytes, for pools of element
 * type dtype.  0 when the call runs in a single pass.  Returns SIZE_MAX on invalid
 * arguments.  Host-only. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, int32_t max_context_len,
                                 int32_t partition_tokens);

/* Decode attention for one layer (definitions as cited at the top of this file).
 *   q              [num_seqs][num_q_heads][head_dim], the pool's act_dtype, device
 *   out            [num_seqs][num_q_heads][head_dim], act_dtype, device; each element
 *                  is the fp32 result rounded to nearest-even
 *   scale          multiplies q . k (normally 1/sqrt(head_dim)), applied in fp32
 *   block_tables   [num_seqs][max_blocks_per_seq] int32, device; entries at index
 *                  >= ceil(context_lens[s] / 16) are never read
 *   context_lens   [num_seqs] int32, device; token count attended by each sequence
 *                  (the step's own token included: append first, then decode)
 *   max_context_len  host-side upper bound of context_lens, sizes the launch grid;
 *                  at most INT32_MAX - 16 (PA_ERR_UNSUPPORTED above)
 *   partition_tokens 0 = automatic; otherwise a positive multiple of 16: the KV axis
 *                  of each sequence is cut into partitions of this many tokens,
 *                  computed independently and merged by the max/normaliser rule
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...) bytes
 *                  (may be NULL when that is 0); contents need no initialisation
 * num_q_heads must be a multiple of the pool's num_kv_heads; q-head h reads kv-head
 * h / (num_q_heads / num_kv_heads).  One call takes at most 65,535 sequences (the
 * launch grid's extent; PA_ERR_UNSUPPORTED above).
 * A sequence with context length 0 gets an all-zero output.  Device-side inconsistency
 * the host cannot see -- a context length < 0, > max_context_len or
 * > max_blocks_per_seq * 16, or a needed table entry outside [0, num_blocks) -- makes
 * that sequence's output NaN; no out-of-bounds memory is ever read. */
pa_status pa_decode(const pa_kv_pool *pool, const void *q, void *out, int32_t num_seqs,
                    int32_t num_q_heads, float scale, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                    int32_t max_context_len, int32_t partition_tokens, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Bytes of the static device buffer pa_decode_noalloc keeps its partials in (16 MiB). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* pa_decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments, results
 * and errors are pa_decode's (the output is bit-identical to pa_decode's for the same
 * arguments), without the workspace: the partials of a split KV axis go to a static
 * device array of PA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing (no hipMalloc, no
 * library allocation).  A call that would need more than that array
 * (pa_decode_workspace_bytes(...) > PA_NOALLOC_SCRATCH_BYTES) returns PA_ERR_SCRATCH and
 * enqueues nothing.  The array belongs to the calling thread's current device, which
 * must be the device of `stream`.  Every call on one GPU shares that GPU's array and
 * leaves its partials there: calls that can overlap in time on one GPU (other streams,
 * other host threads) race on it, so the caller must order them.  No clearing is
 * needed: each call writes every partial it reads. */
pa_status pa_decode_noalloc(const pa_kv_pool *pool, const void *q, void *out, int32_t num_seqs,
                            int32_t num_q_heads, float scale, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, int32_t partition_tokens, void *stream);

/* A decode step's append and attention in one launch: for every sequence b with
 * context_lens[b] >= 1, its new row k_new[b], v_new[b] ([num_seqs][num_kv_heads]
 * [head_dim], the pool's act_dtype, device) becomes token context_lens[b] - 1 -- it is
 * written into the pool at block block_tables[b][(ctx-1)/16], row (ctx-1)%16 (fp8
 * pools store its E4M3 codes, as pa_cache_append does) -- and the attention is
 * pa_decode's over tokens 0 .. ctx-1.  The result, and the pool afterwards, equal
 * pa_cache_append of those rows at those slots followed by pa_decode, bit for bit
 * ("Deep dive into vLLM 06", kernel fusion: the KV-cache write fused with the work
 * around it; LLM-101-CN "推理优化": a decode step appends one token, then attends).
 * The block that receives the row must not be read by another sequence of the same
 * call (copy-on-write keeps a written block private).  Other arguments, errors and
 * the workspace are as for pa_decode; a sequence whose context length or needed
 * table entry is bad gets NaN output and no row is written. */
pa_status pa_decode_append(const pa_kv_pool *pool, const void *q, const void *k_new,
                           const void *v_new, void *out, int32_t num_seqs, int32_t num_q_heads,
                           float scale, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t max_context_len,
                           int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Paged prefill (chunked prefill) attention for one layer: the query rows of prompt
 * chunks attend to the cache through the same pool and block tables as decode
 * (LLM-101-CN "推理优化", section "Chunked Prefill": a chunk's queries attend to the
 * earlier chunks' cache joined with the chunk's own K/V, with the 1/sqrt(d_h) softmax;
 * its mixed prefill/decode batch gives each request its own chunk length.  "Deep dive
 * into vLLM 06", section 4.2: each position is computed from its own prefix, i.e. the
 * attention is causal).
 *   q              [num_query_tokens][num_q_heads][head_dim], act_dtype, device
 *   out            same shape and type; fp32 result rounded to nearest-even
 *   query_start    [num_seqs + 1] int32, device: sequence b owns query rows
 *                  query_start[b] .. query_start[b+1]-1 (non-decreasing, from 0)
 *   num_query_tokens  host: the number of q rows, T
 *   max_query_len  host-side upper bound of the chunk lengths, sizes the launch grid
 *   scale          finite and > 0 (normally 1/sqrt(head_dim)), applied in fp32
 *   block_tables, max_blocks_per_seq, context_lens, max_context_len: as for pa_decode;
 *                  context_lens[b] counts the chunk, whose K/V rows must already be in
 *                  the pool (pa_cache_append first)
 *   key_splits     0 = automatic; otherwise 1 .. 8: the keys each (sequence, kv-head,
 *                  query tile) attends are cut into this many contiguous ranges,
 *                  computed by separate workgroups and merged by the max/normaliser rule
 *                  ("Deep dive into vLLM 06", Flash-Decoding: split the KV axis when the
 *                  grid would leave the GPU's CUs idle, merge the partials exactly).
 *                  Automatic splits only a launch with fewer units than CUs (a single
 *                  long prompt's chunk, a few long decode rows), see pa_prefill_key_splits.
 *                  A split launch takes at most 65,535 sequences (PA_ERR_UNSUPPORTED).
 *   workspace      device scratch of at least pa_prefill_workspace_bytes(...) bytes for
 *                  the same arguments (may be NULL when that is 0); contents need no
 *                  initialisation
 * Query i of sequence b is token context_lens[b] - q_len + i and attends to tokens
 * 0 .. context_lens[b] - q_len + i; a query placed before the context (q_len >
 * context_lens[b]) gets a zero row.  A chunk of one query is exactly a decode step.
 * Supported: 16-bit pools (f16, bf16) and fp8 pools with f16/bf16 activations, head_dim
 * 64, 128 or 256, num_q_heads / num_kv_heads <= 256 (512 at head_dim 64, 128 at 256),
 * num_kv_heads * 16 * head_dim < 2^32 (PA_ERR_UNSUPPORTED otherwise).
 * Device-side inconsistency: a bad context length or a needed table entry outside
 * [0, num_blocks) makes that sequence's rows NaN; a query range that is decreasing,
 * longer than max_query_len or outside [0, num_query_tokens) leaves that sequence's
 * rows unwritten.  Nothing out of bounds is ever read or written. */
pa_status pa_prefill(const pa_kv_pool *pool, const void *q, void *out, int32_t num_seqs,
                     int32_t num_q_heads, float scale, const int32_t *query_start,
                     int32_t num_query_tokens, int32_t max_query_len,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t max_context_len,
                     int32_t key_splits, void *workspace, size_t workspace_bytes,
                     void *stream);

/* The key splits pa_prefill uses when key_splits == 0: as many as bring the launch's
 * (sequence, kv-head, query tile) units up to one per CU of the MI355X (units estimated
 * from these host bounds: at most num_query_tokens / q_tile + num_seqs query tiles per
 * kv-head, q_tile query positions per tile), at most 8, and each split covering at
 * least 1,024 keys of max_context_len; 1 when the units already fill the CUs (the
 * pages' Flash-Decoding rule, "Deep dive into vLLM 06": split the KV axis only where
 * the parallelism is missing).  dtype is the pools' pa_dtype.  Host-only; -1 on bad
 * input. */
int32_t pa_prefill_key_splits(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t dtype, int32_t num_query_tokens,
                              int32_t max_query_len, int32_t max_context_len);

/* Workspace bytes pa_prefill needs for these arguments (key_splits as passed to it):
 * with S > 1 splits, one unnormalised fp32 output row, its running max and normaliser
 * per (query row, q-head, split), i.e. num_query_tokens * num_q_heads * S *
 * (head_dim + 2) * 4 bytes; 0 without a split.  SIZE_MAX on invalid arguments.
 * Host-only. */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t dtype, int32_t num_query_tokens,
                                  int32_t max_query_len, int32_t max_context_len,
                                  int32_t key_splits);

/* Copy whole physical blocks inside the pool: for each pair i, block pairs[2i] (src)
 * is copied to block pairs[2i+1] (dst), every kv-head, in both K and V, bytes
 * unchanged -- the copy half of copy-on-write (LLM-101-CN "推理优化", section
 * "Copy-on-Write 优化": a shared block is copied only when one sharer modifies it).
 *   pairs   [num_pairs][2] int32, device.  A pair with either id outside
 *           [0, num_blocks) is skipped.  Destinations must be distinct and must not be
 *           a source of another pair in the same call (caller error otherwise).
 * num_pairs == 0 is a valid no-op. */
pa_status pa_copy_blocks(const pa_kv_pool *pool, const int32_t *pairs, int32_t num_pairs,
                         void *stream);

/* ---------------------------------------------------------------- host input checks
 * Host-only checks of a batch's index arrays (HOST int32 arrays, read only) against the
 * rules the kernels assume: a sequence's logical block i lives in physical block
 * table[i], token t in block t / 16 at offset t % 16, and an appended row goes to slot
 * block * 16 + offset (LLM-101-CN "推理优化", section "物理块与逻辑块").  The kernels
 * never read or write outside the pool whatever the arrays hold (a bad entry gives NaN
 * rows or a skipped row); these calls name the first offender before anything is
 * launched.  Each returns PA_OK, or PA_ERR_INVALID_ARG with the offender's index in
 * *bad_*_out (if not NULL; -1 when the scalars themselves are wrong), and keeps no state. */

/* Every context length in [0, max_context_len] and at most max_blocks_per_seq * 16, and
 * every table entry a sequence reads (the first ceil(context_lens[b] / 16) of its row of
 * block_tables [num_seqs][max_blocks_per_seq]) in [0, num_blocks). */
pa_status pa_validate_decode_tables(int32_t num_seqs, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t max_context_len, int32_t num_blocks,
                                    int32_t *bad_seq_out);

/* pa_validate_decode_tables' rules, and query_start [num_seqs + 1] starting at 0, never
 * decreasing, each range at most max_query_len rows and ending at num_query_tokens. */
pa_status pa_validate_prefill_batch(int32_t num_seqs, const int32_t *query_start,
                                    int32_t num_query_tokens, int32_t max_query_len,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t max_context_len,
                                    int32_t num_blocks, int32_t *bad_seq_out);

/* Every slot of slot_mapping [num_tokens] negative (a padding row) or in
 * [0, num_blocks * 16), and no slot named twice (two rows written to one slot land in
 * an undefined order).  Allocates num_blocks * 16 bytes of host memory while it runs. */
pa_status pa_validate_slots(const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                            int32_t *bad_token_out);

/* Whether a batch's tables share blocks, for the pool's PA_POOL_SHARED_BLOCKS flag: 1 when
 * some physical block id appears more than once among the entries the sequences read
 * (the first ceil(context_lens[b] / 16) of each row of block_tables
 * [num_seqs][max_blocks_per_seq]; negative ids are skipped), as with forked beams or a
 * shared prompt prefix (LLM-101-CN "推理优化", section "Copy-on-Write 优化"); 0 when
 * every live entry is distinct; -1 on a negative count, a null array with num_seqs > 0,
 * or a context length outside [0, max_blocks_per_seq * 16].  HOST arrays; sorts a copy
 * of the live entries (sum of ceil(context_lens[b] / 16) int32 values). */
int32_t pa_tables_share_blocks(int32_t num_seqs, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens);

/* ---------------------------------------------------------------- host block allocator
 * Bookkeeping of which physical blocks are free, with reference counts so that blocks
 * can be shared by several sequences (beam-search prefixes) and copied on first write
 * (LLM-101-CN "推理优化", sections "物理块与逻辑块" (PageAllocator: a FIFO free
 * pool, acquire takes from the front and fails as a whole when too few blocks are
 * free, release returns blocks to the back) and "Copy-on-Write 优化" (blocks shared
 * with a reference count > 1 are copied only when one sharer writes)).  Host memory
 * only, no device access; one caller at a time per allocator.  Block tables passed
 * here are host int32 rows of max_blocks entries; entries past a sequence's last
 * block are set to -1.  Every call either succeeds completely or changes nothing. */
typedef struct pa_block_allocator pa_block_allocator;

/* A new allocator owning blocks 0 .. num_blocks-1, all free, in that order.  NULL on
 * num_blocks <= 0, on num_blocks * 16 > INT32_MAX (slots are int32, as for the pool),
 * or on allocation failure.  Free it with pa_allocator_destroy. */
pa_block_allocator *pa_allocator_create(int32_t num_blocks);
void pa_allocator_destroy(pa_block_allocator *alloc);

int32_t pa_allocator_num_free(const pa_block_allocator *alloc);

/* Reference count of a block: 0 when free, -1 for an id outside the pool. */
int32_t pa_allocator_ref_count(const pa_block_allocator *alloc, int32_t block);

/* Take count free blocks (front of the free pool first), each with reference count 1,
 * into ids_out[0 .. count).  PA_ERR_OUT_OF_BLOCKS (nothing taken) when fewer are free. */
pa_status pa_allocator_acquire(pa_block_allocator *alloc, int32_t count, int32_t *ids_out);

/* Add one reference to each listed block (all must be in use). */
pa_status pa_allocator_share(pa_block_allocator *alloc, const int32_t *ids, int32_t count);

/* Drop one reference from each listed block (all must be in use); a block whose count
 * reaches 0 goes to the back of the free pool, in list order. */
pa_status pa_allocator_release(pa_block_allocator *alloc, const int32_t *ids, int32_t count);

/* Reserve slots for num_new tokens appended to a sequence of context_len tokens whose
 * blocks are table_row[0 .. ceil(context_len/16)).  Token context_len + i gets
 * slots_out[i] = block * 16 + row, ready for pa_cache_append.  New blocks are acquired
 * when the tokens cross block boundaries.  If the sequence's last block is partly
 * filled and shared (reference count > 1), it is first replaced by a fresh block: the
 * pair (old, new) is written to copy_pairs_out (room for one pair) for
 * pa_copy_blocks, the old block loses this sequence's reference and table_row points
 * at the new block.  *num_copies_out gets 0 or 1.  PA_ERR_OUT_OF_BLOCKS when the pool
 * cannot supply the blocks; PA_ERR_INVALID_ARG when context_len + num_new exceeds
 * max_blocks * 16. */
pa_status pa_seq_reserve(pa_block_allocator *alloc, int32_t *table_row, int32_t max_blocks,
                         int32_t context_len, int32_t num_new, int32_t *slots_out,
                         int32_t *copy_pairs_out, int32_t *num_copies_out);

/* A new sequence sharing every block of another (a beam fork): dst_row gets
 * src_row's first ceil(context_len/16) entries, each block gains one reference, the
 * rest of dst_row (max_blocks entries) is set to -1. */
pa_status pa_seq_fork(pa_block_allocator *alloc, const int32_t *src_row, int32_t *dst_row,
                      int32_t max_blocks, int32_t context_len);

/* Shorten a sequence from context_len to new_len tokens (rolling back rejected
 * speculative tokens, or freeing a finished sequence with new_len = 0): the blocks
 * past ceil(new_len/16) lose this sequence's reference and their entries become -1. */
pa_status pa_seq_truncate(pa_block_allocator *alloc, int32_t *table_row, int32_t max_blocks,
                          int32_t context_len, int32_t new_len);

/* Static, human-readable text for a status code. */
const char *pa_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H */
