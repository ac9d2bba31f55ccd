// pa_common.h -- types and launch declarations shared by the library's HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

constexpr int kBlock = 16;            // tokens per physical block
constexpr int kWave = 64;             // CDNA4 wavefront width

// Online softmax: the running max is moved only when a score exceeds it by more than
// this many doublings (exp2 domain), so weights stay <= 2^kRescaleSlack = 256.
constexpr float kRescaleSlack = 8.0f;

// Arguments of the decode partition kernel (by value, host -> kernel).
struct DecodeArgs {
    const void *k_pool;               // [num_blocks][hkv][16][D]
    const void *v_pool;               // [num_blocks][hkv][D][16]
    const void *q;                    // [B][hq][D]
    void *out;                        // [B][hq][D]           (single-pass mode)
    float *ws_o;                      // [B][hq][P][D]         (split mode)
    float *ws_m;                      // [B][hq][P]   running max, log2 domain
    float *ws_l;                      // [B][hq][P]   normaliser
    const int32_t *block_tables;      // [B][max_blocks]
    const int32_t *context_lens;      // [B]
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t group;                    // hq / hkv
    int32_t head_chunks;              // ceil(group / 16): 16-head chunks (reduce kernel)
    int32_t wg_heads;                 // q-heads one partition workgroup holds (16 x chunks)
    int32_t wg_chunks;                // ceil(group / wg_heads): workgroups per (seq, kv-head, part)
    int32_t max_blocks;
    int32_t max_context_len;
    int32_t part_blocks;              // blocks per partition
    int32_t num_parts;                // P (grid x)
    float scale_log2;                 // scale * log2(e) (* k_scale for fp8 pools)
    float v_scale;                    // multiplies the output (fp8 pools; else 1)
    int32_t split;                    // 1: write partials, 0: write out
    int32_t longest_first;            // 1: workgroup z takes the z-th longest sequence
    // Fused append (pa_decode_append): sequence b's new K/V row, token ctx-1, is
    // written into the pool and used for that token; null for plain decode.
    const void *k_new;                // [B][hkv][D], activation type
    const void *v_new;
    float k_quant;                    // fp8 pools: stored code = E4M3(x / scale)
    float v_quant;
    int32_t act_bf16;                 // fp8 pools: new rows are bf16 (else f16)
    // fp8 pools: per-kv-head scales ([hkv], device) or null.  A non-null k_head_scales
    // multiplies scale_log2 and replaces k_quant for its head (v likewise v_scale).
    const float *k_head_scales;
    const float *v_head_scales;
    // 1: no physical block appears in two sequences' tables, so K/V is streamed with
    // non-temporal loads; 0: ordinary loads, whose repeats the caches serve.
    int32_t stream_kv;
};

// Batches up to this size are dispatched longest sequence first.
constexpr int kLongestFirstMax = 256;

struct AppendArgs {
    void *k_pool;
    void *v_pool;
    const void *k_new;                // [T][hkv][D]
    const void *v_new;
    const int32_t *slot_mapping;      // [T]
    int32_t num_tokens;
    int32_t num_blocks;
    int32_t num_kv_heads;
    float k_scale;                    // fp8 pools: stored code = E4M3(x / scale)
    float v_scale;
    int32_t bf16;                     // fp8 pools: new rows are bf16 (else f16)
    const float *k_head_scales;       // fp8 pools: [hkv] per-head scales, or null
    const float *v_head_scales;
};

// The scale a kv-head's K (or V) uses: its per-head entry when the array is given,
// else the pool's.  A per-head value that is not finite and > 0 is returned as is;
// scale_ok() tells the kernels to poison that head.
__device__ __forceinline__ float head_scale(const float *per_head, float pool_scale, int head)
{
    return per_head ? per_head[head] : pool_scale;
}
__device__ __forceinline__ bool scale_ok(float s) { return s > 0.f && s <= 3.402823466e38f; }

// A float every lane of the wave holds alike, moved to a scalar register.
__device__ __forceinline__ float uniform(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// A global load of K/V.  With NT it carries the non-temporal hint (the `nt` cache-policy
// bit of the CDNA4 load): on MI355X a stream of such loads, each tile read once, moves
// 9-11 % faster than with ordinary loads (a 537 MB decode step: 84 against 94 us), but
// leaves nothing in the L2 or the last-level cache for another workgroup.  Ordinary
// loads serve blocks that several sequences share (their repeats hit in the caches),
// fp32 tiles (whose 16-byte pieces of one cache line arrive over several load
// instructions) and prefill (whose query tiles read each K/V tile again from the L2);
// each measured slower with the hint.
template <bool NT, typename T>
__device__ __forceinline__ T load_kv(const void *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
    else
        return *reinterpret_cast<const T *>(p);
}

// Launchers (return hipSuccess or the launch error).
// dtype: the pools' element type; act_dtype: q / out / new rows (== dtype except for
// fp8 pools, where it is f16 or bf16).
hipError_t launch_decode(int dtype, int act_dtype, int head_dim, const DecodeArgs &a,
                         int num_seqs, hipStream_t stream);
hipError_t launch_append(int dtype, int act_dtype, int head_dim, const AppendArgs &a,
                         hipStream_t stream);
hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                              int32_t num_blocks, size_t block_bytes, hipStream_t stream);

// Decode launch shape for 16-bit K/V with head_dim <= 128: waves per workgroup and
// blocks each wave keeps in flight ahead of the one it is computing.
#ifndef PA_WAVES
#define PA_WAVES 8
#endif
#ifndef PA_PREFETCH
#define PA_PREFETCH 1
#endif
constexpr int kWavesMain = PA_WAVES;
constexpr int kPrefetchMain = PA_PREFETCH;

// Waves per decode workgroup for a head dimension (the other shapes use 4).
constexpr int waves_per_group(int head_dim) { return head_dim <= 128 ? kWavesMain : 4; }

// 16-head chunks of a GQA group one decode workgroup serves.  One for groups up to 16
// q-heads, at head_dim 256 and for fp32 pools: the workgroup's waves walk different
// blocks, and a larger group runs one workgroup per 16 q-heads, whose K/V reads after
// the first come from the XCD's L2.  Above 16 q-heads at head_dim <= 128: for 16-bit
// pools the shared-tile kernel, 2 chunks up to 32 q-heads, else 4, each K/V tile
// staged once in LDS for all of them; for fp8 pools 2 chunks held by every wave of a
// partition workgroup as two MFMA column blocks over the same tile registers (each
// choice measured faster than the alternatives for its pool type).
constexpr int decode_chunks(int dtype, int head_dim, int group)
{
    return (head_dim > 128 || group <= 16 || dtype == DT_F32)
               ? 1
               : (dtype == DT_FP8 || group <= 32 ? 2 : 4);
}

// Whether those chunks share K/V tiles through LDS (the shared-tile kernel) rather than
// as the two column blocks of each wave of a partition workgroup.
constexpr bool decode_shared(int dtype, int head_dim, int group)
{
    return decode_chunks(dtype, head_dim, group) > 1 && (dtype == DT_F16 || dtype == DT_BF16);
}

// Blocks one decode workgroup walks side by side: its waves (partition kernel), or its
// block lanes (8 waves / chunks, shared-tile kernel).  A partition holds at most 64
// blocks per lane (a lane's block ids are one register, one per lane of the wave).
constexpr int decode_lanes(int dtype, int head_dim, int group)
{
    return decode_shared(dtype, head_dim, group) ? 8 / decode_chunks(dtype, head_dim, group)
                                                 : waves_per_group(head_dim);
}

// Fewest decode workgroups the partition choice aims for: one per CU of the MI355X.
#ifndef PA_TARGET_GROUPS
#define PA_TARGET_GROUPS 256
#endif
constexpr int kTargetGroups = PA_TARGET_GROUPS;

}  // namespace pa
