// pa_append.hip -- scatter new K/V rows (a decode step's, or a prompt chunk's) into the
// paged pool, and copy whole blocks for copy-on-write.
//
// Row i of k_new / v_new goes to slot s = slot_mapping[i]: physical block s / 16, row
// s % 16 (the page / offset split of "LLM应用 12 推理优化", PagedKVCache.update, and the
// fill-the-current-page rule of LLM-101-CN "推理优化", KVCachePool.write_tokens).
// Bytes are copied unchanged.  Negative slots are padding; slots past the pool are
// dropped so that no write ever leaves the pool.
//
// Fewer than 16 rows: one thread moves one 16-byte chunk of one (token, kv-head) row:
// a single 16-byte store into the token-major K block, and 16/elem scalar stores into
// the token-minor V block (stride 16 elements).  16 rows or more: groups of 16 rows,
// a whole in-order block written block-wise (see the group kernel).
//
// An fp8 pool stores OCP E4M3 codes of x / scale (the KV-cache write fused with its
// quantisation, one of the fused kernels "Deep dive into vLLM 06" lists): the
// division is IEEE fp32, the code rounds to nearest-even and saturates at 448.  The
// scale is the row's kv-head entry of a per-head array when the pool has one, else the
// pool's; a per-head scale that is not finite and > 0 stores NaN codes.
#include <type_traits>

#include "pa_common.h"
#include "pa_fp8.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int EB, int D>
__global__ __launch_bounds__(256) void pa_cache_append_kernel(AppendArgs a)
{
    constexpr int EPC = 16 / EB;              // elements per 16-byte chunk
    constexpr int CPR = D / EPC;              // chunks per row
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)a.num_tokens * a.num_kv_heads * CPR;
    if (idx >= total)
        return;
    const int c = (int)(idx % CPR);
    const size_t row = idx / CPR;              // token * hkv + head
    const int h = (int)(row % a.num_kv_heads);
    const int i = (int)(row / a.num_kv_heads);
    // The row data and the slot are independent loads: issue all three before the
    // slot decides whether (and where) to store.
    const u32x4 kv = *reinterpret_cast<const u32x4 *>(
        static_cast<const char *>(a.k_new) + (row * D + (size_t)c * EPC) * EB);
    const u32x4 vv = *reinterpret_cast<const u32x4 *>(
        static_cast<const char *>(a.v_new) + (row * D + (size_t)c * EPC) * EB);
    const int32_t slot = a.slot_mapping[i];
    if (slot < 0 || (int64_t)slot >= (int64_t)a.num_blocks * kBlock)
        return;
    const size_t blk = (size_t)(slot / kBlock);
    const int off = slot % kBlock;
    const size_t tile = (blk * a.num_kv_heads + h) * (size_t)kBlock * D;   // element offset

    char *kdst = static_cast<char *>(a.k_pool) + (tile + (size_t)off * D + (size_t)c * EPC) * EB;
    *reinterpret_cast<u32x4 *>(kdst) = kv;
    char *vdst = static_cast<char *>(a.v_pool) + (tile + (size_t)c * EPC * kBlock + off) * EB;
    if constexpr (EB == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            reinterpret_cast<uint32_t *>(vdst)[j * kBlock] = vv[j];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            reinterpret_cast<uint16_t *>(vdst)[(2 * j) * kBlock] = (uint16_t)(vv[j] & 0xFFFFu);
            reinterpret_cast<uint16_t *>(vdst)[(2 * j + 1) * kBlock] = (uint16_t)(vv[j] >> 16);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void pa_cache_append_fp8_kernel(AppendArgs a)
{
    constexpr int CPR = D / 8;                // 8 elements (16 bytes of f16/bf16) per thread
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)a.num_tokens * a.num_kv_heads * CPR;
    if (idx >= total)
        return;
    const int c = (int)(idx % CPR);
    const size_t row = idx / CPR;
    const int h = (int)(row % a.num_kv_heads);
    const int i = (int)(row / a.num_kv_heads);
    const u32x4 kv = *reinterpret_cast<const u32x4 *>(
        static_cast<const uint16_t *>(a.k_new) + row * D + (size_t)c * 8);
    const u32x4 vv = *reinterpret_cast<const u32x4 *>(
        static_cast<const uint16_t *>(a.v_new) + row * D + (size_t)c * 8);
    const int32_t slot = a.slot_mapping[i];
    if (slot < 0 || (int64_t)slot >= (int64_t)a.num_blocks * kBlock)
        return;
    const size_t blk = (size_t)(slot / kBlock);
    const int off = slot % kBlock;
    const size_t tile = (blk * a.num_kv_heads + h) * (size_t)kBlock * D;   // bytes
    const float ks = head_scale(a.k_head_scales, a.k_scale, h);
    const float vs = head_scale(a.v_head_scales, a.v_scale, h);
    uint32_t kc[2] = {0u, 0u};
    uint8_t *vdst = static_cast<uint8_t *>(a.v_pool) + tile + (size_t)c * 8 * kBlock + off;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t kw = (kv[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t vw = (vv[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
        const float kx = a.bf16 ? __uint_as_float(kw << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)kw);
        const float vx = a.bf16 ? __uint_as_float(vw << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)vw);
        kc[j / 4] |= e4m3_scaled(kx, ks) << (8 * (j & 3));
        vdst[j * kBlock] = (uint8_t)e4m3_scaled(vx, vs);
    }
    *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(a.k_pool) + tile + (size_t)off * D +
                               (size_t)c * 8) = make_uint2(kc[0], kc[1]);
}

// Eight consecutive pool elements (a run 8 x element-size bytes long and as aligned)
// written with whole-run vector stores.
template <typename Out>
__device__ __forceinline__ void store_run(Out *dst, const Out (&run)[8])
{
    if constexpr (sizeof(Out) == 1) {
        u32x2 w;
        __builtin_memcpy(&w, run, sizeof(w));
        *reinterpret_cast<u32x2 *>(dst) = w;
    } else {
#pragma unroll
        for (int h = 0; h < (int)sizeof(run) / 16; ++h) {
            u32x4 w;
            __builtin_memcpy(&w, reinterpret_cast<const char *>(run) + 16 * h, sizeof(w));
            reinterpret_cast<u32x4 *>(dst)[h] = w;
        }
    }
}

// Groups of 16 consecutive new rows, one workgroup per (group, kv-head).  A group whose
// 16 slots are one whole block in order (a prompt chunk being ingested) writes that
// block's K rows contiguously and its V^T rows whole: the 16 rows are staged in LDS and
// each store covers 8 consecutive tokens of one V^T row, so no store is a partial-sector
// write.  Any other group writes each row's K pieces to its slot and its V^T elements
// with lanes along the token axis (rows of one block that follow each other coalesce).
// fp8 pools store E4M3(x / scale).
template <int DT, int AT, int D>
__global__ __launch_bounds__(256) void pa_cache_append_group_kernel(AppendArgs a)
{
    using In = typename std::conditional<AT == DT_F32, float, uint16_t>::type;
    using Out = typename std::conditional<DT == DT_F32, float,
                typename std::conditional<DT == DT_FP8, uint8_t, uint16_t>::type>::type;
    constexpr int PC = D / 8;                   // 8-element pieces per row
    __shared__ int s_slot[kBlock];
    __shared__ In s_v[kBlock][D + 8];
    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int i0 = blockIdx.x * kBlock;
    const int n = min(kBlock, a.num_tokens - i0);
    if (tid < kBlock)
        s_slot[tid] = tid < n ? a.slot_mapping[i0 + tid] : -1;
    __syncthreads();
    const int s0 = s_slot[0];
    bool whole = n == kBlock && s0 >= 0 && s0 % kBlock == 0 &&
                 (int64_t)s0 < (int64_t)a.num_blocks * kBlock;
#pragma unroll
    for (int j = 1; j < kBlock; ++j)
        whole = whole && s_slot[j] == s0 + j;

    // fp8 pools: this kv-head's scales (per-head arrays, else the pool's)
    const float ks = DT == DT_FP8 ? head_scale(a.k_head_scales, a.k_scale, h) : 1.f;
    const float vs = DT == DT_FP8 ? head_scale(a.v_head_scales, a.v_scale, h) : 1.f;
    auto conv = [&](In x, float scale) -> Out {
        if constexpr (DT == DT_FP8)
            return (Out)e4m3_of_16(x, a.bf16 != 0, scale);
        else
            return (Out)x;
    };
    const In *kin = static_cast<const In *>(a.k_new);
    const In *vin = static_cast<const In *>(a.v_new);
    Out *kpool = static_cast<Out *>(a.k_pool);
    Out *vpool = static_cast<Out *>(a.v_pool);

    if (whole) {
        const size_t tile = ((size_t)(s0 / kBlock) * a.num_kv_heads + h) * kBlock * D;
        for (int c = tid; c < kBlock * PC; c += blockDim.x) {
            const int j = c / PC, col = (c % PC) * 8;
            const size_t src = ((size_t)(i0 + j) * a.num_kv_heads + h) * D + col;
            In kx[8], vx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kx[e] = kin[src + e];
                vx[e] = vin[src + e];
            }
            Out run[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                run[e] = conv(kx[e], ks);
                s_v[j][col + e] = vx[e];
            }
            store_run(kpool + tile + (size_t)j * D + col, run);
        }
        __syncthreads();
        for (int c = tid; c < D * 2; c += blockDim.x) {
            const int d = c / 2, t0 = (c % 2) * 8;
            // tokens t0 .. t0+7 of V^T row d: one contiguous run
            Out run[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                run[e] = conv(s_v[t0 + e][d], vs);
            store_run(vpool + tile + (size_t)d * kBlock + t0, run);
        }
        return;
    }
    // Any other group: K row pieces go straight to their slots; V rows are staged in
    // LDS and written with lanes along the token axis, so the rows of one block that
    // follow each other in the group land as one run of V^T row d.
    const int64_t slots = (int64_t)a.num_blocks * kBlock;
    for (int c = tid; c < n * PC; c += blockDim.x) {
        const int j = c / PC, col = (c % PC) * 8;
        const size_t src = ((size_t)(i0 + j) * a.num_kv_heads + h) * D + col;
        In kx[8], vx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kx[e] = kin[src + e];
            vx[e] = vin[src + e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s_v[j][col + e] = vx[e];
        const int slot = s_slot[j];
        if (slot < 0 || (int64_t)slot >= slots)
            continue;
        Out run[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            run[e] = conv(kx[e], ks);
        const size_t tile = ((size_t)(slot / kBlock) * a.num_kv_heads + h) * kBlock * D;
        store_run(kpool + tile + (size_t)(slot % kBlock) * D + col, run);
    }
    __syncthreads();
    for (int c = tid; c < D * kBlock; c += blockDim.x) {
        const int d = c / kBlock, j = c % kBlock;
        const int slot = s_slot[j];               // -1 past the last row
        if (slot < 0 || (int64_t)slot >= slots)
            continue;
        const size_t tile = ((size_t)(slot / kBlock) * a.num_kv_heads + h) * kBlock * D;
        vpool[tile + (size_t)d * kBlock + slot % kBlock] = conv(s_v[j][d], vs);
    }
}

template <int DT, int AT, int D>
hipError_t launch_append_group_t(const AppendArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)(((int64_t)a.num_tokens + kBlock - 1) / kBlock), a.num_kv_heads);
    hipLaunchKernelGGL((pa_cache_append_group_kernel<DT, AT, D>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_append_fp8_t(const AppendArgs &a, hipStream_t stream)
{
    const size_t total = (size_t)a.num_tokens * a.num_kv_heads * (D / 8);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL((pa_cache_append_fp8_kernel<D>), dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int EB, int D>
hipError_t launch_append_t(const AppendArgs &a, hipStream_t stream)
{
    constexpr int CPR = D * EB / 16;
    const size_t total = (size_t)a.num_tokens * a.num_kv_heads * CPR;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL((pa_cache_append_kernel<EB, D>), dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Copies whole physical blocks (every kv-head of K and of V) for (src, dst) pairs: the
// copy half of copy-on-write.  A block of either pool is one contiguous run of
// block_bytes bytes; a thread moves one 16-byte unit of each pool.  Pairs with an id
// outside the pool are skipped.
__global__ __launch_bounds__(256) void pa_copy_blocks_kernel(void *k_pool, void *v_pool,
                                                             const int32_t *pairs,
                                                             int32_t num_blocks,
                                                             size_t block_bytes)
{
    const int32_t src = pairs[2 * blockIdx.y];
    const int32_t dst = pairs[2 * blockIdx.y + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
        return;
    const size_t units = block_bytes / 16;
    for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (size_t)gridDim.x * blockDim.x) {
        const size_t so = (size_t)src * block_bytes + u * 16;
        const size_t d = (size_t)dst * block_bytes + u * 16;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(k_pool) + so);
        const u32x4 vv = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(v_pool) + so);
        // the copies are written once and read by a later launch: non-temporal stores
        // (1,024 pairs of 32 KB blocks, no cache reuse between launches: 22.7 us against
        // 30.4 us with ordinary stores; non-temporal loads as well measured slower)
        __builtin_nontemporal_store(kv, reinterpret_cast<u32x4 *>(static_cast<char *>(k_pool) + d));
        __builtin_nontemporal_store(vv, reinterpret_cast<u32x4 *>(static_cast<char *>(v_pool) + d));
    }
}

}  // namespace

hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                              int32_t num_blocks, size_t block_bytes, hipStream_t stream)
{
    const size_t units = block_bytes / 16;
    const unsigned gx = (unsigned)((units + 255) / 256 < 64 ? (units + 255) / 256 : 64);
    hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3(gx, num_pairs), dim3(256), 0, stream, k_pool,
                       v_pool, pairs, num_blocks, block_bytes);
    return hipGetLastError();
}

hipError_t launch_append(int dtype, int act_dtype, int head_dim, const AppendArgs &a,
                         hipStream_t stream)
{
    // 16 rows or more (a prompt chunk): groups of 16, whole blocks written whole
    if (a.num_tokens >= kBlock && a.num_kv_heads <= 65535) {
        AppendArgs b = a;
        b.bf16 = act_dtype == DT_BF16 ? 1 : 0;
#define PA_AG_CASE(DT, AT, D)                                                      \
        if (dtype == DT && act_dtype == AT && head_dim == D)                      \
            return launch_append_group_t<DT, AT, D>(b, stream);
        PA_AG_CASE(DT_F32, DT_F32, 64)
        PA_AG_CASE(DT_F32, DT_F32, 128)
        PA_AG_CASE(DT_F16, DT_F16, 64)
        PA_AG_CASE(DT_F16, DT_F16, 128)
        PA_AG_CASE(DT_F16, DT_F16, 256)
        PA_AG_CASE(DT_BF16, DT_BF16, 64)
        PA_AG_CASE(DT_BF16, DT_BF16, 128)
        PA_AG_CASE(DT_BF16, DT_BF16, 256)
        PA_AG_CASE(DT_FP8, DT_F16, 64)
        PA_AG_CASE(DT_FP8, DT_F16, 128)
        PA_AG_CASE(DT_FP8, DT_F16, 256)
        PA_AG_CASE(DT_FP8, DT_BF16, 64)
        PA_AG_CASE(DT_FP8, DT_BF16, 128)
        PA_AG_CASE(DT_FP8, DT_BF16, 256)
#undef PA_AG_CASE
        return hipErrorInvalidValue;
    }
    if (dtype == DT_FP8) {
        if (act_dtype != DT_F16 && act_dtype != DT_BF16)
            return hipErrorInvalidValue;
        AppendArgs b = a;
        b.bf16 = act_dtype == DT_BF16 ? 1 : 0;
        switch (head_dim) {
        case 64: return launch_append_fp8_t<64>(b, stream);
        case 128: return launch_append_fp8_t<128>(b, stream);
        case 256: return launch_append_fp8_t<256>(b, stream);
        default: return hipErrorInvalidValue;
        }
    }
    const int eb = dtype == DT_F32 ? 4 : 2;
    switch (eb * 1000 + head_dim) {
    case 4064: return launch_append_t<4, 64>(a, stream);
    case 4128: return launch_append_t<4, 128>(a, stream);
    case 2064: return launch_append_t<2, 64>(a, stream);
    case 2128: return launch_append_t<2, 128>(a, stream);
    case 2256: return launch_append_t<2, 256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
