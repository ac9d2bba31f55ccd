// pa_append.hip -- scatter a decode step's new K/V rows into the paged pool.
//
// Row i of k_new / v_new goes to slot s = slot_mapping[i]: physical block s / 16, row
// s % 16 (the page / offset split of "LLM应用 12 推理优化", PagedKVCache.update, and the
// fill-the-current-page rule of LLM-101-CN "推理优化", KVCachePool.write_tokens).
// Bytes are copied unchanged.  Negative slots are padding; slots past the pool are
// dropped so that no write ever leaves the pool.
//
// One thread moves one 16-byte chunk of one (token, kv-head) row: a single 16-byte
// store into the token-major K block, and 16/elem scalar stores into the token-minor
// V block (stride 16 elements).
#include "pa_common.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

template <int EB, int D>
hipError_t launch_append_t(const AppendArgs &a, hipStream_t stream)
{
    constexpr int CPR = D * EB / 16;
    const size_t total = (size_t)a.num_tokens * a.num_kv_heads * CPR;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL((pa_cache_append_kernel<EB, D>), dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int dtype, int head_dim, const AppendArgs &a, hipStream_t stream)
{
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
