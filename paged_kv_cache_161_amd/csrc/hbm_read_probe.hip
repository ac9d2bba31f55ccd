// Measurement helper, not part of the attention path: a plain HBM read kernel whose
// rate is the practical ceiling a streaming kernel can reach on this device.  Each
// thread reads 16 bytes per iteration in a grid-stride loop, with the non-temporal
// hint (on MI355X the faster way to stream data that is read once: 7.2 against
// 6.4 TB/s over 2 GiB with ordinary loads), and folds them with XOR;
// the fold result is stored only when it equals a constant no input here produces, so
// the loads stay (a buffer of repeated bytes, as the benchmark fills it, folds to 0 or
// to that byte repeated, never to the constant).  Built into its own small library and
// called by the benchmark only.
//
//   int32_t pa_probe_read(const void *buf, size_t bytes, uint32_t *sink,
//                         int32_t workgroups, void *stream);
//
// buf: device memory of `bytes` bytes (a multiple of 16, 16-byte aligned); sink: one
// device uint32 (written only if the fold equals the constant); workgroups: grid size (256
// threads each); stream: a hipStream_t or null.  Returns 0, or -1 on a bad argument,
// or the HIP error of the launch.  Asynchronous on the stream.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4 *__restrict__ p, size_t n,
                                                       uint32_t *sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u)   // data-dependent, so the compiler keeps every load
        sink[0] = acc;
}

}  // namespace

extern "C" int32_t pa_probe_read(const void *buf, size_t bytes, uint32_t *sink,
                                 int32_t workgroups, void *stream)
{
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0 || workgroups <= 0)
        return -1;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf),
                       bytes / 16, sink);
    return (int32_t)hipGetLastError();
}
