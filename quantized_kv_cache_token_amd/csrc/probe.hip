// probe.hip -- a streaming read of a large device buffer, the measure of the
// HBM bandwidth a read-only kernel reaches on this part (the context for the
// decode kernels' fractions of the 8 TB/s peak).  Each thread keeps four
// 16-byte loads in flight over a grid-stride loop and folds the words with
// xor; the fold is stored only if it equals a value it cannot be for the
// probe's input (a zero-filled buffer), so the loads stay while nothing is
// written.  NT: loads with the non-temporal hint.
#include "lkv_internal.h"

namespace lkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const u32x4* __restrict__ p, int64_t n, uint32_t* sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t x = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; u++) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4 v = NT ? __builtin_nontemporal_load(p + i) : p[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (x == 0x9E3779B9u) sink[0] = x;
}

hipError_t launch_hbm_read_probe(const void* buf, int64_t bytes, bool nontemporal, uint32_t* sink, hipStream_t stream)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess)
        return hipErrorInvalidDevice;
    const dim3 grid((unsigned)(cus * 8));
    const int64_t n = bytes / 16;
    if (nontemporal) hipLaunchKernelGGL(hbm_read_probe_kernel<true>, grid, dim3(256), 0, stream, (const u32x4*)buf, n, sink);
    else hipLaunchKernelGGL(hbm_read_probe_kernel<false>, grid, dim3(256), 0, stream, (const u32x4*)buf, n, sink);
    return hipGetLastError();
}

}  // namespace lkv
