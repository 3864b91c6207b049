// Read-only streaming kernel: the HBM read bandwidth a scan can reach on this
// device, measured beside the decode scan (which reads the index keys once).
// Built into its own small library; the layer's kernels do not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// Every block reads one contiguous span, 16 bytes per thread and step, eight
// steps in flight, with non-temporal loads (data read once; on this device
// the hint is worth about 15% of read bandwidth).  The values are folded into
// one word that is stored only if it equals a fixed pattern, so the loads
// cannot be removed and almost nothing is written.
__global__ void __launch_bounds__(256) k_read(const uint4* __restrict__ p, int64_t n16,
                                              uint32_t* __restrict__ sink) {
    typedef __attribute__((ext_vector_type(4))) unsigned int u4v;
    constexpr int U = 8;
    uint32_t acc = 0u;
    const int64_t per = n16 / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = blockIdx.x + 1 == gridDim.x ? n16 : lo + per;
    int64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * 256 < hi; i += U * 256) {
        u4v v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load((const u4v*)(p + i + u * 256));
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < hi; i += 256) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

// bytes: a multiple of 16; p: device memory of that size; sink: 4 bytes of device memory.
extern "C" int csa2_calib_read(const void* p, int64_t bytes, void* sink, int blocks,
                               void* stream) {
    if (!p || !sink || bytes < 16 || bytes % 16 || blocks < 1) return 1;
    hipLaunchKernelGGL(k_read, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)p, bytes / 16, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
