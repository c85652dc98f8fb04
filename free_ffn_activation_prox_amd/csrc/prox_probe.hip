// Read-stream probe: the HBM read rate a plain streaming kernel reaches on
// this GPU, the practical ceiling next to the 8 TB/s peak.  Not part of the
// forward; the bench calls it to put the forward's rate in context.
//
// Block b reads one contiguous part of the buffer, 8 KB per load round (512
// threads x 16 bytes), eight rounds in flight per thread (64 KB per block),
// and folds the words into one per thread so the loads stay live.
#include "prox.h"
#include "prox_device.hpp"
#include "prox_internal.hpp"

namespace prox {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 8;

__global__ void __launch_bounds__(kProbeThreads) k_read_probe(const uint4* __restrict__ src, size_t n16,
                                                              uint32_t* __restrict__ sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per, b1 = min(n16, b0 + per);
    uint32_t acc = 0;
    size_t i = b0 + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += kProbeUnroll * kProbeThreads) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * kProbeThreads];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < b1; i += kProbeThreads) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace prox

extern "C" prox_status prox_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
    if (!buf || !sink || blocks < 1 || bytes < 16 || (uintptr_t)buf % 16) return PROX_E_INVALID;
    hipLaunchKernelGGL(prox::k_read_probe, dim3(blocks), dim3(prox::kProbeThreads), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? PROX_OK : PROX_E_HIP;
}
