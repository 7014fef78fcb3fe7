// Streaming-read ceiling of the device: a plain kernel that reads a byte
// range once with 16-byte lane loads (grid-stride, up to eight loads in
// flight per lane) and folds the words into one value per workgroup so the loads are not
// dropped.  Used only to measure the sustained HBM read rate at the byte
// counts the layer's kernels move per launch; not part of the layer.
#include "common.h"
#include "internal.h"

namespace {

template <int U>
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ buf, int64_t n16,
                                                     uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // one value per workgroup: lane 0 of each wave folds in with an atomic on the workgroup's word
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x], acc);
}

}  // namespace

namespace moe {

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int n_blocks, hipStream_t st) {
    const int64_t n16 = bytes / 16, per_thread = n16 / ((int64_t)n_blocks * 256);
    // as many loads in flight per lane as each lane has to issue, up to 8
    if (per_thread >= 8)
        hipLaunchKernelGGL(k_stream_read<8>, dim3(n_blocks), dim3(256), 0, st, static_cast<const uint4 *>(buf), n16, sink);
    else if (per_thread >= 4)
        hipLaunchKernelGGL(k_stream_read<4>, dim3(n_blocks), dim3(256), 0, st, static_cast<const uint4 *>(buf), n16, sink);
    else
        hipLaunchKernelGGL(k_stream_read<2>, dim3(n_blocks), dim3(256), 0, st, static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace moe
