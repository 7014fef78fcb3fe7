// Streaming-read ceiling of the device: a plain kernel that reads a byte
// range once with 16-byte lane loads (grid-stride, four loads in flight per
// lane) and folds the words into one value per workgroup so the loads are not
// dropped.  Used only to measure the sustained HBM read rate at the byte
// counts the layer's kernels move per launch; not part of the layer.
#include "common.h"
#include "internal.h"

namespace {

__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ buf, int64_t n16,
                                                     uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
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
    hipLaunchKernelGGL(k_stream_read, dim3(n_blocks), dim3(256), 0, st, static_cast<const uint4 *>(buf), bytes / 16,
                       sink);
    return hipGetLastError();
}

}  // namespace moe
