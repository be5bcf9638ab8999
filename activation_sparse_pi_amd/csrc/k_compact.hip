// Mask -> neuron table (PowerInfer, "Neuron Placement and Management": each
// kept neuron is mapped back to its position in the original matrix).
//
// One 1024-thread block per list: per token (grid = B) or the OR of the B
// token masks (grid = 1).  Integer-exact; output is ascending.
#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

__global__ __launch_bounds__(1024) void k_compact(const uint32_t* __restrict__ mask, int B, int F,
                                                  int union_mode, int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ count) {
    __shared__ int s_tmp[17];
    const int W = (F + 31) >> 5;
    if (union_mode) {
        block_compact<false>(mask, B, W, F, idx, count, s_tmp);
    } else {
        const int b = blockIdx.x;
        block_compact<false>(mask + (size_t)b * W, 1, W, F, idx + (size_t)b * F, count + b, s_tmp);
    }
}

__global__ __launch_bounds__(256) void k_zero(uint4* __restrict__ p, size_t n16, uint8_t* tail,
                                              int ntail) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_compact(const uint32_t* mask, int B, int F, int mode, int32_t* idx,
                          int32_t* count, hipStream_t s) {
    const int grid = mode == PI_UNION ? 1 : B;
    hipLaunchKernelGGL(k_compact, dim3(grid), dim3(1024), 0, s, mask, B, F,
                       mode == PI_UNION ? 1 : 0, idx, count);
    return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    const int ntail = (int)(bytes % 16);
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<uint4*>(p), n16,
                       reinterpret_cast<uint8_t*>(p) + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace pi
