// Neuron placement on the device: applying a permutation to per-neuron arrays, and the neuron
// table that maps placed ids back to original ones (PowerInfer, "Neuron Placement and
// Management").  Both are plain copies: one pass over the bytes, coalesced.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

// dst row i = src row perm[i]; W bytes per thread (16, 4 or 1), upr units per row
template <int W>
__global__ __launch_bounds__(256) void k_permute_rows(const uint8_t* __restrict__ src,
                                                      uint8_t* __restrict__ dst,
                                                      const int32_t* __restrict__ perm, int n,
                                                      size_t row_bytes, long long upr) {
    const long long total = (long long)n * upr;
    for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < total;
         u += (long long)gridDim.x * 256) {
        const int i = (int)(u / upr);
        const size_t off = (size_t)(u - (long long)i * upr) * W;
        const int s = perm[i];
        uint8_t* q = dst + (size_t)i * row_bytes + off;
        if constexpr (W == 16) {
            *reinterpret_cast<uint4*>(q) = (unsigned)s < (unsigned)n
                ? *reinterpret_cast<const uint4*>(src + (size_t)s * row_bytes + off) : zero4();
        } else if constexpr (W == 4) {
            *reinterpret_cast<uint32_t*>(q) = (unsigned)s < (unsigned)n
                ? *reinterpret_cast<const uint32_t*>(src + (size_t)s * row_bytes + off) : 0u;
        } else {
            *q = (unsigned)s < (unsigned)n ? src[(size_t)s * row_bytes + off] : (uint8_t)0;
        }
    }
}

// out[b, k] = perm[idx[b, k]] for k < count[b]; one block per token
__global__ __launch_bounds__(256) void k_map_ids(const int32_t* idx,   // may be out itself
                                                 const int32_t* __restrict__ count, int F,
                                                 const int32_t* __restrict__ perm,
                                                 int32_t* out) {
    const int b = blockIdx.x;
    const int n = min(max(count[b], 0), F);
    for (int k = threadIdx.x; k < n; k += 256) {
        const int i = idx[(size_t)b * F + k];
        out[(size_t)b * F + k] = (unsigned)i < (unsigned)F ? perm[i] : -1;
    }
}

// counts[i] += number of the B masks (rows of W words) with bit i set, for i < F.  Thread
// = neuron; the 32 lanes of a word read it together (one broadcast load), and every row's
// word is issued before the first is used.
__global__ __launch_bounds__(256) void k_count_active(const uint32_t* __restrict__ mask, int B,
                                                      int F, int32_t* __restrict__ counts) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= F) return;
    const int W = (F + 31) >> 5, w = i >> 5, bit = i & 31;
    int c = 0;
    for (int b0 = 0; b0 < B; b0 += 8) {
        uint32_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = mask[(size_t)min(b0 + k, B - 1) * W + w];
#pragma unroll
        for (int k = 0; k < 8; ++k) c += (b0 + k < B) ? (int)((v[k] >> bit) & 1u) : 0;
    }
    counts[i] += c;
}

}  // namespace

hipError_t launch_count_active(const uint32_t* mask, int B, int F, int32_t* counts, hipStream_t s) {
    hipLaunchKernelGGL(k_count_active, dim3((F + 255) / 256), dim3(256), 0, s, mask, B, F, counts);
    return hipGetLastError();
}

hipError_t launch_permute_rows(const void* src, void* dst, const int32_t* perm, int n,
                               size_t row_bytes, hipStream_t s) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
    const int W = (row_bytes % 16 == 0 && a % 16 == 0) ? 16 : (row_bytes % 4 == 0 && a % 4 == 0) ? 4 : 1;
    const long long upr = (long long)(row_bytes / W);
    const long long total = (long long)n * upr;
    const int grid = (int)std::min<long long>(4096, (total + 255) / 256);
    const uint8_t* sp = static_cast<const uint8_t*>(src);
    uint8_t* dp = static_cast<uint8_t*>(dst);
    if (W == 16)
        hipLaunchKernelGGL(k_permute_rows<16>, dim3(grid), dim3(256), 0, s, sp, dp, perm, n, row_bytes, upr);
    else if (W == 4)
        hipLaunchKernelGGL(k_permute_rows<4>, dim3(grid), dim3(256), 0, s, sp, dp, perm, n, row_bytes, upr);
    else
        hipLaunchKernelGGL(k_permute_rows<1>, dim3(grid), dim3(256), 0, s, sp, dp, perm, n, row_bytes, upr);
    return hipGetLastError();
}

hipError_t launch_map_ids(const int32_t* idx, const int32_t* count, int B, int F,
                          const int32_t* perm, int32_t* out, hipStream_t s) {
    hipLaunchKernelGGL(k_map_ids, dim3(B), dim3(256), 0, s, idx, count, F, perm, out);
    return hipGetLastError();
}

}  // namespace pi
