// Low-rank activation predictor + threshold + neuron-table compaction (gfx950).
//
// PowerInfer, "Adaptive Sparsity Predictors": each layer's predictor marks the
// neurons a token will fire, so the FFN touches only those.  The predictor
// here is the pair l = (x W_p1) W_p2 + b; a neuron is active when l > theta
// (theta = logit of the probability threshold).  "Neuron Placement and
// Management": the active neurons' original positions are written as an
// ascending int32 list.
//
// Both stages are memory-bound GEMVs (B small), so they are tiled for
// coalesced 16-byte loads with fp32 accumulation, not for MFMA:
//   stage 1  z[b, :] = x[b, :] W_p1     W_p1 [d, r] row-major.  Block = 64
//            columns x (32*KU) rows; the row chunks are split-K partials that
//            the last-arriving block of each column group sums in a fixed
//            order (deterministic).
//   stage 2  l[b, :] = z[b, :] W_p2 + b  W_p2 [r, F] row-major.  Block = 64
//            neurons x all r rows; one wave ballot turns 64 decisions into two
//            mask words; the last-arriving block compacts the whole mask.
#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

template <int NB, int KU>
__global__ __launch_bounds__(256) void k_pred_stage1(const uint16_t* __restrict__ x, int B,
                                                     const uint16_t* __restrict__ W1, int d, int r,
                                                     float* __restrict__ part,
                                                     float* __restrict__ z,
                                                     unsigned* __restrict__ counters) {
    __shared__ float s_red[4][NB][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = tid & 7;   // which 8-column piece of the group this lane loads
    const int rl = tid >> 3;   // row lane 0..31
    const int cg = blockIdx.x, chunk = blockIdx.y, nchunk = gridDim.y;
    const int col0 = cg * 64 + sub * 8;
    const bool colok = col0 < r;
    const int kbase = chunk * 32 * KU;

    uint4 w[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        const int k = kbase + rl + 32 * u;
        w[u] = (colok && k < d) ? ld16(W1 + (size_t)k * r + col0) : zero4();
    }

    for (int b0 = 0; b0 < B; b0 += NB) {
        float acc[NB][8];
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int k = kbase + rl + 32 * u;
            if (k < d) {
                const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int t = 0; t < NB; ++t) {
                    const float xv = (b0 + t < B) ? h2f(x[(size_t)(b0 + t) * d + k]) : 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[t][2 * e] = fmaf(xv, lo_f(ww[e]), acc[t][2 * e]);
                        acc[t][2 * e + 1] = fmaf(xv, hi_f(ww[e]), acc[t][2 * e + 1]);
                    }
                }
            }
        }
        // reduce over the 8 row lanes of this wave that share the columns (lane bits 3..5)
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = acc[t][e];
                v += __shfl_xor(v, 8);
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                acc[t][e] = v;
            }
        if (lane < 8) {
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_red[wave][t][lane * 8 + e] = acc[t][e];
        }
        __syncthreads();
        for (int i = tid; i < NB * 64; i += 256) {
            const int t = i >> 6, c = i & 63, col = cg * 64 + c;
            if (b0 + t < B && col < r) {
                const float v = ((s_red[0][t][c] + s_red[1][t][c]) + s_red[2][t][c]) + s_red[3][t][c];
                st_agent(&part[((size_t)chunk * B + b0 + t) * r + col], v);
            }
        }
        __syncthreads();
    }

    if (last_block_arrive(&counters[cg], (unsigned)nchunk)) {
        // z = sum over row chunks, in chunk order split into 4 interleaved runs, then combined
        const int c = tid & 63, qtr = tid >> 6, col = cg * 64 + c;
        for (int b = 0; b < B; ++b) {
            float s = 0.f;
            if (col < r) {
                // 16 partials in flight per thread, summed in chunk order
                for (int base = qtr; base < nchunk; base += 64) {
                    float v[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int ch = base + 4 * j;
                        v[j] = ch < nchunk ? ld_agent(&part[((size_t)ch * B + b) * r + col]) : 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < 16; ++j) s += v[j];
                }
            }
            s_red[qtr][0][c] = s;
            __syncthreads();
            if (qtr == 0 && col < r)
                z[(size_t)b * r + col] =
                    ((s_red[0][0][c] + s_red[1][0][c]) + s_red[2][0][c]) + s_red[3][0][c];
            __syncthreads();
        }
    }
}

template <int NB, int JU>
__global__ __launch_bounds__(256) void k_pred_stage2(const float* __restrict__ z, int B,
                                                     const uint16_t* __restrict__ W2,
                                                     const float* __restrict__ bias, int r, int F,
                                                     float theta, float* __restrict__ logits,
                                                     uint32_t* __restrict__ mask,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ count,
                                                     unsigned* __restrict__ counter) {
    __shared__ float s_red[4][NB][64];
    __shared__ int s_tmp[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = tid & 7, rl = tid >> 3;
    const int n0 = blockIdx.x * 64 + sub * 8;
    const bool nok = n0 < F;
    const int W = (F + 31) >> 5;

    for (int b0 = 0; b0 < B; b0 += NB) {
        float acc[NB][8];
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
        for (int j0 = 0; j0 < r; j0 += 32 * JU) {
            uint4 w[JU];
            float zv[JU][NB];
#pragma unroll
            for (int u = 0; u < JU; ++u) {
                const int j = j0 + rl + 32 * u;
                w[u] = (nok && j < r) ? ld16(W2 + (size_t)j * F + n0) : zero4();
#pragma unroll
                for (int t = 0; t < NB; ++t)
                    zv[u][t] = (j < r && b0 + t < B) ? z[(size_t)(b0 + t) * r + j] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < JU; ++u) {
                const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int t = 0; t < NB; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[t][2 * e] = fmaf(zv[u][t], lo_f(ww[e]), acc[t][2 * e]);
                        acc[t][2 * e + 1] = fmaf(zv[u][t], hi_f(ww[e]), acc[t][2 * e + 1]);
                    }
            }
        }
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = acc[t][e];
                v += __shfl_xor(v, 8);
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                acc[t][e] = v;
            }
        if (lane < 8) {
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_red[wave][t][lane * 8 + e] = acc[t][e];
        }
        __syncthreads();
        // wave t handles token b0 + t: lane = neuron within the 64-neuron tile
        for (int i = tid; i < NB * 64; i += 256) {
            const int t = i >> 6, nn = i & 63, neuron = blockIdx.x * 64 + nn;
            const int b = b0 + t;
            bool act = false;
            if (neuron < F && b < B) {
                const float l =
                    (((s_red[0][t][nn] + s_red[1][t][nn]) + s_red[2][t][nn]) + s_red[3][t][nn]) +
                    bias[neuron];
                act = l > theta;
                if (logits) logits[(size_t)b * F + neuron] = l;
            }
            const unsigned long long bal = __ballot(act);
            if (nn == 0 && b < B) {
                const int wd = blockIdx.x * 2;
                st_agent(&mask[(size_t)b * W + wd], (uint32_t)bal);
                if (wd + 1 < W) st_agent(&mask[(size_t)b * W + wd + 1], (uint32_t)(bal >> 32));
            }
        }
        __syncthreads();
    }

    if (idx != nullptr && last_block_arrive(counter, gridDim.x)) {
        for (int b = 0; b < B; ++b)
            block_compact<true>(mask + (size_t)b * W, 1, W, F, idx + (size_t)b * F, count + b, s_tmp);
    }
}

template <int NB>
hipError_t launch_stage1_ku(int ku, dim3 g, const uint16_t* x, int B, const uint16_t* W1, int d,
                            int r, float* part, float* z, unsigned* cnt, hipStream_t s) {
    switch (ku) {
        case 1: hipLaunchKernelGGL((k_pred_stage1<NB, 1>), g, dim3(256), 0, s, x, B, W1, d, r, part, z, cnt); break;
        case 2: hipLaunchKernelGGL((k_pred_stage1<NB, 2>), g, dim3(256), 0, s, x, B, W1, d, r, part, z, cnt); break;
        case 4: hipLaunchKernelGGL((k_pred_stage1<NB, 4>), g, dim3(256), 0, s, x, B, W1, d, r, part, z, cnt); break;
        default: hipLaunchKernelGGL((k_pred_stage1<NB, 8>), g, dim3(256), 0, s, x, B, W1, d, r, part, z, cnt); break;
    }
    return hipGetLastError();
}

}  // namespace

PredPlan plan_pred(int d, int r, int F, int B) {
    PredPlan p{};
    p.ncg = (r + 63) / 64;
    // at most 64 row chunks, so the last block of a column group sums 16 partials per thread
    p.ku = 1;
    while (p.ku < 8 && (d + 32 * p.ku - 1) / (32 * p.ku) > 64) p.ku *= 2;
    p.nchunk = (d + 32 * p.ku - 1) / (32 * p.ku);
    p.nb = B >= 8 ? 8 : (B >= 4 ? 4 : (B >= 2 ? 2 : 1));
    p.nblk2 = (F + 63) / 64;
    size_t off = COUNTER_BYTES;
    p.off_z = off;
    off = align_up(off + (size_t)B * r * sizeof(float), 256);
    p.off_part = off;
    off = align_up(off + (size_t)p.nchunk * B * r * sizeof(float), 256);
    p.bytes = off;
    return p;
}

hipError_t launch_predict(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x, int B,
                          float theta, float* logits, uint32_t* mask, int32_t* idx, int32_t* count,
                          char* ws, hipStream_t s) {
    unsigned* cnt = reinterpret_cast<unsigned*>(ws);
    float* z = reinterpret_cast<float*>(ws + pl.off_z);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    const dim3 g1(pl.ncg, pl.nchunk);
    hipError_t e;
    switch (pl.nb) {
        case 1: e = launch_stage1_ku<1>(pl.ku, g1, x, B, p.w_p1, p.d, p.r, part, z, cnt + CNT_PRED1, s); break;
        case 2: e = launch_stage1_ku<2>(pl.ku, g1, x, B, p.w_p1, p.d, p.r, part, z, cnt + CNT_PRED1, s); break;
        case 4: e = launch_stage1_ku<4>(pl.ku, g1, x, B, p.w_p1, p.d, p.r, part, z, cnt + CNT_PRED1, s); break;
        default: e = launch_stage1_ku<8>(pl.ku, g1, x, B, p.w_p1, p.d, p.r, part, z, cnt + CNT_PRED1, s); break;
    }
    if (e != hipSuccess) return e;
    const dim3 g2(pl.nblk2);
    switch (pl.nb) {
        case 1: hipLaunchKernelGGL((k_pred_stage2<1, 8>), g2, dim3(256), 0, s, z, B, p.w_p2, p.bias, p.r, p.F, theta, logits, mask, idx, count, cnt + CNT_PRED2); break;
        case 2: hipLaunchKernelGGL((k_pred_stage2<2, 8>), g2, dim3(256), 0, s, z, B, p.w_p2, p.bias, p.r, p.F, theta, logits, mask, idx, count, cnt + CNT_PRED2); break;
        case 4: hipLaunchKernelGGL((k_pred_stage2<4, 4>), g2, dim3(256), 0, s, z, B, p.w_p2, p.bias, p.r, p.F, theta, logits, mask, idx, count, cnt + CNT_PRED2); break;
        default: hipLaunchKernelGGL((k_pred_stage2<8, 4>), g2, dim3(256), 0, s, z, B, p.w_p2, p.bias, p.r, p.F, theta, logits, mask, idx, count, cnt + CNT_PRED2); break;
    }
    return hipGetLastError();
}

}  // namespace pi
