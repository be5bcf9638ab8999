// Batch-1 neuron-aware FFN on gfx950 (PowerInfer, "Neuron-aware Operator":
// work on single row vectors of up/gate and single column vectors of down, read
// in place from the dense neuron-major matrices, no sparse-format conversion).
//
//   up   h[k] = act(W_up[i_k] . x [, W_gate[i_k] . x])   for k < count, i_k = idx[k]
//        One wave per listed neuron.  Lane l owns the 16-byte chunks l, l+64, ...
//        of every row, so its slice of x is loaded once into registers and reused
//        for every neuron the wave handles; every weight byte is read once with a
//        coalesced 16-byte load; the dot product is a 64-lane reduction.
//   down y = sum_k h[k] W_down[i_k, :]
//        2-D tiling: a block owns one column slice (512 fp16 / 2048 int4 columns,
//        one 16-byte chunk per lane) and one neuron split.  Waves of the block
//        take interleaved neurons, sum in registers, combine through LDS, and
//        write one partial row per block; the last-arriving block of each slice
//        adds the partials in split order (deterministic, no float atomics).
//
// int4 group-128 (LLM Runtime page, "01 LLM Runtime"): stored nibble u, value
// (u - 8) * s.  Up: nibbles are widened to fp16 pairs exactly by OR-ing them
// into the mantissa of 1024.0 and subtracting 1032, then dotted with x by
// v_dot2_f32_f16; the per-chunk sum (32 weights, always inside one group) is
// scaled once.  Down: h*s is formed once per neuron and chunk, nibbles are
// converted byte-wise to float, and the -8 offset is applied once at the end
// through the running sum of h*s.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

// ------------------------------------------------------------------------------------------ fp16 up
template <int Q, bool GLU>
__global__ __launch_bounds__(256) void k_up_f16(const uint16_t* __restrict__ x,
                                                const uint16_t* __restrict__ Wg,
                                                const uint16_t* __restrict__ Wu, int d, int F,
                                                const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ count, int dense_F,
                                                float* __restrict__ h) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nw = gridDim.x * 4;
    const int n = dense_F > 0 ? dense_F : min(*count, F);
    if (gw >= n) return;
    const int nc = d >> 3;
    uint4 xr[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = lane + 64 * q;
        xr[q] = c < nc ? ld16(x + 8 * c) : zero4();
    }
    for (int k = gw; k < n; k += nw) {
        const int irow = dense_F > 0 ? k : idx[k];
        if ((unsigned)irow >= (unsigned)F) {   // not a neuron of this layer: contributes 0
            if (lane == 0) h[k] = 0.f;
            continue;
        }
        const size_t row = (size_t)irow;
        const uint16_t* pu = Wu + row * d;
        const uint16_t* pg = GLU ? Wg + row * d : nullptr;
        uint4 wu[Q], wg[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = lane + 64 * q;
            wu[q] = c < nc ? ld16(pu + 8 * c) : zero4();
            if (GLU) wg[q] = c < nc ? ld16(pg + 8 * c) : zero4();
        }
        float au = 0.f, ag = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            au = dot8(wu[q], xr[q], au);
            if (GLU) ag = dot8(wg[q], xr[q], ag);
        }
        au = wave_sum(au);
        if (GLU) ag = wave_sum(ag);
        if (lane == 0) h[k] = GLU ? fmaxf(ag, 0.f) * au : fmaxf(au, 0.f);
    }
}

// ------------------------------------------------------------------------------------------ int4 up
template <int Q, bool GLU>
__global__ __launch_bounds__(256) void k_up_i4(const uint16_t* __restrict__ x,
                                               const uint8_t* __restrict__ Gq,
                                               const uint16_t* __restrict__ Gs,
                                               const uint8_t* __restrict__ Uq,
                                               const uint16_t* __restrict__ Us, int d, int F,
                                               const int32_t* __restrict__ idx,
                                               const int32_t* __restrict__ count, int dense_F,
                                               float* __restrict__ h) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nw = gridDim.x * 4;
    const int n = dense_F > 0 ? dense_F : min(*count, F);
    if (gw >= n) return;
    const int nc = d >> 5;      // 16-byte chunks (32 weights) per row
    const int G = d >> 7;       // scale groups per row
    const size_t rb = (size_t)(d >> 1);
    // x slice of each chunk, regrouped so pair p of word m is (x[8m+p], x[8m+p+4]),
    // matching the nibble pairs (bits 4p and 16+4p) that one AND/OR extracts
    uint32_t xp[Q][16];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = lane + 64 * q;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4 a = c < nc ? ld16(x + 32 * c + 8 * m) : zero4();
            xp[q][4 * m + 0] = (a.x & 0xFFFFu) | (a.z << 16);
            xp[q][4 * m + 1] = (a.x >> 16) | (a.z & 0xFFFF0000u);
            xp[q][4 * m + 2] = (a.y & 0xFFFFu) | (a.w << 16);
            xp[q][4 * m + 3] = (a.y >> 16) | (a.w & 0xFFFF0000u);
        }
    }
    for (int k = gw; k < n; k += nw) {
        const int irow = dense_F > 0 ? k : idx[k];
        if ((unsigned)irow >= (unsigned)F) {
            if (lane == 0) h[k] = 0.f;
            continue;
        }
        const size_t row = (size_t)irow;
        uint4 wu[Q], wg[Q];
        uint32_t su[Q], sg[Q];   // raw fp16 scales, one per register
        // unconditional loads (chunk 0 where a lane has nothing to read, discarded at use):
        // a branch-guarded load is waited for at the end of its branch
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = lane + 64 * q;
            const int cc = c < nc ? c : 0;
            wu[q] = ld16(Uq + row * rb + 16 * cc);
            su[q] = Us[row * G + (cc >> 2)];
            if (GLU) {
                wg[q] = ld16(Gq + row * rb + 16 * cc);
                sg[q] = Gs[row * G + (cc >> 2)];
            }
        }
        float au = 0.f, ag = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (lane + 64 * q < nc) {
                au = fmaf(dot32_i4(wu[q], xp[q]), h2f((uint16_t)su[q]), au);
                if (GLU) ag = fmaf(dot32_i4(wg[q], xp[q]), h2f((uint16_t)sg[q]), ag);
            }
        }
        au = wave_sum(au);
        if (GLU) ag = wave_sum(ag);
        if (lane == 0) h[k] = GLU ? fmaxf(ag, 0.f) * au : fmaxf(au, 0.f);
    }
}

// ------------------------------------------------------------------------------------------ fp16 down
constexpr int DOWN_WAVES_F16 = 16;
constexpr int DOWN_WAVES_I4 = 8;

// G > 0: idx lists groups of G consecutive rows (list entry j stands for rows idx[j] G ..
// idx[j] G + G - 1, *count entries) and h is indexed by row; otherwise h[k] goes with idx[k].
template <int U>
__global__ __launch_bounds__(1024) void k_down_f16(const uint16_t* __restrict__ Wd, int d, int F,
                                                   const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ count, int dense_F,
                                                   int G, const float* __restrict__ h,
                                                   float* __restrict__ part, float* __restrict__ y,
                                                   unsigned* __restrict__ counters) {
    constexpr int NW = DOWN_WAVES_F16;
    __shared__ float4 s_red[NW][128];   // [wave][column / 4] over the 512-column slice
    __shared__ float s_half[512];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slice = blockIdx.x, split = blockIdx.y, nsplit = gridDim.y;
    const int nc = d >> 3;
    const int c = slice * 64 + lane;
    const bool cok = c < nc;
    const int n = dense_F > 0 ? dense_F : G > 0 ? min(*count, F / G) * G : min(*count, F);
    const int stride = nsplit * NW;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int k0 = split * NW + wave; k0 < n; k0 += stride * U) {
        uint4 w[U];
        float hv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * stride;
            int irow = -1;
            if (kk < n) {
                if (dense_F > 0) {
                    irow = kk;
                } else if (G > 0) {
                    const int j = kk / G, g = idx[j];
                    irow = (unsigned)g < (unsigned)(F / G) ? g * G + (kk - j * G) : -1;
                } else {
                    irow = idx[kk];
                }
            }
            if ((unsigned)irow < (unsigned)F) {
                hv[u] = h[G > 0 ? irow : kk];
                w[u] = cok ? ld16(Wd + (size_t)irow * d + 8 * c) : zero4();
            } else {
                hv[u] = 0.f;
                w[u] = zero4();
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = fmaf(hv[u], lo_f(ww[e]), acc[2 * e]);
                acc[2 * e + 1] = fmaf(hv[u], hi_f(ww[e]), acc[2 * e + 1]);
            }
        }
    }
    s_red[wave][2 * lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    s_red[wave][2 * lane + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    __syncthreads();
    // 1024 threads over 512 columns: half hf sums waves [8 hf, 8 hf + 8)
    const int col = tid & 511, hf = tid >> 9;
    const float* sr = reinterpret_cast<const float*>(s_red);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW / 2; ++w) s += sr[(hf * (NW / 2) + w) * 512 + col];
    if (hf == 1) s_half[col] = s;
    __syncthreads();
    const int gcol = slice * 512 + col;
    if (hf == 0 && gcol < d) st_agent(&part[(size_t)split * d + gcol], s + s_half[col]);
    if (last_block_arrive(&counters[slice], (unsigned)nsplit)) {
        float t = 0.f;
        if (gcol < d) {
            for (int base = hf; base < nsplit; base += 32) {   // 16 partials in flight
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int sp = base + 2 * j;
                    v[j] = sp < nsplit ? ld_agent(&part[(size_t)sp * d + gcol]) : 0.f;
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) t += v[j];
            }
        }
        __syncthreads();
        if (hf == 1) s_half[col] = t;
        __syncthreads();
        if (hf == 0 && gcol < d) y[gcol] = t + s_half[col];
    }
}

// ------------------------------------------------------------------------------------------ int4 down
template <int U>
__global__ __launch_bounds__(512) void k_down_i4(const uint8_t* __restrict__ Dq,
                                                 const uint16_t* __restrict__ Ds, int d, int F,
                                                 const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ count, int dense_F,
                                                 const float* __restrict__ h,
                                                 float* __restrict__ part, float* __restrict__ y,
                                                 unsigned* __restrict__ counters) {
    constexpr int NW = DOWN_WAVES_I4;
    __shared__ float4 s_red[NW][512];   // [wave][column / 4] over the 2048-column slice
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slice = blockIdx.x, split = blockIdx.y, nsplit = gridDim.y;
    const int nc = d >> 5;
    const int G = d >> 7;
    const size_t rb = (size_t)(d >> 1);
    const int c = slice * 64 + lane;
    const bool cok = c < nc;
    const int n = dense_F > 0 ? dense_F : min(*count, F);
    const int stride = nsplit * NW;
    float acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.f;
    for (int k0 = split * NW + wave; k0 < n; k0 += stride * U) {
        uint4 w[U];
        float hr[U];
        uint32_t sr[U];          // raw fp16 scales, one per register
        bool ok[U];
        // unconditional loads (row 0 / column 0 where there is nothing to read, zeroed at
        // use): a branch-guarded load is waited for at the end of its branch
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * stride;
            const bool in = kk < n;
            const int irow = in ? (dense_F > 0 ? kk : idx[kk]) : 0;
            ok[u] = in && cok && (unsigned)irow < (unsigned)F;
            const size_t row = ok[u] ? (size_t)irow : 0;
            const int cc = cok ? c : 0;
            w[u] = ld16(Dq + row * rb + 16 * cc);
            sr[u] = Ds[row * G + (cc >> 2)];
            hr[u] = h[in ? kk : 0];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k0 + u * stride >= n) continue;        // empty slots: loaded, never used
            const float hsu = ok[u] ? hr[u] * h2f((uint16_t)sr[u]) : 0.f;
            axpy8_i4(acc, w[u].x, hsu, hsu * 0.0625f);
            axpy8_i4(acc + 8, w[u].y, hsu, hsu * 0.0625f);
            axpy8_i4(acc + 16, w[u].z, hsu, hsu * 0.0625f);
            axpy8_i4(acc + 24, w[u].w, hsu, hsu * 0.0625f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            keep(w[u]);
            keep(sr[u]);
            keep(hr[u]);
        }
    }
#pragma unroll
    for (int j = 0; j < 32; j += 4)
        s_red[wave][8 * lane + j / 4] = make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
    __syncthreads();
    // 512 threads x 4 columns each
    float4 s = s_red[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const float4 t = s_red[w][tid];
        s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    const int gcol = slice * 2048 + 4 * tid;
    if (gcol < d) {
        float* pp = part + (size_t)split * d + gcol;
        st_agent(pp, s.x); st_agent(pp + 1, s.y); st_agent(pp + 2, s.z); st_agent(pp + 3, s.w);
    }
    if (last_block_arrive(&counters[slice], (unsigned)nsplit)) {
        if (gcol < d) {
            float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int base = 0; base < nsplit; base += 8) {     // 32 partials in flight
                float v[8][4];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float* pp = part + (size_t)(base + j) * d + gcol;
                    const bool ok = base + j < nsplit;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[j][e] = ok ? ld_agent(pp + e) : 0.f;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    t.x += v[j][0]; t.y += v[j][1]; t.z += v[j][2]; t.w += v[j][3];
                }
            }
            *reinterpret_cast<float4*>(y + gcol) = t;
        }
    }
}

// ------------------------------------------------------------------------------------------ dispatch
template <bool GLU>
hipError_t up_f16(int q, int blocks, const uint16_t* x, const uint16_t* Wg, const uint16_t* Wu, int d, int F,
                  const int32_t* idx, const int32_t* count, int dense_F, float* h, hipStream_t s,
                  hipEvent_t ev0, hipEvent_t ev1) {
#define PI_UPF16(QQ) case QQ: \
    if (ev0) hipExtLaunchKernelGGL((k_up_f16<QQ, GLU>), dim3(blocks), dim3(256), 0, s, ev0, ev1, 0, x, Wg, Wu, d, F, idx, count, dense_F, h); \
    else hipLaunchKernelGGL((k_up_f16<QQ, GLU>), dim3(blocks), dim3(256), 0, s, x, Wg, Wu, d, F, idx, count, dense_F, h); \
    break;
    switch (q) {
        PI_UPF16(1) PI_UPF16(2) PI_UPF16(3) PI_UPF16(4) PI_UPF16(5) PI_UPF16(6) PI_UPF16(7) PI_UPF16(8)
        PI_UPF16(9) PI_UPF16(10) PI_UPF16(11) PI_UPF16(12) PI_UPF16(13) PI_UPF16(14) PI_UPF16(15) PI_UPF16(16)
        default: return hipErrorInvalidValue;
    }
#undef PI_UPF16
    return hipGetLastError();
}

template <bool GLU>
hipError_t up_i4(int q, int blocks, const uint16_t* x, const uint8_t* Gq, const uint16_t* Gs,
                 const uint8_t* Uq, const uint16_t* Us, int d, int F, const int32_t* idx,
                 const int32_t* count, int dense_F, float* h, hipStream_t s, hipEvent_t ev0,
                 hipEvent_t ev1) {
#define PI_UPI4(QQ) case QQ: \
    if (ev0) hipExtLaunchKernelGGL((k_up_i4<QQ, GLU>), dim3(blocks), dim3(256), 0, s, ev0, ev1, 0, x, Gq, Gs, Uq, Us, d, F, idx, count, dense_F, h); \
    else hipLaunchKernelGGL((k_up_i4<QQ, GLU>), dim3(blocks), dim3(256), 0, s, x, Gq, Gs, Uq, Us, d, F, idx, count, dense_F, h); \
    break;
    switch (q) {
        PI_UPI4(1) PI_UPI4(2) PI_UPI4(3) PI_UPI4(4) PI_UPI4(5) PI_UPI4(6) PI_UPI4(7) PI_UPI4(8)
        default: return hipErrorInvalidValue;
    }
#undef PI_UPI4
    return hipGetLastError();
}

}  // namespace

FfnPlan plan_ffn(int d, int F, int wfmt, int B) {
    FfnPlan p{};
    const bool f16 = wfmt == PI_W_F16;
    p.q = f16 ? (d + 511) / 512 : (d + 2047) / 2048;
    p.up_blocks = (F + 3) / 4 < 1024 ? (F + 3) / 4 : 1024;
    p.cols = f16 ? 512 : 2048;
    p.nslices = (d + p.cols - 1) / p.cols;
    const int wpb = f16 ? DOWN_WAVES_F16 : DOWN_WAVES_I4;
    int ns = 2048 / (p.nslices * wpb);
    p.nsplit = ns < 1 ? 1 : (ns > 32 ? 32 : ns);
    size_t off = COUNTER_BYTES;
    p.off_h = off;
    off = align_up(off + (size_t)F * sizeof(float), 256);
    p.off_part = off;
    off = align_up(off + (size_t)p.nsplit * d * sizeof(float), 256);
    p.u_ncg = p.u_ks = 0;
    p.off_H = p.off_upart = 0;
    if (B > 1) off = plan_union(p, d, F, off);
    p.bytes = off;
    return p;
}

hipError_t launch_up_b1(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x,
                        const int32_t* idx, const int32_t* count, int dense_F, float* h,
                        hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const bool glu = f.act == PI_ACT_REGLU;
    if (f.wfmt == PI_W_F16) {
        const uint16_t* Wg = static_cast<const uint16_t*>(f.w_gate);
        const uint16_t* Wu = static_cast<const uint16_t*>(f.w_up);
        return glu ? up_f16<true>(pl.q, pl.up_blocks, x, Wg, Wu, f.d, f.F, idx, count, dense_F, h, s, ev0, ev1)
                   : up_f16<false>(pl.q, pl.up_blocks, x, Wg, Wu, f.d, f.F, idx, count, dense_F, h, s, ev0, ev1);
    }
    const uint8_t* Gq = static_cast<const uint8_t*>(f.w_gate);
    const uint8_t* Uq = static_cast<const uint8_t*>(f.w_up);
    return glu ? up_i4<true>(pl.q, pl.up_blocks, x, Gq, f.s_gate, Uq, f.s_up, f.d, f.F, idx, count, dense_F, h, s, ev0, ev1)
               : up_i4<false>(pl.q, pl.up_blocks, x, Gq, f.s_gate, Uq, f.s_up, f.d, f.F, idx, count, dense_F, h, s, ev0, ev1);
}

hipError_t launch_down_b1(const pi_ffn_desc& f, const FfnPlan& pl, const int32_t* idx,
                          const int32_t* count, int dense_F, const float* h, float* y, char* ws,
                          hipStream_t s, int group) {
    unsigned* cnt = reinterpret_cast<unsigned*>(ws) + CNT_DOWN;
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    const dim3 gd(pl.nslices, pl.nsplit);
    if (f.wfmt == PI_W_F16) {
        hipLaunchKernelGGL((k_down_f16<4>), gd, dim3(64 * DOWN_WAVES_F16), 0, s,
                           static_cast<const uint16_t*>(f.w_down), f.d, f.F, idx, count, dense_F,
                           group, h, part, y, cnt);
    } else {
        hipLaunchKernelGGL((k_down_i4<4>), gd, dim3(64 * DOWN_WAVES_I4), 0, s,
                           static_cast<const uint8_t*>(f.w_down), f.s_down, f.d, f.F, idx, count,
                           dense_F, h, part, y, cnt);
    }
    return hipGetLastError();
}

hipError_t launch_ffn_b1(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x,
                         const int32_t* idx, const int32_t* count, int dense_F, float* y,
                         char* ws, hipStream_t s) {
    float* h = reinterpret_cast<float*>(ws + pl.off_h);
    hipError_t e = launch_up_b1(f, pl, x, idx, count, dense_F, h, s, nullptr, nullptr);
    if (e != hipSuccess) return e;
    return launch_down_b1(f, pl, idx, count, dense_F, h, y, ws, s);
}

}  // namespace pi
