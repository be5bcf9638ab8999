// The attention side of a layer on gfx950: head-sparse q/k/v and output projections.
//
// PowerInfer, "Adaptive Sparsity Predictors": every layer has a second predictor, for the
// self-attention block, and only the neurons it predicts are computed.  Here the block's
// neurons are its heads (head h owns d_head rows each of W_q, W_k, W_v and d_head rows of W_o^T),
// predicted by pi_predict with one output per head.  "Neuron-aware Operator": the predicted
// heads' rows are read in place out of the dense head-major matrices.
//
//   qkv  qkv[h, m, c] = W_qkv[h, m, c, :] . x for the heads set in the head mask, 0 for the
//        others.  A block owns 8 consecutive rows of one head (4 waves x 2 rows): a block of an
//        inactive head writes its zeros and leaves; an active one keeps its lanes' slice of x in
//        registers and has both rows' 16-byte loads (every chunk of the row) in flight at once.
//        A head's 3 d_head rows are contiguous, so the stream over an active head is one
//        sequential read of 6 d_head d bytes.
//   out  y = sum over predicted heads h, c < d_head of o[h, c] W_o[h, c, :].  Block (s, j) takes
//        entry j of the head table over the 512-column slice s: its head's d_head rows (one
//        contiguous block of W_o), all in flight at once, 8 per wave, 1 KB per row, and stores
//        its column sums as partial row j.  pi_attn_out: agent-scope stores, and the last of the
//        slice's H blocks to arrive (entries past the count arrive without work) sums rows
//        j < count in a fixed order into y.  The executor: plain stores, zero rows for the
//        entries past the count, and the next step's stage-1 kernel -- or, after the last step,
//        a small kernel -- sums the H rows into y, as the FFN decode schedules do: no hand-off
//        between blocks.  The grid's slice dimension is padded to a multiple
//        of 8, so block s + 8k j of the dispatch order -- and with it every block of slice s --
//        lands on XCD s mod 8, and the hand-off stays inside one L2.
#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

constexpr int QKV_WAVES = 4;

template <int Q, int RPW>
__global__ __launch_bounds__(64 * QKV_WAVES) void k_attn_qkv(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ W, int d,
                                                           int dh, const uint32_t* __restrict__ hmask,
                                                           int bph, float* __restrict__ qkv) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x / bph;
    const int nrow = 3 * dh;
    const int r0 = (blockIdx.x - h * bph) * (QKV_WAVES * RPW) + wave * RPW;
    float* out = qkv + (size_t)h * nrow;
    if (!((hmask[h >> 5] >> (h & 31)) & 1u)) {        // a head predicted inactive: zeros
        if (lane < RPW && r0 + lane < nrow) out[r0 + lane] = 0.f;
        return;
    }
    if (r0 >= nrow) return;
    const int nc = d >> 3;                            // 16-byte chunks of a row
    uint4 xr[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = lane + 64 * q;
        xr[q] = c < nc ? ld16(x + 8 * c) : zero4();
    }
    uint4 w[RPW][Q];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const uint16_t* p = W + ((size_t)h * nrow + min(r0 + j, nrow - 1)) * d;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = lane + 64 * q;
            w[j][q] = c < nc ? ld16_nt(p + 8 * c) : zero4();
        }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) acc = dot8(w[j][q], xr[q], acc);
        acc = wave_sum(acc);
        if (lane == 0 && r0 + j < nrow) out[r0 + j] = acc;
    }
}

// l_h = W2t[h, :] . z + bias[h] (fp16 weights, fp32 z): lane i takes elements i, i + 64, ... (four
// in flight), the lanes meet in wave_sum.  Every wave that evaluates head h gets the same bits.
PI_DEV float head_logit(const uint16_t* __restrict__ W2t, const float* __restrict__ z,
                        const float* __restrict__ bias, int r, int h) {
    const int lane = threadIdx.x & 63;
    const uint16_t* w = W2t + (size_t)h * r;
    float acc = 0.f;
    for (int i0 = 0; i0 < r; i0 += 256) {
        uint16_t wv[4];
        float zv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + lane + 64 * u;
            wv[u] = w[i < r ? i : 0];
            zv[u] = z[i < r ? i : 0];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + lane + 64 * u < r) acc = fmaf(h2f(wv[u]), zv[u], acc);
    }
    return wave_sum(acc) + bias[h];
}

// The executor's q/k/v step with the head predictor's second stage folded in (one token,
// H <= 64): every wave computes its head's logit from z and the head's W2t row (an L2 round
// trip) and goes on to the head's rows or its zeros, so no kernel and no mask stand between
// stage 1 and the q/k/v rows.  Block 0 also computes every head's logit (head_logit again, so
// its bits are the ones the blocks acted on) and writes the logits, the mask words, the
// ascending head table and its count.  Rows as in k_attn_qkv.
template <int Q, int RPW>
__global__ __launch_bounds__(64 * QKV_WAVES) void k_attn_pqkv(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, int d, int dh, int bph,
    float* __restrict__ qkv, const float* __restrict__ z, const uint16_t* __restrict__ W2t,
    const float* __restrict__ bias, int r, int H, float theta, float* __restrict__ logits,
    uint32_t* __restrict__ mask, int32_t* __restrict__ heads, int32_t* __restrict__ count) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x / bph;
    const int nrow = 3 * dh;
    const int r0 = (blockIdx.x - h * bph) * (QKV_WAVES * RPW) + wave * RPW;
    float* out = qkv + (size_t)h * nrow;
    const float lh = head_logit(W2t, z, bias, r, h);
    if (blockIdx.x == 0) {
        __shared__ float s_l[64];
        for (int hh = wave; hh < H; hh += QKV_WAVES) {
            const float l = head_logit(W2t, z, bias, r, hh);
            if (lane == 0) s_l[hh] = l;
        }
        __syncthreads();
        if (wave == 0) {
            const float l = lane < H ? s_l[lane] : 0.f;
            const bool act = lane < H && l > theta;
            if (logits != nullptr && lane < H) logits[lane] = l;
            const unsigned long long bal = __ballot(act);
            if (lane == 0) {
                mask[0] = (uint32_t)bal;
                if (H > 32) mask[1] = (uint32_t)(bal >> 32);
                *count = __popcll(bal);
            }
            if (act) heads[__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = lane;
        }
    }
    if (!(lh > theta)) {                              // a head predicted inactive: zeros
        if (lane < RPW && r0 + lane < nrow) out[r0 + lane] = 0.f;
        return;
    }
    if (r0 >= nrow) return;
    const int nc = d >> 3;
    uint4 xr[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = lane + 64 * q;
        xr[q] = c < nc ? ld16(x + 8 * c) : zero4();
    }
    uint4 w[RPW][Q];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const uint16_t* p = W + ((size_t)h * nrow + min(r0 + j, nrow - 1)) * d;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = lane + 64 * q;
            w[j][q] = c < nc ? ld16_nt(p + 8 * c) : zero4();
        }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) acc = dot8(w[j][q], xr[q], acc);
        acc = wave_sum(acc);
        if (lane == 0 && r0 + j < nrow) out[r0 + j] = acc;
    }
}

template <int Q, int RPW>
hipError_t pqkv_launch(const pi_attn_desc& a, const pi_pred_desc& p, const uint16_t* x, const float* z,
                       float theta, float* logits, uint32_t* mask, int32_t* heads, int32_t* count,
                       float* qkv, hipStream_t s) {
    const int bph = (3 * a.dh + QKV_WAVES * RPW - 1) / (QKV_WAVES * RPW);
    hipLaunchKernelGGL((k_attn_pqkv<Q, RPW>), dim3(a.H * bph), dim3(64 * QKV_WAVES), 0, s, x,
                       static_cast<const uint16_t*>(a.w_qkv), a.d, a.dh, bph, qkv, z,
                       static_cast<const uint16_t*>(p.w_p2t), p.bias, p.r, a.H, theta, logits, mask,
                       heads, count);
    return hipGetLastError();
}

template <int Q, int RPW>
hipError_t qkv_launch(const pi_attn_desc& a, const uint16_t* x, const uint32_t* hmask, float* qkv,
                      hipStream_t s) {
    const int bph = (3 * a.dh + QKV_WAVES * RPW - 1) / (QKV_WAVES * RPW);
    hipLaunchKernelGGL((k_attn_qkv<Q, RPW>), dim3(a.H * bph), dim3(64 * QKV_WAVES), 0, s, x,
                       static_cast<const uint16_t*>(a.w_qkv), a.d, a.dh, hmask, bph, qkv);
    return hipGetLastError();
}

constexpr int AO_WAVES = 16;                         // 1024 threads over a 512-column slice
constexpr int AO_COLS = 512;
constexpr int AO_U = 8;                              // rows in flight per wave

template <bool DEFER>
__global__ __launch_bounds__(64 * AO_WAVES) void k_attn_out(const uint16_t* __restrict__ Wo,
                                                          const float* __restrict__ o,
                                                          const int32_t* __restrict__ heads,
                                                          const int32_t* __restrict__ count, int d,
                                                          int H, int dh, int nslices,
                                                          float* __restrict__ part,
                                                          float* __restrict__ y,
                                                          unsigned* __restrict__ counters) {
    __shared__ float4 s_red[AO_WAVES][AO_COLS / 4];
    __shared__ float s_half[AO_COLS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slice = blockIdx.x, j = blockIdx.y;
    if (slice >= nslices) return;                    // padding of the slice dimension
    const int nc = d >> 3;
    const int c = slice * 64 + lane;                 // this lane's 16-byte chunk (8 columns)
    const bool cok = c < nc;
    const int cc = cok ? c : 0;
    const int n = min(*count, H);
    const int col = tid & (AO_COLS - 1), hf = tid >> 9;
    const int gcol = slice * AO_COLS + col;
    if (DEFER && j >= n) {                           // an entry past the count: a zero row
        if (hf == 0 && gcol < d) part[(size_t)j * d + gcol] = 0.f;
        return;
    }
    if (j < n) {
        const int hd = heads[j];
        const bool hok = (unsigned)hd < (unsigned)H;
        const size_t hrow = (size_t)(hok ? hd : 0) * dh;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int i0 = wave; i0 < dh; i0 += AO_WAVES * AO_U) {
            uint4 w[AO_U];
            float ov[AO_U];
            // unconditional clamped loads, discarded at use (a lane-guarded load is waited for
            // on the spot)
#pragma unroll
            for (int u = 0; u < AO_U; ++u) {
                const int i = i0 + AO_WAVES * u;
                const size_t rw = hrow + (i < dh ? i : 0);
                w[u] = ld16(Wo + rw * d + 8 * (size_t)cc);
                ov[u] = o[rw];
            }
#pragma unroll
            for (int u = 0; u < AO_U; ++u) {
                const float hv = (hok && cok && i0 + AO_WAVES * u < dh) ? ov[u] : 0.f;
                const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(hv, lo_f(ww[e]), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(hv, hi_f(ww[e]), acc[2 * e + 1]);
                }
            }
        }
        s_red[wave][2 * lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        s_red[wave][2 * lane + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        __syncthreads();
        // 1024 threads over 512 columns: half hf sums waves [8 hf, 8 hf + 8) in order
        const float* sr = reinterpret_cast<const float*>(s_red);
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < AO_WAVES / 2; ++w) t += sr[(hf * (AO_WAVES / 2) + w) * AO_COLS + col];
        if (hf == 1) s_half[col] = t;
        __syncthreads();
        if (hf == 0 && gcol < d) {
            if (DEFER) part[(size_t)j * d + gcol] = t + s_half[col];
            else st_agent(&part[(size_t)j * d + gcol], t + s_half[col]);
        }
        if (DEFER) return;
    }
    if (!last_block_arrive(&counters[slice], (unsigned)H)) return;
    // rows j < n: half hf takes j = hf, hf + 2, ... (16 loads in flight), then the halves meet
    float t = 0.f;
    if (gcol < d) {
        for (int b0 = hf; b0 < n; b0 += 32) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int jj = b0 + 2 * k;
                v[k] = ld_agent(&part[(size_t)(jj < n ? jj : 0) * d + gcol]);
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (b0 + 2 * k < n) t += v[k];
        }
    }
    __syncthreads();
    if (hf == 1) s_half[col] = t;
    __syncthreads();
    if (hf == 0 && gcol < d) y[gcol] = t + s_half[col];
}

}  // namespace

hipError_t launch_attn_qkv(const pi_attn_desc& a, const uint16_t* x, const uint32_t* hmask,
                           float* qkv, hipStream_t s) {
    const int q = (a.d + 511) / 512;                  // 16-byte chunks per lane of a row
    if (q <= 2) return qkv_launch<2, 2>(a, x, hmask, qkv, s);
    if (q <= 4) return qkv_launch<4, 2>(a, x, hmask, qkv, s);
    if (q <= 8) return qkv_launch<8, 2>(a, x, hmask, qkv, s);
    if (q <= 16) return qkv_launch<16, 2>(a, x, hmask, qkv, s);
    return qkv_launch<32, 1>(a, x, hmask, qkv, s);    // d <= PI_ATTN_MAX_D
}

hipError_t launch_attn_pqkv(const pi_attn_desc& a, const pi_pred_desc& p, const uint16_t* x,
                            const float* z, float theta, float* logits, uint32_t* mask,
                            int32_t* heads, int32_t* count, float* qkv, hipStream_t s) {
    if (a.H > 64 || p.F != a.H || p.pfmt != PI_P_F16) return hipErrorInvalidValue;
    const int q = (a.d + 511) / 512;
    if (q <= 2) return pqkv_launch<2, 2>(a, p, x, z, theta, logits, mask, heads, count, qkv, s);
    if (q <= 4) return pqkv_launch<4, 2>(a, p, x, z, theta, logits, mask, heads, count, qkv, s);
    // 3 rows a wave for d <= 4096: a LLaMA-7B-shaped layer (32 heads x 384 rows) fits one round
    // of waves on the chip (2 rows: 22.2 us per step, 3: 21.8; OPT-30B-shaped d = 7168 keeps 2,
    // 1 row there: 42.8 -> 43.6)
    if (q <= 8) return pqkv_launch<8, 3>(a, p, x, z, theta, logits, mask, heads, count, qkv, s);
    if (q <= 16) return pqkv_launch<16, 2>(a, p, x, z, theta, logits, mask, heads, count, qkv, s);
    return pqkv_launch<32, 1>(a, p, x, z, theta, logits, mask, heads, count, qkv, s);
}

AttnPlan plan_attn(int d, int H, int dh) {
    (void)dh;
    AttnPlan p{};
    p.nslices = (d + AO_COLS - 1) / AO_COLS;          // <= 32 (d <= PI_ATTN_MAX_D)
    p.off_part = align_up(COUNTER_BYTES, 256);
    p.bytes = align_up(p.off_part + (size_t)H * d * sizeof(float), 256);   // H partial rows
    return p;
}

hipError_t launch_attn_out(const pi_attn_desc& a, const AttnPlan& pl, const float* o,
                           const int32_t* heads, const int32_t* count, float* y, char* ws,
                           hipStream_t s) {
    unsigned* cnt = reinterpret_cast<unsigned*>(ws) + CNT_DOWN;
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    const dim3 g((pl.nslices + 7) & ~7, a.H);
    hipLaunchKernelGGL(k_attn_out<false>, g, dim3(64 * AO_WAVES), 0, s, static_cast<const uint16_t*>(a.w_o), o,
                       heads, count, a.d, a.H, a.dh, pl.nslices, part, y, cnt);
    return hipGetLastError();
}

hipError_t launch_attn_out_rows(const pi_attn_desc& a, const AttnPlan& pl, const float* o,
                                const int32_t* heads, const int32_t* count, float* part, hipStream_t s) {
    const dim3 g((pl.nslices + 7) & ~7, a.H);
    hipLaunchKernelGGL(k_attn_out<true>, g, dim3(64 * AO_WAVES), 0, s, static_cast<const uint16_t*>(a.w_o), o,
                       heads, count, a.d, a.H, a.dh, pl.nslices, part, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace pi
