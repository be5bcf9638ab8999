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
//   out  y = sum over predicted heads h, c < d_head of o[h, c] W_o[h, c, :]: the column-sparse
//        axpy of the FFN's down projection over the rows of the predicted heads, run by the
//        batch-1 down kernel with the head table as its list (an entry stands for its head's
//        d_head consecutive rows; o read by row).
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

template <int Q, int RPW>
hipError_t qkv_launch(const pi_attn_desc& a, const uint16_t* x, const uint32_t* hmask, float* qkv,
                      hipStream_t s) {
    const int bph = (3 * a.dh + QKV_WAVES * RPW - 1) / (QKV_WAVES * RPW);
    hipLaunchKernelGGL((k_attn_qkv<Q, RPW>), dim3(a.H * bph), dim3(64 * QKV_WAVES), 0, s, x,
                       static_cast<const uint16_t*>(a.w_qkv), a.d, a.dh, hmask, bph, qkv);
    return hipGetLastError();
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

AttnPlan plan_attn(int d, int H, int dh) {
    AttnPlan p{};
    p.ffn = plan_ffn(d, H * dh, PI_W_F16, 1);
    p.bytes = p.ffn.bytes;
    return p;
}

hipError_t launch_attn_out(const pi_attn_desc& a, const AttnPlan& pl, const float* o,
                           const int32_t* heads, const int32_t* count, float* y, char* ws,
                           hipStream_t s) {
    // the down projection over rows of W_o^T, its list the head table with d_head rows per entry
    pi_ffn_desc f{};
    f.w_down = a.w_o;
    f.d = a.d;
    f.F = a.H * a.dh;
    f.act = PI_ACT_RELU;                              // not read by the down projection
    f.wfmt = PI_W_F16;
    return launch_down_b1(f, pl.ffn, heads, count, 0, o, y, ws, s, a.dh);
}

}  // namespace pi
