// Low-rank activation predictor + threshold + neuron-table compaction (gfx950).
//
// PowerInfer, "Adaptive Sparsity Predictors": each layer's predictor marks the
// neurons a token will fire, so the FFN touches only those.  The predictor is
// the pair l = (x W_p1) W_p2 + b; a neuron is active when l > theta (theta =
// logit of the probability threshold).  "Neuron Placement and Management": the
// active neurons' original positions are written as an ascending int32 list.
//
// Both factors are stored neuron-major / row-contiguous on the device:
//   W1t [r, d]  row j = column j of W_p1   ->  z_j = W1t[j, :] . x
//   W2t [F, r]  row i = column i of W_p2   ->  l_i = W2t[i, :] . z + b_i
// so both stages are row GEMVs over contiguous rows (DRAM-friendly 16-byte
// coalesced loads, no split-K partial sums, no cross-block hand-off), fp32
// accumulation throughout.
//   stage 1  one wave per row j; x slice in registers; 64-lane reduction.
//   stage 2  one block per 64-neuron tile, 8 waves x 8 rows; z staged in LDS;
//            one wave ballot turns the tile's 64 decisions into two mask words;
//            the last-arriving block compacts the mask into the ascending table; with one
//            tile (F <= 64, one token) the single block writes the table from its ballot.
#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

// ------------------------------------------------------------------------------------ stage 1
// z[b, j] = W1t[j, :] . x[b, :].  Block: 4 waves = 4 rows.  The row is read in segments of
// QS 16-byte chunks per lane (all loads of a segment in flight together).  WPR = 4 (batch 1,
// rows of at least 256 chunks): one row per block, its 4 waves taking a quarter of the
// chunks each and meeting in LDS -- four times the blocks, each wave a quarter of the loads.
// CONV (the batch-1 decode executor): the grid also sums the previous step's P partial rows
// into y (reduce_partials), after its own loads are issued.
// P8: int8 rows (a chunk = 16 weights, one fp16 scale per 8 chunks), x read 32 bytes a chunk.
template <int QS, bool CONV, bool P8, int WPR = 1>
__global__ __launch_bounds__(256) void k_p1(const uint16_t* __restrict__ x, int B,
                                            const void* __restrict__ W1t,
                                            const uint16_t* __restrict__ S1, int d, int r,
                                            float* __restrict__ z, const float* __restrict__ part,
                                            float* __restrict__ y, int P) {
    const int lane = threadIdx.x & 63;
    const int j = WPR == 1 ? blockIdx.x * 4 + (threadIdx.x >> 6) : blockIdx.x;
    constexpr int EPC = P8 ? 16 : 8;                  // elements per 16-byte chunk
    const int nc = d / EPC;
    const size_t rowb = P8 ? (size_t)d : (size_t)d * 2;
    const uint8_t* Wb = static_cast<const uint8_t*>(W1t);
    const int ng = d >> 7;                            // int8: scale groups per row
    if constexpr (WPR > 1) {
        // one row per block: wave p takes chunks (p QW + q) 64 + lane
        constexpr int QW = (QS + WPR - 1) / WPR;
        const int p = threadIdx.x >> 6;
        const int jj = j < r ? j : 0;
        const uint8_t* row = Wb + (size_t)jj * rowb;
        uint4 w[QW], xr[QW], xr2[P8 ? QW : 1];
        uint32_t sr[P8 ? QW : 1];
#pragma unroll
        for (int q = 0; q < QW; ++q) {
            const int c = (p * QW + q) * 64 + lane;
            const int cc = c < nc ? c : 0;
            w[q] = ld16(row + 16 * (size_t)cc);
            if constexpr (P8) {
                xr[q] = ld16(x + 16 * cc);
                xr2[q] = ld16(x + 16 * cc + 8);
                sr[q] = S1[(size_t)jj * ng + (cc >> 3)];
            } else {
                xr[q] = ld16(x + 8 * cc);
            }
        }
        if (CONV) reduce_partials(part, P, d, y, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
        if (j >= r) return;                             // the whole block
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < QW; ++q)
            if ((p * QW + q) * 64 + lane < nc) {
                if constexpr (P8)
                    acc = fmaf(h2f((uint16_t)sr[q]), dot16_i8_f16(w[q], xr[q], xr2[q]), acc);
                else
                    acc = dot8(w[q], xr[q], acc);
            }
        acc = wave_sum(acc);
        __shared__ float s_part[WPR];
        if (lane == 0) s_part[p] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = 0.f;
#pragma unroll
            for (int k = 0; k < WPR; ++k) t += s_part[k];
            z[j] = t;
        }
        return;
    }
    if (B == 1 && nc <= 64 * QS) {
        // one segment: row and x chunks all in flight together, issued before the conversion
        // (whose loads would otherwise hold the row loads back by a memory round trip)
        const int jj = j < r ? j : 0;
        const uint8_t* row = Wb + (size_t)jj * rowb;
        uint4 w[QS], xr[QS], xr2[P8 ? QS : 1];
        uint32_t sr[P8 ? QS : 1];
#pragma unroll
        for (int q = 0; q < QS; ++q) {
            const int c = lane + 64 * q;
            const int cc = c < nc ? c : 0;
            w[q] = ld16(row + 16 * (size_t)cc);
            if constexpr (P8) {
                xr[q] = ld16(x + 16 * cc);
                xr2[q] = ld16(x + 16 * cc + 8);
                sr[q] = S1[(size_t)jj * ng + (cc >> 3)];
            } else {
                xr[q] = ld16(x + 8 * cc);
            }
        }
        if (CONV) reduce_partials(part, P, d, y, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
        if (j >= r) return;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < QS; ++q)
            if (lane + 64 * q < nc) {
                if constexpr (P8)
                    acc = fmaf(h2f((uint16_t)sr[q]), dot16_i8_f16(w[q], xr[q], xr2[q]), acc);
                else
                    acc = dot8(w[q], xr[q], acc);
            }
        acc = wave_sum(acc);
        if (lane == 0) z[j] = acc;
        return;
    }
    if (CONV) reduce_partials(part, P, d, y, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
    if (j >= r) return;
    const uint8_t* row = Wb + (size_t)j * rowb;
    for (int b = 0; b < B; ++b) {
        const uint16_t* xb = x + (size_t)b * d;
        float acc = 0.f;
        for (int c0 = 0; c0 < nc; c0 += 64 * QS) {
            uint4 w[QS], xr[QS], xr2[P8 ? QS : 1];
            uint32_t sr[P8 ? QS : 1];
#pragma unroll
            for (int q = 0; q < QS; ++q) {
                const int c = c0 + lane + 64 * q;
                const bool ok = c < nc;
                w[q] = ok ? ld16(row + 16 * (size_t)c) : zero4();
                if constexpr (P8) {
                    xr[q] = ok ? ld16(xb + 16 * c) : zero4();
                    xr2[q] = ok ? ld16(xb + 16 * c + 8) : zero4();
                    sr[q] = (uint32_t)S1[(size_t)j * ng + ((ok ? c : 0) >> 3)];
                } else {
                    xr[q] = ok ? ld16(xb + 8 * c) : zero4();
                }
            }
#pragma unroll
            for (int q = 0; q < QS; ++q) {
                if constexpr (P8)
                    acc = fmaf(h2f((uint16_t)sr[q]), dot16_i8_f16(w[q], xr[q], xr2[q]), acc);
                else
                    acc = dot8(w[q], xr[q], acc);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) z[(size_t)b * r + j] = acc;
    }
}

// ------------------------------------------------------------------------------------ stage 2
// l[b, n] = W2t[n, :] . z[b, :] + bias[n] for the 64 neurons of tile blockIdx.x.
// 512 threads: wave w owns rows n0 + 8w .. n0 + 8w + 7 (tile_logits); z of nbz tokens
// at a time sits in dynamic LDS.
constexpr int P2_WAVES = 8;

template <bool P8>
__global__ __launch_bounds__(P2_WAVES * 64) void k_p2(const float* __restrict__ z, int B,
                                             const void* __restrict__ W2t,
                                             const uint16_t* __restrict__ S2,
                                             const float* __restrict__ bias, int r, int F,
                                             float theta, int nbz, float* __restrict__ logits,
                                             uint32_t* __restrict__ mask,
                                             int32_t* __restrict__ idx,
                                             int32_t* __restrict__ count,
                                             unsigned* __restrict__ counter) {
    extern __shared__ __align__(16) float s_z[];   // [nbz][r]
    __shared__ float s_l[64];
    __shared__ int s_tmp[P2_WAVES + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x;
    const int W = (F + 31) >> 5;
    // the tile's bias, loaded once for every token and not on the threshold's critical path
    const float bv = (wave == 0 && tile * 64 + lane < F) ? bias[tile * 64 + lane] : 0.f;
    for (int b0 = 0; b0 < B; b0 += nbz) {
        const int nb = min(nbz, B - b0);
        for (int i = tid; i < nb * r; i += P2_WAVES * 64) s_z[i] = z[(size_t)b0 * r + i];
        __syncthreads();
        for (int t = 0; t < nb; ++t) {
            tile_logits<P2_WAVES, P8>(W2t, S2, s_z + t * r, r, F, tile, s_l);
            __syncthreads();
            if (wave == 0) {
                const int n = tile * 64 + lane;
                const int b = b0 + t;
                bool act = false;
                if (n < F) {
                    const float l = s_l[lane] + bv;
                    act = l > theta;
                    if (logits) logits[(size_t)b * F + n] = l;
                }
                const unsigned long long bal = __ballot(act);
                if (lane == 0) {
                    st_agent(&mask[(size_t)b * W + 2 * tile], (uint32_t)bal);
                    if (2 * tile + 1 < W) st_agent(&mask[(size_t)b * W + 2 * tile + 1], (uint32_t)(bal >> 32));
                }
            }
            __syncthreads();
        }
    }
    if (idx != nullptr && last_block_arrive(counter, gridDim.x)) {
        for (int b = 0; b < B; ++b)
            block_compact<true>(mask + (size_t)b * W, 1, W, F, idx + (size_t)b * F, count + b, s_tmp);
    }
}

// One token and at most 64 neurons (one tile, so one block: the attention side's head
// predictor has one output per head).  The W2t rows and the bias go out before z is staged,
// and the block writes the mask words and the ascending table straight from its ballot -- no
// arrival counter and no second pass over the mask.
template <bool P8>
__global__ __launch_bounds__(P2_WAVES * 64) void k_p2_one(const float* __restrict__ z,
                                                 const void* __restrict__ W2t,
                                                 const uint16_t* __restrict__ S2,
                                                 const float* __restrict__ bias, int r, int F,
                                                 float theta, float* __restrict__ logits,
                                                 uint32_t* __restrict__ mask,
                                                 int32_t* __restrict__ idx,
                                                 int32_t* __restrict__ count) {
    extern __shared__ __align__(16) float s_z[];   // [r]
    __shared__ float s_l[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    TileRows<P2_WAVES, P8> tr;
    tile_rows_load<P2_WAVES, P8>(tr, W2t, S2, r, F, 0, 0);
    const float bv = bias[lane < F ? lane : 0];
    for (int i = tid; i < r; i += P2_WAVES * 64) s_z[i] = z[i];
    __syncthreads();
    float acc[TileRows<P2_WAVES, P8>::RPW] = {};
    tile_rows_fma<P2_WAVES, P8>(tr, s_z, r, 0, acc);
    for (int c0 = TILE_SEG<P8>; c0 < tile_chunks<P8>(r); c0 += TILE_SEG<P8>) {
        tile_rows_load<P2_WAVES, P8>(tr, W2t, S2, r, F, 0, c0);
        tile_rows_fma<P2_WAVES, P8>(tr, s_z, r, c0, acc);
    }
    tile_rows_store<P2_WAVES>(acc, s_l);
    __syncthreads();
    if (wave != 0) return;
    const float l = s_l[lane] + bv;
    const bool act = lane < F && l > theta;
    if (logits != nullptr && lane < F) logits[lane] = l;
    const unsigned long long bal = __ballot(act);
    if (lane == 0) {
        mask[0] = (uint32_t)bal;
        if (F > 32) mask[1] = (uint32_t)(bal >> 32);
    }
    if (idx != nullptr) {
        if (act) idx[__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = lane;
        if (lane == 0) *count = __popcll(bal);
    }
}

}  // namespace

hipError_t launch_pred_stage1(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x, int B,
                              float* z, hipStream_t s, const float* part, float* y, int P) {
    if (p.pfmt == PI_P_I8G128) {
        int q = (p.d / 16 + 63) / 64;
        q = q < 1 ? 1 : (q > 16 ? 16 : q);
#define PI_P1(QQ) case QQ: \
    if (B == 1 && QQ >= 4 && p.d / 16 <= 64 * QQ) { \
        if (part) hipLaunchKernelGGL((k_p1<QQ, true, true, 4>), dim3(p.r), dim3(256), 0, s, x, B, p.w_p1t, p.s_p1t, p.d, p.r, z, part, y, P); \
        else hipLaunchKernelGGL((k_p1<QQ, false, true, 4>), dim3(p.r), dim3(256), 0, s, x, B, p.w_p1t, p.s_p1t, p.d, p.r, z, nullptr, nullptr, 0); \
    } else if (part) hipLaunchKernelGGL((k_p1<QQ, true, true>), dim3(pl.nblk1), dim3(256), 0, s, x, B, p.w_p1t, p.s_p1t, p.d, p.r, z, part, y, P); \
    else hipLaunchKernelGGL((k_p1<QQ, false, true>), dim3(pl.nblk1), dim3(256), 0, s, x, B, p.w_p1t, p.s_p1t, p.d, p.r, z, nullptr, nullptr, 0); \
    break;
        switch (q) {
            PI_P1(1) PI_P1(2) PI_P1(3) PI_P1(4) PI_P1(5) PI_P1(6) PI_P1(7) PI_P1(8)
            PI_P1(9) PI_P1(10) PI_P1(11) PI_P1(12) PI_P1(13) PI_P1(14) PI_P1(15) PI_P1(16)
            default: return hipErrorInvalidValue;
        }
#undef PI_P1
        return hipGetLastError();
    }
#define PI_P1(QQ) case QQ: \
    if (B == 1 && QQ >= 4 && p.d / 8 <= 64 * QQ) { \
        if (part) hipLaunchKernelGGL((k_p1<QQ, true, false, 4>), dim3(p.r), dim3(256), 0, s, x, B, p.w_p1t, nullptr, p.d, p.r, z, part, y, P); \
        else hipLaunchKernelGGL((k_p1<QQ, false, false, 4>), dim3(p.r), dim3(256), 0, s, x, B, p.w_p1t, nullptr, p.d, p.r, z, nullptr, nullptr, 0); \
    } else if (part) hipLaunchKernelGGL((k_p1<QQ, true, false>), dim3(pl.nblk1), dim3(256), 0, s, x, B, p.w_p1t, nullptr, p.d, p.r, z, part, y, P); \
    else hipLaunchKernelGGL((k_p1<QQ, false, false>), dim3(pl.nblk1), dim3(256), 0, s, x, B, p.w_p1t, nullptr, p.d, p.r, z, nullptr, nullptr, 0); \
    break;
    switch (pl.qs) {
        PI_P1(1) PI_P1(2) PI_P1(3) PI_P1(4) PI_P1(5) PI_P1(6) PI_P1(7) PI_P1(8)
        PI_P1(9) PI_P1(10) PI_P1(11) PI_P1(12) PI_P1(13) PI_P1(14) PI_P1(15) PI_P1(16)
        default: return hipErrorInvalidValue;
    }
#undef PI_P1
    return hipGetLastError();
}

PredPlan plan_pred(int d, int r, int F, int B) {
    PredPlan p{};
    const int q = (d / 8 + 63) / 64;
    p.qs = q < 1 ? 1 : (q > 16 ? 16 : q);
    p.nblk1 = (r + 3) / 4;
    p.nblk2 = (F + 63) / 64;
    int nbz = (32 * 1024) / (r * 4);        // z of nbz tokens in at most 32 KB of LDS
    if (nbz < 1) nbz = 1;
    if (nbz > B) nbz = B;
    p.nbz = nbz;
    p.lds2 = (size_t)nbz * r * sizeof(float);
    size_t off = COUNTER_BYTES;
    p.off_z = off;
    off = align_up(off + (size_t)B * r * sizeof(float), 256);
    p.b_ntile = p.b_nks = 0;
    p.off_zpart = 0;
    if (B > 1) plan_pred_batch(p, d, r, F, off);
    p.bytes = off;
    return p;
}

hipError_t launch_predict(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x, int B,
                          float theta, float* logits, uint32_t* mask, int32_t* idx, int32_t* count,
                          char* ws, hipStream_t s) {
    if (B > 1) {
        hipError_t e = launch_predict_batch(p, pl, x, B, theta, logits, mask, ws, s);
        if (e != hipSuccess || idx == nullptr) return e;
        return launch_compact(mask, B, p.F, PI_PER_TOKEN, idx, count, s);
    }
    hipError_t e = launch_pred_stage1(p, pl, x, B, reinterpret_cast<float*>(ws + pl.off_z), s);
    if (e != hipSuccess) return e;
    return launch_pred_stage2_b1(p, pl, theta, logits, mask, idx, count, ws, s);
}

hipError_t launch_pred_stage2_b1(const pi_pred_desc& p, const PredPlan& pl, float theta, float* logits,
                                 uint32_t* mask, int32_t* idx, int32_t* count, char* ws, hipStream_t s) {
    const int B = 1;
    unsigned* cnt = reinterpret_cast<unsigned*>(ws);
    const float* z = reinterpret_cast<const float*>(ws + pl.off_z);
    if (p.F <= 64 && p.r <= 8192) {      // z (r floats) in LDS next to the static arrays
        if (p.pfmt == PI_P_I8G128)
            hipLaunchKernelGGL(k_p2_one<true>, dim3(1), dim3(P2_WAVES * 64), (size_t)p.r * sizeof(float), s, z,
                               p.w_p2t, p.s_p2t, p.bias, p.r, p.F, theta, logits, mask, idx, count);
        else
            hipLaunchKernelGGL(k_p2_one<false>, dim3(1), dim3(P2_WAVES * 64), (size_t)p.r * sizeof(float), s, z,
                               p.w_p2t, nullptr, p.bias, p.r, p.F, theta, logits, mask, idx, count);
        return hipGetLastError();
    }
    if (p.pfmt == PI_P_I8G128)
        hipLaunchKernelGGL(k_p2<true>, dim3(pl.nblk2), dim3(P2_WAVES * 64), pl.lds2, s, z, B, p.w_p2t, p.s_p2t,
                           p.bias, p.r, p.F, theta, pl.nbz, logits, mask, idx, count, cnt + CNT_PRED2);
    else
        hipLaunchKernelGGL(k_p2<false>, dim3(pl.nblk2), dim3(P2_WAVES * 64), pl.lds2, s, z, B, p.w_p2t, nullptr,
                           p.bias, p.r, p.F, theta, pl.nbz, logits, mask, idx, count, cnt + CNT_PRED2);
    return hipGetLastError();
}

}  // namespace pi
