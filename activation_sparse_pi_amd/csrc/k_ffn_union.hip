// Small-batch (1 < B <= 32) neuron-aware FFN on the union of the token masks, on MFMA.
//
// PowerInfer, "Neuron Aware Operator": only the rows / output vectors of listed
// neurons are read.  With B tokens, the list is the union of their predicted sets
// and every weight byte read serves all B tokens, which makes this a dense
// contraction over the union (about 2B flops per weight byte): MFMA territory.
// Each token still uses its own mask: a neuron outside token b's mask contributes
// nothing to y[b] (its h is zeroed before the down product).
//
// v_mfma_f32_32x32x16_f16 (gfx950) lane layout, checked on the device:
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + j], j < 8
//   B (16 x 32): lane l holds B[8 * (l / 32) + j][l % 32]
//   D (32 x 32): lane l, register r holds D[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32]
// The k slots of one MFMA may be any permutation shared by A and B, which lets a lane
// read long contiguous runs of its row.
//
//   up    Ht[b, k] = act(W_up[u_k] . x_b)  (fp16, token-major [32, F]), zero where neuron
//         u_k is not in token b's mask.  Block = one 32-neuron tile of the union list x
//         all 32 token slots; its 8 waves split d; each lane streams 64-byte runs of its
//         neuron's row and of its token's x (4 MFMAs per run); waves meet in LDS.
//   down  y[b, :] = sum_k Ht[b, k] W_down[u_k, :].  Block = one 32-column slice of y; its
//         8 waves split the union list; per step of 16 neurons a lane loads 16 bytes of
//         one row and writes them transposed into its wave's own LDS tile, so the MFMA B
//         operand (8 consecutive neurons of one column) is one 16-byte LDS read and no
//         block barrier sits in the streaming loop; waves meet in LDS at the end and the
//         block writes its slice of y (no partial sums leave the block).  The two slices
//         sharing a 128-byte line run on blocks of the same XCD.
#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int UN_NW = 8;           // waves per block

PI_DEV half8_t as_h8(const uint4& v) { return __builtin_bit_cast(half8_t, v); }

PI_DEV f32x16_t mfma16(const uint4& a, const uint4& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(a), as_h8(b), c, 0, 0, 0);
}

PI_DEV bool bit_of(const uint32_t* __restrict__ mask, int W, int b, int i) {
    return (mask[(size_t)b * W + (i >> 5)] >> (i & 31)) & 1u;
}

// ------------------------------------------------------------------------------------ up
template <bool GLU>
__global__ __launch_bounds__(UN_NW * 64) void k_union_up(
    const uint16_t* __restrict__ x, int B, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, int d, int F, const int32_t* __restrict__ uidx,
    const int32_t* __restrict__ ucount, const uint32_t* __restrict__ tmask,
    uint16_t* __restrict__ Ht) {
    __shared__ float s_red[UN_NW][16][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int U = min(*ucount, F);
    const int tile = blockIdx.x;
    if (tile * 32 >= U) return;                        // whole block: past the union
    const int mi = lane & 31, half = lane >> 5;
    const int kpos = tile * 32 + mi;                   // this lane's union position (A row)
    int row = kpos < U ? uidx[kpos] : -1;
    if ((unsigned)row >= (unsigned)F) row = -1;
    const int tok = mi;                                // this lane's token (B column)
    const uint8_t* pu = row >= 0 ? reinterpret_cast<const uint8_t*>(Wu + (size_t)row * d) : nullptr;
    const uint8_t* pg = (GLU && row >= 0) ? reinterpret_cast<const uint8_t*>(Wg + (size_t)row * d) : nullptr;
    const uint8_t* px = tok < B ? reinterpret_cast<const uint8_t*>(x + (size_t)tok * d) : nullptr;

    // this wave's share of d, in runs of 64 elements (lane half h reads elements [32h, 32h+32))
    const int nrun = (d + 63) / 64;
    const int per = (nrun + UN_NW - 1) / UN_NW;
    const int r0 = wave * per, r1 = min(nrun, r0 + per);
    f32x16_t cu = {}, cg = {};
    for (int rr = r0; rr < r1; ++rr) {
        const int e0 = rr * 64 + half * 32;            // first element of this lane's run
        uint4 wa[4], ga[4], xb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int e = e0 + 8 * s;
            const bool ok = e < d;
            wa[s] = (ok && pu) ? ld16(pu + 2 * (size_t)e) : zero4();
            if (GLU) ga[s] = (ok && pg) ? ld16(pg + 2 * (size_t)e) : zero4();
            xb[s] = (ok && px) ? ld16(px + 2 * (size_t)e) : zero4();
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            cu = mfma16(wa[s], xb[s], cu);
            if (GLU) cg = mfma16(ga[s], xb[s], cg);
        }
    }
    // Reduce the 8 waves' 32 x 32 tiles.  Thread o covers outputs o and o + 512 with
    // token b = o / 32 and tile row n = o % 32, so 32 neighbouring threads store 32
    // consecutive entries of one H row.  D[n][b] sits in register (n/8)*4 + n%4 of
    // lane b + 32 * ((n/4) % 2).
    float a[2], g[2] = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) s_red[wave][r][lane] = cu[r];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int o = tid + q * UN_NW * 64, b = o >> 5, n = o & 31;
        const int rg = (n >> 3) * 4 + (n & 3), ln = b + 32 * ((n >> 2) & 1);
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < UN_NW; ++w) t += s_red[w][rg][ln];
        a[q] = t;
    }
    if (GLU) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) s_red[wave][r][lane] = cg[r];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int o = tid + q * UN_NW * 64, b = o >> 5, n = o & 31;
            const int rg = (n >> 3) * 4 + (n & 3), ln = b + 32 * ((n >> 2) & 1);
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < UN_NW; ++w) t += s_red[w][rg][ln];
            g[q] = t;
        }
    }
    const int W = (F + 31) >> 5;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int o = tid + q * UN_NW * 64, b = o >> 5, n = o & 31;
        const int k = tile * 32 + n;
        if (b >= B || k >= F) continue;
        // positions from U to the end of the last tile are written as 0: the down
        // product reads H in 8-neuron groups
        float hv = 0.f;
        if (k < U) {
            const int i = uidx[k];
            if ((unsigned)i < (unsigned)F && bit_of(tmask, W, b, i))
                hv = GLU ? fmaxf(g[q], 0.f) * a[q] : fmaxf(a[q], 0.f);
        }
        Ht[(size_t)b * F + k] = __builtin_bit_cast(uint16_t, (_Float16)hv);
    }
}

// ------------------------------------------------------------------------------------ down
PI_DEV int xcd_pair_slice(int b) {
    // slices 2m and 2m+1 (one 128-byte line of every row) on blocks b and b + 8: same XCD
    return ((b >> 4) * 8 + (b & 7)) * 2 + ((b >> 3) & 1);
}

constexpr int DN_PF = 8;   // steps of 16 neurons kept in flight per lane

__global__ __launch_bounds__(UN_NW * 64) void k_union_down(
    const uint16_t* __restrict__ Ht, int B, const uint16_t* __restrict__ Wd, int d, int F,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucount, int nslices,
    float* __restrict__ y) {
    __shared__ __align__(16) uint16_t s_t[UN_NW][32][16];      // per wave: [column][neuron]
    __shared__ float s_red[UN_NW][16][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slice = xcd_pair_slice(blockIdx.x);
    if (slice >= nslices) return;                               // padding block
    const int U = min(*ucount, F);
    const int c0 = slice * 32;                                  // first column of the slice
    const size_t rowb = (size_t)d * 2;
    // loader role: lane -> neuron r = lane / 4 of the step, 8 columns at cc = (lane % 4) * 8
    const int lr = lane >> 2, lcc = (lane & 3) * 8;
    const bool col_ok = c0 + lcc < d;
    // MFMA roles: A = Ht[token = lane % 32][k .. k+8], B = s_t[column = lane % 32][8 half ..]
    const int mtok = lane & 31, khalf = (lane >> 5) * 8;
    const int nsteps = (U + 15) / 16;
    f32x16_t acc = {};
    uint4 wbuf[DN_PF];
    // step s of this wave: global step g = s * UN_NW + wave
    auto load_step = [&](int g, uint4& dst) {
        const int k = g * 16 + lr;
        int row = k < U ? uidx[k] : -1;
        dst = (row >= 0 && row < F && col_ok) ? ld16(reinterpret_cast<const uint8_t*>(Wd) + (size_t)row * rowb + 2 * (size_t)(c0 + lcc))
                                              : zero4();
    };
    const int my_steps = nsteps > wave ? (nsteps - wave + UN_NW - 1) / UN_NW : 0;
#pragma unroll
    for (int p = 0; p < DN_PF; ++p)
        if (p < my_steps) load_step(p * UN_NW + wave, wbuf[p]);
    for (int s = 0; s < my_steps; s += DN_PF) {
#pragma unroll
        for (int p = 0; p < DN_PF; ++p) {
            if (s + p >= my_steps) break;
            const int g = (s + p) * UN_NW + wave;
            // transpose this step's 16 rows x 32 columns into the wave's LDS tile
            const uint32_t ww[4] = {wbuf[p].x, wbuf[p].y, wbuf[p].z, wbuf[p].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s_t[wave][lcc + 2 * j][lr] = (uint16_t)(ww[j] & 0xFFFFu);
                s_t[wave][lcc + 2 * j + 1][lr] = (uint16_t)(ww[j] >> 16);
            }
            // refill this slot with the step DN_PF ahead
            if (s + p + DN_PF < my_steps) load_step((s + p + DN_PF) * UN_NW + wave, wbuf[p]);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes done
            const uint4 bop = *reinterpret_cast<const uint4*>(&s_t[wave][mtok][khalf]);
            const int k = g * 16 + khalf;
            const uint4 aop = (k < U && mtok < B) ? ld16(Ht + (size_t)mtok * F + k) : zero4();
            acc = mfma16(aop, bop, acc);
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s_red[wave][r][lane] = acc[r];
    __syncthreads();
    for (int o = tid; o < 1024; o += UN_NW * 64) {
        const int r = o >> 6, l = o & 63;
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < UN_NW; ++w) t += s_red[w][r][l];
        const int b = (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);    // token (D row)
        const int col = c0 + (l & 31);                           // column (D column)
        if (b < B && col < d) y[(size_t)b * d + col] = t;
    }
}

}  // namespace

hipError_t launch_ffn_union(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x, int B,
                            const int32_t* idx, const int32_t* count, const uint32_t* token_mask,
                            int dense, float* y, char* ws, hipStream_t s) {
    (void)dense;
    uint16_t* Ht = reinterpret_cast<uint16_t*>(ws + pl.off_H);
    const int tiles = (f.F + 31) / 32;
    const uint16_t* Wg = static_cast<const uint16_t*>(f.w_gate);
    const uint16_t* Wu = static_cast<const uint16_t*>(f.w_up);
    if (f.act == PI_ACT_REGLU)
        hipLaunchKernelGGL((k_union_up<true>), dim3(tiles), dim3(UN_NW * 64), 0, s, x, B, Wg, Wu,
                           f.d, f.F, idx, count, token_mask, Ht);
    else
        hipLaunchKernelGGL((k_union_up<false>), dim3(tiles), dim3(UN_NW * 64), 0, s, x, B, Wg, Wu,
                           f.d, f.F, idx, count, token_mask, Ht);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslices = (f.d + 31) / 32;
    const int blocks = (nslices + 15) / 16 * 16;
    hipLaunchKernelGGL(k_union_down, dim3(blocks), dim3(UN_NW * 64), 0, s, Ht, B,
                       static_cast<const uint16_t*>(f.w_down), f.d, f.F, idx, count, nslices, y);
    return hipGetLastError();
}

}  // namespace pi
