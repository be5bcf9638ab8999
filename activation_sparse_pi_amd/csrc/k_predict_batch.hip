// Low-rank activation predictor for 1 < B <= 32 tokens at once, on MFMA (gfx950).
//
// PowerInfer, "Adaptive Sparsity Predictors": l = (x W_p1) W_p2 + b per token; a neuron
// is predicted active when l > theta.  With B tokens both factors are dense
// contractions with B columns:
//   stage 1  z[b, j] = W1t[j, :] . x[b, :]      (W1t = W_p1^T, [r, d] fp16)
//   stage 2  l[b, i] = W2t[i, :] . z[b, :] + b_i (W2t = W_p2^T, [F, r] fp16)
// z stays in fp32 between the stages.  Stage 1 multiplies fp16 by fp16 (products exact in
// fp32, fp32 accumulation).  Stage 2 needs z in fp32 precision on an fp16 MFMA: each token's
// z is scaled by a power of two 2^e (largest |z| brought into [2^14, 2^15)) and split into
// z_hi = fp16(z 2^e) and z_lo = fp16(z 2^e - z_hi), which carry z to 22 bits or better;
// W2t . z_hi + W2t . z_lo is accumulated in fp32 and scaled back by 2^-e (exact).
//
//   stage 1  block = 32 rows of W1t x one of KS shares of d; 8 waves split the share in
//            runs of 64 and stream rows and x through the staged 32 x 32 MFMA tile; the
//            waves meet in LDS; the shares' partial z land in the workspace and a small
//            kernel adds them in share order (a kernel boundary instead of a cross-block
//            hand-off, which costs several round trips to the memory-side cache).
//   stage 2  block = 128 neurons; waves (tile m = w % 4, half of the rank w / 4).  The
//            block's z arrives first, then all of its W2t loads are issued; z is scaled, split
//            and staged in LDS while the W2t rows are in flight; 8 MFMAs per run of 64.  The two halves meet in LDS, the bias is added,
//            and one wave ballot per 64 neurons of a token gives two mask words.  Optionally
//            the block also writes the union of the tokens' masks over its 128 neurons (4
//            words) and each neuron's token word (bit b: the neuron is in token b's mask).
#include "internal.h"
#include "mfma_tile.h"

namespace pi {
namespace {

constexpr int PB_NW = 8;      // waves per block (both stages)
constexpr int ZC = 512;       // rank values of z staged per pass in stage 2
constexpr int PB_KS = 32;     // most stage-1 shares of d
// Row pitch (floats) of a wave's 32 x 32 accumulator tile in LDS: lane l of register q at
// q RP + l.  The reads take one token's 32 rows across the lanes, i.e. 16 registers at one lane
// offset; with a pitch of 64 they would all fall in one bank, with 65 they spread over 16.
constexpr int RP = 65;

// ------------------------------------------------------------------------------------ stage 1
__global__ __launch_bounds__(PB_NW * 64) void k_pb1(const uint16_t* __restrict__ x, int B,
                                                    const uint16_t* __restrict__ W1t, int d, int r,
                                                    int ntile, int nks, float* __restrict__ part,
                                                    float* __restrict__ z) {
    __shared__ uint4 s_st[PB_NW][2][32][8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = blockIdx.x % ntile, ks = blockIdx.x / ntile;
    const int lrow = lane >> 3;
    long long offw[4], offx[4];                       // element offsets, -1 = zero row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = tile * 32 + 8 * q + lrow;
        offw[q] = j < r ? (long long)j * d : -1;
        const int tok = 8 * q + lrow;
        offx[q] = tok < B ? (long long)tok * d : -1;
    }
    // this block's share of the full runs of 64, then this wave's part of it; the partial
    // run, if any, goes to the last wave of the last share
    const int nfull = d >> 6, pb = (nfull + nks - 1) / nks;
    const int b0 = min(nfull, ks * pb), b1 = min(nfull, b0 + pb);
    const int pw = (b1 - b0 + PB_NW - 1) / PB_NW;
    const int r0 = min(b1, b0 + wave * pw), r1 = min(b1, r0 + pw);
    f32x16_t acc[1] = {};
    // full runs through buffer resources (every byte offset below 2^31): rows past r read
    // row 0, tokens past B token 0; neither reaches a stored output
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, B * d * 2);
    const __amdgpu_buffer_rsrc_t rw[1] = {buf_rsrc(W1t, r * d * 2)};
    uint32_t ox[4], ow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        ox[q] = 2u * (uint32_t)(offx[q] < 0 ? 0 : offx[q]) + 16u * (lane & 7);
        ow[q] = 2u * (uint32_t)(offw[q] < 0 ? 0 : offw[q]) + 16u * (lane & 7);
    }
    runs_mfma_full<1, 2>(rx, ox, rw, ow, r0, r1 - r0, 1, s_st[wave], acc);
    if ((d & 63) && ks == nks - 1 && wave == PB_NW - 1) {
        const uint16_t* const Wm[1] = {W1t};
        runs_mfma<1>(x, offx, Wm, offw, d, nfull, nfull + 1, s_st[wave], acc);
    }

    float* red = reinterpret_cast<float*>(&s_st[wave][0][0][0]);   // 16 RP of its 2048 floats
#pragma unroll
    for (int q = 0; q < 16; ++q) red[q * RP + lane] = acc[0][q];
    __syncthreads();
    // outputs (row n of the tile, token b), two per thread, 32 consecutive rows per token
    float v[2];
    int ob[2], oj[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int o = tid + q * PB_NW * 64, b = o >> 5, n = o & 31;
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < PB_NW; ++w)
            t += reinterpret_cast<const float*>(&s_st[w][0][0][0])[d_reg(n) * RP + d_lane(n, b)];
        v[q] = t;
        ob[q] = b;
        oj[q] = tile * 32 + n;
    }
    if (nks == 1) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            if (ob[q] < B && oj[q] < r) z[(size_t)ob[q] * r + oj[q]] = v[q];
        return;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
        if (ob[q] < B && oj[q] < r) part[((size_t)ks * 32 + ob[q]) * r + oj[q]] = v[q];
}

// z[b, j] = the nks shares' partials of (b, j) added in share order; all loads in flight at once.
// Blocks past zblocks sum the previous union pass's deferred down shares into its y instead.
__global__ __launch_bounds__(256) void k_pbz(const float* __restrict__ part, int B, int r, int nks,
                                             float* __restrict__ z, int zblocks,
                                             const float* __restrict__ ypart, int ynks, int yB, int d,
                                             float* __restrict__ y) {
    if ((int)blockIdx.x >= zblocks) {
        reduce_share_rows(ypart, ynks, yB, d, y, (blockIdx.x - zblocks) * 256 + threadIdx.x);
        return;
    }
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= B * r) return;
    const int b = o / r, j = o - b * r;
    float pv[PB_KS];
#pragma unroll
    for (int k = 0; k < PB_KS; ++k) pv[k] = k < nks ? part[((size_t)k * 32 + b) * r + j] : 0.f;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < PB_KS; ++k)
        if (k < nks) t += pv[k];
    z[o] = t;
}

// ------------------------------------------------------------------------------------ stage 2
PI_DEV float absmax4(float m, const float4& v) {
    return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// ONE: the rank fits one pass (r <= ZC), straight-line code, z loaded before W2t
template <bool ONE>
__global__ __launch_bounds__(PB_NW * 64) void k_pb2(const float* __restrict__ z, int B,
                                                    const uint16_t* __restrict__ W2t,
                                                    const float* __restrict__ bias, int r, int F,
                                                    float theta, float* __restrict__ logits,
                                                    uint32_t* __restrict__ mask,
                                                    uint32_t* __restrict__ umask,
                                                    uint32_t* __restrict__ tokbits) {
    __shared__ uint4 s_z[2][32][ZC / 8];     // z_hi, z_lo: [token][chunk of 8, swizzled]
    __shared__ unsigned long long s_u[PB_NW][2];   // per wave: OR of its tokens' ballots
    __shared__ unsigned long long s_bal[32][2];    // per token: its ballots of the 2 x 64 neurons
    __shared__ uint4 s_w[PB_NW][33][8];      // per wave: W2t staging (32 rows), then its
                                             // accumulator tile (16 RP floats)
    __shared__ int s_e[32];                  // per-token exponent e
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 128;
    const int mt = wave & 3, kh = wave >> 2;
    const int lrow = lane >> 3, lch = lane & 7, mi = lane & 31, half = lane >> 5;
    // Every load below is unconditional (a load in a branch makes the next wait a full one):
    // rows past F read row F - 1, rank positions past r read its last 8, tokens past B token
    // 0.  z past r is zeroed before it is staged, so those W2t values meet zeros; rows past F
    // and tokens past B only reach outputs that are never written.
    // the bias of this lane's two neurons in the epilogue (n0 + lane and n0 + 64 + lane), loaded
    // now so that the epilogue's ballots do not each wait for a load
    const float bias0 = bias[min(n0 + lane, F - 1)], bias1 = bias[min(n0 + 64 + lane, F - 1)];
    const uint16_t* wrow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        wrow[q] = W2t + (size_t)min(n0 + mt * 32 + 8 * q + lrow, F - 1) * r;
    // W2t loads of one pass of the rank: this wave's 4 runs of 64, all in flight at once
    uint4 wv[4][4];
    auto load_w = [&](int c0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int e = min(c0 + kh * 256 + rr * 64 + lch * 8, r - 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) wv[rr][q] = ld16_nt(wrow[q] + e);
        }
    };
    // z of one pass: token b = tid / 16 holds chunks sub + 16 i (8 values each), i < 4
    const int b = tid >> 4, sub = tid & 15;
    const float* const zrow = z + (size_t)(b < B ? b : 0) * r;
    float4 zr[2 * (ZC / 128)];
    bool zok[ZC / 128];
    auto load_z = [&](int c0) {
#pragma unroll
        for (int i = 0; i < ZC / 128; ++i) {
            const int k = c0 + 8 * (sub + 16 * i);
            zok[i] = k < r;
            const float* p = zrow + min(k, r - 8);
            zr[2 * i] = *reinterpret_cast<const float4*>(p);
            zr[2 * i + 1] = *reinterpret_cast<const float4*>(p + 4);
        }
    };
    // z first, and waited for before the W2t rows are issued: every block reads the same 64 KB
    // of z, and issued together with the rows of all blocks it would arrive behind most of them
    // (a load also waits for every load issued before it)
    // 1. per-token exponent e: the largest |z| of the token brought into [2^14, 2^15)
    float m = 0.f;
    auto zmax = [&]() {
#pragma unroll
        for (int i = 0; i < 2 * (ZC / 128); ++i) m = zok[i / 2] ? absmax4(m, zr[i]) : m;
    };
    if constexpr (ONE) {                        // the pass's z stays in zr
        load_z(0);
        zmax();
        __builtin_amdgcn_sched_barrier(0);
        load_w(0);
        __builtin_amdgcn_sched_barrier(0);
    } else {
        load_w(0);
        for (int c0 = 0; c0 < r; c0 += ZC) {
            load_z(c0);
            zmax();
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    int E = 0;
    if (m > 0.f) (void)frexpf(m, &E);           // m = f 2^E, f in [0.5, 1)
    const int ez = m > 0.f ? 15 - E : 0;
    if (sub == 0) s_e[b] = ez;
    f32x16_t acc = {};
    for (int c0 = 0; c0 < (ONE ? 1 : r); c0 += ZC) {
        if (!ONE && c0 > 0) load_w(c0);
        if (!ONE) load_z(c0);
        __syncthreads();                       // previous pass's reads done
        // 2. stage z_hi / z_lo of this pass
#pragma unroll
        for (int i = 0; i < ZC / 128; ++i) {
            const int ch = sub + 16 * i;
            const float4 za = zok[i] ? zr[2 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 zb = zok[i] ? zr[2 * i + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float zz[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float s0 = ldexpf(zz[2 * p], ez), s1 = ldexpf(zz[2 * p + 1], ez);
                const _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
                const _Float16 l0 = (_Float16)(s0 - (float)h0), l1 = (_Float16)(s1 - (float)h1);
                hi[p] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                lo[p] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
            }
            s_z[0][b][ch ^ (b & 7)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            s_z[1][b][ch ^ (b & 7)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
        __syncthreads();
        // 3. per run: stage the W2t tile rows, 4 k-steps x (z_hi, z_lo)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
            for (int q = 0; q < 4; ++q) s_w[wave][8 * q + lrow][lch ^ lrow] = wv[rr][q];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 a = s_w[wave][mi][(2 * s + half) ^ (mi & 7)];
                const int zc = (kh * 256 + rr * 64) / 8 + 2 * s + half;
                acc = mfma16(a, s_z[0][mi][zc ^ (mi & 7)], acc);
                acc = mfma16(a, s_z[1][mi][zc ^ (mi & 7)], acc);
            }
        }
    }
    // 4. the two halves of the rank meet in LDS
    float* red = reinterpret_cast<float*>(&s_w[wave][0][0]);
#pragma unroll
    for (int q = 0; q < 16; ++q) red[q * RP + lane] = acc[q];
    __syncthreads();
    const int W = (F + 31) >> 5;
    unsigned long long uor[2] = {0ull, 0ull};
    // every LDS read of the 8 (token, half) items first (unconditional: all addresses lie in
    // the block's tiles), so that their latencies overlap instead of adding up item by item
    float sum[8];
    int es[4];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int tb = wave * 4 + (it >> 1), nh = it & 1;
        const int n = nh * 64 + lane;
        const int m = n >> 5, nl = n & 31;
        const float* r0 = reinterpret_cast<const float*>(&s_w[m][0][0]);
        const float* r1 = reinterpret_cast<const float*>(&s_w[m + 4][0][0]);
        const int o = d_reg(nl) * RP + d_lane(nl, tb);
        sum[it] = r0[o] + r1[o];
        if (nh == 0) es[it >> 1] = s_e[tb];
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int tb = wave * 4 + (it >> 1), nh = it & 1;
        const int i = n0 + nh * 64 + lane;
        bool act = false;
        if (tb < B && i < F) {
            const float l = ldexpf(sum[it], -es[it >> 1]) + (nh ? bias1 : bias0);
            act = l > theta;
            if (logits) logits[(size_t)tb * F + i] = l;
        }
        const unsigned long long bal = __ballot(act);
        uor[nh] |= bal;
        if (lane == 0) s_bal[tb][nh] = bal;           // tb < 32; 0 for tokens past B
        const int w0 = (n0 + nh * 64) >> 5;
        if (lane == 0 && tb < B) {
            if (w0 < W) mask[(size_t)tb * W + w0] = (uint32_t)bal;
            if (w0 + 1 < W) mask[(size_t)tb * W + w0 + 1] = (uint32_t)(bal >> 32);
        }
    }
    if (umask == nullptr && tokbits == nullptr) return;
    // the union over the B tokens of this block's 128 neurons: the OR of every wave's ballots
    if (lane == 0) {
        s_u[wave][0] = uor[0];
        s_u[wave][1] = uor[1];
    }
    __syncthreads();
    // token word of neuron n0 + tid: bit b = neuron in token b's mask (the ballots transposed)
    if (tokbits && tid < 128 && n0 + tid < F) {
        uint32_t t = 0u;
#pragma unroll
        for (int b = 0; b < 32; ++b) t |= (uint32_t)((s_bal[b][tid >> 6] >> (tid & 63)) & 1ull) << b;
        tokbits[n0 + tid] = t;
    }
    if (umask && tid < 4) {                          // mask word n0 / 32 + tid
        const int nh = tid >> 1;
        unsigned long long u = 0ull;
#pragma unroll
        for (int w = 0; w < PB_NW; ++w) u |= s_u[w][nh];
        const int wd = (n0 >> 5) + tid;
        if (wd < W) umask[wd] = (tid & 1) ? (uint32_t)(u >> 32) : (uint32_t)u;
    }
}

}  // namespace

void plan_pred_batch(PredPlan& p, int d, int r, int F, size_t& off) {
    (void)F;
    const int nrun = (d + 63) / 64;
    p.b_ntile = (r + 31) / 32;
    int ks = (128 + p.b_ntile - 1) / p.b_ntile;        // >= 128 stage-1 blocks
    if (ks > PB_KS) ks = PB_KS;
    if (ks > nrun) ks = nrun;
    if (ks < 1) ks = 1;
    p.b_nks = ks;
    p.off_zpart = off;
    if (ks > 1) off = align_up(off + (size_t)ks * 32 * r * sizeof(float), 256);
}

hipError_t launch_predict_batch(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x,
                                int B, float theta, float* logits, uint32_t* mask, char* ws,
                                hipStream_t s, uint32_t* umask, uint32_t* tokbits, const float* ypart,
                                int ynks, int yB, float* yprev) {
    float* z = reinterpret_cast<float*>(ws + pl.off_z);
    float* part = reinterpret_cast<float*>(ws + pl.off_zpart);
    hipLaunchKernelGGL(k_pb1, dim3(pl.b_ntile * pl.b_nks), dim3(PB_NW * 64), 0, s, x, B,
                       static_cast<const uint16_t*>(p.w_p1t),
                       p.d, p.r, pl.b_ntile, pl.b_nks, part, z);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int yblocks = ypart ? (yB * (p.d / 4) + 255) / 256 : 0;
    if (pl.b_nks > 1) {
        const int zblocks = (B * p.r + 255) / 256;
        hipLaunchKernelGGL(k_pbz, dim3(zblocks + yblocks), dim3(256), 0, s, part, B, p.r, pl.b_nks, z,
                           zblocks, ypart, ynks, yB, p.d, yprev);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (ypart && (e = launch_union_yred(ypart, ynks, yB, p.d, yprev, s)) != hipSuccess) {
        return e;
    }
    hipLaunchKernelGGL(p.r <= ZC ? k_pb2<true> : k_pb2<false>, dim3((p.F + 127) / 128),
                       dim3(PB_NW * 64), 0, s, z, B,
                       static_cast<const uint16_t*>(p.w_p2t),
                       p.bias, p.r, p.F, theta, logits, mask, umask, tokbits);
    return hipGetLastError();
}

}  // namespace pi
