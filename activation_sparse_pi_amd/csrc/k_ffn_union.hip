// Small-batch (1 < B <= 32) neuron-aware FFN on the union of the token masks, on MFMA.
//
// PowerInfer, "Neuron Aware Operator": only the rows / output vectors of listed
// neurons are read.  With B tokens, the list is the union of their predicted sets
// and every weight byte read serves all B tokens, which makes this a dense
// contraction over the union (about 2B flops per weight byte): MFMA territory.
// Each token still uses its own mask: a neuron outside token b's mask contributes
// nothing to y[b] (its h is zeroed before the down product).
//
// Global loads are always whole 128-byte lines spread over 8 lanes (16 bytes each);
// operands reach the MFMA layout through a wave-private LDS area (XOR-swizzled so
// that neither the staging writes nor the operand reads conflict).  No block barrier
// sits in either streaming loop: each wave stages and consumes its own data.
//
//   up    one block per 32-neuron tile of the union list; its 8 waves split d in runs
//         of 64 elements.  Per run a wave stages the tile's 32 rows x 128 bytes of
//         W_up (and W_gate) and the 32 tokens' x, then issues 4 (8) MFMAs.  The waves
//         meet in LDS; h = act(.) * [neuron in token b's mask] is rounded to fp16 and
//         written in the down kernel's A-operand order ("H fragments": for each group
//         of 16 union positions, 64 lanes x 16 bytes, lane l holding positions
//         8 (l / 32) .. + 7 of token l % 32), so that operand is one 1 KB load.
//   down  y[b, :] = sum_k H[b, k] W_down[u_k, :].  Block = 64 columns (one 128-byte
//         line of every row) x one of KS interleaved shares of the union list; its 8
//         waves take stages of 64 union positions round-robin.  Per stage a lane loads
//         16 bytes of 8 consecutive rows, transposes the 8 x 8 fp16 block in registers
//         into 8 column vectors of 8 positions (exactly B-operand units) and writes them
//         to LDS; then 4 K-steps x 2 column tiles of MFMA.  The waves meet in LDS; with
//         KS > 1 the shares meet in the workspace and the last-arriving block of the
//         column group adds them in a fixed order (bitwise reproducible).
#include "internal.h"
#include "mfma_tile.h"

namespace pi {
namespace {

constexpr int UP_NW = 8;      // waves per up block
constexpr int DN_NWU = 8;     // waves per down block
constexpr int DN_COLS = 64;   // columns per down block

PI_DEV bool bit_of(const uint32_t* __restrict__ mask, int W, int b, int i) {
    return (mask[(size_t)b * W + (i >> 5)] >> (i & 31)) & 1u;
}

PI_DEV uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// ------------------------------------------------------------------------------------ up
template <bool GLU>
__global__ __launch_bounds__(UP_NW * 64) void k_union_up(
    const uint16_t* __restrict__ x, int B, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, int d, int F, const int32_t* __restrict__ uidx,
    const int32_t* __restrict__ ucount, const uint32_t* __restrict__ tmask,
    uint4* __restrict__ Hf) {
    constexpr int NM = GLU ? 2 : 1;                   // weight matrices: up [, gate]
    __shared__ uint4 s_st[UP_NW][NM + 1][32][8];      // per wave: x, up [, gate] staging
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int U = min(*ucount, F);
    const int tile = blockIdx.x;
    if (tile * 32 >= U) return;                       // whole block: past the union

    // loader slot q (0..3) of a run brings row 8q + lane/8 of the tile and of x
    const int lrow = lane >> 3;
    long long offw[4], offx[4];                       // element offsets, -1 = zero row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int kp = tile * 32 + 8 * q + lrow;
        int row = kp < U ? uidx[kp] : -1;
        if ((unsigned)row >= (unsigned)F) row = -1;
        offw[q] = row < 0 ? -1 : (long long)row * d;
        const int tok = 8 * q + lrow;
        offx[q] = tok < B ? (long long)tok * d : -1;
    }
    const int nrun = (d + 63) / 64, per = (nrun + UP_NW - 1) / UP_NW;
    const int r0 = min(nrun, wave * per), r1 = min(nrun, r0 + per);
    f32x16_t acc[NM] = {};
    if constexpr (GLU) {
        const uint16_t* const Wm[2] = {Wu, Wg};
        runs_mfma<2>(x, offx, Wm, offw, d, r0, r1, s_st[wave], acc);
    } else {
        const uint16_t* const Wm[1] = {Wu};
        runs_mfma<1>(x, offx, Wm, offw, d, r0, r1, s_st[wave], acc);
    }

    // the waves meet in LDS (each wave's staging area holds its own accumulators)
    float* red = reinterpret_cast<float*>(&s_st[wave][0][0][0]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        red[r * 64 + lane] = acc[0][r];
        if constexpr (GLU) red[1024 + r * 64 + lane] = acc[1][r];
    }
    __syncthreads();
    if (tid < 128) {
        // H-fragment lane fl of group 2 tile + gg: token b = fl % 32, positions
        // 16 gg + 8 (fl / 32) + j.  D[n][b] sits in register (n/8)*4 + n%4 of lane
        // b + 32 ((n/4) % 2).
        const int fl = tid & 63, gg = tid >> 6, h = fl >> 5, b = fl & 31;
        const int W = (F + 31) >> 5;
        float hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = gg * 16 + 8 * h + j;
            const int rg = d_reg(n), ln = d_lane(n, b);
            float a = 0.f, g = 0.f;
#pragma unroll
            for (int w = 0; w < UP_NW; ++w) {
                const float* rw = reinterpret_cast<const float*>(&s_st[w][0][0][0]);
                a += rw[rg * 64 + ln];
                if constexpr (GLU) g += rw[1024 + rg * 64 + ln];
            }
            const int k = tile * 32 + gg * 16 + 8 * h + j;
            float v = 0.f;                     // positions past U and tokens past B give 0
            if (k < U && b < B) {
                const int i = uidx[k];
                if ((unsigned)i < (unsigned)F && bit_of(tmask, W, b, i))
                    v = GLU ? fmaxf(g, 0.f) * a : fmaxf(a, 0.f);
            }
            hv[j] = v;
        }
        Hf[(size_t)(tile * 2 + gg) * 64 + fl] =
            make_uint4(pack_h2(hv[0], hv[1]), pack_h2(hv[2], hv[3]), pack_h2(hv[4], hv[5]),
                       pack_h2(hv[6], hv[7]));
    }
}

// ------------------------------------------------------------------------------------ down
// column c of a stage keeps k-block kb in unit kb * 64 + (c ^ ((c >> 3) & 7))
PI_DEV int dn_slot(int c) { return c ^ ((c >> 3) & 7); }

__global__ __launch_bounds__(DN_NWU * 64) void k_union_down(
    const uint4* __restrict__ Hf, int B, const uint16_t* __restrict__ Wd, int d, int F,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucount, int ncg, int nks,
    float* __restrict__ part, unsigned* __restrict__ counter, float* __restrict__ y) {
    __shared__ uint4 s_t[DN_NWU][8][64];             // per wave: k-block, swizzled column unit
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cgi = blockIdx.x % ncg, ks = blockIdx.x / ncg;
    const int U = min(*ucount, F);
    const int c0 = cgi * DN_COLS;
    const int nst = (U + 63) / 64;                    // stages of 64 union positions
    const int nw = nks * DN_NWU;                      // waves sharing the list
    // loader role: lane -> rows 8 rbk .. 8 rbk + 7 of a stage, columns 8 ch .. 8 ch + 7
    const int rbk = lane >> 3, ch = lane & 7;
    const bool col_ok = c0 + ch * 8 < d;
    // MFMA role: B column n of each 32-column tile, k half h
    const int n = lane & 31, h = lane >> 5;
    const int slot0 = dn_slot(n), slot1 = dn_slot(32 + n);
    uint4(*st)[64] = s_t[wave];

    f32x16_t acc0 = {}, acc1 = {};
    int rows[8];
    uint4 R[8], Rn[8], A[4], An[4];
    auto load_rows = [&](int s) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = s * 64 + rbk * 8 + j;
            int r = (s < nst && k < U) ? uidx[k] : -1;
            rows[j] = (unsigned)r < (unsigned)F ? r : -1;
        }
    };
    auto load_w = [&](uint4(&v)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = (rows[j] >= 0 && col_ok) ? ld16(Wd + (size_t)rows[j] * d + c0 + ch * 8) : zero4();
    };
    auto load_a = [&](int s, uint4(&a)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int g = s * 4 + q;                  // group of 16 positions
            a[q] = g * 16 < U ? Hf[(size_t)g * 64 + lane] : zero4();
        }
    };
    int s = ks * DN_NWU + wave;
    if (s < nst) {
        load_rows(s);
        load_w(R);
        load_a(s, A);
        load_rows(s + nw);
    }
    for (; s < nst; s += nw) {
        const int sn = s + nw;
        if (sn < nst) {
            load_w(Rn);
            load_a(sn, An);
            load_rows(sn + nw);
        }
        // 8 x 8 transpose: unit e = column 8 ch + e over rows 8 rbk .. 8 rbk + 7
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t o[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = (&R[2 * p].x)[e >> 1], hi = (&R[2 * p + 1].x)[e >> 1];
                o[p] = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
            }
            st[rbk][8 * ch + (e ^ ch)] = make_uint4(o[0], o[1], o[2], o[3]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kb = 2 * q + h;
            acc0 = mfma16(A[q], st[kb][slot0], acc0);
            acc1 = mfma16(A[q], st[kb][slot1], acc1);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) R[j] = Rn[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) A[q] = An[q];
    }

    // the waves meet in LDS
    float* red = reinterpret_cast<float*>(&s_t[wave][0][0]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        red[r * 64 + lane] = acc0[r];
        red[1024 + r * 64 + lane] = acc1[r];
    }
    __syncthreads();
    // 32 tokens x 64 columns, four per thread; output o: tile o / 1024, register
    // (o / 64) % 16, lane o % 64
    float v[4];
    int ob[4], oc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int o = tid + q * DN_NWU * 64;
        const int nt = o >> 10, r = (o >> 6) & 15, l = o & 63;
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < DN_NWU; ++w)
            t += reinterpret_cast<const float*>(&s_t[w][0][0])[nt * 1024 + r * 64 + l];
        v[q] = t;
        ob[q] = (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
        oc[q] = c0 + nt * 32 + (l & 31);
    }
    if (nks == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (ob[q] < B && oc[q] < d) y[(size_t)ob[q] * d + oc[q]] = v[q];
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (ob[q] < B && oc[q] < d) st_agent(&part[((size_t)ks * 32 + ob[q]) * d + oc[q]], v[q]);
    if (!last_block_arrive(&counter[cgi], nks)) return;
    // the other shares' partials, up to 16 loads in flight per round, added in share order
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nks; k0 += 4) {
        float pv[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k2 = k0 + i;
                pv[q][i] = (k2 < nks && k2 != ks && ob[q] < B && oc[q] < d)
                               ? ld_agent(&part[((size_t)k2 * 32 + ob[q]) * d + oc[q]]) : 0.f;
            }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (k0 + i < nks) t[q] += k0 + i == ks ? v[q] : pv[q][i];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (ob[q] < B && oc[q] < d) y[(size_t)ob[q] * d + oc[q]] = t[q];
}

}  // namespace

size_t plan_union(FfnPlan& p, int d, int F, size_t off) {
    p.off_H = off;
    off = align_up(off + (size_t)((F + 31) / 32) * 2048, 256);   // H fragments, 2 KB per tile
    p.u_ncg = (d + DN_COLS - 1) / DN_COLS;
    int ks = (256 + p.u_ncg - 1) / p.u_ncg;                      // >= 256 down blocks
    p.u_ks = ks < 1 ? 1 : (ks > 16 ? 16 : ks);
    p.off_upart = off;
    if (p.u_ks > 1) off = align_up(off + (size_t)p.u_ks * 32 * d * sizeof(float), 256);
    return off;
}

hipError_t launch_ffn_union(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x, int B,
                            const int32_t* idx, const int32_t* count, const uint32_t* token_mask,
                            float* y, char* ws, hipStream_t s) {
    uint4* Hf = reinterpret_cast<uint4*>(ws + pl.off_H);
    const int tiles = (f.F + 31) / 32;
    const uint16_t* Wg = static_cast<const uint16_t*>(f.w_gate);
    const uint16_t* Wu = static_cast<const uint16_t*>(f.w_up);
    if (f.act == PI_ACT_REGLU)
        hipLaunchKernelGGL((k_union_up<true>), dim3(tiles), dim3(UP_NW * 64), 0, s, x, B, Wg, Wu,
                           f.d, f.F, idx, count, token_mask, Hf);
    else
        hipLaunchKernelGGL((k_union_up<false>), dim3(tiles), dim3(UP_NW * 64), 0, s, x, B, Wg, Wu,
                           f.d, f.F, idx, count, token_mask, Hf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    unsigned* cnt = reinterpret_cast<unsigned*>(ws) + CNT_UNION;
    float* part = reinterpret_cast<float*>(ws + pl.off_upart);
    hipLaunchKernelGGL(k_union_down, dim3(pl.u_ncg * pl.u_ks), dim3(DN_NWU * 64), 0, s, Hf, B,
                       static_cast<const uint16_t*>(f.w_down), f.d, f.F, idx, count, pl.u_ncg,
                       pl.u_ks, part, cnt, y);
    return hipGetLastError();
}

}  // namespace pi
