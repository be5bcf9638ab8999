// 32 x 32 MFMA tiles over rows of fp16 matrices, fed through a wave-private LDS area.
//
// v_mfma_f32_32x32x16_f16 (gfx950) lane layout, checked on the device:
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + j], j < 8
//   B (16 x 32): lane l holds B[8 * (l / 32) + j][l % 32]
//   D (32 x 32): lane l, register r holds D[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32]
// The k slots of one MFMA may be any permutation shared by A and B.
#pragma once

#include "device_common.h"

namespace pi {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

PI_DEV f32x16_t mfma16(const uint4& a, const uint4& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// D[n][b] of a 32 x 32 accumulator: register and lane
PI_DEV int d_reg(int n) { return (n >> 3) * 4 + (n & 3); }
PI_DEV int d_lane(int n, int b) { return b + 32 * ((n >> 2) & 1); }

// acc[m] += W_m[rows] . x[rows]^T over runs [r0, r1) of 64 elements of d-element rows.
// Rows are given per loader slot: load q (0..3) of a run brings row 8q + lane/8 (element
// offsets offw[q] into every W_m, offx[q] into x; -1 = a zero row), 16 bytes at chunk
// lane % 8 of the run, so every global load is 8 full 128-byte lines.  st is the wave's
// staging area, [NM + 1][32][8] units of 16 bytes: row r keeps chunk c in slot c ^ (r % 8),
// which leaves both the staging writes and the operand reads free of bank conflicts.
// Two register sets keep the run after next in flight while one run is consumed.
template <int NM>
PI_DEV void runs_mfma(const uint16_t* __restrict__ x, const long long (&offx)[4],
                      const uint16_t* const (&W)[NM], const long long (&offw)[4], int d, int r0,
                      int r1, uint4 (*st)[32][8], f32x16_t (&acc)[NM]) {
    constexpr int NP = NM + 1;
    const int lane = threadIdx.x & 63;
    const int lrow = lane >> 3, lch = lane & 7;
    const int mi = lane & 31, half = lane >> 5;
    uint4 ra[NP][4], rb[NP][4];
    auto load = [&](int rr, uint4(&v)[NP][4]) {
        const int e = rr * 64 + lch * 8;
        const bool ok = e < d;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[0][q] = (ok && offx[q] >= 0) ? ld16(x + offx[q] + e) : zero4();
#pragma unroll
            for (int m = 0; m < NM; ++m)
                v[m + 1][q] = (ok && offw[q] >= 0) ? ld16_nt(W[m] + offw[q] + e) : zero4();
        }
    };
    auto stage = [&](const uint4(&v)[NP][4]) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) st[p][8 * q + lrow][lch ^ lrow] = v[p][q];
    };
    // k-step s takes chunk 2s + half of row mi: k-slot 8 half + j <-> element 16 s + 8 half + j
    auto compute = [&]() {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int slot = (2 * s + half) ^ (mi & 7);
            const uint4 bx = st[0][mi][slot];
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[m] = mfma16(st[m + 1][mi][slot], bx, acc[m]);
        }
    };
    if (r0 < r1) load(r0, ra);
    if (r0 + 1 < r1) load(r0 + 1, rb);
    for (int rr = r0; rr < r1; rr += 2) {
        stage(ra);
        if (rr + 2 < r1) load(rr + 2, ra);
        compute();
        if (rr + 1 < r1) {
            stage(rb);
            if (rr + 3 < r1) load(rr + 3, rb);
            compute();
        }
    }
}

// runs_mfma over the full runs r0, r0 + rs, .. (n of them, every one inside the rows), rows
// read through buffer resources: loader slot q takes byte offset ox[q] into x (resource rx) and
// ow[q] into every W_m (resource rw[m], non-temporal), plus 128 bytes per run.  NB runs are
// in flight per wave: a run's registers are refilled with the run NB ahead as soon as they
// are staged.  The steady loop issues every load unconditionally and is unrolled NB times so
// the buffers rotate without copies; a scheduling barrier after each run's loads keeps them
// together, so that (vector loads completing in order) waiting for the oldest run never
// waits for younger ones.
template <int NM, int NB>
PI_DEV void runs_mfma_full(__amdgpu_buffer_rsrc_t rx, const uint32_t (&ox)[4],
                           const __amdgpu_buffer_rsrc_t (&rw)[NM], const uint32_t (&ow)[4],
                           int r0, int n, int rs, uint4 (*st)[32][8], f32x16_t (&acc)[NM]) {
    constexpr int NP = NM + 1;
    const int lane = threadIdx.x & 63;
    const int lrow = lane >> 3, lch = lane & 7;
    const int mi = lane & 31, half = lane >> 5;
    uint4 v[NB][NP][4];
    auto load = [&](int j, uint4(&b)[NP][4]) {
        const int so = (r0 + j * rs) * 128;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            b[0][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ox[q], so, 0));
#pragma unroll
            for (int m = 0; m < NM; ++m)
                b[m + 1][q] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw[m], ow[q], so, PI_NT));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage = [&](const uint4(&b)[NP][4]) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) st[p][8 * q + lrow][lch ^ lrow] = b[p][q];
    };
    auto compute = [&]() {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int slot = (2 * s + half) ^ (mi & 7);
            const uint4 bx = st[0][mi][slot];
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[m] = mfma16(st[m + 1][mi][slot], bx, acc[m]);
        }
    };
    const int r1 = n;               // runs are counted from 0 below
    if (r1 < NB) {
        for (int rr = 0; rr < r1; ++rr) {
            load(rr, v[0]);
            stage(v[0]);
            compute();
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) load(k, v[k]);
    int rr = 0;
    for (; rr + 2 * NB - 1 < r1; rr += NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            stage(v[k]);
            load(rr + k + NB, v[k]);
            compute();
        }
    }
    // fewer than 2 NB runs remain, the first NB of them loaded
#pragma unroll
    for (int k = 0; k < 2 * NB - 1; ++k) {
        if (rr + k < r1) {
            stage(v[k % NB]);
            if (rr + k + NB < r1) load(rr + k + NB, v[k % NB]);
            compute();
        }
    }
}

}  // namespace pi
