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
//   up    one block per 32-neuron tile of the union list; its 8 waves split d in runs of 64
//         elements.  The tile's ids come from the union list, or straight from the union mask
//         (a block-wide scan of its words' popcounts locates the tile's 32 positions, which
//         the block writes to the list for the down kernel).  Per token a keep word (bit n:
//         position n of the tile is in that token's mask) comes from the per-neuron token
//         words (loaded with the first rows, transposed after streaming) or, for a given list,
//         from the token masks before streaming.  Per run a wave stages the tile's 32 rows x
//         128 bytes of W_up (and W_gate) and the 32 tokens' x, then issues 4 (8) MFMAs.  The
//         waves meet in LDS; h = act(.) * keep is rounded to fp16 and written in the down kernel's A-operand order ("H fragments": for each group
//         of 16 union positions, 64 lanes x 16 bytes, lane l holding positions
//         8 (l / 32) .. + 7 of token l % 32), so that operand is one 1 KB load.
//   down  y[b, :] = sum_k H[b, k] W_down[u_k, :].  Block = 256 columns (512 contiguous
//         bytes of every row) x one of KS interleaved shares of the union list; its 8 waves
//         take stages of 16 union positions round-robin.  Per stage a lane loads 16 bytes of
//         8 consecutive rows, transposes the 8 x 8 fp16 block in registers into 8 column
//         vectors of 8 positions (exactly B-operand units) and writes them to LDS; then one
//         MFMA per 32-column tile (8 per stage) with the stage's H fragment as A.  Wide
//         blocks read long pieces of each row and re-read the H fragments (from L2) for
//         fewer columns.  The waves meet in LDS; with KS > 1 the shares meet in the
//         workspace and the last-arriving block of the column group adds them in a fixed
//         order (bitwise reproducible).
#include <algorithm>
#include <climits>
#include <map>
#include <mutex>
#include <utility>

#include "internal.h"
#include "mfma_tile.h"

namespace pi {
namespace {

constexpr int UP_NW = 8;      // waves per up block
constexpr int UP_NT = UP_NW * 64;
constexpr int DN_NWU = 4;     // waves per down block (one per SIMD)
constexpr int DN_COLS = 256;  // columns per down block
constexpr int DN_TILES = DN_COLS / 32;   // 32-column MFMA tiles per down block

// The ids at union positions lo .. lo + 31 from the union mask, whose set bits among the first
// F are the union in ascending order: every thread takes runs of 4 consecutive words and an
// exclusive scan of the runs' popcounts gives each run its first position; then each wave walks
// its runs that hold positions of the tile (usually a handful), one word at a time with one
// lane per bit, and writes those ids to s_ids.  Returns the union's size U (block-uniform).
// s_tmp: UP_NW + 1 ints.
PI_DEV int tile_ids_from_mask(const uint32_t* __restrict__ umask, int F, int lo, int* s_ids,
                              int* s_tmp) {
    const int W = (F + 31) >> 5, hi = lo + 32, lane = threadIdx.x & 63;
    int base = 0;
    for (int c0 = 0; c0 < W; c0 += 4 * UP_NT) {
        const int w0 = c0 + 4 * (int)threadIdx.x;
        uint32_t v[4];
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int w = w0 + k;
            uint32_t m = w < W ? umask[w] : 0u;
            if (w == W - 1 && (F & 31)) m &= (1u << (F & 31)) - 1u;       // bits past F
            v[k] = m;
            cnt += __popc(m);
        }
        int total;
        const int pos = base + block_exclusive_scan(cnt, s_tmp, &total);
        unsigned long long hit = __ballot(pos < hi && pos + cnt > lo);
        while (hit) {                                 // wave-uniform
            const int j = __builtin_ctzll(hit);
            hit &= hit - 1ull;
            int r = __builtin_amdgcn_readlane(pos, j);
            const int wj = __builtin_amdgcn_readlane(w0, j);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t vk = (uint32_t)__builtin_amdgcn_readlane((int)v[k], j);
                if (lane < 32 && ((vk >> lane) & 1u)) {
                    const int rank = r + __popc(vk & ((1u << lane) - 1u));
                    if (rank >= lo && rank < hi) s_ids[rank - lo] = ((wj + k) << 5) + lane;
                }
                r += __popc(vk);
            }
        }
        base += total;
    }
    return base;
}

PI_DEV uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// ------------------------------------------------------------------------------------ up
// Block roles.  The first S blocks (S: as many as are resident at once) take whole tiles
// 0 .. S - 1.  The tiles past them would run as a second round behind the first, one block each;
// instead each is split over d into sp parts (sp = 2 when the layer has more than S tiles), so
// the second round has twice the blocks in flight at half the length.  A part stores its
// 32 x 32 pre-activation sums; the last part of the tile to arrive adds the sp partials in part
// order and finishes the tile.  The split blocks go in groups of 8 sp: block r of group g takes
// part r / 8 of tile S + 8 g + r % 8, so the parts of a tile are 8 blocks apart in the dispatch
// order -- on one XCD (S is a multiple of 8), their hand-off inside one L2.  A last group of
// m < 8 tiles pairs block r with tile S + 8 g + r % m, part r / m.
constexpr int UP_SP = 2;
struct UpRole {
    int tile, part, sp;
};
PI_DEV UpRole up_role(int b, int S, int sp, int tiles) {
    if (b < S || sp == 1) return {b, 0, 1};
    const int bb = b - S, g = bb / (8 * sp), r = bb - g * 8 * sp;
    const int m = min(8, tiles - S - 8 * g);
    return {S + 8 * g + r % m, r / m, sp};
}

// ReLU with 32-bit offsets fits 128 registers: two blocks per CU (ReGLU: one).
// FROM_MASK: the tile's ids come from the union mask umask and are written to uidx[32 tile ..]
// (block 0 writes U to *ucount), the keep words from the token words tokbits[F]; otherwise the
// ids are read from the union list uidx[0 .. *ucount) and the keep words from the token masks
// tmask [B, ceil(F / 32)].  S, sp: the block roles above; upart / ucnt: the split tiles'
// partials and arrival counters.
template <bool GLU, bool OFF32, bool FROM_MASK>
__global__ __launch_bounds__(UP_NT, GLU || !OFF32 ? 2 : 4) void k_union_up(
    const uint16_t* __restrict__ x, int B, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, int d, int F, const uint32_t* __restrict__ umask,
    const uint32_t* __restrict__ tokbits, int32_t* __restrict__ uidx, int32_t* __restrict__ ucount,
    const uint32_t* __restrict__ tmask, int S, int sp, float* __restrict__ upart,
    unsigned* __restrict__ ucnt, uint4* __restrict__ Hf) {
    constexpr int NM = GLU ? 2 : 1;                   // weight matrices: up [, gate]
    __shared__ uint4 s_st[UP_NW][NM + 1][32][8];      // per wave: x, up [, gate] staging
    __shared__ int s_ids[32];                         // the tile's neuron ids, -1 past the union
    __shared__ uint32_t s_keep[32];                   // per token: bit n = position n in its mask
    __shared__ int s_tmp[UP_NW + 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < 32) s_ids[tid] = -1;
    const UpRole ro = up_role(blockIdx.x, S, sp, (F + 31) >> 5);
    const int tile = ro.tile, lo = tile * 32;
    uint32_t tok = 0u;             // FROM_MASK, wave 0 lane n < 32: token word of position n
    if constexpr (FROM_MASK) {
        const int U = __builtin_amdgcn_readfirstlane(tile_ids_from_mask(umask, F, lo, s_ids, s_tmp));   // its barriers order the -1s
        if (blockIdx.x == 0 && tid == 0) *ucount = U; // also when the union is empty
        if (lo >= U) return;                          // whole block: past the union
        __syncthreads();
        if (tid < 32) {
            const int id = s_ids[tid];
            if (ro.part == 0 && lo + tid < U) uidx[lo + tid] = id;
            tok = (unsigned)id < (unsigned)F ? tokbits[id] : 0u;        // used after streaming
        }
    } else {
        const int U = min(*ucount, F);
        if (lo >= U) return;
        if (tid < 32 && lo + tid < U) s_ids[tid] = uidx[lo + tid];
        __syncthreads();
        // keep words from the token masks: pair p = (token p / 32, position p % 32), a wave's
        // ballot covers two tokens; every load of a thread is issued before the first ballot
        const int W = (F + 31) >> 5;
        constexpr int NP = 1024 / UP_NT;
        uint32_t wv[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int p = tid + k * UP_NT, b = p >> 5, id = s_ids[p & 31];
            wv[k] = tmask[(size_t)min(b, B - 1) * W + ((unsigned)id < (unsigned)F ? id >> 5 : 0)];
        }
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int p = tid + k * UP_NT, b = p >> 5, id = s_ids[p & 31];
            const bool kb = b < B && (unsigned)id < (unsigned)F && ((wv[k] >> (id & 31)) & 1u);
            const unsigned long long bal = __ballot(kb);
            if (lane == 0) {
                s_keep[b] = (uint32_t)bal;
                s_keep[b + 1] = (uint32_t)(bal >> 32);
            }
        }
    }

    // loader slot q (0..3) of a run brings row 8q + lane/8 of the tile and of x (element
    // offsets, -1 = zero row; recomputed where needed rather than kept across the stream)
    const int lrow = lane >> 3;
    auto offsets = [&](long long(&offw)[4], long long(&offx)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = s_ids[8 * q + lrow];
            offw[q] = (unsigned)row < (unsigned)F ? (long long)row * d : -1;
            const int tk = 8 * q + lrow;
            offx[q] = tk < B ? (long long)tk * d : -1;
        }
    };
    // this part's runs of 64 (the partial run, if any, belongs to the last part), then this
    // wave's share of them
    f32x16_t acc[NM] = {};
    if constexpr (OFF32) {
        long long offw[4], offx[4];
        offsets(offw, offx);
        // full runs through buffer resources (byte offsets of F rows fit 31 bits): zero rows
        // read row 0 of W and x instead, their h is zeroed below; the partial run, if any,
        // goes the general way
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, B * d * 2);
        __amdgpu_buffer_rsrc_t rw[NM];
        rw[0] = buf_rsrc(Wu, F * d * 2);
        if constexpr (GLU) rw[1] = buf_rsrc(Wg, F * d * 2);
        uint32_t ox[4], ow[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ox[q] = 2u * (uint32_t)(offx[q] < 0 ? 0 : offx[q]) + 16u * (lane & 7);
            ow[q] = 2u * (uint32_t)(offw[q] < 0 ? 0 : offw[q]) + 16u * (lane & 7);
        }
        const int nfull = d >> 6;
        const int p0 = ro.part * nfull / ro.sp, p1 = (ro.part + 1) * nfull / ro.sp;
        // the waves take the part's runs in turn (wave w: runs p0 + w, p0 + w + 8, ..), so the
        // block reads neighbouring 128-byte pieces of its 32 rows together
        const int r0 = p0 + wave, nr = r0 < p1 ? (p1 - r0 + UP_NW - 1) / UP_NW : 0;
        runs_mfma_full<NM, 2>(rx, ox, rw, ow, r0, nr, UP_NW, s_st[wave], acc);
        if ((d & 63) && wave == UP_NW - 1 && ro.part == ro.sp - 1) {
            const uint16_t* Wm[NM];
            Wm[0] = Wu;
            if constexpr (GLU) Wm[1] = Wg;
            long long offw2[4], offx2[4];
            offsets(offw2, offx2);
            runs_mfma<NM>(x, offx2, Wm, offw2, d, nfull, nfull + 1, s_st[wave], acc);
        }
    } else {
        long long offw[4], offx[4];
        offsets(offw, offx);
        const int nrun = (d + 63) / 64;
        const int p0 = ro.part * nrun / ro.sp, p1 = (ro.part + 1) * nrun / ro.sp;
        const int per = (p1 - p0 + UP_NW - 1) / UP_NW;
        const int r0 = min(p1, p0 + wave * per), r1 = min(p1, r0 + per);
        const uint16_t* Wm[NM];
        Wm[0] = Wu;
        if constexpr (GLU) Wm[1] = Wg;
        runs_mfma<NM>(x, offx, Wm, offw, d, r0, r1, s_st[wave], acc);
    }

    if constexpr (FROM_MASK) {
        // keep word of token b = bit b of the 32 positions' token words (lanes 32.. hold 0)
        if (wave == 0) {
#pragma unroll
            for (int b = 0; b < 32; ++b) {
                const unsigned long long bal = __ballot((tok >> b) & 1u);
                if (lane == 0) s_keep[b] = b < B ? (uint32_t)bal : 0u;
            }
        }
    }
    // the waves meet in LDS (each wave's staging area holds its own accumulators)
    float* red = reinterpret_cast<float*>(&s_st[wave][0][0][0]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        red[r * 64 + lane] = acc[0][r];
        if constexpr (GLU) red[1024 + r * 64 + lane] = acc[1][r];
    }
    __syncthreads();
    // H-fragment lane fl of group 2 tile + gg: token b = fl % 32, positions 16 gg + 8 (fl / 32)
    // + j.  D[n][b] sits in register (n/8)*4 + n%4 of lane b + 32 ((n/4) % 2).
    const int fl = tid & 63, gg = (tid >> 6) & 1, h = fl >> 5, b = fl & 31;
    float av[8], gv[8];
    if (tid < 128) {
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
            av[j] = a;
            gv[j] = g;
        }
    }
    if (ro.sp > 1) {
        // split tile: this part's sums to the workspace; the last part to arrive adds all of
        // them in part order (its own from registers)
        const size_t slot = (size_t)(tile - S) * ro.sp;
        auto at = [&](int p) { return upart + ((slot + p) * 128 + tid) * (8 * NM); };
        if (tid < 128) {
            float* my = at(ro.part);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                st_agent(my + j, av[j]);
                if constexpr (GLU) st_agent(my + 8 + j, gv[j]);
            }
        }
        if (!last_block_arrive(&ucnt[tile - S], ro.sp)) return;
        if (tid < 128) {
            float pa[UP_SP][8], pg[UP_SP][8];
#pragma unroll
            for (int p = 0; p < UP_SP; ++p) {
                const float* src = at(p < ro.sp ? p : 0);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pa[p][j] = p < ro.sp && p != ro.part ? ld_agent(src + j) : 0.f;
                    pg[p][j] = GLU && p < ro.sp && p != ro.part ? ld_agent(src + 8 + j) : 0.f;
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float a = 0.f, g = 0.f;
#pragma unroll
                for (int p = 0; p < UP_SP; ++p) {
                    if (p >= ro.sp) continue;
                    a += p == ro.part ? av[j] : pa[p][j];
                    g += p == ro.part ? gv[j] : pg[p][j];
                }
                av[j] = a;
                gv[j] = g;
            }
        }
    }
    if (tid < 128) {
        const uint32_t keep = s_keep[b];              // 0 for tokens past B
        float hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = gg * 16 + 8 * h + j;
            // positions past U, invalid ids and tokens past B have no keep bit: h = 0
            hv[j] = (keep >> n) & 1u ? (GLU ? fmaxf(gv[j], 0.f) * av[j] : fmaxf(av[j], 0.f)) : 0.f;
        }
        Hf[(size_t)(tile * 2 + gg) * 64 + fl] =
            make_uint4(pack_h2(hv[0], hv[1]), pack_h2(hv[2], hv[3]), pack_h2(hv[4], hv[5]),
                       pack_h2(hv[6], hv[7]));
    }
}

// ------------------------------------------------------------------------------------ down
// Loads: one instruction brings 512 contiguous bytes (the block's 256 columns) of one row,
// 8 bytes per lane, from a wave-uniform row address (row ids move to scalar registers) and a
// fixed per-lane offset.  Loader lane l takes column chunk pl(l) (4 columns); after 16 rows
// (a stage) it holds 4 columns x 16 positions, transposed in registers into 8 B-operand
// units (column 4 pl + e, k-half hh: 8 positions).
// Stage layout (16-byte units): unit(4 m + e, hh) = hh * DN_HS + 65 e + q(m), with
//   q(m) = g(m / 8) + z(m % 8),  g(t) = 2 (t % 2) + 16 (t / 2),  z(i) = 4 (i % 4) + i / 4,
// so a staging write is base(l) + hh * DN_HS + 65 e and the operand read of tile t is
// base(n) + g(t): one address register each, the rest immediate offsets.  With
//   pl(l) = 8 t + i,  t = 2 (l / 16) + (l / 4) % 2,  i = l % 2 + 2 ((l / 8) % 2) + 4 ((l / 2) % 2)
// both the writes and the reads touch distinct banks within every group of 8 and of 16 lanes.
constexpr int DN_HS = 4 * 65;                 // units per k-half
constexpr int DN_NB = 3;                      // stages in flight per wave
PI_DEV int dn_g(int t) { return 2 * (t & 1) + 16 * (t >> 1); }
PI_DEV int dn_z(int i) { return 4 * (i & 3) + (i >> 2); }

// Pipeline (per wave, its stages s, s + nw, s + 2 nw, ...): DN_NB stages of rows in flight;
// the row ids of a stage are loaded 2 DN_NB - 1 stages ahead, before the rows of the stage
// DN_NB - 1 ahead, so that (loads completing in order) waiting for ids never waits for rows
// in flight.  The steady loop issues every load unconditionally and is unrolled DN_NB times
// so the buffers rotate without copies; the last stages run in a drain whose waits may be
// conservative.
__global__ __launch_bounds__(DN_NWU * 64) void k_union_down(
    const uint4* __restrict__ Hf, int B, const uint16_t* __restrict__ Wd, int d, int F,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucount, int ncg, int nks,
    float* __restrict__ part, unsigned* __restrict__ counter, float* __restrict__ y, int defer) {
    constexpr int NB = DN_NB;
    __shared__ uint4 s_t[DN_NWU][2 * DN_HS];         // per wave: two k-halves x 256 column units
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cgi = blockIdx.x % ncg, ks = blockIdx.x / ncg;
    const int U = min(*ucount, F);
    const int c0 = cgi * DN_COLS;
    const int nst = (U + 15) / 16;                    // stages of 16 union positions
    const int nw = nks * DN_NWU;                      // waves sharing the list
    // loader role: columns 4 pl .. 4 pl + 3 of the block (byte offset voff of each row piece;
    // columns past d read the block's first columns and only reach outputs never written)
    const int pl = 8 * (2 * (lane >> 4) + ((lane >> 2) & 1)) + (lane & 1) + 2 * ((lane >> 3) & 1) +
                   4 * ((lane >> 1) & 1);
    const uint32_t voff = c0 + 4 * pl < d ? 8u * pl : 0u;
    // MFMA role: B column n of each 32-column tile, k half h
    const int n = lane & 31, h = lane >> 5;
    uint4* const stw = s_t[wave] + dn_g(pl >> 3) + dn_z(pl & 7);                        // writes
    const uint4* const str = s_t[wave] + h * DN_HS + 65 * (n & 3) + dn_z(n >> 2);        // reads

    f32x16_t acc[DN_TILES];
#pragma unroll
    for (int t = 0; t < DN_TILES; ++t) acc[t] = f32x16_t{};
    // a stage's 16 row ids: lane l holds the id at position l % 16 (clamped into the list)
    auto load_ids = [&](int st_) { return uidx[min(st_ * 16 + (lane & 15), U - 1)]; };
    // issue the rows of stage st_ and return its (wave-uniform) mask of rows to zero: a
    // position past the union, or holding an id outside [0, F), reads row 0
    auto load_w = [&](int st_, int ids, uint2(&v)[16]) {
        unsigned bad = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int id = __builtin_amdgcn_readlane(ids, j);
            const bool ok = st_ * 16 + j < U && (unsigned)id < (unsigned)F;
            bad |= ok ? 0u : 1u << j;
            const char* row = reinterpret_cast<const char*>(Wd + ((size_t)(ok ? id : 0) * d + c0));
            v[j] = ld8_nt(row + voff);
        }
        return bad;
    };
    auto load_a = [&](int st_) { return Hf[(size_t)st_ * 64 + lane]; };
    // stage: zero the invalid rows, transpose into 8 units (column 4 pl + e, k-half hh), write
    // them to the wave's LDS area, one MFMA per 32-column tile
    auto stage = [&](unsigned bad, uint2(&R)[16], const uint4& A) {
        if (bad) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if ((bad >> j) & 1u) R[j] = make_uint2(0u, 0u);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t o[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint2& lo = R[8 * hh + 2 * p];
                    const uint2& hi = R[8 * hh + 2 * p + 1];
                    o[p] = __builtin_amdgcn_perm((e >> 1) ? hi.y : hi.x, (e >> 1) ? lo.y : lo.x,
                                                 (e & 1) ? 0x07060302u : 0x05040100u);
                }
                stw[hh * DN_HS + 65 * e] = make_uint4(o[0], o[1], o[2], o[3]);
            }
#pragma unroll
        for (int t = 0; t < DN_TILES; ++t) acc[t] = mfma16(A, str[dn_g(t)], acc[t]);
    };

    int s = ks * DN_NWU + wave;
    uint2 R[NB][16];
    uint4 A[NB];
    unsigned bad[NB];
    int ids[NB];
    if (s + (2 * NB - 1) * nw < nst) {
        // ids slot b holds the ids of stage s + (b + NB) nw, buffer b the rows of s + b nw
        int id0[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) id0[b] = load_ids(s + b * nw);
#pragma unroll
        for (int b = 0; b < NB; ++b) ids[b] = load_ids(s + (b + NB) * nw);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            bad[b] = load_w(s + b * nw, id0[b], R[b]);
            A[b] = load_a(s + b * nw);
        }
        do {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                // stage s + b nw: refill its buffer with stage s + (b + NB) nw (ids in slot b),
                // then load the ids of stage s + (b + 2 NB) nw into slot b
                stage(bad[b], R[b], A[b]);
                const int nid = load_ids(s + (b + 2 * NB) * nw);
                asm volatile("" ::: "memory");
                bad[b] = load_w(s + (b + NB) * nw, ids[b], R[b]);
                A[b] = load_a(s + (b + NB) * nw);
                ids[b] = nid;
            }
            s += NB * nw;
        } while (s + (2 * NB - 1) * nw < nst);
        // drain: buffers hold stages s .. s + (NB - 1) nw, slots the ids of the next NB
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (s + b * nw < nst) stage(bad[b], R[b], A[b]);
            if (s + (b + NB) * nw < nst) {
                bad[b] = load_w(s + (b + NB) * nw, ids[b], R[b]);
                A[b] = load_a(s + (b + NB) * nw);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (s + (b + NB) * nw < nst) stage(bad[b], R[b], A[b]);
    } else {
        // fewer than 2 NB - 1 stages: one at a time
        for (; s < nst; s += nw) {
            bad[0] = load_w(s, load_ids(s), R[0]);
            A[0] = load_a(s);
            stage(bad[0], R[0], A[0]);
        }
    }

    // the waves meet in LDS, one column tile at a time (32 tokens x 32 columns); thread o of
    // a tile takes outputs o + q * DN_NWU * 64 (q < DN_OPT): register (o / 64) % 16, lane o % 64
    constexpr int OPT = 1024 / (DN_NWU * 64);         // outputs per thread per tile
    float v[OPT * DN_TILES];
    int ob[OPT], oc[OPT];
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int o = tid + q * DN_NWU * 64, r = (o >> 6) & 15, l = o & 63;
        ob[q] = (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
        oc[q] = l & 31;
    }
    float* red = reinterpret_cast<float*>(&s_t[0][0]);    // DN_NWU waves x 1024 floats
#pragma unroll
    for (int t = 0; t < DN_TILES; ++t) {
        __syncthreads();                              // staging (or the previous tile) read
#pragma unroll
        for (int r = 0; r < 16; ++r) red[wave * 1024 + r * 64 + lane] = acc[t][r];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < OPT; ++q) {
            const int o = tid + q * DN_NWU * 64;
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < DN_NWU; ++w) a += red[w * 1024 + o];
            v[OPT * t + q] = a;
        }
    }
    auto row_of = [&](int i) { return ob[i % OPT]; };                              // token
    auto col = [&](int i) { return c0 + (i / OPT) * 32 + oc[i % OPT]; };          // column
    constexpr int NV = OPT * DN_TILES;
    if (nks == 1) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (row_of(i) < B && col(i) < d) y[(size_t)row_of(i) * d + col(i)] = v[i];
        return;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (row_of(i) < B && col(i) < d) st_agent(&part[((size_t)ks * 32 + row_of(i)) * d + col(i)], v[i]);
    // deferred: a later kernel sums the shares into y (reduce_share_rows), no hand-off here
    if (defer) return;
    if (!last_block_arrive(&counter[cgi], nks)) return;
    // The last block of the column group adds every share's partial (its own included) in
    // share order.  Chunk q = tid + 256 m (m < 8) is token q / 64 (wave-uniform), columns
    // c0 + 4 (q % 64) .. + 3; 32 coherent 16-byte loads are in flight per round (4 chunks x
    // 8 shares).  Loads past the buffer (shares >= nks) return zeros; columns past d are
    // summed but never stored.
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(part, (int)((size_t)nks * 32 * d * sizeof(float)));
    const int j4 = 4 * (tid & 63);
#pragma unroll
    for (int m0 = 0; m0 < 8; m0 += 4) {
        if (wave + 4 * m0 >= B) break;                // tokens of this round: none left
        float4 t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k0 = 0; k0 < nks; k0 += 8) {
            float4 pv[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = wave + 4 * (m0 + i);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int off = (((k0 + kk) * 32 + b) * d + c0 + j4) * (int)sizeof(float);
                    const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16);   // sc1
                    pv[i][kk] = __builtin_bit_cast(float4, r);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    t[i].x += pv[i][kk].x;
                    t[i].y += pv[i][kk].y;
                    t[i].z += pv[i][kk].z;
                    t[i].w += pv[i][kk].w;
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = wave + 4 * (m0 + i);
            if (b < B && c0 + j4 < d) *reinterpret_cast<float4*>(&y[(size_t)b * d + c0 + j4]) = t[i];
        }
    }
}

__global__ __launch_bounds__(256) void k_union_yred(const float* __restrict__ part, int nks, int B, int d,
                                                    float* __restrict__ y) {
    reduce_share_rows(part, nks, B, d, y, blockIdx.x * 256 + threadIdx.x);
}

}  // namespace

hipError_t launch_union_yred(const float* part, int nks, int B, int d, float* y, hipStream_t s) {
    const int nq = B * (d / 4);
    hipLaunchKernelGGL(k_union_yred, dim3((nq + 255) / 256), dim3(256), 0, s, part, nks, B, d, y);
    return hipGetLastError();
}

size_t plan_union(FfnPlan& p, int d, int F, size_t off) {
    p.off_H = off;
    off = align_up(off + (size_t)((F + 31) / 32) * 2048, 256);   // H fragments, 2 KB per tile
    p.u_ncg = (d + DN_COLS - 1) / DN_COLS;
    int ks = (256 + p.u_ncg - 1) / p.u_ncg;                      // >= 256 down blocks
    p.u_ks = ks < 1 ? 1 : (ks > 16 ? 16 : ks);
    p.off_upart = off;
    if (p.u_ks > 1) off = align_up(off + (size_t)p.u_ks * 32 * d * sizeof(float), 256);
    // split up tiles: an arrival counter and UP_SP x 8 KB of partials (ReGLU: 16 KB) per tile
    const size_t tiles = (size_t)(F + 31) / 32;
    p.off_upcnt = off;
    off = align_up(off + tiles * sizeof(unsigned), 256);
    p.off_uppart = off;
    off = align_up(off + tiles * UP_SP * 128 * 8 * 2 * sizeof(float), 256);
    return off;
}

// blocks of one up-kernel variant resident on the whole device at once (queried once per
// device and variant)
template <typename K>
int up_slots(K kern) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, reinterpret_cast<const void*>(kern));
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int per_cu = 0, ncu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), UP_NT, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int S = std::max(1, per_cu * ncu);
    cache[key] = S;
    return S;
}

hipError_t launch_ffn_union(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x, int B,
                            const uint32_t* umask, const uint32_t* tokbits, int32_t* idx,
                            int32_t* count, const uint32_t* token_mask, float* y, char* ws,
                            hipStream_t s, float* defer_part) {
    uint4* Hf = reinterpret_cast<uint4*>(ws + pl.off_H);
    float* upart = reinterpret_cast<float*>(ws + pl.off_uppart);
    unsigned* ucnt = reinterpret_cast<unsigned*>(ws + pl.off_upcnt);
    const int tiles = (f.F + 31) / 32;
    const uint16_t* Wg = static_cast<const uint16_t*>(f.w_gate);
    const uint16_t* Wu = static_cast<const uint16_t*>(f.w_up);
    // 32-bit buffer offsets when every byte of a weight matrix is within 2^31
    const bool off32 = (size_t)f.F * f.d * 2 <= (size_t)INT_MAX;
    const bool glu = f.act == PI_ACT_REGLU;
    hipError_t e = hipSuccess;
    auto up = [&](auto kern) {
        const int S = up_slots(kern);
        if (S <= 0) {
            e = hipErrorInvalidValue;
            return;
        }
        // blocks for every tile the union could have (its size is known on the device only);
        // those past the union return at once
        const int sp = tiles > S ? UP_SP : 1;
        const int grid = tiles > S ? S + (tiles - S) * sp : tiles;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(UP_NT), 0, s, x, B, Wg, Wu, f.d, f.F, umask,
                           tokbits, idx, count, token_mask, S, sp, upart, ucnt, Hf);
        e = hipGetLastError();
    };
    if (umask) {
        if (glu) off32 ? up(k_union_up<true, true, true>) : up(k_union_up<true, false, true>);
        else off32 ? up(k_union_up<false, true, true>) : up(k_union_up<false, false, true>);
    } else {
        if (glu) off32 ? up(k_union_up<true, true, false>) : up(k_union_up<true, false, false>);
        else off32 ? up(k_union_up<false, true, false>) : up(k_union_up<false, false, false>);
    }
    if (e != hipSuccess) return e;
    unsigned* cnt = reinterpret_cast<unsigned*>(ws) + CNT_UNION;
    const bool defer = defer_part != nullptr && pl.u_ks > 1;
    float* part = defer ? defer_part : reinterpret_cast<float*>(ws + pl.off_upart);
    hipLaunchKernelGGL(k_union_down, dim3(pl.u_ncg * pl.u_ks), dim3(DN_NWU * 64), 0, s, Hf, B,
                       static_cast<const uint16_t*>(f.w_down), f.d, f.F, idx, count, pl.u_ncg,
                       pl.u_ks, part, cnt, y, defer ? 1 : 0);
    return hipGetLastError();
}

}  // namespace pi
