// Persistent batch-1 decode on gfx950: a whole run of decode steps in ONE cooperative
// launch, with no kernel boundary between the steps or between their phases.
//
// What each step computes is the PowerInfer online engine for one FFN layer
// ("Adaptive Sparsity Predictors": a per-layer low-rank predictor marks the neurons
// a token will fire; "Neuron Placement and Management": the kept neurons are listed
// by their original positions; "Neuron-aware Operator": only those neurons' rows of
// up/gate and output vectors of down are read, in place).  The schedule is this
// chip's: a kernel boundary costs ~2.4 us of timeline here, about as much as the
// memory time of a whole 35 MB step, so the phases hand over through flags.
//
// Per step (local step k of the launch; replica e, token t):
//   A  stage 1, z = x W_p1.  Block b owns predictor rows j = b + G*i.  Its 512 threads
//      split every row into 16-byte chunks; the chunks of the next step's rows are
//      loaded while the block still waits for the current step to finish.  Wave sums
//      meet in LDS; z goes to the workspace.
//   B  Block b owns the mask words [wb0, wb1) (a balanced split of the F/32 words).
//      The W2t rows of its first 64-neuron tile are loaded at the start of the step;
//      once every z is published the block forms l = W2t z + b, thresholds it
//      (l > theta), writes and publishes its mask words, then gathers the up (and gate)
//      rows of its own predicted-active neurons and writes h (indexed by neuron).
//   C  Block b < nslices * nsplit owns (column slice, word split).  When the B blocks of
//      its split have published their mask words, it compacts the split's words in LDS
//      (ascending: the split's part of the neuron table) and starts loading its slice of
//      the active down rows; when they have published h, it accumulates
//      h_i * W_down[i, slice], writes a partial row, and the last block to arrive on the
//      slice adds the nsplit partials in split order into y (deterministic).
//   The next step's A starts only when every slice of this step's y is written: the
//   layer-to-layer dependency of a real decode stream, kept although the synthetic
//   tokens do not depend on y.
// Hand-offs are monotone step counters in the workspace, stored with agent-coherent
// stores after s_waitcnt has drained the data they cover, and polled with
// agent-coherent loads by one wave per block; all data that crosses blocks is written
// and read with agent-coherent accesses (no L2 writeback / invalidate).  Every wait has
// a spin limit: a wait that outlasts it raises the error word, every later wait then
// returns at once, so the launch always ends, and the last block out fills y with NaN.
// The last block out also resets every counter, so the next launch starts from zero.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

constexpr int RN_NW = 8;             // waves per block
constexpr int RN_NT = RN_NW * 64;    // threads per block
constexpr uint32_t RN_SPIN_LIMIT = 1u << 22;

// wave index as a wave-uniform (scalar) value, so row addresses stay in SGPRs
PI_DEV int uwave() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// 16-byte load at a wave-uniform base plus a 32-bit per-lane byte offset
PI_DEV uint4 ld16u(const void* base, uint32_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + off);
}

// Hand-off flags: bytes from RunPlan::off_flags, each holding a step counter modulo 256.
// A waiter wants counter >= target; no producer can run more than one stage ahead of a
// waiter (every stage of step k + 1 depends on the end of step k), so "(v - target) mod 256
// < 128" decides it exactly.
constexpr int FL_A = 0;              // [G]  z rows of step k written      -> k + 1
constexpr int FL_B = 512;            // [G]  mask words -> 2k + 1, h       -> 2k + 2
constexpr int FL_Y = 1024;           // [nslices] y slice of step k written -> k + 1
constexpr int FL_CNT = 2048;         // uint32 words from here: [nslices] arrival counters
constexpr int FL_EXIT = FL_CNT + 4 * 512;   // uint32: blocks that have left the launch
constexpr int FL_ERR = FL_EXIT + 4;         // uint32: a wait hit its spin limit (sticky)
constexpr int FL_BYTES = FL_ERR + 4;
static_assert(FL_BYTES <= RUN_FLAG_BYTES, "flag area");
static_assert(CNT_RUN * 4 + RUN_FLAG_BYTES <= CNT_TOTAL * 4, "flags inside the counter area");

PI_DEV void set_flag(uint8_t* fl, int i, uint32_t v) {
    __hip_atomic_store(fl + i, (uint8_t)(v & 0xFFu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
PI_DEV uint32_t* fl_word(uint8_t* fl, int byte_off) { return reinterpret_cast<uint32_t*>(fl + byte_off); }

// One wave polls the byte flags fl[lo .. lo+n) until every one has reached `target`, then
// the whole block is released.  Each lane reads 8 flags with one agent-coherent 8-byte
// load, so a window of 512 flags takes one load per lane.  Called by every thread.
PI_DEV void wait_flags(uint8_t* fl, int lo, int n, uint32_t target) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint32_t* err = fl_word(fl, FL_ERR);
        uint32_t spins = 0;
        for (;;) {
            bool done = true;
            for (int base = lo & ~7; base < lo + n; base += 512) {   // 8-byte aligned windows
                const int first = base + 8 * lane;
                const bool mine = first < lo + n && first + 8 > lo;
                const uint64_t v = mine ? __hip_atomic_load(reinterpret_cast<uint64_t*>(fl + first),
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                        : 0ull;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = first + j;
                    const uint32_t f = (uint32_t)(v >> (8 * j)) & 0xFFu;
                    if (mine && i >= lo && i < lo + n) done = done && (((f - target) & 0xFFu) < 128u);
                }
            }
            const uint32_t e = ld_agent(err);
            if (__all(done ? 1 : 0) || e != 0u) break;
            if (++spins >= RN_SPIN_LIMIT) {
                if (lane == 0) st_agent(err, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// After every thread's stores of the covered data have drained, thread 0 sets flag i.
PI_DEV void publish(uint8_t* fl, int i, uint32_t value) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) set_flag(fl, i, value);
}

// An 8-fp16 chunk regrouped as (x0,x4),(x1,x5),(x2,x6),(x3,x7): the pairs one AND/OR
// extracts from an int4 word.  Applied to both operands of a dot, it changes nothing.
PI_DEV uint4 regroup8(const uint4& a) {
    return make_uint4((a.x & 0xFFFFu) | (a.z << 16), (a.x >> 16) | (a.z & 0xFFFF0000u),
                      (a.y & 0xFFFFu) | (a.w << 16), (a.y >> 16) | (a.w & 0xFFFF0000u));
}

// W2t rows of the block's 64-neuron tile (r <= 1024): wave w holds rows n0 + 8w .. n0 + 8w + 7,
// lane the 16-byte chunks lane + 64q (q < 2) of each row; wave 0 lane l the bias of n0 + l.
struct Tile {
    uint4 w[8][2];
    float bias;
};

PI_DEV void tile_load(Tile& t, const uint16_t* __restrict__ W2t, const float* __restrict__ bias,
                      int r, int n0, int n_end) {
    const int lane = threadIdx.x & 63, wave = uwave();
    const int nr = r >> 3;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int n = n0 + wave * 8 + m;                 // wave-uniform row
        const uint16_t* row = W2t + (size_t)n * r;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = lane + 64 * q;
            t.w[m][q] = (n < n_end && c < nr) ? ld16u(row, 16u * (uint32_t)c) : zero4();
        }
    }
    t.bias = (wave == 0 && n0 + lane < n_end) ? bias[n0 + lane] : 0.f;
}

PI_DEV void tile_fma(const Tile& t, const float* s_z, int r, float* acc) {
    const int lane = threadIdx.x & 63;
    const int nr = r >> 3;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = lane + 64 * q;
        if (c < nr) {
            const float4 za = *reinterpret_cast<const float4*>(&s_z[8 * c]);
            const float4 zb = *reinterpret_cast<const float4*>(&s_z[8 * c + 4]);
#pragma unroll
            for (int m = 0; m < 8; ++m) acc[m] += dot8_f32(t.w[m][q], za, zb);
        }
    }
}

template <int WF>
struct RnGeom {
    static constexpr int LB = WF == 0 ? 16 : 8;   // bytes per lane load of a down row
    static constexpr int V = WF == 0 ? 8 : 16;    // columns per lane
    static constexpr int SC = 64 * V;             // columns per slice
};

// -------------------------------------------------------------------------------- one step
// LDS of a block (dynamic part: x, z, then the C region shared by the neuron ids and the
// down reduction).
struct Shm {
    uint4* x;          // d/8 chunks (int4 layers: regrouped)
    float* z;          // r
    int* ids;          // C: the split's active neuron ids
    float* red;        // C: the waves' column sums (aliases ids)
    float* l;          // [64] tile logits before the bias
    float* dot;        // [2][64] gate / up dots of the tile's active neurons
    int* list;         // [64] tile offsets of the active neurons
    int* na;           // active neurons in the tile
    float* asum;       // [NW][4] stage-1 wave sums
    int* tmp;          // [NW + 1] scan scratch
};

// The roles of block b (fixed for a launch, recomputed every step from laundered inputs
// so that nothing of one phase stays live in registers through the others).
struct Roles {
    int G, W, nrb, nA, qa, npa, wb0, wb1, nb0, nb1, ntile;
    bool isC, has_words;
    int slice, split, ws0, ws1, b_lo, b_hi;
    PI_DEV Roles(const RunArgs& a, int b) {
        const RunPlan& pl = a.pl;
        G = pl.G;
        W = pl.W;
        nrb = b < a.r ? (a.r - b + G - 1) / G : 0;           // stage-1 rows b + G*i
        nA = a.r < G ? a.r : G;                              // blocks with stage-1 rows
        qa = pl.qa;                                          // chunks per thread per row
        npa = nrb * qa;                                      // (row, chunk) pairs, <= 4
        wb0 = (int)((long long)b * W / G);
        wb1 = (int)((long long)(b + 1) * W / G);
        nb0 = wb0 * 32;
        nb1 = min(wb1 * 32, a.F);
        ntile = nb1 > nb0 ? 1 : 0;                           // at most 64 neurons (2 words)
        const int nC = pl.nslices * pl.nsplit;
        isC = b < nC;
        slice = isC ? b % pl.nslices : 0;
        split = isC ? b / pl.nslices : 0;
        ws0 = (int)((long long)split * W / pl.nsplit);
        ws1 = (int)((long long)(split + 1) * W / pl.nsplit);
        has_words = isC && ws1 > ws0;
        // B blocks owning the split's words: owner(w) = ceil((w + 1) G / W) - 1
        b_lo = has_words ? (int)(((long long)(ws0 + 1) * G + W - 1) / W) - 1 : 0;
        b_hi = has_words ? (int)(((long long)ws1 * G + W - 1) / W) - 1 : 0;
    }
};

// stage-1 chunk p = (row b + G (p / qa), chunk tid + 512 (p % qa)) of replica R
PI_DEV void load_stage1(uint4 (&wa)[4], const RunRep& R, const Roles& ro, int d, int tid, int b) {
    const int nc8 = d >> 3;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int i = p / ro.qa;
        const int c = tid + RN_NT * (p - i * ro.qa);
        wa[p] = (p < ro.npa && c < nc8) ? ld16u(R.w1t + (size_t)(b + ro.G * i) * d, 16u * (uint32_t)c) : zero4();
    }
}

template <int WF, bool GLU, int Q>
PI_DEV void run_step(const RunArgs& a, int k, int tid, int b, uint4 (&wa)[4], const Shm& sh) {
    using Gm = RnGeom<WF>;
    constexpr int IPW = Q <= 8 ? 2 : 1;           // up/gate rows per wave in flight
    constexpr int M = GLU ? 2 : 1;
    constexpr int U = WF == 0 ? 8 : 12;           // down rows per wave in flight
    const RunPlan& pl = a.pl;
    const int d = a.d, r = a.r;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Roles ro(a, b);
    const int nc8 = d >> 3;
    uint8_t* fl = reinterpret_cast<uint8_t*>(a.ws + pl.off_flags);
    float* zw = reinterpret_cast<float*>(a.ws + pl.off_z);
    float* hw = reinterpret_cast<float*>(a.ws + pl.off_h);
    float* part = reinterpret_cast<float*>(a.ws + pl.off_part);
    const RunRep& R = a.rep[(a.e0 + k) % a.tabn];
    const uint16_t* x = a.x + (size_t)((a.g0 + k) % a.T) * d;

    // ---------------------------------------------------------------- step start
    if (k > 0) wait_flags(fl, FL_Y, pl.nslices, (uint32_t)k);
    for (int c = tid; c < nc8; c += RN_NT) {
        const uint4 v = ld16u(x, 16u * (uint32_t)c);
        sh.x[c] = WF == 0 ? v : regroup8(v);
    }
    __syncthreads();

    // ---------------------------------------------------------------- A: z rows
    if (ro.nrb > 0) {
        float v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int i = p / ro.qa;
            const int c = tid + RN_NT * (p - i * ro.qa);
            v[p] = (p < ro.npa && c < nc8) ? dot8(WF == 0 ? wa[p] : regroup8(wa[p]), sh.x[c], 0.f) : 0.f;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (p < ro.npa) {
                const float s = wave_sum(v[p]);
                if (lane == 0) sh.asum[wave * 4 + p] = s;
            }
        }
        __syncthreads();
        if (tid < ro.nrb) {
            float s = 0.f;
            for (int q = 0; q < ro.qa; ++q)
#pragma unroll
                for (int w = 0; w < RN_NW; ++w) s += sh.asum[w * 4 + tid * ro.qa + q];
            st_agent(zw + (b + ro.G * tid), s);
        }
    }
    // the tile's W2t rows are in flight while z is published and awaited
    Tile tl;
    if (ro.ntile > 0) tile_load(tl, R.w2t, R.bias, r, ro.nb0, ro.nb1);
    publish(fl, FL_A + b, (uint32_t)(k + 1));

    // ---------------------------------------------------------------- B: logits, mask words
    if (ro.ntile > 0) {
        wait_flags(fl, FL_A, ro.nA, (uint32_t)(k + 1));
        for (int j = tid; j < r; j += RN_NT) sh.z[j] = ld_agent(zw + j);
        __syncthreads();
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const float bv = tl.bias;
        tile_fma(tl, sh.z, r, acc);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float s = wave_sum(acc[m]);
            if (lane == 0) sh.l[wave * 8 + m] = s;
        }
        __syncthreads();
        if (wave == 0) {
            const int n = ro.nb0 + lane;
            const bool act = n < ro.nb1 && (sh.l[lane] + bv) > a.theta;
            const unsigned long long bal = __ballot(act);
            const uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
            const int w = ro.nb0 >> 5;
            if (lane == 0) {
                st_agent(a.mask + w, lo);
                if (w + 1 < ro.wb1) st_agent(a.mask + w + 1, hi);
                *sh.na = __popcll(bal);
            }
            if (act) sh.list[__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u))] = lane;
        }
        __syncthreads();
    }
    publish(fl, FL_B + b, (uint32_t)(2 * k + 1));

    // ---------------------------------------------------------------- B: up / gate -> h
    if (ro.ntile > 0) {
        const int nc = WF == 0 ? nc8 : (d >> 5);
        const int Gs = d >> 7;
        const size_t rb = WF == 0 ? (size_t)d * 2 : (size_t)(d >> 1);
        const int n0 = ro.nb0;
        const int na = *sh.na;
        const int items = na * M;
        for (int it0 = wave * IPW; it0 < items; it0 += RN_NW * IPW) {
            uint4 wr[IPW][Q];
            uint32_t sr[IPW][Q];   // raw fp16 scales, one per register
            // unconditional loads (chunk 0 of the row, or row 0 for an empty slot, where a lane
            // has nothing to read; discarded at use): a branch-guarded load is waited for at
            // the end of its branch
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int it = it0 + i;
                const bool valid = it < items;
                const int kk = GLU ? (it >> 1) : it;
                const int mat = GLU ? (it & 1) : 1;      // 0 = gate, 1 = up
                const size_t row = valid ? (size_t)__builtin_amdgcn_readfirstlane(n0 + sh.list[kk < 64 ? kk : 63]) : 0;
                const uint8_t* base = static_cast<const uint8_t*>(mat ? R.wu : R.wg) + row * rb;
                const uint16_t* sbase = WF == 1 ? (mat ? R.su : R.sg) + row * Gs : nullptr;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int c = lane + 64 * q;
                    const int cc = c < nc ? c : 0;
                    wr[i][q] = ld16u(base, 16u * (uint32_t)cc);
                    if (WF == 1) sr[i][q] = (uint32_t)sbase[cc >> 2];
                }
            }
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int it = it0 + i;
                if (it >= items) break;
                float dot = 0.f;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int c = lane + 64 * q;
                    if (c < nc) {
                        if (WF == 0) {
                            dot = dot8(wr[i][q], sh.x[c], dot);
                        } else {
                            uint32_t xp[16];
#pragma unroll
                            for (int m = 0; m < 4; ++m) {
                                const uint4 t = sh.x[4 * c + m];
                                xp[4 * m] = t.x; xp[4 * m + 1] = t.y; xp[4 * m + 2] = t.z; xp[4 * m + 3] = t.w;
                            }
                            dot = fmaf(dot32_i4(wr[i][q], xp), h2f((uint16_t)sr[i][q]), dot);
                        }
                    }
                }
                dot = wave_sum(dot);
                if (lane == 0) sh.dot[(GLU ? (it & 1) : 1) * 64 + (GLU ? (it >> 1) : it)] = dot;
            }
        }
        __syncthreads();
        for (int kk = tid; kk < na; kk += RN_NT) {
            const float av = sh.dot[64 + kk];
            st_agent(hw + n0 + sh.list[kk], GLU ? fmaxf(sh.dot[kk], 0.f) * av : fmaxf(av, 0.f));
        }
    }
    publish(fl, FL_B + b, (uint32_t)(2 * k + 2));

    // ---------------------------------------------------------------- C: down
    if (ro.isC) {
        // the split's mask words -> ascending neuron ids in LDS
        if (ro.has_words) wait_flags(fl, FL_B + ro.b_lo, ro.b_hi - ro.b_lo + 1, (uint32_t)(2 * k + 1));
        uint32_t mw = 0;
        if (ro.ws0 + tid < ro.ws1) mw = ld_agent(a.mask + ro.ws0 + tid);
        int n_loc;
        int pos = block_exclusive_scan(__popc(mw), sh.tmp, &n_loc);
        while (mw) {
            sh.ids[pos++] = ((ro.ws0 + tid) << 5) + (__ffs(mw) - 1);
            mw &= mw - 1u;
        }
        __syncthreads();

        const size_t rowb = WF == 0 ? (size_t)d * 2 : (size_t)(d >> 1);
        const uint32_t boff = ((uint32_t)ro.slice * 64u + (uint32_t)lane) * Gm::LB;
        const bool cok = boff < rowb;
        const int Gs = d >> 7;
        const int sg = (ro.slice * Gm::SC + lane * Gm::V) >> 7;   // int4 scale group of the lane
        const uint8_t* Wb = static_cast<const uint8_t*>(R.wd);
        float acc[Gm::V];
#pragma unroll
        for (int v = 0; v < Gm::V; ++v) acc[v] = 0.f;
        uint4 w16[U];
        uint2 w8[U];
        uint32_t sr[U];            // raw fp16 scales, one per register
        float hv[U];
        int rows[U];
        // one round: U rows per wave (items k0 + u*NW); their h only once it is published.
        // Unconditional loads (row 0 / column 0 where there is nothing to read, zeroed at use):
        // a branch-guarded load is waited for at the end of its branch.
        auto load_round = [&](int k0, bool with_h) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kk = k0 + u * RN_NW;
                const bool valid = kk < n_loc;
                const int row = valid ? __builtin_amdgcn_readfirstlane(sh.ids[kk < RUN_WPS_MAX * 32 ? kk : 0]) : 0;
                rows[u] = row;
                const uint32_t off = cok ? boff : 0u;
                if (with_h) hv[u] = ld_agent(hw + row);
                if (WF == 0) {
                    w16[u] = ld16u(Wb + (size_t)row * rowb, off);
                } else {
                    w8[u] = *reinterpret_cast<const uint2*>(Wb + (size_t)row * rowb + off);
                    sr[u] = (uint32_t)R.sd[(size_t)row * Gs + (cok ? sg : 0)];
                }
            }
        };
        load_round(wave, false);
        if (ro.has_words) wait_flags(fl, FL_B + ro.b_lo, ro.b_hi - ro.b_lo + 1, (uint32_t)(2 * k + 2));
        for (int k0 = wave; k0 < n_loc; k0 += RN_NW * U) {
            if (k0 == wave) {
#pragma unroll
                for (int u = 0; u < U; ++u) hv[u] = ld_agent(hw + rows[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float hu = (k0 + u * RN_NW < n_loc && cok) ? hv[u] : 0.f;
                if (WF == 0) {
                    const uint32_t ww[4] = {w16[u].x, w16[u].y, w16[u].z, w16[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[2 * e] = fmaf(hu, lo_f(ww[e]), acc[2 * e]);
                        acc[2 * e + 1] = fmaf(hu, hi_f(ww[e]), acc[2 * e + 1]);
                    }
                } else {
                    const float hs = hu * h2f((uint16_t)sr[u]);
                    axpy8_i4(acc, w8[u].x, hs, hs * 0.0625f);
                    axpy8_i4(acc + 8, w8[u].y, hs, hs * 0.0625f);
                }
            }
            if (k0 + RN_NW * U < n_loc) load_round(k0 + RN_NW * U, true);
        }
        __syncthreads();                      // the ids are dead: their LDS takes the sums
        {
            float4* dst = reinterpret_cast<float4*>(&sh.red[wave * Gm::SC + lane * Gm::V]);
#pragma unroll
            for (int v = 0; v < Gm::V; v += 4) dst[v / 4] = make_float4(acc[v], acc[v + 1], acc[v + 2], acc[v + 3]);
        }
        __syncthreads();
        // the waves' sums -> this block's partial row of the slice (fixed order)
        constexpr int CPT = Gm::SC / RN_NT;   // columns per thread: 1 (fp16) or 2 (int4)
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int col = tid + RN_NT * j;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < RN_NW; ++w) s += sh.red[w * Gm::SC + col];
            const int gcol = ro.slice * Gm::SC + col;
            if (gcol < d) st_agent(&part[(size_t)ro.split * d + gcol], s);
        }
        if (last_block_arrive(fl_word(fl, FL_CNT + 4 * ro.slice), (unsigned)pl.nsplit)) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int gcol = ro.slice * Gm::SC + tid + RN_NT * j;
                if (gcol < d) {
                    float t = 0.f;
                    for (int base = 0; base < pl.nsplit; base += 16) {   // 16 partials in flight
                        float pv[16];
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int sp = base + i;
                            pv[i] = sp < pl.nsplit ? ld_agent(&part[(size_t)sp * d + gcol]) : 0.f;
                        }
#pragma unroll
                        for (int i = 0; i < 16; ++i) t += pv[i];
                    }
                    // agent-coherent: the slice's last block differs from step to step (and
                    // from XCD to XCD), and a write-back store could land after a later one
                    st_agent(&a.y[gcol], t);
                }
            }
            publish(fl, FL_Y + ro.slice, (uint32_t)(k + 1));
        }
    }

    // the next step's stage-1 rows are loaded while the block waits for this step's y
    if (k + 1 < a.L) load_stage1(wa, a.rep[(a.e0 + k + 1) % a.tabn], ro, d, tid, b);
}

// -------------------------------------------------------------------------------- the kernel
// WF: 0 = fp16 rows, 1 = int4 group-128 rows.  Q: 16-byte chunks per lane of an up/gate row.
template <int WF, bool GLU, int Q>
__global__ __launch_bounds__(RN_NT, 4) void k_run(RunArgs args) {
    // The arguments are read in place from the kernarg segment (the only explicit argument
    // sits at offset 0): indexing the replica table of a by-value copy would move the whole
    // struct to private memory and make every pointer taken from it a per-lane value.
#if defined(__HIP_DEVICE_COMPILE__)
    const RunArgs* ap0 = (const RunArgs*)__builtin_amdgcn_kernarg_segment_ptr();
#else
    const RunArgs* ap0 = &args;
#endif
    extern __shared__ __align__(16) char smem[];
    __shared__ float s_l[64];
    __shared__ float s_dot[2 * 64];
    __shared__ int s_list[64];
    __shared__ int s_na;
    __shared__ float s_asum[RN_NW * 4];
    __shared__ int s_tmp[RN_NW + 1];
    __shared__ int s_exit;
    const int d0 = ap0->d, r0 = ap0->r;
    char* s_c = smem + (size_t)d0 * 2 + align16i(r0 * 4);
    const Shm sh{reinterpret_cast<uint4*>(smem), reinterpret_cast<float*>(smem + (size_t)d0 * 2),
                 reinterpret_cast<int*>(s_c), reinterpret_cast<float*>(s_c), s_l, s_dot, s_list,
                 &s_na, s_asum, s_tmp};

    uint4 wa[4];
    {
        const Roles ro(*ap0, blockIdx.x);
        load_stage1(wa, ap0->rep[ap0->e0 % ap0->tabn], ro, d0, threadIdx.x, blockIdx.x);
    }
    const int L = ap0->L;
    for (int k = 0; k < L; ++k) {
        // fresh copies every step: nothing derived from them is hoisted out of the loop
        const RunArgs* ap = ap0;
        int tid = threadIdx.x, b = blockIdx.x;
        asm volatile("" : "+s"(ap), "+v"(tid), "+s"(b));
        run_step<WF, GLU, Q>(*ap, k, tid, b, wa, sh);
    }

    // ---- end of the launch: the last block out resets the counters and writes the table
    const RunArgs& a = *ap0;
    const int tid = threadIdx.x;
    uint8_t* fl = reinterpret_cast<uint8_t*>(a.ws + a.pl.off_flags);
    wait_flags(fl, FL_Y, a.pl.nslices, (uint32_t)L);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(fl_word(fl, FL_EXIT), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_exit = prev == gridDim.x - 1u;
    }
    __syncthreads();
    if (s_exit) {
        // every block has passed its last wait: nobody reads a flag any more
        const bool err = ld_agent(fl_word(fl, FL_ERR)) != 0u;
        for (int i = tid; i < FL_CNT / 4; i += RN_NT) st_agent(fl_word(fl, 4 * i), 0u);   // byte flags
        if (err) {
            for (int i = tid; i < a.d; i += RN_NT) st_agent(&a.y[i], __builtin_nanf(""));
            if (tid == 0 && a.count != nullptr) *a.count = -1;
        } else if (a.idx != nullptr) {
            // the last step's neuron table, ascending, from its mask
            block_compact<true>(a.mask, 1, a.pl.W, a.F, a.idx, a.count, s_tmp);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) st_agent(fl_word(fl, FL_EXIT), 0u);
    }
}

template <int WF, bool GLU, int Q>
const void* run_kernel() {
    return reinterpret_cast<const void*>(&k_run<WF, GLU, Q>);
}

template <int WF, bool GLU>
const void* pick_q(int q) {
    if constexpr (WF == 0) {
        switch (q) {
            case 2: return run_kernel<0, GLU, 2>();
            case 4: return run_kernel<0, GLU, 4>();
            case 8: return run_kernel<0, GLU, 8>();
            case 16: return run_kernel<0, GLU, 16>();
            default: return nullptr;
        }
    } else {
        switch (q) {
            case 1: return run_kernel<1, GLU, 1>();
            case 2: return run_kernel<1, GLU, 2>();
            case 4: return run_kernel<1, GLU, 4>();
            case 8: return run_kernel<1, GLU, 8>();
            default: return nullptr;
        }
    }
}

}  // namespace

const void* run_kernel_for(int wfmt, int act, int q) {
    const bool glu = act == PI_ACT_REGLU;
    if (wfmt == PI_W_F16) return glu ? pick_q<0, true>(q) : pick_q<0, false>(q);
    return glu ? pick_q<1, true>(q) : pick_q<1, false>(q);
}

RunPlan plan_run(int d, int r, int F, int wfmt, int G) {
    RunPlan p{};
    const bool f16 = wfmt == PI_W_F16;
    p.G = G;
    p.W = (F + 31) / 32;
    const int sc = f16 ? RnGeom<0>::SC : RnGeom<1>::SC;
    p.nslices = (d + sc - 1) / sc;
    // about 128 down blocks: enough rows in flight, few enough partials per slice
    int ns = (128 + p.nslices - 1) / p.nslices;
    const int ns_min = (p.W + RUN_WPS_MAX - 1) / RUN_WPS_MAX;
    if (ns > 16) ns = 16;
    if (ns > p.W) ns = p.W;
    if (ns < ns_min) ns = ns_min;
    if (ns < 1) ns = 1;
    p.nsplit = ns;
    p.qa = (d / 8 + RN_NT - 1) / RN_NT;
    p.nrb = G > 0 ? (r + G - 1) / G : 0;
    const int wpb = G > 0 ? (p.W + G - 1) / G : 0;           // words per block, at most
    p.tpb = (wpb * 32 + 63) / 64;
    const int nc = f16 ? d / 8 : d / 32;
    const int q = (nc + 63) / 64;
    int qb = f16 ? 2 : 1;
    while (qb < q) qb *= 2;
    p.q = qb;
    const size_t c_region = std::max((size_t)RUN_WPS_MAX * 32 * 4, (size_t)RN_NW * sc * 4);
    p.lds = (size_t)d * 2 + (size_t)align16i(r * 4) + c_region;
    // the flags live in the reserved counter area, which no other path writes
    p.off_flags = (size_t)CNT_RUN * sizeof(unsigned);
    size_t off = COUNTER_BYTES;
    p.off_z = off;
    off = align_up(off + (size_t)r * 4, 256);
    p.off_h = off;
    off = align_up(off + (size_t)F * 4, 256);
    p.off_part = off;
    off = align_up(off + (size_t)p.nsplit * d * 4, 256);
    p.bytes = off;
    return p;
}

bool run_fits(const RunPlan& p, int d, int r, int F, int wfmt) {
    const int maxq = wfmt == PI_W_F16 ? 16 : 8;
    return p.G >= 1 && p.G <= 512 && r <= 1024 && p.nrb * p.qa <= 4 &&
           p.tpb <= 1 && p.nslices <= 512 && p.nslices * p.nsplit <= p.G &&
           (p.W + p.nsplit - 1) / p.nsplit <= RUN_WPS_MAX && p.q <= maxq && p.lds <= 65536 &&
           d % 8 == 0;
}

hipError_t launch_run(const RunArgs& ra, hipStream_t s) {
    const void* fn = run_kernel_for(ra.wfmt, ra.act, ra.pl.q);
    if (!fn) return hipErrorInvalidValue;
    void* args[] = {const_cast<RunArgs*>(&ra)};
    return hipLaunchCooperativeKernel(fn, dim3(ra.pl.G), dim3(RN_NT), args, (unsigned)ra.pl.lds, s);
}

int run_grid(int wfmt, int act, int q, size_t lds) {
    const void* fn = run_kernel_for(wfmt, act, q);
    if (!fn) return 0;
    int dev = 0, cus = 0, nb = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, RN_NT, lds) != hipSuccess) return 0;
    if (nb > 2) nb = 2;
    const int g = cus * nb;
    return g > 512 ? 512 : g;
}

}  // namespace pi
