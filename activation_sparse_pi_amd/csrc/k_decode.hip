// Batch-1 decode step on gfx950: two or three kernels per token.
//
// PowerInfer (online engine, "Adaptive Sparsity Predictors", "Neuron Placement
// and Management", "Neuron-aware Operator"): predict the neurons a token will
// fire, compute only their rows of up/gate and their output vectors of down,
// and keep a table of their original positions.
//
// On this GPU a kernel boundary costs 1.1-1.4 us of timeline between dependent
// kernels, so the step is cut only where a global dependency forces it (every
// tile's logits need all of z):
//   A  predictor stage 1, z_j = W1t[j, :] . x (one wave per predictor column, the
//      kernel pi_predict uses); its grid also sums the previous step's partial rows
//      into y.
//   B  one block per 64-neuron tile: the tile's 64 contiguous W2t rows (and biases)
//      are already in flight while z is staged in LDS; l = W2t[tile] . z + b,
//      active = l > theta, a wave ballot writes the tile's two mask words and lists
//      its active neurons; the block computes h for them from their gate/up rows
//      (x staged in LDS).
// The down projection y = sum_k h_k W_down[k, :] is computed as P fp32 partial rows of d
// columns (plain stores, no atomics), which the next step's first kernel -- or, after the last
// step, a small finishing kernel -- sums in a fixed order into y (reduce_partials), in one of
// two ways:
//   fused (two kernels per step): B itself reads its active neurons' down rows and stores
//      its d column sums as partial row `tile` (P = number of tiles).
//   split (three kernels per step): B writes h; C, a 2-D grid of (range of mask words, column
//      slice) blocks, compacts its range of the mask in LDS, reduces its rows over 16 waves and
//      stores its slice of partial row `range` (P = number of ranges).
// The fused step saves a kernel boundary but writes (and the reduction reads) ntile * d
// partial sums, against nsplit * d for the split step, so it is chosen where ntile * d is
// small.  The finishing kernel also writes the last step's ascending neuron table.
#include <hip/hip_ext.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace pi {
namespace {

constexpr int DEC_IDCAP = 4096;   // neuron ids one split-schedule down block holds (128 mask words)

// --------------------------------------------------------------------------------------- B
// WF: 0 = fp16 rows, 1 = int4 group-128 rows.  Q: 16-byte chunks per lane per row.
// Dynamic LDS: z (r floats) then x (d/8 uint4; for int4 regrouped per 8 elements as
// (x0,x4),(x1,x5),(x2,x6),(x3,x7) to match the nibble pairs one AND/OR extracts).
constexpr int B_WAVES = 8;   // waves per tile block (two blocks fit on a CU)

// Columns per lane of the fused down chunks: 8 fp16 (16-byte loads) or 16 int4 (8-byte loads)
// where the layer is wide enough to give each of the 8 waves a chunk, fewer below that.
constexpr int down_cols_per_lane(int wf, int q) {
    return wf == 0 ? (q <= 2 ? 2 : q <= 4 ? 4 : 8) : (q <= 2 ? 8 : 16);
}

// P8: int8 predictor rows W2t with fp16 scales S2 (one per 128 columns).  (Holding the int8
// variants to 128 VGPRs, for two tile blocks per CU, makes them spill: slower on every shape.)
template <int WF, bool GLU, int Q, bool FUSED, bool P8>
__global__ __launch_bounds__(B_WAVES * 64) void k_dec_stage2_up(
    const float* __restrict__ z, const void* __restrict__ W2t, const uint16_t* __restrict__ S2,
    const float* __restrict__ bias, int r, int F, float theta, float* __restrict__ logits,
    uint32_t* __restrict__ mask, const uint16_t* __restrict__ x, const void* __restrict__ Wg,
    const uint16_t* __restrict__ Sg, const void* __restrict__ Wu,
    const uint16_t* __restrict__ Su, int d, float* __restrict__ h, const void* __restrict__ Wd,
    const uint16_t* __restrict__ Sd, float* __restrict__ part, int nhot) {
    constexpr int NT = B_WAVES * 64;
    // row items per wave in flight, so that a tile with up to 3 (fp16, d <= 4096; int4,
    // d <= 8192) times 8 items needs one memory round trip.  The items are dealt round-robin
    // (wave w: items w, w + 8, ..), so the dot products of a round are spread over all the
    // waves; a slot past the tile's items still loads (a row already in L2), so int4 rows take
    // 3 slots rather than the 4 the registers would allow (LLaMA-70B-shaped layer: 4 slots in
    // blocks of 4 items per wave 32.47, round-robin 32.22, with 3 slots 31.70 us per step)
    constexpr int IPW = Q <= 4 ? (WF == 1 ? 3 : 4) : Q <= 8 ? (WF == 0 ? 3 : 2) : 1;
    extern __shared__ __align__(16) char smem[];
    float* s_z = reinterpret_cast<float*>(smem);
    uint4* s_x = reinterpret_cast<uint4*>(smem + align16i(r * 4));
    __shared__ __align__(16) float s_red[256];   // per tile row, four 16-lane partial sums
    __shared__ float s_dot[2][64];
    __shared__ int s_list[64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: item indices stay scalar
    const int tile = blockIdx.x;
    const int W = (F + 31) >> 5;

    // --- hot block (split schedule): neurons [0, nhot) are computed densely, whether or not the
    // predictor marks them, so their up/gate rows need not wait for the logits.  Wave w of block
    // b takes hot neuron b + ntile w (at most one per wave); its rows go straight into the
    // wave's LDS slot (no registers held), issued before the W2t rows, and are used after the
    // logits, by which time they have landed.  h of a hot neuron is written unmasked: the down
    // projection reads h only for neurons set in the mask.
    constexpr int M = GLU ? 2 : 1;
    const int nc = WF == 0 ? (d >> 3) : (d >> 5);   // 16-byte chunks per row
    const int G = d >> 7;
    const size_t rb = WF == 0 ? (size_t)d * 2 : (size_t)(d >> 1);
    const size_t hslot = (rb + 1023) & ~(size_t)1023;       // one row's LDS slot
    const int hn = tile + (int)gridDim.x * wave;              // this wave's hot neuron
    const bool hot_w = !FUSED && hn < nhot;                   // wave-uniform
    char* s_hot = smem + align16i(r * 4) + (size_t)(d / 8) * 16 + (size_t)wave * M * hslot;
    uint32_t hsc[M][WF == 1 ? Q : 1];                         // int4 scales of the hot rows
    if (hot_w) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int mat = GLU ? m : 1;                      // 0 = gate, 1 = up
            const uint8_t* rowp = static_cast<const uint8_t*>(mat ? Wu : Wg) + (size_t)hn * rb;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int c = lane + 64 * q;
                if (c < nc)        // lane c of instruction q lands at slot offset 16 c
                    __builtin_amdgcn_global_load_lds(rowp + 16 * (size_t)c,
                        (__attribute__((address_space(3))) void*)(s_hot + m * hslot + 1024 * q), 16, 0, 0);
                if constexpr (WF == 1)
                    hsc[m][q] = (uint32_t)((mat ? Su : Sg) + (size_t)hn * G)[(c < nc ? c : 0) >> 2];
            }
        }
    }

    // --- logits of the tile: the first segment of its W2t rows (and the tile's bias) goes out
    // first, then z and x.  fp16 rows, r <= 1024 and d <= 8192: two values of each per thread,
    // all in flight together and staged after one wait (staged in a loop, each iteration waits
    // for everything issued before it); the stores go to clamped addresses (a thread past r or
    // d rewrites the last value), so no branch takes the loads with it.  (Measured: OPT-30B
    // layer -0.55 us per step, LLaMA-7B -0.1; the int4 LLaMA-70B layer +1.3 us, so int4 rows
    // keep the loop.)
    TileRows<B_WAVES, P8> tr;
    tile_rows_load<B_WAVES, P8>(tr, W2t, S2, r, F, tile, 0);
    const float bv = tile * 64 + lane < F ? bias[tile * 64 + lane] : 0.f;   // every wave thresholds
    const int nc8 = d >> 3;
    auto regroup = [](uint4 a) {
        return WF == 0 ? a
                       : make_uint4((a.x & 0xFFFFu) | (a.z << 16), (a.x >> 16) | (a.z & 0xFFFF0000u),
                                    (a.y & 0xFFFFu) | (a.w << 16), (a.y >> 16) | (a.w & 0xFFFF0000u));
    };
    // int4 rows without a hot block stage x after the ballot, where only the dot products need
    // it, instead of behind the W2t rows (the hot block dots its rows with x before the ballot)
    const bool late_x = WF == 1 && nhot == 0;          // block-uniform
    if (WF == 0 && r <= 2 * NT && nc8 <= 2 * NT) {   // block-uniform
        float zr[2];
        uint4 xq[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            zr[k] = z[min(tid + NT * k, r - 1)];
            xq[k] = ld16(x + 8 * min(tid + NT * k, nc8 - 1));
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            s_z[min(tid + NT * k, r - 1)] = zr[k];
            s_x[min(tid + NT * k, nc8 - 1)] = regroup(xq[k]);
        }
    } else if (late_x && r <= 2 * NT) {
        // z in one round (two values per thread, clamped as above); x comes after the ballot
        // (measured: the LLaMA-70B-shaped layer 33.57 -> 33.40 us per step)
        float zr[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) zr[k] = z[min(tid + NT * k, r - 1)];
#pragma unroll
        for (int k = 0; k < 2; ++k) s_z[min(tid + NT * k, r - 1)] = zr[k];
    } else {
        for (int j = tid; j < r; j += NT) s_z[j] = z[j];
        if (!late_x)
            for (int c = tid; c < nc8; c += NT) s_x[c] = regroup(ld16(x + 8 * c));
    }
    __syncthreads();
    float acc[TileRows<B_WAVES, P8>::RPW] = {};
    tile_rows_fma<B_WAVES, P8>(tr, s_z, r, 0, acc);
    for (int c0 = TILE_SEG<P8>; c0 < tile_chunks<P8>(r); c0 += TILE_SEG<P8>) {
        tile_rows_load<B_WAVES, P8>(tr, W2t, S2, r, F, tile, c0);
        tile_rows_fma<B_WAVES, P8>(tr, s_z, r, c0, acc);
    }
    tile_rows_store4<B_WAVES>(acc, s_red);
    __syncthreads();

    // --- the wave's hot neuron: its rows are in LDS by now (issued before the W2t rows, whose
    // data the logits have consumed); the wait below makes that explicit
    if (hot_w) {
        __builtin_amdgcn_s_waitcnt(0);
        float hd[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float dot = 0.f;
            const char* slot = s_hot + m * hslot;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int c = lane + 64 * q;
                if (c < nc) {
                    const uint4 w = *reinterpret_cast<const uint4*>(slot + 16 * c);
                    if (WF == 0) {
                        dot = dot8(w, s_x[c], dot);
                    } else {
                        uint32_t xp[16];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint4 t = s_x[4 * c + k];
                            xp[4 * k] = t.x; xp[4 * k + 1] = t.y; xp[4 * k + 2] = t.z; xp[4 * k + 3] = t.w;
                        }
                        dot = fmaf(dot32_i4(w, xp), h2f((uint16_t)hsc[m][q]), dot);
                    }
                }
            }
            hd[m] = wave_sum(dot);
        }
        if (lane == 0) h[hn] = GLU ? fmaxf(hd[0], 0.f) * hd[M - 1] : fmaxf(hd[0], 0.f);
    }

    // --- threshold: every wave forms the tile's ballot from the logits in LDS (lane = neuron
    // of the tile) and finds its own items' neurons in it (kth_set_bit), with no barrier before
    // the gather; wave 0 also writes the mask words, the logits and the list the phases after
    // the gather read
    const int n = tile * 64 + lane;
    bool act = false;
    float lg = 0.f;
    if (n < F) {
        lg = tile_row_sum(s_red, lane) + bv;
        act = lg > theta;
    }
    const unsigned long long bal = __ballot(act);
    // the row list holds the active neurons outside the hot block (all of them when fused)
    const bool listed = act && (FUSED || n >= nhot);
    const unsigned long long bl = __ballot(listed);
    if (wave == 0) {
        if (logits && n < F) logits[n] = lg;
        if (lane == 0) {
            mask[2 * tile] = (uint32_t)bal;
            if (2 * tile + 1 < W) mask[2 * tile + 1] = (uint32_t)(bal >> 32);
        }
        const uint32_t lo = (uint32_t)bl, hi = (uint32_t)(bl >> 32);
        if (listed) s_list[__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u))] = lane;
    }

    // --- rows of the active neurons: (neuron, matrix) items, IPW per wave in flight
    const int na = __popcll(bl);
    const int items = na * M;
    if (late_x) {                                     // x for the dot products (block-uniform)
        for (int c = tid; c < nc8; c += NT) s_x[c] = regroup(ld16(x + 8 * c));
        __syncthreads();
    }
    for (int it0 = wave; it0 < items; it0 += B_WAVES * IPW) {
        uint4 wr[IPW][Q];
        uint32_t sr[IPW][Q];   // raw fp16 scales, one per register
        // Every load is issued unconditionally, from chunk 0 of the row (row 0 for an empty
        // slot) where a lane has nothing to read, and its value is discarded at use: a load
        // guarded by a branch is waited for at the end of the branch, which would turn the
        // round's loads into one memory round trip each.
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int it = it0 + i * B_WAVES;
            const bool valid = it < items;
            const int k = GLU ? (it >> 1) : it;
            const int mat = GLU ? (it & 1) : 1;        // 0 = gate, 1 = up
            const size_t row = valid ? (size_t)(tile * 64 + kth_set_bit(bl, k)) : 0;
            const uint8_t* base = static_cast<const uint8_t*>(mat ? Wu : Wg) + row * rb;
            const uint16_t* sbase = WF == 1 ? (mat ? Su : Sg) + row * G : nullptr;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int c = lane + 64 * q;
                const int cc = c < nc ? c : 0;
                wr[i][q] = ld16(base + 16 * (size_t)cc);
                if (WF == 1) sr[i][q] = (uint32_t)sbase[cc >> 2];
            }
        }
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int it = it0 + i * B_WAVES;
            if (it >= items) break;
            float dot = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int c = lane + 64 * q;
                if (c < nc) {
                    if (WF == 0) {
                        dot = dot8(wr[i][q], s_x[c], dot);
                    } else {
                        uint32_t xp[16];
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const uint4 t = s_x[4 * c + m];
                            xp[4 * m] = t.x; xp[4 * m + 1] = t.y; xp[4 * m + 2] = t.z; xp[4 * m + 3] = t.w;
                        }
                        dot = fmaf(dot32_i4(wr[i][q], xp), h2f((uint16_t)sr[i][q]), dot);
                    }
                }
            }
            dot = wave_sum(dot);
            if (lane == 0) s_dot[GLU ? (it & 1) : 1][GLU ? (it >> 1) : it] = dot;
        }
    }
    __syncthreads();
    if constexpr (!FUSED) {
        for (int k = tid; k < na; k += NT) {
            const float a = s_dot[1][k];
            h[tile * 64 + s_list[k]] = GLU ? fmaxf(s_dot[0][k], 0.f) * a : fmaxf(a, 0.f);
        }
        return;
    }
    __shared__ float s_h[64];
    for (int k = tid; k < na; k += NT) {
        const float a = s_dot[1][k];
        s_h[k] = GLU ? fmaxf(s_dot[0][k], 0.f) * a : fmaxf(a, 0.f);
    }
    __syncthreads();

    // --- down: partial row `tile` = sum over the tile's active neurons of h_k W_down[row_k, :]
    // (all zero for a tile with none).  Wave w takes column chunks w, w + 8, ... (64 V columns:
    // V fp16 or int4 weights per lane of each row, V as large as leaves no wave without a
    // chunk) and reads that chunk of every active row at once (DN_ROWS in flight; empty slots
    // re-read the first row's chunk, an L2 hit, and count zero); a lane's V column sums are V
    // consecutive floats of the partial row, so the wave's stores are contiguous.
    constexpr int V = down_cols_per_lane(WF, Q);     // columns per lane
    constexpr int CH = 64 * V;
    constexpr int NB = WF == 0 ? 2 * V : V / 2;      // bytes per lane per row
    // 12 rows in flight: a tile holds ~6 active neurons on average and up to ~12 on the
    // busiest placed tiles, whose round sets the kernel's end (LLaMA-7B-shaped layer, µs per
    // step: 16 rows 16.44, 12 16.30, 10 16.78, 8 16.78)
    constexpr int DN_ROWS = 12;
    const int nch = (d + CH - 1) / CH;
    const size_t rowb = WF == 0 ? (size_t)d * 2 : (size_t)(d >> 1);
    float* prow = part + (size_t)tile * d;
    const uint8_t* Wb = static_cast<const uint8_t*>(Wd);
    for (int j = wave; j < nch; j += B_WAVES) {
        const int col0 = j * CH + lane * V;
        const bool cok = col0 < d;                  // d % 8 (fp16) / % 128 (int4): all V or none
        const size_t boff = cok ? (WF == 0 ? (size_t)col0 * 2 : (size_t)(col0 >> 1)) : 0;
        const int sg = cok ? (col0 >> 7) : 0;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.f;
        for (int k0 = 0; k0 < na; k0 += DN_ROWS) {
            uint4 wv[DN_ROWS];         // NB bytes used
            uint32_t sr[DN_ROWS];
            float hv[DN_ROWS];
#pragma unroll
            for (int u = 0; u < DN_ROWS; ++u) {
                const int k = k0 + u;
                const int kk = k < na ? k : 0;
                const size_t row = (size_t)(tile * 64 + s_list[kk]);
                hv[u] = (k < na && cok) ? s_h[kk] : 0.f;
                wv[u] = ld_n<NB>(Wb + row * rowb + boff);
                if (WF == 1) sr[u] = (uint32_t)Sd[row * G + sg];
            }
#pragma unroll
            for (int u = 0; u < DN_ROWS; ++u) {
                if (k0 + u >= na) continue;              // empty slots: loaded, never used
                const uint32_t ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
                if (WF == 0) {
#pragma unroll
                    for (int e = 0; e < V / 2; ++e) {
                        acc[2 * e] = fmaf(hv[u], lo_f(ww[e]), acc[2 * e]);
                        acc[2 * e + 1] = fmaf(hv[u], hi_f(ww[e]), acc[2 * e + 1]);
                    }
                } else {
                    const float hs = hv[u] * h2f((uint16_t)sr[u]);
#pragma unroll
                    for (int e = 0; e < V / 8; ++e) axpy8_i4(acc + 8 * e, ww[e], hs, hs * 0.0625f);
                }
            }
#pragma unroll
            for (int u = 0; u < DN_ROWS; ++u) {
                keep_n<NB>(wv[u]);
                if (WF == 1) keep(sr[u]);
            }
        }
        if (cok) {
            if constexpr (V == 2) {
                *reinterpret_cast<float2*>(prow + col0) = make_float2(acc[0], acc[1]);
            } else {
#pragma unroll
                for (int v = 0; v < V; v += 4)
                    *reinterpret_cast<float4*>(prow + col0 + v) =
                        make_float4(acc[v], acc[v + 1], acc[v + 2], acc[v + 3]);
            }
        }
    }
}


// --------------------------------------------------------------------------------------- C
// Split schedule: the down projection straight from the mask, 2-D tiled.  Block (split,
// slice) owns the neuron ids of a range of mask words and a column slice of y (64 lanes x one
// load each: 512 fp16 columns with 16-byte loads, or 1024 int4 columns with 8-byte loads).  It
// compacts its range in LDS, its 16 waves take interleaved active neurons (U rows in flight
// per wave), the waves' sums meet in LDS in a fixed order, and the block stores its slice of
// partial row `split`.  The range is the grid's fast index, so the blocks of one range (which
// read the same mask words, the same h entries and the same lines of int4 scales) go to the
// same XCD and share its L2.
constexpr int DN_NW = 16;

template <int WF>
struct DnGeom {
    static constexpr int LB = WF == 0 ? 16 : 8;      // bytes per lane load
    static constexpr int V = WF == 0 ? 8 : 16;       // columns per lane
    static constexpr int SC = 64 * V;                // columns per slice
};

// Block-local compaction of mask words [w0, w1) into s_ids (ascending); returns the count.
PI_DEV int range_compact(const uint32_t* __restrict__ mask, int w0, int w1, int F, int* s_ids,
                         int* s_tmp) {
    const int W = (F + 31) >> 5;
    const int t = threadIdx.x;
    if (w1 - w0 <= 64) {                             // block-uniform: wave 0 alone, one barrier
        if (t < 64) {
            uint32_t v = 0;
            if (w0 + t < w1) {
                v = mask[w0 + t];
                if (w0 + t == W - 1 && (F & 31)) v &= (1u << (F & 31)) - 1u;
            }
            const int c = __popc(v);
            const int inc = wave_inclusive_scan(c);
            int pos = inc - c;
            while (v) {
                const int b = __ffs(v) - 1;
                s_ids[pos++] = ((w0 + t) << 5) + b;
                v &= v - 1u;
            }
            if (t == 63) s_tmp[0] = inc;
        }
        __syncthreads();
        return s_tmp[0];
    }
    uint32_t v = 0;
    if (w0 + t < w1) {
        v = mask[w0 + t];
        if (w0 + t == W - 1 && (F & 31)) v &= (1u << (F & 31)) - 1u;
    }
    int total;
    int pos = block_exclusive_scan(__popc(v), s_tmp, &total);
    while (v) {
        const int b = __ffs(v) - 1;
        s_ids[pos++] = ((w0 + t) << 5) + b;
        v &= v - 1u;
    }
    __syncthreads();
    return total;
}

template <int WF, int U>
__global__ __launch_bounds__(DN_NW * 64) void k_dec_down(
    const uint32_t* __restrict__ mask, int F, const float* __restrict__ h,
    const void* __restrict__ Wd, const uint16_t* __restrict__ Sd, int d, int wps,
    float* __restrict__ part, int Wh, int wps_hot, int Rh) {
    using Gm = DnGeom<WF>;
    __shared__ int s_ids[DEC_IDCAP];
    __shared__ __align__(16) float s_red[DN_NW * Gm::SC];
    __shared__ float s_half[512];
    __shared__ int s_tmp[DN_NW + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, slice = blockIdx.y;
    const int W = (F + 31) >> 5;
    // ranges: the first Rh cover the hot block's mask words [0, Wh) wps_hot at a time (a hot
    // word holds ~8 times the active neurons of a cold one), the rest the cold words wps at a time
    const int w0 = split < Rh ? split * wps_hot : min(W, Wh + (split - Rh) * wps);
    const int w1 = split < Rh ? min(Wh, w0 + wps_hot) : min(W, w0 + wps);   // wps: the cold width
    const int n_loc = range_compact(mask, w0, w1, F, s_ids, s_tmp);

    const size_t rowb = WF == 0 ? (size_t)d * 2 : (size_t)(d >> 1);
    const size_t boff = ((size_t)slice * 64 + lane) * Gm::LB;
    const bool cok = boff < rowb;
    const int G = d >> 7;
    const int sg = (slice * Gm::SC + lane * Gm::V) >> 7;   // int4 scale group of this lane
    const uint8_t* Wb = static_cast<const uint8_t*>(Wd);
    float acc[Gm::V];
#pragma unroll
    for (int v = 0; v < Gm::V; ++v) acc[v] = 0.f;
    for (int k0 = wave; k0 < n_loc; k0 += DN_NW * U) {
        float hr[U];
        uint32_t sr[U];        // raw fp16 scales, one per register
        uint4 w16[U];
        uint2 w8[U];
        // unconditional loads (row 0 / column 0 where there is nothing to read), and no use
        // of a loaded value until all of them are issued: a branch-guarded load, or one whose
        // value is consumed at once (even by a select), is waited for on the spot, and in-order
        // completion then makes every row of the round a memory round trip of its own
        int rid[U];            // the round's row ids (row 0 for an empty slot; n_loc >= 1 here)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u * DN_NW;
            rid[u] = s_ids[k < n_loc ? k : 0];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t row = (size_t)__builtin_amdgcn_readfirstlane(rid[u]);
            const size_t off = row * rowb + (cok ? boff : 0);
            hr[u] = h[row];
            if (WF == 0) {
                w16[u] = ld16(Wb + off);
            } else {
                w8[u] = *reinterpret_cast<const uint2*>(Wb + off);
                sr[u] = (uint32_t)Sd[row * G + (cok ? sg : 0)];
            }
        }
        float hv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) hv[u] = (k0 + u * DN_NW < n_loc && cok) ? hr[u] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k0 + u * DN_NW >= n_loc) continue;     // empty slots: loaded, never used
            if (WF == 0) {
                const uint32_t ww[4] = {w16[u].x, w16[u].y, w16[u].z, w16[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(hv[u], lo_f(ww[e]), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(hv[u], hi_f(ww[e]), acc[2 * e + 1]);
                }
            } else {
                const float hs = hv[u] * h2f((uint16_t)sr[u]);
                axpy8_i4(acc, w8[u].x, hs, hs * 0.0625f);
                axpy8_i4(acc + 8, w8[u].y, hs, hs * 0.0625f);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (WF == 0) {
                keep(w16[u]);
            } else {
                keep(w8[u]);
                keep(sr[u]);
            }
        }
    }
    {
        float4* dst = reinterpret_cast<float4*>(&s_red[wave * Gm::SC + lane * Gm::V]);
#pragma unroll
        for (int v = 0; v < Gm::V; v += 4) dst[v / 4] = make_float4(acc[v], acc[v + 1], acc[v + 2], acc[v + 3]);
    }
    __syncthreads();
    // waves' sums -> this block's partial row of the slice (fixed order)
    float s = 0.f;
    int col;
    if (WF == 0) {                       // 512 columns: two half-sums per column
        col = tid & 511;
        const int hf = tid >> 9;
#pragma unroll
        for (int w = 0; w < DN_NW / 2; ++w) s += s_red[(hf * (DN_NW / 2) + w) * Gm::SC + col];
        if (hf == 1) s_half[col] = s;
        __syncthreads();
        if (hf == 0) s += s_half[col];
    } else {                             // 1024 columns: one per thread
        col = tid;
#pragma unroll
        for (int w = 0; w < DN_NW; ++w) s += s_red[w * Gm::SC + col];
    }
    // the block's column sums are its slice of partial row `split` (a later kernel sums the rows)
    const int gcol = slice * Gm::SC + col;
    const bool writer = WF == 0 ? (tid < 512) : true;
    if (writer && gcol < d) part[(size_t)split * d + gcol] = s;
}

// After the last step: y = the fixed-order sum of the P partial rows; block 0 also writes the
// last step's ascending neuron table from its mask.
__global__ __launch_bounds__(256) void k_dec_finish(const float* __restrict__ part, int P, float* __restrict__ y,
                                                    int d, const uint32_t* __restrict__ mask, int F,
                                                    int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ int s_tmp[256 / 64 + 1];
    reduce_partials(part, P, d, y, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4);
    if (blockIdx.x == 0 && idx != nullptr) block_compact<false>(mask, 1, (F + 31) >> 5, F, idx, count, s_tmp);
}

// --------------------------------------------------------------------------------------- dispatch
template <int WF, bool GLU, int Q, bool FUSED, bool P8>
hipError_t launch_b8(dim3 g, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const float* z,
               const pi_pred_desc& p, float theta, float* logits, uint32_t* mask,
               const uint16_t* x, const pi_ffn_desc& f, float* h, float* part) {
    if (lds > 65536) {
        // a hot block's LDS slots can take the tile block past the default 64 KB of dynamic
        // LDS (a gfx950 CU has 160 KB); raise this kernel's limit to what the launch needs
        static size_t raised = 65536;
        if (lds > raised) {
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void*>(&k_dec_stage2_up<WF, GLU, Q, FUSED, P8>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = lds;
        }
    }
    if (e0)
        hipExtLaunchKernelGGL((k_dec_stage2_up<WF, GLU, Q, FUSED, P8>), g, dim3(B_WAVES * 64), (uint32_t)lds, s,
                              e0, e1, 0, z, p.w_p2t, p.s_p2t, p.bias, p.r, p.F, theta, logits, mask, x,
                              f.w_gate, f.s_gate, f.w_up, f.s_up, f.d, h, f.w_down, f.s_down, part, FUSED ? 0 : f.nhot);
    else
        hipLaunchKernelGGL((k_dec_stage2_up<WF, GLU, Q, FUSED, P8>), g, dim3(B_WAVES * 64), lds, s, z, p.w_p2t,
                           p.s_p2t, p.bias, p.r, p.F, theta, logits, mask, x, f.w_gate, f.s_gate, f.w_up,
                           f.s_up, f.d, h, f.w_down, f.s_down, part, FUSED ? 0 : f.nhot);
    return hipSuccess;
}

template <int WF, bool GLU, int Q, bool FUSED>
hipError_t launch_b(dim3 g, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const float* z,
              const pi_pred_desc& p, float theta, float* logits, uint32_t* mask,
              const uint16_t* x, const pi_ffn_desc& f, float* h, float* part) {
    if (p.pfmt == PI_P_I8G128)
        return launch_b8<WF, GLU, Q, FUSED, true>(g, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part);
    return launch_b8<WF, GLU, Q, FUSED, false>(g, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part);
}

template <int WF, bool GLU, bool FUSED>
hipError_t dispatch_b(int q, dim3 g, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                      const float* z, const pi_pred_desc& p, float theta, float* logits,
                      uint32_t* mask, const uint16_t* x, const pi_ffn_desc& f, float* h,
                      float* part) {
#define PI_B(QQ) case QQ: { \
        const hipError_t le = launch_b<WF, GLU, QQ, FUSED>(g, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part); \
        if (le != hipSuccess) return le; } break;
    if constexpr (WF == 0) {
        switch (q) {
            PI_B(1) PI_B(2) PI_B(3) PI_B(4) PI_B(5) PI_B(6) PI_B(7) PI_B(8)
            PI_B(9) PI_B(10) PI_B(11) PI_B(12) PI_B(13) PI_B(14) PI_B(15) PI_B(16)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (q) {
            PI_B(1) PI_B(2) PI_B(3) PI_B(4) PI_B(5) PI_B(6) PI_B(7) PI_B(8)
            default: return hipErrorInvalidValue;
        }
    }
#undef PI_B
    return hipGetLastError();
}

template <bool FUSED>
hipError_t dispatch_b_fmt(const DecPlan& pl, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const float* z,
                          const pi_pred_desc& p, float theta, float* logits, uint32_t* mask,
                          const uint16_t* x, const pi_ffn_desc& f, float* h, float* part) {
    const bool glu = f.act == PI_ACT_REGLU;
    const dim3 gb(pl.ntile);
    const size_t lds = pl.lds_b + (FUSED ? 0 : hot_lds_bytes(f, pl.ntile));
    if (f.wfmt == PI_W_F16)
        return glu ? dispatch_b<0, true, FUSED>(pl.q, gb, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part)
                   : dispatch_b<0, false, FUSED>(pl.q, gb, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part);
    return glu ? dispatch_b<1, true, FUSED>(pl.q, gb, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part)
               : dispatch_b<1, false, FUSED>(pl.q, gb, lds, s, e0, e1, z, p, theta, logits, mask, x, f, h, part);
}

}  // namespace

// The plan's nsplit ranges (about one down block per CU) are shared between the hot and the cold
// words in proportion to their expected active neurons, a hot word taken as DOWN_HOT_DENSITY
// times as dense as a cold one (profiled hot blocks fire on 70-99% of tokens, the cold rest on
// 3-7%: ratios of 14 to 30 on the workloads here).
constexpr int DOWN_HOT_DENSITY = 16;

DownRanges down_ranges(const DecPlan& pl, int nhot, int F) {
    DownRanges r{};
    const int W = (F + 31) / 32;
    r.Wh = nhot > 0 ? std::min(W, (nhot + 31) / 32) : 0;
    if (r.Wh == 0) {
        r.wps_hot = 1;
        r.Rh = 0;
        r.P = pl.nsplit;
        r.wps_cold = pl.wps;
        return r;
    }
    const double wh = (double)DOWN_HOT_DENSITY * r.Wh, wc = (double)(W - r.Wh);
    int rh = (int)std::lround(pl.nsplit * wh / (wh + wc));
    rh = std::max(1, std::min(rh, std::min(r.Wh, pl.nsplit - (W > r.Wh ? 1 : 0))));
    r.wps_hot = (r.Wh + rh - 1) / rh;
    r.Rh = (r.Wh + r.wps_hot - 1) / r.wps_hot;
    const int rc = std::max(1, pl.nsplit - r.Rh);
    const int wps_c = std::max(pl.wps, (W - r.Wh + rc - 1) / rc);   // never more words than fit in LDS
    r.P = r.Rh + (W - r.Wh + wps_c - 1) / wps_c;
    r.wps_cold = wps_c;
    return r;
}

size_t hot_lds_bytes(const pi_ffn_desc& f, int ntile) {
    if (f.nhot <= 0) return 0;
    const size_t rb = f.wfmt == PI_W_F16 ? (size_t)f.d * 2 : (size_t)f.d / 2;
    const size_t hslot = (rb + 1023) & ~(size_t)1023;
    const int hpb = (f.nhot + ntile - 1) / ntile;               // hot neurons (waves) per tile block
    return (size_t)hpb * (f.act == PI_ACT_REGLU ? 2 : 1) * hslot;
}

// the most ranges any hot block (nhot <= 8 ceil(F / 64)) can give the split down projection
static int max_down_ranges(const DecPlan& p, int F) {
    return down_ranges(p, std::min(F, 8 * p.ntile), F).P;
}

DecPlan plan_decode(int d, int r, int F, int wfmt) {
    DecPlan p{};
    p.pred = plan_pred(d, r, F, 1);
    p.ntile = (F + 63) / 64;
    const bool f16 = wfmt == PI_W_F16;
    p.q = f16 ? (d + 511) / 512 : (d + 2047) / 2048;
    p.lds_b = (size_t)align16i(r * 4) + (size_t)(d / 8) * 16;
    // fused down: ntile * d partial sums per step; the split schedule's nsplit * d and its
    // extra kernel boundary win above about 2^20 (between the LLaMA-7B-shaped layer, 0.7M,
    // faster fused, and the OPT-30B-shaped one, 3.2M, faster split)
    p.fused_default = (long long)p.ntile * d <= (1LL << 20);
    const int sc = f16 ? DnGeom<0>::SC : DnGeom<1>::SC;
    p.nslices = (d + sc - 1) / sc;
    const int W = (F + 31) / 32;
    // down blocks: every range adds one partial row of d floats.  int4 rows: about 256, one per
    // CU (the block's LDS leaves room for one; 512 would run as two rounds: LLaMA-70B-shaped
    // layer 31.6 -> 36.1 us per step); fp16 rows: about 512, two per CU at once (OPT-30B-shaped
    // layer 24.28 -> 23.62; 768: 26.2)
    const int nblk = f16 ? 512 : 256, ns_max = f16 ? 64 : 32;
    int ns = (nblk + p.nslices - 1) / p.nslices;
    const int ns_min = (W + (DEC_IDCAP / 32) - 1) / (DEC_IDCAP / 32);
    if (ns > ns_max) ns = ns_max;
    if (ns > W) ns = W;
    if (ns < ns_min) ns = ns_min;
    if (ns < 1) ns = 1;
    p.wps = (W + ns - 1) / ns;
    p.nsplit = (W + p.wps - 1) / p.wps;
    size_t off = COUNTER_BYTES;
    p.off_z = off;
    off = align_up(off + (size_t)r * sizeof(float), 256);
    p.off_h = off;
    off = align_up(off + (size_t)F * sizeof(float), 256);
    p.off_part = off;          // partial rows of either schedule (a hot block adds ranges)
    off = align_up(off + (size_t)std::max(p.ntile, max_down_ranges(p, F)) * d * sizeof(float), 256);
    p.bytes = off;
    return p;
}

hipError_t launch_decode_step(const pi_pred_desc& p, const pi_ffn_desc& f, const DecPlan& pl, bool fused,
                              const uint16_t* x, float theta, float* logits, uint32_t* mask,
                              float* y, bool convert_prev, char* ws, hipStream_t s,
                              hipEvent_t e0, hipEvent_t e1) {
    float* z = reinterpret_cast<float*>(ws + pl.off_z);
    float* h = reinterpret_cast<float*>(ws + pl.off_h);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    // the previous step (same schedule) left its partial rows: stage 1 sums them into y
    hipError_t e = launch_pred_stage1(p, pl.pred, x, 1, z, s, convert_prev ? part : nullptr, y,
                                      fused ? pl.ntile : down_ranges(pl, f.nhot, f.F).P);
    if (e != hipSuccess) return e;
    if (fused) return dispatch_b_fmt<true>(pl, s, e0, e1, z, p, theta, logits, mask, x, f, h, part);
    if ((e = dispatch_b_fmt<false>(pl, s, e0, e1, z, p, theta, logits, mask, x, f, h, part)) != hipSuccess)
        return e;
    const DownRanges dr = down_ranges(pl, f.nhot, f.F);
    const dim3 gc(dr.P, pl.nslices);          // range fastest: one range's blocks on one XCD
    // rows in flight per wave (16 waves): enough slots for a range's active rows in one round
    // and few empty ones (each still loads); LLaMA-70B-shaped int4 layer, µs per step: 12 rows
    // 31.67, 10 31.37, 8 31.13, 7 31.07, 6 31.41; OPT-30B-shaped fp16: 8 rows 23.64, 6 23.26,
    // 4 23.09, 3 23.10, 2 23.33
    if (f.wfmt == PI_W_F16)
        hipLaunchKernelGGL((k_dec_down<0, 4>), gc, dim3(DN_NW * 64), 0, s, mask, f.F, h, f.w_down,
                           f.s_down, f.d, dr.wps_cold, part, dr.Wh, dr.wps_hot, dr.Rh);
    else
        hipLaunchKernelGGL((k_dec_down<1, 8>), gc, dim3(DN_NW * 64), 0, s, mask, f.F, h, f.w_down,
                           f.s_down, f.d, dr.wps_cold, part, dr.Wh, dr.wps_hot, dr.Rh);
    return hipGetLastError();
}

hipError_t launch_reduce_rows(const float* part, int P, int d, float* y, hipStream_t s) {
    const int nq = d / 4;                         // one 4-column quad per wave
    hipLaunchKernelGGL(k_dec_finish, dim3((nq + 3) / 4), dim3(256), 0, s, part, P, y, d, nullptr, 0,
                       nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_decode_finish(const DecPlan& pl, bool fused, int nhot, int d, int F, const uint32_t* mask,
                                int32_t* idx, int32_t* count, float* y, char* ws, hipStream_t s) {
    const float* part = reinterpret_cast<const float*>(ws + pl.off_part);
    const int nq = d / 4;                         // one 4-column quad per wave
    hipLaunchKernelGGL(k_dec_finish, dim3((nq + 3) / 4), dim3(256), 0, s, part,
                       fused ? pl.ntile : down_ranges(pl, nhot, F).P, y, d, mask, F, idx, count);
    return hipGetLastError();
}

}  // namespace pi
