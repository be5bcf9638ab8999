// Device helpers shared by the gfx950 kernels of the sparse FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

#define PI_DEV __device__ __forceinline__

// ---- fp16 ------------------------------------------------------------------------
PI_DEV float h2f(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
PI_DEV float lo_f(uint32_t v) { return h2f((uint16_t)(v & 0xFFFFu)); }
PI_DEV float hi_f(uint32_t v) { return h2f((uint16_t)(v >> 16)); }

// a.x*b.x + a.y*b.y + acc with fp16 inputs and fp32 products / accumulation (v_dot2_f32_f16)
PI_DEV float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), acc, false);
}
PI_DEV float dot8(const uint4& a, const uint4& b, float acc) {
    acc = dot2(a.x, b.x, acc);
    acc = dot2(a.y, b.y, acc);
    acc = dot2(a.z, b.z, acc);
    return dot2(a.w, b.w, acc);
}

__host__ __device__ constexpr int align16i(int v) { return (v + 15) & ~15; }

// (a & m) | c in one v_and_or_b32 (the compiler splits it in two when both constants are
// literals, which gfx9 VOP3 encodings cannot hold); m in an SGPR, c in a VGPR
PI_DEV uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

// sum over the 32 int4 weights of one 16-byte chunk of (u - 8) * x, with x given as the 16
// fp16 pairs (x[8m+p], x[8m+p+4]), m = word, p = nibble pair.  Each pair is widened exactly by
// OR-ing it into the mantissa of fp16 1024.0: the nibbles at bits 0-3 (pairs 0 and 2, the
// latter after a shift by 8) give 1024 + u, those at bits 4-7 (pairs 1 and 3) 1024 + 16 u; one
// packed fp16 subtraction makes that u - 8 or 16 (u - 8), both exact, and v_dot2_f32_f16
// dots them with x in fp32 (the factor 16 comes out of the second sum exactly at the end).
PI_DEV float dot32_i4(const uint4& w, const uint32_t* xp) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    const h2_t o0 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2_t o1 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t mg = 0x64006400u;
    float a1 = 0.f, a16 = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t v = ws[m], v8 = v >> 8;
        const h2_t q0 = __builtin_bit_cast(h2_t, and_or(v, 0x000F000Fu, mg)) - o0;
        const h2_t q1 = __builtin_bit_cast(h2_t, and_or(v, 0x00F000F0u, mg)) - o1;
        const h2_t q2 = __builtin_bit_cast(h2_t, and_or(v8, 0x000F000Fu, mg)) - o0;
        const h2_t q3 = __builtin_bit_cast(h2_t, and_or(v8, 0x00F000F0u, mg)) - o1;
        a1 = __builtin_amdgcn_fdot2(q0, __builtin_bit_cast(h2_t, xp[4 * m]), a1, false);
        a16 = __builtin_amdgcn_fdot2(q1, __builtin_bit_cast(h2_t, xp[4 * m + 1]), a16, false);
        a1 = __builtin_amdgcn_fdot2(q2, __builtin_bit_cast(h2_t, xp[4 * m + 2]), a1, false);
        a16 = __builtin_amdgcn_fdot2(q3, __builtin_bit_cast(h2_t, xp[4 * m + 3]), a16, false);
    }
    return fmaf(a16, 0.0625f, a1);
}

// acc[n] += hs * (u_n - 8) for the 8 int4 weights u_n of word v (nibble n = column n; hs16 =
// hs / 16).  Each nibble pair (n, n + 4) is widened exactly by OR-ing it into the mantissa of
// fp16 1024.0: the nibbles at bits 0-3 give 1024 + u, those at bits 4-7 give 1024 + 16 u, and
// one packed fp16 subtraction of 1032 or 1152 makes that u - 8 or 16 (u - 8), both exact; the
// fp32 FMAs take the fp16 operand directly (v_fma_mix_f32), the 16 folded into hs16.
PI_DEV void axpy8_i4(float* acc, uint32_t v, float hs, float hs16) {
    const h2_t o0 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2_t o1 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t v8 = v >> 8;
    const uint32_t mg = 0x64006400u;
    const h2_t q0 = __builtin_bit_cast(h2_t, and_or(v, 0x000F000Fu, mg)) - o0;
    const h2_t q1 = __builtin_bit_cast(h2_t, and_or(v, 0x00F000F0u, mg)) - o1;
    const h2_t q2 = __builtin_bit_cast(h2_t, and_or(v8, 0x000F000Fu, mg)) - o0;
    const h2_t q3 = __builtin_bit_cast(h2_t, and_or(v8, 0x00F000F0u, mg)) - o1;
    acc[0] = fmaf(hs, (float)q0.x, acc[0]);
    acc[4] = fmaf(hs, (float)q0.y, acc[4]);
    acc[1] = fmaf(hs16, (float)q1.x, acc[1]);
    acc[5] = fmaf(hs16, (float)q1.y, acc[5]);
    acc[2] = fmaf(hs, (float)q2.x, acc[2]);
    acc[6] = fmaf(hs, (float)q2.y, acc[6]);
    acc[3] = fmaf(hs16, (float)q3.x, acc[3]);
    acc[7] = fmaf(hs16, (float)q3.y, acc[7]);
}

// sum of the 8 fp16 values of w times 8 fp32 values (za, zb), fp32 FMAs
PI_DEV float dot8_f32(const uint4& w, const float4& za, const float4& zb) {
    float a = lo_f(w.x) * za.x;
    a = fmaf(hi_f(w.x), za.y, a);
    a = fmaf(lo_f(w.y), za.z, a);
    a = fmaf(hi_f(w.y), za.w, a);
    a = fmaf(lo_f(w.z), zb.x, a);
    a = fmaf(hi_f(w.z), zb.y, a);
    a = fmaf(lo_f(w.w), zb.z, a);
    return fmaf(hi_f(w.w), zb.w, a);
}

// ---- int8 predictor rows (one 16-byte chunk = 16 signed weights) -----------------------------
PI_DEV float i8f(uint32_t w, int k) { return (float)(int8_t)(uint8_t)(w >> (8 * k)); }

// sum over the 16 bytes of w of (signed byte) * v, v = a, b, c, e (fp32, in byte order)
PI_DEV float dot16_i8_f32(const uint4& w, const float4& a, const float4& b, const float4& c,
                          const float4& e) {
    float s = 0.f;
    s = fmaf(i8f(w.x, 0), a.x, s); s = fmaf(i8f(w.x, 1), a.y, s);
    s = fmaf(i8f(w.x, 2), a.z, s); s = fmaf(i8f(w.x, 3), a.w, s);
    s = fmaf(i8f(w.y, 0), b.x, s); s = fmaf(i8f(w.y, 1), b.y, s);
    s = fmaf(i8f(w.y, 2), b.z, s); s = fmaf(i8f(w.y, 3), b.w, s);
    s = fmaf(i8f(w.z, 0), c.x, s); s = fmaf(i8f(w.z, 1), c.y, s);
    s = fmaf(i8f(w.z, 2), c.z, s); s = fmaf(i8f(w.z, 3), c.w, s);
    s = fmaf(i8f(w.w, 0), e.x, s); s = fmaf(i8f(w.w, 1), e.y, s);
    s = fmaf(i8f(w.w, 2), e.z, s); s = fmaf(i8f(w.w, 3), e.w, s);
    return s;
}

// the same with 16 fp16 values (x0: elements 0-7, x1: 8-15)
PI_DEV float dot16_i8_f16(const uint4& w, const uint4& x0, const uint4& x1) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    const uint32_t xx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s = fmaf(i8f(ww[i], 0), lo_f(xx[2 * i]), s);
        s = fmaf(i8f(ww[i], 1), hi_f(xx[2 * i]), s);
        s = fmaf(i8f(ww[i], 2), lo_f(xx[2 * i + 1]), s);
        s = fmaf(i8f(ww[i], 3), hi_f(xx[2 * i + 1]), s);
    }
    return s;
}

// An empty use of a loaded value, placed after the loop that consumes it under a uniform
// condition: with a use outside the condition the compiler cannot sink the load into the
// conditional block (where it would be waited for at once, one memory round trip per row).
PI_DEV void keep(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
PI_DEV void keep(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }
PI_DEV void keep(uint32_t& v) { asm volatile("" : "+v"(v)); }
PI_DEV void keep(float& v) { asm volatile("" : "+v"(v)); }
// keep() for the NB loaded bytes of an ld_n value
template <int NB>
PI_DEV void keep_n(uint4& v) {
    if constexpr (NB == 16) {
        keep(v);
    } else if constexpr (NB == 8) {
        asm volatile("" : "+v"(v.x), "+v"(v.y));
    } else {
        asm volatile("" : "+v"(v.x));
    }
}

// 16-byte global load
PI_DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// NB-byte (16, 8 or 4) global load into the low words of a uint4 (the rest zero)
template <int NB>
PI_DEV uint4 ld_n(const void* p) {
    if constexpr (NB == 16) {
        return *reinterpret_cast<const uint4*>(p);
    } else if constexpr (NB == 8) {
        const uint2 t = *reinterpret_cast<const uint2*>(p);
        return make_uint4(t.x, t.y, 0u, 0u);
    } else {
        return make_uint4(*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u);
    }
}
PI_DEV uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// On the batch path weight rows are read once per step while x, the H fragments and the
// partial sums are read many times: non-temporal loads of the rows (and buffer loads with
// the nt cache-policy bit, PI_NT) keep them from evicting the reused data from L2.
constexpr int PI_NT = 2;
// A raw buffer resource over `bytes` bytes at p (loads past them return 0).  Word 3 names a
// 32-bit data format: with a zero format every load would return 0.
PI_DEV __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
PI_DEV uint4 ld16_nt(const void* p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
PI_DEV uint2 ld8_nt(const void* p) {
    const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(t.x, t.y);
}

// ---- wave-level (DPP: cross-lane moves inside the VALU, no LDS round trip) ----------------------
// update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl): lanes whose source lane is
// outside the row, or whose row is masked off, get `old`.
template <int CTRL, int ROW_MASK = 0xF>
PI_DEV int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
PI_DEV float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
PI_DEV float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over the 64 lanes, returned (wave-uniform) to every lane.  Pairs, quads, half rows and
// rows of 16 are summed with DPP quad_perm / row_half_mirror / row_mirror; the four row sums
// are then read from lanes 0, 16, 32, 48.  Fixed order, so the result is deterministic.
PI_DEV float wave_sum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);   // row_half_mirror
    v += dpp_f<0x140>(v);   // row_mirror
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Position of the k-th (from 0) set bit of m (k < popcount(m)): a binary search on popcounts,
// scalar when m and k are wave-uniform.
PI_DEV int kth_set_bit(unsigned long long m, int k) {
    int pos = 0;
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) {
        const unsigned long long low = m & ((1ull << s) - 1ull);
        const int c = __popcll(low);
        if (k >= c) {
            k -= c;
            m >>= s;
            pos += s;
        } else {
            m = low;
        }
    }
    return pos;
}

// Inclusive prefix sum over the 64 lanes (integers): row_shr 1, 2, 4, 8 inside each row of
// 16, then row_bcast 15 / 31 carry row totals into the rows above.
PI_DEV int wave_inclusive_scan(int v) {
    v += dpp_i<0x111>(v);          // row_shr:1
    v += dpp_i<0x112>(v);          // row_shr:2
    v += dpp_i<0x114>(v);          // row_shr:4
    v += dpp_i<0x118>(v);          // row_shr:8
    v += dpp_i<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
    v += dpp_i<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
    return v;
}

// ---- cross-block "last arrival" ------------------------------------------------------------
// Blocks hand partial results to one another through memory.  An agent-scope
// fence here would write back and invalidate the whole L2 of the XCD for every
// block, so instead the partials are written and read with relaxed agent-scope
// atomic stores / loads: on gfx950 these are plain stores / loads with the sc1
// (agent coherence) bit, coherent across the XCDs' L2s by themselves.
PI_DEV void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
PI_DEV void st_agent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
PI_DEV float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
PI_DEV uint32_t ld_agent(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- deterministic cross-block sums: fp32 partial rows, reduced in a fixed order -------------
// Producers (blocks that each own a share of the neurons) store their d column sums as one
// partial row part[p, 0 .. d) with plain stores; a later kernel turns the P rows into y.  The
// order of that sum is a function of P alone -- not of the grid that runs it -- so every
// kernel that reduces the same rows gets the same bits, and repeated runs are bit-identical.
// Values are fp32 throughout: relative (not absolute) precision, and NaN / Inf propagate.

// y[c] = sum over p < P of part[p * d + c] (d % 4 == 0; part and y 16-byte aligned).  A unit is
// one 4-column quad, taken by a whole wave: lane j adds the rows p = j, j + 64, j + 128, ... in
// ascending order (all of a lane's loads in flight together, eight at a time), and the 64 lane
// sums meet in wave_sum's fixed pattern.  gw / nw: this wave's index in the grid and the
// grid's number of waves (quads are dealt out round-robin).  Every lane of the wave must call
// it (it uses cross-lane moves).
PI_DEV void reduce_partials(const float* __restrict__ part, int P, int d, float* __restrict__ y,
                            int gw, int nw) {
    const int lane = threadIdx.x & 63;
    const int nq = d >> 2;
    for (int q = gw; q < nq; q += nw) {
        const float* src = part + (size_t)q * 4;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int p0 = 0; p0 < P; p0 += 64 * 8) {
            float4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int p = p0 + 64 * k + lane;
                v[k] = *reinterpret_cast<const float4*>(src + (size_t)(p < P ? p : 0) * d);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (p0 + 64 * k + lane < P) {
                    s.x += v[k].x;
                    s.y += v[k].y;
                    s.z += v[k].z;
                    s.w += v[k].w;
                }
            }
        }
        s.x = wave_sum(s.x);
        s.y = wave_sum(s.y);
        s.z = wave_sum(s.z);
        s.w = wave_sum(s.w);
        if (lane == 0) *reinterpret_cast<float4*>(y + 4 * q) = s;
    }
}

// Batch rows: y[b, c] = the nks shares' partials part[(k * 32 + b) * d + c] added in share order,
// from 0, in groups of 8 with zeros for the shares past nks -- bit for bit the sum the union down
// kernel's last block forms.  Unit q (one 4-column quad of one token, q < B d / 4) per thread;
// its nks loads are in flight together, 8 at a time.  d % 4 == 0, part and y 16-byte aligned.
PI_DEV void reduce_share_rows(const float* __restrict__ part, int nks, int B, int d,
                              float* __restrict__ y, int q) {
    const int nq = d >> 2;
    if (q >= B * nq) return;
    const int b = q / nq, c = 4 * (q - b * nq);
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < nks; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = *reinterpret_cast<const float4*>(part + ((size_t)(k0 + k < nks ? k0 + k : 0) * 32 + b) * d + c);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool ok = k0 + k < nks;
            t.x += ok ? v[k].x : 0.f;
            t.y += ok ? v[k].y : 0.f;
            t.z += ok ? v[k].z : 0.f;
            t.w += ok ? v[k].w : 0.f;
        }
    }
    *reinterpret_cast<float4*>(y + (size_t)b * d + c) = t;
}

// Every block calls this once, after all its threads issued their st_agent
// partials.  The barrier drains the stores (vmcnt(0)) before thread 0 bumps the
// arrival counter, so the block that sees the final count reads complete
// partials with ld_agent.  Exactly that last block gets true; it resets the
// counter, which therefore starts at zero for the next launch on the stream.
PI_DEV bool last_block_arrive(unsigned* counter, unsigned nblocks) {
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == nblocks - 1u);
        if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    return s_last != 0;
}

// ---- block-wide exclusive scan of one int per thread --------------------------------------
// s_tmp needs (blockDim.x / 64 + 1) ints.  Returns the exclusive prefix; *total gets the sum.
PI_DEV int block_exclusive_scan(int v, int* s_tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int inc = wave_inclusive_scan(v);
    if (lane == 63) s_tmp[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            int t = s_tmp[w];
            s_tmp[w] = run;
            run += t;
        }
        s_tmp[nw] = run;
    }
    __syncthreads();
    const int excl = inc - v + s_tmp[wave];
    *total = s_tmp[nw];
    __syncthreads();
    return excl;
}

// ---- neuron-table compaction by one block ------------------------------------------------------
// Writes, in ascending order, the positions of the set bits among the first F
// bits of the mask (the OR of `nrows` masks of W words each, rows `stride`
// words apart) to out[0 .. n), and n to *count.  Each thread owns a run of
// consecutive words, so an exclusive scan of per-thread popcounts gives every
// thread its first output slot.
template <bool COHERENT>
PI_DEV uint32_t mask_word(const uint32_t* mask, int nrows, int stride, int w, int W, int F) {
    auto ld = [&](int b) {
        const uint32_t* p = mask + (size_t)b * stride + w;
        return COHERENT ? ld_agent(p) : *p;
    };
    uint32_t v = 0;
    if (nrows == 1) {
        v = ld(0);
    } else {
        // the rows' words in groups of 16 loads, all issued before the first is used (one
        // memory round trip per group); rows past the last repeat it, which leaves the OR as it
        // is and keeps every load unconditional (a load under a condition is waited for at once)
        for (int b0 = 0; b0 < nrows; b0 += 16) {
            uint32_t t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = ld(min(b0 + i, nrows - 1));
#pragma unroll
            for (int i = 0; i < 16; ++i) v |= t[i];
        }
    }
    if (w == W - 1 && (F & 31)) v &= (1u << (F & 31)) - 1u;
    return v;
}

// Ascending ids of the set bits of the OR of nrows masks (F bits each, row stride `stride`
// words) -> out[0 .. count).  Rounds of blockDim.x words, one word per thread; after the
// block scan each wave writes its words' ids two words at a time (lanes 0-31 one word,
// 32-63 the next, lane = bit), so a store instruction covers up to 64 consecutive ids.
template <bool COHERENT>
PI_DEV void block_compact(const uint32_t* mask, int nrows, int stride, int F, int32_t* out,
                          int32_t* count, int* s_tmp) {
    const int W = (F + 31) >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bit = lane & 31, sel = lane >> 5;
    int base = 0;
    for (int r0 = 0; r0 < W; r0 += (int)blockDim.x) {
        const int w = r0 + (int)threadIdx.x;
        const uint32_t v = w < W ? mask_word<COHERENT>(mask, nrows, stride, w, W, F) : 0u;
        int total;
        const int pos = base + block_exclusive_scan(__popc(v), s_tmp, &total);
        const int wb = r0 + wave * 64;            // this wave's first word
        for (int j = 0; j < 64; j += 2) {
            const uint32_t v0 = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
            const uint32_t v1 = (uint32_t)__builtin_amdgcn_readlane((int)v, j + 1);
            if ((v0 | v1) == 0u) continue;        // wave-uniform
            const int p0 = __builtin_amdgcn_readlane(pos, j);
            const int p1 = __builtin_amdgcn_readlane(pos, j + 1);
            const uint32_t vv = sel ? v1 : v0;
            if ((vv >> bit) & 1u)
                out[(sel ? p1 : p0) + __popc(vv & ((1u << bit) - 1u))] = ((wb + j + sel) << 5) + bit;
        }
        base += total;
    }
    if (threadIdx.x == 0) *count = base;
}

// ---- predictor stage 2 on one 64-neuron tile (blocks of NW waves) ------------------------------
// Wave w owns rows n0 + w*RPW .. n0 + w*RPW + RPW - 1 of W2t [F, r] (row n = neuron n's
// predictor weights, contiguous), RPW = 64 / NW.  A row is read by all 64 lanes in segments
// of 128 16-byte chunks (1024 predictor columns in fp16, 2048 in int8), so a segment's loads
// are all in flight.  P8: int8 rows with one fp16 scale per 128 columns (per 8 chunks).
template <bool P8>
PI_DEV int tile_chunks(int r) { return P8 ? (r >> 4) : (r >> 3); }
// chunks per lane per row in one segment (int8 rows are half as long: one chunk a lane
// covers 1024 columns), and chunks per segment
template <bool P8> constexpr int TILE_QC = P8 ? 1 : 2;
template <bool P8> constexpr int TILE_SEG = 64 * TILE_QC<P8>;

template <int NW, bool P8 = false>
struct TileRows {
    static constexpr int RPW = 64 / NW;
    uint4 w[RPW][2];
};

template <int NW>
struct TileRows<NW, true> {
    static constexpr int RPW = 64 / NW;
    uint4 w[RPW][1];
    uint32_t s[RPW][1];                           // raw fp16 scales (int8 rows)
};

template <int NW, bool P8 = false>
PI_DEV void tile_rows_load(TileRows<NW, P8>& tr, const void* __restrict__ W2t,
                           const uint16_t* __restrict__ S2, int r, int F, int tile, int c0) {
    constexpr int RPW = TileRows<NW, P8>::RPW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nr = tile_chunks<P8>(r);
#pragma unroll
    for (int m = 0; m < RPW; ++m) {
        const int n = tile * 64 + wave * RPW + m;
#pragma unroll
        for (int q = 0; q < TILE_QC<P8>; ++q) {
            const int c = c0 + lane + 64 * q;
            if constexpr (P8) {
                // the row's bases are wave-uniform (scalar registers); lanes add their offsets
                // the scale load is unconditional (clamped row and chunk): a load merged with
                // a constant under a lane condition is waited for on the spot
                const int nu = __builtin_amdgcn_readfirstlane(n);
                const int8_t* W8 = static_cast<const int8_t*>(W2t) + (size_t)nu * r;
                const uint16_t* s8 = S2 + (size_t)(nu < F ? nu : 0) * (r >> 7);
                tr.w[m][q] = (nu < F && c < nr) ? ld16(W8 + 16 * c) : zero4();
                tr.s[m][q] = (uint32_t)s8[(c < nr ? c : 0) >> 3];
            } else {
                const uint16_t* W16 = static_cast<const uint16_t*>(W2t);
                tr.w[m][q] = (n < F && c < nr) ? ld16(W16 + (size_t)n * r + 8 * c) : zero4();
            }
        }
    }
}

// acc[m] += row m . z over the segment starting at chunk c0 (z in LDS, fp32)
template <int NW, bool P8 = false>
PI_DEV void tile_rows_fma(const TileRows<NW, P8>& tr, const float* s_z, int r, int c0, float* acc) {
    constexpr int RPW = TileRows<NW, P8>::RPW;
    const int lane = threadIdx.x & 63;
    const int nr = tile_chunks<P8>(r);
#pragma unroll
    for (int q = 0; q < TILE_QC<P8>; ++q) {
        const int c = c0 + lane + 64 * q;
        if (c < nr) {
            if constexpr (P8) {
                const float4* zp = reinterpret_cast<const float4*>(&s_z[16 * c]);
                const float4 za = zp[0], zb = zp[1], zc = zp[2], zd = zp[3];
#pragma unroll
                for (int m = 0; m < RPW; ++m)
                    acc[m] = fmaf(h2f((uint16_t)tr.s[m][q]), dot16_i8_f32(tr.w[m][q], za, zb, zc, zd), acc[m]);
            } else {
                const float4 za = *reinterpret_cast<const float4*>(&s_z[8 * c]);
                const float4 zb = *reinterpret_cast<const float4*>(&s_z[8 * c + 4]);
#pragma unroll
                for (int m = 0; m < RPW; ++m) acc[m] += dot8_f32(tr.w[m][q], za, zb);
            }
        }
    }
}

// Finish a tile: reduce each wave's RPW row sums and store them to s_l[64].  Caller syncs.
template <int NW>
PI_DEV void tile_rows_store(const float* acc, float* s_l) {
    constexpr int RPW = TileRows<NW>::RPW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < RPW; ++m) {
        const float v = wave_sum(acc[m]);
        if (lane == 0) s_l[wave * RPW + m] = v;
    }
}

// The same 64 row sums through a transposed butterfly (8 rows per wave): a lane swaps half of
// what it holds with the lane 1, 2 and then 4 apart, keeping (and adding) the other half --
// one add per kept row instead of a whole-wave reduction per row -- and then adds the value of
// the lane 8 apart.  Lane l of each row of 16 then holds the 16-lane sum of the wave's row
// 4 b0 + 2 b1 + b2 (b: bits of l); the lanes with b3 = 0 store it as s4[4 k + l / 16] for tile
// row k.  tile_row_sum(s4, k) adds the four in a fixed order.  Caller syncs between the two.
template <int NW>
PI_DEV void tile_rows_store4(const float* acc, float* s4) {
    static_assert(TileRows<NW>::RPW == 8, "8 rows per wave");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1;
    float a4[4], a2[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {                       // keep rows 4 b0 + i
        const float keep = b0 ? acc[i + 4] : acc[i], send = b0 ? acc[i] : acc[i + 4];
        a4[i] = keep + dpp_f<0xB1>(send);               // quad_perm [1,0,3,2]: lane ^ 1
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {                       // keep rows 4 b0 + 2 b1 + j
        const float keep = b1 ? a4[j + 2] : a4[j], send = b1 ? a4[j] : a4[j + 2];
        a2[j] = keep + dpp_f<0x4E>(send);               // quad_perm [2,3,0,1]: lane ^ 2
    }
    float v = (b2 ? a2[1] : a2[0]) + __shfl_xor(b2 ? a2[0] : a2[1], 4);
    v += dpp_f<0x128>(v);                               // row_ror:8: lane ^ 8 within 16
    if ((lane & 8) == 0) s4[(wave * 8 + 4 * b0 + 2 * b1 + b2) * 4 + (lane >> 4)] = v;
}
PI_DEV float tile_row_sum(const float* s4, int k) {
    const float4 q = reinterpret_cast<const float4*>(s4)[k];
    return (q.x + q.y) + (q.z + q.w);
}

// s_l[k] = W2t[tile*64 + k, :] . z for k < 64 (before the bias); z in LDS.  Caller syncs after.
template <int NW, bool P8 = false>
PI_DEV void tile_logits(const void* __restrict__ W2t, const uint16_t* __restrict__ S2, const float* s_z,
                        int r, int F, int tile, float* s_l) {
    float acc[TileRows<NW, P8>::RPW] = {};
    for (int c0 = 0; c0 < tile_chunks<P8>(r); c0 += TILE_SEG<P8>) {
        TileRows<NW, P8> tr;
        tile_rows_load<NW, P8>(tr, W2t, S2, r, F, tile, c0);
        tile_rows_fma<NW, P8>(tr, s_z, r, c0, acc);
    }
    tile_rows_store<NW>(acc, s_l);
}
