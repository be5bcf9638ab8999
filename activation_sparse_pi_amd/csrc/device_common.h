// Device helpers shared by the gfx950 kernels of the sparse FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// 16-byte global load
PI_DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
PI_DEV uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// ---- wave-level ------------------------------------------------------------------------
PI_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---- cross-block "last arrival" --------------------------------------------------------------
// Every block calls this once after writing its partial results.  Exactly one
// block (the last to arrive) gets true, after an agent-scope acquire, and may
// then read every other block's writes.  The counter is reset to zero by that
// block, so it starts at zero for the next launch on the stream.
PI_DEV bool last_block_arrive(unsigned* counter, unsigned nblocks) {
    __shared__ int s_last;
    __threadfence();                 // release this thread's writes (agent scope)
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned prev = atomicAdd(counter, 1u);
        int last = (prev == nblocks - 1u);
        if (last) atomicExch(counter, 0u);
        s_last = last;
    }
    __syncthreads();
    const bool last = s_last != 0;
    if (last) __threadfence();       // acquire the other blocks' writes
    return last;
}

// ---- block-wide exclusive scan of one int per thread --------------------------------------
// s_tmp needs (blockDim.x / 64 + 1) ints.  Returns the exclusive prefix; *total gets the sum.
PI_DEV int block_exclusive_scan(int v, int* s_tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
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
PI_DEV uint32_t mask_word(const uint32_t* mask, int nrows, int stride, int w, int W, int F) {
    uint32_t v = 0;
    for (int b = 0; b < nrows; ++b) v |= mask[(size_t)b * stride + w];
    if (w == W - 1 && (F & 31)) v &= (1u << (F & 31)) - 1u;
    return v;
}

PI_DEV void block_compact(const uint32_t* mask, int nrows, int stride, int F, int32_t* out,
                          int32_t* count, int* s_tmp) {
    const int W = (F + 31) >> 5;
    const int per = (W + (int)blockDim.x - 1) / (int)blockDim.x;
    const int w0 = threadIdx.x * per;
    int c = 0;
    for (int i = 0; i < per; ++i) {
        const int w = w0 + i;
        if (w < W) c += __popc(mask_word(mask, nrows, stride, w, W, F));
    }
    int total;
    int pos = block_exclusive_scan(c, s_tmp, &total);
    for (int i = 0; i < per; ++i) {
        const int w = w0 + i;
        if (w >= W) break;
        uint32_t v = mask_word(mask, nrows, stride, w, W, F);
        while (v) {
            const int b = __ffs(v) - 1;
            out[pos++] = (w << 5) + b;
            v &= v - 1u;
        }
    }
    if (threadIdx.x == 0) *count = total;
}
