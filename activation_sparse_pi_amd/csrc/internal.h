// Internal interface between the C ABI layer (pi_abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pi.h"

namespace pi {

// ---- arrival-counter slots inside the workspace (unsigned ints) ------------------------------
constexpr int CNT_PRED1 = 0;      // (free: 256 slots)
constexpr int CNT_PRED2 = 256;    // one for stage 2's compaction
constexpr int CNT_DOWN = 512;     // one per down-projection column slice (<= 512)
constexpr int CNT_UNION = 1024;   // union path, down-product column groups (<= 512)
constexpr int CNT_TOTAL = 4096;
constexpr size_t COUNTER_BYTES = CNT_TOTAL * sizeof(unsigned);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- predictor launch plan ----------------------------------------------------------------------
struct PredPlan {
    int qs;       // stage-1 16-byte chunks per lane per row segment
    int nblk1;    // stage-1 blocks (4 rows each)
    int nblk2;    // stage-2 blocks (64 neurons each)
    int nbz;      // tokens whose z is staged in LDS at a time (stage 2)
    size_t lds2;  // stage-2 dynamic LDS
    size_t off_z, bytes;
    // 1 < B <= 32 (MFMA stages): stage-1 row tiles of 32, shares of d, share partial sums
    int b_ntile, b_nks;
    size_t off_zpart;
};
PredPlan plan_pred(int d, int r, int F, int B);
// appends the batch predictor's workspace to p from offset off (advanced in place)
void plan_pred_batch(PredPlan& p, int d, int r, int F, size_t& off);

// ---- batch-1 FFN launch plan ----------------------------------------------------------------------
struct FfnPlan {
    int q;         // 16-byte chunks per lane per row in the up kernel
    int up_blocks; // 256-thread blocks of the up kernel
    int cols;      // columns per down slice
    int nslices, nsplit;
    size_t off_h, off_part, bytes;
    // union (B > 1) path: H fragments, down-product column groups and list shares,
    // the shares' partial sums (all 0 when B == 1)
    int u_ncg, u_ks;
    size_t off_H, off_upart, off_upcnt, off_uppart;
};
FfnPlan plan_ffn(int d, int F, int wfmt, int B);
// appends the union path's workspace to p from offset off; returns the new end
size_t plan_union(FfnPlan& p, int d, int F, size_t off);

// ---- fused batch-1 decode step (three kernels) --------------------------------------------
struct DecPlan {
    PredPlan pred;
    int ntile, q;              // tiles of 64 neurons, chunks per lane per up/gate row
    size_t lds_b;              // dynamic LDS of the tile kernel
    bool fused_default;        // the schedule chosen for this shape
    int nslices, nsplit, wps;  // split schedule's down grid: column slices, ranges, mask words per range
    size_t off_z, off_h, off_part, bytes;   // off_part: max(ntile, nsplit) partial rows of d floats
};
DecPlan plan_decode(int d, int r, int F, int wfmt);
// The split schedule's down ranges: Rh ranges of wps_hot mask words over the hot block's words
// [0, Wh), then ranges of wps_cold words over the rest; P partial rows in all.
struct DownRanges {
    int Wh, wps_hot, Rh, P, wps_cold;
};
DownRanges down_ranges(const DecPlan& pl, int nhot, int F);
// Dynamic LDS of the split schedule's hot-block slots: ceil(nhot / ntile) waves per tile block,
// one 1 KB-aligned row slot per matrix (gate, up); 0 without a hot block.
size_t hot_lds_bytes(const pi_ffn_desc& f, int ntile);
constexpr int DEC_LDS_MAX = 160 * 1024;   // LDS of a gfx950 CU
// One step: two kernels (fused: each tile block stores its down projection as one partial row
// of d floats) or three (split: a down kernel over ranges of the mask, one partial row per
// range).  When convert_prev is set, the first kernel sums the previous step's partial rows
// into y (same schedule), in a fixed order.
hipError_t launch_decode_step(const pi_pred_desc& p, const pi_ffn_desc& f, const DecPlan& pl, bool fused,
                              const uint16_t* x, float theta, float* logits, uint32_t* mask,
                              float* y, bool convert_prev, char* ws, hipStream_t s,
                              hipEvent_t e0, hipEvent_t e1);
// After the last step: y = the fixed-order sum of its partial rows, and the last step's neuron
// table (idx, count; skipped when idx is NULL) from its mask.
hipError_t launch_decode_finish(const DecPlan& pl, bool fused, int nhot, int d, int F, const uint32_t* mask,
                                int32_t* idx, int32_t* count, float* y, char* ws, hipStream_t s);

// ---- launchers (return hipError_t of the launch) ---------------------------------------------------
hipError_t launch_predict(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x, int B,
                          float theta, float* logits, uint32_t* mask, int32_t* idx, int32_t* count,
                          char* ws, hipStream_t s);

// 1 < B <= 32: stage 1 and stage 2 with threshold and mask words (no neuron tables); umask
// (optional, ceil(F/32) words): the OR of the B tokens' masks
// yprev (optional): the previous union pass's deferred down shares -- ynks shares of 32 rows of d
// floats at ypart -- are summed into yprev [yB, d] by this pass's predictor (its share-summing
// kernel, or a kernel of its own where stage 1 has no shares)
hipError_t launch_predict_batch(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x,
                                int B, float theta, float* logits, uint32_t* mask, char* ws,
                                hipStream_t s, uint32_t* umask = nullptr,
                                uint32_t* tokbits = nullptr, const float* ypart = nullptr,
                                int ynks = 0, int yB = 0, float* yprev = nullptr);

// part / y (batch-1 decode executor only): also sum the previous step's P partial rows of d
// floats into y (reduce_partials)
hipError_t launch_pred_stage1(const pi_pred_desc& p, const PredPlan& pl, const uint16_t* x, int B,
                              float* z, hipStream_t s, const float* part = nullptr,
                              float* y = nullptr, int P = 0);

// stage 2 of one token from the z that stage 1 left at pl.off_z: logits, mask, table
hipError_t launch_pred_stage2_b1(const pi_pred_desc& p, const PredPlan& pl, float theta, float* logits,
                                 uint32_t* mask, int32_t* idx, int32_t* count, char* ws, hipStream_t s);
// y = the fixed-order sum of P partial rows of d floats (reduce_partials)
hipError_t launch_reduce_rows(const float* part, int P, int d, float* y, hipStream_t s);

hipError_t launch_compact(const uint32_t* mask, int B, int F, int mode, int32_t* idx,
                          int32_t* count, hipStream_t s);

// B == 1 sparse (idx/count) or dense (dense_F > 0: neuron k is row k, count = dense_F)
hipError_t launch_ffn_b1(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x,
                         const int32_t* idx, const int32_t* count, int dense_F, float* y,
                         char* ws, hipStream_t s);

// the two batch-1 operators on their own (one kernel each)
hipError_t launch_up_b1(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x,
                        const int32_t* idx, const int32_t* count, int dense_F, float* h,
                        hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// group > 0 (fp16 weights): idx lists groups of `group` consecutive rows and h is indexed by row
hipError_t launch_down_b1(const pi_ffn_desc& f, const FfnPlan& pl, const int32_t* idx,
                          const int32_t* count, int dense_F, const float* h, float* y, char* ws,
                          hipStream_t s, int group = 0);

// 1 < B <= 32 union-mask path on MFMA.  With umask == nullptr the union list idx[0 .. *count)
// is read; otherwise the list is built from the union mask umask and written to idx / count,
// and tokbits[F] (per neuron, bit b: in token b's mask) stands in for the token masks.
// defer_part (optional, with pl.u_ks > 1): the down shares' partials go there (pl.u_ks shares
// of 32 rows of d floats) and y is left to a later reduce_share_rows (launch_union_yred or the
// next pass's predictor) instead of the down kernel's last blocks.
hipError_t launch_ffn_union(const pi_ffn_desc& f, const FfnPlan& pl, const uint16_t* x, int B,
                            const uint32_t* umask, const uint32_t* tokbits, int32_t* idx,
                            int32_t* count, const uint32_t* token_mask, float* y, char* ws,
                            hipStream_t s, float* defer_part = nullptr);
hipError_t launch_union_yred(const float* part, int nks, int B, int d, float* y, hipStream_t s);

// ---- attention side ----------------------------------------------------------------------
struct AttnPlan {
    int nslices;              // 512-column slices of the output projection
    size_t off_part;          // pi_attn_out's partial rows: H x d floats
    size_t bytes;
};
AttnPlan plan_attn(int d, int H, int dh);
// the executor's step for H <= 64: head predictor stage 2 folded into the q/k/v kernel (z from
// launch_pred_stage1); writes mask, heads, count (and logits when not null) as pi_predict does
hipError_t launch_attn_pqkv(const pi_attn_desc& a, const pi_pred_desc& p, const uint16_t* x,
                            const float* z, float theta, float* logits, uint32_t* mask,
                            int32_t* heads, int32_t* count, float* qkv, hipStream_t s);
// the executor's output projection: H partial rows of d floats at part (rows of entries past
// the count are zeros), summed into y by the next step's stage 1 or launch_reduce_rows
hipError_t launch_attn_out_rows(const pi_attn_desc& a, const AttnPlan& pl, const float* o,
                                const int32_t* heads, const int32_t* count, float* part, hipStream_t s);
hipError_t launch_attn_qkv(const pi_attn_desc& a, const uint16_t* x, const uint32_t* hmask,
                           float* qkv, hipStream_t s);
hipError_t launch_attn_out(const pi_attn_desc& a, const AttnPlan& pl, const float* o,
                           const int32_t* heads, const int32_t* count, float* y, char* ws,
                           hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_permute_rows(const void* src, void* dst, const int32_t* perm, int n,
                               size_t row_bytes, hipStream_t s);
hipError_t launch_count_active(const uint32_t* mask, int B, int F, int32_t* counts, hipStream_t s);
hipError_t launch_map_ids(const int32_t* idx, const int32_t* count, int B, int F,
                          const int32_t* perm, int32_t* out, hipStream_t s);

}  // namespace pi
