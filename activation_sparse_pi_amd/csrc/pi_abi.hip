// C ABI of the predictor-gated sparse FFN: host-side validation, workspace
// planning and launches.  Every check runs before the first HIP call, so an
// invalid request enqueues nothing and leaves the outputs untouched.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

using namespace pi;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return PI_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_pred(const pi_pred_desc* p) {
    if (!p) return fail(PI_ERR_NULL, "pred descriptor is NULL");
    if (!p->w_p1t || !p->w_p2t || !p->bias) return fail(PI_ERR_NULL, "pred weights/bias NULL");
    if (p->d <= 0 || p->r <= 0 || p->F <= 0)
        return fail(PI_ERR_SHAPE, "pred sizes must be positive (d=%d r=%d F=%d)", p->d, p->r, p->F);
    if (p->d % 8 || p->r % 8 || p->F % 8)
        return fail(PI_ERR_SHAPE, "pred sizes need d, r, F %% 8 == 0 (d=%d r=%d F=%d)", p->d, p->r, p->F);
    if (p->r > 16384) return fail(PI_ERR_UNSUPPORTED, "predictor rank %d > 16384", p->r);
    if (!aligned16(p->w_p1t) || !aligned16(p->w_p2t))
        return fail(PI_ERR_ALIGN, "predictor weights must be 16-byte aligned");
    if (!(p->threshold > 0.f && p->threshold < 1.f))
        return fail(PI_ERR_SHAPE, "threshold must be a probability in (0,1), got %g", (double)p->threshold);
    if (p->pfmt != PI_P_F16 && p->pfmt != PI_P_I8G128)
        return fail(PI_ERR_DTYPE, "unknown predictor format %d", p->pfmt);
    if (p->pfmt == PI_P_I8G128) {
        if (!p->s_p1t || !p->s_p2t) return fail(PI_ERR_NULL, "int8 predictor needs s_p1t / s_p2t");
        if (p->d % 128 || p->r % 128)
            return fail(PI_ERR_SHAPE, "int8 predictor needs d, r %% 128 == 0 (d=%d r=%d)", p->d, p->r);
        if ((reinterpret_cast<uintptr_t>(p->s_p1t) | reinterpret_cast<uintptr_t>(p->s_p2t)) & 1u)
            return fail(PI_ERR_ALIGN, "predictor scales must be 2-byte aligned");
    }
    return PI_OK;
}

int check_ffn(const pi_ffn_desc* f, int B) {
    if (!f) return fail(PI_ERR_NULL, "ffn descriptor is NULL");
    if (f->act != PI_ACT_RELU && f->act != PI_ACT_REGLU)
        return fail(PI_ERR_DTYPE, "unknown activation %d", f->act);
    if (f->wfmt != PI_W_F16 && f->wfmt != PI_W_I4G128)
        return fail(PI_ERR_DTYPE, "unknown weight format %d", f->wfmt);
    if (!f->w_up || !f->w_down) return fail(PI_ERR_NULL, "w_up / w_down NULL");
    if (f->act == PI_ACT_REGLU && !f->w_gate) return fail(PI_ERR_NULL, "ReGLU needs w_gate");
    if (f->wfmt == PI_W_I4G128) {
        if (!f->s_up || !f->s_down) return fail(PI_ERR_NULL, "int4 needs s_up / s_down");
        if (f->act == PI_ACT_REGLU && !f->s_gate) return fail(PI_ERR_NULL, "int4 ReGLU needs s_gate");
    }
    if (f->d <= 0 || f->F <= 0) return fail(PI_ERR_SHAPE, "ffn sizes must be positive (d=%d F=%d)", f->d, f->F);
    if (f->wfmt == PI_W_F16 && f->d % 8) return fail(PI_ERR_SHAPE, "fp16 needs d %% 8 == 0 (d=%d)", f->d);
    if (f->wfmt == PI_W_I4G128 && f->d % 128) return fail(PI_ERR_SHAPE, "int4 needs d %% 128 == 0 (d=%d)", f->d);
    if (f->F % 8) return fail(PI_ERR_SHAPE, "ffn needs F %% 8 == 0 (F=%d)", f->F);
    if (f->wfmt == PI_W_F16 && f->d > PI_MAX_D_F16)
        return fail(PI_ERR_UNSUPPORTED, "fp16 d=%d > %d", f->d, PI_MAX_D_F16);
    if (f->wfmt == PI_W_I4G128 && f->d > PI_MAX_D_I4)
        return fail(PI_ERR_UNSUPPORTED, "int4 d=%d > %d", f->d, PI_MAX_D_I4);
    const void* ptrs[6] = {f->w_gate, f->w_up, f->w_down, f->s_gate, f->s_up, f->s_down};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return fail(PI_ERR_ALIGN, "ffn weights must be 16-byte aligned");
    if (B > 1 && f->wfmt != PI_W_F16)
        return fail(PI_ERR_UNSUPPORTED, "batch > 1 union path is fp16 only");
    if (f->nhot < 0 || f->nhot > f->F || f->nhot > 8 * ((f->F + 63) / 64))
        return fail(PI_ERR_SHAPE, "nhot=%d outside 0..min(F, 8 ceil(F/64)) (F=%d)", f->nhot, f->F);
    return PI_OK;
}

int check_batch(int B) {
    if (B < 1 || B > PI_MAX_BATCH) return fail(PI_ERR_SHAPE, "batch %d outside 1..%d", B, PI_MAX_BATCH);
    return PI_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
    if (!ws) return fail(PI_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(PI_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (have < need) return fail(PI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return PI_OK;
}

size_t ffn_bytes(const pi_ffn_desc& f, int B) {
    FfnPlan p = plan_ffn(f.d, f.F, f.wfmt, B);
    return p.bytes;
}

// The region every call shares (each plan starts its own layout at COUNTER_BYTES; the calls run
// one after another on a stream), for batches of 1 .. B_max tokens.  0 on invalid descriptors.
size_t ws_base(const pi_pred_desc* pred, const pi_ffn_desc* ffn, int B_max) {
    size_t need = COUNTER_BYTES;
    if (pred) {
        if (check_pred(pred) != PI_OK) return 0;
        for (int B = 1; B <= B_max; ++B) {
            const size_t b = plan_pred(pred->d, pred->r, pred->F, B).bytes;
            if (b > need) need = b;
        }
    }
    if (ffn) {
        if (check_ffn(ffn, 1) != PI_OK) return 0;
        for (int B = 1; B <= B_max; ++B) {
            const size_t b = ffn_bytes(*ffn, B);
            if (b > need) need = b;
        }
    }
    if (pred && ffn && pred->d == ffn->d && pred->F == ffn->F) {
        const size_t b = plan_decode(pred->d, pred->r, pred->F, ffn->wfmt).bytes;
        if (b > need) need = b;
    }
    return need;
}

// pi_batch_run's union path keeps the batch's union mask, token words, list and count past the shared region
// (they live from the predictor's launch to the union FFN's, which uses that region)
struct BatchWs {
    size_t off_umask, off_tokbits, off_uidx, off_ucount, off_ypart, bytes;
    int yks;    // union down shares whose partials a pass leaves for the next pass to sum (0: none)
};
BatchWs batch_ws(size_t base, int F, int d) {
    BatchWs w{};
    w.off_umask = align_up(base, 256);
    w.off_tokbits = align_up(w.off_umask + (size_t)((F + 31) / 32) * 4, 256);
    w.off_uidx = align_up(w.off_tokbits + (size_t)F * 4, 256);
    w.off_ucount = align_up(w.off_uidx + (size_t)F * 4, 256);
    w.off_ypart = w.off_ucount + 256;
    const int ks = plan_ffn(d, F, PI_W_F16, 2).u_ks;
    w.yks = ks > 1 ? ks : 0;
    w.bytes = align_up(w.off_ypart + (size_t)w.yks * 32 * d * sizeof(float), 256);
    return w;
}

// The batch-size dispatch estimate (pi_batch_plan, pi_batch_run's automatic choice).  The fixed
// costs and bandwidth fractions are fitted (least squares on relative error) to pi_batch_run's
// own step times on MI355X over three layers -- d 4096 / F 11008 ReGLU, d 7168 / F 28672 ReLU,
// d 8192 / F 32768 ReLU, fp16, B = 1 .. 64, predictor included: a token through the batch-1
// kernel schedule costs ~9 us plus its rows and predictor at ~69% of peak; a union pass ~52 us
// (five dependent kernels) plus the union's rows and one predictor pass at ~84%.  The fit is
// within 17% of every measured step and picks the faster schedule at every point but one, where
// the two differ by 1%.  B > 32 runs as union passes of at most 32 tokens.
constexpr double BATCH_TOK_FIXED_US = 9.0, BATCH_TOK_EFF = 0.69;
constexpr double BATCH_UNION_FIXED_US = 51.8, BATCH_UNION_EFF = 0.845;

int batch_groups(int B) { return (B + PI_MAX_BATCH - 1) / PI_MAX_BATCH; }
// size of group g of B tokens split into batch_groups(B) near-equal groups
int group_size(int B, int g) {
    const int G = batch_groups(B);
    return B / G + (g < B % G ? 1 : 0);
}

int batch_plan_impl(const pi_ffn_desc* ffn, int B, const float* rate, double hbm_gbs,
                    pi_batch_plan_t* plan) {
    int st;
    if ((st = check_ffn(ffn, 1)) != PI_OK) return st;
    if (!rate || !plan) return fail(PI_ERR_NULL, "rate / plan NULL");
    if (B < 1 || B > PI_MAX_BATCH_RUN) return fail(PI_ERR_SHAPE, "batch %d outside 1..%d", B, PI_MAX_BATCH_RUN);
    if (!(hbm_gbs > 0.0)) return fail(PI_ERR_SHAPE, "hbm_gbs must be positive, got %g", hbm_gbs);
    const int G = batch_groups(B);
    double n = 0.0, ug[2] = {0.0, 0.0};
    const int b0 = group_size(B, 0), b1 = G > 1 ? group_size(B, 1) : 0;
    for (int i = 0; i < ffn->F; ++i) {
        const double p = rate[i];
        if (!(p >= 0.0 && p <= 1.0)) return fail(PI_ERR_SHAPE, "rate[%d] = %g outside [0, 1]", i, p);
        n += p;
        ug[0] += 1.0 - std::pow(1.0 - p, (double)b0);
        if (G > 1) ug[1] += 1.0 - std::pow(1.0 - p, (double)b1);
    }
    const int m = ffn->act == PI_ACT_REGLU ? 3 : 2;
    const double w = ffn->wfmt == PI_W_F16 ? 2.0 : 0.5 + 2.0 / 128.0;
    const double row = (double)m * ffn->d * w;                    // bytes per listed neuron
    const double bw = hbm_gbs * 1e3;                               // bytes per us
    plan->n_mean = n;
    plan->u_mean = G > 1 ? (ug[0] + ug[1]) * 0.5 : ug[0];
    plan->t_tokens_us = B * (BATCH_TOK_FIXED_US + n * row / (BATCH_TOK_EFF * bw));
    const bool union_ok = B > 1 && ffn->wfmt == PI_W_F16;
    double tu = 0.0;
    for (int g = 0; g < G; ++g)
        tu += BATCH_UNION_FIXED_US + ug[g == 0 ? 0 : 1] * row / (BATCH_UNION_EFF * bw);
    plan->t_union_us = union_ok ? tu : HUGE_VAL;
    plan->choice = plan->t_union_us < plan->t_tokens_us ? PI_BATCH_UNION : PI_BATCH_TOKENS;
    return ok();
}

// ---- scratch of pi_decode_run_noalloc -------------------------------------------------------
// The one entry point that allocates nothing keeps its scratch (z, h, the partial rows) in this
// file-scope device array: PI_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held until
// the process ends.  In host code `scratch` only names the array; its device address on the
// current GPU comes from hipGetSymbolAddress, looked up once per device (with that device
// current) and kept in g_scratch_ptr, and only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[PI_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<char*> g_scratch_ptr;    // indexed by device ordinal

hipError_t scratch_ptr(char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// pi_decode_run and pi_decode_run_noalloc.  Every check, the workspace size included, runs
// before the first HIP call.  noalloc: ws / ws_bytes are ignored and the scratch array above is
// used (kernel schedules only).
int decode_run_impl(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep, const uint16_t* x,
                    int T, long long s0, int nsteps, int mode, uint32_t* mask, int32_t* idx,
                    int32_t* count, float* y, void* const* events, void* const* kernel_events,
                    void* ws, size_t ws_bytes, void* stream, bool noalloc);

}  // namespace

extern "C" {

const char* pi_status_string(int status) {
    switch (status) {
        case PI_OK: return "ok";
        case PI_ERR_NULL: return "null pointer";
        case PI_ERR_SHAPE: return "bad shape";
        case PI_ERR_ALIGN: return "misaligned pointer";
        case PI_ERR_DTYPE: return "bad enum";
        case PI_ERR_UNSUPPORTED: return "unsupported";
        case PI_ERR_WORKSPACE: return "bad workspace";
        case PI_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* pi_last_error(void) { return g_last_error.c_str(); }

int pi_version(void) { return 100; }

size_t pi_workspace_bytes(const pi_pred_desc* pred, const pi_ffn_desc* ffn, int B_max) {
    if (B_max < 1 || B_max > PI_MAX_BATCH) return 0;
    const size_t base = ws_base(pred, ffn, B_max);
    if (base == 0) return 0;
    // with both descriptors and B_max > 1: also pi_batch_run's union mask, list and count
    if (pred && ffn && B_max > 1 && pred->F == ffn->F) return batch_ws(base, ffn->F, ffn->d).bytes;
    return base;
}

int pi_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return fail(PI_ERR_NULL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(PI_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes == 0) return ok();
    hipError_t e = launch_zero(ws, ws_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "workspace zero fill");
    return ok();
}

int pi_predict(const pi_pred_desc* pred, const uint16_t* x, int B, float* logits, uint32_t* mask,
               int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
    int st;
    if ((st = check_pred(pred)) != PI_OK) return st;
    if ((st = check_batch(B)) != PI_OK) return st;
    if (!x || !mask) return fail(PI_ERR_NULL, "x and mask are required");
    if ((idx == nullptr) != (count == nullptr)) return fail(PI_ERR_NULL, "idx and count go together");
    if (!aligned16(x)) return fail(PI_ERR_ALIGN, "x must be 16-byte aligned");
    if (pred->pfmt == PI_P_I8G128 && B > 1)
        return fail(PI_ERR_UNSUPPORTED, "the int8 predictor runs at batch 1 (B=%d)", B);
    if (B > 1 && (size_t)pred->r * pred->d * 2 > (size_t)INT_MAX)
        return fail(PI_ERR_UNSUPPORTED, "the batch predictor needs r * d * 2 < 2^31 bytes (r=%d d=%d)",
                    pred->r, pred->d);
    const PredPlan pl = plan_pred(pred->d, pred->r, pred->F, B);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != PI_OK) return st;
    const double tau = pred->threshold;
    const float theta = (float)std::log(tau / (1.0 - tau));
    hipError_t e = launch_predict(*pred, pl, x, B, theta, logits, mask, idx, count,
                                  static_cast<char*>(ws), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_predict launch");
    return ok();
}

int pi_compact(const uint32_t* mask, int B, int F, int mode, int32_t* idx, int32_t* count,
               void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    int st;
    if (!mask || !idx || !count) return fail(PI_ERR_NULL, "mask, idx and count are required");
    if ((st = check_batch(B)) != PI_OK) return st;
    if (F <= 0) return fail(PI_ERR_SHAPE, "F must be positive (F=%d)", F);
    if (mode != PI_PER_TOKEN && mode != PI_UNION) return fail(PI_ERR_DTYPE, "unknown compaction mode %d", mode);
    hipError_t e = launch_compact(mask, B, F, mode, idx, count, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_compact launch");
    return ok();
}

int pi_sparse_ffn(const pi_ffn_desc* ffn, const uint16_t* x, int B, const int32_t* idx,
                  const int32_t* count, const uint32_t* token_mask, float* y, void* ws,
                  size_t ws_bytes, void* stream) {
    int st;
    if ((st = check_batch(B)) != PI_OK) return st;
    if (!x || !idx || !count || !y) return fail(PI_ERR_NULL, "x, idx, count and y are required");
    if (B == 1 && token_mask) return fail(PI_ERR_SHAPE, "token_mask must be NULL at batch 1");
    if (B > 1 && !token_mask) return fail(PI_ERR_NULL, "token_mask is required for batch > 1");
    if ((st = check_ffn(ffn, B)) != PI_OK) return st;
    if (!aligned16(x) || !aligned16(y)) return fail(PI_ERR_ALIGN, "x and y must be 16-byte aligned");
    const FfnPlan pl = plan_ffn(ffn->d, ffn->F, ffn->wfmt, B);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != PI_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (B == 1) {
        e = launch_ffn_b1(*ffn, pl, x, idx, count, 0, y, static_cast<char*>(ws), s);
    } else {
        // the list is only read (umask == nullptr)
        e = launch_ffn_union(*ffn, pl, x, B, nullptr, nullptr, const_cast<int32_t*>(idx),
                             const_cast<int32_t*>(count), token_mask, y, static_cast<char*>(ws), s);
    }
    if (e != hipSuccess) return hip_fail(e, "pi_sparse_ffn launch");
    return ok();
}

int pi_ffn_up(const pi_ffn_desc* ffn, const uint16_t* x, const int32_t* idx, const int32_t* count,
              float* h, void* stream) {
    int st;
    if ((st = check_ffn(ffn, 1)) != PI_OK) return st;
    if (!x || !idx || !count || !h) return fail(PI_ERR_NULL, "x, idx, count and h are required");
    if (!aligned16(x)) return fail(PI_ERR_ALIGN, "x must be 16-byte aligned");
    const FfnPlan pl = plan_ffn(ffn->d, ffn->F, ffn->wfmt, 1);
    hipError_t e = launch_up_b1(*ffn, pl, x, idx, count, 0, h, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_up launch");
    return ok();
}

int pi_ffn_down(const pi_ffn_desc* ffn, const int32_t* idx, const int32_t* count, const float* h,
                float* y, void* ws, size_t ws_bytes, void* stream) {
    int st;
    if ((st = check_ffn(ffn, 1)) != PI_OK) return st;
    if (!idx || !count || !h || !y) return fail(PI_ERR_NULL, "idx, count, h and y are required");
    if (!aligned16(y)) return fail(PI_ERR_ALIGN, "y must be 16-byte aligned");
    const FfnPlan pl = plan_ffn(ffn->d, ffn->F, ffn->wfmt, 1);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != PI_OK) return st;
    hipError_t e = launch_down_b1(*ffn, pl, idx, count, 0, h, y, static_cast<char*>(ws),
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_down launch");
    return ok();
}

}  // extern "C"

namespace {

int decode_run_impl(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep, const uint16_t* x,
                    int T, long long s0, int nsteps, int mode, uint32_t* mask, int32_t* idx,
                    int32_t* count, float* y, void* const* events, void* const* kernel_events,
                    void* ws, size_t ws_bytes, void* stream, bool noalloc) {
    int st;
    if (!preds || !ffns) return fail(PI_ERR_NULL, "descriptor arrays are required");
    if (nrep < 1) return fail(PI_ERR_SHAPE, "nrep must be >= 1 (nrep=%d)", nrep);
    if (T < 1 || nsteps < 0 || s0 < 0) return fail(PI_ERR_SHAPE, "need T >= 1, nsteps >= 0, s0 >= 0");
    if (mode != PI_RUN_AUTO && mode != PI_RUN_KERNELS && mode != PI_RUN_FUSED && mode != PI_RUN_SPLIT)
        return fail(PI_ERR_DTYPE, "unknown run mode %d", mode);
    if (!x || !mask || !y) return fail(PI_ERR_NULL, "x, mask and y are required");
    if ((idx == nullptr) != (count == nullptr)) return fail(PI_ERR_NULL, "idx and count go together");
    if (!aligned16(x) || !aligned16(y)) return fail(PI_ERR_ALIGN, "x and y must be 16-byte aligned");
    for (int i = 0; i < nrep; ++i) {
        if ((st = check_pred(&preds[i])) != PI_OK) return st;
        if ((st = check_ffn(&ffns[i], 1)) != PI_OK) return st;
        if (preds[i].d != ffns[i].d || preds[i].F != ffns[i].F || preds[i].d != preds[0].d ||
            preds[i].F != preds[0].F || preds[i].r != preds[0].r || ffns[i].act != ffns[0].act ||
            ffns[i].wfmt != ffns[0].wfmt || preds[i].threshold != preds[0].threshold ||
            preds[i].pfmt != preds[0].pfmt)
            return fail(PI_ERR_SHAPE, "replica %d does not match replica 0 / its ffn", i);
    }
    if (preds[0].F > 131072) return fail(PI_ERR_UNSUPPORTED, "pi_decode_run supports F <= 131072");
    if (events && (!events[0] || !events[1])) return fail(PI_ERR_NULL, "events must hold two events");
    if (kernel_events)
        for (int i = 0; i < 2 * nsteps; ++i)
            if (!kernel_events[i]) return fail(PI_ERR_NULL, "kernel_events[%d] is NULL", i);
    const int d = preds[0].d, r = preds[0].r, F = preds[0].F;
    const int wfmt = ffns[0].wfmt;
    // PI_RUN_AUTO and PI_RUN_KERNELS take the fused or the split kernel schedule by shape
    const DecPlan pl = plan_decode(d, r, F, wfmt);
    // a hot block runs in the split schedule (the fused one computes every neuron from the
    // predicted set, hot or not)
    const bool fused = mode == PI_RUN_FUSED || (mode != PI_RUN_SPLIT && ffns[0].nhot == 0 && pl.fused_default);
    for (int i = 0; i < nrep; ++i)
        if (ffns[i].nhot != ffns[0].nhot) return fail(PI_ERR_SHAPE, "replica %d has another hot block", i);
    if (!fused && pl.lds_b + hot_lds_bytes(ffns[0], pl.ntile) > (size_t)DEC_LDS_MAX)
        return fail(PI_ERR_UNSUPPORTED, "the hot block needs %zu bytes of LDS per tile block, more than %d",
                    pl.lds_b + hot_lds_bytes(ffns[0], pl.ntile), DEC_LDS_MAX);
    // the kernel schedules use the partial rows of the schedule they run (the workspace from
    // pi_workspace_bytes holds those of either)
    const size_t need = pl.off_part + (size_t)(fused ? pl.ntile : down_ranges(pl, ffns[0].nhot, F).P) *
                                          d * sizeof(float);
    if (noalloc) {
        if (need > (size_t)PI_NOALLOC_SCRATCH_BYTES)
            return fail(PI_ERR_WORKSPACE, "this layer's decode scratch is %zu bytes, more than the %u "
                        "bytes of the static scratch (d=%d r=%d F=%d, %s schedule)", need,
                        (unsigned)PI_NOALLOC_SCRATCH_BYTES, d, r, F, fused ? "fused" : "split");
        char* sp = nullptr;
        hipError_t e = scratch_ptr(&sp);          // the first HIP call of this path
        if (e != hipSuccess) return hip_fail(e, "static scratch address");
        ws = sp;
        ws_bytes = PI_NOALLOC_SCRATCH_BYTES;
    }
    if ((st = check_ws(ws, ws_bytes, need)) != PI_OK) return st;
    const double tau = preds[0].threshold;
    const float theta = (float)std::log(tau / (1.0 - tau));
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    hipError_t e;
    if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s)) != hipSuccess)
        return hip_fail(e, "pi_decode_run start event");
    if (nsteps > 0) {
        // every step leaves its down projection as fp32 partial rows; the next step's first
        // kernel sums them into y in a fixed order, and a small kernel does so after the last
        for (int i = 0; i < nsteps; ++i) {
            const long long g = s0 + i;
            const int t = (int)(g % T), rep = (int)(g % nrep);
            hipEvent_t k0 = kernel_events ? static_cast<hipEvent_t>(kernel_events[2 * i]) : nullptr;
            hipEvent_t k1 = kernel_events ? static_cast<hipEvent_t>(kernel_events[2 * i + 1]) : nullptr;
            e = launch_decode_step(preds[rep], ffns[rep], pl, fused, x + (size_t)t * d, theta, nullptr, mask,
                                   y, i > 0, w, s, k0, k1);
            if (e != hipSuccess) return hip_fail(e, "pi_decode_run launch");
        }
        if ((e = launch_decode_finish(pl, fused, ffns[0].nhot, d, F, mask, idx, count, y, w, s)) != hipSuccess)
            return hip_fail(e, "pi_decode_run final y");
    }
    if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[1]), s)) != hipSuccess)
        return hip_fail(e, "pi_decode_run end event");
    return ok();
}

}  // namespace

extern "C" {

int pi_decode_run(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep, const uint16_t* x,
                  int T, long long s0, int nsteps, int mode, uint32_t* mask, int32_t* idx,
                  int32_t* count, float* y, void* const* events, void* const* kernel_events,
                  void* ws, size_t ws_bytes, void* stream) {
    return decode_run_impl(preds, ffns, nrep, x, T, s0, nsteps, mode, mask, idx, count, y, events,
                           kernel_events, ws, ws_bytes, stream, false);
}

int pi_decode_run_noalloc(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep,
                          const uint16_t* x, int T, long long s0, int nsteps, int mode,
                          uint32_t* mask, int32_t* idx, int32_t* count, float* y,
                          void* const* events, void* const* kernel_events, void* stream) {
    return decode_run_impl(preds, ffns, nrep, x, T, s0, nsteps, mode, mask, idx, count, y, events,
                           kernel_events, nullptr, 0, stream, true);
}

int pi_ffn_dense_ref_gpu(const pi_ffn_desc* ffn, const uint16_t* x, int B, float* y, void* ws,
                         size_t ws_bytes, void* stream) {
    int st;
    if ((st = check_batch(B)) != PI_OK) return st;
    if ((st = check_ffn(ffn, 1)) != PI_OK) return st;
    if (!x || !y) return fail(PI_ERR_NULL, "x and y are required");
    if (!aligned16(x) || !aligned16(y)) return fail(PI_ERR_ALIGN, "x and y must be 16-byte aligned");
    const FfnPlan pl = plan_ffn(ffn->d, ffn->F, ffn->wfmt, 1);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != PI_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int b = 0; b < B; ++b) {
        hipError_t e = launch_ffn_b1(*ffn, pl, x + (size_t)b * ffn->d, nullptr, nullptr, ffn->F,
                                     y + (size_t)b * ffn->d, static_cast<char*>(ws), s);
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_dense_ref_gpu launch");
    }
    return ok();
}

int pi_place_neurons(const int32_t* counts, int F, int32_t* perm) {
    if (!counts || !perm) return fail(PI_ERR_NULL, "counts / perm NULL");
    if (F <= 0) return fail(PI_ERR_SHAPE, "F must be positive (F=%d)", F);
    for (int i = 0; i < F; ++i)
        if (counts[i] < 0) return fail(PI_ERR_SHAPE, "negative count %d at neuron %d", counts[i], i);
    // rank: descending count, ties by ascending original index
    std::vector<int32_t> order(F);
    for (int i = 0; i < F; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
    // deal the ranks over the 64-neuron tiles in serpentine order, skipping full tiles
    const int T = (F + 63) / 64;
    std::vector<int> fill(T, 0);
    auto cap = [&](int t) { return t == T - 1 ? F - 64 * (T - 1) : 64; };
    int t = 0, dir = 1;
    auto advance = [&]() {
        t += dir;
        if (t == T) { t = T - 1; dir = -1; }
        if (t < 0) { t = 0; dir = 1; }
    };
    for (int k = 0; k < F; ++k) {
        while (fill[t] == cap(t)) advance();
        perm[t * 64 + fill[t]] = order[k];
        ++fill[t];
        advance();
    }
    return ok();
}

int pi_batch_plan(const pi_ffn_desc* ffn, int B, const float* rate, double hbm_gbs,
                  pi_batch_plan_t* plan) {
    return batch_plan_impl(ffn, B, rate, hbm_gbs, plan);
}

int pi_batch_run(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep, const uint16_t* x,
                 int T, int B, long long s0, int nsteps, int schedule, const float* rate,
                 double hbm_gbs, uint32_t* mask, float* y, void* const* events,
                 void* const* kernel_events, void* ws, size_t ws_bytes, void* stream) {
    int st;
    if (!preds || !ffns) return fail(PI_ERR_NULL, "descriptor arrays are required");
    if (nrep < 1) return fail(PI_ERR_SHAPE, "nrep must be >= 1 (nrep=%d)", nrep);
    if (T < 1 || nsteps < 0 || s0 < 0) return fail(PI_ERR_SHAPE, "need T >= 1, nsteps >= 0, s0 >= 0");
    if (B < 1 || B > PI_MAX_BATCH_RUN) return fail(PI_ERR_SHAPE, "batch %d outside 1..%d", B, PI_MAX_BATCH_RUN);
    if (schedule != PI_BATCH_TOKENS && schedule != PI_BATCH_UNION && schedule != PI_BATCH_AUTO)
        return fail(PI_ERR_DTYPE, "unknown batch schedule %d", schedule);
    if (!x || !mask || !y) return fail(PI_ERR_NULL, "x, mask and y are required");
    if (!aligned16(x) || !aligned16(y)) return fail(PI_ERR_ALIGN, "x and y must be 16-byte aligned");
    for (int i = 0; i < nrep; ++i) {
        if ((st = check_pred(&preds[i])) != PI_OK) return st;
        if ((st = check_ffn(&ffns[i], 1)) != PI_OK) return st;
        if (preds[i].d != ffns[i].d || preds[i].F != ffns[i].F || preds[i].d != preds[0].d ||
            preds[i].F != preds[0].F || preds[i].r != preds[0].r || ffns[i].act != ffns[0].act ||
            ffns[i].wfmt != ffns[0].wfmt || preds[i].threshold != preds[0].threshold ||
            preds[i].pfmt != preds[0].pfmt || ffns[i].nhot != ffns[0].nhot)
            return fail(PI_ERR_SHAPE, "replica %d does not match replica 0 / its ffn", i);
    }
    if (events && (!events[0] || !events[1])) return fail(PI_ERR_NULL, "events must hold two events");
    const int d = preds[0].d, r = preds[0].r, F = preds[0].F, W = (F + 31) / 32;
    int sched = schedule;
    if (sched == PI_BATCH_AUTO) {
        if (!rate) return fail(PI_ERR_NULL, "PI_BATCH_AUTO needs the activation rates");
        pi_batch_plan_t pl{};
        if ((st = batch_plan_impl(&ffns[0], B, rate, hbm_gbs, &pl)) != PI_OK) return st;
        // the token schedule also runs the predictor once per token, the union schedule once per
        // pass: its bytes (2 d r + 2 r F, fp16) at each schedule's bandwidth fraction
        const double pb = 2.0 * d * r + 2.0 * r * F, bw = hbm_gbs * 1e3;
        const double tt = pl.t_tokens_us + B * pb / (BATCH_TOK_EFF * bw);
        const double tu = pl.t_union_us + batch_groups(B) * pb / (BATCH_UNION_EFF * bw);
        sched = tu < tt ? PI_BATCH_UNION : PI_BATCH_TOKENS;
    }
    if (sched == PI_BATCH_UNION && B == 1) sched = PI_BATCH_TOKENS;     // nothing to unite
    if (kernel_events) {
        if (sched != PI_BATCH_UNION || batch_groups(B) != 1)
            return fail(PI_ERR_SHAPE, "kernel_events need the union schedule in one pass (2 <= B <= %d)",
                        PI_MAX_BATCH);
        for (int i = 0; i < 2 * nsteps; ++i)
            if (!kernel_events[i]) return fail(PI_ERR_NULL, "kernel_events[%d] is NULL", i);
    }
    if (sched == PI_BATCH_UNION) {
        if (ffns[0].wfmt != PI_W_F16 || preds[0].pfmt != PI_P_F16)
            return fail(PI_ERR_UNSUPPORTED, "the union schedule takes fp16 weights and an fp16 predictor");
        if ((size_t)r * d * 2 > (size_t)INT_MAX)
            return fail(PI_ERR_UNSUPPORTED, "the batch predictor needs r * d * 2 < 2^31 bytes");
    }
    const int Gmax = sched == PI_BATCH_UNION ? group_size(B, 0) : 1;   // the largest group
    const size_t base = ws_base(&preds[0], &ffns[0], Gmax);
    const BatchWs bw = batch_ws(base, F, d);
    const size_t need = sched == PI_BATCH_UNION ? bw.bytes : base;
    if ((st = check_ws(ws, ws_bytes, need)) != PI_OK) return st;
    const DecPlan dpl = plan_decode(d, r, F, ffns[0].wfmt);
    const bool fused = ffns[0].nhot == 0 && dpl.fused_default;
    const double tau = preds[0].threshold;
    const float theta = (float)std::log(tau / (1.0 - tau));
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    uint32_t* umask = reinterpret_cast<uint32_t*>(w + bw.off_umask);
    uint32_t* tokbits = reinterpret_cast<uint32_t*>(w + bw.off_tokbits);
    int32_t* uidx = reinterpret_cast<int32_t*>(w + bw.off_uidx);
    int32_t* ucount = reinterpret_cast<int32_t*>(w + bw.off_ucount);
    // one union pass per step with its down projection in shares: the pass leaves the shares'
    // partials and the next pass's predictor (after the last step, a small kernel) sums them
    // into y -- bit for bit the down kernel's own sum, without its cross-block hand-off
    const bool defer = sched == PI_BATCH_UNION && batch_groups(B) == 1 && bw.yks > 0;
    float* ypart = reinterpret_cast<float*>(w + bw.off_ypart);
    hipError_t e;
    if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s)) != hipSuccess)
        return hip_fail(e, "pi_batch_run start event");
    for (int i = 0; i < nsteps; ++i) {
        const long long g = s0 + i;
        const int rep = (int)(g % nrep);
        const uint16_t* xs = x + (size_t)(g % T) * B * d;
        const pi_pred_desc& P = preds[rep];
        const pi_ffn_desc& Fd = ffns[rep];
        if (sched == PI_BATCH_TOKENS) {
            // every token through the batch-1 kernel schedule; a token's first kernel sums the
            // previous token's partial rows into that token's row of y
            for (int b = 0; b < B; ++b) {
                const bool first = i == 0 && b == 0;
                float* yprev = y + (size_t)(b == 0 ? B - 1 : b - 1) * d;
                e = launch_decode_step(P, Fd, dpl, fused, xs + (size_t)b * d, theta, nullptr,
                                       mask + (size_t)b * W, yprev, !first, w, s, nullptr, nullptr);
                if (e != hipSuccess) return hip_fail(e, "pi_batch_run token step");
            }
        } else {
            for (int gi = 0, b0 = 0; gi < batch_groups(B); b0 += group_size(B, gi), ++gi) {
                const int Bg = group_size(B, gi);
                const PredPlan ppl = plan_pred(d, r, F, Bg);
                const FfnPlan fpl = plan_ffn(d, F, Fd.wfmt, Bg);
                // the union FFN builds the union's list from the union mask itself
                const bool yprev = defer && i > 0;
                if ((e = launch_predict_batch(P, ppl, xs + (size_t)b0 * d, Bg, theta, nullptr,
                                              mask + (size_t)b0 * W, w, s, umask, tokbits,
                                              yprev ? ypart : nullptr, bw.yks, B, y)) != hipSuccess)
                    return hip_fail(e, "pi_batch_run union pass");
                if (kernel_events &&
                    (e = hipEventRecord(static_cast<hipEvent_t>(kernel_events[2 * i]), s)) != hipSuccess)
                    return hip_fail(e, "pi_batch_run kernel event");
                if ((e = launch_ffn_union(Fd, fpl, xs + (size_t)b0 * d, Bg, umask, tokbits, uidx, ucount,
                                          mask + (size_t)b0 * W, y + (size_t)b0 * d, w, s,
                                          defer ? ypart : nullptr)) != hipSuccess)
                    return hip_fail(e, "pi_batch_run union pass");
                if (kernel_events &&
                    (e = hipEventRecord(static_cast<hipEvent_t>(kernel_events[2 * i + 1]), s)) != hipSuccess)
                    return hip_fail(e, "pi_batch_run kernel event");
            }
        }
    }
    if (defer && nsteps > 0 && (e = launch_union_yred(ypart, bw.yks, B, d, y, s)) != hipSuccess)
        return hip_fail(e, "pi_batch_run final y");
    if (sched == PI_BATCH_TOKENS && nsteps > 0 &&
        (e = launch_decode_finish(dpl, fused, ffns[0].nhot, d, F, mask + (size_t)(B - 1) * W, nullptr,
                                  nullptr, y + (size_t)(B - 1) * d, w, s)) != hipSuccess)
        return hip_fail(e, "pi_batch_run final y");
    if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[1]), s)) != hipSuccess)
        return hip_fail(e, "pi_batch_run end event");
    return ok();
}

int pi_permute_rows(const void* src, void* dst, const int32_t* perm, int n, size_t row_bytes,
                    void* stream) {
    if (!src || !dst || !perm) return fail(PI_ERR_NULL, "src / dst / perm NULL");
    if (n <= 0 || row_bytes == 0) return fail(PI_ERR_SHAPE, "need n > 0 and row_bytes > 0 (n=%d)", n);
    const hipError_t e = launch_permute_rows(src, dst, perm, n, row_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "pi_permute_rows");
}

int pi_place_neurons_hot(const int32_t* counts, int F, int ntok, float hot_rate, int32_t* perm,
                         int32_t* nhot) {
    if (!counts || !perm || !nhot) return fail(PI_ERR_NULL, "counts / perm / nhot NULL");
    if (F <= 0 || ntok <= 0) return fail(PI_ERR_SHAPE, "need F > 0 and ntok > 0 (F=%d ntok=%d)", F, ntok);
    if (!(hot_rate > 0.f && hot_rate <= 1.f)) return fail(PI_ERR_SHAPE, "hot_rate %g outside (0, 1]", (double)hot_rate);
    for (int i = 0; i < F; ++i)
        if (counts[i] < 0 || counts[i] > ntok) return fail(PI_ERR_SHAPE, "count %d at neuron %d outside 0..ntok", counts[i], i);
    std::vector<int32_t> order(F);
    for (int i = 0; i < F; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
    const int T = (F + 63) / 64;
    int H = 0;
    while (H < F && H < 8 * T && (double)counts[order[H]] >= (double)hot_rate * ntok) ++H;
    for (int k = 0; k < H; ++k) perm[k] = order[k];           // the hot block, hottest first
    // the cold neurons, by descending count, dealt in serpentine order over the tiles' free
    // positions (those from H on), so every cold tile expects about the same number active
    std::vector<int> next(T), end(T);
    std::vector<int> tiles;
    for (int t = 0; t < T; ++t) {
        next[t] = std::max(64 * t, H);
        end[t] = std::min(64 * t + 64, F);
        if (next[t] < end[t]) tiles.push_back(t);
    }
    const int nt = (int)tiles.size();
    int j = 0, dir = 1;
    for (int k = H; k < F; ++k) {
        while (next[tiles[j]] == end[tiles[j]]) {
            j += dir;
            if (j == nt) { j = nt - 1; dir = -1; }
            if (j < 0) { j = 0; dir = 1; }
        }
        perm[next[tiles[j]]++] = order[k];
        j += dir;
        if (j == nt) { j = nt - 1; dir = -1; }
        if (j < 0) { j = 0; dir = 1; }
    }
    *nhot = H;
    return ok();
}

int pi_count_active(const uint32_t* mask, int B, int F, int32_t* counts, void* stream) {
    if (!mask || !counts) return fail(PI_ERR_NULL, "mask / counts NULL");
    if (F <= 0) return fail(PI_ERR_SHAPE, "F must be positive (F=%d)", F);
    if (int st = check_batch(B); st != PI_OK) return st;
    const hipError_t e = launch_count_active(mask, B, F, counts, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "pi_count_active");
}

int pi_map_ids(const int32_t* idx, const int32_t* count, int B, int F, const int32_t* perm,
               int32_t* out, void* stream) {
    if (!idx || !count || !perm || !out) return fail(PI_ERR_NULL, "idx / count / perm / out NULL");
    if (F <= 0) return fail(PI_ERR_SHAPE, "F must be positive (F=%d)", F);
    if (int st = check_batch(B); st != PI_OK) return st;
    const hipError_t e = launch_map_ids(idx, count, B, F, perm, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "pi_map_ids");
}

}  // extern "C"

namespace {

int check_attn(const pi_attn_desc* a) {
    if (!a) return fail(PI_ERR_NULL, "attention descriptor is NULL");
    if (!a->w_qkv || !a->w_o) return fail(PI_ERR_NULL, "w_qkv and w_o are required");
    if (!aligned16(a->w_qkv) || !aligned16(a->w_o)) return fail(PI_ERR_ALIGN, "attention weights must be 16-byte aligned");
    if (a->d < 8 || a->d % 8 || a->d > PI_ATTN_MAX_D)
        return fail(PI_ERR_SHAPE, "attention needs 8 <= d <= %d with d %% 8 == 0 (d=%d)", PI_ATTN_MAX_D, a->d);
    if (a->H < 1 || a->H > PI_ATTN_MAX_HEADS)
        return fail(PI_ERR_SHAPE, "attention needs 1 <= H <= %d (H=%d)", PI_ATTN_MAX_HEADS, a->H);
    if (a->dh < 1 || (long long)a->H * a->dh * 3 > INT_MAX / a->d)
        return fail(PI_ERR_SHAPE, "attention needs d_head >= 1 and 3 H d_head d < 2^31 (H=%d d_head=%d d=%d)",
                    a->H, a->dh, a->d);
    return PI_OK;
}

}  // namespace

extern "C" {

size_t pi_attn_workspace_bytes(const pi_attn_desc* a) {
    if (check_attn(a) != PI_OK) return 0;
    return plan_attn(a->d, a->H, a->dh).bytes;
}

int pi_attn_qkv(const pi_attn_desc* a, const uint16_t* x, const uint32_t* head_mask, float* qkv,
                void* stream) {
    int st;
    if ((st = check_attn(a)) != PI_OK) return st;
    if (!x || !head_mask || !qkv) return fail(PI_ERR_NULL, "x, head_mask and qkv are required");
    if (!aligned16(x)) return fail(PI_ERR_ALIGN, "x must be 16-byte aligned");
    const hipError_t e = launch_attn_qkv(*a, x, head_mask, qkv, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "pi_attn_qkv launch");
}

int pi_attn_out(const pi_attn_desc* a, const float* o, const int32_t* heads, const int32_t* count,
                float* y, void* ws, size_t ws_bytes, void* stream) {
    int st;
    if ((st = check_attn(a)) != PI_OK) return st;
    if (!o || !heads || !count || !y) return fail(PI_ERR_NULL, "o, heads, count and y are required");
    if (!aligned16(y)) return fail(PI_ERR_ALIGN, "y must be 16-byte aligned");
    const AttnPlan pl = plan_attn(a->d, a->H, a->dh);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != PI_OK) return st;
    const hipError_t e = launch_attn_out(*a, pl, o, heads, count, y, static_cast<char*>(ws),
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "pi_attn_out launch");
}

int pi_attn_run(const pi_pred_desc* preds, const pi_attn_desc* attns, int nrep, const uint16_t* x,
                const float* o, int T, long long s0, int nsteps, uint32_t* mask, int32_t* idx,
                int32_t* count, float* qkv, float* y, void* const* events,
                void* const* kernel_events, void* ws, size_t ws_bytes, void* stream) {
    int st;
    if (!preds || !attns) return fail(PI_ERR_NULL, "descriptor arrays are required");
    if (nrep < 1) return fail(PI_ERR_SHAPE, "nrep must be >= 1 (nrep=%d)", nrep);
    if (T < 1 || nsteps < 0 || s0 < 0) return fail(PI_ERR_SHAPE, "need T >= 1, nsteps >= 0, s0 >= 0");
    if (!x || !o || !mask || !idx || !count || !qkv || !y)
        return fail(PI_ERR_NULL, "x, o, mask, idx, count, qkv and y are required");
    if (!aligned16(x) || !aligned16(y)) return fail(PI_ERR_ALIGN, "x and y must be 16-byte aligned");
    for (int i = 0; i < nrep; ++i) {
        if ((st = check_pred(&preds[i])) != PI_OK) return st;
        if ((st = check_attn(&attns[i])) != PI_OK) return st;
        if (preds[i].pfmt != PI_P_F16) return fail(PI_ERR_UNSUPPORTED, "the head predictor takes fp16 factors");
        if (preds[i].F != attns[i].H || preds[i].d != attns[i].d)
            return fail(PI_ERR_SHAPE, "replica %d: the head predictor needs F = H and the same d", i);
        if (preds[i].d != preds[0].d || preds[i].r != preds[0].r || attns[i].H != attns[0].H ||
            attns[i].dh != attns[0].dh || preds[i].threshold != preds[0].threshold)
            return fail(PI_ERR_SHAPE, "replica %d does not match replica 0", i);
    }
    if (events && (!events[0] || !events[1])) return fail(PI_ERR_NULL, "events must hold two events");
    if (kernel_events)
        for (int i = 0; i < 2 * nsteps; ++i)
            if (!kernel_events[i]) return fail(PI_ERR_NULL, "kernel_events[%d] is NULL", i);
    const int d = attns[0].d, H = attns[0].H, dh = attns[0].dh;
    const PredPlan ppl = plan_pred(d, preds[0].r, H, 1);
    const AttnPlan apl = plan_attn(d, H, dh);
    // the output projection's partial rows sit past the predictor's area (the next step's stage 1
    // reads them while it writes z)
    const size_t off_rows = align_up(ppl.bytes, 256);
    const int P = H;                             // one partial row per head-table entry
    if ((st = check_ws(ws, ws_bytes, off_rows + (size_t)P * d * sizeof(float))) != PI_OK) return st;
    const double tau = preds[0].threshold;
    const float theta = (float)std::log(tau / (1.0 - tau));
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    hipError_t e;
    if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s)) != hipSuccess)
        return hip_fail(e, "pi_attn_run start event");
    float* rows = reinterpret_cast<float*>(w + off_rows);
    for (int i = 0; i < nsteps; ++i) {
        const long long g = s0 + i;
        const int rep = (int)(g % nrep), t = (int)(g % T);
        const uint16_t* xs = x + (size_t)t * d;
        const float* os = o + (size_t)t * H * dh;
        // stage 1 (which also sums the previous step's partial rows into y); with H <= 64 one
        // kernel then takes the heads' logits, mask, table and q/k/v, else stage 2 runs first
        const bool fold = H <= 64;
        if ((e = launch_pred_stage1(preds[rep], ppl, xs, 1, reinterpret_cast<float*>(w + ppl.off_z), s,
                                    i > 0 ? rows : nullptr, y, P)) != hipSuccess ||
            (!fold && (e = launch_pred_stage2_b1(preds[rep], ppl, theta, nullptr, mask, idx, count, w, s)) != hipSuccess))
            return hip_fail(e, "pi_attn_run head predictor");
        if (kernel_events && (e = hipEventRecord(static_cast<hipEvent_t>(kernel_events[2 * i]), s)) != hipSuccess)
            return hip_fail(e, "pi_attn_run kernel event");
        if ((e = fold ? launch_attn_pqkv(attns[rep], preds[rep], xs, reinterpret_cast<const float*>(w + ppl.off_z),
                                         theta, nullptr, mask, idx, count, qkv, s)
                      : launch_attn_qkv(attns[rep], xs, mask, qkv, s)) != hipSuccess)
            return hip_fail(e, "pi_attn_run q/k/v");
        if (kernel_events && (e = hipEventRecord(static_cast<hipEvent_t>(kernel_events[2 * i + 1]), s)) != hipSuccess)
            return hip_fail(e, "pi_attn_run kernel event");
        if ((e = launch_attn_out_rows(attns[rep], apl, os, idx, count, rows, s)) != hipSuccess)
            return hip_fail(e, "pi_attn_run output projection");
    }
    if (nsteps > 0 && (e = launch_reduce_rows(rows, P, d, y, s)) != hipSuccess)
        return hip_fail(e, "pi_attn_run final y");
    if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[1]), s)) != hipSuccess)
        return hip_fail(e, "pi_attn_run end event");
    return ok();
}

}  // extern "C"
