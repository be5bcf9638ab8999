"""ctypes binding of libpi.so (the C ABI declared in include/pi.h).

Argument marshalling only: every function forwards integers (device
addresses, sizes, the hipStream_t handle) to the library and returns its
status code.  Nothing here computes any part of the sparse FFN, and there is
no fallback: if libpi.so is missing or fails to load, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpi.so")

PI_OK, PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_ALIGN, PI_ERR_DTYPE = 0, 1, 2, 3, 4
PI_ERR_UNSUPPORTED, PI_ERR_WORKSPACE, PI_ERR_HIP = 5, 6, 7
PI_ACT_RELU, PI_ACT_REGLU = 0, 1
PI_W_F16, PI_W_I4G128 = 0, 1
PI_P_F16, PI_P_I8G128 = 0, 1
PI_PER_TOKEN, PI_UNION = 0, 1
PI_RUN_AUTO, PI_RUN_KERNELS, PI_RUN_FUSED, PI_RUN_SPLIT = 0, 2, 3, 4
PI_MAX_BATCH = 32
PI_BATCH_TOKENS, PI_BATCH_UNION, PI_BATCH_AUTO = 0, 1, 2
PI_MAX_BATCH_RUN = 64

EXPORTS = ("pi_status_string", "pi_last_error", "pi_version", "pi_workspace_bytes",
           "pi_workspace_init", "pi_predict", "pi_compact", "pi_sparse_ffn",
           "pi_ffn_up", "pi_ffn_down", "pi_decode_run", "pi_ffn_dense_ref_gpu",
           "pi_place_neurons", "pi_permute_rows", "pi_map_ids", "pi_batch_plan",
           "pi_count_active", "pi_decode_run_noalloc", "pi_place_neurons_hot", "pi_batch_run",
           "pi_attn_workspace_bytes", "pi_attn_qkv", "pi_attn_out", "pi_attn_run")
PI_ATTN_MAX_HEADS, PI_ATTN_MAX_D = 1024, 16384
PI_NOALLOC_SCRATCH_BYTES = 4 << 20


class PredDesc(ctypes.Structure):
    _fields_ = [("w_p1t", c_void_p), ("w_p2t", c_void_p), ("bias", c_void_p),
                ("d", c_int32), ("r", c_int32), ("F", c_int32), ("threshold", c_float),
                ("pfmt", c_int32), ("s_p1t", c_void_p), ("s_p2t", c_void_p)]


class FfnDesc(ctypes.Structure):
    _fields_ = [("w_gate", c_void_p), ("w_up", c_void_p), ("w_down", c_void_p),
                ("s_gate", c_void_p), ("s_up", c_void_p), ("s_down", c_void_p),
                ("d", c_int32), ("F", c_int32), ("act", c_int32), ("wfmt", c_int32),
                ("nhot", c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("d", c_int32), ("H", c_int32),
                ("dh", c_int32)]


class BatchPlan(ctypes.Structure):
    _fields_ = [("n_mean", ctypes.c_double), ("u_mean", ctypes.c_double),
                ("t_tokens_us", ctypes.c_double), ("t_union_us", ctypes.c_double),
                ("choice", c_int32)]


class PiError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"[{status}] {detail}")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libpi.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        try:
            # torch ships its own HIP runtime (file libamdhip64.so, soname libamdhip64.so.7);
            # loading it first lets libpi.so's libamdhip64.so.7 bind to that same copy, so
            # the process holds one HIP runtime whatever the import order
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.pi_status_string.argtypes, L.pi_status_string.restype = [c_int], ctypes.c_char_p
        L.pi_last_error.argtypes, L.pi_last_error.restype = [], ctypes.c_char_p
        L.pi_version.argtypes, L.pi_version.restype = [], c_int
        L.pi_workspace_bytes.argtypes = [P(PredDesc), P(FfnDesc), c_int]
        L.pi_workspace_bytes.restype = c_size_t
        L.pi_workspace_init.argtypes, L.pi_workspace_init.restype = [c_void_p, c_size_t, c_void_p], c_int
        L.pi_predict.argtypes = [P(PredDesc), c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_size_t, c_void_p]
        L.pi_predict.restype = c_int
        L.pi_compact.argtypes = [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                 c_size_t, c_void_p]
        L.pi_compact.restype = c_int
        L.pi_sparse_ffn.argtypes = [P(FfnDesc), c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]
        L.pi_sparse_ffn.restype = c_int
        L.pi_ffn_up.argtypes = [P(FfnDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.pi_ffn_up.restype = c_int
        L.pi_ffn_down.argtypes = [P(FfnDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_size_t, c_void_p]
        L.pi_ffn_down.restype = c_int
        L.pi_decode_run.argtypes = [P(PredDesc), P(FfnDesc), c_int, c_void_p, c_int,
                                    ctypes.c_longlong, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.pi_decode_run.restype = c_int
        L.pi_ffn_dense_ref_gpu.argtypes = [P(FfnDesc), c_void_p, c_int, c_void_p, c_void_p,
                                           c_size_t, c_void_p]
        L.pi_ffn_dense_ref_gpu.restype = c_int
        L.pi_place_neurons.argtypes = [c_void_p, c_int, c_void_p]
        L.pi_place_neurons.restype = c_int
        L.pi_permute_rows.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_size_t, c_void_p]
        L.pi_permute_rows.restype = c_int
        L.pi_map_ids.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]
        L.pi_map_ids.restype = c_int
        L.pi_decode_run_noalloc.argtypes = [P(PredDesc), P(FfnDesc), c_int, c_void_p, c_int,
                                            ctypes.c_longlong, c_int, c_int, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.pi_decode_run_noalloc.restype = c_int
        L.pi_place_neurons_hot.argtypes = [c_void_p, c_int, c_int, c_float, c_void_p, c_void_p]
        L.pi_place_neurons_hot.restype = c_int
        L.pi_batch_run.argtypes = [P(PredDesc), P(FfnDesc), c_int, c_void_p, c_int, c_int,
                                   ctypes.c_longlong, c_int, c_int, c_void_p, ctypes.c_double,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.pi_batch_run.restype = c_int
        L.pi_count_active.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p]
        L.pi_count_active.restype = c_int
        L.pi_batch_plan.argtypes = [ctypes.POINTER(FfnDesc), c_int, c_void_p, ctypes.c_double,
                                    ctypes.POINTER(BatchPlan)]
        L.pi_batch_plan.restype = c_int
        L.pi_attn_workspace_bytes.argtypes = [P(AttnDesc)]
        L.pi_attn_workspace_bytes.restype = c_size_t
        L.pi_attn_qkv.argtypes = [P(AttnDesc), c_void_p, c_void_p, c_void_p, c_void_p]
        L.pi_attn_qkv.restype = c_int
        L.pi_attn_out.argtypes = [P(AttnDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_size_t, c_void_p]
        L.pi_attn_out.restype = c_int
        L.pi_attn_run.argtypes = [P(PredDesc), P(AttnDesc), c_int, c_void_p, c_void_p, c_int,
                                  ctypes.c_longlong, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.pi_attn_run.restype = c_int
        _LIB = L
    return _LIB


def _p(desc):
    return None if desc is None else ctypes.byref(desc)


def pi_status_string(status: int) -> str:
    return lib().pi_status_string(status).decode()


def pi_last_error() -> str:
    return lib().pi_last_error().decode()


def pi_version() -> int:
    return lib().pi_version()


def pi_workspace_bytes(pred, ffn, B_max: int) -> int:
    return lib().pi_workspace_bytes(_p(pred), _p(ffn), B_max)


def pi_workspace_init(ws: int, ws_bytes: int, stream: int) -> int:
    return lib().pi_workspace_init(ws, ws_bytes, stream)


def pi_predict(pred, x, B, logits, mask, idx, count, ws, ws_bytes, stream) -> int:
    return lib().pi_predict(_p(pred), x, B, logits, mask, idx, count, ws, ws_bytes, stream)


def pi_compact(mask, B, F, mode, idx, count, ws, ws_bytes, stream) -> int:
    return lib().pi_compact(mask, B, F, mode, idx, count, ws, ws_bytes, stream)


def pi_sparse_ffn(ffn, x, B, idx, count, token_mask, y, ws, ws_bytes, stream) -> int:
    return lib().pi_sparse_ffn(_p(ffn), x, B, idx, count, token_mask, y, ws, ws_bytes, stream)


def pi_ffn_up(ffn, x, idx, count, h, stream) -> int:
    return lib().pi_ffn_up(_p(ffn), x, idx, count, h, stream)


def pi_ffn_down(ffn, idx, count, h, y, ws, ws_bytes, stream) -> int:
    return lib().pi_ffn_down(_p(ffn), idx, count, h, y, ws, ws_bytes, stream)


def pi_decode_run(preds, ffns, nrep, x, T, s0, nsteps, mode, mask, idx, count, y, events,
                  kernel_events, ws, ws_bytes, stream) -> int:
    """preds / ffns: ctypes arrays of PredDesc / FfnDesc; events: ctypes array of two
    hipEvent_t handles (c_void_p) or None; kernel_events: ctypes array of 2*nsteps
    handles or None."""
    return lib().pi_decode_run(preds, ffns, nrep, x, T, s0, nsteps, mode, mask, idx, count, y,
                               events, kernel_events, ws, ws_bytes, stream)


def pi_ffn_dense_ref_gpu(ffn, x, B, y, ws, ws_bytes, stream) -> int:
    return lib().pi_ffn_dense_ref_gpu(_p(ffn), x, B, y, ws, ws_bytes, stream)


def check(status: int) -> None:
    """Raise PiError with the library's message for a non-zero status."""
    if status != PI_OK:
        raise PiError(status, f"{pi_status_string(status)}: {pi_last_error()}")


def pi_place_neurons(counts: int, F: int, perm: int) -> int:
    """counts and perm are host addresses (int32 [F]), e.g. ndarray.ctypes.data."""
    return lib().pi_place_neurons(counts, F, perm)


def pi_batch_plan(desc, B: int, rate: int, hbm_gbs: float, plan) -> int:
    """rate is a host address (float32 [F]); plan a BatchPlan, filled on success."""
    return lib().pi_batch_plan(_p(desc), B, rate, hbm_gbs, _p(plan))


def pi_permute_rows(src, dst, perm, n, row_bytes, stream) -> int:
    return lib().pi_permute_rows(src, dst, perm, n, row_bytes, stream)


def pi_map_ids(idx, count, B, F, perm, out, stream) -> int:
    return lib().pi_map_ids(idx, count, B, F, perm, out, stream)


def pi_count_active(mask, B, F, counts, stream) -> int:
    return lib().pi_count_active(mask, B, F, counts, stream)


def pi_decode_run_noalloc(preds, ffns, nrep, x, T, s0, nsteps, mode, mask, idx, count, y, events,
                          kernel_events, stream) -> int:
    """pi_decode_run without a workspace (the library's static scratch); arguments as there."""
    return lib().pi_decode_run_noalloc(preds, ffns, nrep, x, T, s0, nsteps, mode, mask, idx, count,
                                       y, events, kernel_events, stream)


def pi_place_neurons_hot(counts: int, F: int, ntok: int, hot_rate: float, perm: int, nhot) -> int:
    """counts / perm host addresses (int32 [F]); nhot a ctypes.c_int32, set on success."""
    return lib().pi_place_neurons_hot(counts, F, ntok, hot_rate, perm, ctypes.byref(nhot))


def pi_batch_run(preds, ffns, nrep, x, T, B, s0, nsteps, schedule, rate, hbm_gbs, mask, y, events,
                 kernel_events, ws, ws_bytes, stream) -> int:
    """preds / ffns: ctypes arrays; rate: host address (float32 [F]) or None; events: ctypes array
    of two hipEvent_t handles or None; kernel_events: ctypes array of 2 nsteps handles or None."""
    return lib().pi_batch_run(preds, ffns, nrep, x, T, B, s0, nsteps, schedule, rate, hbm_gbs, mask,
                              y, events, kernel_events, ws, ws_bytes, stream)


def pi_attn_workspace_bytes(a) -> int:
    return lib().pi_attn_workspace_bytes(_p(a))


def pi_attn_qkv(a, x, head_mask, qkv, stream) -> int:
    return lib().pi_attn_qkv(_p(a), x, head_mask, qkv, stream)


def pi_attn_out(a, o, heads, count, y, ws, ws_bytes, stream) -> int:
    return lib().pi_attn_out(_p(a), o, heads, count, y, ws, ws_bytes, stream)


def pi_attn_run(preds, attns, nrep, x, o, T, s0, nsteps, mask, idx, count, qkv, y, events,
                kernel_events, ws, ws_bytes, stream) -> int:
    return lib().pi_attn_run(preds, attns, nrep, x, o, T, s0, nsteps, mask, idx, count, qkv, y, events,
                             kernel_events, ws, ws_bytes, stream)
