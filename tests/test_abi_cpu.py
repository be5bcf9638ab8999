"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from activation_sparse_pi_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi.h")

# fake, 256-byte aligned "device" addresses: validation never dereferences them
A = 0x7F0000000000


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(pi_[a-z_]+)\s*\(", src)))


def test_header_declarations_match_exports():
    declared = _declared()
    assert set(declared) == set(L.EXPORTS), declared


def test_library_exports_every_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in _declared():
        assert name in syms, name
        getattr(L.lib(), name)


def pred(**kw):
    a = dict(w_p1=A, w_p2=A + 0x100000, bias=A + 0x200000, d=1024, r=128, F=4096, threshold=0.5)
    a.update(kw)
    return L.PredDesc(a["w_p1"], a["w_p2"], a["bias"], a["d"], a["r"], a["F"], a["threshold"])


def ffn(**kw):
    a = dict(w_gate=None, w_up=A, w_down=A + 0x1000000, s_gate=None, s_up=None, s_down=None,
             d=1024, F=4096, act=L.PI_ACT_RELU, wfmt=L.PI_W_F16, nhot=0)
    a.update(kw)
    return L.FfnDesc(a["w_gate"], a["w_up"], a["w_down"], a["s_gate"], a["s_up"], a["s_down"],
                     a["d"], a["F"], a["act"], a["wfmt"], a["nhot"])


def test_status_strings_and_version():
    assert L.pi_status_string(0) == "ok"
    assert L.pi_status_string(L.PI_ERR_WORKSPACE) == "bad workspace"
    assert L.pi_status_string(99) == "unknown status"
    assert L.pi_version() >= 100


def test_workspace_bytes():
    n = L.pi_workspace_bytes(pred(), ffn(), 1)
    assert n > 0 and n % 256 == 0
    # batch > 1 adds the union path's H fragments (2 KB per 32 neurons) and partial sums
    assert L.pi_workspace_bytes(None, ffn(), 32) >= L.pi_workspace_bytes(None, ffn(), 1) + 32 * 4096 * 2
    assert L.pi_workspace_bytes(pred(), ffn(), 32) >= n
    assert L.pi_workspace_bytes(pred(), ffn(), 0) == 0
    assert L.pi_workspace_bytes(pred(d=1001), None, 1) == 0
    assert L.pi_workspace_bytes(None, ffn(act=7), 1) == 0


WS = A + 0x10000000
WSB = 1 << 30


@pytest.mark.parametrize("kw,code", [
    (dict(desc=None), L.PI_ERR_NULL),
    (dict(desc=pred(w_p1=None)), L.PI_ERR_NULL),
    (dict(desc=pred(d=0)), L.PI_ERR_SHAPE),
    (dict(desc=pred(r=12)), L.PI_ERR_SHAPE),
    (dict(desc=pred(F=1001)), L.PI_ERR_SHAPE),
    (dict(desc=pred(w_p2=A + 8)), L.PI_ERR_ALIGN),
    (dict(desc=pred(threshold=1.0)), L.PI_ERR_SHAPE),
    (dict(desc=pred(threshold=0.0)), L.PI_ERR_SHAPE),
    (dict(B=0), L.PI_ERR_SHAPE),
    (dict(B=33), L.PI_ERR_SHAPE),
    (dict(x=None), L.PI_ERR_NULL),
    (dict(mask=None), L.PI_ERR_NULL),
    (dict(x=A + 2), L.PI_ERR_ALIGN),
    (dict(idx=None), L.PI_ERR_NULL),
    (dict(ws=None), L.PI_ERR_WORKSPACE),
    (dict(ws=WS + 16), L.PI_ERR_WORKSPACE),
    (dict(wsb=1024), L.PI_ERR_WORKSPACE),
    # batch predictor: r * d * 2 must stay below 2^31 bytes
    (dict(desc=pred(d=131072, r=8192), B=2), L.PI_ERR_UNSUPPORTED),
])
def test_predict_validation(kw, code):
    a = dict(desc=pred(), x=A + 0x3000000, B=1, logits=None, mask=A + 0x4000000,
             idx=A + 0x5000000, count=A + 0x6000000, ws=WS, wsb=WSB)
    a.update(kw)
    st = L.pi_predict(a["desc"], a["x"], a["B"], a["logits"], a["mask"], a["idx"], a["count"],
                      a["ws"], a["wsb"], None)
    assert st == code, L.pi_last_error()
    assert L.pi_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(desc=None), L.PI_ERR_NULL),
    (dict(desc=ffn(act=3)), L.PI_ERR_DTYPE),
    (dict(desc=ffn(wfmt=5)), L.PI_ERR_DTYPE),
    (dict(desc=ffn(act=L.PI_ACT_REGLU)), L.PI_ERR_NULL),
    (dict(desc=ffn(wfmt=L.PI_W_I4G128)), L.PI_ERR_NULL),
    (dict(desc=ffn(wfmt=L.PI_W_I4G128, s_up=A, s_down=A, d=1000)), L.PI_ERR_SHAPE),
    (dict(desc=ffn(d=1020)), L.PI_ERR_SHAPE),
    (dict(desc=ffn(F=4095)), L.PI_ERR_SHAPE),
    (dict(desc=ffn(d=8200)), L.PI_ERR_UNSUPPORTED),
    (dict(desc=ffn(w_down=A + 4)), L.PI_ERR_ALIGN),
    (dict(desc=ffn(nhot=-1)), L.PI_ERR_SHAPE),
    (dict(desc=ffn(nhot=4097)), L.PI_ERR_SHAPE),
    (dict(B=2, token_mask=None), L.PI_ERR_NULL),
    (dict(B=2, token_mask=A, desc=ffn(wfmt=L.PI_W_I4G128, s_up=A, s_down=A)), L.PI_ERR_UNSUPPORTED),
    (dict(B=32, token_mask=A, wsb="batch1"), L.PI_ERR_WORKSPACE),
    (dict(token_mask=A), L.PI_ERR_SHAPE),
    (dict(idx=None), L.PI_ERR_NULL),
    (dict(count=None), L.PI_ERR_NULL),
    (dict(y=A + 8), L.PI_ERR_ALIGN),
    (dict(ws=None), L.PI_ERR_WORKSPACE),
    (dict(wsb=256), L.PI_ERR_WORKSPACE),
])
def test_sparse_ffn_validation(kw, code):
    a = dict(desc=ffn(), x=A + 0x3000000, B=1, idx=A + 0x5000000, count=A + 0x6000000,
             token_mask=None, y=A + 0x7000000, ws=WS, wsb=WSB)
    a.update(kw)
    if a["wsb"] == "batch1":     # sized for batch 1 only (evaluated here, not at collection)
        a["wsb"] = L.pi_workspace_bytes(None, ffn(), 1)
    st = L.pi_sparse_ffn(a["desc"], a["x"], a["B"], a["idx"], a["count"], a["token_mask"], a["y"],
                         a["ws"], a["wsb"], None)
    assert st == code, L.pi_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), L.PI_ERR_NULL),
    (dict(B=0), L.PI_ERR_SHAPE),
    (dict(F=0), L.PI_ERR_SHAPE),
    (dict(mode=9), L.PI_ERR_DTYPE),
    (dict(count=None), L.PI_ERR_NULL),
])
def test_compact_validation(kw, code):
    a = dict(mask=A, B=1, F=4096, mode=L.PI_PER_TOKEN, idx=A + 0x100000, count=A + 0x200000)
    a.update(kw)
    st = L.pi_compact(a["mask"], a["B"], a["F"], a["mode"], a["idx"], a["count"], None, 0, None)
    assert st == code, L.pi_last_error()


def test_dense_ref_validation():
    st = L.pi_ffn_dense_ref_gpu(ffn(), A, 1, A + 0x100, None, 0, None)
    assert st == L.PI_ERR_WORKSPACE
    st = L.pi_ffn_dense_ref_gpu(ffn(F=0), A, 1, A + 0x100, WS, WSB, None)
    assert st == L.PI_ERR_SHAPE


def test_workspace_init_validation():
    assert L.pi_workspace_init(None, 1024, None) == L.PI_ERR_NULL
    assert L.pi_workspace_init(A + 64, 1024, None) == L.PI_ERR_WORKSPACE


def _run_noalloc(p, f, mode):
    preds = (L.PredDesc * 1)(p)
    ffns = (L.FfnDesc * 1)(f)
    return L.pi_decode_run_noalloc(preds, ffns, 1, A + 0x3000000, 4, 0, 2, mode, A + 0x4000000,
                                   A + 0x5000000, A + 0x6000000, A + 0x7000000, None, None, None)


def test_decode_run_noalloc_validation():
    """The static-scratch decode entry point rejects, before any HIP call, a layer whose scratch
    exceeds PI_NOALLOC_SCRATCH_BYTES (here a fused step of 2048 tiles x 8192 columns of partial
    rows: 64 MiB), besides pi_decode_run's own argument checks (mode 1 is not assigned)."""
    big_p, big_f = pred(d=8192, r=512, F=131072), ffn(d=8192, F=131072)
    assert _run_noalloc(big_p, big_f, L.PI_RUN_FUSED) == L.PI_ERR_WORKSPACE, L.pi_last_error()
    assert "static scratch" in L.pi_last_error()
    assert _run_noalloc(pred(), ffn(), 1) == L.PI_ERR_DTYPE
    assert _run_noalloc(pred(d=1001), ffn(), L.PI_RUN_KERNELS) == L.PI_ERR_SHAPE
    assert _run_noalloc(pred(), ffn(), 17) == L.PI_ERR_DTYPE



def _batch_run(p, f, B=4, schedule=L.PI_BATCH_UNION, ws=WS, wsb=WSB, rate=None, **kw):
    preds = (L.PredDesc * 1)(p)
    ffns = (L.FfnDesc * 1)(f)
    a = dict(x=A + 0x3000000, mask=A + 0x4000000, y=A + 0x7000000)
    a.update(kw)
    return L.pi_batch_run(preds, ffns, 1, a["x"], 4, B, 0, 2, schedule, rate, 8000.0, a["mask"],
                          a["y"], None, a.get("kev"), ws, wsb, None)


def test_batch_run_validation():
    """pi_batch_run rejects bad arguments before any HIP call: batch range, schedule enum,
    missing rates for the automatic choice, int4 weights on the union schedule, alignment and
    the workspace."""
    import numpy as np
    assert _batch_run(pred(), ffn(), B=0) == L.PI_ERR_SHAPE
    assert _batch_run(pred(), ffn(), B=65) == L.PI_ERR_SHAPE
    assert _batch_run(pred(), ffn(), schedule=9) == L.PI_ERR_DTYPE
    assert _batch_run(pred(), ffn(), schedule=L.PI_BATCH_AUTO) == L.PI_ERR_NULL
    i4 = ffn(wfmt=L.PI_W_I4G128, s_up=A, s_down=A)
    assert _batch_run(pred(), i4, schedule=L.PI_BATCH_UNION) == L.PI_ERR_UNSUPPORTED
    assert _batch_run(pred(), ffn(), x=A + 2) == L.PI_ERR_ALIGN
    assert _batch_run(pred(), ffn(), mask=None) == L.PI_ERR_NULL
    assert _batch_run(pred(), ffn(), ws=None) == L.PI_ERR_WORKSPACE
    need = L.pi_workspace_bytes(pred(), ffn(), 32)
    assert need > L.pi_workspace_bytes(pred(), None, 32)
    assert _batch_run(pred(), ffn(), B=64, wsb=need - 256) == L.PI_ERR_WORKSPACE
    rate = np.full(4096, 0.1, np.float32)
    assert _batch_run(pred(), ffn(), schedule=L.PI_BATCH_AUTO, rate=rate.ctypes.data, ws=None) == \
        L.PI_ERR_WORKSPACE
    import ctypes
    kev = (ctypes.c_void_p * 4)(A, A, A, A)
    assert _batch_run(pred(), ffn(), B=40, kev=kev) == L.PI_ERR_SHAPE                  # two passes
    assert _batch_run(pred(), ffn(), schedule=L.PI_BATCH_TOKENS, kev=kev) == L.PI_ERR_SHAPE
    assert _batch_run(pred(), ffn(), kev=(ctypes.c_void_p * 4)(A, None, A, A)) == L.PI_ERR_NULL


def attn(**kw):
    a = dict(w_qkv=A, w_o=A + 0x1000000, d=4096, H=32, dh=128)
    a.update(kw)
    return L.AttnDesc(a["w_qkv"], a["w_o"], a["d"], a["H"], a["dh"])


def test_attn_workspace_bytes():
    n = L.pi_attn_workspace_bytes(attn())
    # the arrival counters and one partial row of d floats per head-table entry
    assert n > 32 * 4096 * 4 and n % 256 == 0
    assert L.pi_attn_workspace_bytes(attn(H=8, dh=24, d=200)) > 0
    for bad in (dict(d=12), dict(d=0), dict(d=L.PI_ATTN_MAX_D + 8), dict(H=0),
                dict(H=L.PI_ATTN_MAX_HEADS + 1), dict(dh=0), dict(w_qkv=None), dict(w_o=A + 8)):
        assert L.pi_attn_workspace_bytes(attn(**bad)) == 0, bad


@pytest.mark.parametrize("kw,code", [
    (dict(desc=None), L.PI_ERR_NULL),
    (dict(x=None), L.PI_ERR_NULL),
    (dict(mask=None), L.PI_ERR_NULL),
    (dict(qkv=None), L.PI_ERR_NULL),
    (dict(x=A + 8), L.PI_ERR_ALIGN),
    (dict(desc=attn(w_qkv=A + 4)), L.PI_ERR_ALIGN),
    (dict(desc=attn(d=100)), L.PI_ERR_SHAPE),
    (dict(desc=attn(H=2000)), L.PI_ERR_SHAPE),
    (dict(desc=attn(dh=0)), L.PI_ERR_SHAPE),
    (dict(desc=attn(d=16384, H=1024, dh=1024)), L.PI_ERR_SHAPE),
])
def test_attn_qkv_validation(kw, code):
    a = dict(desc=attn(), x=A, mask=A + 0x100, qkv=A + 0x200)
    a.update(kw)
    assert L.pi_attn_qkv(a["desc"], a["x"], a["mask"], a["qkv"], None) == code, L.pi_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), L.PI_ERR_NULL),
    (dict(heads=None), L.PI_ERR_NULL),
    (dict(count=None), L.PI_ERR_NULL),
    (dict(y=None), L.PI_ERR_NULL),
    (dict(y=A + 4), L.PI_ERR_ALIGN),
    (dict(ws=None), L.PI_ERR_WORKSPACE),
    (dict(ws=A + 64), L.PI_ERR_WORKSPACE),
    (dict(ws_bytes=1024), L.PI_ERR_WORKSPACE),
    (dict(desc=attn(d=4100)), L.PI_ERR_SHAPE),
])
def test_attn_out_validation(kw, code):
    d = attn()
    a = dict(desc=d, o=A, heads=A + 0x100, count=A + 0x180, y=A + 0x200, ws=A + 0x10000,
             ws_bytes=L.pi_attn_workspace_bytes(d))
    a.update(kw)
    assert L.pi_attn_out(a["desc"], a["o"], a["heads"], a["count"], a["y"], a["ws"], a["ws_bytes"],
                         None) == code, L.pi_last_error()


def test_attn_run_validation():
    import ctypes
    d = attn(d=4096, H=32, dh=128)
    p = L.PredDesc(A + 0x3000000, A + 0x4000000, A + 0x5000000, 4096, 128, 32, 0.5)
    preds, attns = (L.PredDesc * 1)(p), (L.AttnDesc * 1)(d)
    ws_need = L.pi_workspace_bytes(p, None, 1) + L.pi_attn_workspace_bytes(d)
    base = dict(preds=preds, attns=attns, nrep=1, x=A, o=A + 0x10000, T=4, s0=0, n=2, mask=A + 0x20000,
                idx=A + 0x20100, count=A + 0x20200, qkv=A + 0x30000, y=A + 0x40000, ev=None, kev=None,
                ws=A + 0x100000, ws_bytes=ws_need)

    def call(**kw):
        a = dict(base, **kw)
        return L.pi_attn_run(a["preds"], a["attns"], a["nrep"], a["x"], a["o"], a["T"], a["s0"], a["n"],
                             a["mask"], a["idx"], a["count"], a["qkv"], a["y"], a["ev"], a["kev"],
                             a["ws"], a["ws_bytes"], None)
    assert call(preds=None) == L.PI_ERR_NULL
    assert call(nrep=0) == L.PI_ERR_SHAPE
    assert call(T=0) == L.PI_ERR_SHAPE
    assert call(o=None) == L.PI_ERR_NULL
    assert call(x=A + 8) == L.PI_ERR_ALIGN
    # the predictor's area alone leaves no room for the output projection's partial rows
    assert call(ws_bytes=L.pi_workspace_bytes(p, None, 1)) == L.PI_ERR_WORKSPACE
    bad = L.PredDesc(A + 0x3000000, A + 0x4000000, A + 0x5000000, 4096, 128, 40, 0.5)   # F != H
    assert call(preds=(L.PredDesc * 1)(bad)) == L.PI_ERR_SHAPE, L.pi_last_error()
    i8 = L.PredDesc(A + 0x3000000, A + 0x4000000, A + 0x5000000, 4096, 128, 32, 0.5, L.PI_P_I8G128,
                    A + 0x6000000, A + 0x7000000)
    assert call(preds=(L.PredDesc * 1)(i8)) == L.PI_ERR_UNSUPPORTED, L.pi_last_error()
    assert call(ev=(ctypes.c_void_p * 2)(None, None)) == L.PI_ERR_NULL
    assert call(kev=(ctypes.c_void_p * 4)(A, A, None, A)) == L.PI_ERR_NULL
