"""The ABI's validation of the int8 group-128 predictor format (no HIP call: validation runs
before any launch and never dereferences the fake addresses)."""
import pytest

from activation_sparse_pi_amd import _lib as L

A = 0x7F0000000000


def pred8(**kw):
    a = dict(w_p1=A, w_p2=A + 0x100000, bias=A + 0x200000, d=1024, r=128, F=4096, threshold=0.5,
             pfmt=L.PI_P_I8G128, s_p1=A + 0x300000, s_p2=A + 0x400000)
    a.update(kw)
    return L.PredDesc(a["w_p1"], a["w_p2"], a["bias"], a["d"], a["r"], a["F"], a["threshold"],
                      a["pfmt"], a["s_p1"], a["s_p2"])


WS, WSB = A + 0x10000000, 1 << 30


@pytest.mark.parametrize("kw,B,code", [
    (dict(), 2, L.PI_ERR_UNSUPPORTED),               # int8 predictor: batch 1 only
    (dict(pfmt=2), 1, L.PI_ERR_DTYPE),
    (dict(s_p1=None), 1, L.PI_ERR_NULL),
    (dict(s_p2=None), 1, L.PI_ERR_NULL),
    (dict(d=1032), 1, L.PI_ERR_SHAPE),
    (dict(r=136), 1, L.PI_ERR_SHAPE),
    (dict(s_p2=A + 0x400001), 1, L.PI_ERR_ALIGN),
])
def test_predict_int8_validation(kw, B, code):
    st = L.pi_predict(pred8(**kw), A + 0x3000000, B, None, A + 0x4000000, None, None, WS, WSB, None)
    assert st == code, L.pi_last_error()
