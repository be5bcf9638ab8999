"""The decode schedules' y against the oracle outside the workloads' value range (needs an MI355X).

pi_decode_run's kernel schedules store each block's down-projection column sums as fp32 partial
rows and sum the rows in a fixed order, so y carries relative fp32 rounding at any scale and
non-finite values propagate as in any fp32 sum.  Checked here, through the C ABI:

* x scaled by 2^-12 and by 2^8 (ReGLU y then scales by 2^-24 and 2^16): index sets and y
  against the oracle on the same scaled fp16 x, in both the fused and the split schedule;
* an Inf planted in one predicted-active neuron's up row (fp16 layers): the predictor is
  untouched, and y's NaN / +Inf / -Inf pattern equals the oracle's exactly.
"""
import sys

import numpy as np
import pytest

from synth import configs, gen

from . import _parity as P
import oracle.pi_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    configs.tiny("reglu", "f16", d=1032, F=2000, r=48, T=3, seed=21),
    configs.tiny("relu", "f16", d=384, F=1000, r=40, T=3, seed=22),
    configs.tiny("reglu", "i4g128", d=2176, F=2000, r=48, T=3, seed=23),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _modes():
    from activation_sparse_pi_amd import _lib as L
    return {"fused": L.PI_RUN_FUSED, "split": L.PI_RUN_SPLIT}


def _layer(inputs, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inputs, **kw)


def _one_step(layer, xs, t, mode):
    bufs = layer.buffers(1)
    layer.decode_run(xs.data_ptr(), xs.shape[0], t, 1, bufs, mode=mode)
    torch.cuda.synchronize()
    n = int(bufs["count"][0].item())
    return (bufs["idx"][0, :n].cpu().numpy().astype(np.int64),
            bufs["mask"][0].cpu().numpy().view(np.uint32), bufs["y"][0].cpu().numpy().copy())


@pytest.mark.parametrize("scale_log2", [-12, 8])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_scaled_x(cfg, scale_log2):
    say(f"[gpu] y contract: {cfg.name}, x * 2^{scale_log2}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    X = (inp["x"][:, 0, :].astype(np.float32) * np.float32(2.0 ** scale_log2)).astype(np.float16)
    assert np.all(np.isfinite(X))
    layer = _layer(inp, replicas=1)
    xs = torch.from_numpy(X.copy()).to(layer.device)
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    for mname, m in _modes().items():
        for t in range(cfg.T):
            idx, mask, y = _one_step(layer, xs, t, m)
            ctx = f"{cfg.name} x*2^{scale_log2} {mname} t={t}"
            P.check_index_set(idx, mask, ref_L[t], cfg.F, ctx=ctx)
            ref = O.ffn_neurons(W, X[t], idx)
            e = P.rel_l2(y, ref)
            say(f"  {ctx}: n={idx.size} |y_ref|={np.linalg.norm(ref):.3e} rel-L2={e:.2e}")
            assert e <= P.REL_TOL, f"{ctx}: rel-L2 {e:.3e}"


@pytest.mark.parametrize("cfg", [c for c in CASES if c.wfmt == "f16"], ids=lambda c: c.name)
def test_nonfinite_weight_propagates(cfg):
    say(f"[gpu] y contract: {cfg.name}, Inf in an active neuron's up row")
    inp = gen.make(cfg)
    X = inp["x"][:, 0, :]
    t = 0
    lg = O.predictor_logits(X[t], inp["w_p1"], inp["w_p2"], inp["bias"])
    act = O.compact(O.predicted_active(lg) & ~O.exclusion_band(lg))
    assert act.size > 0
    i0 = int(act[act.size // 2])
    c0 = int(np.flatnonzero(X[t] != 0)[0])
    w_up = inp["w_up"].copy()
    w_up[i0, c0] = np.float16(np.inf if X[t][c0] > 0 else -np.inf)     # a_i0 = +Inf
    bad = dict(inp, w_up=w_up)
    W = O.Weights.from_inputs(bad)
    layer = _layer(bad, replicas=1)
    xs = torch.from_numpy(X.copy()).to(layer.device)
    for mname, m in _modes().items():
        idx, mask, y = _one_step(layer, xs, t, m)
        ctx = f"{cfg.name} Inf weight {mname}"
        P.check_index_set(idx, mask, lg, cfg.F, ctx=ctx)
        assert i0 in set(idx.tolist()), f"{ctx}: the planted neuron is not listed"
        with np.errstate(invalid="ignore", over="ignore"):
            ref = O.ffn_neurons(W, X[t], idx)
        assert not np.all(np.isfinite(ref)), "the planted Inf should reach the oracle's y"
        for name, f in (("NaN", np.isnan), ("+Inf", np.isposinf), ("-Inf", np.isneginf)):
            assert np.array_equal(f(y), f(ref)), f"{ctx}: {name} pattern differs"
        fin = np.isfinite(ref)
        if fin.any():
            assert P.rel_l2(y[fin], ref[fin]) <= P.REL_TOL, f"{ctx}: finite columns"
        say(f"  {ctx}: {int(np.isnan(y).sum())} NaN, {int(np.isinf(y).sum())} Inf of {y.size}")
