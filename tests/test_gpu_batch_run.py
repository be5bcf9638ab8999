"""pi_batch_run, the native small-batch executor, against the oracle (needs an MI355X).

Every token of a step keeps its own predicted neurons whatever the schedule: its mask is checked
against the oracle's index set (outside the exclusion band) and its y against the oracle's FFN
over that token's own list.  Union passes of more than 32 tokens split into near-equal groups
(33 = 17 + 16, 64 = 32 + 32).  A run of several steps ends bit-identical to a one-step run of
its last step.  The automatic schedule follows the estimate it documents.
"""
import sys

import numpy as np
import pytest

from synth import configs, gen

from . import _parity as P
import oracle.pi_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _L():
    from activation_sparse_pi_amd import _lib as L
    return L


def _layer(inputs, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inputs, **kw)


def _run(layer, cfg, xd, B, s0, n, schedule, rate=None):
    W = (cfg.F + 31) // 32
    mask = torch.full((B, W), -1, dtype=torch.int32, device="cuda")
    y = torch.full((B, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    layer.batch_run(xd.data_ptr(), cfg.T, B, s0, n, mask.data_ptr(), y.data_ptr(), schedule=schedule,
                    rate=rate)
    torch.cuda.synchronize()
    return mask.cpu().numpy().view(np.uint32), y.cpu().numpy().astype(np.float64)


def _check_step(inp, W, X, mask, y, ctx):
    """Every token of one step against the oracle: index set and y over its own list."""
    cfg = inp["cfg"]
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    worst = 0.0
    for b in range(X.shape[0]):
        act = O.words_to_active(mask[b], cfg.F)
        idx = np.flatnonzero(act)
        P.check_index_set(idx, mask[b], ref_L[b], cfg.F, ctx=f"{ctx} b={b}")
        worst = max(worst, P.check_ffn(y[b], W, X[b], idx, ctx=f"{ctx} b={b}"))
    return worst


CASES = [
    (configs.tiny("relu", "f16", d=384, F=1000, r=40, B=64, T=3, seed=71), [2, 7, 33, 64]),
    (configs.tiny("reglu", "f16", d=1032, F=2000, r=48, B=40, T=2, seed=72), [5, 40]),
]


@pytest.mark.parametrize("sched", ["union", "tokens"])
@pytest.mark.parametrize("cfg,Bs", CASES, ids=lambda c: c.name if hasattr(c, "name") else "")
def test_batch_run_tiny(cfg, Bs, sched):
    L = _L()
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=2, B_max=32)
    s = {"union": L.PI_BATCH_UNION, "tokens": L.PI_BATCH_TOKENS}[sched]
    for B in Bs:
        say(f"[gpu] batch_run {sched} {cfg.name} B={B}")
        Xall = np.ascontiguousarray(inp["x"][:, :B, :])               # [T, B, d]
        xd = torch.from_numpy(Xall).cuda()
        for t in range(cfg.T):
            mask, y = _run(layer, cfg, xd, B, t, 1, s)
            worst = _check_step(inp, W, Xall[t], mask, y, f"{cfg.name} {sched} B={B} t={t}")
        say(f"  worst rel-L2 {worst:.2e}")
        m1, y1 = _run(layer, cfg, xd, B, 1, 5, s)        # steps 1..5, ends on token set 5 % T
        m2, y2 = _run(layer, cfg, xd, B, 5, 1, s)
        assert np.array_equal(m1, m2) and np.array_equal(y1, y2), f"{sched} B={B}: long run"


def test_batch_run_int4_tokens_and_auto():
    """int4 weights run the token schedule; the automatic choice takes it too (no union path)."""
    L = _L()
    cfg = configs.tiny("reglu", "i4g128", d=384, F=1000, r=40, B=6, T=2, seed=73)
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=1, B_max=32)
    xd = torch.from_numpy(np.ascontiguousarray(inp["x"])).cuda()
    rate = np.full(cfg.F, 0.2, np.float32)
    for s in (L.PI_BATCH_TOKENS, L.PI_BATCH_AUTO):
        mask, y = _run(layer, cfg, xd, cfg.B, 0, 1, s, rate=rate)
        _check_step(inp, W, inp["x"][0], mask, y, f"int4 sched={s}")
    with pytest.raises(L.PiError) as e:
        _run(layer, cfg, xd, cfg.B, 0, 1, L.PI_BATCH_UNION)
    assert e.value.status == L.PI_ERR_UNSUPPORTED


@pytest.mark.parametrize("B", [32, 64])
def test_batch_run_c4_shape(B):
    """The Falcon-40B-shaped batch layer: B = 32 (one union pass) and 64 (two), every token's set
    and y against the oracle on one step; the automatic choice is the union schedule here (the
    token schedule would read the 42 MB predictor once per token)."""
    L = _L()
    cfg = configs.C4.with_(B=B, T=2)
    say(f"[gpu] batch_run c4 shape B={B}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=1, B_max=32)
    xd = torch.from_numpy(np.ascontiguousarray(inp["x"])).cuda()
    mask, y = _run(layer, cfg, xd, B, 1, 1, L.PI_BATCH_AUTO, rate=inp["rates"].astype(np.float32))
    worst = _check_step(inp, W, inp["x"][1], mask, y, f"c4 B={B}")
    mu, yu = _run(layer, cfg, xd, B, 1, 1, L.PI_BATCH_UNION)
    assert np.array_equal(mu, mask) and np.array_equal(yu, y), "AUTO must have taken the union schedule"
    if B <= L.PI_MAX_BATCH:
        # events around each step's union FFN change nothing in the results and all complete
        W = (cfg.F + 31) // 32
        mk = torch.full((B, W), -1, dtype=torch.int32, device="cuda")
        yk = torch.full((B, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        kev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        layer.batch_run(xd.data_ptr(), cfg.T, B, 0, 2, mk.data_ptr(), yk.data_ptr(),
                        schedule=L.PI_BATCH_UNION, kernel_events=kev)
        torch.cuda.synchronize()
        assert np.array_equal(mk.cpu().numpy().view(np.uint32), mask) and \
            np.array_equal(yk.cpu().numpy().astype(np.float64), y), "kernel events changed the results"
        assert all(kev[2 * i].elapsed_time(kev[2 * i + 1]) > 0 for i in range(2))
    say(f"  worst rel-L2 {worst:.2e}")


@pytest.mark.parametrize("sched", ["union", "tokens"])
def test_batch_run_empty_union(sched):
    """A step where no token has an active neuron (x = 0 and every bias below the threshold):
    masks and y are all zero, also right after a step with a non-empty union on the same
    workspace, and the next non-empty step is unaffected."""
    L = _L()
    cfg = configs.tiny("relu", "f16", d=384, F=1000, r=40, B=8, T=2, seed=74)
    inp = gen.make(cfg)
    inp["bias"] = np.minimum(inp["bias"], np.float32(-1e-3))      # x = 0 gives l = bias < 0
    W = O.Weights.from_inputs(inp)
    assert not np.any(O.predicted_active(inp["bias"])), "x = 0 must predict no neuron"
    layer = _layer(inp, replicas=1, B_max=8)
    s = {"union": L.PI_BATCH_UNION, "tokens": L.PI_BATCH_TOKENS}[sched]
    X = np.ascontiguousarray(inp["x"][:1])                           # [1, B, d]
    xd = torch.from_numpy(X).cuda()
    zd = torch.zeros_like(xd)
    m1, y1 = _run(layer, cfg, xd, cfg.B, 0, 1, s)
    _check_step(inp, W, X[0], m1, y1, f"empty-union {sched}: before")
    assert m1.any(), "the regular step should have active neurons"
    m0, y0 = _run(layer, cfg, zd, cfg.B, 0, 1, s)
    assert not m0.any(), f"{sched}: masks of x = 0 must be empty"
    assert np.array_equal(y0, np.zeros_like(y0)), f"{sched}: y of an empty union must be 0"
    m2, y2 = _run(layer, cfg, xd, cfg.B, 0, 1, s)
    assert np.array_equal(m1, m2) and np.array_equal(y1, y2), f"{sched}: step after the empty one"
