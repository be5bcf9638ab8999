"""Small-batch (1 < B <= 32) path vs the CPU oracle, through the C ABI (needs an MI355X).

Per step: pi_predict(B) gives every token's mask and neuron table, pi_compact(UNION)
their union, pi_sparse_ffn(B) the union FFN on MFMA in which token b only receives the
neurons of its own mask.  Each token's y is compared with the oracle's FFN over that
token's own GPU list (rel-L2 <= 1e-3: h is rounded to fp16 on this path, a relative
error of at most 2^-11 per neuron).
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


def _np(t):
    return t.detach().cpu().numpy()


def _layer(inputs, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inputs, **kw)


def _dev_list(layer, idx):
    n = len(idx)
    t = torch.zeros(max(1, layer.F), dtype=torch.int32, device=layer.device)
    if n:
        t[:n] = torch.from_numpy(np.asarray(idx, np.int32)).to(layer.device)
    return t, torch.tensor([n], dtype=torch.int32, device=layer.device)


def _dev_masks(layer, active):
    return torch.from_numpy(O.mask_words(active).view(np.int32)).to(layer.device)


def run_batch(layer, xb, B, bufs):
    """One batch step; returns per-token logits, masks, lists, the union and y."""
    layer.batch_step(xb.data_ptr(), B, bufs)
    torch.cuda.synchronize()
    cnt = _np(bufs["count"][:B])
    un = int(_np(bufs["ucount"])[0])
    return dict(logits=_np(bufs["logits"][:B]), mask=_np(bufs["mask"][:B]).view(np.uint32),
                idx=[_np(bufs["idx"][b, :cnt[b]]).astype(np.int64) for b in range(B)],
                uidx=_np(bufs["uidx"][:un]).astype(np.int64), y=_np(bufs["y"][:B]).copy())


def check_batch(g, inp, W, X, F, ctx, ffn_tokens=None):
    B = X.shape[0]
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    assert np.max(np.abs(g["logits"] - ref_L)) < 5e-5, ctx
    act = np.zeros((B, F), bool)
    for b in range(B):
        P.check_index_set(g["idx"][b], g["mask"][b], ref_L[b], F, ctx=f"{ctx} b={b}")
        act[b, g["idx"][b]] = True
    # the union list is exactly the OR of the GPU's own token masks
    assert np.array_equal(g["uidx"], O.compact(O.union_active(act))), f"{ctx}: union list"
    worst = 0.0
    for b in (range(B) if ffn_tokens is None else ffn_tokens):
        worst = max(worst, P.check_ffn(g["y"][b], W, X[b], g["idx"][b], ctx=f"{ctx} b={b}"))
    return worst


UNION_TINY = [
    configs.tiny("relu", "f16", d=384, F=1000, r=40, B=5, T=2, seed=21),
    configs.tiny("reglu", "f16", d=1032, F=2000, r=48, B=32, T=2, seed=22),
    configs.tiny("relu", "f16", d=8, F=8, r=8, B=3, T=2, seed=23, mean_rate=0.5),
    configs.tiny("relu", "f16", d=2048, F=4104, r=64, B=2, T=2, seed=24, mean_rate=0.05),
]


@pytest.mark.parametrize("cfg", UNION_TINY, ids=lambda c: c.name + f"_b{c.B}")
def test_union_tiny(cfg):
    say(f"[gpu] union tiny {cfg.name} B={cfg.B}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, B_max=cfg.B)
    bufs = layer.buffers(cfg.B)
    xd = torch.from_numpy(inp["x"]).to(layer.device)
    for t in range(cfg.T):
        g = run_batch(layer, xd[t], cfg.B, bufs)
        check_batch(g, inp, W, inp["x"][t], cfg.F, ctx=f"{cfg.name} t={t}")


def test_union_invariants():
    """Degenerate and special cases of the union operator (fed given lists and masks)."""
    cfg = configs.tiny("reglu", "f16", d=384, F=1000, r=40, B=7, T=1, seed=25)
    say(f"[gpu] union invariants {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    B, F = cfg.B, cfg.F
    layer = _layer(inp, B_max=32)
    X = inp["x"][0]
    xd = torch.from_numpy(X.copy()).to(layer.device)
    y = torch.full((32, cfg.d), 7.0, dtype=torch.float32, device=layer.device)

    def ffn(lst, active, nb=B):
        i, c = _dev_list(layer, lst)
        m = _dev_masks(layer, active)
        layer.sparse_ffn(xd.data_ptr(), nb, i.data_ptr(), c.data_ptr(), m.data_ptr(), y.data_ptr())
        torch.cuda.synchronize()
        return _np(y[:nb]).copy()

    rng = np.random.default_rng(5)
    full = np.arange(F)
    # every neuron listed and set in every mask: the dense FFN of each token
    yy = ffn(full, np.ones((B, F), bool))
    for b in range(B):
        assert P.rel_l2(yy[b], O.ffn_dense(W, X[b])) <= P.REL_TOL
    # empty list, and a full list with all masks clear: exactly zero
    assert np.all(ffn([], np.zeros((B, F), bool)) == 0.0)
    assert np.all(ffn(full, np.zeros((B, F), bool)) == 0.0)
    # a list wider than the masks: neurons outside token b's mask give nothing to y[b]
    act = rng.random((B, F)) < 0.1
    wide = np.flatnonzero(act.any(0) | (rng.random(F) < 0.3))
    yy = ffn(wide, act)
    for b in range(B):
        P.check_ffn(yy[b], W, X[b], O.compact(act[b]), ctx=f"wide b={b}")
    # each token equals the batch-1 operator on its own list
    layer1 = _layer(inp)
    y1 = torch.empty((1, cfg.d), dtype=torch.float32, device=layer.device)
    for b in range(B):
        i, c = _dev_list(layer1, O.compact(act[b]))
        layer1.sparse_ffn(xd[b].data_ptr(), 1, i.data_ptr(), c.data_ptr(), None, y1.data_ptr())
        torch.cuda.synchronize()
        assert P.rel_l2(yy[b], _np(y1[0])) <= P.REL_TOL, b
    # a wide call followed by a narrow one reuses the workspace: no stale H survives
    act2 = rng.random((2, F)) < 0.02
    y2 = ffn(O.compact(act2.any(0)), act2, nb=2)
    for b in range(2):
        P.check_ffn(y2[b], W, X[b], O.compact(act2[b]), ctx=f"narrow b={b}")
    # the kernels are deterministic
    assert np.array_equal(ffn(wide, act), yy)


def test_union_c4_sampled():
    """The batch-32 workload shape: every token's index set on two steps, the FFN of
    eight tokens per step against the oracle."""
    cfg = configs.get("c4")
    say(f"[gpu] union {cfg.name}: generating")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, B_max=cfg.B)
    bufs = layer.buffers(cfg.B)
    for t in (0, cfg.T - 1):
        xb = torch.from_numpy(inp["x"][t].copy()).to(layer.device)
        g = run_batch(layer, xb, cfg.B, bufs)
        worst = check_batch(g, inp, W, inp["x"][t], cfg.F, ctx=f"c4 t={t}",
                            ffn_tokens=[0, 5, 9, 14, 18, 23, 27, 31])
        say(f"[gpu] c4 t={t}: union {g['uidx'].size} of {cfg.F}, "
            f"mean per-token {np.mean([len(i) for i in g['idx']]):.0f}, worst rel-L2 {worst:.2e}")
