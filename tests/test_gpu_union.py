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


PRED_CASES = [
    configs.tiny("relu", "f16", d=640, F=1000, r=1040, B=4, T=1, seed=31),     # 3 passes of the rank
    configs.tiny("relu", "f16", d=8, F=8, r=8, B=32, T=1, seed=32, mean_rate=0.5),
    configs.tiny("relu", "f16", d=1032, F=2056, r=96, B=17, T=1, seed=33),
]


def _predict_only(cfg, inp, B, want_idx=True):
    """pi_predict at batch B straight through the C ABI (predictor weights only)."""
    from activation_sparse_pi_amd import _lib as L
    dev = torch.device("cuda")
    w1 = torch.from_numpy(np.ascontiguousarray(inp["w_p1"].T)).to(dev)
    w2 = torch.from_numpy(np.ascontiguousarray(inp["w_p2"].T)).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev)
    x = torch.from_numpy(inp["x"][0].copy()).to(dev)
    pred = L.PredDesc(w1.data_ptr(), w2.data_ptr(), bias.data_ptr(), cfg.d, cfg.r, cfg.F, 0.5)
    nb = L.pi_workspace_bytes(pred, None, B)
    assert nb > 0, L.pi_last_error()
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    L.check(L.pi_workspace_init(ws.data_ptr(), nb, stream))
    W = (cfg.F + 31) // 32
    logits = torch.empty((B, cfg.F), dtype=torch.float32, device=dev)
    mask = torch.full((B, W), -1, dtype=torch.int32, device=dev)
    idx = torch.full((B, cfg.F), -7, dtype=torch.int32, device=dev)
    cnt = torch.zeros(B, dtype=torch.int32, device=dev)
    for _ in range(2):                          # twice: counters and partials are reused
        L.check(L.pi_predict(pred, x.data_ptr(), B, logits.data_ptr(), mask.data_ptr(),
                             idx.data_ptr() if want_idx else None,
                             cnt.data_ptr() if want_idx else None, ws.data_ptr(), nb, stream))
    torch.cuda.synchronize()
    c = _np(cnt)
    lists = [_np(idx[b, :c[b]]).astype(np.int64) for b in range(B)] if want_idx else None
    return _np(logits), _np(mask).view(np.uint32), lists


@pytest.mark.parametrize("cfg", PRED_CASES, ids=lambda c: f"{c.name}_b{c.B}")
def test_predict_batch(cfg):
    say(f"[gpu] batch predictor {cfg.name} B={cfg.B}")
    inp = gen.make(cfg, ffn=False)
    X = inp["x"][0]
    lg, mk, lists = _predict_only(cfg, inp, cfg.B)
    ref = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    assert np.max(np.abs(lg - ref)) < 5e-5
    for b in range(cfg.B):
        P.check_index_set(lists[b], mk[b], ref[b], cfg.F, ctx=f"b={b}")


def test_predict_batch_c5_shape():
    """The batch predictor at the largest rank of the workloads (d=8192, r=1024,
    F=28672), 32 tokens, masks only (no neuron tables)."""
    import dataclasses
    cfg = dataclasses.replace(configs.C5, B=32, T=1)
    say(f"[gpu] batch predictor at {cfg.name} shape, B=32")
    inp = gen.make(cfg, ffn=False)
    X = inp["x"][0]
    lg, mk, _ = _predict_only(cfg, inp, 32, want_idx=False)
    ref = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    err = np.max(np.abs(lg - ref))
    say(f"[gpu] c5-shape batch predictor max |dl| {err:.2e}")
    assert err < 5e-5
    for b in range(32):
        gpu_active = O.words_to_active(mk[b], cfg.F)
        P.check_index_set(O.compact(gpu_active), mk[b], ref[b], cfg.F, ctx=f"b={b}")


@pytest.mark.parametrize("cfg", [
    configs.tiny("relu", "f16", d=1032, F=2056, r=96, B=6, T=1, seed=41),
    configs.tiny("reglu", "f16", d=384, F=1000, r=40, B=3, T=1, seed=42),
], ids=lambda c: f"{c.name}_b{c.B}")
def test_batch_schedules_agree(cfg):
    """The two schedules pi_batch_plan chooses between: every token through the batch-1
    operators with its own list, and one union pass.  Both match the oracle on each token's
    own list; pi_batch_plan takes the layer's descriptor (at rates of 0 and 1 its expected
    union is the union's size)."""
    from activation_sparse_pi_amd import _lib as L
    say(f"[gpu] batch schedules {cfg.name} B={cfg.B}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, B_max=cfg.B)
    bufs = layer.buffers(cfg.B)
    xd = torch.from_numpy(inp["x"]).to(layer.device)
    g = run_batch(layer, xd[0], cfg.B, bufs)                 # union schedule
    check_batch(g, inp, W, inp["x"][0], cfg.F, ctx=f"{cfg.name} union")
    yt = torch.zeros((cfg.B, cfg.d), dtype=torch.float32, device=layer.device)
    for b in range(cfg.B):                                   # token schedule, own lists
        layer.sparse_ffn(xd[0, b].data_ptr(), 1, bufs["idx"][b].data_ptr(), bufs["count"][b:].data_ptr(),
                         None, yt[b].data_ptr())
    torch.cuda.synchronize()
    y_tok = _np(yt)
    for b in range(cfg.B):
        P.check_ffn(y_tok[b], W, inp["x"][0, b], g["idx"][b], ctx=f"{cfg.name} tokens b={b}")
    rate = np.zeros(cfg.F, np.float32)                       # every neuron at rate 0 or 1
    for b in range(cfg.B):
        rate[g["idx"][b]] = 1.0
    p = L.BatchPlan()
    L.check(L.pi_batch_plan(layer.ffn[0], cfg.B, rate.ctypes.data, 8000.0, p))
    assert p.u_mean == pytest.approx(len(g["uidx"]))


def test_union_past_2gb_rows():
    """Weight matrices larger than 2^31 bytes (F = 131080, d = 8192: rows from 131072 on start
    past 2 GB) take the union kernels' general loop; token lists that include the last rows,
    checked against the oracle on each token's own list (the oracle holds only the listed
    rows, renumbered)."""
    from activation_sparse_pi_amd import _lib as L
    F, d, B = 131080, 8192, 4
    assert F * d * 2 > 2**31 - 1
    say(f"[gpu] union past 2 GB: F={F} d={d} B={B}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(51)
    w_up = torch.empty((F, d), dtype=torch.float16, device=dev).normal_(0.0, 0.02, generator=g)
    w_dn = torch.empty((F, d), dtype=torch.float16, device=dev).normal_(0.0, 0.02, generator=g)
    rng = np.random.default_rng(52)
    x = rng.standard_normal((B, d)).astype(np.float16)
    act = np.zeros((B, F), bool)
    for b in range(B):
        act[b, rng.choice(F, 60, replace=False)] = True
        act[b, F - 1 - b] = True                            # the last rows, past 2 GB
        act[b, 131072 + 2 * b] = True
    act[:, 5] = True                                         # one neuron shared by every token
    desc = L.FfnDesc(None, w_up.data_ptr(), w_dn.data_ptr(), None, None, None, d, F,
                     L.PI_ACT_RELU, L.PI_W_F16)
    nws = L.pi_workspace_bytes(None, desc, B)
    assert nws > 0, L.pi_last_error()
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    L.check(L.pi_workspace_init(ws.data_ptr(), nws, stream))
    xd = torch.from_numpy(x).to(dev)
    md = torch.from_numpy(O.mask_words(act).view(np.int32)).to(dev)
    uidx = torch.empty((F,), dtype=torch.int32, device=dev)
    ucnt = torch.empty((1,), dtype=torch.int32, device=dev)
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    L.check(L.pi_compact(md.data_ptr(), B, F, L.PI_UNION, uidx.data_ptr(), ucnt.data_ptr(), None, 0, stream))
    L.check(L.pi_sparse_ffn(desc, xd.data_ptr(), B, uidx.data_ptr(), ucnt.data_ptr(), md.data_ptr(),
                            y.data_ptr(), ws.data_ptr(), nws, stream))
    torch.cuda.synchronize()
    un = O.compact(O.union_active(act))
    assert np.array_equal(_np(uidx[: int(_np(ucnt)[0])]).astype(np.int64), un)
    sel = torch.from_numpy(un).to(dev)
    Wsmall = O.Weights("relu", "f16", {"w_up": _np(w_up[sel]), "w_down": _np(w_dn[sel])})
    pos = {int(n): k for k, n in enumerate(un)}
    yg = _np(y)
    for b in range(B):
        own = np.array([pos[int(n)] for n in O.compact(act[b])], np.int64)
        P.check_ffn(yg[b], Wsmall, x[b], own, ctx=f"past 2 GB b={b}")
    del w_up, w_dn
    torch.cuda.empty_cache()
