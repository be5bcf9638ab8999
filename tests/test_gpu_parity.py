"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Cases: ragged tiny shapes (several tiles plus a tail in every dimension) for
each activation and weight format, and the full workload shapes with every
token's index set checked and sampled tokens' FFN outputs checked.
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


def _layer(inputs, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inputs, **kw)


def _to_np(t):
    return t.detach().cpu().numpy()


def gpu_token(layer, xdev, bufs, rep=0):
    layer.step(xdev.data_ptr(), bufs, rep)
    torch.cuda.synchronize()
    n = int(bufs["count"][0].item())
    return dict(logits=_to_np(bufs["logits"][0]), mask=_to_np(bufs["mask"][0]).view(np.uint32),
                idx=_to_np(bufs["idx"][0, :n]).astype(np.int64), y=_to_np(bufs["y"][0]).copy())


def gpu_ffn_on(layer, xdev, idx_np, bufs):
    """pi_sparse_ffn fed an externally given neuron list."""
    n = len(idx_np)
    idx = torch.zeros(max(1, layer.F), dtype=torch.int32, device=layer.device)
    if n:
        idx[:n] = torch.from_numpy(np.asarray(idx_np, np.int32)).to(layer.device)
    cnt = torch.tensor([n], dtype=torch.int32, device=layer.device)
    layer.sparse_ffn(xdev.data_ptr(), 1, idx.data_ptr(), cnt.data_ptr(), None, bufs["y"].data_ptr())
    torch.cuda.synchronize()
    return _to_np(bufs["y"][0]).copy()


TINY = [
    configs.tiny("relu", "f16", d=384, F=1000, r=40),
    configs.tiny("reglu", "f16", d=1032, F=2000, r=48, seed=9),
    configs.tiny("relu", "i4g128", d=384, F=1000, r=40, seed=10),
    configs.tiny("reglu", "i4g128", d=2176, F=1000, r=40, seed=11),
    configs.tiny("relu", "f16", d=8, F=8, r=8, seed=12, mean_rate=0.5),
]


@pytest.mark.parametrize("cfg", TINY, ids=lambda c: c.name)
def test_tiny_end_to_end(cfg):
    say(f"[gpu] tiny end-to-end {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp)
    bufs = layer.buffers(1)
    xd = torch.from_numpy(inp["x"]).to(layer.device)
    for t in range(cfg.T):
        x = inp["x"][t, 0]
        g = gpu_token(layer, xd[t, 0], bufs)
        ref_l = O.predictor_logits(x, inp["w_p1"], inp["w_p2"], inp["bias"])
        assert np.max(np.abs(g["logits"] - ref_l)) < 5e-5
        P.check_index_set(g["idx"], g["mask"], ref_l, cfg.F, ctx=f"{cfg.name} t={t}")
        P.check_ffn(g["y"], W, x, g["idx"], ctx=f"{cfg.name} t={t} e2e")
        ref_idx = O.compact(O.predicted_active(ref_l))
        P.check_ffn(gpu_ffn_on(layer, xd[t, 0], ref_idx, bufs), W, x, ref_idx, ctx="oracle idx")
        # all neurons listed == the dense reference kernel, and both == the oracle's dense FFN
        y_all = gpu_ffn_on(layer, xd[t, 0], np.arange(cfg.F), bufs)
        layer.dense(xd[t, 0].data_ptr(), 1, bufs["y"].data_ptr())
        torch.cuda.synchronize()
        y_dense = _to_np(bufs["y"][0]).copy()
        assert np.array_equal(y_all, y_dense), "all-ones list must equal the dense kernel bit for bit"
        P.check_ffn(y_dense, W, x, np.arange(cfg.F), ctx="dense")
        # the true support of the activation reproduces the dense FFN
        pa = O.preact(W, x)
        sup = np.flatnonzero(pa["g" if cfg.act == "reglu" else "a"] > 0)
        assert P.rel_l2(gpu_ffn_on(layer, xd[t, 0], sup, bufs), O.ffn_dense(W, x)) <= P.REL_TOL
        # an empty list gives exactly zero
        assert np.all(gpu_ffn_on(layer, xd[t, 0], [], bufs) == 0.0)


@pytest.mark.parametrize("F", [8, 1000, 1024, 4096, 28672, 32768])
@pytest.mark.parametrize("B", [1, 3, 32])
def test_compact_gpu(F, B):
    from activation_sparse_pi_amd import _lib as L
    say(f"[gpu] compact F={F} B={B}")
    rng = np.random.default_rng(F * 100 + B)
    W = (F + 31) // 32
    for p in (0.0, 0.03, 0.5, 1.0):
        act = rng.random((B, F)) < p
        words = O.mask_words(act)
        # garbage above F in the last word must be ignored
        if F % 32:
            words[:, -1] |= np.uint32(0xFFFFFFFF) << np.uint32(F % 32)
        md = torch.from_numpy(words.view(np.int32)).to("cuda")
        idx = torch.full((B, F), -7, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
        L.check(L.pi_compact(md.data_ptr(), B, F, L.PI_PER_TOKEN, idx.data_ptr(), cnt.data_ptr(),
                             None, 0, torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        ci, cc = _to_np(idx), _to_np(cnt)
        for b in range(B):
            want = O.compact(act[b])
            assert cc[b] == want.size and np.array_equal(ci[b, :cc[b]], want), (F, B, p, b)
        uidx = torch.full((F,), -7, dtype=torch.int32, device="cuda")
        ucnt = torch.zeros(1, dtype=torch.int32, device="cuda")
        L.check(L.pi_compact(md.data_ptr(), B, F, L.PI_UNION, uidx.data_ptr(), ucnt.data_ptr(),
                             None, 0, torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        want = O.compact(O.union_active(act))
        n = int(_to_np(ucnt)[0])
        assert n == want.size and np.array_equal(_to_np(uidx)[:n], want), (F, B, p, "union")


_CACHE = {}


def _full(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = gen.make(configs.get(name))
    return _CACHE[name]


SAMPLED = {"c1": 64, "c2": 6, "c3": 4, "c5": 3}


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_config_end_to_end(name):
    cfg = configs.get(name)
    say(f"[gpu] full config {cfg.name}: generating")
    inp = _full(name)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp)
    bufs = layer.buffers(1)
    xd = torch.from_numpy(inp["x"]).to(layer.device)
    X = inp["x"][:, 0, :]
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])   # [T, F]
    sample = set(np.linspace(0, cfg.T - 1, SAMPLED[name]).astype(int).tolist())
    say(f"[gpu] full config {cfg.name}: {cfg.T} tokens, FFN checked on {sorted(sample)}")
    band_total, worst = 0, 0.0
    for t in range(cfg.T):
        g = gpu_token(layer, xd[t, 0], bufs)
        band_total += P.check_index_set(g["idx"], g["mask"], ref_L[t], cfg.F, ctx=f"{name} t={t}")
        if t in sample:
            worst = max(worst, P.check_ffn(g["y"], W, X[t], g["idx"], ctx=f"{name} t={t}"))
            ref_idx = O.compact(O.predicted_active(ref_L[t]))
            P.check_ffn(gpu_ffn_on(layer, xd[t, 0], ref_idx, bufs), W, X[t], ref_idx,
                        ctx=f"{name} t={t} oracle idx")
    say(f"[gpu] {name}: band disagreements {band_total}, worst rel-L2 {worst:.2e}")


def _run_modes():
    from activation_sparse_pi_amd import _lib as L
    return {"fused": L.PI_RUN_FUSED, "split": L.PI_RUN_SPLIT}


def _decode_single_steps(layer, inp, W, xd, tokens, mode, ctx):
    """Each token as a one-step run, checked against the oracle (index set, table, mask, y)."""
    cfg = inp["cfg"]
    X = inp["x"][:, 0, :]
    ref_L = O.predictor_logits(X[tokens], inp["w_p1"], inp["w_p2"], inp["bias"])
    bufs = layer.buffers(1)
    for i, t in enumerate(tokens):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=mode)
        torch.cuda.synchronize()
        n = int(bufs["count"][0].item())
        gidx = _to_np(bufs["idx"][0, :n]).astype(np.int64)
        gmask = _to_np(bufs["mask"][0]).view(np.uint32)
        P.check_index_set(gidx, gmask, ref_L[i], cfg.F, ctx=f"{ctx} t={t}")
        P.check_ffn(_to_np(bufs["y"][0]), W, X[t], gidx, ctx=f"{ctx} t={t}")


def _decode_long_run(layer, cfg, xd, s0, nsteps, mode):
    """A multi-step run ends with exactly what a one-step run of its last token gives
    (the kernels are deterministic and a step does not depend on earlier ones)."""
    bufs, ref = layer.buffers(1), layer.buffers(1)
    layer.decode_run(xd.data_ptr(), cfg.T, s0, nsteps, bufs, mode=mode)
    layer.decode_run(xd.data_ptr(), cfg.T, s0 + nsteps - 1, 1, ref, mode=mode)
    torch.cuda.synchronize()
    c = int(ref["count"][0].item())
    assert int(bufs["count"][0].item()) == c
    assert torch.equal(bufs["idx"][0, :c], ref["idx"][0, :c])
    assert torch.equal(bufs["mask"], ref["mask"])
    assert torch.equal(bufs["y"], ref["y"])


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_decode_run(name, mode):
    """pi_decode_run as two (fused) or three (split) kernels per step, against the oracle on
    single steps; a 17-step run over 3 replicas ends with the one-step result of its last
    token, bit for bit."""
    cfg = configs.get(name)
    say(f"[gpu] decode_run {mode} on {cfg.name}")
    inp = _full(name)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=3)
    xd = torch.from_numpy(inp["x"][:, 0, :].copy()).to(layer.device)
    tokens = sorted(set(np.linspace(0, cfg.T - 1, 5).astype(int).tolist()))
    m = _run_modes()[mode]
    _decode_single_steps(layer, inp, W, xd, tokens, m, f"{name} {mode}")
    _decode_long_run(layer, cfg, xd, 40, 17, m)


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("cfg", TINY, ids=lambda c: c.name)
def test_decode_run_tiny(cfg, mode):
    """Both schedules on ragged shapes (tails in d, F and r; F = 8): every token as a
    one-step run against the oracle, then a long run that must end on the one-step result
    of its last token."""
    say(f"[gpu] decode_run {mode} tiny {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=2)
    xd = torch.from_numpy(inp["x"][:, 0, :].copy()).to(layer.device)
    m = _run_modes()[mode]
    _decode_single_steps(layer, inp, W, xd, list(range(cfg.T)), m, f"{cfg.name} {mode}")
    _decode_long_run(layer, cfg, xd, 3, 40, m)


def test_decode_run_modes_agree_on_tables():
    """The two kernel schedules share their mask kernel: on c2 tokens they give the same neuron
    tables, equal to the oracle's outside the band, and y agreeing to fp32 rounding."""
    inp = _full("c2")
    cfg = inp["cfg"]
    layer = _layer(inp, replicas=1)
    xd = torch.from_numpy(inp["x"][:, 0, :].copy()).to(layer.device)
    X = inp["x"][:, 0, :]
    modes = _run_modes()
    for t in (0, 100, 255):
        out = {}
        for mname, m in modes.items():
            b = layer.buffers(1)
            layer.decode_run(xd.data_ptr(), cfg.T, t, 1, b, mode=m)
            torch.cuda.synchronize()
            n = int(b["count"][0].item())
            out[mname] = (_to_np(b["idx"][0, :n]).astype(np.int64), _to_np(b["y"][0]).copy(),
                          _to_np(b["mask"][0]).view(np.uint32).copy())
        ref_l = O.predictor_logits(X[t], inp["w_p1"], inp["w_p2"], inp["bias"])
        assert np.array_equal(out["fused"][0], out["split"][0]), f"t={t}: fused and split tables differ"
        P.check_index_set(out["fused"][0], out["fused"][2], ref_l, cfg.F, ctx=f"c2 t={t}")
        assert P.rel_l2(out["fused"][1], out["split"][1]) <= 1e-5


def test_operators_match_sparse_ffn():
    """pi_ffn_up + pi_ffn_down give, bit for bit, what pi_sparse_ffn gives."""
    cfg = configs.C1
    inp = _full("c1")
    layer = _layer(inp)
    bufs, ref = layer.buffers(1), layer.buffers(1)
    xd = torch.from_numpy(inp["x"][:, 0, :].copy()).to(layer.device)
    for t in (0, 7, 33):
        layer.step(xd[t].data_ptr(), ref, logits=False)
        layer.ffn_up(xd[t].data_ptr(), ref["idx"].data_ptr(), ref["count"].data_ptr(),
                     bufs["h"].data_ptr())
        layer.ffn_down(ref["idx"].data_ptr(), ref["count"].data_ptr(), bufs["h"].data_ptr(),
                       bufs["y"].data_ptr())
        torch.cuda.synchronize()
        assert torch.equal(bufs["y"], ref["y"])


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_decode_run_graph_replay(mode):
    """A run captured into a HIP graph (the library records kernels only: no memset, no host
    sync) replays bit-identically to the same run enqueued eagerly, three times, with eager
    runs of other steps in between."""
    cfg = configs.C1
    inp = _full("c1")
    layer = _layer(inp, replicas=3)
    xd = torch.from_numpy(inp["x"][:, 0, :].copy()).to(layer.device)
    m = _run_modes()[mode]
    bufs = layer.buffers(1)
    layer.decode_run(xd.data_ptr(), cfg.T, 5, 9, bufs, mode=m)
    torch.cuda.synchronize()
    ref = {k: bufs[k].clone() for k in ("y", "mask", "idx", "count")}
    side = torch.cuda.Stream(device=layer.device)
    side.wait_stream(torch.cuda.current_stream(layer.device))
    with torch.cuda.stream(side):
        layer.decode_run(xd.data_ptr(), cfg.T, 0, 2, bufs, mode=m)
    torch.cuda.current_stream(layer.device).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.decode_run(xd.data_ptr(), cfg.T, 5, 9, bufs, mode=m)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        c = int(ref["count"][0].item())
        assert int(bufs["count"][0].item()) == c, f"replay {rep}: count"
        assert torch.equal(bufs["idx"][0, :c], ref["idx"][0, :c]), f"replay {rep}: table"
        assert torch.equal(bufs["mask"], ref["mask"]) and torch.equal(bufs["y"], ref["y"]), f"replay {rep}"
        layer.decode_run(xd.data_ptr(), cfg.T, 20 + rep, 4, bufs, mode=m)   # eager work in between
        torch.cuda.synchronize()
