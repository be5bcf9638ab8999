"""The int8 group-128 predictor on the GPU against the oracle of the same predictor.

The oracle dequantizes the stored int8 factors itself (``dequant_int8``) and runs the
unchanged fp64 predictor, threshold, table and FFN; the parity contract is the fp16 one
(index sets equal outside the 1e-4 band of the oracle's logits, rel-L2 <= 1e-3 for y).
How close the int8 predictor's masks come to the fp16 predictor's is reported, not
asserted: that is a property of the quantization, not of the kernels.
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


def _L():
    from activation_sparse_pi_amd import _lib as L
    return L


def _inputs(cfg):
    inp = gen.make(cfg)
    inp.update(gen.predictor_int8(inp))
    W1, W2 = O.predictor_from_int8(inp["q_p1t"], inp["s_p1t"], inp["q_p2t"], inp["s_p2t"])
    return inp, W1, W2


def _layer(inp, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inp, pred_format="i8g128", **kw)


TINY8 = [
    configs.tiny("relu", "f16", d=384, F=1000, r=128, seed=51),
    configs.tiny("reglu", "f16", d=1024, F=2000, r=256, seed=52),
    configs.tiny("reglu", "i4g128", d=384, F=1000, r=128, seed=53),
    configs.tiny("relu", "f16", d=128, F=8, r=128, seed=54, mean_rate=0.5),
    configs.tiny("reglu", "f16", d=256, F=64, r=256, seed=56, mean_rate=0.4),   # one full tile
    # d >= 3200: stage 1 takes one row per block with four waves (208 chunks of 16 weights,
    # split raggedly: the fourth wave holds 16), also in the multi-step conversion variant
    configs.tiny("reglu", "f16", d=3328, F=1000, r=256, seed=55),
]


@pytest.mark.parametrize("cfg", TINY8, ids=lambda c: c.name)
def test_int8_operator_path(cfg):
    """pi_predict (B = 1, compaction fused) + pi_sparse_ffn: logits, mask, list, y."""
    say(f"[gpu] int8 predictor operators {cfg.name}")
    inp, W1, W2 = _inputs(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp)
    X = inp["x"][:, 0, :]
    ref_L = O.predictor_logits(X, W1, W2, inp["bias"])
    bufs = layer.buffers(1)
    agree = []
    for t in range(cfg.T):
        xd = torch.from_numpy(X[t].copy()).cuda()
        layer.step(xd.data_ptr(), bufs)
        torch.cuda.synchronize()
        n = int(bufs["count"][0].item())
        gidx = _np(bufs["idx"][0, :n]).astype(np.int64)
        assert np.max(np.abs(_np(bufs["logits"][0]) - ref_L[t])) < 5e-5, f"{cfg.name} t={t}: logits"
        P.check_index_set(gidx, _np(bufs["mask"][0]).view(np.uint32), ref_L[t], cfg.F, ctx=f"{cfg.name} t={t}")
        P.check_ffn(_np(bufs["y"][0]), W, X[t], gidx, ctx=f"{cfg.name} t={t}")
        l16 = O.predictor_logits(X[t], inp["w_p1"], inp["w_p2"], inp["bias"])
        agree.append(np.mean((l16 > 0) == (ref_L[t] > 0)))
    say(f"[gpu] {cfg.name}: int8 vs fp16 predictor mask agreement {np.mean(agree):.4f}")


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("cfg", TINY8, ids=lambda c: c.name)
def test_int8_decode_run(cfg, mode):
    """Every token as a one-step pi_decode_run, then a 40-step run that must end on the
    one-step result of its last token."""
    L = _L()
    say(f"[gpu] int8 predictor decode {mode} {cfg.name}")
    inp, W1, W2 = _inputs(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=2)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    ref_L = O.predictor_logits(X, W1, W2, inp["bias"])
    m = {"fused": L.PI_RUN_FUSED, "split": L.PI_RUN_SPLIT}[mode]
    bufs = layer.buffers(1)
    for t in range(cfg.T):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=m)
        torch.cuda.synchronize()
        n = int(bufs["count"][0].item())
        gidx = _np(bufs["idx"][0, :n]).astype(np.int64)
        P.check_index_set(gidx, _np(bufs["mask"][0]).view(np.uint32), ref_L[t], cfg.F, ctx=f"{cfg.name} t={t}")
        P.check_ffn(_np(bufs["y"][0]), W, X[t], gidx, ctx=f"{cfg.name} {mode} t={t}")
    ref = layer.buffers(1)
    layer.decode_run(xd.data_ptr(), cfg.T, 3, 40, bufs, mode=m)
    layer.decode_run(xd.data_ptr(), cfg.T, 42, 1, ref, mode=m)
    torch.cuda.synchronize()
    assert torch.equal(bufs["y"], ref["y"]) and torch.equal(bufs["mask"], ref["mask"])


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_int8_decode_full(name):
    """The LLaMA-7B- and LLaMA-70B-shaped layers (fp16 and int4 FFN) with the int8 predictor,
    the default kernel schedule, on sampled tokens."""
    L = _L()
    cfg = configs.get(name)
    say(f"[gpu] int8 predictor decode {cfg.name}")
    inp, W1, W2 = _inputs(cfg)
    W = O.Weights.from_inputs(inp)
    layer = _layer(inp, replicas=2)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    tokens = [0, cfg.T // 2, cfg.T - 1]
    ref_L = O.predictor_logits(X[tokens], W1, W2, inp["bias"])
    bufs = layer.buffers(1)
    band = 0
    for i, t in enumerate(tokens):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=L.PI_RUN_KERNELS)
        torch.cuda.synchronize()
        n = int(bufs["count"][0].item())
        gidx = _np(bufs["idx"][0, :n]).astype(np.int64)
        band += P.check_index_set(gidx, _np(bufs["mask"][0]).view(np.uint32), ref_L[i], cfg.F, ctx=f"{name} t={t}")
        P.check_ffn(_np(bufs["y"][0]), W, X[t], gidx, ctx=f"{name} t={t}")
    say(f"[gpu] {name}: band disagreements {band}")
    # a 17-step run (every step after the first sums its predecessor's partial rows in the
    # stage-1 kernel) ends bit-identical to a one-step run of its last token, against the oracle
    s0, n = 5, 17
    last = s0 + n - 1
    ref = layer.buffers(1)
    layer.decode_run(xd.data_ptr(), cfg.T, s0, n, bufs, mode=L.PI_RUN_KERNELS)
    layer.decode_run(xd.data_ptr(), cfg.T, last, 1, ref, mode=L.PI_RUN_KERNELS)
    torch.cuda.synchronize()
    c = int(ref["count"][0].item())
    assert int(bufs["count"][0].item()) == c and torch.equal(bufs["idx"][0, :c], ref["idx"][0, :c])
    assert torch.equal(bufs["mask"], ref["mask"]) and torch.equal(bufs["y"], ref["y"])
    gidx = _np(bufs["idx"][0, :c]).astype(np.int64)
    ref_last = O.predictor_logits(X[last % cfg.T], W1, W2, inp["bias"])
    P.check_index_set(gidx, _np(bufs["mask"][0]).view(np.uint32), ref_last, cfg.F, ctx=f"{name} run")
    P.check_ffn(_np(bufs["y"][0]), W, X[last % cfg.T], gidx, ctx=f"{name} run")


def test_int8_placed():
    """A placed layer with the int8 predictor (its W2t rows and scales permuted)."""
    L = _L()
    cfg = TINY8[1]
    say(f"[gpu] int8 predictor placed {cfg.name}")
    inp, W1, W2 = _inputs(cfg)
    W = O.Weights.from_inputs(inp)
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 100, cfg.F).astype(np.int32)
    perm = np.empty(cfg.F, np.int32)
    L.check(L.pi_place_neurons(counts.ctypes.data, cfg.F, perm.ctypes.data))
    layer = _layer(inp, perm=perm)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    ref_L = O.predictor_logits(X, W1, W2, inp["bias"])
    bufs = layer.buffers(1)
    table = torch.empty_like(bufs["idx"])
    for t in range(cfg.T):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=L.PI_RUN_SPLIT)
        layer.map_ids(bufs["idx"].data_ptr(), bufs["count"].data_ptr(), 1, table.data_ptr())
        torch.cuda.synchronize()
        n = int(bufs["count"][0].item())
        orig = np.sort(_np(table[0, :n]).astype(np.int64))
        act = np.zeros(cfg.F, bool)
        act[orig] = True
        P.check_index_set(orig, O.mask_words(act), ref_L[t], cfg.F, ctx=f"placed t={t}")
        P.check_ffn(_np(bufs["y"][0]), W, X[t], orig, ctx=f"placed t={t}")


def test_int8_unsupported_paths_raise():
    L = _L()
    cfg = TINY8[0]
    inp, _, _ = _inputs(cfg)
    layer = _layer(inp, B_max=2)
    bufs = layer.buffers(2)
    xd = torch.from_numpy(inp["x"][:, 0, :].copy()).cuda()
    with pytest.raises(L.PiError) as e:
        layer.predict(xd.data_ptr(), 2, None, bufs["mask"].data_ptr(), None, None)
    assert e.value.status == L.PI_ERR_UNSUPPORTED
