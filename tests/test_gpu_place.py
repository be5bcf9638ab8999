"""Neuron placement on the GPU (pi_permute_rows, pi_map_ids) and placed layers vs the oracle.

A placed layer holds every per-neuron array permuted by pi_place_neurons' layout; its masks,
lists and logits are in placed order, and the neuron table (pi_map_ids) names the original
neurons.  The oracle is unchanged: the original layer's logits, active sets and FFN output.
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


def _layer(inputs, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inputs, **kw)


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("n,row_bytes,shift", [(1000, 768, 0), (1000, 4, 0), (37, 6, 0), (5, 64, 0),
                                               (300, 32, 4), (1, 2, 0)])
def test_permute_rows_bit_exact(n, row_bytes, shift):
    """16-byte, 4-byte and byte copies (a source 4 bytes off 16-byte alignment takes the
    4-byte path); an entry outside [0, n) gives a zero row."""
    L = _L()
    say(f"[gpu] permute_rows n={n} row_bytes={row_bytes} shift={shift}")
    rng = np.random.default_rng(n + row_bytes)
    src_h = rng.integers(0, 256, size=n * row_bytes + shift, dtype=np.uint8)
    perm = rng.permutation(n).astype(np.int32)
    if n > 3:
        perm[2] = n + 5                                          # out of range: zero row
    src = torch.from_numpy(src_h).cuda()
    dst = torch.full((n * row_bytes,), 0xAB, dtype=torch.uint8, device="cuda")
    pd = torch.from_numpy(perm).cuda()
    L.check(L.pi_permute_rows(src.data_ptr() + shift, dst.data_ptr(), pd.data_ptr(), n, row_bytes, _stream()))
    torch.cuda.synchronize()
    rows = src_h[shift:].reshape(n, row_bytes)
    want = np.zeros((n, row_bytes), np.uint8)
    ok = (perm >= 0) & (perm < n)
    want[ok] = rows[perm[ok]]
    assert np.array_equal(_np(dst).reshape(n, row_bytes), want)


def test_map_ids_table_and_in_place():
    L = _L()
    say("[gpu] map_ids")
    B, F = 3, 100
    rng = np.random.default_rng(5)
    perm = rng.permutation(F).astype(np.int32)
    idx = np.full((B, F), -5, np.int32)
    cnt = np.array([0, 17, F], np.int32)
    for b in range(B):
        idx[b, :cnt[b]] = np.sort(rng.choice(F, cnt[b], replace=False))
    idx[1, 3] = F + 1                                             # outside [0, F): -1
    di, dc, dp = (torch.from_numpy(a).cuda() for a in (idx, cnt, perm))
    out = torch.full((B, F), -9, dtype=torch.int32, device="cuda")
    L.check(L.pi_map_ids(di.data_ptr(), dc.data_ptr(), B, F, dp.data_ptr(), out.data_ptr(), _stream()))
    L.check(L.pi_map_ids(di.data_ptr(), dc.data_ptr(), B, F, dp.data_ptr(), di.data_ptr(), _stream()))
    torch.cuda.synchronize()
    want = np.full((B, F), -9, np.int32)
    for b in range(B):
        k = idx[b, :cnt[b]]
        want[b, :cnt[b]] = np.where((k >= 0) & (k < F), perm[np.clip(k, 0, F - 1)], -1)
    assert np.array_equal(_np(out), want)
    inplace = idx.copy()
    for b in range(B):
        inplace[b, :cnt[b]] = want[b, :cnt[b]]
    assert np.array_equal(_np(di), inplace)


@pytest.mark.parametrize("F,B", [(1000, 1), (1000, 3), (33, 32), (4096, 32), (28672, 17)])
def test_count_active_matches_oracle_masks(F, B):
    """pi_count_active adds, per neuron, the number of masks in which it is set: bit-exact
    against the column sums of oracle-built masks, accumulated over two calls, with garbage
    bits above F in the last word ignored."""
    L = _L()
    say(f"[gpu] count_active F={F} B={B}")
    rng = np.random.default_rng(F * 7 + B)
    rate = rng.random(F) ** 3                                   # skewed, like the Zipf rates
    acts = [rng.random((B, F)) < rate for _ in range(2)]
    W = (F + 31) // 32
    counts = torch.full((F,), 5, dtype=torch.int32, device="cuda")
    for a in acts:
        words = O.mask_words(a).astype(np.uint32)
        if F % 32:
            words[:, -1] |= np.uint32(0xFFFFFFFF) << np.uint32(F % 32)
        md = torch.from_numpy(words.view(np.int32).reshape(B, W).copy()).cuda()
        L.check(L.pi_count_active(md.data_ptr(), B, F, counts.data_ptr(), _stream()))
    torch.cuda.synchronize()
    want = 5 + sum(a.sum(axis=0) for a in acts)
    assert np.array_equal(_np(counts), want.astype(np.int32))


def test_activation_counts_profiling_run():
    """The profiling run (pi_predict masks counted by pi_count_active) against the oracle's
    predicted sets on the same calibration tokens, outside the exclusion band."""
    cfg = configs.tiny("reglu", "f16", d=1032, F=2000, r=48, T=1, seed=9)
    inp = gen.make(cfg)
    L = _L()
    prof = _layer(inp, B_max=L.PI_MAX_BATCH)
    xc = gen.calibration_x(cfg, 70)
    got = prof.activation_counts(torch.from_numpy(xc).cuda())
    lg = O.predictor_logits(xc, inp["w_p1"], inp["w_p2"], inp["bias"])
    want = O.predicted_active(lg).sum(axis=0)
    slack = O.exclusion_band(lg).sum(axis=0)
    assert np.all(np.abs(got.astype(np.int64) - want) <= slack), "counts outside the band slack"


def _placement(inp, ncal=64):
    """pi_place_neurons from a profiling run of the unplaced layer on calibration tokens."""
    L = _L()
    cfg = inp["cfg"]
    prof = _layer(inp, B_max=L.PI_MAX_BATCH)
    cal = torch.from_numpy(gen.calibration_x(cfg, ncal)).cuda()
    counts = prof.activation_counts(cal)
    perm = np.empty(cfg.F, np.int32)
    L.check(L.pi_place_neurons(counts.ctypes.data, cfg.F, perm.ctypes.data))
    return perm, counts


def _check_placed(layer, perm, bufs, b, ref_logits, W, x, F, ctx, logits=None):
    """Token b of a placed layer's outputs against the oracle of the original layer."""
    n = int(bufs["count"][b].item())
    placed = _np(bufs["idx"][b, :n]).astype(np.int64)
    pact = np.zeros(F, bool)
    pact[placed] = True
    assert n == 0 or np.all(np.diff(placed) > 0), f"{ctx}: placed list not ascending"
    assert np.array_equal(_np(bufs["mask"][b]).view(np.uint32), O.mask_words(pact)), f"{ctx}: mask"
    table = torch.empty_like(bufs["idx"])
    layer.map_ids(bufs["idx"].data_ptr(), bufs["count"].data_ptr(), bufs["count"].numel(), table.data_ptr())
    torch.cuda.synchronize()
    orig = _np(table[b, :n]).astype(np.int64)
    assert np.array_equal(orig, perm[placed]), f"{ctx}: neuron table"
    orig = np.sort(orig)
    oact = np.zeros(F, bool)
    oact[orig] = True
    P.check_index_set(orig, O.mask_words(oact), ref_logits, F, ctx=ctx)
    if logits is not None:
        assert np.max(np.abs(logits - ref_logits[perm])) < 5e-5, f"{ctx}: logits"
    return P.check_ffn(_np(bufs["y"][b]), W, x, orig, ctx=ctx)


PLACE_TINY = [
    configs.tiny("relu", "f16", d=384, F=1000, r=40, seed=41),
    configs.tiny("reglu", "i4g128", d=384, F=1000, r=40, seed=42),
    configs.tiny("reglu", "f16", d=1032, F=2000, r=48, seed=43),
]


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("cfg", PLACE_TINY, ids=lambda c: c.name)
def test_placed_decode_tiny(cfg, mode):
    """Every token of a placed layer as a one-step pi_decode_run against the oracle of the
    original layer: the active set through the neuron table, the placed mask and list, y."""
    L = _L()
    say(f"[gpu] placed decode {mode} tiny {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm, _ = _placement(inp)
    assert not np.array_equal(perm, np.arange(cfg.F))
    layer = _layer(inp, replicas=2, perm=perm)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    m = {"fused": L.PI_RUN_FUSED, "split": L.PI_RUN_SPLIT}[mode]
    bufs = layer.buffers(1)
    for t in range(cfg.T):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=m)
        torch.cuda.synchronize()
        _check_placed(layer, perm, bufs, 0, ref_L[t], W, X[t], cfg.F, f"{cfg.name} {mode} t={t}")


def test_placed_step_logits_tiny():
    """The operator path (pi_predict + pi_sparse_ffn) on a placed layer: logits in placed
    order equal the original logits permuted."""
    cfg = PLACE_TINY[0]
    say(f"[gpu] placed step {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm, _ = _placement(inp)
    layer = _layer(inp, perm=perm)
    X = inp["x"][:, 0, :]
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    bufs = layer.buffers(1)
    for t in range(cfg.T):
        xd = torch.from_numpy(X[t].copy()).cuda()
        layer.step(xd.data_ptr(), bufs)
        torch.cuda.synchronize()
        _check_placed(layer, perm, bufs, 0, ref_L[t], W, X[t], cfg.F, f"{cfg.name} t={t}",
                      logits=_np(bufs["logits"][0]))


def test_placed_decode_c2():
    """The LLaMA-7B-shaped layer placed from 256 calibration tokens, two-kernel schedule, on
    sampled tokens of its stream."""
    L = _L()
    cfg = configs.get("c2")
    say(f"[gpu] placed decode {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm, counts = _placement(inp, ncal=256)
    layer = _layer(inp, replicas=2, perm=perm)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    tokens = [0, 77, 255]
    ref_L = O.predictor_logits(X[tokens], inp["w_p1"], inp["w_p2"], inp["bias"])
    bufs = layer.buffers(1)
    for i, t in enumerate(tokens):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=L.PI_RUN_KERNELS)
        torch.cuda.synchronize()
        _check_placed(layer, perm, bufs, 0, ref_L[i], W, X[t], cfg.F, f"c2 t={t}")
    # the placement's purpose: the calibration counts are spread evenly over the tiles
    sums = counts[perm].astype(np.int64).reshape(-1, 64).sum(1)
    assert sums.max() - sums.min() <= counts.max()


def test_placed_union_tiny():
    """A placed layer on the batch path: every token's set through the neuron table and its
    y against the oracle."""
    cfg = configs.tiny("relu", "f16", d=384, F=1000, r=40, B=7, T=2, seed=44)
    say(f"[gpu] placed union {cfg.name}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm, _ = _placement(inp)
    layer = _layer(inp, B_max=cfg.B, perm=perm)
    bufs = layer.buffers(cfg.B)
    for t in range(cfg.T):
        X = inp["x"][t]
        xd = torch.from_numpy(X.copy()).cuda()
        layer.batch_step(xd.data_ptr(), cfg.B, bufs)
        torch.cuda.synchronize()
        ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
        for b in range(cfg.B):
            _check_placed(layer, perm, bufs, b, ref_L[b], W, X[b], cfg.F, f"union t={t} b={b}")


# ----------------------------------------------------------------------------- hot block
def _placement_hot(inp, ncal=64, rate=0.5):
    """pi_place_neurons_hot from a profiling run of the unplaced layer on calibration tokens."""
    import ctypes
    L = _L()
    cfg = inp["cfg"]
    prof = _layer(inp, B_max=L.PI_MAX_BATCH)
    cal = torch.from_numpy(gen.calibration_x(cfg, ncal)).cuda()
    counts = prof.activation_counts(cal)
    perm = np.empty(cfg.F, np.int32)
    nh = ctypes.c_int32(0)
    L.check(L.pi_place_neurons_hot(counts.ctypes.data, cfg.F, ncal, rate, perm.ctypes.data, nh))
    return perm, nh.value, counts


HOT_TINY = [
    configs.tiny("relu", "f16", d=384, F=1000, r=40, seed=61, mean_rate=0.25),
    configs.tiny("reglu", "i4g128", d=384, F=1000, r=40, seed=62, mean_rate=0.25),
    configs.tiny("reglu", "f16", d=1032, F=2000, r=48, seed=63, mean_rate=0.25),
    configs.tiny("reglu", "i4g128", d=2176, F=1000, r=40, seed=64, mean_rate=0.3),
]


@pytest.mark.parametrize("mode", ["split", "kernels", "fused"])
@pytest.mark.parametrize("cfg", HOT_TINY, ids=lambda c: c.name)
def test_hot_block_decode_tiny(cfg, mode):
    """A layer with a hot block (its hot neurons computed densely, before the predictor's
    decision, in the split schedule): every token as a one-step run against the oracle of the
    original layer through the neuron table, then a 40-step run that must end bit-identical to
    a one-step run of its last token.  The fused schedule ignores the hot block."""
    L = _L()
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm, nhot, counts = _placement_hot(inp)
    say(f"[gpu] hot block decode {mode} {cfg.name}: nhot={nhot}")
    assert 0 < nhot < cfg.F
    layer = _layer(inp, replicas=2, perm=perm, nhot=nhot)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    m = {"split": L.PI_RUN_SPLIT, "kernels": L.PI_RUN_KERNELS, "fused": L.PI_RUN_FUSED}[mode]
    bufs = layer.buffers(1)
    for t in range(cfg.T):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=m)
        torch.cuda.synchronize()
        _check_placed(layer, perm, bufs, 0, ref_L[t], W, X[t], cfg.F, f"{cfg.name} hot {mode} t={t}")
    ref = layer.buffers(1)
    layer.decode_run(xd.data_ptr(), cfg.T, 1, 40, bufs, mode=m)
    layer.decode_run(xd.data_ptr(), cfg.T, 40, 1, ref, mode=m)
    torch.cuda.synchronize()
    assert torch.equal(bufs["y"], ref["y"]) and torch.equal(bufs["mask"], ref["mask"])


@pytest.mark.parametrize("name,rate", [("c2", 0.85), ("c5", 0.7)])
def test_hot_block_decode_full(name, rate):
    """The LLaMA-7B- and LLaMA-70B-shaped layers with a hot block from 256 calibration tokens,
    in the default kernel schedule (split, since the layer has a hot block), on sampled
    tokens; the hot block holds the neurons the profile saw firing on >= rate of the tokens."""
    L = _L()
    cfg = configs.get(name)
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm, nhot, counts = _placement_hot(inp, ncal=256, rate=rate)
    say(f"[gpu] hot block decode {cfg.name}: nhot={nhot}")
    assert nhot > 300
    layer = _layer(inp, replicas=2, perm=perm, nhot=nhot)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).cuda()
    tokens = [0, cfg.T // 2, cfg.T - 1]
    ref_L = O.predictor_logits(X[tokens], inp["w_p1"], inp["w_p2"], inp["bias"])
    bufs = layer.buffers(1)
    for i, t in enumerate(tokens):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=L.PI_RUN_KERNELS)
        torch.cuda.synchronize()
        _check_placed(layer, perm, bufs, 0, ref_L[i], W, X[t], cfg.F, f"{name} hot t={t}")
