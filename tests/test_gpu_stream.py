"""The benchmarked paths over whole token streams, as bench.py runs them (needs an MI355X).

* c2, c3 and c5 through pi_decode_run in its kernel schedule (two kernels per step on c2, three
  on c3 and c5) with the bench's replica count: every token of the stream as a one-step run
  (token t on replica t mod R) -- its index set against the oracle outside the 1e-4 band, its
  mask equal to the bitmask of its table, its y against the oracle's FFN over its own table
  (every token on c2, every fourth on c3, every sixteenth on c5, whose int4 oracle takes
  seconds a token) -- and then one run over the whole stream that must end bit-identical to the
  one-step run of its last token.  Every layer also as the bench times it, with the neurons
  dealt over the tiles (placed): every token's set mapped back to original ids against the
  oracle, and y with the table from pi_map_ids on sampled tokens.
* c4 through pi_batch_run's union schedule at B = 32: every step of the 64-step stream as a
  one-step run, all 32 tokens' index sets against the oracle, y for one token every other step
  (a different slot b each time).
* a2 and a3 (the attention side) through pi_attn_run with the bench's replica count: every
  token of the stream as a one-step run -- its head set against the oracle outside the band,
  the mask equal to the table's bitmask, q/k/v of the listed heads and y against the oracle
  over the GPU's own head table -- and a run over the stream that must end bit-identical to
  the one-step run of its last token.
"""
import math
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


def _replicas(cfg):
    import bench
    return max(2, math.ceil(bench.CACHE_BUST_BYTES / bench.bytes_model(cfg, cfg.mean_rate * cfg.F)["total"]))


@pytest.mark.parametrize("name,y_every,placed", [("c2", 1, False), ("c3", 4, False), ("c5", 16, False),
                                                  ("c1", 1, True), ("c2", 4, True), ("c3", 8, True),
                                                  ("c5", 32, True)])
def test_decode_stream(name, y_every, placed):
    """placed: the layer as the bench times it -- neurons dealt over the tiles from 256
    calibration tokens -- checked through its neuron table against the oracle of the original
    layer."""
    from activation_sparse_pi_amd import _lib as L
    from activation_sparse_pi_amd.layer import DeviceLayer
    from .test_gpu_place import _check_placed, _placement
    cfg = configs.get(name)
    R = _replicas(cfg)
    say(f"[gpu] stream {cfg.name}: {cfg.T} tokens, {R} replicas{', dealt placement' if placed else ''}")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    perm = _placement(inp, ncal=256)[0] if placed else None
    layer = DeviceLayer(inp, replicas=R, perm=perm)
    X = inp["x"][:, 0, :]
    xd = torch.from_numpy(X.copy()).to(layer.device)
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    bufs = layer.buffers(1)
    worst, band = 0.0, 0
    for t in range(cfg.T):
        layer.decode_run(xd.data_ptr(), cfg.T, t, 1, bufs, mode=L.PI_RUN_KERNELS)
        torch.cuda.synchronize()
        ctx = f"{name} t={t} replica {t % R}"
        if placed:
            if t % y_every == 0:
                worst = max(worst, _check_placed(layer, perm, bufs, 0, ref_L[t], W, X[t], cfg.F, ctx))
            else:                                     # the index set, mapped back on the host
                n = int(bufs["count"][0].item())
                orig = np.sort(perm[bufs["idx"][0, :n].cpu().numpy()].astype(np.int64))
                act = np.zeros(cfg.F, bool)
                act[orig] = True
                band += P.check_index_set(orig, O.mask_words(act), ref_L[t], cfg.F, ctx=ctx)
            continue
        n = int(bufs["count"][0].item())
        idx = bufs["idx"][0, :n].cpu().numpy().astype(np.int64)
        band += P.check_index_set(idx, bufs["mask"][0].cpu().numpy().view(np.uint32), ref_L[t], cfg.F, ctx=ctx)
        if t % y_every == 0:
            worst = max(worst, P.check_ffn(bufs["y"][0].cpu().numpy().astype(np.float64), W, X[t], idx, ctx=ctx))
    say(f"  every token checked: band differences {band}, worst rel-L2 {worst:.2e}")
    # the whole stream in one run ends on the one-step result of its last token
    long, one = layer.buffers(1), layer.buffers(1)
    layer.decode_run(xd.data_ptr(), cfg.T, 0, 2 * cfg.T + 3, long, mode=L.PI_RUN_KERNELS)
    layer.decode_run(xd.data_ptr(), cfg.T, 2 * cfg.T + 2, 1, one, mode=L.PI_RUN_KERNELS)
    torch.cuda.synchronize()
    c = int(one["count"][0].item())
    assert int(long["count"][0].item()) == c
    assert torch.equal(long["idx"][0, :c], one["idx"][0, :c]) and torch.equal(long["mask"], one["mask"])
    assert torch.equal(long["y"], one["y"]), f"{name}: a long run differs from its last one-step run"


def test_batch_stream_c4():
    from activation_sparse_pi_amd import _lib as L
    from activation_sparse_pi_amd.layer import DeviceLayer
    cfg = configs.C4
    B, T = cfg.B, cfg.T
    say(f"[gpu] stream {cfg.name}: {T} steps of {B} tokens")
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    layer = DeviceLayer(inp, replicas=2, B_max=B)
    xd = torch.from_numpy(inp["x"].copy()).to(layer.device)            # [T, B, d]
    Wd = (cfg.F + 31) // 32
    mask = torch.empty((B, Wd), dtype=torch.int32, device=layer.device)
    y = torch.empty((B, cfg.d), dtype=torch.float32, device=layer.device)
    ref_all = O.predictor_logits(inp["x"].reshape(T * B, cfg.d), inp["w_p1"], inp["w_p2"],
                                 inp["bias"]).reshape(T, B, cfg.F)
    worst, band = 0.0, 0
    for t in range(T):
        layer.batch_run(xd.data_ptr(), T, B, t, 1, mask.data_ptr(), y.data_ptr(), schedule=L.PI_BATCH_UNION)
        torch.cuda.synchronize()
        m = mask.cpu().numpy().view(np.uint32)
        yh = y.cpu().numpy().astype(np.float64)
        X = inp["x"][t]
        for b in range(B):
            idx = np.flatnonzero(O.words_to_active(m[b], cfg.F))
            band += P.check_index_set(idx, m[b], ref_all[t, b], cfg.F, ctx=f"c4 t={t} b={b}")
            if t % 2 == 0 and b == (t // 2 * 7) % B:
                worst = max(worst, P.check_ffn(yh[b], W, X[b], idx, ctx=f"c4 t={t} b={b}"))
    say(f"  all {T * B} tokens' sets checked: band differences {band}, worst rel-L2 {worst:.2e}")


@pytest.mark.parametrize("name", ["a2", "a3"])
def test_attn_stream(name):
    import bench
    from synth import attn as SA
    import oracle.attn_oracle as A
    from activation_sparse_pi_amd.layer import DeviceAttn
    cfg = SA.get(name)
    R = max(2, math.ceil(bench.CACHE_BUST_BYTES / bench.bytes_model_attn(cfg, cfg.mean_rate * cfg.H)["total"]))
    say(f"[gpu] attention stream {cfg.name}: {cfg.T} tokens, {R} replicas")
    inp = SA.make(cfg)
    att = DeviceAttn(inp, replicas=R)
    xd = torch.from_numpy(inp["x"].copy()).to(att.device)
    od = torch.from_numpy(inp["o"].copy()).to(att.device)
    ref_L = A.head_logits(inp["x"], inp["w_a1"], inp["w_a2"], inp["bias_a"])
    bufs = att.buffers()
    worst = 0.0
    for t in range(cfg.T):
        att.run(xd.data_ptr(), od.data_ptr(), cfg.T, t, 1, bufs)
        torch.cuda.synchronize()
        n = int(bufs["count"][0].item())
        heads = bufs["idx"][:n].cpu().numpy().astype(np.int64)
        ctx = f"{name} t={t} replica {t % R}"
        P.check_index_set(heads, bufs["mask"].cpu().numpy().view(np.uint32), ref_L[t], cfg.H, ctx=ctx)
        qkv = bufs["qkv"].cpu().numpy().astype(np.float64)
        off = np.setdiff1d(np.arange(cfg.H), heads)
        assert not np.any(qkv[off]), f"{ctx}: unlisted heads not 0"
        if heads.size:
            ref_qkv = A.qkv_heads(inp["w_qkv"], inp["x"][t], heads)
            worst = max(worst, P.rel_l2(qkv[heads], ref_qkv[heads]))
            worst = max(worst, P.rel_l2(bufs["y"].cpu().numpy().astype(np.float64),
                                        A.out_heads(inp["w_o"], inp["o"][t], heads)))
        else:
            assert not np.any(bufs["y"].cpu().numpy()), f"{ctx}: y of no head must be 0"
        assert worst <= P.REL_TOL, f"{ctx}: rel-L2 {worst:.3e}"
    say(f"  every token checked: worst rel-L2 {worst:.2e}")
    long, one = att.buffers(), att.buffers()
    att.run(xd.data_ptr(), od.data_ptr(), cfg.T, 0, 2 * cfg.T + 3, long)
    att.run(xd.data_ptr(), od.data_ptr(), cfg.T, 2 * cfg.T + 2, 1, one)
    torch.cuda.synchronize()
    for k in ("mask", "count", "qkv", "y"):
        assert torch.equal(long[k], one[k]), f"{name}: {k} of a long run differs from its last one-step run"
    c = int(one["count"][0].item())
    assert torch.equal(long["idx"][:c], one["idx"][:c])
