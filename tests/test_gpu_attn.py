"""The attention side (head predictor, pi_attn_qkv, pi_attn_out) against the oracle, through the
C ABI (needs an MI355X).

Per token: pi_predict with one output per head gives the head mask and the ascending head
table; the head set must equal the oracle's outside the 1e-4 band (bit-exact otherwise), and
the mask must be the bitmask of the table.  pi_attn_qkv: every listed head's q, k, v against
the oracle (rel-L2 <= 1e-3 over the listed heads; fp32 accumulation of fp16 products), every
other head exactly 0.  pi_attn_out: y against the oracle's projection over the GPU's own head
table (rel-L2 <= 1e-3).  Shapes: ragged tiny layers (d not a multiple of 64 or 512, head widths
not a multiple of 8 rows per block), a layer where every head fires (= the dense projections),
one where none does (exact zeros, also right after a call with heads), and the LLaMA-7B and
OPT-30B attention shapes.  Two runs of a token are bitwise identical.
"""
import sys

import numpy as np
import pytest

from synth import attn as SA

from . import _parity as P
import oracle.attn_oracle as A

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev_attn(inp, **kw):
    from activation_sparse_pi_amd.layer import DeviceAttn
    return DeviceAttn(inp, **kw)


def _step(att, xd, od, bufs):
    att.predict(xd.data_ptr(), bufs)
    att.qkv(xd.data_ptr(), bufs)
    att.out(od.data_ptr(), bufs)
    torch.cuda.synchronize()
    n = int(bufs["count"][0].item())
    return dict(logits=bufs["logits"].cpu().numpy().astype(np.float64),
                heads=bufs["idx"][:n].cpu().numpy().astype(np.int64),
                mask=bufs["mask"].cpu().numpy().view(np.uint32).copy(),
                qkv=bufs["qkv"].cpu().numpy().astype(np.float64), y=bufs["y"].cpu().numpy().astype(np.float64))


def _check(inp, g, x, o, ctx):
    cfg = inp["cfg"]
    ref_L = A.head_logits(x, inp["w_a1"], inp["w_a2"], inp["bias_a"])
    assert np.max(np.abs(g["logits"] - ref_L)) < 5e-5, f"{ctx}: logits"
    P.check_index_set(g["heads"], g["mask"], ref_L, cfg.H, ctx=ctx)
    heads = g["heads"]
    ref_qkv = A.qkv_heads(inp["w_qkv"], x, heads)
    off = np.setdiff1d(np.arange(cfg.H), heads)
    assert np.array_equal(g["qkv"][off], np.zeros_like(g["qkv"][off])), f"{ctx}: unlisted heads not 0"
    eq = P.rel_l2(g["qkv"][heads], ref_qkv[heads]) if heads.size else 0.0
    assert eq <= P.REL_TOL, f"{ctx}: qkv rel-L2 {eq:.3e}"
    ref_y = A.out_heads(inp["w_o"], o, heads)
    if heads.size == 0:
        assert np.array_equal(g["y"], np.zeros(cfg.d)), f"{ctx}: y of no head must be 0"
        ey = 0.0
    else:
        ey = P.rel_l2(g["y"], ref_y)
    assert ey <= P.REL_TOL, f"{ctx}: y rel-L2 {ey:.3e}"
    return eq, ey, heads.size


TINY = [
    SA.tiny(d=200, H=8, dh=24, r=16, T=4, seed=41),
    SA.tiny(d=1032, H=16, dh=40, r=24, T=4, seed=42),
    SA.tiny(d=520, H=24, dh=3, r=8, T=4, seed=43, mean_rate=0.3),
    SA.tiny(d=8, H=8, dh=1, r=8, T=3, seed=44),
]


@pytest.mark.parametrize("cfg", TINY, ids=lambda c: c.name)
def test_attn_tiny(cfg):
    inp = SA.make(cfg)
    att = _dev_attn(inp)
    bufs = att.buffers()
    xd = torch.from_numpy(inp["x"].copy()).cuda()
    od = torch.from_numpy(inp["o"].copy()).cuda()
    for t in range(cfg.T):
        g = _step(att, xd[t], od[t], bufs)
        eq, ey, n = _check(inp, g, inp["x"][t], inp["o"][t], f"{cfg.name} t={t}")
        say(f"[gpu] {cfg.name} t={t}: {n}/{cfg.H} heads, qkv {eq:.2e}, y {ey:.2e}")
    g2 = _step(att, xd[cfg.T - 1], od[cfg.T - 1], bufs)
    assert np.array_equal(g2["qkv"], g["qkv"]) and np.array_equal(g2["y"], g["y"]), "not reproducible"


@pytest.mark.parametrize("which", ["all", "none"])
def test_attn_all_or_no_heads(which):
    """Every head firing gives the dense projections; none firing gives exact zeros, also on a
    workspace that just served a call with heads."""
    cfg = SA.tiny(d=264, H=16, dh=16, r=16, T=2, seed=45)
    inp = SA.make(cfg)
    base = dict(inp)
    shifted = dict(inp, bias_a=inp["bias_a"] + np.float32(1e3 if which == "all" else -1e3))
    att0 = _dev_attn(base)
    att = _dev_attn(shifted)
    att.ws = att0.ws                                       # the same workspace for both layers
    att.ws_bytes = min(att.ws_bytes, att0.ws_bytes)
    bufs = att.buffers()
    xd = torch.from_numpy(inp["x"].copy()).cuda()
    od = torch.from_numpy(inp["o"].copy()).cuda()
    _step(att0, xd[0], od[0], bufs)                        # some heads: fills the workspace
    g = _step(att, xd[1], od[1], bufs)
    x, o = inp["x"][1], inp["o"][1]
    if which == "all":
        assert list(g["heads"]) == list(range(cfg.H))
        assert P.rel_l2(g["qkv"], A.qkv_dense(inp["w_qkv"], x)) <= P.REL_TOL
        assert P.rel_l2(g["y"], A.out_dense(inp["w_o"], o)) <= P.REL_TOL
    else:
        assert g["heads"].size == 0 and not g["mask"].any()
        assert np.array_equal(g["qkv"], np.zeros_like(g["qkv"])) and np.array_equal(g["y"], np.zeros(cfg.d))


@pytest.mark.parametrize("name,steps", [("a2", 8), ("a3", 4)])
def test_attn_model_shapes(name, steps):
    cfg = SA.get(name).with_(T=steps)
    inp = SA.make(cfg)
    att = _dev_attn(inp)
    bufs = att.buffers()
    xd = torch.from_numpy(inp["x"].copy()).cuda()
    od = torch.from_numpy(inp["o"].copy()).cuda()
    for t in range(cfg.T):
        g = _step(att, xd[t], od[t], bufs)
        eq, ey, n = _check(inp, g, inp["x"][t], inp["o"][t], f"{cfg.name} t={t}")
        say(f"[gpu] {cfg.name} t={t}: {n}/{cfg.H} heads, qkv {eq:.2e}, y {ey:.2e}")


RUN = [
    TINY[1],
    SA.tiny(d=264, H=40, dh=8, r=16, T=4, seed=48),    # two mask words, logits folded into q/k/v
    SA.tiny(d=200, H=72, dh=4, r=16, T=3, seed=49),    # H > 64: pi_predict, then the q/k/v kernel
    SA.get("a2").with_(T=6),
    SA.get("a3").with_(T=4),
]


@pytest.mark.parametrize("cfg", RUN, ids=lambda c: c.name)
def test_attn_run(cfg):
    """pi_attn_run over several tokens and two replicas: the last step's outputs equal a one-step
    run of that token bit for bit, and the oracle's (up to H = 64 the step computes the heads'
    logits inside its q/k/v kernel, above that through pi_predict)."""
    inp = SA.make(cfg)
    att = _dev_attn(inp, replicas=2)
    xd = torch.from_numpy(inp["x"].copy()).cuda()
    od = torch.from_numpy(inp["o"].copy()).cuda()
    b1, b2 = att.buffers(), att.buffers()
    n = 2 * cfg.T + 1                                   # ends on token (n - 1) % T, replica 0
    att.run(xd.data_ptr(), od.data_ptr(), cfg.T, 0, n, b1)
    att.run(xd.data_ptr(), od.data_ptr(), cfg.T, n - 1, 1, b2)
    torch.cuda.synchronize()
    for k in ("mask", "idx", "count", "qkv", "y"):
        c = int(b1["count"][0].item())
        a1, a2 = b1[k].cpu().numpy(), b2[k].cpu().numpy()
        if k == "idx":
            a1, a2 = a1[:c], a2[:c]
        assert np.array_equal(a1, a2), f"{cfg.name}: {k} differs between the long and the one-step run"
    t = (n - 1) % cfg.T
    c = int(b1["count"][0].item())
    g = dict(logits=A.head_logits(inp["x"][t], inp["w_a1"], inp["w_a2"], inp["bias_a"]),
             heads=b1["idx"][:c].cpu().numpy().astype(np.int64),
             mask=b1["mask"].cpu().numpy().view(np.uint32), qkv=b1["qkv"].cpu().numpy().astype(np.float64),
             y=b1["y"].cpu().numpy().astype(np.float64))
    eq, ey, nh = _check(inp, g, inp["x"][t], inp["o"][t], f"{cfg.name} run")
    say(f"[gpu] {cfg.name} pi_attn_run: {nh} heads, qkv {eq:.2e}, y {ey:.2e}")


ONE_TILE = [
    SA.tiny(d=16384, H=64, dh=1, r=1000, T=3, seed=45, mean_rate=0.4),   # two row segments, 250 blocks
    SA.tiny(d=4104, H=40, dh=2, r=8, T=3, seed=46),                      # two blocks, F past one word
    SA.tiny(d=264, H=64, dh=1, r=64, T=3, seed=47, mean_rate=0.9),
]


@pytest.mark.parametrize("cfg", ONE_TILE, ids=lambda c: c.name)
def test_head_predictor_one_tile(cfg):
    """pi_predict at one token and F <= 64 (one launch, logits summed from per-block partial rows
    by the last block): logits within 5e-5 of the oracle's fp64 logits, the head set equal to the
    oracle's outside the band, the mask the bitmask of the table; every call of a token gives the
    same bits (the arrival counter resets itself), with or without the logits output."""
    say(f"[gpu] one-tile predictor {cfg.name}")
    inp = SA.make(cfg)
    att = _dev_attn(inp)
    xd = torch.from_numpy(inp["x"].copy()).to(att.device)
    first = None
    for rnd in range(2):
        for t in range(cfg.T):
            bufs = att.buffers()
            att.predict(xd[t].data_ptr(), bufs, logits=(rnd == 0))
            torch.cuda.synchronize()
            n = int(bufs["count"][0].item())
            heads = bufs["idx"][:n].cpu().numpy().astype(np.int64)
            mask = bufs["mask"].cpu().numpy().view(np.uint32).copy()
            ref_L = A.head_logits(inp["x"][t], inp["w_a1"], inp["w_a2"], inp["bias_a"])
            if rnd == 0:
                lg = bufs["logits"].cpu().numpy().astype(np.float64)
                assert np.max(np.abs(lg - ref_L)) < 5e-5, f"{cfg.name} t={t}: logits"
                P.check_index_set(heads, mask, ref_L, cfg.H, ctx=f"{cfg.name} t={t}")
                first = first or {}
                first[t] = (heads, mask)
            else:
                assert np.array_equal(heads, first[t][0]) and np.array_equal(mask, first[t][1]), \
                    f"{cfg.name} t={t}: a second call differs"
