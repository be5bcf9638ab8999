"""The union FFN with more 32-neuron tiles than up-kernel blocks resident at once (MI355X).

On this chip the ReLU up kernel holds 512 blocks at once and the ReGLU one 256.  When a layer
has more tiles than that, every tile past the resident ones is split over d into two parts whose
partial pre-activations the last-arriving part adds in part order.  The shapes below (B = 32
tokens at rate 0.2: the union is ~90% of F) land at

    ReLU  d=200  F=18000: 521 tiles (9 split)      d=1032 F=21000: 611 (99 split)
    ReLU  d=200  F=30000: 851 tiles (339 split)
    ReGLU d=200  F=10000: 293 tiles (37 split)     d=1032 F=12504: 362 (106 split)

and the layers' F also leaves whole-tile blocks past the union.  d = 200 is 3 runs of 64 plus
8: the first part holds one run, the last two and the ragged one.  Both entries are checked:
pi_batch_run (the list built from the union mask) and the operators pi_predict / pi_compact /
pi_sparse_ffn (the list given).  Every token's index set and y against the oracle (y over the
token's own list), and the union list against the OR of the token masks.
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
    configs.tiny("relu", "f16", d=200, F=18000, r=40, B=32, T=1, seed=81),
    configs.tiny("relu", "f16", d=1032, F=21000, r=40, B=32, T=1, seed=82),
    configs.tiny("relu", "f16", d=200, F=30000, r=40, B=32, T=1, seed=83),
    configs.tiny("reglu", "f16", d=200, F=10000, r=40, B=32, T=1, seed=84),
    configs.tiny("reglu", "f16", d=1032, F=12504, r=48, B=32, T=1, seed=85),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_union_split_tiles(cfg):
    from activation_sparse_pi_amd import _lib as L
    from activation_sparse_pi_amd.layer import DeviceLayer
    inp = gen.make(cfg)
    W = O.Weights.from_inputs(inp)
    X = inp["x"][0]                                                    # [B, d]
    B, F = cfg.B, cfg.F
    ref_L = O.predictor_logits(X, inp["w_p1"], inp["w_p2"], inp["bias"])
    layer = DeviceLayer(inp, replicas=1, B_max=B)
    xd = torch.from_numpy(np.ascontiguousarray(inp["x"])).cuda()      # [1, B, d]
    Wd = (F + 31) // 32

    # pi_batch_run, union schedule
    mask = torch.full((B, Wd), -1, dtype=torch.int32, device="cuda")
    y = torch.full((B, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    layer.batch_run(xd.data_ptr(), 1, B, 0, 1, mask.data_ptr(), y.data_ptr(), schedule=L.PI_BATCH_UNION)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().view(np.uint32)
    yr = y.cpu().numpy().astype(np.float64)
    act = np.zeros((B, F), bool)
    for b in range(B):
        act[b] = O.words_to_active(m[b], F)
    U = int(act.any(axis=0).sum())
    say(f"[gpu] {cfg.name}: union {U}, {(U + 31) // 32} tiles")
    worst = 0.0
    for b in range(B):
        idx = np.flatnonzero(act[b])
        P.check_index_set(idx, m[b], ref_L[b], F, ctx=f"{cfg.name} run b={b}")
        worst = max(worst, P.check_ffn(yr[b], W, X[b], idx, ctx=f"{cfg.name} run b={b}"))
    say(f"  pi_batch_run worst rel-L2 {worst:.2e}")

    # the operators: the union list is given to the FFN
    bufs = layer.buffers(B)
    layer.batch_step(xd[0].data_ptr(), B, bufs)
    torch.cuda.synchronize()
    un = int(bufs["ucount"][0].item())
    uidx = bufs["uidx"][:un].cpu().numpy().astype(np.int64)
    m2 = bufs["mask"][:B].cpu().numpy().view(np.uint32)
    assert np.array_equal(m2, m), "operators and pi_batch_run disagree on the masks"
    assert np.array_equal(uidx, O.compact(O.union_active(act))), "union list"
    y2 = bufs["y"][:B].cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(B):
        worst = max(worst, P.check_ffn(y2[b], W, X[b], np.flatnonzero(act[b]), ctx=f"{cfg.name} ops b={b}"))
    say(f"  operators worst rel-L2 {worst:.2e}")
