"""pi_decode_run_noalloc (static scratch, no workspace) against pi_decode_run (needs an MI355X).

Two calls in a row through the C ABI -- a larger layer, then a smaller one that reuses the
scratch the first left behind -- must give what pi_decode_run gives with its own workspace,
bit for bit (the same kernels in the same order): the last step's mask, neuron table, count and
y, for the fused and the split schedule.  The decode path itself is checked against the oracle
in the parity tests.
"""
import sys

import numpy as np
import pytest

from synth import configs, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _layer(inputs, **kw):
    from activation_sparse_pi_amd.layer import DeviceLayer
    return DeviceLayer(inputs, **kw)


LAYERS = [
    configs.C2,                                                              # 2.9 MB of scratch (fused)
    configs.tiny("relu", "i4g128", d=384, F=1000, r=40, T=5, seed=31),      # then a smaller layer
]


@pytest.mark.parametrize("mode_name", ["fused", "split"])
def test_noalloc_matches_workspace_run(mode_name):
    from activation_sparse_pi_amd import _lib as L
    mode = {"fused": L.PI_RUN_FUSED, "split": L.PI_RUN_SPLIT}[mode_name]
    for cfg in LAYERS:
        say(f"[gpu] noalloc {mode_name} on {cfg.name}")
        inp = gen.make(cfg)
        layer = _layer(inp, replicas=2)
        xd = torch.from_numpy(inp["x"][:, 0, :].copy()).to(layer.device)
        s0, n = 3, 6
        ref, out = layer.buffers(1), layer.buffers(1)
        for b in (ref, out):
            for k in ("mask", "idx", "count"):
                b[k].fill_(-7)
            b["y"].fill_(float("nan"))
        layer.decode_run(xd.data_ptr(), cfg.T, s0, n, ref, mode=mode)
        layer.decode_run_noalloc(xd.data_ptr(), cfg.T, s0, n, out, mode=mode)
        torch.cuda.synchronize()
        c = int(ref["count"][0].item())
        assert c >= 0 and int(out["count"][0].item()) == c, (cfg.name, mode_name, "count")
        assert torch.equal(out["idx"][0, :c], ref["idx"][0, :c]), (cfg.name, mode_name, "table")
        assert torch.equal(out["mask"], ref["mask"]), (cfg.name, mode_name, "mask")
        assert torch.equal(out["y"], ref["y"]), (cfg.name, mode_name, "y")
        assert bool(torch.isfinite(out["y"]).all())
        say(f"  {cfg.name} {mode_name}: n={c}, y identical")
