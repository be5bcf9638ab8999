"""Benchmark of the predictor-gated sparse FFN decode step on one MI355X.

One step = one batch-1 decode token through the whole hot path of one FFN
layer: predictor stage 1 + stage 2 with fused threshold and neuron-table
compaction (pi_predict), the row operator over the active up/gate rows
(pi_ffn_up) and the column operator over the active down rows (pi_ffn_down).
Tokens are consumed strictly one after another (no batching across tokens).

Default workload: the LLaMA-7B-shaped ReGLU layer (d=4096, ffn=11008, predictor
rank 256, fp16 weights, fp32 accumulation, Zipf(1.2) rates with a 5% hot set,
~10% active, 256-token stream).  Weights are held in R byte-identical replicas
and token s uses replica s mod R, standing in for the distinct layers of a real
model: the touched bytes of consecutive steps never share cache lines, so they
come from HBM and not from the 256 MB Infinity Cache.

The token loop is captured once in a HIP graph (through torch.cuda.CUDAGraph)
and replayed; inputs are resident in HBM before the timed region starts.
Events around every pi_ffn_up launch inside the graph give the dominant
kernel's average duration; its algorithmic bytes (the active rows, x, the
neuron table and h) over that duration give the roofline fraction.

Prints one JSON line.  --gpus N with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
CACHE_BUST_BYTES = 576e6    # 2 x (256 MB Infinity Cache + 8 x 4 MB L2)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5440)
    ap.add_argument("--warmup", type=int, default=1088)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to bust the caches")
    ap.add_argument("--mode", choices=("native", "graph", "eager"), default="native",
                    help="native: one pi_decode_run call enqueues the timed steps (default); "
                         "graph: torch HIP-graph replay; eager: one Python call per kernel")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget, 0 = skip")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter scaling runs)")
    return ap.parse_args()


parse_defaults = {"steps": 5440, "warmup": 1088}


# ------------------------------------------------------------------------------- byte accounting
def bytes_model(cfg, n):
    """Algorithmic bytes of one step with n active neurons.

    Whole step: predictor weights 2dr + 2rF, bias 4F, active rows m*n*d*w_b (m = 3 for
    ReGLU, 2 for ReLU; w_b = 2 for fp16, 0.5 + 2/128 for int4 with its scales), x 2d,
    y 4d, the neuron table 4n and the mask F/8.  Per kernel of the fused step:
      A (stage-1 partials): 2dr + 2d;
      B (stage 2 + up/gate of the active rows): 2rF + 4F + (m-1)*n*d*w_b + 2d + F/8 + 4n;
      C (down from the mask, neuron table): n*d*w_b + F/8 + 4n (h) + 4n (table) + 4d.
    Per kernel of the unfused operators: up = (m-1)*n*d*w_b + 2d + 8n.
    """
    d, F, r = cfg.d, cfg.F, cfg.r
    wb = 2.0 if cfg.wfmt == "f16" else 0.5 + 2.0 / 128.0
    m_up = 2 if cfg.act == "reglu" else 1
    a = 2 * d * r + 2 * d
    b = 2 * r * F + 4 * F + m_up * n * d * wb + 2 * d + F / 8 + 4 * n
    c = n * d * wb + F / 8 + 8 * n + 4 * d
    up = m_up * n * d * wb + 2 * d + 8 * n
    return dict(A=a, B=b, C=c, up=up, total=a + b + c)


def bytes_model_batch(cfg, n_tok, U):
    """Algorithmic bytes of one batch step (B tokens, union size U; n_tok, the per-token
    active counts, is not needed: the step writes no per-token tables).
    Predictor: 2dr + 2rF + 4F + B*2d (x) + B*F/8 (masks).
    Union compaction: B*F/8 + 4U.  Union FFN (the two MFMA kernels): the U gathered rows of
    each matrix, m*U*d*2 (m = 3 for ReGLU, 2 for ReLU), x B*2d, the union table twice 8U,
    the masks B*F/8, H written and read 2*B*U*2, y 4*B*d."""
    d, F, r, B = cfg.d, cfg.F, cfg.r, cfg.B
    m = 3 if cfg.act == "reglu" else 2
    pred = 2 * d * r + 2 * r * F + 4 * F + B * 2 * d + B * F / 8
    comp = B * F / 8 + 4 * U
    ffn = m * U * d * 2 + B * 2 * d + 8 * U + B * F / 8 + 4 * B * U + 4 * B * d
    return dict(pred=pred, compact=comp, ffn=ffn, total=pred + comp + ffn)


def src_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_sparse_pi_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str):
    """HBM bytes per launch from the committed counter summary, if it is still current."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel_key)
    if not ent or ent.get("src_sha") != src_sha():
        return None
    return ent.get("hbm_bytes_per_launch")


def copy_probe(mb, dev):
    """Three plain device copies of mb MiB: the reference dispatches for scaling the
    FETCH_SIZE / WRITE_SIZE counters of the same run."""
    if not mb:
        return
    import torch
    src = torch.empty(mb << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------- CPU baseline
def cpu_baseline(inputs, budget_s):
    import numpy as np

    import oracle.pi_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    W = O.Weights.from_inputs(inputs)
    X = inputs["x"][:, 0, :]
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s and n < X.shape[0] * 4:
        O.token_step(inputs, W, X[n % X.shape[0]])
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} tokens of the same stream (wrapping), one at a time, "
                      f"numpy float64, {dt:.1f} s"}


# ------------------------------------------------------------------------------- batch path
def cpu_baseline_batch(inputs, budget_s):
    import oracle.pi_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    W = O.Weights.from_inputs(inputs)
    X = inputs["x"]                      # [T, B, d]
    T, B = X.shape[0], X.shape[1]
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s and n < T * B:
        O.token_step(inputs, W, X[(n // B) % T, n % B])
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} tokens of step 0 onwards, each through its own predicted "
                      f"neuron list (what the union path computes per token), numpy float64, "
                      f"{dt:.1f} s"}


def bench_batch(a, cfg):
    """Small-batch decode: one step = pi_predict(B, masks only) -> pi_compact(UNION) ->
    pi_sparse_ffn(B) over one batch of B independent tokens (the union FFN runs on MFMA)."""
    import torch

    from activation_sparse_pi_amd.layer import DeviceLayer
    from synth import gen

    dev = torch.device("cuda:0")
    inputs = gen.make(cfg)
    B, T = cfg.B, cfg.T
    K = a.steps if a.steps != parse_defaults["steps"] else 640
    Wm = a.warmup if a.warmup != parse_defaults["warmup"] else 64
    xd = torch.from_numpy(inputs["x"].copy()).to(dev)                    # [T, B, d] in HBM
    probe = bytes_model_batch(cfg, np.full(B, cfg.mean_rate * cfg.F), 0.6 * cfg.F)
    R = a.replicas or max(2, math.ceil(CACHE_BUST_BYTES / probe["total"]))
    layer = DeviceLayer(inputs, replicas=R, B_max=B, device=dev)
    bufs = layer.buffers(B)
    # per-step active counts and union sizes (replicas are identical)
    n_tok = np.zeros((T, B)); U = np.zeros(T)
    for t in range(T):
        layer.batch_step(xd[t].data_ptr(), B, bufs, logits=False)
        n_tok[t] = bufs["count"][:B].cpu().numpy()
        U[t] = int(bufs["ucount"][0].item())

    def step(s, ev=None):
        t, rep = s % T, s % R
        xp = xd[t].data_ptr()
        # masks only: the union FFN needs the per-token masks and their union list
        layer.predict(xp, B, None, bufs["mask"].data_ptr(), None, None, rep)
        layer.compact(bufs["mask"].data_ptr(), B, 1, bufs["uidx"].data_ptr(), bufs["ucount"].data_ptr())
        if ev is not None:
            ev[0].record()
        layer.sparse_ffn(xp, B, bufs["uidx"].data_ptr(), bufs["ucount"].data_ptr(),
                         bufs["mask"].data_ptr(), bufs["y"].data_ptr(), rep)
        if ev is not None:
            ev[1].record()

    for s in range(Wm):
        step(s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(K):
        step(Wm + s, ev[s])
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ffn_ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    steps = (Wm + np.arange(K)) % T
    ffn_bytes = float(np.mean([bytes_model_batch(cfg, n_tok[t], U[t])["ffn"] for t in steps]))
    path_bytes = float(np.mean([bytes_model_batch(cfg, n_tok[t], U[t])["total"] for t in steps]))
    ms_per_step = total_ms / K
    achieved = ffn_bytes / (float(ffn_ms.mean()) * 1e-3) / 1e9
    path_gbs = path_bytes / (ms_per_step * 1e-3) / 1e9
    kernel_key = f"k_union_up[{cfg.act}] + k_union_down {cfg.name}"
    copy_probe(a.copy_probe_mb, dev)
    out = {
        "metric": f"sparse-FFN decode tokens/sec at batch {B} (union path) + effective HBM GB/s (% of peak)",
        "value": round(K * B / (total_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one FFN layer, d={cfg.d}, ffn={cfg.F}, {cfg.act}, fp16 weights, "
                        f"fp32 accumulate, predictor rank {cfg.r}, batch {B} independent tokens per "
                        f"step, {T}-step stream, union FFN on MFMA",
            "batch": B, "d": cfg.d, "ffn": cfg.F, "rank": cfg.r, "replicas": R,
            "mean_active_per_token": round(float(n_tok.mean()), 1),
            "mean_union": round(float(U.mean()), 1),
            "launch": "three ABI calls per step from Python (pi_predict, pi_compact, pi_sparse_ffn)",
        },
        "effective_hbm": {"GB/s": round(path_gbs, 1), "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_step": round(path_bytes)},
        "roofline": {
            "bound": "hbm", "kernel": kernel_key,
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profiles(kernel_key),
            "avg_us": round(float(ffn_ms.mean()) * 1e3, 3),
            "bytes_per_launch": round(ffn_bytes),
            "mfma_tflops": round((3 if cfg.act == "reglu" else 2) * 2 * B * U[steps].mean() * cfg.d
                                 / (float(ffn_ms.mean()) * 1e-3) / 1e12, 1),
        },
    }
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline_batch(inputs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------------------- main
def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "the sparse FFN layer is not sharded in this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from activation_sparse_pi_amd.layer import DeviceLayer
    from synth import configs, gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = configs.get(a.config)
    if cfg.B != 1:
        return bench_batch(a, cfg)
    dev = torch.device("cuda:0")
    inputs = gen.make(cfg)
    probe = bytes_model(cfg, cfg.mean_rate * cfg.F)
    R = a.replicas or max(2, math.ceil(CACHE_BUST_BYTES / probe["total"]))
    layer = DeviceLayer(inputs, replicas=R, device=dev)
    T = cfg.T
    xd = torch.from_numpy(inputs["x"][:, 0, :].copy()).to(dev)     # [T, d] resident in HBM
    bufs = layer.buffers(1)
    mask, idx, cnt, h, y = (bufs[k].data_ptr() for k in ("mask", "idx", "count", "h", "y"))

    # active count of every token (replicas are identical, so token t always gives n_t)
    counts = np.zeros(T, dtype=np.int64)
    for t in range(T):
        layer.predict(xd[t].data_ptr(), 1, None, mask, idx, cnt)
        counts[t] = int(bufs["count"][0].item())

    L = R * math.ceil(T / R)            # graph length: whole replica cycles, phase-continuous

    def step(s, ev=None):
        t, rep = s % T, s % R
        xp = xd[t].data_ptr()
        layer.predict(xp, 1, None, mask, idx, cnt, rep)
        if ev is not None:
            ev[0].record()
        layer.ffn_up(xp, idx, cnt, h, rep)
        if ev is not None:
            ev[1].record()
        layer.ffn_down(idx, cnt, h, y, rep)

    K, Wm = a.steps, a.warmup
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if a.mode == "native":
        # timed region: one native call enqueues all K fused steps; the stage-2 + up kernel
        # of every step (the one that moves the most bytes) carries its own start/end events
        ev_up = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
        for e in ev_up:                        # materialise the events before handing them over
            e.record()
        layer.decode_run(xd.data_ptr(), T, 0, Wm, bufs)          # untimed warmup
        torch.cuda.synchronize()
        t0.record()
        layer.decode_run(xd.data_ptr(), T, Wm, K, bufs, events=ev_up)
        t1.record()
        torch.cuda.synchronize()
        up_ms = [ev_up[2 * i].elapsed_time(ev_up[2 * i + 1]) for i in range(K)]
        ev_steps = timed_steps = [Wm + i for i in range(K)]
    elif a.mode == "eager":
        for s in range(Wm):
            step(s)
        ev_up = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(K)]
        torch.cuda.synchronize()
        t0.record()
        for s in range(K):
            step(Wm + s, ev_up[s])
        t1.record()
        torch.cuda.synchronize()
        up_ms = [e0.elapsed_time(e1) for e0, e1 in ev_up]
        ev_steps = timed_steps = [Wm + s for s in range(K)]
    else:                                       # graph: whole-step throughput only
        for s in range(Wm):
            step(s)
        nfull, tail = divmod(K, L)
        s_cap = torch.cuda.Stream(dev)
        s_cap.wait_stream(torch.cuda.current_stream(dev))
        graphs = []
        with torch.cuda.stream(s_cap):
            for length in (L, tail):
                g = None
                if length:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s_cap):
                        for s in range(length):
                            step(Wm + s)
                graphs.append(g)
        torch.cuda.current_stream(dev).wait_stream(s_cap)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(nfull):
            graphs[0].replay()
        if tail:
            graphs[1].replay()
        t1.record()
        torch.cuda.synchronize()
        up_ms = []
        ev_steps = []
        timed_steps = [Wm + s for s in range(L)] * nfull + [Wm + s for s in range(tail)]
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / K
    tok_s = K / (total_ms / 1e3)

    dom = "B" if a.mode == "native" else "up"
    if up_ms:
        n_ev = counts[np.array(ev_steps) % T].astype(np.float64)
        up_bytes = float(np.mean(bytes_model(cfg, n_ev)[dom]))
        up_avg_ms = float(np.mean(up_ms))
        achieved = up_bytes / (up_avg_ms * 1e-3) / 1e9
    else:
        up_bytes = up_avg_ms = achieved = float("nan")
    n_all = counts[np.array(timed_steps) % T]
    path_bytes = float(np.mean(bytes_model(cfg, n_all.astype(np.float64))["total"]))
    path_gbs = path_bytes / (ms_per_step * 1e-3) / 1e9

    kernel_key = (f"k_dec_stage2_up[{cfg.wfmt},{cfg.act}] {cfg.name}" if dom == "B"
                  else f"k_up_{cfg.wfmt}[{cfg.act}] {cfg.name}")
    traffic = traffic_from_profiles(kernel_key)

    copy_probe(a.copy_probe_mb, dev)

    out = {
        "metric": "sparse-FFN decode tokens/sec at batch 1 + effective HBM GB/s (% of peak)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg.wfmt == "f16" else "int4-g128",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one FFN layer, d={cfg.d}, ffn={cfg.F}, {cfg.act}, "
                        f"{cfg.wfmt} weights, fp32 accumulate, predictor rank {cfg.r}, batch 1, "
                        f"{T}-token stream",
            "batch": 1, "d": cfg.d, "ffn": cfg.F, "rank": cfg.r, "replicas": R,
            "mean_active": round(float(counts.mean()), 1),
            "launch": {"native": "one pi_decode_run call (native loop, events on the up kernel)",
                       "graph": f"torch HIP graph of {L} steps, replayed",
                       "eager": "one Python call per ABI function"}[a.mode],
        },
        "effective_hbm": {"GB/s": round(path_gbs, 1), "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_step": round(path_bytes)},
        "roofline": {
            "bound": "hbm", "kernel": kernel_key,
            "achieved": None if math.isnan(achieved) else round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": None if math.isnan(achieved) else round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_us": None if math.isnan(up_avg_ms) else round(up_avg_ms * 1e3, 3),
            "bytes_per_launch": None if math.isnan(up_bytes) else round(up_bytes),
        },
    }
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inputs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
