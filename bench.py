"""Benchmark of the predictor-gated sparse FFN decode step on one MI355X.

One step = one batch-1 decode token through the whole hot path of one FFN
layer: predictor stage 1 and stage 2 with the strict threshold, the neuron
table, the row operator over the predicted-active up/gate rows and the column
operator over their down rows.  Tokens are consumed strictly one after another:
a step starts only when the previous step's y is complete (no batching across
tokens).

Default workload: the largest batch-1 layer, LLaMA-70B-shaped ReGLU (d=8192,
ffn=28672, weight-only int4 with one fp16 scale per 128 along d, fp16 predictor of
rank 1024, fp32 accumulation, Zipf(1.2) rates, ~10% active, 128-token stream);
--config c1 / c2 / c3 select the smaller batch-1 layers, c4 the batch-32 one.  Weights are held in R byte-identical replicas
and token s uses replica s mod R, standing in for the distinct layers of a real
model: the touched bytes of consecutive steps never share cache lines, so they
come from HBM and not from the 256 MB Infinity Cache.

Modes (--mode): "kernels" (default) enqueues the K timed steps with one
pi_decode_run call in the kernel schedule the library picks for the shape: "fused"
(two kernels per step, the tile kernel also does the down rows) where
ceil(F/64) * d <= 2^20, else "split" (three kernels per step, the down projection
its own kernel); "fused" and "split" force one of them; "eager" makes one Python call
per ABI function.  Inputs are
resident in HBM before the timed region starts; two events recorded on the library's
stream around the enqueued steps time them.  The roofline figure is the tile kernel
(the one that moves the most bytes): its algorithmic bytes over its average duration,
taken in a second pass over the same stream in which that kernel of every step
carries its own start/end events (those events slow the step down, so the headline
value comes from the first pass, which has none).

Prints one JSON line.  --gpus N with N > 1 exits: the layer runs on one GPU.
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
    ap.add_argument("--config", default="c5", help="c1..c5 (FFN), a2 / a3 (attention side)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to bust the caches")
    ap.add_argument("--mode", choices=("kernels", "fused", "split", "eager"), default="kernels",
                    help="kernels: one pi_decode_run call, the schedule the library picks (default); "
                         "fused / split: one pi_decode_run call in that schedule; "
                         "eager: one Python call per ABI function")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget, 0 = skip")
    ap.add_argument("--placement", choices=("auto", "none", "dealt", "hot"), default="auto",
                    help="dealt: neurons dealt over the 64-neuron tiles by their activation counts "
                         "on calibration tokens (pi_place_neurons); hot: the neurons firing on at "
                         "least --hot-rate of them form a hot block computed without waiting for "
                         "the predictor, the rest dealt (pi_place_neurons_hot); auto (default): "
                         "dealt (it balances the tile kernel's tiles); batch 1 only")
    ap.add_argument("--hot-rate", type=float, default=0.7, help="profiled rate of the hot block")
    ap.add_argument("--calib-tokens", type=int, default=256, help="calibration tokens for --placement")
    ap.add_argument("--pred-format", choices=("f16", "i8g128"), default="f16",
                    help="i8g128: the predictor factors in int8 with one fp16 scale per 128 (batch 1)")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="pi_batch_run per schedule for B = 1, 2, 4, ... up to --batch-max")
    ap.add_argument("--batch-max", type=int, default=0, help="--batch-sweep: largest B (0 = max(batch, 64))")
    ap.add_argument("--passes", type=int, default=5,
                    help="also time this many whole passes over the T-token stream and report "
                         "their median (0 = skip)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter scaling runs)")
    return ap.parse_args()


parse_defaults = {"steps": 5440, "warmup": 1088}


# ------------------------------------------------------------------------------- byte accounting
def bytes_model(cfg, n, pb=2.0):
    """Algorithmic bytes of one batch-1 step with n active neurons: predictor weights
    pb*(dr + rF) (pb = 2 for fp16, 1 + 2/128 for int8 with its scales), bias 4F, the active rows m*n*d*w_b (m = 3 for ReGLU, 2 for ReLU; w_b = 2
    for fp16, 0.5 + 2/128 for int4 with its scales), x 2d, y 4d, the mask F/8 and the
    neuron table 4n.  (The unfused up operator alone: (m-1)*n*d*w_b + 2d + 8n.)"""
    d, F, r = cfg.d, cfg.F, cfg.r
    wb = 2.0 if cfg.wfmt == "f16" else 0.5 + 2.0 / 128.0
    m = 3 if cfg.act == "reglu" else 2
    pred = pb * d * r + pb * r * F + 4 * F
    ffn = m * n * d * wb
    total = pred + ffn + 2 * d + 4 * d + F / 8 + 4 * n
    up = (m - 1) * n * d * wb + 2 * d + 8 * n
    # the tile kernel of the split step: W2t + bias, z, x, the up (and gate) rows of the
    # active neurons, the mask words and h written
    stage2 = pb * r * F + 4 * F + 4 * r + 2 * d + (m - 1) * n * d * wb + F / 8 + 4 * n
    # the tile kernel of the fused step: the same without h, plus the down rows and y
    tile_fused = stage2 - 4 * n + n * d * wb + 4 * d
    return dict(pred=pred, ffn=ffn, up=up, stage2=stage2, tile_fused=tile_fused, total=total)


def kernel_schedule(cfg, nhot=0) -> str:
    """The schedule PI_RUN_KERNELS takes for this shape (documented in include/pi.h): split for a
    layer with a hot block."""
    return "fused" if nhot == 0 and ((cfg.F + 63) // 64) * cfg.d <= (1 << 20) else "split"


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
def cpu_model() -> str:
    """The host CPU's model name as lscpu prints it (falling back to /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpus() -> dict:
    """CPUs the host has, and the ones this process may run on."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"host_cpus": os.cpu_count(), "usable_cpus": usable,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _oracle_rate(inputs, W, X, budget_s, limit):
    import oracle.pi_oracle as O
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s and n < limit:
        O.token_step(inputs, W, X[n % X.shape[0]])
        n += 1
    return n, time.perf_counter() - t0


def cpu_baseline(inputs, budget_s):
    """The oracle on the host: about two thirds of the budget with every BLAS thread, the rest
    with one thread (reported beside it)."""
    import oracle.pi_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    W = O.Weights.from_inputs(inputs)
    X = inputs["x"][:, 0, :]
    n, dt = _oracle_rate(inputs, W, X, budget_s * 2 / 3, X.shape[0] * 4)
    out = {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"first {n} tokens of the same stream (wrapping), one at a time, "
                     f"numpy float64 with its BLAS pool of {threads} threads, {dt:.1f} s",
           "cpu_model": cpu_model(), **host_cpus()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, dt1 = _oracle_rate(inputs, W, X, budget_s / 3, X.shape[0] * 4)
        out["single_thread"] = {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                                "sample": f"first {n1} tokens, one BLAS thread, {dt1:.1f} s"}
    return out


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
                      f"neuron list (what the union path computes per token), numpy float64 with "
                      f"its BLAS pool of {threads} threads, {dt:.1f} s",
            "cpu_model": cpu_model(), **host_cpus()}


def bench_batch(a, cfg):
    """Small-batch decode: one step = the B independent tokens of one batch through the union
    schedule of pi_batch_run (batch predictor with per-token masks and their union, the union's
    neuron table, the union FFN on MFMA where every token gets only its own neurons).  The K
    timed steps are one pi_batch_run call; the roofline comes from a second call with events
    around every step's union FFN (its two kernels)."""
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

    from activation_sparse_pi_amd import _lib as L
    mask_r = torch.empty((B, (cfg.F + 31) // 32), dtype=torch.int32, device=dev)
    y_r = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
    layer.batch_run(xd.data_ptr(), T, B, 0, Wm, mask_r.data_ptr(), y_r.data_ptr(),
                    schedule=L.PI_BATCH_UNION)                                   # untimed warmup
    t01 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    layer.batch_run(xd.data_ptr(), T, B, Wm, K, mask_r.data_ptr(), y_r.data_ptr(),
                    schedule=L.PI_BATCH_UNION, events=t01)                       # timed: K steps
    torch.cuda.synchronize()
    total_ms = t01[0].elapsed_time(t01[1])
    # roofline pass: the same call with events around every step's union FFN
    Kr = min(K, 128)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * Kr)]
    torch.cuda.synchronize()
    layer.batch_run(xd.data_ptr(), T, B, Wm + K, Kr, mask_r.data_ptr(), y_r.data_ptr(),
                    schedule=L.PI_BATCH_UNION, kernel_events=kev)
    torch.cuda.synchronize()
    ffn_ms = np.array([kev[2 * i].elapsed_time(kev[2 * i + 1]) for i in range(Kr)])
    steps = (Wm + np.arange(K)) % T
    rsteps = (Wm + K + np.arange(Kr)) % T
    ffn_bytes = float(np.mean([bytes_model_batch(cfg, n_tok[t], U[t])["ffn"] for t in rsteps]))
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
            "launch": "one pi_batch_run call, union schedule: per step the batch predictor (per-token "
                      "masks and their union), the union's neuron table and the union FFN on MFMA",
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
            "mfma_tflops": round((3 if cfg.act == "reglu" else 2) * 2 * B * U[rsteps].mean() * cfg.d
                                 / (float(ffn_ms.mean()) * 1e-3) / 1e12, 1),
        },
    }
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline_batch(inputs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_batch_sweep(a, cfg):
    """Batch-size dispatch on a layer of the workload's shape: for B = 1, 2, 4, ... up to
    --batch-max, one decode step of B tokens (predictor, tables, FFN) through pi_batch_run with
    each schedule -- token by token on the batch-1 kernel schedule, union passes of at most 32
    tokens on MFMA, and the automatic choice -- next to pi_batch_plan's FFN estimates.  The
    schedule the automatic choice ran is read off its y, which equals bit for bit the y of the
    schedule it took (each schedule sums in a fixed order).  The activation rates it decides on
    are the predicted masks' rates over the sampled steps."""
    import torch

    from activation_sparse_pi_amd import _lib as L
    from activation_sparse_pi_amd.layer import DeviceLayer
    from synth import gen

    dev = torch.device("cuda:0")
    Bmax = a.batch_max or max(cfg.B, 64)
    S = 16                                                # distinct steps cycled through
    cfg = cfg.with_(B=Bmax, T=S)
    inputs = gen.make(cfg)
    F, W = cfg.F, (cfg.F + 31) // 32
    R = a.replicas or 2
    layer = DeviceLayer(inputs, replicas=R, B_max=min(Bmax, 32), device=dev)
    xall = torch.from_numpy(inputs["x"].copy()).to(dev)                  # [S, Bmax, d]
    # activation rates from the predicted masks (batches of at most 32 tokens)
    m = torch.empty((32, W), dtype=torch.int32, device=dev)
    hits = np.zeros(F)
    ntok = 0
    for t in range(S):
        for b0 in range(0, Bmax, 32):
            nb = min(32, Bmax - b0)
            layer.predict(xall[t, b0].data_ptr(), nb, None, m.data_ptr(), None, None)
            bits = np.unpackbits(m[:nb].cpu().numpy().view(np.uint8), axis=-1, bitorder="little")[:, :F]
            hits += bits.sum(axis=0)
            ntok += nb
    rate = np.ascontiguousarray(hits / ntok, dtype=np.float32)
    mask = torch.empty((Bmax, W), dtype=torch.int32, device=dev)
    y = torch.empty((Bmax, cfg.d), dtype=torch.float32, device=dev)
    K, Wm = 16, 4
    names = {L.PI_BATCH_TOKENS: "tokens", L.PI_BATCH_UNION: "union", L.PI_BATCH_AUTO: "auto"}

    def timed(x, B, sched):
        layer.batch_run(x.data_ptr(), S, B, 0, Wm, mask.data_ptr(), y.data_ptr(), schedule=sched, rate=rate)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in ev:
            e.record()                                    # creates the underlying events
        torch.cuda.synchronize()
        layer.batch_run(x.data_ptr(), S, B, Wm, K, mask.data_ptr(), y.data_ptr(), schedule=sched,
                        rate=rate, events=ev)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / K * 1e3, y[:B].clone()      # us per step, last y

    rows = []
    B = 1
    while B <= Bmax:
        x = xall[:, :B].contiguous()                                   # [S, B, d]
        t_tok, y_tok = timed(x, B, L.PI_BATCH_TOKENS)
        t_uni, y_uni = timed(x, B, L.PI_BATCH_UNION) if B > 1 and cfg.wfmt == "f16" else (None, None)
        t_auto, y_auto = timed(x, B, L.PI_BATCH_AUTO)
        ran = ("tokens" if torch.equal(y_auto, y_tok) else
               "union" if y_uni is not None and torch.equal(y_auto, y_uni) else "neither")
        best = "tokens" if t_uni is None or t_tok <= t_uni else "union"
        p = L.BatchPlan()
        L.check(L.pi_batch_plan(layer.ffn[0], B, rate.ctypes.data, HBM_PEAK_GBS, p))
        rows.append({
            "B": B, "tokens_us": round(t_tok, 2), "union_us": None if t_uni is None else round(t_uni, 2),
            "auto_us": round(t_auto, 2), "auto_ran": ran, "best": best,
            "ffn_plan": {"tokens_us": round(p.t_tokens_us, 2),
                         "union_us": None if math.isinf(p.t_union_us) else round(p.t_union_us, 2),
                         "n_mean": round(p.n_mean, 1), "u_mean": round(p.u_mean, 1)},
        })
        print(f"# B={B}: tokens {t_tok:.1f} us, union {t_uni} us, auto {t_auto:.1f} us ran {ran}, "
              f"best {best}", file=sys.stderr, flush=True)
        B = B * 2 if B * 2 <= Bmax or B == Bmax else Bmax
    out = {
        "metric": "batch-size dispatch: one decode step of B tokens through pi_batch_run per schedule (us per step)",
        "unit": "us", "n_gpus": 1, "data": "synthetic", "dtype": "f16",
        "config": {"workload": f"{cfg.name}: one layer, d={cfg.d}, ffn={F}, rank {cfg.r}, {cfg.act}, "
                               f"{cfg.wfmt} weights; the first B of each step's {Bmax} tokens, {S} steps "
                               f"cycled, {R} replicas", "steps": K, "warmup": Wm},
        "rows": rows,
        "auto_took_best": sum(r["auto_ran"] == r["best"] for r in rows),
    }
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------------------- attention side
def bytes_model_attn(cfg, n):
    """Algorithmic bytes of one attention-side step with n predicted heads, by kernel.
    Predictor stage 1: W_p1 2dr, x 2d, z written 4r.  Stage 2: W_p2 2rH, bias 4H, z read 4r, the
    mask words and the head table with its count written (4 ceil(H/32) + 4H + 4).  q/k/v: the n
    heads' 3 d_head rows of d fp16 (n 3 dh d 2), x 2d, qkv written for every head (4 H 3 dh: zeros
    for the others), and the mask read -- or, with H <= 64, stage 2 itself, which the step runs
    inside its q/k/v kernel.  Output: the n heads' d_head rows of W_o^T (n dh d 2), their o values
    (4 n dh), the head table (4 n + 4), y 4d."""
    d, H, dh, r = cfg.d, cfg.H, cfg.dh, cfg.r
    mw = 4 * ((H + 31) // 32)
    stage1 = 2 * d * r + 2 * d + 4 * r
    stage2 = 2 * r * H + 4 * H + 4 * r + mw + 4 * H + 4
    rows = n * 3 * dh * d * 2 + 2 * d + 4 * H * 3 * dh
    if H <= 64:
        pred, qkv = stage1, rows + stage2
    else:
        pred, qkv = stage1 + stage2, rows + mw
    out = n * dh * d * 2 + 4 * n * dh + 4 * n + 4 + 4 * d
    return dict(pred=pred, qkv=qkv, out=out, total=pred + qkv + out)


def cpu_baseline_attn(inputs, budget_s):
    import oracle.attn_oracle as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    X, Ob = inputs["x"], inputs["o"]
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s and n < 4 * X.shape[0]:
        A.attn_step(inputs, X[n % X.shape[0]], Ob[n % X.shape[0]])
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} tokens of the same stream (wrapping), one at a time through the "
                      f"attention-side oracle (head predictor, q/k/v and output projection of the "
                      f"predicted heads), numpy float64, {dt:.1f} s",
            "cpu_model": cpu_model(), **host_cpus()}


def bench_attn(a, cfg):
    """The attention side at batch 1: one step = the head predictor (pi_predict, one output per
    head), the q/k/v projections of the predicted heads (pi_attn_qkv) and the output projection
    over them (pi_attn_out) of one token, the attention core's output standing in as a seeded
    input; K steps through one pi_attn_run call.  The roofline is the q/k/v kernel's, from
    events around it in every step of a second pi_attn_run."""
    import numpy as np
    import torch

    from activation_sparse_pi_amd.layer import DeviceAttn
    from synth import attn as SA

    dev = torch.device("cuda:0")
    inputs = SA.make(cfg)
    T = cfg.T
    probe = bytes_model_attn(cfg, cfg.mean_rate * cfg.H)
    R = a.replicas or max(2, math.ceil(CACHE_BUST_BYTES / probe["total"]))
    att = DeviceAttn(inputs, replicas=R, device=dev)
    bufs = att.buffers()
    xd = torch.from_numpy(inputs["x"].copy()).to(dev)                 # [T, d] in HBM
    od = torch.from_numpy(inputs["o"].copy()).to(dev)                 # [T, H, dh]
    heads = np.zeros(T)
    for t in range(T):
        att.predict(xd[t].data_ptr(), bufs, logits=False)
        heads[t] = int(bufs["count"][0].item())
    K = a.steps if a.steps != parse_defaults["steps"] else 2048
    Wm = a.warmup if a.warmup != parse_defaults["warmup"] else 256
    att.run(xd.data_ptr(), od.data_ptr(), T, 0, Wm, bufs)             # untimed warmup
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    att.run(xd.data_ptr(), od.data_ptr(), T, Wm, K, bufs, events=ev)  # timed: K steps
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[1])
    Kr = min(K, 512)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * Kr)]
    torch.cuda.synchronize()
    att.run(xd.data_ptr(), od.data_ptr(), T, Wm + K, Kr, bufs, kernel_events=kev)
    torch.cuda.synchronize()
    qkv_ms = np.array([kev[2 * i].elapsed_time(kev[2 * i + 1]) for i in range(Kr)])
    steps = (Wm + np.arange(K)) % T
    rsteps = (Wm + K + np.arange(Kr)) % T
    path_bytes = float(np.mean([bytes_model_attn(cfg, heads[t])["total"] for t in steps]))
    qkv_bytes = float(np.mean([bytes_model_attn(cfg, heads[t])["qkv"] for t in rsteps]))
    ms_per_step = total_ms / K
    path_gbs = path_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = qkv_bytes / (float(qkv_ms.mean()) * 1e-3) / 1e9
    kernel_key = f"{'k_attn_pqkv' if cfg.H <= 64 else 'k_attn_qkv'} {cfg.name}"
    copy_probe(a.copy_probe_mb, dev)
    out = {
        "metric": "attention-side decode tokens/sec at batch 1 (predicted heads only) + effective HBM GB/s (% of peak)",
        "value": round(K / (total_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one attention block's predictor and projections, d={cfg.d}, "
                        f"{cfg.H} heads of {cfg.dh}, fp16 weights, fp32 accumulate, head predictor "
                        f"rank {cfg.r}, batch 1, {T}-token stream; the attention core's output is a "
                        f"seeded input",
            "d": cfg.d, "heads": cfg.H, "d_head": cfg.dh, "rank": cfg.r, "replicas": R,
            "mean_predicted_heads": round(float(heads.mean()), 2),
            "launch": ("one pi_attn_run call: per step the head predictor's stage 1 (one kernel), its "
                       "stage 2 folded into the q/k/v kernel of the predicted heads (one kernel), the output "
                       "projection over the head table (one kernel)") if cfg.H <= 64 else
                      ("one pi_attn_run call: per step the head predictor (two kernels), q/k/v of the "
                       "predicted heads (one kernel), the output projection over the head table (one kernel)"),
        },
        "effective_hbm": {"GB/s": round(path_gbs, 1), "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_step": round(path_bytes)},
        "roofline": {
            "bound": "hbm", "kernel": kernel_key,
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profiles(kernel_key),
            "avg_us": round(float(qkv_ms.mean()) * 1e3, 3),
            "bytes_per_launch": round(qkv_bytes),
        },
    }
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline_attn(inputs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------------------- main
def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "the sparse FFN layer is not sharded over GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from activation_sparse_pi_amd import _lib as L
    from activation_sparse_pi_amd.layer import DeviceLayer
    from synth import configs, gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from synth import attn as SA
    if a.config in SA.SHORT or a.config in SA.CONFIGS:
        return bench_attn(a, SA.get(a.config))
    cfg = configs.get(a.config)
    if a.batch_sweep:
        return bench_batch_sweep(a, cfg)
    if cfg.B != 1:
        return bench_batch(a, cfg)
    dev = torch.device("cuda:0")
    inputs = gen.make(cfg)
    p8 = a.pred_format == "i8g128"
    pb = 1.0 + 2.0 / 128.0 if p8 else 2.0
    if p8:
        inputs.update(gen.predictor_int8(inputs))
    probe = bytes_model(cfg, cfg.mean_rate * cfg.F, pb)
    R = a.replicas or max(2, math.ceil(CACHE_BUST_BYTES / probe["total"]))
    perm, nhot = None, 0
    if a.placement == "auto":
        a.placement = "dealt"
    if a.placement in ("dealt", "hot"):
        # profiling run on calibration tokens of their own (none of the timed stream), then
        # the placement; the timed layer holds the placed weights
        prof = DeviceLayer(inputs, replicas=1, B_max=1 if p8 else L.PI_MAX_BATCH, device=dev,
                           pred_format=a.pred_format)
        cal = torch.from_numpy(gen.calibration_x(cfg, a.calib_tokens)).to(dev)
        cal_counts = prof.activation_counts(cal)
        del prof, cal
        torch.cuda.empty_cache()
        perm = np.empty(cfg.F, dtype=np.int32)
        if a.placement == "dealt":
            L.check(L.pi_place_neurons(cal_counts.ctypes.data, cfg.F, perm.ctypes.data))
        else:
            import ctypes
            nh = ctypes.c_int32(0)
            L.check(L.pi_place_neurons_hot(cal_counts.ctypes.data, cfg.F, a.calib_tokens, a.hot_rate,
                                           perm.ctypes.data, nh))
            nhot = nh.value
    layer = DeviceLayer(inputs, replicas=R, device=dev, perm=perm, pred_format=a.pred_format, nhot=nhot)
    T = cfg.T
    xd = torch.from_numpy(inputs["x"][:, 0, :].copy()).to(dev)     # [T, d] resident in HBM
    bufs = layer.buffers(1)
    mask, idx, cnt, h, y = (bufs[k].data_ptr() for k in ("mask", "idx", "count", "h", "y"))

    # active count of every token (replicas are identical, so token t always gives n_t)
    counts = np.zeros(T, dtype=np.int64)
    for t in range(T):
        layer.predict(xd[t].data_ptr(), 1, None, mask, idx, cnt)
        counts[t] = int(bufs["count"][0].item())

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
    up_ms = []
    passes_ms = []
    sched = a.mode if a.mode in ("fused", "split") else kernel_schedule(cfg, nhot)
    sched_desc = ("two kernels per step (fused down)" if sched == "fused"
                  else "three kernels per step (split down)")
    if a.mode in ("kernels", "fused", "split"):
        mode = {"kernels": L.PI_RUN_KERNELS, "fused": L.PI_RUN_FUSED, "split": L.PI_RUN_SPLIT}[a.mode]
        layer.decode_run(xd.data_ptr(), T, 0, Wm, bufs, mode=mode)            # untimed warmup
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in ev:                 # torch creates the HIP event on first record
            e.record()
        torch.cuda.synchronize()
        layer.decode_run(xd.data_ptr(), T, Wm, K, bufs, events=ev, mode=mode)  # timed: K steps
        torch.cuda.synchronize()
        total_ms = ev[0].elapsed_time(ev[1])
        passes_ms = []
        for _ in range(a.passes):
            # a whole pass over the stream: tokens 0 .. T-1, replicas rotating as in the timed run
            pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for e in pe:
                e.record()
            torch.cuda.synchronize()
            layer.decode_run(xd.data_ptr(), T, 0, T, bufs, events=pe, mode=mode)
            torch.cuda.synchronize()
            passes_ms.append(pe[0].elapsed_time(pe[1]))
        # roofline pass: the tile kernel of every step carries its own start/end events
        Kr = min(K, 1088)
        kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * Kr)]
        for e in kev:
            e.record()
        torch.cuda.synchronize()
        layer.decode_run(xd.data_ptr(), T, Wm + K, Kr, bufs, mode=mode, kernel_events=kev)
        torch.cuda.synchronize()
        up_ms = [kev[2 * i].elapsed_time(kev[2 * i + 1]) for i in range(Kr)]
        roof_steps = (Wm + K + np.arange(Kr)) % T
    else:
        for s in range(Wm):
            step(s)
        ev_up = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(K)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for s in range(K):
            step(Wm + s, ev_up[s])
        t1.record()
        torch.cuda.synchronize()
        total_ms = t0.elapsed_time(t1)
        up_ms = [e0.elapsed_time(e1) for e0, e1 in ev_up]
    timed = (Wm + np.arange(K)) % T
    ms_per_step = total_ms / K
    tok_s = K / (total_ms / 1e3)
    n_all = counts[timed].astype(np.float64)
    bm = bytes_model(cfg, n_all, pb)
    path_bytes = float(np.mean(bm["total"]))
    path_gbs = path_bytes / (ms_per_step * 1e-3) / 1e9
    ffn_gbs = float(np.mean(bm["ffn"])) / (ms_per_step * 1e-3) / 1e9
    if a.mode == "eager":
        kernel_key = f"k_up_{cfg.wfmt}[{cfg.act}] {cfg.name}"
        launch_bytes, launch_ms = float(np.mean(bm["up"])), float(np.mean(up_ms))
    else:
        kernel_key = f"k_dec_stage2_up[{cfg.wfmt},{cfg.act},{sched}{',p8' if p8 else ''}{',hot' if nhot else ''}] {cfg.name}"
        bm_r = bytes_model(cfg, counts[roof_steps].astype(np.float64), pb)
        launch_bytes = float(np.mean(bm_r["tile_fused" if sched == "fused" else "stage2"]))
        launch_ms = float(np.mean(up_ms))
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(kernel_key) if kernel_key else None

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
            "launch": {"kernels": f"one pi_decode_run call: {sched_desc}",
                       "fused": f"one pi_decode_run call: {sched_desc}",
                       "split": f"one pi_decode_run call: {sched_desc}",
                       "eager": "one Python call per ABI function"}[a.mode],
            "predictor": "int8 group-128, fp16 scales" if p8 else "fp16",
            "placement": ("none" if perm is None else
                          f"neurons dealt over the 64-neuron tiles by their activation counts on "
                          f"{a.calib_tokens} calibration tokens (pi_place_neurons)" if nhot == 0 else
                          f"hot block of {nhot} neurons (profiled rate >= {a.hot_rate} on "
                          f"{a.calib_tokens} calibration tokens) computed before the predictor's "
                          f"decision, the rest dealt over the tiles (pi_place_neurons_hot)"),
        },
        "effective_hbm": {"GB/s": round(path_gbs, 1), "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_step": round(path_bytes),
                          "sparse_ffn_GB/s": round(ffn_gbs, 1),
                          "sparse_ffn_bytes_per_step": round(float(np.mean(bm["ffn"])))},
        "roofline": {
            "bound": "hbm", "kernel": kernel_key,
            "achieved": None if math.isnan(achieved) else round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": None if math.isnan(achieved) else round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_us": None if math.isnan(launch_ms) else round(launch_ms * 1e3, 3),
            "bytes_per_launch": None if math.isnan(launch_bytes) else round(launch_bytes),
        },
    }
    if passes_ms:
        med = float(np.median(passes_ms))
        out["stream_passes"] = {
            "passes": len(passes_ms), "tokens_per_pass": T,
            "median_us_per_step": round(med / T * 1e3, 3),
            "median_tokens_per_s": round(T / (med / 1e3), 1),
            "us_per_step_each": [round(p / T * 1e3, 3) for p in passes_ms],
            "GB/s_median": round(float(np.mean(bytes_model(cfg, counts.astype(np.float64), pb)["total"]))
                                 / (med / T * 1e-3) / 1e9, 1)}
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inputs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
