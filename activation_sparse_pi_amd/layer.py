"""Device-side holder of one FFN layer for the C ABI: weights, descriptors, workspace.

PyTorch is used only to own device memory and to name the stream; every step
of the method runs in libpi.so.  ``replicas`` keeps R byte-identical copies of
the weights so that a token stream can rotate through them: each copy stands
for another layer of a real model, so weights are fetched from HBM rather
than from the 256 MB Infinity Cache or the L2 of a previous token.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _event_handle(e):
    """The hipEvent_t of a torch event (torch creates it lazily, at the first record)."""
    if not e.cuda_event:
        e.record()
    return e.cuda_event


class DeviceLayer:
    def __init__(self, inputs: dict, replicas: int = 1, B_max: int = 1, device="cuda",
                 threshold: float = 0.5, perm: np.ndarray | None = None, pred_format: str = "f16",
                 nhot: int = 0):
        """perm: optional neuron placement (int32 [F], placed position p holds original
        neuron perm[p], from ``pi_place_neurons`` or ``pi_place_neurons_hot``): every per-neuron
        array is permuted on the device with ``pi_permute_rows``; ``map_ids`` turns placed ids
        back into original ones.  nhot: the hot block's size (placed positions [0, nhot)), from
        ``pi_place_neurons_hot``; it goes into every FFN descriptor.
        pred_format: "f16", or "i8g128" for the int8 group-128 predictor, whose factors come in
        ``inputs`` as q_p1t, s_p1t, q_p2t, s_p2t (one row per predictor output)."""
        cfg = inputs["cfg"]
        self.cfg, self.d, self.F, self.r = cfg, cfg.d, cfg.F, cfg.r
        self.act = L.PI_ACT_REGLU if cfg.act == "reglu" else L.PI_ACT_RELU
        self.wfmt = L.PI_W_F16 if cfg.wfmt == "f16" else L.PI_W_I4G128
        self.device = torch.device(device)
        if pred_format not in ("f16", "i8g128"):
            raise ValueError(f"unknown predictor format {pred_format}")
        self.pfmt = L.PI_P_I8G128 if pred_format == "i8g128" else L.PI_P_F16
        names = ["w_p1", "w_p2", "bias"] if pred_format == "f16" else ["q_p1t", "s_p1t", "q_p2t", "s_p2t", "bias"]
        mats = ("gate", "up", "down") if cfg.act == "reglu" else ("up", "down")
        for m in mats:
            names += ["w_" + m] if cfg.wfmt == "f16" else ["q_" + m, "s_" + m]
        host = {k: inputs[k] for k in names}
        # predictor factors go to the device transposed: one contiguous row per output
        if pred_format == "f16":
            host["w_p1"] = np.ascontiguousarray(inputs["w_p1"].T)    # [r, d]
            host["w_p2"] = np.ascontiguousarray(inputs["w_p2"].T)    # [F, r]
        base = {k: _dev(v, self.device) for k, v in host.items()}
        self.perm = None
        self.nhot = nhot
        if nhot and perm is None:
            raise ValueError("a hot block needs the placement that laid it out (perm)")
        if perm is not None:
            perm = np.ascontiguousarray(perm, dtype=np.int32)
            if perm.shape != (cfg.F,):
                raise ValueError(f"perm must be int32 [{cfg.F}]")
            self.perm = _dev(perm, self.device)
            for k in names:                     # every array here is one row per neuron but W_p1^T
                if k in ("w_p1", "q_p1t", "s_p1t"):
                    continue
                src = base[k]
                dst = torch.empty_like(src)
                L.check(L.pi_permute_rows(src.data_ptr(), dst.data_ptr(), self.perm.data_ptr(), cfg.F,
                                          src.numel() * src.element_size() // cfg.F, self.stream()))
                base[k] = dst
        self.tensors = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(replicas - 1)]
        self.pred, self.ffn = [], []
        for t in self.tensors:
            if pred_format == "f16":
                self.pred.append(L.PredDesc(t["w_p1"].data_ptr(), t["w_p2"].data_ptr(), t["bias"].data_ptr(),
                                            cfg.d, cfg.r, cfg.F, threshold))
            else:
                self.pred.append(L.PredDesc(t["q_p1t"].data_ptr(), t["q_p2t"].data_ptr(), t["bias"].data_ptr(),
                                            cfg.d, cfg.r, cfg.F, threshold, L.PI_P_I8G128,
                                            t["s_p1t"].data_ptr(), t["s_p2t"].data_ptr()))
            if cfg.wfmt == "f16":
                g = t["w_gate"].data_ptr() if "w_gate" in t else None
                self.ffn.append(L.FfnDesc(g, t["w_up"].data_ptr(), t["w_down"].data_ptr(), None, None,
                                          None, cfg.d, cfg.F, self.act, self.wfmt, nhot))
            else:
                g = t["q_gate"].data_ptr() if "q_gate" in t else None
                sg = t["s_gate"].data_ptr() if "s_gate" in t else None
                self.ffn.append(L.FfnDesc(g, t["q_up"].data_ptr(), t["q_down"].data_ptr(), sg,
                                          t["s_up"].data_ptr(), t["s_down"].data_ptr(), cfg.d, cfg.F,
                                          self.act, self.wfmt, nhot))
        self.ws_bytes = L.pi_workspace_bytes(self.pred[0], self.ffn[0], B_max)
        if self.ws_bytes == 0:
            raise L.PiError(L.PI_ERR_SHAPE, "pi_workspace_bytes rejected the layer: " + L.pi_last_error())
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        L.check(L.pi_workspace_init(self.ws.data_ptr(), self.ws_bytes, self.stream()))

    @property
    def replicas(self) -> int:
        return len(self.tensors)

    def weight_bytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.tensors[0].values())

    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    # ---- thin forwards to the C ABI (pointers are tensor.data_ptr() values) -------------
    def predict(self, x, B, logits, mask, idx, count, rep: int = 0) -> None:
        L.check(L.pi_predict(self.pred[rep], x, B, logits, mask, idx, count, self.ws.data_ptr(),
                             self.ws_bytes, self.stream()))

    def compact(self, mask, B, mode, idx, count) -> None:
        L.check(L.pi_compact(mask, B, self.F, mode, idx, count, None, 0, self.stream()))

    def sparse_ffn(self, x, B, idx, count, token_mask, y, rep: int = 0) -> None:
        L.check(L.pi_sparse_ffn(self.ffn[rep], x, B, idx, count, token_mask, y, self.ws.data_ptr(),
                                self.ws_bytes, self.stream()))

    def ffn_up(self, x, idx, count, h, rep: int = 0) -> None:
        L.check(L.pi_ffn_up(self.ffn[rep], x, idx, count, h, self.stream()))

    def ffn_down(self, idx, count, h, y, rep: int = 0) -> None:
        L.check(L.pi_ffn_down(self.ffn[rep], idx, count, h, y, self.ws.data_ptr(), self.ws_bytes,
                              self.stream()))

    def map_ids(self, idx, count, B: int, out) -> None:
        """Neuron table of a placed layer: out[b, k] = perm[idx[b, k]] for k < count[b]."""
        if self.perm is None:
            raise ValueError("the layer has no placement")
        L.check(L.pi_map_ids(idx, count, B, self.F, self.perm.data_ptr(), out, self.stream()))

    def activation_counts(self, x: torch.Tensor) -> np.ndarray:
        """Profiling run: how often each neuron (in this layer's order) is predicted active over
        the tokens x (fp16 [n, d] on the device), in batches of up to 32 tokens (1 with the int8
        predictor) through pi_predict, counted on the device by pi_count_active.  Returns
        int32 [F] on the host."""
        n = x.shape[0]
        W = (self.F + 31) // 32
        bmax = 1 if self.pfmt == L.PI_P_I8G128 else L.PI_MAX_BATCH      # int8: batch 1 only
        mask = torch.empty((bmax, W), dtype=torch.int32, device=self.device)
        counts = torch.zeros((self.F,), dtype=torch.int32, device=self.device)
        for t0 in range(0, n, bmax):
            B = min(bmax, n - t0)
            self.predict(x[t0:t0 + B].data_ptr(), B, None, mask.data_ptr(), None, None)
            L.check(L.pi_count_active(mask.data_ptr(), B, self.F, counts.data_ptr(), self.stream()))
        return counts.cpu().numpy()

    def dense(self, x, B, y, rep: int = 0) -> None:
        L.check(L.pi_ffn_dense_ref_gpu(self.ffn[rep], x, B, y, self.ws.data_ptr(), self.ws_bytes,
                                       self.stream()))

    def decode_run(self, x, T: int, s0: int, nsteps: int, bufs: dict, events=None,
                   mode: int = L.PI_RUN_AUTO, kernel_events=None) -> None:
        """Enqueue nsteps batch-1 steps from native code (token (s0+i) % T, replica
        (s0+i) % R).  events: None or two torch.cuda.Event objects recorded around the
        enqueued work; kernel_events: None or 2*nsteps events attached to the tile kernel
        of every step.  Events must have been recorded
        once already (torch creates the HIP event on first record).
        mode: PI_RUN_AUTO / PI_RUN_KERNELS / PI_RUN_FUSED / PI_RUN_SPLIT."""
        import ctypes
        if not hasattr(self, "_pred_arr"):
            self._pred_arr = (L.PredDesc * self.replicas)(*self.pred)
            self._ffn_arr = (L.FfnDesc * self.replicas)(*self.ffn)

        def handles(evs):
            return None if evs is None else (ctypes.c_void_p * len(evs))(*[_event_handle(e) for e in evs])

        L.check(L.pi_decode_run(self._pred_arr, self._ffn_arr, self.replicas, x, T, s0, nsteps,
                                mode, bufs["mask"].data_ptr(), bufs["idx"].data_ptr(),
                                bufs["count"].data_ptr(), bufs["y"].data_ptr(),
                                handles(events), handles(kernel_events), self.ws.data_ptr(),
                                self.ws_bytes, self.stream()))

    def batch_run(self, x, T: int, B: int, s0: int, nsteps: int, mask, y,
                  schedule: int = L.PI_BATCH_AUTO, rate=None, hbm_gbs: float = 8000.0,
                  events=None, kernel_events=None) -> None:
        """pi_batch_run: nsteps steps of B tokens (x: device address of fp16 [T, B, d]); mask /
        y: device addresses of [B, ceil(F/32)] u32 and [B, d] fp32 (the last step's); rate: host
        float32 ndarray [F] (for PI_BATCH_AUTO) or None; events: None or two torch events;
        kernel_events: None or 2 nsteps torch events around each step's union FFN."""
        import ctypes
        if not hasattr(self, "_pred_arr"):
            self._pred_arr = (L.PredDesc * self.replicas)(*self.pred)
            self._ffn_arr = (L.FfnDesc * self.replicas)(*self.ffn)
        ev = None if events is None else (ctypes.c_void_p * 2)(*[_event_handle(e) for e in events])
        kev = None if kernel_events is None else \
            (ctypes.c_void_p * len(kernel_events))(*[_event_handle(e) for e in kernel_events])
        rp = None if rate is None else np.ascontiguousarray(rate, dtype=np.float32)
        L.check(L.pi_batch_run(self._pred_arr, self._ffn_arr, self.replicas, x, T, B, s0, nsteps,
                               schedule, None if rp is None else rp.ctypes.data, hbm_gbs, mask, y, ev,
                               kev, self.ws.data_ptr(), self.ws_bytes, self.stream()))

    def decode_run_noalloc(self, x, T: int, s0: int, nsteps: int, bufs: dict,
                           mode: int = L.PI_RUN_AUTO) -> None:
        """decode_run through pi_decode_run_noalloc: the library's static scratch instead of this
        layer's workspace (kernel schedules only)."""
        if not hasattr(self, "_pred_arr"):
            self._pred_arr = (L.PredDesc * self.replicas)(*self.pred)
            self._ffn_arr = (L.FfnDesc * self.replicas)(*self.ffn)
        L.check(L.pi_decode_run_noalloc(self._pred_arr, self._ffn_arr, self.replicas, x, T, s0, nsteps,
                                        mode, bufs["mask"].data_ptr(), bufs["idx"].data_ptr(),
                                        bufs["count"].data_ptr(), bufs["y"].data_ptr(), None, None,
                                        self.stream()))

    def step(self, x, bufs: dict, rep: int = 0, logits: bool = True) -> None:
        """One batch-1 decode step: predict + compact (fused), then the sparse FFN.

        x is the device address of one fp16 token; results land in ``bufs``
        (see ``buffers``).  Nothing is synchronised and count stays on the device.
        """
        self.predict(x, 1, bufs["logits"].data_ptr() if logits else None, bufs["mask"].data_ptr(),
                     bufs["idx"].data_ptr(), bufs["count"].data_ptr(), rep)
        self.sparse_ffn(x, 1, bufs["idx"].data_ptr(), bufs["count"].data_ptr(), None,
                        bufs["y"].data_ptr(), rep)

    def batch_step(self, x, B: int, bufs: dict, rep: int = 0, logits: bool = True) -> None:
        """One small-batch step (1 < B <= 32): per-token masks and tables, their union,
        then the union FFN where token b only receives the neurons of its own mask."""
        self.predict(x, B, bufs["logits"].data_ptr() if logits else None, bufs["mask"].data_ptr(),
                     bufs["idx"].data_ptr(), bufs["count"].data_ptr(), rep)
        self.compact(bufs["mask"].data_ptr(), B, L.PI_UNION, bufs["uidx"].data_ptr(),
                     bufs["ucount"].data_ptr())
        self.sparse_ffn(x, B, bufs["uidx"].data_ptr(), bufs["ucount"].data_ptr(),
                        bufs["mask"].data_ptr(), bufs["y"].data_ptr(), rep)

    # ---- output buffers --------------------------------------------------------------------
    def buffers(self, B: int) -> dict:
        W = (self.F + 31) // 32
        dev = self.device
        return dict(
            logits=torch.empty((B, self.F), dtype=torch.float32, device=dev),
            mask=torch.empty((B, W), dtype=torch.int32, device=dev),
            idx=torch.empty((B, self.F), dtype=torch.int32, device=dev),
            count=torch.empty((B,), dtype=torch.int32, device=dev),
            uidx=torch.empty((self.F,), dtype=torch.int32, device=dev),
            ucount=torch.empty((1,), dtype=torch.int32, device=dev),
            y=torch.empty((B, self.d), dtype=torch.float32, device=dev),
            h=torch.empty((self.F,), dtype=torch.float32, device=dev),
        )


class DeviceAttn:
    """The attention side of one layer on the device: the head predictor (pi_predict with one
    output per head) and the head-major projections for pi_attn_qkv / pi_attn_out.

    ``inputs``: w_a1 fp16 [d, r], w_a2 fp16 [r, H], bias_a fp32 [H], w_qkv fp16 [H, 3, dh, d],
    w_o fp16 [H, dh, d] and ``cfg`` (d, H, dh, r).  Replicas are independent copies (the bench
    cycles through them so each step streams its weights from HBM)."""

    def __init__(self, inputs: dict, replicas: int = 1, device: str = "cuda:0", threshold: float = 0.5):
        cfg = inputs["cfg"]
        self.cfg, self.d, self.H, self.dh, self.r = cfg, cfg.d, cfg.H, cfg.dh, cfg.r
        self.device = torch.device(device)
        self.replicas = replicas
        host = {"w_a1": np.ascontiguousarray(inputs["w_a1"].T),      # [r, d]
                "w_a2": np.ascontiguousarray(inputs["w_a2"].T),      # [H, r]
                "bias_a": inputs["bias_a"], "w_qkv": inputs["w_qkv"], "w_o": inputs["w_o"]}
        base = {k: _dev(v, self.device) for k, v in host.items()}
        self.tensors = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(replicas - 1)]
        self.pred = [L.PredDesc(t["w_a1"].data_ptr(), t["w_a2"].data_ptr(), t["bias_a"].data_ptr(),
                                cfg.d, cfg.r, cfg.H, threshold) for t in self.tensors]
        self.attn = [L.AttnDesc(t["w_qkv"].data_ptr(), t["w_o"].data_ptr(), cfg.d, cfg.H, cfg.dh)
                     for t in self.tensors]
        pb = L.pi_workspace_bytes(self.pred[0], None, 1)
        ab = L.pi_attn_workspace_bytes(self.attn[0])
        if pb == 0 or ab == 0:
            raise L.PiError(L.PI_ERR_SHAPE, "the library rejected the attention layer: " + L.pi_last_error())
        self.ws_bytes = pb + ab            # pi_attn_run: the predictor's area, then the partial rows
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        L.check(L.pi_workspace_init(self.ws.data_ptr(), self.ws_bytes, self.stream()))

    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def buffers(self) -> dict:
        W = (self.H + 31) // 32
        z = dict(dtype=torch.float32, device=self.device)
        return {"logits": torch.empty(self.H, **z), "mask": torch.zeros(W, dtype=torch.int32, device=self.device),
                "idx": torch.empty(self.H, dtype=torch.int32, device=self.device),
                "count": torch.empty(1, dtype=torch.int32, device=self.device),
                "qkv": torch.empty((self.H, 3, self.dh), **z), "y": torch.empty(self.d, **z)}

    def predict(self, x, bufs: dict, rep: int = 0, logits: bool = True) -> None:
        """pi_predict with the head predictor: head mask, head table (ascending) and count."""
        L.check(L.pi_predict(self.pred[rep], x, 1, bufs["logits"].data_ptr() if logits else None,
                             bufs["mask"].data_ptr(), bufs["idx"].data_ptr(), bufs["count"].data_ptr(),
                             self.ws.data_ptr(), self.ws_bytes, self.stream()))

    def qkv(self, x, bufs: dict, rep: int = 0) -> None:
        L.check(L.pi_attn_qkv(self.attn[rep], x, bufs["mask"].data_ptr(), bufs["qkv"].data_ptr(), self.stream()))

    def out(self, o, bufs: dict, rep: int = 0) -> None:
        """o: device address of fp32 [H, dh] (the attention core's per-head output); the head
        table is the one ``predict`` wrote into bufs."""
        L.check(L.pi_attn_out(self.attn[rep], o, bufs["idx"].data_ptr(), bufs["count"].data_ptr(),
                              bufs["y"].data_ptr(), self.ws.data_ptr(), self.ws_bytes, self.stream()))

    def run(self, x, o, T: int, s0: int, nsteps: int, bufs: dict, events=None, kernel_events=None) -> None:
        """pi_attn_run: nsteps steps over tokens x (device fp16 [T, d]) and attention outputs o
        (device fp32 [T, H, dh]), replicas rotating; events: None or two torch events;
        kernel_events: None or 2 nsteps torch events around each step's q/k/v kernel."""
        import ctypes
        if not hasattr(self, "_pred_arr"):
            self._pred_arr = (L.PredDesc * self.replicas)(*self.pred)
            self._attn_arr = (L.AttnDesc * self.replicas)(*self.attn)

        def handles(evs):
            return None if evs is None else (ctypes.c_void_p * len(evs))(*[_event_handle(e) for e in evs])

        L.check(L.pi_attn_run(self._pred_arr, self._attn_arr, self.replicas, x, o, T, s0, nsteps,
                              bufs["mask"].data_ptr(), bufs["idx"].data_ptr(), bufs["count"].data_ptr(),
                              bufs["qkv"].data_ptr(), bufs["y"].data_ptr(), handles(events),
                              handles(kernel_events), self.ws.data_ptr(), self.ws_bytes, self.stream()))
