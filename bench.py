"""Benchmark of the INT4 (group 32) weight-only MoE layer on one MI355X.

One step = one layer call over one batch through moe_w4a16_layer: routing,
FC1 (gate/up, SiLU*mul) and FC2 with the weighted combine (two kernels for
small batches, up to four above). The headline workload is the
384-expert layer (hidden 7168, intermediate 2048, top-8) at M = 1 token
(one decoding stream), the shape of "The Throughput Lever: Quantifying the MoE
GEMM and Mapping the Road to B300", section "The Result: Two Regimes", table
row M = 1. A sweep over M = 4, 9, 90, 256, 512, 1024, the skewed M = 1024
batch and prefill chunks of 2048-8192 tokens is reported in the same JSON
line, and (mxfp4_sweep) the same layer with MXFP4 expert weights through
moe_mxfp4_layer at M = 1, 4, 9, 256, 1024, 4096 (context: the headline is INT4).

Weights are synthetic (random INT4 codes, fp16 scales in [0.005, 0.02]) and
resident in HBM before timing starts. To keep the 256 MB last-level cache from
serving a step's weights out of the previous step, the timed loop cycles
through R copies of the layer's weights at different addresses (a model with R
MoE layers); each step reads copy i % R.

Timing: W untimed warm-up steps, then K steps bracketed by
torch.cuda.synchronize(), queued behind a GPU spin of device copies (busy, so
the clock stays up) and max(10, K/4) untimed steps so that they run back to back as
under a HIP graph; HIP events on the launch stream bracket the K steps; K more steps carry events around every FC1 launch (for the roofline
figure). The same K steps
replayed from one captured HIP graph are reported as context. The CPU oracle is timed on a bounded sample of
the same workload (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--replicas R] [--no-sweep] [--no-mxfp4] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak
HEADLINE = "k26_m1"
SWEEP = ["k26_m4", "k26_m9", "k26_m90", "k26_m256", "k26_m512", "k26_m1024", "k26_m1024_skew",
         "k26_m2048", "k26_m4096", "k26_m8192"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_k26_m1_traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=8)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--sweep-steps", type=int, default=200)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--sweep-list", default=None,
                   help="comma-separated workloads to sweep instead of the default list (for profiling runs)")
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replay context figure")
    p.add_argument("--no-mxfp4", action="store_true", help="skip the MXFP4-weight sweep")
    p.add_argument("--weights", choices=("int4", "mxfp4"), default="int4",
                   help="expert weight format of the headline and the sweep (mxfp4: for profiling that path)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 1 GiB device-to-device copy (to scale HBM counters)")
    return p.parse_args()


def kernel_source_sha() -> str:
    """Hash of every kernel source: counters taken on other sources do not apply."""
    d = os.path.join(ROOT, "int4_weight_only_moe_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# weight bytes per weight: INT4 codes + an fp16 scale per 32 (9/16), MXFP4
# codes + an E8M0 byte per 32 (17/32)
WEIGHT_BYTES = {"int4": (9, 16), "mxfp4": (17, 32)}
MXFP4_SWEEP = ["k26_m1", "k26_m4", "k26_m9", "k26_m256", "k26_m1024", "k26_m4096"]


def _wbytes(n, fmt):
    num, den = WEIGHT_BYTES[fmt]
    return n * num // den


def layer_bytes(D, M, s, fmt="int4"):
    """Algorithmic bytes of one layer call: touched experts' codes + scales,
    x in and out (bf16), logits (fp32), ids and weights."""
    per_expert = _wbytes(2 * s.I * s.H + s.H * s.I, fmt)
    return D * per_expert + 4 * M * s.H + 4 * M * s.E + 8 * M * s.k


def fc1_bytes(D, M, s, fmt="int4"):
    """Algorithmic bytes of one FC1 launch: touched experts' W13 codes + scales,
    the x rows, and the bf16 activations it writes."""
    return D * _wbytes(2 * s.I * s.H, fmt) + 2 * M * s.H + 2 * M * s.k * s.I


def fc2_bytes(D, M, s, fmt="int4"):
    """Algorithmic bytes of one FC2 stage: touched experts' W2 codes + scales, the
    bf16 activations it reads and the bf16 output."""
    return D * _wbytes(s.H * s.I, fmt) + 2 * M * s.k * s.I + 2 * M * s.H


def flops(M, s):
    return 2 * M * s.k * (2 * s.I * s.H + s.H * s.I)


class HipEvent:
    """A raw hipEvent_t (the library records it on the launch stream)."""
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreate(ctypes.byref(self.ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.handle = self.ev.value

    def elapsed_ms(self, end: "HipEvent") -> float:
        t = self._ct.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._ct.byref(t), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return t.value

    def __del__(self):
        hip = getattr(type(self), "_hip", None)  # module globals may be gone at interpreter exit
        if hip is not None and self.ev:
            hip.hipEventDestroy(self.ev)


class Bench:
    def __init__(self, replicas: int):
        self._spin_bufs = None
        import torch
        import int4_weight_only_moe_amd as moe
        import workloads as wl

        self.torch, self.moe, self.wl = torch, moe, wl
        self.s = wl.K26
        t0 = time.time()
        w13, s13, w2, s2 = wl.layer_weights(self.s, 2026)
        self.host = (w13, s13, w2, s2)
        dev = "cuda"
        q13 = torch.from_numpy(w13).to(dev)
        sc13 = torch.from_numpy(s13).to(dev)
        p13 = moe.repack(q13, sc13, moe.KIND_W13)
        del q13, sc13
        q2 = torch.from_numpy(w2).to(dev)
        sc2 = torch.from_numpy(s2).to(dev)
        p2 = moe.repack(q2, sc2, moe.KIND_W2)
        del q2, sc2
        torch.cuda.synchronize()
        t1 = time.time()
        # repack time on its own (one more repack of W13 + W2 from device copies)
        self.repack_ms = self._time_repack(w13, s13, w2, s2)
        self.layers = [(p13, p2)] + [(p13.clone(), p2.clone()) for _ in range(replicas - 1)]
        self.fmt_layers = {"int4": self.layers}
        self.replicas = replicas
        torch.cuda.synchronize()
        print(f"# weights: generated + repacked in {t1 - t0:.1f} s, {replicas} copies "
              f"({replicas * (p13.numel() + p2.numel()) / 1e9:.1f} GB)", file=sys.stderr, flush=True)

    def mxfp4_layers(self):
        """The same layer with seeded MXFP4 weights (built on first use), as many copies."""
        if "mxfp4" not in self.fmt_layers:
            torch, moe, wl = self.torch, self.moe, self.wl
            t0 = time.time()
            w13, s13, w2, s2 = wl.layer_weights(self.s, 2026, fmt="mxfp4")
            p13 = moe.repack_mxfp4(torch.from_numpy(w13).cuda(), torch.from_numpy(s13).cuda(), moe.KIND_W13)
            p2 = moe.repack_mxfp4(torch.from_numpy(w2).cuda(), torch.from_numpy(s2).cuda(), moe.KIND_W2)
            del w13, s13, w2, s2
            self.fmt_layers["mxfp4"] = [(p13, p2)] + [(p13.clone(), p2.clone()) for _ in range(self.replicas - 1)]
            torch.cuda.synchronize()
            print(f"# MXFP4 weights: generated + repacked in {time.time() - t0:.1f} s, {self.replicas} copies "
                  f"({self.replicas * (p13.numel() + p2.numel()) / 1e9:.1f} GB)", file=sys.stderr, flush=True)
        return self.fmt_layers["mxfp4"]

    def _time_repack(self, w13, s13, w2, s2):
        torch, moe = self.torch, self.moe
        q13, sc13 = torch.from_numpy(w13).cuda(), torch.from_numpy(s13).cuda()
        q2, sc2 = torch.from_numpy(w2).cuda(), torch.from_numpy(s2).cuda()
        o13 = torch.empty(moe.moe_w4a16_packed_bytes(self.s.E, 2 * self.s.I, self.s.H), dtype=torch.uint8, device="cuda")
        o2 = torch.empty(moe.moe_w4a16_packed_bytes(self.s.E, self.s.H, self.s.I), dtype=torch.uint8, device="cuda")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moe.moe_w4a16_repack(q13, sc13, moe.KIND_W13, o13)
        moe.moe_w4a16_repack(q2, sc2, moe.KIND_W2, o2)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        del q13, sc13, q2, sc2, o13, o2
        return ms

    def prepare(self, name):
        torch, moe, wl = self.torch, self.moe, self.wl
        w = wl.WORKLOADS[name]
        s = w.shape
        t = wl.workload_tokens(w)
        B = moe.moe_w4a16_preferred_block_m(w.M, s.E, s.H, s.I, s.k)
        rb = moe.alloc_route_buffers(w.M, s.E, s.k, B)
        logits = torch.from_numpy(t.logits).cuda()
        x = torch.from_numpy(t.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        ws = torch.empty(moe.moe_w4a16_workspace_bytes(w.M, s.E, s.H, s.I, s.k), dtype=torch.uint8, device="cuda")
        out = torch.empty((w.M, s.H), dtype=torch.bfloat16, device="cuda")
        D = int(len(np.unique(self._oracle_free_ids(t.logits, s.k))))
        return dict(w=w, t=t, B=B, rb=rb, logits=logits, x=x, ws=ws, out=out, D=D)

    @staticmethod
    def _oracle_free_ids(logits, k):
        # touched experts for the byte count: the k largest logits per row
        return np.argsort(-logits, axis=1, kind="stable")[:, :k]

    def step(self, c, layer, ev=None, fmt="int4"):
        """One layer call: moe_w4a16_layer or moe_mxfp4_layer (routing + FC1 +
        FC2); ev = optional pair of HIP events recorded around its FC1 stage."""
        s = self.s
        self.moe.layer(c["logits"], c["x"], c["rb"], s.I, layer[0], layer[1], workspace=c["ws"], out=c["out"],
                       stage_events=None if ev is None else (ev[0].handle, ev[1].handle), fmt=fmt)

    def spin(self, seconds):
        """Keep the GPU busy for about `seconds` ahead of the host: device
        copies of 512 MB (each far more GPU time than host time to launch).
        An idle wait would let the clock drop, and the first timed steps
        would then run slower than in steady operation."""
        torch = self.torch
        if self._spin_bufs is None:
            self._spin_bufs = (torch.empty(1 << 29, dtype=torch.uint8, device="cuda"),
                               torch.empty(1 << 29, dtype=torch.uint8, device="cuda"))
            self._spin_bufs[0].fill_(1)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(8):
                self._spin_bufs[1].copy_(self._spin_bufs[0])
            torch.cuda.synchronize()
            self._spin_copy_s = (time.perf_counter() - t) / 8
        for _ in range(max(1, int(seconds / self._spin_copy_s))):
            self._spin_bufs[1].copy_(self._spin_bufs[0])

    def run(self, name, steps, warmup, replicas, fmt="int4"):
        """W eager warm-up steps, then K timed steps launched back to back, then
        K more steps with HIP events on the FC1 stage.

        The Python host needs longer to launch a step than the GPU needs to run
        it at small M, so the timed steps are queued behind a GPU spin of known
        length: by the time the GPU reaches the start event, every step is
        already in the queue and runs without host gaps (as under a HIP graph).
        The spin is device copies (an idle wait lets the clock drop), and
        untimed steps between it and the start event bring the pipeline into
        its steady state.
        The first K steps carry no instrumentation (they give the per-call
        time); the second K steps each record a pair of events around their
        FC1 kernel (the kernel's own start and end timestamps) for the roofline
        figure of that kernel.
        """
        torch = self.torch
        c = self.prepare(name)
        layers = self.mxfp4_layers() if fmt == "mxfp4" else self.layers
        R = min(replicas, len(layers))
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for i in range(warmup):
            self.step(c, layers[i % R], fmt=fmt)
        host_per_step = (time.perf_counter() - h0) / max(warmup, 1)
        torch.cuda.synchronize()
        # Untimed steps queued between the spin and the start event: the
        # timed region starts in steady operation.
        ramp = max(10, steps // 4)
        # generous cover: a host that falls behind the GPU would put launch
        # gaps into the timed region (checked below)
        spin_s = min(4.0, 4.0 * host_per_step * (steps + ramp) + 5e-3)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.spin(spin_s)
        for i in range(ramp):
            self.step(c, layers[i % R], fmt=fmt)
        start.record()
        for i in range(steps):
            self.step(c, layers[i % R], fmt=fmt)
        stop.record()
        enqueue_s = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if enqueue_s > spin_s:
            print(f"# warning: {name}: enqueueing took {enqueue_s * 1e3:.1f} ms, longer than the "
                  f"{spin_s * 1e3:.1f} ms spin; the timed steps may include host gaps", file=sys.stderr)
        total_ms = start.elapsed_time(stop)
        evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
        self.spin(spin_s)
        for i in range(ramp):
            self.step(c, layers[i % R], fmt=fmt)
        for i in range(steps):
            self.step(c, layers[i % R], evs[i], fmt=fmt)
        torch.cuda.synchronize()
        fc1 = np.array([a.elapsed_ms(b) for a, b in evs]) * 1e3
        return c, total_ms / steps, fc1, wall

    def run_graph(self, name, steps, replicas, fmt="int4"):
        """The same K steps captured in one HIP graph and replayed (context)."""
        torch = self.torch
        c = self.prepare(name)
        layers = self.mxfp4_layers() if fmt == "mxfp4" else self.layers
        R = min(replicas, len(layers))
        self.step(c, layers[0], fmt=fmt)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                self.step(c, layers[i % R], fmt=fmt)
        g.replay()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        g.replay()
        stop.record()
        torch.cuda.synchronize()
        del g
        return start.elapsed_time(stop) / steps

    def record(self, name, steps, warmup, replicas, fmt="int4"):
        c, ms, fc1, wall = self.run(name, steps, warmup, replicas, fmt)
        fc1_us = float(np.mean(fc1))
        w, s, D = c["w"], self.s, c["D"]
        us = ms * 1e3
        lb = layer_bytes(D, w.M, s, fmt)
        r = dict(
            workload=name, M=w.M, block_m=c["B"], experts_touched=D, us_per_call=round(us, 2),
            us_per_token=round(us / w.M, 3), hbm_TBps=round(lb / (us * 1e-6) / 1e12, 3),
            mfma_pct=round(100 * flops(w.M, s) / (us * 1e-6) / (MFMA_BF16_PEAK_TFS * 1e12), 2),
            roofline_frac=round(max(lb / (HBM_PEAK_GBS * 1e9),
                                    flops(w.M, s) / (MFMA_BF16_PEAK_TFS * 1e12)) / (us * 1e-6), 4),
            fc1_us=round(fc1_us, 2), fc1_GBps=round(fc1_bytes(D, w.M, s, fmt) / (fc1_us * 1e-6) / 1e9, 1),
            fc1_us_p10_p50_p90=[round(float(v), 2) for v in np.percentile(fc1, [10, 50, 90])],
            replicas=min(replicas, len(self.layers)), wall_s=round(wall, 3))
        # the batch's grouping as the library computed it, and the inputs' hashes
        rb = c["rb"]
        ids = rb.topk_ids.cpu().numpy().reshape(-1)
        r["npp"] = int(rb.num_tokens_post_pad.item())
        r["max_per_expert"] = int(np.bincount(ids, minlength=s.E).max())
        t = c["t"]
        r["inputs_sha256_16"] = {"logits": hashlib.sha256(t.logits.tobytes()).hexdigest()[:16],
                                 "x_bf16": hashlib.sha256(t.x_bits.tobytes()).hexdigest()[:16]}
        if fmt != "int4":
            r["weights"] = fmt
        return r, c

    def cpu_baseline(self, c, budget_s=12.0):
        """The oracle (as it stands) on the headline batch, repeated for about
        budget_s seconds on one thread (BLAS limited to one thread), and the
        two costs the per-workload estimates are built from: dequantising one
        expert (W13 and W2, float64) and one expert MLP on one token."""
        import oracle
        import workloads as wl
        from threadpoolctl import threadpool_limits
        w13, s13, w2, s2 = self.host
        t = c["t"]
        x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
        with threadpool_limits(limits=1):
            cache = oracle.DequantCache(lambda e: (w13[e], s13[e], w2[e], s2[e]), max_items=0)
            tokens, n = 0, 0
            t0 = time.perf_counter()
            while True:
                oracle.layer(x, t.logits, self.s.k, cache)
                tokens += t.logits.shape[0]
                n += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            el = time.perf_counter() - t0
            # the parts: one expert's dequantisation, one expert MLP on one token
            reps = 3
            t1 = time.perf_counter()
            for e in range(reps):
                W13, W2 = cache(e)
            t_deq = (time.perf_counter() - t1) / reps
            t2 = time.perf_counter()
            for _ in range(20):
                oracle.expert_mlp(x[0], W13, W2)
            t_mlp = (time.perf_counter() - t2) / 20
        self.oracle_parts = (t_deq, t_mlp)
        host = len(os.sched_getaffinity(0))
        return {"value": round(el / tokens * 1e6, 1), "unit": "us/token", "cores": 1, "kind": "oracle",
                "host_cores": host, "blas_threads": 1,
                "dequant_expert_s": round(t_deq, 4), "expert_mlp_token_s": round(t_mlp, 5),
                "sample": f"{n} full oracle calls (route, dequantise the 8 experts in float64, expert MLPs, "
                          f"combine) on the {c['w'].M}-token batch, {el:.1f} s on one thread (numpy, BLAS limited "
                          f"to one thread) of a {host}-core host"}

    def cpu_estimate(self, r):
        """Oracle time per token for a sweep entry from the measured parts: each
        touched expert dequantised once (a cache holding the batch's experts)
        plus one expert MLP per (token, slot); one thread."""
        t_deq, t_mlp = self.oracle_parts
        M, D = r["M"], r["experts_touched"]
        return round((D * t_deq + M * self.s.k * t_mlp) / M * 1e6, 1)

    def attainable(self):
        """Attainable peaks measured here with the library's measurement
        kernels: the HBM read rate of one pass over 2 GiB (non-temporal 16-byte
        loads, the best of three grid sizes) and the fp16 matrix-core rate of
        back-to-back v_mfma_f32_16x16x32_f16 on register operands (~10 ms per
        launch, so the clock settles at its power limit). These are the
        denominators of frac_attainable. An 8192^3 torch bf16 matmul is
        reported as context."""
        torch, moe = self.torch, self.moe
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(fn, reps):
            fn()
            torch.cuda.synchronize()
            best = float("inf")
            for _ in range(reps):
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e-3)
            return best

        nbytes = 2 << 30
        buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        read = {}
        for per_cu in (2, 4, 8):
            sink = torch.empty(cus * per_cu * 256, dtype=torch.int32, device="cuda")
            read[per_cu] = nbytes / timed(lambda: moe.moe_calib_hbm_read(buf, sink), 5) / 1e9
            del sink
        del buf
        iters, wgs = 40000, 4 * cus
        sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        mfma = wgs * 4 * iters * 8 * 16384 / timed(lambda: moe.moe_calib_mfma_f16(iters, sink), 3) / 1e12
        del sink
        a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        tf = 2 * 8192 ** 3 / timed(lambda: torch.matmul(a, b), 5) / 1e12
        del a, b
        best = max(read, key=read.get)
        return {"hbm_GBps": round(read[best], 1), "f16_mfma_TFps": round(mfma, 1),
                "torch_bf16_matmul_TFps": round(tf, 1),
                "how": f"HBM: moe_calib_hbm_read over 2 GiB, best of {sorted(read)} workgroups per CU "
                       f"(best {best}); matrix core: moe_calib_mfma_f16, {iters} x 8 MFMAs per wave, "
                       f"{wgs} workgroups of 4 waves; torch matmul: 8192^3 bf16 (context)"}


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hip": torch.version.hip}


def traffic_for(launch_bytes_alg):
    """HBM bytes per FC1 launch from committed rocprofv3 counter runs, if they
    were taken on the current FC1 source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    return d.get("traffic_bytes_per_launch")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported "
              "(the library implements the one-GPU layer; sharding it over GPUs is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    b = Bench(a.replicas)
    if a.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fmt = a.weights
    head, c = b.record(a.workload, a.steps, a.warmup, a.replicas, fmt)
    s, D, M = b.s, c["D"], c["w"].M
    fc1_alg = fc1_bytes(D, M, s, fmt)
    fc1_s = head["fc1_us"] * 1e-6
    sweep = []
    if not a.no_sweep:
        for name in (a.sweep_list.split(",") if a.sweep_list else SWEEP):
            r, _ = b.record(name, a.sweep_steps, 5, a.replicas, fmt)
            sweep.append(r)
            print(f"# {json.dumps(r)}", file=sys.stderr, flush=True)
        warm, _ = b.record(a.workload, a.sweep_steps, 5, 1, fmt)
        warm["note"] = "one weight copy: consecutive steps may hit the last-level cache (context only)"
        sweep.append(warm)
    mxfp4 = []
    if not a.no_mxfp4 and fmt == "int4":
        for name in ([a.workload] if a.no_sweep else MXFP4_SWEEP):
            r, _ = b.record(name, a.sweep_steps, 5, a.replicas, fmt="mxfp4")
            mxfp4.append(r)
            print(f"# {json.dumps(r)}", file=sys.stderr, flush=True)
    cpu = None if a.no_cpu_baseline else b.cpu_baseline(c)
    att = b.attainable()
    for r in [head] + sweep + mxfp4:
        lb = layer_bytes(r["experts_touched"], r["M"], b.s, r.get("weights", "int4"))
        r["frac_attainable"] = round(max(lb / (att["hbm_GBps"] * 1e9), flops(r["M"], b.s) / (att["f16_mfma_TFps"] * 1e12))
                                     / (r["us_per_call"] * 1e-6), 4)
        if cpu is not None and r.get("weights", "int4") == "int4":
            r["cpu_us_per_token"] = b.cpu_estimate(r)
            r["cpu_cores"] = 1
    line = {
        "metric": "MoE layer us/token (+ achieved HBM TB/s, MFMA %) on the 384-expert INT4 g32 layer",
        "value": head["us_per_token"],
        "unit": "us/token",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random INT4 weights and router logits, bf16 N(0,1) activations)",
        "config": {"workload": f"{a.workload}: E=384, H=7168, I=2048, top-8, "
                               f"{'INT4 g32' if fmt == 'int4' else 'MXFP4'}, M={M} tokens",
                   "global_batch": M, "block_m": head["block_m"], "experts_touched": D,
                   "npp": head["npp"], "max_per_expert": head["max_per_expert"],
                   "inputs_sha256_16": head["inputs_sha256_16"],
                   "weight_copies_cycled": head["replicas"],
                   "launch": "eager, queued ahead of the GPU"},
        "graph_us_per_call": None if a.no_graph else round(b.run_graph(a.workload, a.steps, a.replicas, fmt) * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(fc1_alg / fc1_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(fc1_alg / fc1_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(fc1_alg) if fmt == "int4" else None,
                     "kernel": "FC1 stage (fc1_decode_kernel at M = 1, fc1_routed_kernel for few touched experts, "
                               "else the grouped FC1 kernel)",
                     "kernel_avg_us": head["fc1_us"], "algorithmic_bytes": fc1_alg},
        "layer": {k: head[k] for k in ("us_per_call", "hbm_TBps", "mfma_pct", "roofline_frac", "frac_attainable",
                                       "fc1_us_p10_p50_p90")},
        "attainable_peaks": att,
        "device": device_info(torch),
        "repack_ms": round(b.repack_ms, 2),
        "sweep": sweep,
        "mxfp4_sweep": mxfp4,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
