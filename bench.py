"""Benchmark of the quantized GEMV / mmq hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
quantize the activations to Q8_1 on the GPU, then run the product on the
quantized weights.  Default workload: the Q4_K decode GEMV at a Llama-3-8B FFN
shape (n = 14336, k = 4096).  Other workloads: --workload q8_0_gemv,
q6_k_gemv, q4_k_mmq, moe_q4_k, or all (one JSON line each); prefill products
with the other weight types q6_k_mmq, q8_0_mmq, q5_k_mmq; the Q5_K GEMV
q5_k_gemv (14336 x 4096); the 32-value types q4_0_gemv, q5_0_gemv (14336 x
4096), q4_0_mmq, q5_0_mmq; the RMSNorm + quantize
prologue rmsnorm_q8_1; the MoE router router_topk; small-batch GEMVs
<fmt>_gemv_b<B> (the GEMV workload's weights against B <= 8 activation rows),
or batch for the standard set of them.

Inputs are resident in HBM before timing starts.  The weights are replicated
into enough copies (>= 512 MB in total) that consecutive steps read different
copies, so the 256 MB Infinity Cache cannot serve them (--warm disables this).

Printed per workload: one JSON line with the step throughput (`value`), the
dominant kernel's roofline position measured with HIP events on the launch
stream, and the CPU oracle's throughput on a bounded sample of the same work
(the median of three runs on all the oracle's threads, and of three on one).

The default run (the Q4_K GEMV line) also carries `configs`: the same figures
for the five headline workloads (Q4_K, Q8_0 and Q6_K GEMVs, the Q4_K mmq and
the MoE), each against the published peak and against a peak measured in the
same run -- the best streaming read of the workload's own byte count (HBM) or
a loop of int8 MFMAs (mmq) -- listed under `peaks`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMV HBM GB/s (% of peak) and tokens/s-equivalent; mmq TOPS at M=512"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published
COLD_BYTES = 512 << 20       # rotate weight copies until at least this much
MALL_BYTES = 256 << 20       # MI355X Infinity Cache
PROFILE_DIR = os.path.join(ROOT, "profiles")


def q81_bytes(k):
    return (k // 32) * 36


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, run_s):
    """The oracle on the host cores: three runs on all its OpenMP threads and
    three on one; each run repeats the workload's bounded sample for at least
    run_s seconds.  `value` is the median over the all-threads runs."""
    import statistics

    import oracle
    fn, work, unit, sample = wl.cpu_sample()
    all_threads = oracle.max_threads()
    out = {}
    for threads in (all_threads, 1):
        oracle.set_threads(threads)
        rates, reps_done, secs = [], 0, 0.0
        for _ in range(3):
            reps, t = _repeat(fn, run_s)
            rates.append(reps * work / t / (1e9 if unit == "GB/s" else 1e12))
            reps_done, secs = reps_done + reps, secs + t
        out[threads] = (statistics.median(rates), reps_done, secs)
    oracle.set_threads(all_threads)
    v, reps, secs = out[all_threads]
    v1, reps1, secs1 = out[1]
    return dict(value=v, unit=unit, cores=all_threads, kind="oracle",
                sample=f"{sample}; median of 3 runs of >= {run_s:g} s ({reps} repetitions, {secs:.1f} s)",
                single_thread={"value": v1, "cores": 1, "repetitions": reps1, "seconds": round(secs1, 2)},
                nproc=os.cpu_count(), cpu_model=_cpu_model())


KERNEL_SOURCES = {
    "q4_k_gemv": ["qg_gemv.hip"], "q8_0_gemv": ["qg_gemv.hip"], "q6_k_gemv": ["qg_gemv.hip"],
    "q5_k_gemv": ["qg_gemv.hip"], "q4_0_gemv": ["qg_gemv.hip"], "q5_0_gemv": ["qg_gemv.hip"],
    "q4_0_mmq": ["qg_mmq.hip"], "q5_0_mmq": ["qg_mmq.hip"],
    "q4_k_mmq": ["qg_mmq.hip"], "q6_k_mmq": ["qg_mmq.hip"], "q8_0_mmq": ["qg_mmq.hip"], "q5_k_mmq": ["qg_mmq.hip"],
    "rmsnorm_q8_1": ["qg_quant.hip", "qg_quant.h"],
    "moe_q4_k": ["qg_moe.hip", "qg_quant.h"],
    "router_topk": ["qg_router.hip"],
}
GEMV_KERNEL = {"q8_0": "gemv_q8_0_pair_kernel", "q4_k": "gemv_q4k_kernel", "q6_k": "gemv_q6k_kernel",
               "q5_k": "gemv_q5k_kernel", "q4_0": "gemv_q4_0_kernel", "q5_0": "gemv_q5_0_kernel"}
BATCH_WORKLOADS = ["q8_0_gemv_b8", "q4_k_gemv_b2", "q4_k_gemv_b4", "q4_k_gemv_b8", "q6_k_gemv_b4", "q6_k_gemv_b8"]


def _sources(workload):
    if "_gemv_b" in workload:
        return ["qg_gemv_batch.hip", "qg_gemv_mfma.hip"]
    return KERNEL_SOURCES[workload]


def kernel_source_hash(workload):
    """sha256 over the kernel sources a workload's dominant kernel is built from."""
    import hashlib
    csrc = os.path.join(ROOT, "gemm_gguf_block_amd", "csrc")
    h = hashlib.sha256()
    for f in _sources(workload) + ["qg_blocks.h", "qg_device.h"]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def _traffic(workload):
    """HBM bytes per launch of the dominant kernel(s), from the committed
    counter summary: FETCH_SIZE and WRITE_SIZE, each scaled by what the same
    counter reads for a plain device copy of known size.  None when there is no
    summary or the kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))["workloads"].get(workload)
    except Exception:
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash(workload):
        return None
    return rec.get("bytes_per_launch")


def _repeat(fn, budget_s):
    """Run fn() until budget_s seconds have passed (at least once); (reps, secs)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        t = time.perf_counter() - t0
        if t >= budget_s:
            return reps, t


# ---------------------------------------------------------------- workloads
class Workload:
    """Holds device inputs and issues one step; subclasses define the work."""

    name = ""
    dominant = ""        # kernel name the roofline refers to

    def step(self, i):
        raise NotImplementedError

    def dominant_call(self, i):
        raise NotImplementedError


class Gemv(Workload):
    def __init__(self, qg, torch, name, warm):
        from gemm_gguf_block_amd import synth
        p = synth.WORKLOADS[name]
        self.name, self.fmt, self.n, self.k = name, p["fmt"], p["n"], p["k"]
        self.seed = p["seed"]
        self.qg, self.torch = qg, torch
        dev = torch.device("cuda:0")
        w = synth.weights(self.fmt, self.n, self.k, self.seed)
        self.w_host = w
        self.x_host = synth.normal(self.seed, synth.T_X, (self.k,))
        wbytes = w.nbytes
        self.copies = 1 if warm else max(1, math.ceil(COLD_BYTES / wbytes))
        W0 = torch.from_numpy(w).to(dev)
        self.W = [W0] + [W0.clone() for _ in range(self.copies - 1)]
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.xq = torch.empty(q81_bytes(self.k), dtype=torch.uint8, device=dev)
        self.y = torch.empty(self.n, dtype=torch.float32, device=dev)
        self.fn = getattr(qg, "qgemv_" + self.fmt)
        self.dominant = GEMV_KERNEL[self.fmt]
        # algorithmic bytes: every weight byte once, the activation, the output
        self.kernel_bytes = wbytes + q81_bytes(self.k) + 4 * self.n
        self.step_bytes = self.kernel_bytes + 4 * self.k + q81_bytes(self.k)  # + quantize's f32 read / Q8_1 write
        self.tokens_per_step = 1
        self.unit, self.bound = "GB/s", "hbm"

    def step(self, i):
        self.qg.quantize_q8_1(self.x, self.xq)
        self.fn(self.W[i % self.copies], self.xq, self.n, self.k, y=self.y)

    def dominant_call(self, i):
        self.fn(self.W[i % self.copies], self.xq, self.n, self.k, y=self.y)

    def value(self, sec_per_step):
        return self.step_bytes / sec_per_step / 1e9

    def kernel_rate(self, sec):
        return self.kernel_bytes / sec / 1e9

    def cpu_sample(self):
        import numpy as np

        import oracle
        xq = oracle.quantize_q8_1(self.x_host[None])[0]
        sel = np.arange(min(self.n, 16384), dtype=np.int64)
        nb = sel.size * self.w_host.shape[1] + q81_bytes(self.k) + 4 * sel.size
        return (lambda: oracle.qgemv(self.fmt, self.w_host, xq, self.n, self.k, rows=sel), nb, "GB/s",
                f"rows 0..{sel.size - 1} of {self.n} (plain double dequant-and-dot)")


class GemvBatch(Gemv):
    """`<fmt>_gemv_b<B>`: the batch-1 workload's weights against B activation
    rows (B concurrent decode sequences); weights are read once per step."""

    def __init__(self, qg, torch, name, warm):
        base, b = name.rsplit("_b", 1)
        super().__init__(qg, torch, base, warm)
        from gemm_gguf_block_amd import synth
        self.name, self.b = name, int(b)
        dev = torch.device("cuda:0")
        self.x_host = synth.normal(self.seed, synth.T_X, (self.b, self.k))
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.xq = torch.empty((self.b, q81_bytes(self.k)), dtype=torch.uint8, device=dev)
        self.y = torch.empty((self.b, self.n), dtype=torch.float32, device=dev)
        self.fn = getattr(qg, "qgemv_" + self.fmt + "_batch")
        # the kernel the batch call dispatches to at these shapes (k a multiple of 256): the
        # matrix cores for Q4_K from 2 rows, Q6_K from 3, Q8_0 from 5
        mfma = self.b > {"q4_k": 1, "q6_k": 2, "q8_0": 4}[self.fmt]
        self.dominant = ({"q8_0": "gemv_batch_mfma_q8_0", "q4_k": "gemv_batch_mfma_q4k",
                          "q6_k": "gemv_batch_mfma_q6k"}[self.fmt] if mfma else "gemv_batch_kernel")
        wbytes = self.w_host.nbytes
        self.kernel_bytes = wbytes + self.b * (q81_bytes(self.k) + 4 * self.n)
        self.step_bytes = self.kernel_bytes + self.b * (4 * self.k + q81_bytes(self.k))
        self.tokens_per_step = self.b

    def step(self, i):
        self.qg.quantize_q8_1(self.x, self.xq)
        self.fn(self.W[i % self.copies], self.xq, self.b, self.n, self.k, y=self.y)

    def dominant_call(self, i):
        self.fn(self.W[i % self.copies], self.xq, self.b, self.n, self.k, y=self.y)

    def cpu_sample(self):
        import numpy as np

        import oracle
        xq = oracle.quantize_q8_1(self.x_host)
        sel = np.arange(min(self.n, 16384 // self.b), dtype=np.int64)

        def once():
            for i in range(self.b):
                oracle.qgemv(self.fmt, self.w_host, xq[i], self.n, self.k, rows=sel)
        nb = sel.size * self.w_host.shape[1] + self.b * (q81_bytes(self.k) + 4 * sel.size)
        return (once, nb, "GB/s", f"rows 0..{sel.size - 1} of {self.n} against {self.b} activation rows "
                                  f"(plain double dequant-and-dot per row)")


class RmsnormQ81(Workload):
    """`rmsnorm_q8_1`: x (f32 [rows][k]) -> Q8_1((x * r) * gamma) per row in one
    launch.  The same work as two launches (torch's rms_norm writing f32, then
    quantize_q8_1) is timed alongside as `alt_call`."""

    def __init__(self, qg, torch, warm):
        from gemm_gguf_block_amd import synth
        p = synth.WORKLOADS["rmsnorm_q8_1"]
        self.name, self.rows, self.k, self.eps = "rmsnorm_q8_1", p["rows"], p["k"], p["eps"]
        self.qg, self.torch = qg, torch
        dev = torch.device("cuda:0")
        self.x_host = synth.normal(p["seed"], synth.T_X, (self.rows, self.k))
        self.g_host = (1.0 + 0.25 * synth.normal(p["seed"], synth.T_W, (self.k,))).astype("float32")
        self.copies = 1 if warm else max(1, math.ceil(COLD_BYTES / self.x_host.nbytes))
        X0 = torch.from_numpy(self.x_host).to(dev)
        self.X = [X0] + [X0.clone() for _ in range(self.copies - 1)]
        self.gamma = torch.from_numpy(self.g_host).to(dev)
        self.xq = torch.empty((self.rows, q81_bytes(self.k)), dtype=torch.uint8, device=dev)
        self.dominant = "rmsnorm_quantize_q8_1_kernel"
        self.kernel_bytes = self.x_host.nbytes + 4 * self.k + self.rows * q81_bytes(self.k)
        self.step_bytes = self.kernel_bytes
        self.tokens_per_step = self.rows
        self.unit, self.bound = "GB/s", "hbm"

    def step(self, i):
        self.qg.rmsnorm_quantize_q8_1(self.X[i % self.copies], self.gamma, self.eps, xq=self.xq)

    def dominant_call(self, i):
        self.step(i)

    def alt_call(self, i):
        F = self.torch.nn.functional
        y = F.rms_norm(self.X[i % self.copies], (self.k,), self.gamma, self.eps)
        self.qg.quantize_q8_1(y, self.xq)

    alt_what = "torch rms_norm (f32 out), then quantize_q8_1"

    def value(self, sec_per_step):
        return self.step_bytes / sec_per_step / 1e9

    def kernel_rate(self, sec):
        return self.kernel_bytes / sec / 1e9

    def cpu_sample(self):
        import numpy as np

        import oracle
        rows = min(self.rows, 64)
        x = self.x_host[:rows]

        def once():
            r = oracle.rms_scale(x, self.eps).astype(np.float32)
            oracle.quantize_q8_1((x * r[:, None]) * self.g_host[None, :])
        return (once, rows * (4 * self.k + q81_bytes(self.k)), "GB/s",
                f"rows 0..{rows - 1} of {self.rows} (double RMS scale, f32 products, quantize)")


class Mmq(Workload):
    def __init__(self, qg, torch, name, warm):
        from gemm_gguf_block_amd import synth
        p = synth.WORKLOADS[name]
        self.name, self.fmt, self.m, self.n, self.k = name, p["fmt"], p["m"], p["n"], p["k"]
        self.qg, self.torch = qg, torch
        self.fn = getattr(qg, f"qgemm_{self.fmt}_mmq")
        dev = torch.device("cuda:0")
        w = synth.weights(self.fmt, self.n, self.k, p["seed"])
        self.w_host = w
        self.a_host = synth.normal(p["seed"], synth.T_X, (self.m, self.k))
        self.copies = 1 if warm else max(1, math.ceil(COLD_BYTES / w.nbytes))
        W0 = torch.from_numpy(w).to(dev)
        self.W = [W0] + [W0.clone() for _ in range(self.copies - 1)]
        self.a = torch.from_numpy(self.a_host).to(dev)
        self.aq = torch.empty((self.m, q81_bytes(self.k)), dtype=torch.uint8, device=dev)
        self.c = torch.empty((self.m, self.n), dtype=torch.float32, device=dev)
        self.dominant = f"mmq_kernel<{self.fmt}>"
        self.ops = 2.0 * self.m * self.n * self.k
        self.kernel_bytes = w.nbytes + self.m * q81_bytes(self.k) + 4 * self.m * self.n
        self.tokens_per_step = self.m
        self.unit, self.bound = "TOPS", "mfma"

    def step(self, i):
        self.qg.quantize_q8_1(self.a, self.aq)
        self.fn(self.W[i % self.copies], self.aq, self.m, self.n, self.k, c=self.c)

    def dominant_call(self, i):
        self.fn(self.W[i % self.copies], self.aq, self.m, self.n, self.k, c=self.c)

    def value(self, sec_per_step):
        return self.ops / sec_per_step / 1e12

    def kernel_rate(self, sec):
        return self.ops / sec / 1e12

    def cpu_sample(self):
        import numpy as np

        import oracle
        aq = oracle.quantize_q8_1(self.a_host)
        g = np.random.default_rng(0)
        cnt = 1 << 14
        pairs = np.stack([g.integers(0, self.m, cnt), g.integers(0, self.n, cnt)], 1)
        return (lambda: oracle.qgemm(self.fmt, self.w_host, aq, self.m, self.n, self.k, pairs=pairs),
                2.0 * cnt * self.k, "TOPS", f"{cnt} random entries of C[{self.m}][{self.n}] (plain double "
                                            f"dequant-and-dot)")


class Moe(Workload):
    def __init__(self, qg, torch, warm):
        import numpy as np

        from gemm_gguf_block_amd import synth
        p = synth.WORKLOADS["moe_q4_k"]
        self.name = "moe_q4_k"
        self.E, self.F, self.H, self.T, self.K = p["n_expert"], p["n_ff"], p["n_embd"], p["n_tok"], p["top_k"]
        self.qg, self.torch = qg, torch
        dev = torch.device("cuda:0")
        inp = synth.workload("moe_q4_k")
        self.inp = inp
        wbytes = inp["w_gu"].nbytes + inp["w_down"].nbytes
        self.copies = 1 if warm else max(1, math.ceil(COLD_BYTES / wbytes))
        gu0, dn0 = torch.from_numpy(inp["w_gu"]).to(dev), torch.from_numpy(inp["w_down"]).to(dev)
        self.Wgu = [gu0] + [gu0.clone() for _ in range(self.copies - 1)]
        self.Wdn = [dn0] + [dn0.clone() for _ in range(self.copies - 1)]
        self.x = torch.from_numpy(inp["x"]).to(dev)
        self.ids = torch.from_numpy(inp["ids"]).to(dev)
        self.rw = torch.from_numpy(inp["weights"]).to(dev)
        self.xq = torch.empty((self.T, q81_bytes(self.H)), dtype=torch.uint8, device=dev)
        self.out = torch.empty((self.T, self.H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(qg.moe_qgemv_q4_k_workspace_size(self.T, self.K, self.E, self.F, self.H),
                              dtype=torch.uint8, device=dev)
        self.distinct = int(np.unique(inp["ids"]).size)
        per_expert = wbytes // self.E
        self.dominant = f"moe ({qg.moe_launches(self.T, self.K, self.E, self.F, self.H)} kernels)"
        self.kernel_bytes = self.distinct * per_expert + self.T * q81_bytes(self.H) + 4 * self.T * self.H
        self.step_bytes = self.kernel_bytes + 4 * self.T * self.H + self.T * q81_bytes(self.H)
        self.tokens_per_step = self.T
        self.unit, self.bound = "GB/s", "hbm"

    def _moe(self, i):
        c = i % self.copies
        self.qg.moe_qgemv_q4_k(self.Wgu[c], self.Wdn[c], self.xq, self.ids, self.rw, self.T, self.K, self.E, self.F,
                               self.H, out=self.out, workspace=self.ws)

    def step(self, i):
        self.qg.quantize_q8_1(self.x, self.xq)
        self._moe(i)

    def dominant_call(self, i):
        self._moe(i)

    def value(self, sec_per_step):
        return self.step_bytes / sec_per_step / 1e9

    def kernel_rate(self, sec):
        return self.kernel_bytes / sec / 1e9

    def cpu_sample(self):
        import oracle
        inp = self.inp
        T = self.T
        xq = oracle.quantize_q8_1(inp["x"])
        nb = self.distinct * (inp["w_gu"].nbytes + inp["w_down"].nbytes) // self.E
        return (lambda: oracle.moe_q4_k(inp["w_gu"], inp["w_down"], xq, inp["ids"], inp["weights"], T, self.K,
                                        self.E, self.F, self.H), nb, "GB/s",
                f"all {T} tokens ({self.distinct} distinct experts)")


class Router(Workload):
    """`router_topk`: logits of an f32 router, then top-k and softmax."""

    def __init__(self, qg, torch, warm):
        from gemm_gguf_block_amd import synth
        inp = synth.workload("router_topk")
        self.inp, self.name = inp, "router_topk"
        self.E, self.H, self.T, self.K = inp["n_expert"], inp["n_embd"], inp["n_tok"], inp["top_k"]
        self.qg, self.torch = qg, torch
        dev = torch.device("cuda:0")
        wr = inp["w_router"]
        self.copies = 1 if warm else max(1, math.ceil(COLD_BYTES / wr.nbytes))
        W0 = torch.from_numpy(wr).to(dev)
        self.W = [W0] + [W0.clone() for _ in range(self.copies - 1)]
        self.x = torch.from_numpy(inp["x"]).to(dev)
        self.ids = torch.empty((self.T, self.K), dtype=torch.int32, device=dev)
        self.rw = torch.empty((self.T, self.K), dtype=torch.float32, device=dev)
        self.logits = torch.empty((self.T, self.E), dtype=torch.float32, device=dev)
        self.dominant = "router (2 kernels)"
        # router and tokens read, logits written and read back, ids and weights written
        self.kernel_bytes = wr.nbytes + inp["x"].nbytes + 8 * self.T * self.E + 8 * self.T * self.K
        self.step_bytes = self.kernel_bytes
        self.tokens_per_step = self.T
        self.unit, self.bound = "GB/s", "hbm"

    def step(self, i):
        self.qg.moe_router_topk(self.W[i % self.copies], self.x, self.K, ids=self.ids, weights=self.rw,
                                logits=self.logits)

    def dominant_call(self, i):
        self.step(i)

    def value(self, sec_per_step):
        return self.step_bytes / sec_per_step / 1e9

    def kernel_rate(self, sec):
        return self.kernel_bytes / sec / 1e9

    def cpu_sample(self):
        import oracle
        inp = self.inp

        def once():
            oracle.route_topk(oracle.router_logits(inp["w_router"], inp["x"]).astype("float32"), self.K)
        return once, self.kernel_bytes, "GB/s", f"all {self.T} tokens (double logits, top-k, softmax)"


def make(name, qg, torch, warm):
    if "_gemv_b" in name:
        return GemvBatch(qg, torch, name, warm)
    if name.endswith("_gemv"):
        return Gemv(qg, torch, name, warm)
    if name.endswith("_mmq"):
        return Mmq(qg, torch, name, warm)
    if name == "rmsnorm_q8_1":
        return RmsnormQ81(qg, torch, warm)
    if name == "moe_q4_k":
        return Moe(qg, torch, warm)
    if name == "router_topk":
        return Router(qg, torch, warm)
    raise SystemExit(f"unknown workload {name}")


# ---------------------------------------------------------------- timing
def _time(fn, first, count, warmup, torch, graph, spinup):
    """Average ms per call of fn(i) over `count` calls, timed with HIP events on
    the stream the calls launch on.  With graph=True the calls are captured in a
    HIP graph (after `warmup` eager calls) and the graph is replayed untimed,
    then once timed: the device work is identical, host launch overhead is
    removed.  The untimed part lasts at least `spinup` seconds of back-to-back
    work, so the timed calls run at the clock the GPU sustains under load
    rather than one still ramping up from idle."""
    if not graph:
        t0 = time.perf_counter()
        i = 0
        while i < warmup or time.perf_counter() - t0 < spinup:
            fn(i)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(count):
            fn(first + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / count
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                fn(first + i)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        t0 = time.perf_counter()
        while True:
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= spinup:
                break
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / count


def run(wl, steps, warmup, torch, graph, spinup):
    ms_step = _time(wl.step, warmup, steps, warmup, torch, graph, spinup)
    ms_kernel = _time(wl.dominant_call, warmup, steps, warmup, torch, graph, spinup)
    return ms_step, ms_kernel


def bench_one(name, args, qg, torch, cpu_run_s=None):
    t_setup = time.time()
    wl = make(name, qg, torch, args.warm)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    ms_step, ms_kernel = run(wl, args.steps, args.warmup, torch, not args.no_graph, args.spinup)
    value = wl.value(ms_step / 1e3)
    achieved = wl.kernel_rate(ms_kernel / 1e3)
    peak = HBM_PEAK_GBS if wl.unit == "GB/s" else INT8_PEAK_TOPS
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": wl.unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": name, "hip_graph": not args.no_graph, "spinup_s": args.spinup},
        "tokens_per_s_equiv": round(wl.tokens_per_step / (ms_step / 1e3), 1),
        "roofline": {
            "bound": wl.bound,
            "kernel": wl.dominant,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "GB/s" if wl.unit == "GB/s" else "TOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": _traffic(name),
            "ms_per_launch": round(ms_kernel, 6),
            "algorithmic_per_launch": wl.kernel_bytes if wl.unit == "GB/s" else wl.ops,
        },
    }
    if wl.unit == "GB/s":
        rec["pct_of_hbm_peak"] = round(100.0 * value / HBM_PEAK_GBS, 2)
    cfg = rec["config"]
    for key in ("fmt", "b", "m", "n", "k", "rows", "E", "F", "H", "T", "K"):
        if hasattr(wl, key):
            cfg[key] = getattr(wl, key)
    cfg["weight_copies"] = wl.copies
    if name == "moe_q4_k":
        cfg["distinct_experts"] = wl.distinct
    if hasattr(wl, "alt_call"):
        ms_alt = _time(wl.alt_call, args.warmup, args.steps, args.warmup, torch, not args.no_graph, args.spinup)
        rec["comparison"] = {"what": wl.alt_what, "ms_per_step": round(ms_alt, 6)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_run if cpu_run_s is None else cpu_run_s)
    print(f"[bench] {name}: setup {setup_s:.1f} s, step {ms_step * 1e3:.2f} us, "
          f"{wl.dominant} {ms_kernel * 1e3:.2f} us/launch", file=sys.stderr, flush=True)
    del wl
    torch.cuda.empty_cache()
    return rec


def warm_figure(name, args, qg, torch):
    """The dominant kernel with one weight copy, reused call after call, so
    that weights of up to 256 MB stay in the Infinity Cache (MALL) between
    calls: a labelled side figure, never the headline."""
    wl = make(name, qg, torch, True)
    torch.cuda.synchronize()
    ms_kernel = _time(wl.dominant_call, args.warmup, args.steps, args.warmup, torch, not args.no_graph, args.spinup)
    achieved = wl.kernel_rate(ms_kernel / 1e3)
    fits = wl.unit != "GB/s" or wl.kernel_bytes <= MALL_BYTES
    out = {"us_per_launch": round(ms_kernel * 1e3, 3), "achieved": round(achieved, 3),
           "unit": "GB/s" if wl.unit == "GB/s" else "TOP/s",
           "what": "one weight copy reused by every call" +
                   ("; it fits the 256 MB Infinity Cache" if fits else "; larger than the 256 MB Infinity Cache")}
    del wl
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ measured peaks
# Launch shapes of the streaming-read reference: grid x threads, loads in
# flight per thread, non-temporal or plain.
READ_SWEEP = [(g, t, l, nt) for g in (256, 512, 1024) for t in (256, 512) for l in (4, 8) for nt in (1, 0)]


def peak_read(qg, torch, nbytes, args):
    """Best rate (GB/s) of the streaming-read reference over READ_SWEEP for a
    buffer of nbytes (rounded up to 16), on copies rotating past the Infinity
    Cache like the weights of the workloads; each shape timed as a HIP graph of
    args.steps launches after args.spinup seconds of untimed replays."""
    nbytes = (nbytes + 15) // 16 * 16
    copies = 1 if args.warm else max(1, math.ceil(COLD_BYTES / nbytes))
    dev = torch.device("cuda:0")
    bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.empty(max(g for g, _, _, _ in READ_SWEEP), dtype=torch.int32, device=dev)
    best = None
    for j, (g, t, l, nt) in enumerate(READ_SWEEP):
        def call(i):
            qg.peak_read(bufs[i % copies], g, t, l, nt, sink)
        # the first shape spins the clock up; the rest follow back to back
        ms = _time(call, args.warmup, args.steps, args.warmup, torch, not args.no_graph,
                   args.spinup if j == 0 else min(args.spinup, 0.05))
        rate = nbytes / (ms / 1e3) / 1e9
        if best is None or rate > best["GB/s"]:
            best = {"GB/s": round(rate, 1), "us": round(ms * 1e3, 3), "grid": g, "threads": t, "loads": l,
                    "nontemporal": bool(nt)}
    del bufs
    torch.cuda.empty_cache()
    best["bytes"] = nbytes
    best["copies"] = copies
    return best


def peak_mfma_i8(qg, torch, args, iters=1000):
    """Rate (TOP/s) of a loop of int8 MFMAs filling every SIMD."""
    dev = torch.device("cuda:0")
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    ops = qg.peak_mfma_i8(iters, sink)
    ms = _time(lambda i: qg.peak_mfma_i8(iters, sink), args.warmup, args.steps, args.warmup, torch,
               not args.no_graph, args.spinup)
    return {"TOP/s": round(ops / (ms / 1e3) / 1e12, 1), "us": round(ms * 1e3, 3), "ops_per_launch": ops}


HEADLINE = ["q4_k_gemv", "q8_0_gemv", "q6_k_gemv", "q4_k_mmq", "moe_q4_k"]


def config_entry(rec, peak):
    """The compact per-workload figures of the `configs` list."""
    rf = rec["roofline"]
    meas = peak["GB/s"] if rf["unit"] == "GB/s" else peak["TOP/s"]
    e = {
        "workload": rec["config"]["workload"],
        "config": {k: v for k, v in rec["config"].items() if k not in ("workload", "hip_graph", "spinup_s")},
        "kernel": rf["kernel"],
        "us_per_launch": round(rf["ms_per_launch"] * 1e3, 3),
        "us_per_step": round(rec["ms_per_step"] * 1e3, 3),
        "achieved": rf["achieved"],
        "unit": rf["unit"],
        "frac_of_published_peak": rf["frac"],
        "measured_peak": meas,
        "frac_of_measured_peak": round(rf["achieved"] / meas, 4),
        "step_value": rec["value"],
        "step_unit": rec["unit"],
        "tokens_per_s_equiv": rec["tokens_per_s_equiv"],
        "algorithmic_per_launch": rf["algorithmic_per_launch"],
        "traffic": rf["traffic"],
    }
    if "cpu_baseline" in rec:
        e["cpu_baseline"] = rec["cpu_baseline"]
    return e


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--spinup", type=float, default=1.0,
                    help="minimum seconds of untimed back-to-back calls before each timed region")
    ap.add_argument("--workload", default="q4_k_gemv",
                    help="q4_k_gemv (default; with the `configs` list), q8_0_gemv, q6_k_gemv, q4_k_mmq, moe_q4_k, "
                         "all (these five, one line each), "
                         "q6_k_mmq, q8_0_mmq, rmsnorm_q8_1, q5_k_gemv, q5_k_mmq, router_topk, q4_0_gemv, q5_0_gemv, "
                         "q4_0_mmq, q5_0_mmq, "
                         "a small-batch GEMV <fmt>_gemv_b<B> (B <= 8), or batch (" + ", ".join(BATCH_WORKLOADS) + ")")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload only: leave out the `configs` list and the measured peaks")
    ap.add_argument("--warm", action="store_true", help="one weight copy (Infinity-Cache-resident for small ones)")
    ap.add_argument("--no-graph", action="store_true", help="launch every call from the host (no HIP graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-run", type=float, default=1.5,
                    help="seconds per oracle timing run of the printed workload (3 runs on all threads, 3 on one)")
    ap.add_argument("--cpu-run-configs", type=float, default=0.4,
                    help="seconds per oracle timing run of each other entry of the `configs` list")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="instead of benchmarking, run 10 plain device copies of MiB mebibytes (a kernel of known "
                         "traffic, to scale HBM counters by) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import gemm_gguf_block_amd as qg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 10}))
        return
    if args.workload == "q4_k_gemv" and not args.no_configs:
        t0 = time.time()
        recs = {}
        for name in HEADLINE:
            run_s = args.cpu_run if name == "q4_k_gemv" else args.cpu_run_configs
            recs[name] = bench_one(name, args, qg, torch, cpu_run_s=run_s)
        peaks = {"hbm_read": {}, "mfma_i8": peak_mfma_i8(qg, torch, args)}
        entries = []
        for name in HEADLINE:
            rec = recs[name]
            if rec["roofline"]["unit"] == "GB/s":
                nb = rec["roofline"]["algorithmic_per_launch"]
                pk = peaks["hbm_read"].setdefault(name, peak_read(qg, torch, nb, args))
            else:
                pk = peaks["mfma_i8"]
            entries.append(config_entry(rec, pk))
            entries[-1]["warm"] = warm_figure(name, args, qg, torch)
            print(f"[bench] {name}: {entries[-1]['frac_of_published_peak']:.3f} of published, "
                  f"{entries[-1]['frac_of_measured_peak']:.3f} of measured peak; warm "
                  f"{entries[-1]['warm']['us_per_launch']:.2f} us/launch", file=sys.stderr, flush=True)
        head = recs["q4_k_gemv"]
        head["configs"] = entries
        head["peaks"] = peaks
        head["roofline"]["measured_peak"] = entries[0]["measured_peak"]
        head["roofline"]["frac_of_measured_peak"] = entries[0]["frac_of_measured_peak"]
        head["bench_wall_s"] = round(time.time() - t0, 1)
        print(json.dumps(head), flush=True)
        return
    names = (HEADLINE if args.workload == "all"
             else BATCH_WORKLOADS if args.workload == "batch" else [args.workload])
    for name in names:
        rec = bench_one(name, args, qg, torch)
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
