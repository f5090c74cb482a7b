"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one moe_layer_forward (route, permute, grouped gate/up + SiLU*mul GEMM,
grouped down GEMM, combine) over the workload's seeded synthetic batch, all inputs
resident in HBM. The default workload is the largest single-GPU layer, the DeepSeek-V3-style
one (T=16384, d=7168, f=2048, E=256 routed experts, top-8, sigmoid gates, one shared expert,
22.6 GB of bf16 weights). Prints ONE JSON line (rank 0):
  value      routed tokens per second (T * K / elapsed over the K timed steps)
  roofline   the gated grouped GEMM (the dominant kernel): algorithmic FLOPs per launch
             (4 d f N_kept, + 4 d f_s T for the shared experts) / its average launch time,
             HIP events recorded around that launch on the layer's stream inside the timed
             steps, against 2.5 PFLOP/s
  routing    expert loads, drops and near-tie tokens of the batch (outside the timed steps)
  parity     the run's output against the oracle on the CPU baseline's tokens
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
Decode workloads (T <= 64) are bound by the touched experts' weight bytes (the weight-streaming
kernels; bf16 batches averaging 8 or more rows per expert take the tiled GEMM): there the
roofline is the gated launch's algorithmic bytes (touched experts' gate and up weights as
stored, token rows in, h out) per launch time, against 8 TB/s. The mixtral_decode_fp8_*
workloads run the same layer with FP8 E4M3 expert weights (moe_layer_forward_fp8).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
SMALL_BATCH_TOKENS = 64  # decode batches: up to this size the step is bound by the weight bytes
SMALL_ROWS_PER_EXPERT = 8  # bf16 decode batches with T*k < 8*E take the weight-streaming kernels


def weight_streaming(T: int, k: int, E: int, fp8: bool) -> bool:
    """Whether the library runs a decode batch on its weight-streaming kernels (FP8 weights
    always; bf16 while the experts average fewer than 8 rows) rather than the tiled GEMM."""
    return T <= SMALL_BATCH_TOKENS and (fp8 or T * k < SMALL_ROWS_PER_EXPERT * E)
METRIC = "routed tokens/sec per MoE layer; % of bf16 MFMA peak (prefill) / HBM peak (decode)"


class HipEvents:
    """hipEvent_t pairs through the HIP runtime (recorded by libmoe on its launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> ctypes.c_void_p:
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b) -> float:
        assert self.hip.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def kernel_source_hash(name: str) -> str:
    from sparse_mixture_experts_29_amd.traffic_summary import source_hash
    return source_hash(os.path.join(ROOT, "sparse_mixture_experts_29_amd", "csrc", name))


def graph_steps(step, K: int, warmup: int, torch):
    """One call of step() captured in a HIP graph (torch.cuda.CUDAGraph), then warmup + K
    replays on the current stream, each timed with a pair of events. Returns per-replay ms."""
    import numpy as np
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def traffic_from_profile(kernel_file: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current source of the kernel; otherwise None."""
    p = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        rec = d.get(workload)
        if rec and rec.get("source_sha256_16") == kernel_source_hash(kernel_file):
            return rec.get("hbm_bytes_per_launch")
    except (ValueError, OSError):
        return None
    return None


def time_steps(step, K: int, warmup: int, stream, kernel=None):
    """Warm up, then time exactly K calls of step() on `stream`, bracketing one launch of
    `kernel` (default: the gated launch) in each with HIP events (moe_time_next_launch).
    Returns (wall seconds, per-step ms, per-step ms of that launch)."""
    import numpy as np
    import torch

    from sparse_mixture_experts_29_amd import binding
    if kernel is None:
        kernel = binding.MOE_KERNEL_GATE_UP
    ev = HipEvents()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    begins = [ev.create() for _ in range(K)]
    ends = [ev.create() for _ in range(K)]
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ev[0].record(stream)
    for i in range(K):
        binding.moe_time_next_launch(kernel, begins[i], ends[i])
        step()
        step_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = np.array([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(K)])
    gate_up_ms = np.array([ev.elapsed_ms(begins[i], ends[i]) for i in range(K)])
    for e in begins + ends:
        ev.destroy(e)
    return elapsed, step_ms, gate_up_ms


# an oracle run shorter than this is repeated three times (median reported)
CPU_REPEAT_BELOW_S = 5.0


def blas_name(info) -> str:
    """The BLAS library numpy runs the oracle's products on (threadpoolctl's report)."""
    libs = [f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info if i.get("user_api") == "blas"]
    return ", ".join(libs) or "unknown"


def sample_clocks(step, want: int = 2, seconds: float = 8.0) -> dict:
    """rocm-smi's current clocks, read (want times, at most `seconds`) while step() runs in a
    loop on the GPU after the timed steps; the clocks are not controlled. On any failure the
    reason is returned instead of samples."""
    import shutil
    import subprocess
    import threading

    import torch
    tool = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    samples, errors = [], []

    def poll():
        t_end = time.time() + seconds
        while time.time() < t_end and len(samples) < want:
            try:
                r = subprocess.run([tool, "--showclocks", "--json"], capture_output=True, text=True,
                                   timeout=seconds)
                got = {}
                for card in json.loads(r.stdout).values():  # every card-like entry
                    if isinstance(card, dict):
                        # "<clk> clock speed:" holds the frequency, "<clk> clock level:" the DPM
                        # level; keep both under distinct names
                        for key, v in card.items():
                            kl = key.lower()
                            if "clk" not in kl and "clock" not in kl:
                                continue
                            name = key.split(" clock")[0].strip() + ("_level" if "level" in kl else "")
                            got[name] = str(v).strip("()")
                if not got:
                    errors.append("no clock fields in: " + r.stdout[:200])
                    return
                samples.append(got)
            except Exception as e:  # the tool is missing, refused or printed something else
                errors.append(f"{type(e).__name__}: {e}"[:200])
                return

    th = threading.Thread(target=poll)
    th.start()
    while th.is_alive():
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    th.join()
    out = {"tool": "rocm-smi --showclocks --json", "while": "layer steps after the timed ones", "samples": samples}
    if errors:
        out["error"] = errors[0]
    return out


def cold_steps(step, K: int, stream, flush_mib: int, mode: str = "read"):
    """K steps, each after streaming a flush_mib MiB scratch buffer through the caches so that
    the MALL holds none of the weights; each step timed alone with events around it (the flush
    is not timed). mode "read" sums the buffer (clean lines only); "write" fills it, which
    also leaves dirty lines whose write-back then lands inside the step.
    Returns (per-step ms, per-step ms of the gated launch)."""
    import numpy as np
    import torch

    from sparse_mixture_experts_29_amd import binding
    ev = HipEvents()
    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda:0")
    begins = [ev.create() for _ in range(K)]
    ends = [ev.create() for _ in range(K)]
    se = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    buf.fill_(1)
    for i in range(K):
        if mode == "write":
            buf.fill_(i & 0xFF)
        else:
            buf.sum()
        se[i][0].record(stream)
        binding.moe_time_next_launch(binding.MOE_KERNEL_GATE_UP, begins[i], ends[i])
        step()
        se[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in se])
    gate_ms = np.array([ev.elapsed_ms(begins[i], ends[i]) for i in range(K)])
    for e in begins + ends:
        ev.destroy(e)
    del buf
    return step_ms, gate_ms


def shard_bench(args, w):
    """One GPU's share of an expert-parallel layer: route the whole layer on the GPU, keep
    the rows whose experts this shard owns, and time moe_expert_shard_forward on them."""
    import numpy as np
    import torch

    from sparse_mixture_experts_29_amd import binding
    from sparse_mixture_experts_29_amd.device import ExpertShard, host_to_device, shard_rows
    from sparse_mixture_experts_29_amd.inputs import make_inputs

    cfg = w.layer
    binding.load_library()
    li = make_inputs(cfg)
    dev = torch.device("cuda:0")
    x = host_to_device(li.x, cfg, dev)
    wr = host_to_device(li.w_router, cfg, dev)
    bias = None if li.router_bias is None else torch.from_numpy(li.router_bias).to(dev)
    idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    binding.moe_route(cfg, x, wr, bias, idx, gate, None)
    tok, slot, local = shard_rows(idx.cpu().numpy(), w.n_shards, w.shard, cfg.n_experts)
    del wr, idx, gate
    sh = ExpertShard.from_inputs(li, w.n_shards, w.shard, x, tok, local, threads=16)
    torch.cuda.synchronize()
    R = len(tok)
    per = cfg.n_experts // w.n_shards
    loads = np.bincount(local, minlength=per)
    elapsed, step_ms, gate_up_ms = time_steps(sh.forward, args.steps, args.warmup, torch.cuda.current_stream())
    K = args.steps
    es = 2 if cfg.dtype == "bf16" else 4
    flops_gate_up = 4.0 * cfg.d_model * cfg.d_ff * R
    if cfg.dtype == "bf16" and R <= SMALL_BATCH_TOKENS:
        touched = int((loads > 0).sum())
        bytes_gate_up = float(touched * cfg.gate_up_bytes(cfg.d_ff)) + R * cfg.d_model * es + R * cfg.d_ff * es
        achieved = bytes_gate_up / (gate_up_ms.mean() * 1e-3) / 1e9
        kname = ("small_m_kernel<gated> (weight-streaming gate/up + SiLU*mul)"
                 if weight_streaming(R, 1, per, False) else "grouped_gemm_bf16<gated> (gate/up GEMM + SiLU*mul)")
        roofline = {"kernel": kname, "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                    "avg_launch_ms": round(float(gate_up_ms.mean()), 4), "bytes_per_launch": bytes_gate_up}
    else:
        achieved = flops_gate_up / (gate_up_ms.mean() * 1e-3) / 1e12
        roofline = {"kernel": "grouped_gemm_bf16<gated> (gate/up GEMM + SiLU*mul)", "bound": "mfma",
                    "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "avg_launch_ms": round(float(gate_up_ms.mean()), 4), "flops_per_launch": flops_gate_up}
    shard_flops = cfg.expert_flops_per_pair() * R
    out = {
        "metric": "received rows/sec of one expert-parallel shard (moe_expert_shard_forward)",
        "value": round(R * K / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) random-init weights)",
        "config": {"workload": w.name, "layer": cfg.name, "n_shards": w.n_shards, "shard": w.shard,
                   "rows": R, "local_experts": per, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "parallelism": "one GPU's expert shard (the exchanges are not run)"},
        "roofline": roofline,
        "layer": {
            "step_ms_p50": round(float(np.percentile(step_ms, 50)), 4),
            "step_ms_p95": round(float(np.percentile(step_ms, 95)), 4),
            "step_ms_p99": round(float(np.percentile(step_ms, 99)), 4),
            "shard_tflops": round(shard_flops / (np.median(step_ms) * 1e-3) / 1e12, 2),
            "max_over_mean_load": round(float(loads.max() / max(loads.mean(), 1e-9)), 3),
            "experts_touched": int((loads > 0).sum()),
        },
    }
    print(json.dumps(out), flush=True)


def backward_bench(args, cfg):
    """Training step of one layer: moe_layer_forward then moe_layer_backward (which recomputes
    the routing and the gate/up products) for the seeded output gradient, inputs resident in
    HBM. value = tokens per second of the step; roofline = the longest backward GEMM launch."""
    import numpy as np
    import torch

    from sparse_mixture_experts_29_amd import binding
    from sparse_mixture_experts_29_amd.device import DeviceLayer, LayerGrads, host_to_device
    from sparse_mixture_experts_29_amd.inputs import make_inputs, output_grad

    binding.load_library()
    li = make_inputs(cfg)
    dev = DeviceLayer(li, device="cuda:0", threads=16)
    dy = host_to_device(output_grad(cfg), cfg, dev.device)
    grads = LayerGrads(dev)
    aux = args.aux_coef
    stream = torch.cuda.current_stream()
    b = dev.stage_buffers()
    dev.route(b, logits=False)
    dev.permute(b)
    torch.cuda.synchronize()
    n_kept = int(b["offsets"][-1].item())
    del b

    def step():
        dev.forward()
        dev.backward(dy, aux, grads)

    # per-kernel launch times (outside the timed steps): each backward GEMM in its own pass
    kernels = [("recompute x Wg | x Wu", binding.MOE_KERNEL_BWD_RECOMPUTE, 4),
               ("down dgrad u = dy Wd", binding.MOE_KERNEL_BWD_DOWN_DGRAD, 2),
               ("gate/up dgrad (da|db)(Wg|Wu)", binding.MOE_KERNEL_BWD_GATE_UP_DGRAD, 4),
               ("down wgrad", binding.MOE_KERNEL_BWD_DOWN_WGRAD, 2),
               ("gate wgrad", binding.MOE_KERNEL_BWD_GATE_WGRAD, 2),
               ("up wgrad", binding.MOE_KERNEL_BWD_UP_WGRAD, 2)]
    per = {}
    for name, kid, mult in kernels:
        _, _, ms = time_steps(step, 5, 1 if per else args.warmup, stream, kernel=kid)
        flops = mult * (cfg.d_model * cfg.d_ff * n_kept + cfg.d_model * cfg.d_ff_shared * cfg.T * cfg.n_shared)
        per[name] = dict(kernel_id=kid, avg_launch_ms=round(float(ms.mean()), 4), flops_per_launch=float(flops),
                         tflops=round(flops / (ms.mean() * 1e-3) / 1e12, 1))
    dom_name = max(per, key=lambda n: per[n]["avg_launch_ms"])
    dom = per[dom_name]
    elapsed, step_ms, dom_ms = time_steps(step, args.steps, 0, stream, kernel=dom["kernel_id"])
    K = args.steps
    achieved = dom["flops_per_launch"] / (dom_ms.mean() * 1e-3) / 1e12
    train_flops = 22.0 * cfg.d_model * cfg.d_ff * n_kept + 22.0 * cfg.d_model * cfg.d_ff_shared * cfg.T * cfg.n_shared
    out = {
        "metric": "training-step tokens/sec per MoE layer (forward + backward with recompute)",
        "value": round(cfg.T * K / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and output gradient, N(0,1/sqrt(fan_in)) random-init weights)",
        "config": {"workload": cfg.name + "_train", "T": cfg.T, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "gating": cfg.gating,
                   "capacity_factor": cfg.capacity_factor, "n_shared": cfg.n_shared,
                   "d_ff_shared": cfg.d_ff_shared, "aux_coef": aux, "parallelism": "single GPU"},
        "roofline": {"kernel": f"grouped_gemm_bf16 ({dom_name})", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(float(dom_ms.mean()), 4),
                     "flops_per_launch": dom["flops_per_launch"]},
        "layer": {
            "step_ms_p50": round(float(np.percentile(step_ms, 50)), 4),
            "step_ms_p95": round(float(np.percentile(step_ms, 95)), 4),
            "step_ms_p99": round(float(np.percentile(step_ms, 99)), 4),
            "train_step_tflops": round(train_flops / (np.median(step_ms) * 1e-3) / 1e12, 2),
            "n_kept": n_kept,
            "backward_gemms": per,
        },
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_backward(li, min(args.cpu_tokens, cfg.T), aux)
    print(json.dumps(out), flush=True)


def cpu_baseline_backward(li, n_tokens: int, aux: float):
    """The oracle's forward and backward (as they stand) on the first n_tokens of the workload."""
    import threadpoolctl

    import oracle
    from sparse_mixture_experts_29_amd.inputs import output_grad
    c = li.cfg
    x = li.values(li.x[:n_tokens])
    dy = li.values(output_grad(c)[:n_tokens])
    wr = li.values(li.w_router)
    experts = [li.expert_values(e) for e in range(c.n_experts)]  # input generation: untimed
    shared = [li.shared_values(s) for s in range(c.n_shared)]
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    oracle.forward(x, wr, li.router_bias, top_k=c.top_k, gating=c.gating, capacity_factor=c.capacity_factor,
                   experts=experts, shared=shared, n_shared=c.n_shared)
    oracle.backward(x, wr, li.router_bias, dy, top_k=c.top_k, gating=c.gating, capacity_factor=c.capacity_factor,
                    experts=experts, shared=shared, n_shared=c.n_shared, aux_coef=aux)
    dt = time.perf_counter() - t0
    return dict(value=n_tokens / dt, unit="tokens/s", cores=int(threads), kind="oracle", blas=blas_name(info),
                sample=f"forward + backward of the first {n_tokens} of {c.T} tokens of {c.name} "
                       f"(capacity and balancing loss over that sample); {dt:.1f} s", seconds=round(dt, 2))


def cpu_baseline(li, n_tokens: int):
    """The oracle (as it stands) on the first n_tokens of the workload, on host cores.
    Returns the record and the oracle's result on those tokens (its routing and y)."""
    import numpy as np
    import threadpoolctl

    import oracle
    c = li.cfg
    x = li.values(li.x[:n_tokens])
    wr = li.values(li.w_router)
    if c.fp8:
        # codes and scales drawn untimed; the oracle decodes them inside the timed region
        codes = [li.expert_fp8(e) for e in range(c.n_experts)]
        scodes = [li.shared_fp8(s) for s in range(c.n_shared)]
        experts = lambda e: oracle.fp8_expert(*codes[e])  # noqa: E731
        shared = lambda s: oracle.fp8_expert(*scodes[s])  # noqa: E731
    else:
        # stored weights (bf16 bit patterns, 2 bytes each) drawn untimed; the chosen experts'
        # values are widened inside the timed region
        store = [None] * c.n_experts

        def put(e, w):
            store[e] = w

        li.for_each_expert(put, 16)
        sstore = [li.shared(s) for s in range(c.n_shared)]
        experts = lambda e: tuple(li.values(w) for w in store[e])  # noqa: E731
        shared = lambda s: tuple(li.values(w) for w in sstore[s])  # noqa: E731
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    # the median of 3 runs when one run is short (the small and decode batches), else one run
    times = []
    res = None
    while len(times) < (3 if not times or times[0] < CPU_REPEAT_BELOW_S else 1):
        t0 = time.perf_counter()
        res = oracle.forward(x, wr, li.router_bias, top_k=c.top_k, gating=c.gating,
                             capacity_factor=c.capacity_factor, experts=experts, shared=shared,
                             n_shared=c.n_shared)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    rec = dict(value=n_tokens / dt, unit="tokens/s", cores=int(threads), kind="oracle", blas=blas_name(info),
               sample=f"first {n_tokens} of {c.T} tokens of {c.name}, the chosen experts' "
                      f"weights {'decoded from FP8' if c.fp8 else 'widened'} to float64 inside the timed "
                      f"region; median of {len(times)} run(s), {dt:.3g} s each",
               runs=len(times), seconds=round(dt, 2))
    return rec, res, (experts, shared)


def routing_telemetry(li, counts, drop, idx_g, n_kept):
    """Expert loads and drops of the timed batch (the library's own counts), and its near-tie
    tokens: the oracle's float64 logits of every token, the k-th/(k+1)-th gap and adjacent
    chosen logits closer than 1e-4, and how many tokens the GPU routed to another expert set
    or in another order. Outside the timed steps."""
    import numpy as np

    import oracle
    c = li.cfg
    logits = oracle.router_logits(li.values(li.x), li.values(li.w_router), li.router_bias)
    idx_o = oracle.select_topk(logits, c.top_k)
    srt_o = -np.sort(-logits, axis=1)
    gap = srt_o[:, c.top_k - 1] - srt_o[:, c.top_k] if c.top_k < c.n_experts else np.full(c.T, np.inf)
    sel = np.take_along_axis(logits, idx_o, axis=1)
    adj = ((sel[:, :-1] - sel[:, 1:]) < 1e-4).any(axis=1) if c.top_k > 1 else np.zeros(c.T, bool)
    same_set = (np.sort(idx_g, axis=1) == np.sort(idx_o, axis=1)).all(axis=1)
    pairs = c.T * c.top_k
    cap = oracle.expert_capacity(c.capacity_factor, c.T, c.top_k, c.n_experts)
    kept = counts if cap is None else np.minimum(counts, cap)
    nz = counts[counts > 0]
    return {
        "pairs": pairs, "n_kept": n_kept, "capacity": cap,
        "dropped": int(drop.sum()), "drop_rate": round(float(drop.sum()) / pairs, 6),
        "experts_touched": int((counts > 0).sum()),
        "load": {"max": int(counts.max()), "min": int(counts.min()), "min_nonzero": int(nz.min()) if nz.size else 0,
                 "mean": round(float(counts.mean()), 2), "p50": float(np.percentile(counts, 50)),
                 "p99": float(np.percentile(counts, 99)), "max_over_mean": round(float(counts.max() / counts.mean()), 3),
                 "cv": round(float(counts.std() / counts.mean()), 4), "experts_over_capacity":
                 None if cap is None else int((counts > cap).sum()),
                 "kept_max_over_mean": round(float(kept.max() / max(kept.mean(), 1e-9)), 3)},
        "near_tie_tokens": int((gap < 1e-4).sum()),
        "adjacent_near_tie_tokens": int((adj & (gap >= 1e-4)).sum()),
        "tokens_routed_to_another_set": int((~same_set).sum()),
        "order_flips": int(((idx_g != idx_o).any(axis=1) & same_set).sum()),
        "near_tie_rule": "float64 oracle logits: k-th/(k+1)-th gap < 1e-4, or adjacent chosen logits < 1e-4 apart",
    }, (logits, idx_o)


def parity_against_oracle(li, y_dev, idx_g, drop_g, base_res, weights, oracle_routing):
    """The run's y on the CPU baseline's tokens against the oracle (its own routing). Tokens
    the GPU routed to another expert set, or whose kept experts differ, are near ties: counted
    and left out. Dropless layers reuse the baseline's y; with a capacity the oracle's token
    outputs are recomputed with the drops of the whole batch."""
    import numpy as np

    import oracle
    c = li.cfg
    n = base_res["y"].shape[0]
    if c.dropless:
        idx_o, y_o = base_res["idx"], base_res["y"]
        keep_o = np.ones_like(idx_o, dtype=bool)
    else:
        logits, idx_all = oracle_routing
        gate_all = oracle.gate_values(logits, idx_all, c.gating)
        cap = oracle.expert_capacity(c.capacity_factor, c.T, c.top_k, c.n_experts)
        keep_all = oracle.permute(idx_all, c.n_experts, cap)["drop"].reshape(c.T, c.top_k) == 0
        idx_o, keep_o = idx_all[:n], keep_all[:n]
        y_o = oracle.token_outputs(li.values(li.x[:n]), idx_o, gate_all[:n], keep_o, weights[0], weights[1],
                                   c.n_shared)
    keep_g = drop_g.reshape(c.T, c.top_k)[:n] == 0
    ig = idx_g[:n]
    same = (np.sort(ig, axis=1) == np.sort(idx_o, axis=1)).all(axis=1)
    kept_same = np.array([sorted(ig[t][keep_g[t]]) == sorted(idx_o[t][keep_o[t]]) for t in range(n)])
    ok = same & kept_same
    got = y_dev[:n].float().cpu().numpy().astype(np.float64)[ok]
    want = np.asarray(y_o, np.float64)[ok]
    diff = got - want
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30))
    mx = float(np.abs(diff).max(initial=0))
    bf16 = c.dtype == "bf16"
    tol = {"rel_l2": 1e-2, "max_abs": 5e-2} if bf16 else {"max_abs": 1e-4}
    return {"tokens": int(n), "compared": int(ok.sum()), "near_tie_excluded": int((~ok).sum()),
            "y_max_abs": mx, "y_rel_l2": rel, "tolerance": tol,
            "within_tolerance": bool(mx <= tol["max_abs"] and (not bf16 or rel <= tol["rel_l2"]))}


def library_record():
    """Which libmoe.so this process loaded (path, size and hash of the file)."""
    import hashlib

    from sparse_mixture_experts_29_amd import binding
    path = os.path.realpath(binding.LIB_PATH)
    h = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    return {"path": os.path.relpath(path, ROOT) if path.startswith(ROOT) else path, "sha256_16": h,
            "bytes": os.path.getsize(path), "moe_lib_override": bool(os.environ.get("MOE_LIB"))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="name of a configs.ALL or configs.SHARDS entry")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--backward", action="store_true",
                    help="time the training step (forward + moe_layer_backward) of the workload")
    ap.add_argument("--aux-coef", type=float, default=0.01, help="balancing-loss coefficient (--backward)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="also time K cold steps, each after streaming this many MiB of scratch through "
                         "the caches (read, or written with --flush-mode write), so the MALL holds no "
                         "weights at the step's start; reported under 'cold', not in value")
    ap.add_argument("--flush-mode", choices=("read", "write"), default="read")
    ap.add_argument("--graph", action="store_true",
                    help="also time K replays of one layer step captured in a HIP graph (reported under "
                         "'graph', never in value)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the timed steps, copy a buffer of this many MiB once (a plain copy "
                         "kernel of known size, to scale the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(expert parallelism is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mixture_experts_29_amd import binding, configs
    from sparse_mixture_experts_29_amd.device import DeviceLayer
    from sparse_mixture_experts_29_amd.inputs import make_inputs

    if args.workload in configs.SHARDS:
        return shard_bench(args, configs.SHARDS[args.workload])
    cfg = configs.ALL[args.workload] if args.workload else configs.DEEPSEEK_V3
    if args.backward:
        if args.cpu_tokens == 4096:
            args.cpu_tokens = 512
        return backward_bench(args, cfg)
    binding.load_library()
    li = make_inputs(cfg)
    t_gen = time.perf_counter()
    dev = DeviceLayer(li, device="cuda:0", threads=16)
    print(f"# inputs resident in HBM ({cfg.total_weight_bytes() / 1e9:.2f} GB weights) "
          f"in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    # routing statistics of this batch (outside the timed region)
    b = dev.stage_buffers()
    dev.route(b, logits=False)
    dev.permute(b)
    torch.cuda.synchronize()
    counts = b["counts"].cpu().numpy()
    n_kept = int(b["offsets"][-1].item())
    touched = int((counts > 0).sum())
    idx_g = b["idx"].cpu().numpy().astype(np.int64)
    drop_g = b["drop"].cpu().numpy()
    del b

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    elapsed, step_ms, gate_up_ms = time_steps(dev.forward, args.steps, args.warmup, stream)
    K = args.steps
    value = cfg.T * K / elapsed
    # after the timed steps: the down launch in a pass of its own, then the clocks while the
    # layer runs
    _, _, down_ms = time_steps(dev.forward, K, 1, stream, kernel=binding.MOE_KERNEL_DOWN)
    # counter runs (--copy-mib) skip it: under a counter profiler every child process loads the
    # profiler, and the tool's own interpreter start (a script run through env) is then refused
    clocks = (sample_clocks(dev.forward) if not args.copy_mib else
              {"tool": "rocm-smi --showclocks --json", "samples": [], "error": "not sampled in counter runs (--copy-mib)"})
    flops_gate_up = 4.0 * cfg.d_model * cfg.d_ff * n_kept + 4.0 * cfg.d_model * cfg.d_ff_shared * cfg.T * cfg.n_shared
    flops_down = flops_gate_up / 2
    layer_flops = (cfg.expert_flops_per_pair() * n_kept + cfg.shared_flops() + cfg.router_flops())
    es = 2 if cfg.dtype == "bf16" else 4
    small_batch = cfg.dtype == "bf16" and cfg.T <= SMALL_BATCH_TOKENS
    if small_batch:
        # decode batch: HBM-bound on either path; algorithmic bytes of the gated launch = the
        # touched experts' gate and up weights as stored (+ shared; FP8: codes and row scales),
        # the token rows read, the h rows written
        bytes_gate_up = (float(touched * cfg.gate_up_bytes(cfg.d_ff))
                         + cfg.n_shared * cfg.gate_up_bytes(cfg.d_ff_shared)
                         + cfg.T * cfg.d_model * es + n_kept * cfg.d_ff * es
                         + cfg.n_shared * cfg.T * cfg.d_ff_shared * es)
        achieved = bytes_gate_up / (gate_up_ms.mean() * 1e-3) / 1e9
        roofline = {
            "kernel": (("small_m_kernel<gated, fp8>" if cfg.fp8 else "small_m_kernel<gated>")
                       + " (weight-streaming gate/up + SiLU*mul)")
            if weight_streaming(cfg.T, cfg.top_k, cfg.n_experts, cfg.fp8)
            else "grouped_gemm_bf16<gated> (tiled gate/up GEMM + SiLU*mul, weight-bound at this batch)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profile("grouped_mlp_small.hip" if weight_streaming(
                cfg.T, cfg.top_k, cfg.n_experts, cfg.fp8) else "grouped_mlp.hip", cfg.name),
            "avg_launch_ms": round(float(gate_up_ms.mean()), 4),
            "bytes_per_launch": bytes_gate_up,
        }
    else:
        achieved = flops_gate_up / (gate_up_ms.mean() * 1e-3) / 1e12
        roofline = {
            "kernel": "grouped_gemm_bf16<gated> (gate/up GEMM + SiLU*mul)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_from_profile("grouped_mlp.hip", cfg.name),
            "avg_launch_ms": round(float(gate_up_ms.mean()), 4),
            "flops_per_launch": flops_gate_up,
        }
    # whole-layer algorithmic bytes (weights of touched experts, router, x in and y out)
    layer_bytes = (float(touched * cfg.expert_weight_bytes())
                   + cfg.n_shared * (cfg.gate_up_bytes(cfg.d_ff_shared) + cfg.down_bytes(cfg.d_ff_shared))
                   + cfg.d_model * cfg.n_experts * es + 2.0 * cfg.T * cfg.d_model * es)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "gating": cfg.gating,
                   "capacity_factor": cfg.capacity_factor, "n_shared": cfg.n_shared,
                   "d_ff_shared": cfg.d_ff_shared, "expert_weights": "fp8_e4m3" if cfg.fp8 else cfg.dtype,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "layer": {
            "step_ms_p50": round(float(np.percentile(step_ms, 50)), 4),
            "step_ms_p95": round(float(np.percentile(step_ms, 95)), 4),
            "step_ms_p99": round(float(np.percentile(step_ms, 99)), 4),
            "layer_tflops": round(layer_flops / (np.median(step_ms) * 1e-3) / 1e12, 2),
            "layer_mfma_frac": round(layer_flops / (np.median(step_ms) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "layer_hbm_frac": round(layer_bytes / (np.median(step_ms) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "pairs_per_s": round(n_kept / (np.median(step_ms) * 1e-3), 1),
            "gate_up_avg_ms": round(float(gate_up_ms.mean()), 4),
            "down_avg_ms": round(float(down_ms.mean()), 4),
            "n_kept": n_kept,
            "experts_touched": touched,
            "max_over_mean_load": round(float(counts.max() / max(counts.mean(), 1e-9)), 3),
        },
        "clocks": clocks,
        "library": library_record(),
    }
    if cfg.dtype == "bf16" and not small_batch:
        # both grouped launches (gate/up, down; shared experts ride in them as extra groups)
        gemm_tflops = (flops_gate_up + flops_down) / ((gate_up_ms.mean() + down_ms.mean()) * 1e-3) / 1e12
        out["layer"]["grouped_gemm_tflops"] = round(gemm_tflops, 2)
        out["layer"]["grouped_gemm_mfma_frac"] = round(gemm_tflops / BF16_PEAK_TFLOPS, 4)
    if args.flush_mib:
        cold_ms, cold_gate = cold_steps(dev.forward, K, stream, args.flush_mib, args.flush_mode)
        cold = {"flush_mib": args.flush_mib, "flush_mode": args.flush_mode,
                "ms_per_step": round(float(cold_ms.mean()), 4),
                "value": round(cfg.T / (cold_ms.mean() * 1e-3), 1),
                "step_ms_p50": round(float(np.percentile(cold_ms, 50)), 4),
                "gate_up_avg_ms": round(float(cold_gate.mean()), 4)}
        if small_batch:
            cold["gate_up_gbps"] = round(roofline["bytes_per_launch"] / (cold_gate.mean() * 1e-3) / 1e9, 1)
            cold["layer_hbm_frac"] = round(layer_bytes / (cold_ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        out["cold"] = cold
    if args.graph:
        g_ms = graph_steps(dev.forward, K, args.warmup, torch)
        out["graph"] = {"ms_per_step": round(float(g_ms.mean()), 4),
                        "value": round(cfg.T / (g_ms.mean() * 1e-3), 1),
                        "step_ms_p50": round(float(np.percentile(g_ms, 50)), 4)}
    y_dev = dev.forward()
    torch.cuda.synchronize()
    out["routing"], oracle_routing = routing_telemetry(li, counts, drop_g, idx_g, n_kept)
    if not args.no_cpu:
        out["cpu_baseline"], base_res, weights = cpu_baseline(li, min(args.cpu_tokens, cfg.T))
        out["parity"] = parity_against_oracle(li, y_dev, idx_g, drop_g, base_res, weights, oracle_routing)
        del base_res, weights
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
