"""Benchmark: decode layer-steps/s of one tensor-parallel shard on one MI355X.

A step is one pass of the whole shard step for rank 0 of the workload:
attention stage (RMSNorm, QKV, RoPE + KV append, GQA attention, W_O, int8
wire when configured) -> merge of the T shard partials (rank 0's own plus
the T-1 wires the other ranks produced, standing in for what would arrive
over xGMI) -> FFN stage (RMSNorm, W1/W3 + SwiGLU, W2) -> merge. By default
each merge is done by the kernel that produces rank 0's own partial
(decode_merge_step); --merge separate runs it as a kernel of its own
(merge_partials). The output of a step is the next step's input. R layer
copies (distinct weights, caches and workspaces in HBM, R x step bytes > 3 x
the 256 MB Infinity Cache) are used in rotation, step i on copy i mod R, so
no step reads what the previous one left in the cache.

Timing: one pass over the R copies is captured as a HIP graph (and the first
k mod R steps as another), so exactly --steps steps run per timed repeat,
after exactly --warmup untimed steps; each repeat is bracketed by a device
synchronisation and HIP events on the launch stream, and `value` is the
median of --repeats repeats (min and median both reported). Per-kernel
durations come from the library's HIP event pairs around each launch in an
eager pass that starts behind a device-side sleep, so the host's launch
calls never leave the GPU idle inside a pair.

Prints ONE JSON line: the primary workload (the 7B shard by default) with
the other configurations of the same metric as sub-results under "configs".
Inputs are seeded synthetic tensors of the workloads' shapes (no trained
weights exist here), resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time
from typing import Callable, Dict, List, Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode layer-steps/s per TP shard + achieved HBM GB/s (% peak), 7B/70B shapes"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# the other configurations of the metric, reported next to the primary one
SUB_CONFIGS = ("tiny_llama_tp2_b1", "llama2_7b_tp4_b1_q8", "llama2_70b_tp8_b16",
               "palm540b_ffn2d_b512", "palm540b_ffn2d_prefill8192")

PROFILES = os.path.join(ROOT, "profiles")


def measured_traffic(profile: str, sources) -> Optional[int]:
    """HBM bytes per launch of a kernel from its committed counter summary
    (profiles/<profile>: FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a
    copy of known size), or None when the summary is missing or the kernel's
    sources changed since the counters were taken."""
    path = os.path.join(PROFILES, profile)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch",
                                                                  "source_sha256"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if "traffic_bytes_per_launch" not in fields or "source_sha256" not in fields:
        return None
    if fields["source_sha256"] != sources_sha256(sources):
        return None
    return int(fields["traffic_bytes_per_launch"])


def sources_sha256(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


GEMV_SOURCES = ("tensor_tp_shard_amd/csrc/k_gemv.hip", "tensor_tp_shard_amd/csrc/gemv_lds.h",
                "tensor_tp_shard_amd/csrc/common.h")
# batch 5..16 with bf16 weights: the MFMA projections
GEMV_MFMA_SOURCES = ("tensor_tp_shard_amd/csrc/k_gemv_mfma.hip", "tensor_tp_shard_amd/csrc/common.h")
FFN2D_SOURCES = ("tensor_tp_shard_amd/csrc/k_ffn2d.hip", "tensor_tp_shard_amd/csrc/common.h")


def calib_copy(mib: int):
    """A plain device-to-device copy of `mib` MiB (fp32, torch's copy kernel),
    three times: the reference for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n * 4, "copies": 3}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


# ---------------------------------------------------------------- timing

class Stepper:
    """Runs k steps of a workload whose step i uses copy i mod R: each full
    pass over the R copies replays one captured graph, the k mod R steps
    left replay a graph of the first k mod R steps (eager mode: plain
    calls). Graphs are captured on first use, outside any timed region."""

    def __init__(self, step: Callable[[int], None], R: int, mode: str, stream):
        self.step, self.R, self.mode, self.stream = step, R, mode, stream
        self.graphs = {}

    def prepare(self, *counts):
        import torch
        with torch.cuda.stream(self.stream):
            for i in range(self.R):  # one eager pass before any capture
                self.step(i)
        torch.cuda.synchronize()
        if self.mode == "graph":
            for k in counts:
                for n in {self.R if k >= self.R else 0, k % self.R} - {0}:
                    self._graph(n)

    def _graph(self, n: int):
        import torch
        if n not in self.graphs:
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    self.step(i)
            torch.cuda.synchronize()
            self.graphs[n] = g
        return self.graphs[n]

    def run(self, k: int):
        import torch
        with torch.cuda.stream(self.stream):
            if self.mode == "eager":
                for i in range(k):
                    self.step(i % self.R)
                return
            full, rem = divmod(k, self.R)
            if full:
                g = self._graph(self.R)
                for _ in range(full):
                    g.replay()
            if rem:
                self._graph(rem).replay()


def time_steps(st: Stepper, steps: int, warmup: int, repeats: int) -> List[float]:
    """Milliseconds of `steps` steps, `repeats` times, after `warmup` steps."""
    import torch
    st.prepare(steps, warmup)
    st.run(warmup)
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st.stream)
        st.run(steps)
        e1.record(st.stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


_SLEEP_CYCLES_PER_MS = None


def _sleep_cycles_per_ms() -> float:
    """Calibrates torch.cuda._sleep (a device-side spin) in cycles per ms."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        import torch
        n = 2_000_000
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(n)  # first call loads the kernel
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = n / max(e0.elapsed_time(e1), 1e-3)
    return _SLEEP_CYCLES_PER_MS


def kernel_times(handles, st: Stepper, steps: int, names) -> Dict[str, float]:
    """Average duration (us) of each named kernel over an eager pass of
    `steps` steps, from the library's event pairs on the launch stream. The
    pass is enqueued behind a device-side sleep longer than the host needs to
    enqueue it, so the kernels run back to back as in the graph."""
    import torch
    import tensor_tp_shard_amd as tp
    ids = tp.kernel_names()
    t0 = time.perf_counter()
    with torch.cuda.stream(st.stream):
        for i in range(steps):
            st.step(i % st.R)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3
    out = {}
    for name in names:
        kid = ids.index(name)
        for h in handles:
            tp.kernel_timing_arm(h, kid)
        with torch.cuda.stream(st.stream):
            torch.cuda._sleep(int(_sleep_cycles_per_ms() * min(3 * host_ms + 2, 250)))
            for i in range(steps):
                st.step(i % st.R)
        torch.cuda.synchronize()
        tot, n = 0.0, 0
        for h in handles:
            t_, n_ = tp.kernel_timing_read(h)
            tot += t_
            n += n_
            tp.kernel_timing_arm(h, -1)
        if n:
            out[name] = round(tot / n * 1e3, 3)
    return out


def measured_peaks() -> Dict[str, float]:
    """The denominators measured on this GPU by the library's probes: a read
    stream over 2 GiB (16-byte nontemporal loads, the best of three grid
    sizes) and a bf16 MFMA loop with no memory traffic (the best of two
    occupancies), each the best of 5 timed launches after a warm-up."""
    import torch
    import tensor_tp_shard_amd as tp

    def best_ms(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    nbytes = 1 << 31
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    gbps = max(nbytes / (best_ms(lambda: tp.probe_read(buf, nbytes, sink, blocks)) * 1e-3) / 1e9
               for blocks in (1024, 2048, 4096))
    del buf
    iters = 2000
    fout = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    tflops = max(blocks * 4 * iters * 4 * 32768 /
                 (best_ms(lambda: tp.probe_mfma(blocks, iters, fout)) * 1e-3) / 1e12
                 for blocks in (512, 1024))
    del fout, sink
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(gbps, 1), "bf16_mfma_TFLOPs": round(tflops, 1),
            "how": "library probes: 2 GiB read with 16-byte nontemporal loads (best of 1024/2048/4096 "
                   "workgroups); bf16 32x32x16 MFMA loop from registers (best of 2 and 4 waves a SIMD)"}


def summarize(ms: List[float], steps: int, unit_per_step: float = 1.0) -> dict:
    med, mn = statistics.median(ms), min(ms)
    return {"value": round(unit_per_step * steps / (med * 1e-3), 2),
            "ms_per_step": round(med / steps, 6), "ms_per_step_min": round(mn / steps, 6),
            "ms_per_step_median": round(med / steps, 6), "repeats": len(ms)}


# ---------------------------------------------------------------- oracle baseline

def cpu_info() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(one_step: Callable[[], None], seconds: float, unit: str, per_step: float,
                 what: str) -> dict:
    """The oracle as it stands, timed on this host: the OpenMP build (the
    same source, independent rows on every thread; `value`) and the plain
    single-threaded build, each repeating one step of `what` for about
    `seconds` (at least once). per_step scales steps to the unit."""
    import oracle

    def run(omp: bool):
        threads = oracle.use_threads(omp)
        n, t0 = 0, time.perf_counter()
        while True:
            one_step()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return n, el, threads

    n1, el1, _ = run(False)
    nm, elm, threads = run(True)
    oracle.use_threads(False)
    return {"value": round(per_step * nm / elm, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{nm} {what} by the fp64 C oracle built with OpenMP ({threads} threads) "
                      f"in {elm:.1f} s",
            "single_thread": {"value": round(per_step * n1 / el1, 6), "cores": 1,
                              "sample": f"{n1} {what} by the plain single-threaded build in "
                                        f"{el1:.1f} s"},
            **cpu_info()}


# ---------------------------------------------------------------- Llama shard layer step

def llama_config(tp, w, rank):
    dt = {synth.F32: tp.TP_F32, synth.BF16: tp.TP_BF16}
    return tp.make_config(kind=tp.TP_LLAMA_BLOCK, dim=w.dim, n_heads=w.n_heads,
                          n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn_hidden=w.ffn_hidden,
                          tp_size=w.tp, tp_rank=rank, max_batch=w.batch, max_ctx=w.max_ctx,
                          w_dtype=dt[w.w_dtype], kv_dtype=dt[w.kv_dtype], quant=w.quant,
                          quant_block=32, rope_theta=w.rope_theta, norm_eps=w.norm_eps)


def llama_bytes(w, lens):
    """Algorithmic HBM bytes of rank 0's layer step: every packed weight of the
    shard once, plus the cached K and V of the past positions of the shard's
    kv heads (each kv head once, however many q heads share it)."""
    # int8 weights: one byte per weight plus a 4-byte scale per 32
    e = 1.125 if w.quant & synth.Q_WEIGHTS else 2 if w.w_dtype == synth.BF16 else 4
    kve = 2 if w.kv_dtype == synth.BF16 else 4
    T, D, hd = w.tp, w.dim, w.head_dim
    Hq_s, Hkv_s, Fs = w.n_heads // T, w.n_kv_heads // T, w.ffn_hidden // T
    weights = int(((Hq_s + 2 * Hkv_s) * hd * D + D * Hq_s * hd + 2 * Fs * D + D * Fs) * e)
    kv = int(np.sum(lens)) * Hkv_s * hd * 2 * kve
    w13 = int(2 * Fs * D * e)
    return weights, kv, w13


def llama_rank0(w):
    """Rank 0's layer of workload w and the other ranks' partials for its
    input (what rank 0 would receive): -> (inputs, shard builder, x, lens,
    attention wires, FFN wires of ranks 1..T-1)."""
    import torch
    import tensor_tp_shard_amd as tp
    T, B = w.tp, w.batch
    t_gen = time.time()
    d = synth.llama_inputs(w)
    log(f"generated inputs of {w.name} in {time.time() - t_gen:.1f}s")
    W = {k: dev(d[k]) for k in ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_att", "g_ffn")}
    hs = w.n_kv_heads // T

    def shard(rank):
        sh = tp.Shard(llama_config(tp, w, rank), caches=False)
        sh.load(W, k_cache=dev(d["kcache"][:, rank * hs:(rank + 1) * hs]).reshape(-1),
                v_cache=dev(d["vcache"][:, rank * hs:(rank + 1) * hs]).reshape(-1))
        return sh

    x0 = dev(d["x"])
    lens = dev(d["lens"])
    # the other ranks' partials for this input (what rank 0 would receive)
    others = [shard(r) for r in range(1, T)]
    s0 = shard(0)
    wa = [sh.new_wire() for sh in [s0] + others]
    for sh, wr in zip([s0] + others, wa):
        sh.step(tp.TP_STAGE_ATTN, x0, lens, B, wr)
    h0 = torch.empty_like(x0)
    s0.merge(tp.TP_STAGE_ATTN, wa, x0, h0, B)
    wf = [sh.new_wire() for sh in [s0] + others]
    for sh, wr in zip([s0] + others, wf):
        sh.step(tp.TP_STAGE_FFN, h0, None, B, wr)
    torch.cuda.synchronize()
    return d, shard, s0, x0, lens, wa[1:], wf[1:]


def wdtype(w):
    return "int8" if w.quant & synth.Q_WEIGHTS else "bf16" if w.w_dtype == synth.BF16 else "f32"


def run_llama(args, w, with_cpu=True):
    import torch
    import tensor_tp_shard_amd as tp
    T, B = w.tp, w.batch
    d, shard, s0, x0, lens, other_att, other_ffn = llama_rank0(w)
    wbytes, kvbytes, w13bytes = llama_bytes(w, d["lens"])
    step_bytes = wbytes + kvbytes
    # (at most 64: the 2 MB tiny block is latency-bound, its copies stay cached)
    R = args.copies or min(64, max(2, int(np.ceil(3 * 256e6 / step_bytes))))
    copies = [s0] + [shard(0) for _ in range(R - 1)]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    wires_a = [c.new_wire() for c in copies]
    wires_f = [c.new_wire() for c in copies]
    xs = [torch.empty_like(x0) for _ in range(R)]
    hs_ = [torch.empty_like(x0) for _ in range(R)]
    xs[0].copy_(x0)

    def step_fused(r):
        # layer copy r reads xs[r] and writes xs[r+1]; each merge is done by
        # the kernel that produces rank 0's own partial of that stage
        c, xin, xout = copies[r], xs[r], xs[(r + 1) % R]
        c.step_merge(tp.TP_STAGE_ATTN, xin, lens, B, wires_a[r], [wires_a[r]] + other_att, hs_[r])
        c.step_merge(tp.TP_STAGE_FFN, hs_[r], None, B, wires_f[r], [wires_f[r]] + other_ffn, xout)

    def step_separate(r):
        c, xin, xout = copies[r], xs[r], xs[(r + 1) % R]
        c.step(tp.TP_STAGE_ATTN, xin, lens, B, wires_a[r])
        c.merge(tp.TP_STAGE_ATTN, [wires_a[r]] + other_att, xin, hs_[r], B)
        c.step(tp.TP_STAGE_FFN, hs_[r], None, B, wires_f[r])
        c.merge(tp.TP_STAGE_FFN, [wires_f[r]] + other_ffn, hs_[r], xout, B)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    st = Stepper(step_fused if args.merge == "fused" else step_separate, R, args.mode, stream)
    ms = time_steps(st, args.steps, args.warmup, args.repeats)
    assert torch.isfinite(xs[0]).all().item(), "non-finite layer output"
    names = ["rmsnorm", "gemv_qkv", "qkv_attention", "attention", "gemv_wo", "q8_wire", "gemv_w13_swiglu", "gemv_w2",
             "merge"]
    kt = kernel_times([c.handle for c in copies], st, max(args.steps, R), names)
    s = summarize(ms, args.steps)
    ms_step = s["ms_per_step"]
    k_us = kt["gemv_w13_swiglu"]
    achieved = w13bytes / (k_us * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": s["value"], "unit": "layer-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wdtype(w),
        "data": "synthetic",
        "config": {"workload": w.name, "shard": f"rank 0 of TP={T}", "batch": B,
                   "kv_positions": [int(d["lens"].min()), int(d["lens"].max())],
                   "quant": w.quant, "layer_copies": R, "launch": args.mode,
                   "merge": ("fused into the producer of rank 0's partial" if args.merge == "fused"
                             else "kernel of its own"),
                   "step_bytes": int(step_bytes)},
        "ms_per_step_min": s["ms_per_step_min"], "ms_per_step_median": s["ms_per_step_median"],
        "repeats": s["repeats"],
        "achieved_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels_us": kt,
        "roofline": {"kernel": "gemv_w13_swiglu", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(
                         f"traffic_gemv_w13_swiglu_{w.name}.md",
                         GEMV_MFMA_SOURCES if w.w_dtype == synth.BF16 and B > 4 else GEMV_SOURCES),
                     "bytes_per_launch": int(w13bytes), "avg_launch_us": k_us},
    }
    if with_cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_llama(w, d, args.cpu_seconds)
    return res


def llama_oracle_step(w, d):
    """One rank-0 layer step of the oracle (attention stage, wire, merge, FFN
    stage, wire, merge; the other ranks' partials taken as zeros)."""
    import dataclasses
    import oracle
    x = d["x"].astype(np.float64)
    kc, vc = d["kcache"].copy(), d["vcache"].copy()
    if w.quant & synth.Q_WEIGHTS:
        # the weights' int8 round trip is a load-time step (as in load_weights):
        # done once, the timed steps then run on the dequantised weights
        d = dict(d)
        for k in ("wq", "wk", "wv", "wo", "w1", "w3", "w2"):
            d[k] = oracle.q8_weights(d[k], w.w_dtype)[2]
        w = dataclasses.replace(w, w_dtype=synth.F32, quant=w.quant & ~synth.Q_WEIGHTS)
    zeros = np.zeros((w.tp - 1, w.batch, w.dim))

    def one():
        a = oracle.attn_shard(w, d, 0, x, d["lens"], kc, vc)
        da, _, _ = oracle.wire(a["p"], w.quant)
        h = oracle.merge(x, np.concatenate([da[None], zeros]))
        f = oracle.ffn_shard(w, d, 0, h)
        df, _, _ = oracle.wire(f["p"], w.quant)
        oracle.merge(h, np.concatenate([df[None], zeros]))
    return one


def cpu_baseline_llama(w, d, seconds):
    return cpu_baseline(llama_oracle_step(w, d), seconds, "layer-steps/s", 1.0,
                        f"rank-0 shard layer steps of {w.name} (attention stage, wire, merge, "
                        f"FFN stage, wire, merge)")


# ---------------------------------------------------------------- PaLM 2D FFN block

def run_ffn2d(args, w, with_cpu=True):
    """One step = the block's up-projection + SwiGLU and down-projection for
    the workload's token count, over R rotating weight copies."""
    import torch
    import tensor_tp_shard_amd as tp
    B, E, F = w.batch, w.e_blk, w.f_blk
    d = synth.ffn2d_inputs(w)
    W = {"w1": dev(d["w_gate"]), "w3": dev(d["w_in"]), "w2": dev(d["w_out"])}
    cfg = tp.make_config(kind=tp.TP_FFN_2D, dim=E, ffn_hidden=F, tp_size=1, tp_rank=0,
                         max_batch=B, w_dtype=tp.TP_BF16)
    wbytes = 3 * E * F * 2
    R = args.copies or max(2, int(np.ceil(3 * 256e6 / wbytes)))
    copies = []
    for _ in range(R):
        sh = tp.Shard(cfg, caches=False)
        sh.load(W)
        copies.append(sh)
    del W
    x = dev(d["x"])
    ys = [torch.empty((B, E), dtype=torch.float32, device="cuda") for _ in range(R)]
    flops = 2.0 * B * E * F * 3
    up_flops = 2.0 * B * E * 2 * F

    def step(r):
        copies[r].step(tp.TP_STAGE_FFN, x, None, B, ys[r])

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    st = Stepper(step, R, args.mode, stream)
    ms = time_steps(st, args.steps, args.warmup, args.repeats)
    kt = kernel_times([c.handle for c in copies], st, max(args.steps, R), ["ffn2d_up", "ffn2d_down"])
    s = summarize(ms, args.steps)
    ms_step = s["ms_per_step"]
    ach = up_flops / (kt["ffn2d_up"] * 1e-6) / 1e12
    res = {
        "metric": METRIC, "value": s["value"], "unit": "ffn-block-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": B, "E_block": E, "F_block": F, "layer_copies": R,
                   "launch": args.mode},
        "ms_per_step_min": s["ms_per_step_min"], "ms_per_step_median": s["ms_per_step_median"],
        "repeats": s["repeats"],
        "achieved_TFLOPs": round(flops / (ms_step * 1e-3) / 1e12, 1),
        "mfma_frac": round(flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "kernels_us": kt,
        "roofline": {"kernel": "ffn2d_up", "bound": "mfma", "achieved": round(ach, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(f"traffic_ffn2d_up_{w.name}.md", FFN2D_SOURCES),
                     "flops_per_launch": up_flops, "avg_launch_us": kt["ffn2d_up"]},
    }
    if with_cpu and not args.no_cpu_baseline:
        import oracle
        rows = [0]
        nr = 16

        def one():  # a few token rows of the block (rows are independent)
            oracle.ffn2d(d["x"], d["w_gate"], d["w_in"], d["w_out"], row0=rows[0] % B, nrows=nr)
            rows[0] += nr
        res["cpu_baseline"] = cpu_baseline(one, args.cpu_seconds, "ffn-block-steps/s", nr / B,
                                           f"groups of {nr} token rows of {w.name}, scaled to "
                                           f"{B} rows,")
    return res


# ---------------------------------------------------------------- final stage

def logits_config(tp, w, rank):
    dt = {synth.F32: tp.TP_F32, synth.BF16: tp.TP_BF16}
    return tp.make_config(kind=tp.TP_LOGITS, dim=w.dim, ffn_hidden=w.vocab, tp_size=w.tp,
                          tp_rank=rank, max_batch=w.batch, w_dtype=dt[w.w_dtype], quant=w.quant,
                          quant_block=32, norm_eps=w.norm_eps)


def run_logits(args, w, with_cpu=True):
    """The final stage of rank 0: final RMSNorm + its V/T logits (+ int8 wire),
    then the merge of all T slices into full rows (the other ranks' wires
    computed once beforehand, standing in for what would arrive). R copies of
    rank 0's classifier slice in rotation, as for the layer step."""
    import torch
    import tensor_tp_shard_amd as tp
    T, B, D, Vs = w.tp, w.batch, w.dim, w.vocab // w.tp
    t_gen = time.time()
    d = synth.logits_inputs(w)
    log(f"generated inputs of {w.name} in {time.time() - t_gen:.1f}s")
    W = {"w1": dev(d["w_cls"]), "g_att": dev(d["g_final"])}

    def shard(rank):
        sh = tp.Shard(logits_config(tp, w, rank), caches=False)
        sh.load(W)
        return sh

    x = dev(d["x"])
    others = [shard(r) for r in range(1, T)]
    other_w = [sh.new_wire() for sh in others]
    for sh, wr in zip(others, other_w):
        sh.step(tp.TP_STAGE_LOGITS, x, None, B, wr)
    torch.cuda.synchronize()
    del others
    e = 1.125 if w.quant & synth.Q_WEIGHTS else 2 if w.w_dtype == synth.BF16 else 4
    cls_bytes = int(Vs * D * e)
    R = args.copies or max(2, int(np.ceil(3 * 256e6 / cls_bytes)))
    copies = [shard(0) for _ in range(R)]
    del W
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    wires = [c.new_wire() for c in copies]
    outs = [torch.empty((B, w.vocab), dtype=torch.float32, device="cuda") for _ in range(R)]

    def step(r):
        copies[r].step(tp.TP_STAGE_LOGITS, x, None, B, wires[r])
        copies[r].merge_logits([wires[r]] + other_w, outs[r], B)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    st = Stepper(step, R, args.mode, stream)
    ms = time_steps(st, args.steps, args.warmup, args.repeats)
    assert torch.isfinite(outs[0]).all().item(), "non-finite logits"
    kt = kernel_times([c.handle for c in copies], st, max(args.steps, R),
                      ["rmsnorm", "gemv_logits", "q8_wire", "merge_logits"])
    s = summarize(ms, args.steps)
    ms_step = s["ms_per_step"]
    achieved = cls_bytes / (kt["gemv_logits"] * 1e-6) / 1e9
    res = {
        "metric": "final-stage steps/s of one TP shard (final RMSNorm, vocabulary-split logits, "
                  "wire, merge of all slices)",
        "value": s["value"], "unit": "logits-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wdtype(w), "data": "synthetic",
        "config": {"workload": w.name, "shard": f"rank 0 of TP={T}", "batch": B, "vocab": w.vocab,
                   "quant": w.quant, "copies": R, "launch": args.mode, "step_bytes": cls_bytes},
        "ms_per_step_min": s["ms_per_step_min"], "ms_per_step_median": s["ms_per_step_median"],
        "repeats": s["repeats"],
        "achieved_GBps": round(cls_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(cls_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels_us": kt,
        "roofline": {"kernel": "gemv_logits", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(
                         f"traffic_gemv_logits_{w.name}.md",
                         GEMV_MFMA_SOURCES if w.w_dtype == synth.BF16 and B > 4 else GEMV_SOURCES),
                     "bytes_per_launch": cls_bytes, "avg_launch_us": kt["gemv_logits"]},
    }
    if with_cpu and not args.no_cpu_baseline:
        import oracle

        def one():
            z = oracle.logits_shard(d["w_cls"], d["g_final"], d["x"], T, 0, w.norm_eps, w.w_dtype)["z"]
            dz, _, _ = oracle.wire(z, w.quant)
            oracle.merge_logits(np.concatenate([dz[None], np.zeros((T - 1, B, Vs))]))
        res["cpu_baseline"] = cpu_baseline(one, args.cpu_seconds, "logits-steps/s", 1.0,
                                           f"rank-0 final-stage steps of {w.name} (final norm, "
                                           f"logits slice, wire, merge)")
    return res


# ---------------------------------------------------------------- batch-sharded attention

def attn_batch_config(tp, w, rank):
    dt = {synth.F32: tp.TP_F32, synth.BF16: tp.TP_BF16}
    return tp.make_config(kind=tp.TP_ATTN_BATCH, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads,
                          head_dim=w.head_dim, tp_size=w.tp, tp_rank=rank, max_batch=w.batch,
                          max_ctx=w.max_ctx, kv_dtype=dt[w.kv_dtype], rope_theta=w.rope_theta)


def run_attn_batch(args, w, with_cpu=True):
    """Rank 0's batch-sharded attention step: the all-to-all of the queries
    from the T head shards into its attention input rows, attention of every
    head over its sequences' caches, and the all-to-all of the outputs back
    into head shard 0's rows (the other batch shards' outputs computed once).
    R copies of rank 0's caches in rotation."""
    import torch
    import tensor_tp_shard_amd as tp
    T, B, hd, Hq, Hkv = w.tp, w.batch, w.head_dim, w.n_heads, w.n_kv_heads
    nb, C = B // T, Hq // T * hd
    d = synth.attn_batch_inputs(w)
    kve = 2 if w.kv_dtype == synth.BF16 else 4

    def shard(rank):
        rows = slice(rank * nb, (rank + 1) * nb)
        sh = tp.Shard(attn_batch_config(tp, w, rank), caches=False)
        sh.load({}, k_cache=dev(np.ascontiguousarray(d["kcache"][rows])).reshape(-1),
                v_cache=dev(np.ascontiguousarray(d["vcache"][rows])).reshape(-1))
        return sh

    qh = [dev(np.ascontiguousarray(d["qkv"][:, i * C:(i + 1) * C])) for i in range(T)]
    ld_q = (Hq + 2 * Hkv) * hd
    outs = []
    for r in range(1, T):   # the other batch shards' outputs for head shard 0
        sh = shard(r)
        x = dev(np.ascontiguousarray(d["qkv"][r * nb:(r + 1) * nb]))
        att = torch.empty((nb, Hq * hd), device="cuda")
        sh.step(tp.TP_STAGE_ATTN, x, dev(d["lens"][r * nb:(r + 1) * nb]), nb, att)
        outs.append(att)
    torch.cuda.synchronize()
    kv_bytes = int(np.sum(d["lens"][:nb]) + nb) * Hkv * hd * 2 * kve
    R = args.copies or max(2, int(np.ceil(3 * 256e6 / max(kv_bytes, 1))))
    R = min(R, 64)
    copies = [shard(0) for _ in range(R)]
    lens0 = dev(d["lens"][:nb])
    xs = [dev(np.ascontiguousarray(d["qkv"][:nb])) for _ in range(R)]
    atts = [torch.empty((nb, Hq * hd), device="cuda") for _ in range(R)]
    backs = [torch.empty((B, C), device="cuda") for _ in range(R)]
    torch.cuda.synchronize()

    def step(r):
        c = copies[r]
        tp.all_to_all(c.handle, tp.TP_A2A_HEADS_TO_BATCH, qh, C, xs[r], ld_q)
        c.step(tp.TP_STAGE_ATTN, xs[r], lens0, nb, atts[r])
        tp.all_to_all(c.handle, tp.TP_A2A_BATCH_TO_HEADS, [atts[r]] + outs, Hq * hd, backs[r], C)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    st = Stepper(step, R, args.mode, stream)
    ms = time_steps(st, args.steps, args.warmup, args.repeats)
    assert torch.isfinite(backs[0]).all().item(), "non-finite attention output"
    kt = kernel_times([c.handle for c in copies], st, max(args.steps, R), ["attention", "all_to_all"])
    s = summarize(ms, args.steps)
    ms_step = s["ms_per_step"]
    achieved = kv_bytes / (kt["attention"] * 1e-6) / 1e9
    res = {
        "metric": "batch-sharded attention steps/s of one shard (all-to-all in, RoPE + KV append + "
                  "GQA attention over every head of its sequences, all-to-all out)",
        "value": s["value"], "unit": "attention-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if w.kv_dtype == synth.F32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "shard": f"rank 0 of TP={T}", "sequences": nb,
                   "heads": [Hq, Hkv], "kv_positions": [int(x) for x in d["lens"][:nb]],
                   "copies": R, "launch": args.mode, "step_bytes": kv_bytes},
        "ms_per_step_min": s["ms_per_step_min"], "ms_per_step_median": s["ms_per_step_median"],
        "repeats": s["repeats"], "kernels_us": kt,
        "roofline": {"kernel": "attention (+ combine)", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": kv_bytes, "avg_launch_us": kt["attention"]},
    }
    if with_cpu and not args.no_cpu_baseline:
        import oracle
        kc, vc = d["kcache"][:nb].copy(), d["vcache"][:nb].copy()
        heads = np.stack([d["qkv"][:, i * C:(i + 1) * C] for i in range(T)])

        def one():
            q = oracle.a2a_heads_to_batch(heads, 0)
            rows = d["qkv"][:nb].astype(np.float64)
            rows[:, :Hq * hd] = q
            att = oracle.attn_batch_shard(rows, d["lens"][:nb], kc, vc, Hq, Hkv, hd, w.kv_dtype)
            oracle.a2a_batch_to_heads(np.concatenate([att[None], np.zeros((T - 1, nb, Hq * hd))]), 0)
        res["cpu_baseline"] = cpu_baseline(one, args.cpu_seconds, "attention-steps/s", 1.0,
                                           f"rank-0 batch-sharded attention steps of {w.name} "
                                           f"(all-to-all, attention, all-to-all)")
    return res


# ---------------------------------------------------------------- whole decode step

def run_decode(args, wd, with_cpu=True):
    """One token through rank 0's shard of the whole model: n_layers layer
    steps (distinct packed weights and KV caches per layer, each merge done by
    the kernel producing rank 0's partial) feeding each other, then the final
    stage (final norm, logits slice, wire, merge of all T slices). The other
    ranks' partials are computed once for the first layer's input and stand
    in for what every layer would receive. A step is one token."""
    import torch
    import tensor_tp_shard_amd as tp
    w, wl, L = wd.block, wd.logits, wd.n_layers
    T, B = w.tp, w.batch
    d, shard, s0, x0, lens, other_att, other_ffn = llama_rank0(w)
    layers = [s0] + [shard(0) for _ in range(L - 1)]
    dl = synth.logits_inputs(wl)
    WL = {"w1": dev(dl["w_cls"]), "g_att": dev(dl["g_final"])}
    lsh = []
    for r in range(T):
        sh = tp.Shard(logits_config(tp, wl, r), caches=False)
        sh.load(WL)
        lsh.append(sh)
    xl = dev(dl["x"][:B])
    other_lw = [sh.new_wire() for sh in lsh[1:]]
    for sh, wr in zip(lsh[1:], other_lw):
        sh.step(tp.TP_STAGE_LOGITS, xl, None, B, wr)
    torch.cuda.synchronize()
    l0 = lsh[0]
    del lsh, WL
    torch.cuda.empty_cache()
    wires_a = [c.new_wire() for c in layers]
    wires_f = [c.new_wire() for c in layers]
    xs = [torch.empty_like(x0) for _ in range(L + 1)]
    hs_ = [torch.empty_like(x0) for _ in range(L)]
    xs[0].copy_(x0)
    lwire = l0.new_wire()
    logits = torch.empty((B, wl.vocab), dtype=torch.float32, device="cuda")

    def one_token(_r):
        for i, c in enumerate(layers):
            c.step_merge(tp.TP_STAGE_ATTN, xs[i], lens, B, wires_a[i], [wires_a[i]] + other_att, hs_[i])
            c.step_merge(tp.TP_STAGE_FFN, hs_[i], None, B, wires_f[i], [wires_f[i]] + other_ffn,
                         xs[i + 1])
        l0.step(tp.TP_STAGE_LOGITS, xs[L], None, B, lwire)
        l0.merge_logits([lwire] + other_lw, logits, B)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    st = Stepper(one_token, 1, args.mode, stream)
    ms = time_steps(st, args.steps, args.warmup, args.repeats)
    assert torch.isfinite(logits).all().item(), "non-finite logits"
    kt = kernel_times([c.handle for c in layers], st, 1, ["gemv_w13_swiglu"])
    s = summarize(ms, args.steps)
    ms_tok = s["ms_per_step"]
    wbytes, kvbytes, w13bytes = llama_bytes(w, d["lens"])
    ecls = 1.125 if wl.quant & synth.Q_WEIGHTS else 2 if wl.w_dtype == synth.BF16 else 4
    tok_bytes = L * (wbytes + kvbytes) + int(wl.vocab // T * wl.dim * ecls)
    achieved = w13bytes / (kt["gemv_w13_swiglu"] * 1e-6) / 1e9
    res = {
        "metric": "decode tokens/s of one TP shard through the whole model (all layers + final stage)",
        "value": round(1e3 / ms_tok * B, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_tok, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wdtype(w), "data": "synthetic",
        "config": {"workload": wd.name, "shard": f"rank 0 of TP={T}", "batch": B, "layers": L,
                   "vocab": wl.vocab, "kv_positions": [int(d["lens"].min()), int(d["lens"].max())],
                   "launch": args.mode, "token_bytes": int(tok_bytes)},
        "ms_per_step_min": s["ms_per_step_min"], "ms_per_step_median": s["ms_per_step_median"],
        "repeats": s["repeats"],
        "achieved_GBps": round(tok_bytes / (ms_tok * 1e-3) / 1e9, 1),
        "hbm_frac": round(tok_bytes / (ms_tok * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": "gemv_w13_swiglu", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(
                         f"traffic_gemv_w13_swiglu_{w.name}.md",
                         GEMV_MFMA_SOURCES if w.w_dtype == synth.BF16 and B > 4 else GEMV_SOURCES),
                     "bytes_per_launch": int(w13bytes), "avg_launch_us": kt["gemv_w13_swiglu"]},
    }
    if with_cpu and not args.no_cpu_baseline:
        import oracle
        layer = llama_oracle_step(w, d)
        Vs = wl.vocab // T

        def final():
            z = oracle.logits_shard(dl["w_cls"], dl["g_final"], dl["x"][:B], T, 0, wl.norm_eps,
                                    wl.w_dtype)["z"]
            dz, _, _ = oracle.wire(z, wl.quant)
            oracle.merge_logits(np.concatenate([dz[None], np.zeros((T - 1, B, Vs))]))
        tl = cpu_baseline(layer, args.cpu_seconds / 2, "layer-steps/s", 1.0, "layer steps")
        tf = cpu_baseline(final, args.cpu_seconds / 2, "final-steps/s", 1.0, "final stages")
        res["cpu_baseline"] = {
            "value": round(B / (L / tl["value"] + 1 / tf["value"]), 6), "unit": "tokens/s",
            "cores": tl["cores"], "kind": "oracle",
            "sample": f"{tl['sample']}; {tf['sample']}; tokens/s = B / ({L} x layer step + "
                      f"final stage)",
            "single_thread": {"value": round(B / (L / tl["single_thread"]["value"]
                                                  + 1 / tf["single_thread"]["value"]), 6),
                              "cores": 1},
            **cpu_info()}
    return res


RUNS = {"ffn2d": run_ffn2d, "logits": run_logits, "llama": run_llama, "decode": run_decode,
        "attn_batch": run_attn_batch}


def sub_result(res: dict, peaks: dict) -> dict:
    """The figures of one configuration kept under the primary line's "configs"."""
    keep = ("value", "unit", "ms_per_step", "ms_per_step_min", "ms_per_step_median", "repeats",
            "dtype", "achieved_GBps", "hbm_frac", "achieved_TFLOPs", "mfma_frac", "kernels_us",
            "roofline", "cpu_baseline")
    out = {k: res[k] for k in keep if k in res}
    out["config"] = res["config"]
    add_measured_fracs(out, peaks)
    return out


def add_measured_fracs(res: dict, peaks: dict):
    """Fractions of the measured peaks next to those of the spec peaks."""
    if not peaks:
        return
    if "achieved_GBps" in res:
        res["hbm_frac_of_measured"] = round(res["achieved_GBps"] / peaks["hbm_read_GBps"], 4)
    if "achieved_TFLOPs" in res:
        res["mfma_frac_of_measured"] = round(res["achieved_TFLOPs"] / peaks["bf16_mfma_TFLOPs"], 4)
    rf = res.get("roofline")
    if rf:
        den = peaks["hbm_read_GBps"] if rf["unit"] == "GB/s" else peaks["bf16_mfma_TFLOPs"]
        rf["frac_of_measured"] = round(rf["achieved"] / den, 4)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400, help="timed steps per repeat")
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps before the first repeat")
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats (value = median)")
    ap.add_argument("--workload", default="llama2_7b_tp4_b1", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--configs", default="auto",
                    help="sub-configurations to add under 'configs': 'all' (the other configurations "
                         "of the metric), 'none', or a comma list of workloads; 'auto' = all for the "
                         "default workload, none otherwise")
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"])
    ap.add_argument("--copies", type=int, default=0, help="layer copies in rotation (0 = auto)")
    ap.add_argument("--merge", default="fused", choices=["fused", "separate"],
                    help="merge of a stage's partials by the kernel that produces rank 0's own "
                         "partial (decode_merge_step) or as a kernel of its own (merge_partials)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the shard step runs every shard in turn on one device "
              "and uses no collectives; --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.repeats < 1:
        print("--steps and --repeats must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)
        return
    w = synth.get(args.workload)
    res = RUNS[w.kind](args, w)
    peaks = {} if args.no_peaks else measured_peaks()
    if peaks:
        res["measured_peaks"] = peaks
        add_measured_fracs(res, peaks)
    subs = args.configs
    if subs == "auto":
        subs = "all" if args.workload == "llama2_7b_tp4_b1" else "none"
    names = [] if subs == "none" else list(SUB_CONFIGS) if subs == "all" else subs.split(",")
    configs = {}
    for name in names:
        if name == args.workload:
            continue
        log(f"sub-configuration {name}")
        ws = synth.get(name)
        sargs = argparse.Namespace(**vars(args))
        sargs.cpu_seconds = min(args.cpu_seconds, 3.0)
        configs[name] = sub_result(RUNS[ws.kind](sargs, ws), peaks)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if configs:
        res["configs"] = configs
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
