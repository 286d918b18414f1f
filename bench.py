#!/usr/bin/env python3
"""Benchmark of the TwoTower block-diffusion hot path on one MI355X.

One step = one whole block of Algorithm 2 (Nemotron-TwoTower, arXiv 2606.26493,
section 2.2) over a batch: the block starts fully masked; each denoising step
r = 1..T runs the Eq. (1) block attention of all six attention layers (each
against its own layer-aligned context cache) and then one ConfidenceSample
(threshold gamma, steps left T-r+1); the loop stops once every position is
committed. Every call is launched from the host; --graph replays each step from a HIP graph
captured once per step instead (after checking that the graphs reproduce the host-launched
loop exactly). The denoiser layers between attention and the logits need trained
weights and are not part of this path: each step's logits are synthetic
(N(0,1) plus a spike of height 0.5*t at a fixed target), drawn in advance and
resident in HBM, as are the six caches.

Default workload ("loop"): batch 32, block S=16, T=16, prefix 8192 tokens,
32 query / 2 KV heads, head_dim 128, bf16, vocabulary 131072, gamma 0.8,
temperature 0.1. The JSON line reports noisy-block tokens per second per
attention layer (B*S*layers*steps / time), the attention call's roofline, and
the CPU oracle on a bounded sample as a baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload loop|tiny|single|ragged|long|...]
    python bench.py --copy-calibration   # a plain device copy of known size, for counter scaling

The default run (loop workload) also times the other four workloads and reports them in
"per_config", one entry per workload: the tiny fp32 call and its unmask step (us), the
single-layer call cold (a 512 MB buffer read before each call) and warm, the ragged
batch and its 64 x 16 x 131072 unmask step, and the long-prefix call against the bf16 MFMA
roof; every entry has the median, p10 and p90 of at least 20 calls timed one by one and the
oracle on a bounded sample at one thread and at every host thread. The loop itself also runs
at gamma 0.5 and 0.95 (blocks/s and steps per block).

roofline.traffic is the HBM traffic of one attention call measured with
rocprofv3 FETCH_SIZE / WRITE_SIZE counters, scaled by the ratio the same
counters give for the plain copy; it is read from profiles/attn_loop_hbm_traffic.txt
and reported only while the kernel source still hashes to the value recorded
there (otherwise null).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import shutil
import subprocess
import sys
import threading
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_eq_block_amd import api, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_loop_hbm_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "attention_eq_block_amd", "csrc", "attn_bf16.hip")
BUILD_SCRIPT = os.path.join(ROOT, "attention_eq_block_amd", "build.py")
COPY_BYTES = 1 << 30


def kernel_source_hash():
    """Hash of the attention kernel's source and of the build script (its compiler flags)."""
    h = hashlib.sha256()
    for path in (KERNEL_SOURCE, BUILD_SCRIPT):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention call from the committed counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None
METRIC = "noisy-block tokens/s per attn layer (S=16); achieved HBM TB/s vs peak"
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
SCRUB_BYTES = 512 << 20    # read between timed calls so that the next one reads HBM, not the 256 MB MALL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    """q-th percentile (0..100) of a list, linear interpolation."""
    ys = sorted(xs)
    if not ys:
        return float("nan")
    k = (len(ys) - 1) * q / 100.0
    lo, hi = int(math.floor(k)), int(math.ceil(k))
    return ys[lo] + (ys[hi] - ys[lo]) * (k - lo)


def spread_us(ms):
    """median, p10 and p90 of per-call times (ms) in microseconds."""
    return {"median": pct(ms, 50) * 1e3, "p10": pct(ms, 10) * 1e3, "p90": pct(ms, 90) * 1e3, "n": len(ms)}


class Scrub:
    """A 512 MB buffer read between timed calls (outside their events). Reading, not writing: a
    write would leave dirty lines in the caches whose write-back the next timed call would pay."""

    def __init__(self):
        self.buf = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros((), dtype=torch.float32, device="cuda")

    def __call__(self):
        torch.sum(self.buf, dim=0, out=self.sink)


def time_each(call, stream, reps, warmup, scrub=None):
    """Per-call times (ms): HIP events on the stream the kernels run on, around each call only."""
    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        if scrub is not None:
            scrub()
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


class Layer:
    """One attention layer's inputs on the GPU plus its prepared call."""

    def __init__(self, case, layer, workspace=None):
        inp = synth.make_attn_inputs(case, seed=0, layer=layer, device="cuda")
        self.inp = inp
        self.case = case
        self.p = api.attn_params(inp["Q"], inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp["Kd"],
                                 inp["Vd"], page_size=inp["page_size"], max_ctx_len=case.max_ctx_len,
                                 scale=inp["scale"])
        self.out, self.lse = self.p._keep
        nb = api.block_attn_workspace_bytes(self.p)
        self.ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                                      device="cuda")
        self.nb = nb

    def __call__(self, stream):
        rc = api.lib().tt_block_attn(self.p, self.ws.data_ptr(), self.nb, stream)
        if rc:
            raise RuntimeError(f"tt_block_attn failed: {api.status_string(rc)}")

    def cpu_sub(self, b0, b1):
        """The inputs of sequences b0..b1-1 on the CPU (their pages only)."""
        inp = self.inp
        pages = inp["page_table"][b0:b1].cpu()
        used = pages[pages >= 0]
        lo, hi = int(used.min()), int(used.max()) + 1
        return dict(Q=inp["Q"][b0:b1].cpu(), Kc=inp["Kc"][lo:hi].cpu(), Vc=inp["Vc"][lo:hi].cpu(),
                    page_table=torch.where(pages >= 0, pages - lo, pages).to(torch.int32),
                    ctx_len=inp["ctx_len"][b0:b1].cpu(),
                    Kd=None if inp["Kd"] is None else inp["Kd"][b0:b1].cpu(),
                    Vd=None if inp["Vd"] is None else inp["Vd"][b0:b1].cpu(), page_size=inp["page_size"],
                    scale=inp["scale"])


def oracle_attn_time(d, rows=None, threads=None):
    """Seconds the float64 oracle takes for Eq. (1) over the given inputs (all rows or a sample)."""
    import oracle
    if threads is not None:
        oracle.set_num_threads(threads)
    t0 = time.perf_counter()
    oracle.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Kd"], d["Vd"],
                      page_size=d["page_size"], scale=d["scale"], rows=rows)
    return time.perf_counter() - t0


def host_threads():
    """Threads for the oracle's all-threads figure: the process's CPU share (OMP_NUM_THREADS when
    the environment sets it, else the CPUs this process may run on)."""
    import oracle
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    oracle.set_num_threads(max(1, n))
    return oracle.num_threads()


def attn_roofline(case, call_ms, bound):
    """Roofline of one attention call: algorithmic bytes against HBM, or flops against bf16 MFMA."""
    if bound == "mfma":
        ach = case.flops() / (call_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / MFMA_PEAK_TFLOPS, "traffic": None, "flops": case.flops(),
                "hbm_frac": case.algorithmic_bytes() / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    ach = case.algorithmic_bytes() / (call_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
            "traffic": None, "algorithmic_bytes": case.algorithmic_bytes()}


def unmask_timing(ucase, stream, args, scrub, logits=None):
    """One ConfidenceSample step over all-masked rows (mask_out separate, so every call sees the same
    state), timed per call; bytes are the masked logit rows read once."""
    B, S = ucase.B, ucase.S
    x = logits if logits is not None else synth.make_logits(ucase, seed=0, device="cuda")
    mask = torch.ones(B, S, dtype=torch.uint8, device="cuda")
    mask_out = torch.empty_like(mask)
    tokens = torch.full((B, S), synth.MASK_TOKEN_ID, dtype=torch.int32, device="cuda")
    p = api.unmask_params(x, mask, tokens, gamma=ucase.gamma, temperature=ucase.temperature, steps_left=16,
                          mask_out=mask_out)
    ws = torch.empty(max(16, api.conf_unmask_workspace_bytes(p)), dtype=torch.uint8, device="cuda")
    lib = api.lib()
    sh = stream.cuda_stream

    def call():
        rc = lib.tt_conf_unmask(p, ws.data_ptr(), ws.numel(), sh)
        if rc:
            raise RuntimeError(f"tt_conf_unmask failed: {api.status_string(rc)}")

    ms = time_each(call, stream, max(20, args.reps), 5, scrub)
    med = pct(ms, 50)
    algo = ucase.algorithmic_bytes(B * S)
    ach = algo / (med * 1e-3) / 1e9
    return x, {"rows": B * S, "V": ucase.V, "call_us": spread_us(ms), "masked_rows_per_s": B * S / (med * 1e-3),
               "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": ach / HBM_PEAK_GBS, "algorithmic_bytes": algo}}


def oracle_unmask_time(x, ucase, threads=None):
    import oracle
    if threads is not None:
        oracle.set_num_threads(threads)
    tok, mk = synth.make_mask_state(x.shape[0], x.shape[1])
    t0 = time.perf_counter()
    oracle.conf_unmask(x, mk, tok, gamma=oracle.f32(ucase.gamma), temperature=oracle.f32(ucase.temperature),
                       steps_left=16)
    return time.perf_counter() - t0


# --------------------------------------------------------------------------- single-call workloads

CONFIG_OF = {"tiny": "C1", "single": "C2", "ragged": "C3", "long": "C4", "loop": "C5"}


def run_single(args, name, stream):
    """One attention layer of a workload, timed call by call (median, p10, p90). 'single' is also
    timed warm (no scrub: its 4.5 MB stay in the MALL); 'ragged' and 'tiny' add their unmask step;
    'long' is reported against the bf16 MFMA roof, the others against HBM."""
    case = synth.attn_case(name)
    L = Layer(case, 0)
    scrub = Scrub()
    sh = stream.cuda_stream
    reps = max(20, args.reps)
    ms = time_each(lambda: L(sh), stream, reps, 5, None if name == "tiny" else scrub)
    med = pct(ms, 50)
    bound = "mfma" if name == "long" else "hbm"
    res = {"config": CONFIG_OF[name], "metric": METRIC, "value": case.B * case.S / (med * 1e-3),
           "unit": "tokens/s", "dtype": "f32" if case.dtype == torch.float32 else "bf16",
           "workload": f"single attention layer, {name}: B={case.B}, S={case.S}, {case.Hq}/{case.Hkv} heads, "
                       f"d={case.D}, prefix {case.max_ctx_len}" + (" (ragged, shuffled pages)" if name == "ragged"
                                                                   else ""),
           "call_us": spread_us(ms), "tflops": case.flops() / (med * 1e-3) / 1e12,
           "roofline": attn_roofline(case, med, bound),
           "timing": "per call between HIP events; a 512 MB buffer read before each call"
           if name != "tiny" else "per call between HIP events"}
    if name == "tiny":
        res["roofline"] = {"bound": "latency", "note": "66 KB per call: launch latency, reported in us"}
    if name == "single":
        wm = time_each(lambda: L(sh), stream, reps, 5, None)
        res["warm_call_us"] = spread_us(wm)
        res["warm_value"] = case.B * case.S / (pct(wm, 50) * 1e-3)
        res["warm_roofline"] = attn_roofline(case, pct(wm, 50), "hbm")
        res["warm_note"] = "back to back: the 4.5 MB working set stays in the 256 MB MALL"
    ucase = None
    if name in ("tiny", "ragged"):
        ucase = synth.unmask_case(name, temperature=args.temperature, gamma=args.gamma)
        x, res["unmask"] = unmask_timing(ucase, stream, args, None if name == "tiny" else scrub)
    del scrub
    if not args.no_cpu:
        res["cpu_baseline"] = single_cpu_baseline(name, case, L, med, x if ucase is not None else None, ucase)
    return res


def single_cpu_baseline(name, case, L, gpu_ms, logits, ucase):
    """The float64 oracle on a bounded sample of the same call, at one thread and at every host
    thread, scaled to the same unit (tokens/s per attention layer)."""
    import oracle
    B, S, Hq = case.B, case.S, case.Hq
    nth = host_threads()
    out = {"kind": "oracle", "unit": "tokens/s"}
    if name in ("tiny", "single"):
        d = L.cpu_sub(0, B)
        t1 = oracle_attn_time(d, threads=1)
        tn = oracle_attn_time(d, threads=nth)
        out.update(value=B * S / tn, cores=nth, one_thread=B * S / t1, sample="the whole call")
        if logits is not None:
            out["unmask_s"] = {"1": oracle_unmask_time(logits.cpu(), ucase, 1),
                               str(nth): oracle_unmask_time(logits.cpu(), ucase, nth)}
    elif name == "ragged":
        n = 4
        d = L.cpu_sub(0, n)
        keys = int(d["ctx_len"].sum()) + n * S
        frac = keys / (sum(case.ctx_lens) + B * S)  # share of the call's work
        tn = oracle_attn_time(d, threads=nth)
        rows1 = oracle.all_rows(1, Hq, S)
        t1 = oracle_attn_time(L.cpu_sub(0, 1), rows=rows1, threads=1)
        frac1 = (int(case.ctx_lens[0]) + S) / (sum(case.ctx_lens) + B * S)
        out.update(value=B * S / (tn / frac), cores=nth, one_thread=B * S / (t1 / frac1),
                   sample=f"{n} of {B} sequences at {nth} threads, 1 sequence at 1 thread, scaled by their share "
                          f"of the call's keys")
        xs = logits[:n].cpu()
        tu = oracle_unmask_time(xs, ucase, nth)
        out["unmask"] = {"masked_rows_per_s": n * S / tu, "cores": nth,
                         "sample": f"{n} of {B} sequences (all {n * S} rows masked)"}
    else:  # long: a sample of rows of sequence 0
        d = L.cpu_sub(0, 1)
        rows_n = oracle.all_rows(1, Hq, S)
        tn = oracle_attn_time(d, rows=rows_n, threads=nth)
        rows_1 = rows_n[:: 16]
        t1 = oracle_attn_time(d, rows=rows_1, threads=1)
        total = B * Hq * S
        out.update(value=B * S / (tn * total / len(rows_n)), cores=nth,
                   one_thread=B * S / (t1 * total / len(rows_1)),
                   sample=f"{len(rows_n)} of {total} query rows at {nth} threads, {len(rows_1)} at 1 thread, "
                          f"scaled to the whole call")
    oracle.set_num_threads(nth)
    out["vs_gpu"] = "gpu/oracle = %.0fx" % ((B * S / (gpu_ms * 1e-3)) / out["value"])
    return out


# --------------------------------------------------------------------------- the denoise loop


def cpu_baseline_loop(layers, logits, case, ucase, steps_gpu, budget_s=12.0, uniforms=None):
    """The float64 oracle running one whole block of Algorithm 2 (gamma and temperature of the run)
    on n of the B sequences at every host thread: T steps of six Eq. (1) layers plus one
    ConfidenceSample, stopping when the block is clean. Also one step of one sequence at one thread.
    Reported in the same unit: noisy tokens per second per attention layer."""
    import oracle
    S, T, NL = case.S, synth.LOOP_STEPS, synth.LOOP_LAYERS
    nth = host_threads()
    one = [L.cpu_sub(0, 1) for L in layers]
    t1 = oracle_attn_time(one[0], threads=1)
    tu1 = oracle_unmask_time(logits[0][:1].cpu(), ucase, 1)
    step1 = NL * t1 + tu1
    oracle.set_num_threads(nth)
    tn = oracle_attn_time(one[0], threads=nth)
    n = max(1, min(case.B, int(budget_s / max(1e-3, steps_gpu * NL * tn))))
    subs = [L.cpu_sub(0, n) for L in layers]
    xs = [lg[:n].cpu() for lg in logits]
    us = None if uniforms is None else [u[:n].cpu() for u in uniforms]
    tok, mk = synth.make_mask_state(n, S)
    tok, mk = tok.numpy(), mk.numpy()
    t0 = time.perf_counter()
    steps = 0
    for r in range(1, T + 1):
        for d in subs:
            oracle.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Kd"], d["Vd"],
                              page_size=d["page_size"], scale=d["scale"])
        res = oracle.conf_unmask(xs[r - 1], mk, tok, gamma=oracle.f32(ucase.gamma),
                                 temperature=oracle.f32(ucase.temperature), steps_left=T - r + 1,
                                 uniforms=None if us is None else us[r - 1])
        tok, mk = res["tokens"], res["mask"]
        steps = r
        if int(mk.sum()) == 0:
            break
    wall = time.perf_counter() - t0
    return dict(value=n * S * NL * steps / wall, unit="tokens/s", cores=nth, kind="oracle",
                sample=f"one whole block of Algorithm 2 on {n} of {case.B} sequences ({steps} steps of 6 Eq. (1) "
                       f"layers plus one ConfidenceSample, prefix {case.ctx_lens[0]}, S={S}, 32/2 heads, d={case.D}) "
                       f"in {wall:.1f} s at {nth} threads",
                blocks_per_s=n / wall, steps_per_block=steps,
                one_thread={"value": S * NL / step1, "unit": "tokens/s", "cores": 1,
                            "sample": f"one denoising step of 1 sequence (6 layers at {t1:.2f} s each, unmask "
                                      f"{tu1:.3f} s); extrapolated to a block by its step count"},
                per_step_s_all_threads=wall / steps)


def run_loop(args, stream):
    case = synth.attn_case("loop")
    ucase = synth.unmask_case("loop", temperature=args.temperature, gamma=args.gamma)
    B, S, T, NL = case.B, case.S, synth.LOOP_STEPS, synth.LOOP_LAYERS
    log(f"[bench] building {NL} layer caches of {case.kv_bytes() / 1e6:.0f} MB and {T} logit steps on the GPU")
    layers = []
    for i in range(NL):
        layers.append(Layer(case, i, workspace=layers[0].ws if layers else None))
    targets = synth.spike_targets(B, S, ucase.V, seed=0, device="cuda")
    logits = [synth.make_logits(ucase, seed=0, step=r, spike=0.5 * r, targets=targets, device="cuda")
              for r in range(1, T + 1)]
    tokens = torch.empty((B, S), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, S), dtype=torch.uint8, device="cuda")
    nmask = torch.empty((B,), dtype=torch.int32, device="cuda")
    nm_host = torch.empty((B,), dtype=torch.int32, pin_memory=True)
    # --sample: each step draws its tokens from softmax(logits / temperature) with fresh uniforms
    unis = [synth.make_uniforms(B, S, seed=0, step=r, device="cuda") for r in range(1, T + 1)] if args.sample else None
    up = api.unmask_params(logits[0], mask, tokens, gamma=ucase.gamma, temperature=ucase.temperature,
                           steps_left=T, num_masked=nmask, uniforms=unis[0] if unis else None)
    uws = torch.empty(max(16, api.conf_unmask_workspace_bytes(up)), dtype=torch.uint8, device="cuda")
    lib = api.lib()
    sh = stream.cuda_stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T)]

    def enqueue_step(r, gamma, handle, timing=False):
        """Step r of Algorithm 2 on the stream `handle`: six Eq. (1) layers, one ConfidenceSample,
        and the copy of the masked counts to pinned host memory."""
        if timing:
            ev[r - 1][0].record(stream)
        for L in layers:
            L(handle)
        if timing:
            ev[r - 1][1].record(stream)
        up.gamma = gamma
        up.logits = logits[r - 1].data_ptr()
        up.steps_left = T - r + 1
        if unis:
            up.uniforms = unis[r - 1].data_ptr()
        rc = lib.tt_conf_unmask(up, uws.data_ptr(), uws.numel(), handle)
        if rc:
            raise RuntimeError(f"tt_conf_unmask failed: {api.status_string(rc)}")
        nm_host.copy_(nmask, non_blocking=True)

    # --graph: one HIP graph per step and gamma (the step's kernel arguments are fixed), so that
    # after the host reads a step's masked count the next step starts with one graph launch rather
    # than fourteen library calls. The library allocates and clears nothing, so a step captures
    # whole. On MI355X the replays measured slower than host launches (4.52 against 4.44 ms per
    # block), so they are not the default.
    graphs = {}

    def step_graphs(gamma):
        if gamma not in graphs:
            torch.cuda.synchronize()
            cs = torch.cuda.Stream()
            gs = []
            for r in range(1, T + 1):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    enqueue_step(r, gamma, cs.cuda_stream)
                gs.append(g)
            torch.cuda.synchronize()
            graphs[gamma] = gs
        return graphs[gamma]

    nm_view = nm_host.numpy()  # the pinned counts, read without a torch op
    done = torch.cuda.Event()

    def block(gamma, timing=False, graph=False):
        tokens.fill_(synth.MASK_TOKEN_ID)
        mask.fill_(1)
        gs = step_graphs(gamma) if graph else None
        steps = 0
        for r in range(1, T + 1):
            if gs:
                gs[r - 1].replay()
            else:
                enqueue_step(r, gamma, sh, timing)
            steps = r
            # the step's end (the masked counts in pinned memory), polled: the wake-up costs less
            # than a blocking stream synchronisation (4.122 against 4.137 ms per block)
            done.record(stream)
            while not done.query():
                pass
            if not nm_view.any():
                break
        return steps

    def timed_blocks(gamma, k, warmup, graph):
        for _ in range(warmup):
            block(gamma, graph=graph)
        torch.cuda.synchronize()
        total_steps = 0
        t0 = time.perf_counter()
        for _ in range(k):
            total_steps += block(gamma, graph=graph)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, total_steps

    def timed_calls(gamma, k):
        """Per-call attention times: HIP events around each step's six calls, eager launches."""
        per_call = []
        for _ in range(k):
            n = block(gamma, timing=True)
            torch.cuda.synchronize()
            per_call += [ev[r][0].elapsed_time(ev[r][1]) / NL for r in range(n)]
        return per_call

    use_graph = args.graph
    if use_graph:
        # the graphs must reproduce the eager block exactly
        n_e = block(args.gamma)
        ref = (tokens.clone(), mask.clone(), nmask.clone())
        n_g = block(args.gamma, graph=True)
        torch.cuda.synchronize()
        if n_g != n_e or not all(torch.equal(x, y) for x, y in zip(ref, (tokens, mask, nmask))):
            raise RuntimeError("graph replay of the denoise loop differs from the eager loop")
    log("[bench] warmup and timed blocks" + (" (one graph launch per step)" if use_graph else ""))
    wall, total_steps = timed_blocks(args.gamma, args.steps, args.warmup, use_graph)
    per_call = timed_calls(args.gamma, max(3, args.steps // 2))
    ms_per_block = wall * 1e3 / args.steps
    steps_per_block = total_steps / args.steps
    value = B * S * NL * total_steps / wall
    call_ms = sum(per_call) / len(per_call)
    algo = case.algorithmic_bytes()
    achieved = algo / (call_ms * 1e-3) / 1e9
    assert torch.isfinite(layers[0].out.float()).all()
    log(f"[bench] {steps_per_block:.2f} steps/block, {ms_per_block:.3f} ms/block, attention call {call_ms * 1e3:.1f} us")
    sweep = {}
    if not args.sample and math.isfinite(args.gamma):
        for g in (0.5, 0.8, 0.95):
            if g == args.gamma:
                sweep[str(g)] = {"blocks_per_s": B * args.steps / wall, "steps_per_block": steps_per_block,
                                 "tokens_per_s": value}
                continue
            k = max(3, args.steps // 2)
            w, ts = timed_blocks(g, k, 1, use_graph)
            sweep[str(g)] = {"blocks_per_s": B * k / w, "steps_per_block": ts / k,
                             "tokens_per_s": B * S * NL * ts / w}
    wl = ("full-block denoise loop (Algorithm 2): batch 32, S=16, T=16, 6 attention layers, prefix 8192, "
          f"32 q / 2 kv heads, head_dim 128, V=131072, gamma {args.gamma:g}, temperature {args.temperature:g}"
          + (", stochastic draws" if args.sample else ""))
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_block, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "global_batch": B, "seq_len": case.ctx_lens[0] + S, "parallelism": "none",
                   "denoise_steps_per_block": steps_per_block, "blocks_per_s": B * args.steps / wall,
                   "attn_call_us": call_ms * 1e3, "attn_call_tokens_per_s": B * S / (call_ms * 1e-3),
                   "attn_call_us_spread": spread_us(per_call),
                   "launch": "one HIP graph per denoising step (checked against the eager loop)" if use_graph
                   else "each call launched from the host",
                   "attn_call_timing": "HIP events around each step's six calls, eager launches, in blocks run "
                                       "right after the timed ones"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "tt_block_attn (attn_bf16_kernel + attn_bf16_finalize), one layer",
                     "algorithmic_bytes": algo},
    }
    if sweep:
        res["config"]["gamma_sweep"] = sweep
    if not args.no_power:
        log("[bench] board power during the loop")
        res["power"] = board_power(lambda: block(args.gamma, graph=use_graph))
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle): one whole block")
        cb = cpu_baseline_loop(layers, [lg for lg in logits], case, ucase, steps_per_block, uniforms=unis)
        if sweep:
            # n sequences per measured step: blocks/s = n / (steps at this gamma * seconds per step)
            n_seq = cb["blocks_per_s"] * cb["steps_per_block"] * cb["per_step_s_all_threads"]
            cb["gamma_sweep_extrapolated"] = {
                g: {"blocks_per_s": n_seq / (v["steps_per_block"] * cb["per_step_s_all_threads"]),
                    "note": "the measured gamma 0.8 step time times the GPU run's step count at this gamma"}
                for g, v in sweep.items()}
        res["cpu_baseline"] = cb
    return res, layers


def parse_power_clock(text):
    """(board watts or None, [shader clock in MHz of each GFX_n domain]) from the text that
    `amd-smi metric --power --clock` prints for one GPU."""
    m = re.search(r"SOCKET_POWER:\s+(\d+)\s*W", text)
    clocks = [int(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s+(\d+)\s*MHz", text)]
    return (int(m.group(1)) if m else None), clocks


def board_power(work, settle_s=3.0, samples=3):
    """Board power and shader clocks while `work()` is called back to back on a second host thread:
    `amd-smi metric --power --clock` read `samples` times after `settle_s` seconds, and the power cap
    from `rocm-smi --showmaxpower`. Both tools only read counters. None if amd-smi is missing."""
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    stop = threading.Event()
    errors = []

    def runner():
        try:
            while not stop.is_set():
                work()
        except Exception as e:  # reported, and the readings dropped
            errors.append(repr(e))

    th = threading.Thread(target=runner, daemon=True)
    watts, clocks = [], []
    th.start()
    try:
        time.sleep(settle_s)
        for _ in range(samples):
            out = subprocess.run([exe, "metric", "--power", "--clock"], capture_output=True, text=True,
                                 timeout=30).stdout
            w, c = parse_power_clock(out)
            if w is not None:
                watts.append(w)
            clocks += c
            time.sleep(0.5)
    except (OSError, subprocess.SubprocessError) as e:  # a tool that fails or hangs: no readings
        errors.append(repr(e))
    finally:
        stop.set()
        th.join()
        if torch.cuda.is_available():
            torch.cuda.synchronize()
    if errors or not watts:
        return None
    cap = None
    smi = shutil.which("rocm-smi")
    if smi:
        try:
            m = re.search(r"Max Graphics Package Power \(W\):\s*([\d.]+)",
                          subprocess.run([smi, "--showmaxpower"], capture_output=True, text=True,
                                         timeout=30).stdout)
            cap = float(m.group(1)) if m else None
        except (OSError, subprocess.SubprocessError):
            cap = None
    return {"board_w": watts, "cap_w": cap,
            "shader_mhz": {"min": min(clocks), "mean": sum(clocks) / len(clocks), "max": max(clocks)} if clocks
            else None,
            "sample": f"amd-smi, {samples} readings {settle_s:g} s into a run of the same blocks after the timed ones"}


APPEND_METRIC = "committed-block KV rows appended per s (one layer); achieved HBM GB/s vs peak"


def run_append(args):
    """Commit-time cache append (Algorithm 1's context update) at the denoise loop's shape: the
    S = 16 committed rows of 32 sequences with prefix 8192, 2 KV heads, d = 128, bf16, 16-token
    pages, a fresh page taken from the pool per sequence. Each call is timed on its own (HIP events
    on the stream); the cache state is restored between calls outside the timed region."""
    B, S, Hkv, D, P = 32, 16, 2, 128, 16
    L0 = 8192 - 8  # mid-page: every sequence fills its last page and takes one more
    inp = synth.make_append_inputs(B, S, Hkv, D, P, max_pages=520, ctx_lens=[L0] * B, spare_pages=64, seed=0)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    table0, ctx0 = d["page_table"].clone(), d["ctx_len"].clone()
    pc = torch.tensor([inp["pool_count"]], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = api.append_params(d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Knew"], d["Vnew"], pool=d["pool"],
                          pool_count=pc, status=status)
    lib = api.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def reset():
        d["page_table"].copy_(table0)
        d["ctx_len"].copy_(ctx0)
        pc.fill_(inp["pool_count"])

    for _ in range(args.warmup):
        reset()
        assert lib.tt_kv_append(p, sh) == 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        reset()
        e0.record(stream)
        rc = lib.tt_kv_append(p, sh)
        e1.record(stream)
        if rc:
            raise RuntimeError(f"tt_kv_append failed: {api.status_string(rc)}")
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(d["ctx_len"][0].item()) == L0 + S
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    esz = 2
    algo = 2 * 2 * B * S * Hkv * D * esz + B * (2 * 4 + 2 * 4)  # rows read and written; ctx_len and table entries
    achieved = algo / (call_ms * 1e-3) / 1e9
    res = {"metric": APPEND_METRIC, "value": B * S / (call_ms * 1e-3), "unit": "rows/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": call_ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"kv append: B={B}, S={S}, {Hkv} kv heads, d={D}, 16-token pages, prefix {L0}",
                      "global_batch": B, "seq_len": L0 + S, "parallelism": "none", "call_us": call_ms * 1e3},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": algo,
                        "note": "two launches (plan, copy) of under 1 MB: launch latency, not bandwidth"}}
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 2.0:
            r = oracle.kv_append(inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp["Knew"], inp["Vnew"],
                                 pool=inp["pool"].tolist(), pool_count=inp["pool_count"])
            assert r["status"] == 0
            n += 1
        dt = (time.perf_counter() - t0) / n
        res["cpu_baseline"] = {"value": B * S / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole call, {n} runs (each copies the caches first)"}
    return res


NLL_METRIC = "masked positions scored per s (L_MD, Eq. 4); achieved HBM GB/s vs peak"
SAMPLE_METRIC = "masked rows per s of the stochastic unmask step (temperature draw); achieved HBM GB/s vs peak"


def run_nll(args):
    """L_MD (Eq. 4) over the denoise loop's logits: 32 x 16 positions, all masked, V = 131072, bf16.
    Each call is timed between HIP events; the bytes are the logit rows read once."""
    c = synth.unmask_case("loop")
    targets = synth.spike_targets(c.B, c.S, c.V, seed=0, device="cuda").to(torch.int32)
    x = synth.make_logits(c, seed=0, step=3, spike=1.5, targets=targets, device="cuda")
    mask = torch.ones(c.B, c.S, dtype=torch.uint8, device="cuda")
    nll = torch.empty(c.B, c.S, device="cuda")
    loss = torch.zeros(1, device="cuda")
    p = api.nll_params(x, targets, mask, nll=nll, loss=loss)
    ws = torch.empty(max(16, api.lib().tt_masked_nll_workspace_bytes(p)), dtype=torch.uint8, device="cuda")
    lib = api.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for _ in range(args.warmup):
        assert lib.tt_masked_nll(p, ws.data_ptr(), ws.numel(), sh) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        rc = lib.tt_masked_nll(p, ws.data_ptr(), ws.numel(), sh)
        if rc:
            raise RuntimeError(f"tt_masked_nll failed: {api.status_string(rc)}")
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / args.steps
    n = c.B * c.S
    algo = n * c.V * 2 + n * (4 + 1 + 4)  # logit rows, targets, mask, nll
    achieved = algo / (call_ms * 1e-3) / 1e9
    res = {"metric": NLL_METRIC, "value": n / (call_ms * 1e-3), "unit": "positions/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": call_ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"masked NLL: B={c.B}, S={c.S}, V={c.V}, all masked", "global_batch": c.B,
                      "seq_len": c.S, "parallelism": "none", "call_us": call_ms * 1e3, "loss": float(loss.item())},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": algo}}
    if not args.no_cpu:
        import oracle
        xs, ts, ms = x[:2].cpu(), targets[:2].cpu(), mask[:2].cpu()
        t0 = time.perf_counter()
        r = oracle.masked_nll(xs, ts, ms)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": r["count"] / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
                               "sample": f"2 of {c.B} sequences ({r['count']} positions)"}
    return res


def run_sample(args):
    """One ConfidenceSample step with the stochastic draw (caller uniforms) on the denoise loop's
    first-step logits: 32 x 16 positions, all masked, V = 131072 bf16, gamma and temperature as
    given, 16 steps left. Each call is timed between HIP events (mask_out is a separate buffer, so
    every call sees the same all-masked state); the greedy step is timed the same way beside it.
    The bytes are the masked logit rows read once, as for the greedy step."""
    c = synth.unmask_case("loop")
    targets = synth.spike_targets(c.B, c.S, c.V, seed=0, device="cuda")
    x = synth.make_logits(c, seed=0, step=1, spike=0.5, targets=targets, device="cuda")
    mask = torch.ones(c.B, c.S, dtype=torch.uint8, device="cuda")
    mask_out = torch.empty_like(mask)
    tokens = torch.full((c.B, c.S), synth.MASK_TOKEN_ID, dtype=torch.int32, device="cuda")
    u = synth.make_uniforms(c.B, c.S, seed=0, step=1, device="cuda")
    lib = api.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def timed(uniforms):
        p = api.unmask_params(x, mask, tokens, gamma=args.gamma, temperature=args.temperature, steps_left=16,
                              mask_out=mask_out, uniforms=uniforms)
        ws = torch.empty(max(16, api.conf_unmask_workspace_bytes(p)), dtype=torch.uint8, device="cuda")
        for _ in range(args.warmup):
            assert lib.tt_conf_unmask(p, ws.data_ptr(), ws.numel(), sh) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            rc = lib.tt_conf_unmask(p, ws.data_ptr(), ws.numel(), sh)
            if rc:
                raise RuntimeError(f"tt_conf_unmask failed: {api.status_string(rc)}")
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    greedy_ms = timed(None)
    call_ms = timed(u)
    n = c.B * c.S
    algo = n * c.V * 2 + n * (4 + 1 + 1 + 4 + 4)  # logit rows, uniform, mask in/out, token, conf
    achieved = algo / (call_ms * 1e-3) / 1e9
    res = {"metric": SAMPLE_METRIC, "value": n / (call_ms * 1e-3), "unit": "masked rows/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": call_ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"stochastic unmask step: B={c.B}, S={c.S}, V={c.V}, all masked, "
                                  f"gamma {args.gamma}, temperature {args.temperature}",
                      "global_batch": c.B, "seq_len": c.S, "parallelism": "none", "call_us": call_ms * 1e3,
                      "greedy_call_us": greedy_ms * 1e3},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": algo}}
    if not args.no_cpu:
        import oracle
        xs, ms, ts, us = x[:2].cpu(), mask[:2].cpu(), tokens[:2].cpu(), u[:2].cpu()
        t0 = time.perf_counter()
        oracle.conf_unmask(xs, ms, ts, gamma=args.gamma, temperature=args.temperature, steps_left=16, uniforms=us)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": 2 * c.S / dt, "unit": "masked rows/s", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": f"2 of {c.B} sequences ({2 * c.S} masked rows)"}
    return res


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, five times: the counter reference
    for FETCH_SIZE / WRITE_SIZE (each launch reads and writes COPY_BYTES). Also reports
    the copy's bandwidth and that of a plain read-only reduction over the same buffer
    (PyTorch kernels), as references for what streaming HBM reaches on the box."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    fsrc = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    copy_ms, read_ms = [], []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.sum(fsrc, dim=0, out=sink)
        e1.record()
        torch.cuda.synchronize()
        read_ms.append(e0.elapsed_time(e1))
    cm, rm = pct(copy_ms, 50), pct(read_ms, 50)
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5,
                      "copy_GBps": 2 * COPY_BYTES / (cm * 1e-3) / 1e9, "read_GBps": COPY_BYTES / (rm * 1e-3) / 1e9,
                      "note": "median of 5; copy counts bytes read plus written"}))


def gemm_reference(seconds):
    """Dense bf16 GEMMs (8192 x 8192 x 8192 through torch.matmul, contiguous operands) back to back for
    about `seconds`: a compute reference. Board power sampled while it runs gives the energy of dense
    MFMA work on the box, beside that of the attention loop and of a plain HBM stream."""
    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    z = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, y, out=z)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters = 0
    t0 = time.perf_counter()
    e0.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            torch.matmul(x, y, out=z)
        iters += 20
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    print(json.dumps({"gemm": f"bf16 {n}x{n}x{n}", "iters": iters, "seconds": ms / 1e3,
                      "tflops": 2 * n ** 3 * iters / (ms * 1e-3) / 1e12}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="loop",
                    choices=["loop", "tiny", "single", "ragged", "long", "append", "nll", "sample"])
    ap.add_argument("--reps", type=int, default=30, help="timed calls per single-call workload (at least 20)")
    ap.add_argument("--gamma", type=float, default=0.8)
    ap.add_argument("--temperature", type=float, default=0.1)
    ap.add_argument("--sample", action="store_true",
                    help="loop workload: draw tokens at the temperature (caller uniforms) instead of the argmax")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-power", action="store_true",
                    help="loop workload: skip the board power readings taken after the timed blocks")
    ap.add_argument("--no-configs", action="store_true",
                    help="loop workload only: skip the per-config lines of the other four workloads")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the counter-reference copy")
    ap.add_argument("--gemm-reference", type=float, default=0.0, metavar="SECONDS",
                    help="run only dense bf16 GEMMs for this long (a compute reference for power readings)")
    ap.add_argument("--graph", action="store_true",
                    help="loop workload: replay each denoising step from a HIP graph instead of launching its calls "
                         "from the host (measured slower on MI355X)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the data-parallel "
              "sharding exists as a design only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_reference > 0:
        gemm_reference(args.gemm_reference)
        return
    stream = torch.cuda.current_stream()
    if args.workload == "loop":
        res, layers = run_loop(args, stream)
        del layers
        if not args.no_configs and not args.sample:
            per = []
            for name in ("tiny", "single", "ragged", "long"):
                log(f"[bench] config {CONFIG_OF[name]} ({name})")
                torch.cuda.empty_cache()
                per.append(run_single(args, name, stream))
            c5 = {"config": "C5", "metric": METRIC, "value": res["value"], "unit": "tokens/s", "dtype": "bf16",
                  "workload": res["config"]["workload"], "call_us": res["config"]["attn_call_us_spread"],
                  "blocks_per_s": res["config"]["blocks_per_s"], "roofline": res["roofline"]}
            if "cpu_baseline" in res:
                c5["cpu_baseline"] = res["cpu_baseline"]
            per.append(c5)
            res["per_config"] = per
    elif args.workload == "append":
        res = run_append(args)
    elif args.workload == "sample":
        res = run_sample(args)
    elif args.workload == "nll":
        res = run_nll(args)
    else:
        r = run_single(args, args.workload, stream)
        res = {"metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1, "steps": max(20, args.reps),
               "warmup": 5, "ms_per_step": r["call_us"]["median"] / 1e3, "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": r["dtype"], "data": "synthetic",
               "config": {k: v for k, v in r.items() if k not in ("roofline", "cpu_baseline", "metric", "value",
                                                                   "unit", "dtype")},
               "roofline": r["roofline"]}
        if "cpu_baseline" in r:
            res["cpu_baseline"] = r["cpu_baseline"]
    print(json.dumps(res))


if __name__ == "__main__":
    main()
