#!/usr/bin/env python3
"""Benchmark of the TwoTower block-diffusion hot path on one MI355X.

One step = one whole block of Algorithm 2 (Nemotron-TwoTower, arXiv 2606.26493,
section 2.2) over a batch: the block starts fully masked; each denoising step
r = 1..T runs the Eq. (1) block attention of all six attention layers (each
against its own layer-aligned context cache) and then one ConfidenceSample
(threshold gamma, steps left T-r+1); the loop stops once every position is
committed. The denoiser layers between attention and the logits need trained
weights and are not part of this path: each step's logits are synthetic
(N(0,1) plus a spike of height 0.5*t at a fixed target), drawn in advance and
resident in HBM, as are the six caches.

Default workload ("loop"): batch 32, block S=16, T=16, prefix 8192 tokens,
32 query / 2 KV heads, head_dim 128, bf16, vocabulary 131072, gamma 0.8,
temperature 0.1. The JSON line reports noisy-block tokens per second per
attention layer (B*S*layers*steps / time), the attention call's roofline, and
the CPU oracle on a bounded sample as a baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload loop|single|ragged|long]
    python bench.py --copy-calibration   # a plain device copy of known size, for counter scaling

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
import sys
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
        self.ws = workspace if workspace is not None else torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.nb = nb

    def __call__(self, stream):
        rc = api.lib().tt_block_attn(self.p, self.ws.data_ptr(), self.nb, stream)
        if rc:
            raise RuntimeError(f"tt_block_attn failed: {api.status_string(rc)}")


def cpu_baseline_loop(layers, logits, case, ucase, budget_s=12.0, uniforms=None):
    """The float64 oracle on whole sequences of the same workload (one layer's attention
    per sequence plus one unmask step), scaled to tokens/s per attention layer."""
    import oracle

    S = case.S
    L0 = layers[0].inp
    per = case.pages_of(case.ctx_lens[0])

    def sub(b0, b1):
        pages = L0["page_table"][b0:b1].cpu()
        lo = int(pages.min())
        hi = int(pages.max()) + 1
        return dict(Q=L0["Q"][b0:b1].cpu(), Kc=L0["Kc"][lo:hi].cpu(), Vc=L0["Vc"][lo:hi].cpu(),
                    page_table=(pages - lo).to(torch.int32), ctx_len=L0["ctx_len"][b0:b1].cpu(),
                    Kd=L0["Kd"][b0:b1].cpu(), Vd=L0["Vd"][b0:b1].cpu())

    def run(n):
        d = sub(0, n)
        t0 = time.perf_counter()
        oracle.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Kd"], d["Vd"],
                          page_size=case.page_size, scale=1.0 / math.sqrt(case.D))
        t1 = time.perf_counter()
        x = logits[0][:n].cpu()
        tok, mk = synth.make_mask_state(n, S)
        oracle.conf_unmask(x, mk, tok, gamma=oracle.f32(ucase.gamma), temperature=oracle.f32(ucase.temperature),
                           steps_left=synth.LOOP_STEPS, uniforms=None if uniforms is None else uniforms[:n].cpu())
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    ta, tu = run(1)
    n = max(1, min(case.B, int(budget_s / max(1e-3, synth.LOOP_LAYERS * ta + tu))))
    if n > 1:
        ta, tu = run(n)
    per_seq_step = synth.LOOP_LAYERS * ta + tu  # one denoising step of n sequences (6 layers + unmask)
    value = n * S * synth.LOOP_LAYERS / per_seq_step
    del per
    return dict(value=value, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} of {case.B} sequences: one layer's Eq. (1) attention (prefix {case.ctx_lens[0]}, "
                       f"S={S}, 32/2 heads, d={case.D}) timed {ta:.2f} s and one unmask step timed {tu:.2f} s; "
                       f"a denoising step counted as 6 attention layers plus one unmask")


def run_loop(args):
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
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T)]

    def block(timing=False):
        tokens.fill_(synth.MASK_TOKEN_ID)
        mask.fill_(1)
        steps = 0
        for r in range(1, T + 1):
            if timing:
                ev[r - 1][0].record(stream)
            for L in layers:
                L(sh)
            if timing:
                ev[r - 1][1].record(stream)
            up.logits = logits[r - 1].data_ptr()
            up.steps_left = T - r + 1
            if unis:
                up.uniforms = unis[r - 1].data_ptr()
            rc = lib.tt_conf_unmask(up, uws.data_ptr(), uws.numel(), sh)
            if rc:
                raise RuntimeError(f"tt_conf_unmask failed: {api.status_string(rc)}")
            steps = r
            nm_host.copy_(nmask, non_blocking=True)
            stream.synchronize()
            if int(nm_host.sum()) == 0:
                break
        return steps

    log("[bench] warmup")
    for _ in range(args.warmup):
        block()
    torch.cuda.synchronize()
    log("[bench] timed")
    attn_ms, n_attn_steps, total_steps = 0.0, 0, 0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        n = block(timing=True)
        total_steps += n
        torch.cuda.synchronize()
        for r in range(n):
            attn_ms += ev[r][0].elapsed_time(ev[r][1])
        n_attn_steps += n
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_block = wall * 1e3 / args.steps
    steps_per_block = total_steps / args.steps
    value = B * S * NL * total_steps / wall
    call_ms = attn_ms / (n_attn_steps * NL)
    algo = case.algorithmic_bytes()
    achieved = algo / (call_ms * 1e-3) / 1e9
    assert torch.isfinite(layers[0].out.float()).all()
    log(f"[bench] {steps_per_block:.2f} steps/block, {ms_per_block:.3f} ms/block, attention call {call_ms * 1e3:.1f} us")
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_block, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full-block denoise loop (Algorithm 2): batch 32, S=16, T=16, 6 attention layers, "
                               "prefix 8192, 32 q / 2 kv heads, head_dim 128, V=131072, "
                               f"gamma {args.gamma:g}, temperature {args.temperature:g}"
                               + (", stochastic draws" if args.sample else ""),
                   "global_batch": B, "seq_len": case.ctx_lens[0] + S, "parallelism": "none",
                   "denoise_steps_per_block": steps_per_block, "blocks_per_s": B * args.steps / wall,
                   "attn_call_us": call_ms * 1e3, "attn_call_tokens_per_s": B * S / (call_ms * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "tt_block_attn (attn_bf16_kernel + attn_bf16_finalize), one layer",
                     "algorithmic_bytes": algo},
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline_loop(layers, logits, case, ucase, uniforms=unis[0] if unis else None)
    return res


def run_single(args, name):
    """Diagnostic: one attention layer of another workload (plus its unmask for 'ragged')."""
    case = synth.attn_case(name)
    L = Layer(case, 0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for _ in range(args.warmup):
        L(sh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        L(sh)
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / args.steps
    algo = case.algorithmic_bytes()
    achieved = algo / (call_ms * 1e-3) / 1e9
    flops = case.flops()
    res = {"metric": METRIC, "value": case.B * case.S / (call_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": call_ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"single attention layer, {name}: B={case.B}, S={case.S}, "
                                  f"{case.Hq}/{case.Hkv} heads, d={case.D}, max prefix {case.max_ctx_len}",
                      "global_batch": case.B, "seq_len": case.max_ctx_len + case.S, "parallelism": "none",
                      "tflops": flops / (call_ms * 1e-3) / 1e12},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None}}
    return res


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
    for FETCH_SIZE / WRITE_SIZE (each launch reads and writes COPY_BYTES)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="loop", choices=["loop", "single", "ragged", "long", "append", "nll", "sample"])
    ap.add_argument("--gamma", type=float, default=0.8)
    ap.add_argument("--temperature", type=float, default=0.1)
    ap.add_argument("--sample", action="store_true",
                    help="loop workload: draw tokens at the temperature (caller uniforms) instead of the argmax")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the counter-reference copy")
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
    if args.workload == "loop":
        res = run_loop(args)
    elif args.workload == "append":
        res = run_append(args)
    elif args.workload == "sample":
        res = run_sample(args)
    elif args.workload == "nll":
        res = run_nll(args)
    else:
        res = run_single(args, args.workload)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
