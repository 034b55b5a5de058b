"""Benchmark of the renderer hot path on one MI355X.

A step is one ff_render_attend call at steady state: publish of the chunk's
K/V into its stage bank (Tail_H) plus segmented attention over the Gamma(i)
anchors, the H = 5 history chunks and the chunk itself, host bookkeeping
included.  The default workload is the 480p-shaped step: 12 heads, head_dim
128, T = 1560 tokens per latent, chunk 5 (Gamma = 2 anchors + 5 history
chunks + own = 20 latents: 4680 queries x 31200 keys).  Steps rotate over the
S = 4 stage banks (4 distinct key sets, 0.77 GB, more than the 256 MB
last-level cache); before each round the four banks are rewound by one chunk
(ff_stage_bank_rewind) so the same steady-state call repeats, with the
in-flight Q/K/V alternating between two input sets per stage from round to
round (8 distinct publish sources).

`--workload plan480` measures the planner role instead: one step is one
denoising ff_plan_attend call of planner block 8 of a 261-latent clip
(staging of its K/V + attention over 6 earlier blocks' anchors and its own
3 latents: 4680 queries x 32760 keys).

Prints one JSON line.  `value` = attention TFLOP/s of the whole step
(algorithmic 4*Lq*Lk*d*nh FLOPs / wall time per step).  `roofline` = the
attention kernel alone, from HIP events on the launch stream.  `cpu_baseline`
= the float64 CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E

WORKLOADS = {
    # name: (T, nh, chunk, n_latents, S, description)
    "step480": (1560, 12, 5, 81, 4, "480p renderer step: chunk 5, 4680 queries x 31200 keys "
                                     "(2 anchors + 5 history chunks + own 3 latents), 12 heads x 128"),
    "step480_21": (1560, 12, 13, 81, 4, "480p renderer step at the 21-latent cap: chunk 13, 4680 queries x "
                                         "32760 keys (3 anchors + 5 history + own), 12 heads x 128"),
    "step720": (3600, 40, 5, 81, 1, "720p renderer step: chunk 5, 10800 queries x 72000 keys "
                                    "(2 anchors + 5 history + own), 40 heads x 128"),
    "step720_21": (3600, 40, 13, 81, 1, "720p renderer step at the 21-latent cap: chunk 13, 10800 queries x "
                                         "75600 keys (3 anchors + 5 history + own), 40 heads x 128"),
    "step480_warm": (1560, 12, 5, 81, 1, "480p renderer step, warm: chunk 5 repeated on one stage bank "
                                         "(31200 keys, key set resident in the last-level cache)"),
    # whole rollouts (T, nh, -, n_latents, S, description)
    "rollout480": (1560, 12, 0, 81, 4, "480p 81-latent rollout: 9 anchors published, then 27 chunks x 4 stages "
                                       "= 108 ff_render_attend calls in wavefront order, one call per launch"),
    "rollout480_grouped": (1560, 12, 0, 81, 4, "480p 81-latent rollout as 30 grouped anti-diagonal launches "
                                               "(108 calls)"),
    "rollout65s": (1560, 12, 0, 261, 4, "480p 65 s rollout: 261 latents, 27 anchors, 87 chunks x 4 stages = "
                                        "348 calls in 90 grouped anti-diagonal launches"),
    # planner role: block 8 of a 261-latent clip (27 anchors, 9 blocks of 3)
    "plan480": (1560, 12, 8, 261, 1, "480p planner block step: block 8 of 261 latents, 4680 queries x 32760 "
                                     "keys (18 anchors of 6 earlier blocks + own 3 latents), 12 heads x 128"),
    # block-causal training form: forward + backward of one stage over a whole clip
    "bc480": (1560, 12, 0, 81, 1, "480p block-causal training pass: forward + backward of one stage over the "
                                  "81-latent clip (27 chunks of 4680 queries, 9 anchors), 12 heads x 128"),
    "bc720": (3600, 40, 0, 81, 1, "720p block-causal training pass: forward + backward of one stage over the "
                                  "81-latent clip (27 chunks of 10800 queries, 9 anchors), 40 heads x 128"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload, kernel="attn", source="ff_kernels.hip", field="traffic_bytes_per_dispatch"):
    """HBM bytes of `kernel` (`field`: per dispatch, or per step for the whole
    backward) from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or
    None when the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    src = os.path.join(ROOT, "chunked_kv_cache_amd", "csrc", "hip", source)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "-", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if fields.get("kernel_source_sha256_16") != h or field not in fields:
        return None
    return float(fields[field])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="step480", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads in the CPU oracle sample")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed region, run a plain 256 MiB device copy (read + write of known size) "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs one GPU's share; the stage-sharded multi-GPU layout is a design only)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic as syn
    from chunked_kv_cache_amd import ff

    if args.workload.startswith("plan"):
        return run_planner(args)
    if args.workload.startswith("bc"):
        return run_block_causal(args)
    if args.workload.startswith("rollout"):
        return run_rollout(args)
    T, nh, chunk, n_latents, S, desc = WORKLOADS[args.workload]
    d, H = 128, 5
    torch.cuda.set_device(0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).cuda()
    shape = ff.make_shape(n_heads=nh, head_dim=d, tokens_per_latent=T, n_latents=n_latents)
    banks = ff.StageBanks(shape, S, H)
    ctx = banks.ctx
    Lq = 3 * T

    t0 = time.time()
    n_anchor = (n_latents + 9) // 10
    for a0 in range(0, n_anchor, 3):
        blk = list(range(a0, min(a0 + 3, n_anchor)))
        K, V = syn.anchor_kv(T=T, n_heads=nh, head_dim=d, anchors=blk)
        ff.ff_anchor_bank_publish(ctx, blk[0], len(blk), dev(K), dev(V))
    # fill every stage bank with chunks 0..chunk in wavefront order
    step_inputs = {}
    scratch_o = torch.empty((Lq, nh, d), dtype=torch.bfloat16, device="cuda")
    for t in range(chunk + S):
        for k in range(S):
            i = t - k
            if 0 <= i <= chunk:
                q, kk, vv = syn.chunk_qkv(T=T, n_heads=nh, head_dim=d, chunk=i, stage=k)
                qd, kd, vd = dev(q), dev(kk), dev(vv)
                if i == chunk:
                    step_inputs[k] = (qd, kd, vd, q, kk, vv)
                ff.ff_render_attend(ctx, i, k, qd, kd, vd, scratch_o)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s")

    outs = [torch.empty((Lq, nh, d), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    lses = [torch.empty((nh, Lq), dtype=torch.float32, device="cuda") for _ in range(S)]
    stream = torch.cuda.current_stream().cuda_stream

    def rewind_all():
        for k in reversed(range(S)):
            ff.ff_stage_bank_rewind(ctx, k)

    # A second input set per stage (seeded N(0,1) bf16 drawn on the device): the
    # rounds alternate between the two, so the publishes read 8 distinct
    # 28.75 MB source sets in turn (and each publish follows an attention that
    # streamed a 192 MB key set), which keeps the sources out of the 256 MB
    # last-level cache.
    gen = torch.Generator(device="cuda").manual_seed(1)
    randn = lambda: torch.randn((Lq, nh, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    alt_inputs = {k: (randn(), randn(), randn()) for k in range(S)}

    def one_step(j):
        k = j % S
        if k == 0:
            rewind_all()
        qd, kd, vd = (step_inputs[k][:3] if (j // S) % 2 == 0 else alt_inputs[k])
        ff.ff_render_attend(ctx, chunk, k, qd, kd, vd, outs[k], lses[k], stream=stream)

    # the stage banks currently hold chunk `chunk` published once; start a round
    key_plan = None
    rewind_all()
    for k in range(S):
        if key_plan is None:
            key_plan = ff.ff_key_plan(ctx, chunk, k)
        qd, kd, vd = step_inputs[k][:3]
        ff.ff_render_attend(ctx, chunk, k, qd, kd, vd, outs[k], lses[k], stream=stream)
    Lk = key_plan.key_tokens
    flops = 4.0 * Lq * Lk * d * nh
    pub_bytes = 2 * 2 * Lq * nh * d * 2          # K and V, read + write, bf16

    steps_done = S
    for _ in range(args.warmup):
        one_step(steps_done)
        steps_done += 1
    # align the timed region to the start of a round
    while steps_done % S:
        one_step(steps_done)
        steps_done += 1
    torch.cuda.synchronize()

    # Inside the timed region the library brackets only the attention kernel
    # (the roofline's kernel) with HIP events; every event pair costs stream
    # time, so the merge and publish kernels are timed in a pass of their own
    # right after it.
    ff.ff_profile_families(ctx, ff.PROF_ATTN)
    ff.ff_profile_enable(ctx, True)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    clocks = ClockSampler().start()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for j in range(args.steps):
        events[j][0].record()
        one_step(steps_done + j)
        events[j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    clock_info = clocks.stop()
    prof = ff.ff_profile_read(ctx)
    steps_done += args.steps
    steps_ms = step_stats(events)

    ff.ff_profile_families(ctx, ff.PROF_MERGE | ff.PROF_PUBLISH)
    ff.ff_profile_enable(ctx, True)           # resets the totals
    n_detail = max(S, min(args.steps, 40) // S * S)
    for j in range(n_detail):
        one_step(steps_done + j)
    steps_done += n_detail
    detail = ff.ff_profile_read(ctx)
    ff.ff_profile_enable(ctx, False)
    ff.ff_profile_families(ctx, ff.PROF_ALL)

    ms_per_step = wall * 1e3 / args.steps
    tflops = flops * args.steps / wall / 1e12
    attn_ms = prof["attn_ms"] / max(prof["attn_launches"], 1)
    merge_ms = detail["merge_ms"] / detail["merge_launches"] if detail["merge_launches"] else 0.0
    pub_ms = detail["publish_ms"] / max(detail["publish_launches"], 1)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    pub_gbps = pub_bytes / (pub_ms * 1e-3) / 1e9
    log(f"attention kernel {attn_ms:.3f} ms ({attn_tflops:.1f} TFLOP/s), merge {merge_ms:.3f} ms, "
        f"publish {pub_ms * 1e3:.1f} us ({pub_gbps:.0f} GB/s), step {ms_per_step:.3f} ms "
        f"(median {steps_ms['median']:.3f}, min {steps_ms['min']:.3f}); clocks {clock_info}")

    copy_us, copy_med_us = publish_copy_reference(one_step, steps_done, pub_bytes)
    copy_gbps = pub_bytes / (copy_us * 1e-6) / 1e9
    log(f"device copy of the publish's bytes after a step: {copy_us:.1f} us ({copy_gbps:.0f} GB/s); "
        f"publish / copy rate {pub_gbps / copy_gbps:.2f}")

    if args.calibration_copy:
        calibration_copy()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(ctx, step_inputs[0][3:], chunk, T, nh, d, args.cpu_heads, n_latents)

    out = {
        "metric": "renderer chunk-attention TFLOP/s (% bf16 MFMA peak) + chunk-steps/s; publish GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shapes of the 480p/720p renderer)",
        "config": {"workload": desc, "queries": Lq, "keys": Lk, "heads": nh, "head_dim": d,
                   "tokens_per_latent": T, "chunk": chunk, "stage_banks": S, "history": H,
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "chunk_steps_per_s": round(args.steps / wall, 2),
        "step_ms": steps_ms,
        "clocks": clock_info,
        "attention_kernel_ms": round(attn_ms, 4),
        "merge_kernel_ms": round(merge_ms, 4),
        "publish_kernel_us": round(pub_ms * 1e3, 2),
        "publish_gbps": round(pub_gbps, 1),
        "publish_pct_hbm": round(100 * pub_gbps / PEAK_HBM_GBPS, 2),
        "publish_copy_reference": {
            "what": "one hipMemcpyAsync (torch copy_) of the same bytes (a chunk's K and V, read once and written "
                    "once), event-timed right after a step, 8 rotating sources",
            "us": round(copy_us, 2), "median_us": round(copy_med_us, 2), "gbps": round(copy_gbps, 1),
            "pct_hbm": round(100 * copy_gbps / PEAK_HBM_GBPS, 2),
            "publish_over_copy": round(pub_gbps / copy_gbps, 3)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    banks.close()


class ClockSampler:
    """Samples the GPU's current shader and memory clock levels (the entries
    marked '*' in the driver's pp_dpm_sclk / pp_dpm_mclk files) every 20 ms
    in a thread while the timed region runs; reports their range and mode."""

    def __init__(self):
        import glob
        self.files = {k: sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{k}")) for k in ("sclk", "mclk")}
        self.samples = {"sclk": [], "mclk": []}
        self._stop = None
        self._thread = None

    @staticmethod
    def _current_mhz(path):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return int("".join(ch for ch in line.split(":", 1)[1] if ch.isdigit()))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, paths in self.files.items():
                vals = [v for v in (self._current_mhz(p) for p in paths) if v]
                if vals:
                    self.samples[k].append(max(vals))
            self._stop.wait(0.02)

    def start(self):
        import threading
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()
        out = {}
        for k, v in self.samples.items():
            if v:
                out[f"{k}_mhz"] = {"min": min(v), "max": max(v), "mode": max(set(v), key=v.count),
                                   "samples": len(v)}
            else:
                out[f"{k}_mhz"] = None
        out["source"] = "pp_dpm_sclk / pp_dpm_mclk current level, sampled every 20 ms" \
            if any(self.files.values()) else "not readable on this host"
        return out


def step_stats(events):
    """Median / min / mean of per-step device times from (start, end) event pairs."""
    ms = sorted(a.elapsed_time(b) for a, b in events)
    return {"median": round(ms[len(ms) // 2], 4), "min": round(ms[0], 4), "mean": round(sum(ms) / len(ms), 4),
            "n": len(ms)}


def publish_copy_reference(one_step, j0, n_bytes, n=40):
    """The platform's device copy of the publish's bytes, for comparison: after
    each of n further steps, one hipMemcpyAsync (torch copy_) of n_bytes/2
    bytes (a chunk's K and V: n_bytes counts each byte read and written)
    between buffers that rotate over 8 sources and 4 destinations, bracketed
    by its own events -- the conditions of the publish, which also follows a
    step's kernels.  Returns the mean and median time in us."""
    import torch
    half = n_bytes // 2
    srcs = [torch.randint(0, 255, (half,), dtype=torch.uint8, device="cuda") for _ in range(8)]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(4)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for j in range(n):
        one_step(j0 + j)
        ev[j][0].record()
        dsts[j % 4].copy_(srcs[j % 8])
        ev[j][1].record()
    torch.cuda.synchronize()
    us = sorted(1e3 * a.elapsed_time(b) for a, b in ev)
    return sum(us) / n, us[n // 2]


def calibration_copy():
    """A plain device copy of known size after the timed region: its rocprofv3
    FETCH_SIZE / WRITE_SIZE scale those counters to bytes."""
    import torch
    n = 64 << 20                                   # 64 Mi floats = 256 MiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log("calibration copy: 3 x (256 MiB read + 256 MiB write), kernel vectorized_elementwise add")


def run_rollout(args):
    """Whole-rollout workloads: anchors published (untimed), then every
    (chunk, stage) call of the wavefront schedule, timed end to end.  Inputs
    come from a pool of 8 seeded N(0,1) bf16 Q/K/V sets drawn on the device
    (values do not change the work; the pool keeps setup short)."""
    import torch

    from chunked_kv_cache_amd import ff

    T, nh, _, n_latents, S, desc = WORKLOADS[args.workload]
    d, H = 128, 5
    grouped = args.workload != "rollout480"
    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda").manual_seed(0)
    Lq = 3 * T
    randn = lambda n: torch.randn((n, nh, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pool = [(randn(Lq), randn(Lq), randn(Lq)) for _ in range(8)]
    shape = ff.make_shape(n_heads=nh, head_dim=d, tokens_per_latent=T, n_latents=n_latents)
    banks = ff.StageBanks(shape, S, H)
    # The library's own wavefront schedule and planner blocks.
    counts = ff.ff_clip_layout(shape, S)
    sched = [ff.ff_wavefront(shape, S, t) for t in range(counts["n_diagonals"])]
    n_calls = sum(len(x) for x in sched)
    outs = [torch.empty((Lq, nh, d), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    blocks = [ff.ff_planner_block(shape, b) for b in range(counts["n_planner_blocks"])]
    anchor_kv = [(randn(len(b) * T), randn(len(b) * T)) for b in blocks]
    stream = torch.cuda.current_stream().cuda_stream

    def rollout():
        banks.close()
        banks.ctx = ff.ff_stage_bank_create(shape, S, H, banks.workspace, banks.ws_bytes)
        ctx = banks.ctx
        for b, (K, V) in zip(blocks, anchor_kv):
            ff.ff_anchor_bank_publish(ctx, b[0], len(b), K, V, stream=stream)
        torch.cuda.synchronize()
        flops = 0.0
        j = 0
        t0 = time.perf_counter()
        for diag in sched:
            plans = [ff.ff_key_plan(ctx, i, k) for i, k in diag]
            flops += sum(4.0 * Lq * p.key_tokens * d * nh for p in plans)
            sets = [pool[(j + n) % 8] for n in range(len(diag))]
            j += len(diag)
            if grouped:
                ff.ff_render_attend_grouped(ctx, [i for i, _ in diag], [k for _, k in diag],
                                            [x[0] for x in sets], [x[1] for x in sets], [x[2] for x in sets],
                                            [outs[k] for _, k in diag], stream=stream)
            else:
                for (i, k), x in zip(diag, sets):
                    ff.ff_render_attend(ctx, i, k, x[0], x[1], x[2], outs[k], stream=stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, flops

    reps = max(1, min(args.steps, 5))
    for _ in range(max(1, min(args.warmup, 2))):
        rollout()
    times = []
    for _ in range(reps):
        dt, flops = rollout()
        times.append(dt)
    dt = sorted(times)[len(times) // 2]
    tflops = flops / dt / 1e12
    log(f"rollout: {n_calls} calls in {len(sched)} diagonals, median {dt * 1e3:.1f} ms "
        f"(min {min(times) * 1e3:.1f}), {flops / 1e12:.1f} TFLOP, {tflops:.1f} TFLOP/s, "
        f"{n_calls / dt:.0f} chunk-steps/s")
    # One more rollout with per-kernel HIP events (outside the timed ones): the
    # Tail_H publishes of a grouped launch move every pair's K/V at once.
    orig_create = ff.ff_stage_bank_create

    def create_profiled(*a, **k):
        ctx = orig_create(*a, **k)
        ff.ff_profile_enable(ctx, True)
        return ctx
    ff.ff_stage_bank_create = create_profiled
    try:
        rollout()
    finally:
        ff.ff_stage_bank_create = orig_create
    prof = ff.ff_profile_read(banks.ctx)
    pub_bytes = n_calls * 2 * 2 * Lq * nh * d * 2                # K and V of every call, read + write
    pub_gbps = pub_bytes / (prof["publish_ms"] * 1e-3) / 1e9
    attn_tflops = flops / (prof["attn_ms"] * 1e-3) / 1e12
    log(f"kernels: attention {prof['attn_ms']:.1f} ms ({attn_tflops:.1f} TFLOP/s) in {prof['attn_launches']} "
        f"launches; publish {prof['publish_ms']:.2f} ms in {prof['publish_launches']} launches "
        f"({pub_gbps:.0f} GB/s, {100 * pub_gbps / PEAK_HBM_GBPS:.1f}% of HBM)")
    res = {
        "metric": "renderer rollout TFLOP/s (% bf16 MFMA peak) + chunk-steps/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": max(1, min(args.warmup, 2)),
        "ms_per_step": round(dt * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, a pool of 8 Q/K/V sets drawn on the device)",
        "config": {"workload": desc, "calls": n_calls, "launches": len(sched) if grouped else n_calls,
                   "heads": nh, "head_dim": d, "tokens_per_latent": T, "stage_banks": S, "history": H,
                   "rollout_tflop": round(flops / 1e12, 2), "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "chunk_steps_per_s": round(n_calls / dt, 1),
        "attention_kernel_tflops": round(attn_tflops, 1),
        "publish_launches": prof["publish_launches"],
        "publish_gbps": round(pub_gbps, 1),
        "publish_pct_hbm": round(100 * pub_gbps / PEAK_HBM_GBPS, 2),
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)
    banks.close()


def run_planner(args):
    """Planner-role workload: one step = one denoising ff_plan_attend call of a
    planner block (staging of its K/V in the anchor bank + segmented attention
    over the earlier blocks' anchors and its own latents).  The anchors of the
    earlier blocks are published once; the repeated call changes no state, as
    the denoising steps of one block do."""
    import numpy as np
    import torch

    import synthetic as syn
    from chunked_kv_cache_amd import ff

    T, nh, block, n_latents, _, desc = WORKLOADS[args.workload]
    d = 128
    torch.cuda.set_device(0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).cuda()
    shape = ff.make_shape(n_heads=nh, head_dim=d, tokens_per_latent=T, n_latents=n_latents)
    banks = ff.StageBanks(shape, 1, 5)
    ctx = banks.ctx
    t0 = time.time()
    for a0 in range(0, 3 * block, 3):
        blk = [a0, a0 + 1, a0 + 2]
        K, V = syn.anchor_kv(T=T, n_heads=nh, head_dim=d, anchors=blk)
        ff.ff_anchor_bank_publish(ctx, a0, 3, dev(K), dev(V))
    host = syn.planner_qkv(T=T, n_heads=nh, head_dim=d, block=block, step=0, n_latents=3)
    qd, kd, vd = (dev(x) for x in host)
    Lq = 3 * T
    out = torch.empty((Lq, nh, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((nh, Lq), dtype=torch.float32, device="cuda")
    plan = ff.ff_plan_key_plan(ctx, block)
    Lk = plan.key_tokens
    flops = 4.0 * Lq * Lk * d * nh
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s")
    for _ in range(args.warmup):
        ff.ff_plan_attend(ctx, block, qd, kd, vd, out, lse, stream=stream)
    torch.cuda.synchronize()
    # As in the renderer step: only the attention kernel carries event pairs
    # inside the timed region; the staging copy is timed in a pass after it.
    ff.ff_profile_families(ctx, ff.PROF_ATTN)
    ff.ff_profile_enable(ctx, True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        ff.ff_plan_attend(ctx, block, qd, kd, vd, out, lse, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    prof = ff.ff_profile_read(ctx)
    ff.ff_profile_families(ctx, ff.PROF_ANCHOR)
    ff.ff_profile_enable(ctx, True)
    for _ in range(min(args.steps, 40)):
        ff.ff_plan_attend(ctx, block, qd, kd, vd, out, lse, stream=stream)
    detail = ff.ff_profile_read(ctx)
    ff.ff_profile_enable(ctx, False)
    ff.ff_profile_families(ctx, ff.PROF_ALL)
    ms_per_step = wall * 1e3 / args.steps
    tflops = flops * args.steps / wall / 1e12
    attn_ms = prof["attn_ms"] / max(prof["attn_launches"], 1)
    stage_us = 1e3 * detail["anchor_ms"] / max(detail["anchor_launches"], 1)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    log(f"attention kernel {attn_ms:.3f} ms ({attn_tflops:.1f} TFLOP/s), staging {stage_us:.1f} us, "
        f"step {ms_per_step:.3f} ms")
    if args.calibration_copy:
        calibration_copy()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_planner(host, block, T, nh, d, args.cpu_heads, n_latents)
    res = {
        "metric": "planner block-attention TFLOP/s (% bf16 MFMA peak)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V and anchors, 480p planner shapes)",
        "config": {"workload": desc, "queries": Lq, "keys": Lk, "heads": nh, "head_dim": d,
                   "tokens_per_latent": T, "block": block, "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "attention_kernel_ms": round(attn_ms, 4),
        "staging_kernel_us": round(stage_us, 2),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    banks.close()


def run_block_causal(args):
    """Block-causal training form: one step = ff_bc_forward + ff_bc_backward of
    one stage over the whole clip (operand copies, the segmented attention
    over every chunk's key set, row statistics, dQ and dK/dV kernels)."""
    import torch

    from chunked_kv_cache_amd import ff

    T, nh, _, n_latents, _, desc = WORKLOADS[args.workload]
    d, H = 128, 5
    torch.cuda.set_device(0)
    shape = ff.make_shape(n_heads=nh, head_dim=d, tokens_per_latent=T, n_latents=n_latents)
    counts = ff.ff_clip_layout(shape)
    nc, na, L = counts["n_chunks"], counts["n_anchors"], shape.chunk_latents * T
    bc = ff.BlockCausal(shape, H)
    t0 = time.time()
    # Seeded N(0,1) bf16 drawn on the device (the clip is 1.6 GB of inputs).
    gen = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda rows: torch.randn((rows, nh, d), generator=gen, device="cuda").to(torch.bfloat16)
    Ka, Va = rnd(na * T), rnd(na * T)
    Q, K, V, dO = rnd(nc * L), rnd(nc * L), rnd(nc * L), rnd(nc * L)
    O = torch.empty_like(Q)
    lse = torch.empty((nc, nh, L), dtype=torch.float32, device="cuda")
    dQ, dK, dV, dKa, dVa = (torch.empty_like(x) for x in (Q, K, V, Ka, Va))
    keys = [ff.ff_bc_key_plan(bc.ctx, i).key_tokens for i in range(nc)]
    pair_flops = float(sum(L * lk for lk in keys)) * d * nh          # sum of Lq*Lk*d*nh
    fwd_flops, bwd_flops = 4.0 * pair_flops, 10.0 * pair_flops         # backward = 2.5 x forward
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s; {fwd_flops / 1e12:.2f} TFLOP forward, {bwd_flops / 1e12:.2f} backward")

    def step():
        ff.ff_bc_forward(bc.ctx, Ka, Va, Q, K, V, O, lse, stream=stream)
        ff.ff_bc_backward(bc.ctx, Ka, Va, Q, K, V, O, lse, dO, dQ, dK, dV, dKa, dVa, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ff.ff_bc_profile_enable(bc.ctx, True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    prof = ff.ff_bc_profile_read(bc.ctx)
    ff.ff_bc_profile_enable(bc.ctx, False)
    ms_per_step = wall * 1e3 / args.steps
    tflops = (fwd_flops + bwd_flops) * args.steps / wall / 1e12
    per = lambda k: prof[f"{k}_ms"] / args.steps                     # ms per step of a kernel family
    kern = {"attention": (per("attn"), fwd_flops), "dq": (per("bwd_dq"), 6.0 * pair_flops),
            "dk": (per("bwd_dk"), 6.0 * pair_flops), "dv": (per("bwd_dv"), 4.0 * pair_flops)}
    for k, (ms, fl) in kern.items():
        log(f"{k}: {ms:.2f} ms per step, {fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    log(f"merge {per('merge'):.3f} ms, copies {per('layout'):.3f} ms, row statistics {per('bwd_pre'):.3f} ms; "
        f"step {ms_per_step:.2f} ms")
    # The roofline describes the backward as one unit on the method's own count
    # (10P; the kernels' recomputation of S and dP is not counted as work).
    bwd_ms = per("bwd_dq") + per("bwd_dk") + per("bwd_dv")
    achieved = bwd_flops / (bwd_ms * 1e-3) / 1e12
    log(f"backward (dQ + dK + dV kernels): {bwd_ms:.2f} ms per step, {achieved:.1f} TFLOP/s on the 10P count")
    if args.calibration_copy:
        calibration_copy()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_block_causal(T, nh, d, n_latents, H, 1)

    res = {
        "metric": "block-causal training attention TFLOP/s (forward + backward, % bf16 MFMA peak)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V/dO and anchors drawn on the device, clip shapes of the "
                "workload)",
        "config": {"workload": desc, "chunks": nc, "anchors": na, "queries_per_chunk": L, "heads": nh,
                   "head_dim": d, "history": H, "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "forward_tflops": round(fwd_flops / (sum(per(k) for k in ("layout", "attn", "merge")) * 1e-3) / 1e12, 1),
        "kernel_ms_per_step": {k: round(v[0], 3) for k, v in kern.items()} |
                              {"merge": round(per("merge"), 3), "copies": round(per("layout"), 3),
                               "row_statistics": round(per("bwd_pre"), 3)},
        "roofline": {"bound": "mfma", "kernel": "backward: bc_dq + bc_dk + bc_dv, one launch each per step",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, "bc_dk", "ff_bc_kernels.hip",
                                                 "backward_traffic_bytes_per_step"),
                     "algorithmic_work": "10P = 10 x sum over chunks of Lq*Lk*d*nh (dQ, dK, dV and the dP, S "
                                         "products of the standard backward count)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    bc.close()


def cpu_baseline_block_causal(T, nh, d, n_latents, H, n_heads_sample, chunk=5):
    """The float64 oracle's block-causal forward and backward restricted to
    the query rows of one steady-state chunk, on `n_heads_sample` heads."""
    import oracle as orc
    import synthetic as syn
    threads = _threads()
    cfg = orc.FFConfig(tokens_per_latent=T, n_heads=n_heads_sample, head_dim=d, n_latents=n_latents, history=H)
    nc, na = orc.n_chunks(cfg), orc.n_anchors(cfg)
    srcs = orc.bc_key_sources(cfg, chunk)
    need = [j for k, j in srcs if k == "chunk"]
    hs = slice(0, n_heads_sample)
    Ka, Va = (syn.as_f64(x, "bf16")[:, hs] for x in syn.anchor_kv(T=T, n_heads=nh, head_dim=d, anchors=range(na)))
    Q, K, V, dO = (syn.as_f64(x, "bf16")[:, hs]
                   for x in syn.clip_tensors(T=T, n_heads=nh, head_dim=d, n_chunks=nc, chunks=need))
    t0 = time.perf_counter()
    orc.bc_forward(cfg, Ka, Va, Q, K, V, chunks=[chunk])
    orc.bc_backward(cfg, Ka, Va, Q, K, V, dO, chunks=[chunk])
    dt = time.perf_counter() - t0
    n_keys = sum(T if k == "anchor" else 3 * T for k, _ in srcs)
    flops = 14.0 * 3 * T * n_keys * d * n_heads_sample
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle block-causal forward + backward for the queries of chunk {chunk} "
                      f"({n_keys} keys), {n_heads_sample} of {nh} heads: {flops / 1e9:.0f} GFLOP in {dt:.1f} s"}


def cpu_baseline_planner(host_qkv, block, T, nh, d, n_heads_sample, n_latents):
    """The float64 oracle's planner call for the same block on the first
    `n_heads_sample` heads (key-source gather + attention)."""
    import oracle as orc
    import synthetic as syn
    threads = _threads()
    cfg = orc.FFConfig(tokens_per_latent=T, n_heads=n_heads_sample, head_dim=d, n_latents=n_latents, n_stages=1)
    ro = orc.Rollout(cfg)
    hs = slice(0, n_heads_sample)
    f64 = lambda x: syn.as_f64(x, "bf16")[:, hs]
    for a in range(3 * block):
        K, V = syn.anchor_kv(T=T, n_heads=nh, head_dim=d, anchors=[a])
        ro.anchors[a] = (f64(K), f64(V))
    q, kk, vv = (f64(x) for x in host_qkv)
    n_keys = T * len(ro.plan_key_sources(block))
    t0 = time.perf_counter()
    ro.plan_attend(block, q, kk, vv)
    dt = time.perf_counter() - t0
    flops = 4.0 * q.shape[0] * n_keys * d * n_heads_sample
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle planner call for block {block} ({n_keys} keys), {n_heads_sample} of "
                      f"{nh} heads: {flops / 1e9:.0f} GFLOP in {dt:.1f} s"}


def _host_info():
    """CPU model and the BLAS the oracle's numpy runs on (threadpoolctl)."""
    import numpy  # noqa: F401  (loads the BLAS so threadpoolctl can see it)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')} ({libs[0].get('threading_layer')})"
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "affinity_cores": len(os.sched_getaffinity(0))}


def tiny_rollout_one_thread():
    """The float64 oracle's whole tiny rollout (fp32 inputs: T = 16, 2 heads,
    d = 64, 81 latents, 9 anchors, 27 chunks x 4 stages = 108 calls) on one
    BLAS thread: seconds and GFLOP/s."""
    import oracle as orc
    import synthetic as syn
    from threadpoolctl import threadpool_limits
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=64)
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        ro = orc.Rollout(cfg)
        for blk in orc.planner_blocks(cfg):
            K, V = syn.anchor_kv(T=16, n_heads=2, head_dim=64, anchors=blk, dtype="f32")
            ro.publish_anchors(blk[0], syn.as_f64(K, "f32"), syn.as_f64(V, "f32"))
        flops = 0.0
        for diag in orc.schedule(cfg):
            for i, k in diag:
                q, kk, vv = (syn.as_f64(x, "f32") for x in syn.chunk_qkv(T=16, n_heads=2, head_dim=64, chunk=i,
                                                                          stage=k, dtype="f32"))
                nk = sum(16 if kind == "anchor" else 48 for kind, _ in ro.key_sources(i, k))
                ro.render_attend(i, k, q, kk, vv)
                flops += 4.0 * 48 * nk * 64 * 2
        dt = time.perf_counter() - t0
    return {"seconds": round(dt, 3), "gflops": round(flops / dt / 1e9, 3), "calls": 108,
            "what": "float64 oracle, whole tiny fp32 rollout (inputs, Tail_H banks, 108 calls), 1 BLAS thread"}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                   default=len(os.sched_getaffinity(0)))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(ctx, host_qkv, chunk, T, nh, d, n_heads_sample, n_latents):
    """The float64 oracle on a bounded sample of the same workload: its whole
    renderer call (order checks, gather of the key sources, attention, Tail_H
    publish) for two consecutive steady-state chunks (`chunk`, `chunk`+1, both
    20 key latents at 480p), on the first `n_heads_sample` heads."""
    import numpy as np
    import oracle as orc
    import synthetic as syn
    threads = _threads()
    cfg = orc.FFConfig(tokens_per_latent=T, n_heads=n_heads_sample, head_dim=d, n_latents=n_latents, n_stages=1)
    ro = orc.Rollout(cfg)
    hs = slice(0, n_heads_sample)
    f64 = lambda x: syn.as_f64(x, "bf16")[:, hs]
    for a in sorted(set(orc.gamma(cfg, chunk)) | set(orc.gamma(cfg, chunk + 1))):
        K, V = syn.anchor_kv(T=T, n_heads=nh, head_dim=d, anchors=[a])
        ro.anchors[a] = (f64(K), f64(V))
    for i in range(max(0, chunk - cfg.history), chunk):
        _, kk, vv = syn.chunk_qkv(T=T, n_heads=nh, head_dim=d, chunk=i, stage=0)
        ro.banks[0].append((i, f64(kk), f64(vv)))
    ro.next_chunk[0] = chunk
    calls = [(chunk, [f64(x) for x in host_qkv]),
             (chunk + 1, [f64(x) for x in syn.chunk_qkv(T=T, n_heads=nh, head_dim=d, chunk=chunk + 1, stage=0)])]
    flops = 0.0
    t0 = time.perf_counter()
    for i, (q, kk, vv) in calls:
        ro.render_attend(i, 0, q, kk, vv)
    dt = time.perf_counter() - t0
    for i in (chunk, chunk + 1):
        flops += 4.0 * 3 * T * T * orc.key_latents(cfg, i, cfg.history) * d * n_heads_sample
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle renderer calls for chunks {chunk} and {chunk + 1} (stage 0, 20 key "
                      f"latents each), {n_heads_sample} of {nh} heads: {flops / 1e9:.0f} GFLOP in {dt:.1f} s",
            "seconds_per_chunk_step": round(dt / 2 * nh / n_heads_sample, 2),
            **_host_info(), "tiny_rollout_1_thread": tiny_rollout_one_thread()}


if __name__ == "__main__":
    main()
