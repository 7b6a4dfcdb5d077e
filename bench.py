#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
routing (router logits, top-K, renormalised weights), grouping, the experts'
SwiGLU and the weighted combine -- one moe_layer call.  The headline workload
is the speculative verify step: 5 tokens (4 drafted + 1, the pages' `--spec
4`), hidden 2048, 512 experts, top-10, expert width 512, bf16 weights, fp32
router, rotating over 8 independently generated weight sets so the 256 MB
Infinity Cache cannot serve the ~300 MB a step reads.  Further workloads are
reported under "also": the 8192-token prefill chunk, the pruning statistic over
48 x 262144 x 512 logits with the expert profile built from it, the pruned
48-layer int4 stack (plain and with 41 steered layers), the verify layer and
stack with int4 / int3 / int2 experts, and the measured HBM / MFMA ceilings.

--steps K / --warmup W are honoured exactly for the headline (W untimed steps,
then K timed steps between two HIP events on the launch stream); the per-step
median / p10 / p90 come from a further max(200, K) individually timed steps.
Every workload's oracle (single-threaded C, fp64) is timed on a bounded sample
on one host core.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W]
                    [--workloads verify,prefill,freq,stack,lowbit,peaks,copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "routed tokens/s per MoE layer (8192-tok prefill; 5-tok verify); % HBM/MFMA peak"
N_SETS = 8                     # rotating weight sets: 8 x 3.2 GB defeats the 256 MB MALL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "routed_expert_ffn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# kernel sources behind each measured call (the counter summary of a call is
# void once any of them changes)
SRC = {
    "verify_step": ("verify.hip", "route.hip", "stream.h", "common.h", "api.hip"),
    "ffn_prefill": ("ffn_gemm.hip", "ffn.hip", "common.h"),
    "freq": ("freq.hip", "common.h"),
}


def measured_traffic(key):
    """HBM bytes per call from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE of the call's kernels at this call's shape, each
    scaled by the same counter's reading on a plain copy of known size), if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if key is None or not os.path.exists(p):
        return None
    try:
        d = json.load(open(p)).get(key)
    except (OSError, ValueError):
        return None
    if not d or d.get("src_sha") != src_hash(*SRC[key]):
        return None
    return d.get("bytes_per_call")


def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(cpu_model=model, nproc=os.cpu_count(), cpus_usable=len(os.sched_getaffinity(0)))


class Timer:
    """HIP events on the current stream (the one the library calls launch on),
    bracketed by device synchronisation."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, reps=1):
        torch = self.torch
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return s.elapsed_time(e) / 1e3, wall

    def per_step(self, fns, n, start=0):
        """Durations (us) of n steps, each between its own pair of events; step i runs fns[(start + i) % len]."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            a, b = evs[i]
            a.record()
            fns[(start + i) % len(fns)]()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]


def dist(us):
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return dict(runs=len(us), median_us=round(float(np.median(a)), 2), p10_us=round(float(np.percentile(a, 10)), 2),
                p90_us=round(float(np.percentile(a, 90)), 2), mean_us=round(float(a.mean()), 2))


def capture(torch, fn):
    """Capture fn() (a sequence of library calls on the current stream) in a HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # warm: allocations and lazy init happen outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# ------------------------------------------------------------------ verify / prefill layers
def layer_bytes_and_flops(s, counts_list, expert_bytes, residual=False):
    """Algorithmic (compulsory) HBM bytes and flops of one layer step from the
    run's actual routing: the router, the input rows, every touched expert's
    three matrices once, the output rows (and the residual), the routing and
    grouping outputs.  Intermediates that stay in the caches are not counted."""
    n = s.T * s.K
    out = []
    for counts in counts_list:
        touched = int((counts > 0).sum())
        b_router = s.E * s.H * 4 + s.T * s.H * 2
        b_experts = touched * expert_bytes
        b_io = s.T * s.H * 2 * (2 if residual else 1) + n * 4 * 4 + s.E * 8
        f_router = 2.0 * s.T * s.H * s.E
        f_ffn = 2.0 * n * 3 * s.H * s.F
        out.append(dict(touched=touched, b_router=b_router, b_experts=b_experts,
                        b_step=b_router + b_experts + b_io, f_router=f_router, f_ffn=f_ffn))
    return out


def bench_layer(torch, moe, synth, shape, cfg_id, steps, warmup, sets, use_graph, name, stat_runs=0, parts=True):
    """W untimed then K timed steps (one moe_layer call each, rotating over the
    weight sets), the per-step distribution over stat_runs more, and (parts)
    the separate calls of the same layer for reference."""
    dev = torch.device("cuda:0")
    log(f"[{name}] generating {sets} weight set(s) of {shape}")
    layers = [synth.make_device_layer(shape, seed=0, cfg=cfg_id, layer=i, device=dev) for i in range(sets)]
    x = layers[0].x
    for L in layers[1:]:
        L.x = x
    torch.cuda.synchronize()
    wdt = {"bf16": moe.BF16, "int4": moe.INT4_B32, "int3": moe.INT3_B32, "int2": moe.INT2_B32}[shape.wdt]
    lw = moe.LayerWorkspace(shape.T, shape.H, shape.E, shape.K, shape.F, x_dtype=x.dtype, w_dtype=wdt)

    def step(L):
        return moe.layer(L.x, L.wr, L.wg, L.wu, L.wd, shape.K, bias=L.bias, sg=L.sg, su=L.su, sd=L.sd, lw=lw)

    # per-set routing (for the algorithmic byte counts and the per-call timings)
    per_set = []
    for L in layers:
        _, r = step(L)
        per_set.append({k: v.clone() for k, v in r.items()})
    torch.cuda.synchronize()
    counts = [p["counts"].cpu().numpy() for p in per_set]
    acct = layer_bytes_and_flops(shape, counts, synth.expert_bytes(shape))

    fns = [(capture(torch, lambda L=L: step(L)).replay if use_graph else (lambda L=L: step(L))) for L in layers]
    # consecutive steps run as one graph of consecutive layer calls in rotation
    # order (as a model's consecutive layers would), so that a step does not
    # carry a whole graph launch: one graph per run of sets j .. j + m - 1
    # (m up to the end of the rotation), captured beforehand, so that any step
    # count replays as whole runs (a full rotation is the run from set 0)
    runs = {}
    if use_graph and sets > 1:
        for j0 in range(sets):
            for m in range(2, sets - j0 + 1):
                runs[(j0, m)] = capture(torch, lambda j0=j0, m=m: [step(L) for L in layers[j0:j0 + m]]).replay
    run_all = runs.get((0, sets))

    def run_steps(n, start):
        i = 0
        while i < n:
            j = (start + i) % sets
            m = min(sets - j, n - i)
            if m > 1 and (j, m) in runs:
                runs[(j, m)]()
            else:
                m = 1
                fns[j]()
            i += m

    timer = Timer(torch)
    if warmup > 0:
        timer.run(lambda: run_steps(warmup, 0))
    dt, wall = timer.run(lambda: run_steps(steps, warmup))
    ms = dt / steps * 1e3
    stats = dist(timer.per_step(fns, stat_runs, warmup + steps)) if stat_runs else None
    b_step = sum(a["b_step"] for a in acct) / len(acct)
    f_ffn = acct[0]["f_ffn"]
    f_all = acct[0]["f_ffn"] + acct[0]["f_router"]
    touched = sum(a["touched"] for a in acct) / len(acct)
    res = dict(name=name, T=shape.T, ms_per_step=ms, value=shape.T / (ms / 1e3), steps=steps, warmup=warmup,
               wall_s=wall, step_us=stats, layers_per_graph=sets if run_all is not None else 1,
               touched_experts=touched, bytes_per_step=b_step,
               bytes_experts=sum(a["b_experts"] for a in acct) / len(acct), flops_ffn=f_ffn, flops_step=f_all,
               hbm_frac_step=b_step / (ms / 1e3) / (HBM_PEAK_GBS * 1e9),
               mfma_frac_step=f_all / (ms / 1e3) / (BF16_PEAK_TFLOPS * 1e12),
               mfma_frac_experts=f_ffn / (ms / 1e3) / (BF16_PEAK_TFLOPS * 1e12))
    if parts:
        res["separate_calls_us"] = separate_calls(torch, moe, synth, shape, layers, per_set, lw, use_graph)
    res["_layers"] = layers
    res["_per_set"] = per_set
    return res


def separate_calls(torch, moe, synth, shape, layers, per_set, lw, use_graph):
    """The layer as separate calls (route + group, ffn, combine, steered
    combine), each captured alone over the rotating sets: us per step."""
    dev = layers[0].x.device
    y = lw.y

    def calls_route_group():
        for L in layers:
            moe.route_group(L.x, L.wr, shape.K, bias=L.bias, workspace=lw.group_ws, out=lw.route_out + lw.perm_out)

    def calls_ffn():
        for L, p in zip(layers, per_set):
            moe.ffn(L.x, L.wg, L.wu, L.wd, p["offsets"], p["perm"], shape.K, L.sg, L.su, L.sd, out=y,
                    workspace=lw.ffn_ws)

    def calls_combine():
        for p in per_set:
            moe.combine(y, p["inv"], p["w"], out=lw.out)

    v = torch.from_numpy(synth.steer_vector(shape.H)).to(dev)

    def calls_combine_steer():
        for p in per_set:
            moe.combine(y, p["inv"], p["w"], out=lw.out, steer_v=v)

    timer = Timer(torch)
    out = {}
    for pname, f in (("route_group", calls_route_group), ("ffn", calls_ffn), ("combine", calls_combine),
                     ("combine_steer", calls_combine_steer)):
        gf = capture(torch, f).replay if use_graph else f
        timer.run(gf, 2)
        t, _ = timer.run(gf, 8)
        out[pname] = round(t / (8 * len(layers)) * 1e6, 2)
    return out


def layer_roofline(res, kernel, key):
    """HBM roofline of the whole layer call (the step): compulsory bytes per
    call over the call's average duration in the timed region."""
    a = res["bytes_per_step"] / (res["ms_per_step"] / 1e3) / 1e9
    return dict(bound="hbm", achieved=round(a, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(a / HBM_PEAK_GBS, 4),
                traffic=measured_traffic(key), kernel=kernel, algorithmic_bytes_per_launch=int(res["bytes_per_step"]),
                launch_us=round(res["ms_per_step"] * 1e3, 2))


def ffn_mfma_roofline(res):
    """MFMA roofline of the expert call (moe_ffn, the grouped GEMMs) of the
    prefill chunk, timed alone: expert flops over its average duration."""
    t = res["separate_calls_us"]["ffn"] / 1e6
    a = res["flops_ffn"] / t / 1e12
    return dict(bound="mfma", achieved=round(a, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(a / BF16_PEAK_TFLOPS, 4), traffic=measured_traffic("ffn_prefill"),
                kernel="moe_ffn (plan + gate/up + down launches)", algorithmic_flops_per_launch=res["flops_ffn"],
                launch_us=res["separate_calls_us"]["ffn"])


# ------------------------------------------------------------------ pruning statistic
def bench_freq(torch, moe, synth, steps, warmup, use_graph, cpu):
    L, T, E, K, keep = synth.FREQ_L, synth.FREQ_T, synth.FREQ_E, synth.FREQ_K, synth.FREQ_KEEP
    log(f"[freq] generating {L} x {T} x {E} fp32 logits")
    lg = torch.empty((L, T, E), dtype=torch.float32, device="cuda")
    for l in range(L):
        synth.make_device_logits_layer(T, E, seed=0, cfg=4, layer=l, device="cuda", out=lg[l])
    counts = torch.zeros((L, E), dtype=torch.int64, device="cuda")
    rank_of = torch.empty((L, E), dtype=torch.int32, device="cuda")
    keep_map = torch.empty((L, keep), dtype=torch.int32, device="cuda")
    lib = moe.load()

    def step():
        rc = lib.moe_expert_freq(moe._ptr(lg), L, T, E, K, moe._ptr(counts), 0, keep, moe._ptr(rank_of),
                                 moe._ptr(keep_map), moe._stream())
        assert rc == 0
    timer = Timer(torch)
    fn = capture(torch, step).replay if use_graph else step
    timer.run(fn, max(1, warmup))
    n = max(3, steps)
    dt, wall = timer.run(fn, n)
    ms = dt / n * 1e3
    nbytes = L * T * E * 4 + L * E * 8 * 2
    a = nbytes / (ms / 1e3) / 1e9
    res = dict(name="pruning statistic 48x262144x512 fp32 logits, top-10, keep 256", ms_per_step=ms,
               value=L * T / (ms / 1e3), unit="logit rows/s", steps=n, warmup=max(1, warmup), wall_s=wall,
               roofline=dict(bound="hbm", achieved=round(a, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=round(a / HBM_PEAK_GBS, 4), kernel="moe_expert_freq (one call, 48 layers)",
                             algorithmic_bytes_per_launch=nbytes, launch_us=round(ms * 1e3, 1),
                             traffic=measured_traffic("freq")))
    if cpu:
        res["cpu_baseline"] = cpu_baseline_freq(lg)
    prof = bench_profile(torch, moe, lg, K)
    del lg
    return res, prof


def bench_profile(torch, moe, lg, K, slots=2537, n_eval=8192):
    """The expert profile on the statistic's logits: counts of the first half of
    the calibration tokens, their global (layer, expert) ranking, and the share
    of the routed reads of held-out tokens (the second half) that the first
    `slots` ranked pairs serve, next to the share a profile unrelated to the
    routing would serve (slots / pairs).  The held-out trace is the library's
    own routing of those rows: moe_route with the logits as activations and the
    identity as router (every logit reproduced exactly, then selected by the
    routing rule)."""
    L, T, E = lg.shape
    half = T // 2
    counts = torch.zeros((L, E), dtype=torch.int64, device="cuda")
    for l in range(L):
        moe.expert_freq(lg[l, :half], K, counts=counts[l:l + 1])
    eye = torch.eye(E, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.route_workspace_size(n_eval, E, E, K, moe.F32), dtype=torch.uint8, device="cuda")
    trace = torch.empty((L, n_eval, K), dtype=torch.int32, device="cuda")
    w = torch.empty((n_eval, K), dtype=torch.float32, device="cuda")
    for l in range(L):
        moe.route(lg[l, half:half + n_eval], eye, K, workspace=ws, out=(trace[l], w))
    pws = torch.empty(moe.load().moe_profile_workspace_size(L, E), dtype=torch.uint8, device="cuda")
    rank, pairs = moe.profile_rank(counts, workspace=pws)
    hits = moe.profile_hits(trace, rank, slots)
    torch.cuda.synchronize()
    timer = Timer(torch)
    reps = 20
    dt_r, _ = timer.run(lambda: moe.profile_rank(counts, workspace=pws), reps)
    dt_h, _ = timer.run(lambda: moe.profile_hits(trace, rank, slots), reps)
    rate = int(hits.item()) / trace.numel()
    log(f"[profile] rank {dt_r / reps * 1e6:.1f} us, hits {dt_h / reps * 1e6:.1f} us, hit rate of the first {slots} "
        f"pairs {rate:.3f} (unrelated profile: {slots / (L * E):.3f})")
    return dict(name=f"expert profile: global rank of {L} x {E} pairs, hit rate of the first {slots} on "
                     f"{L} x {n_eval} held-out tokens x top-{K} (trace from moe_route)",
                rank_us=round(dt_r / reps * 1e6, 2), hits_us=round(dt_h / reps * 1e6, 2),
                hit_rate=round(rate, 4), unrelated_profile_rate=round(slots / (L * E), 4))


# ------------------------------------------------------------------ measured ceilings
def bench_copy(torch, steps):
    """A plain 1 GiB device-to-device copy: the reference reading of the HBM
    byte counters (1 GiB fetched and 1 GiB written per launch)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    timer = Timer(torch)
    timer.run(lambda: b.copy_(a), 2)
    reps = max(3, steps // 20)
    dt, wall = timer.run(lambda: b.copy_(a), reps)
    ms = dt / reps * 1e3
    del a, b
    return dict(name="device copy 1 GiB (counter calibration)", ms_per_step=ms, steps=reps, wall_s=wall,
                value=round(2 * n / (ms / 1e3) / 1e9, 1), unit="GB/s (read + write)", bytes_read=n, bytes_written=n)


def bench_peaks(torch):
    """Ceilings measured on this GPU with library code, next to the published
    peaks: a 1 GiB copy (read + write), a 4 GiB read (a sum), and an 8192^3
    bf16 GEMM (torch.matmul, hipBLASLt)."""
    timer = Timer(torch)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    timer.run(lambda: b.copy_(a), 3)
    dt, _ = timer.run(lambda: b.copy_(a), 10)
    copy_gbs = 2 * n / (dt / 10) / 1e9
    del a, b
    r = torch.ones(1 << 31, dtype=torch.bfloat16, device="cuda")       # 4 GiB
    timer.run(lambda: r.sum(dtype=torch.float32), 2)
    dt, _ = timer.run(lambda: r.sum(dtype=torch.float32), 5)
    read_gbs = r.numel() * 2 / (dt / 5) / 1e9
    del r
    m = 8192
    A = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    B = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((m, m), dtype=torch.bfloat16, device="cuda")
    timer.run(lambda: torch.matmul(A, B, out=C), 3)
    dt, _ = timer.run(lambda: torch.matmul(A, B, out=C), 10)
    gemm_tf = 2.0 * m ** 3 / (dt / 10) / 1e12
    del A, B, C
    torch.cuda.empty_cache()
    res = dict(name="measured ceilings (library code on this GPU) vs published peaks",
               hbm_copy_gbs=round(copy_gbs, 1), hbm_read_gbs=round(read_gbs, 1), hbm_peak_gbs=HBM_PEAK_GBS,
               bf16_gemm_8192_tflops=round(gemm_tf, 1), bf16_peak_tflops=BF16_PEAK_TFLOPS)
    log(f"[peaks] copy {copy_gbs:.0f} GB/s, read {read_gbs:.0f} GB/s, bf16 GEMM 8192^3 {gemm_tf:.0f} TFLOP/s")
    return res


# ------------------------------------------------------------------ pruned 48-layer stack
def bench_stack(torch, moe, synth, shape, steps, warmup, use_graph, name, steered=41, cpu=False):
    """The 48-layer stack, each layer's output added to the stream in place;
    timed plain and with the first `steered` layers steered (the pages steer
    41 layers without naming them)."""
    Ls = synth.STACK_INT4_LAYERS
    log(f"[{name}] generating {Ls} {shape.wdt} layers")
    layers = [synth.make_device_layer(shape, seed=0, cfg=5, layer=l, device="cuda") for l in range(Ls)]
    vs = [torch.from_numpy(synth.steer_vector(shape.H, layer=l)).cuda() if l < steered else None for l in range(Ls)]
    x0 = layers[0].x
    torch.cuda.synchronize()
    wdt = {"int4": moe.INT4_B32, "int3": moe.INT3_B32, "int2": moe.INT2_B32}[shape.wdt]
    lw = moe.LayerWorkspace(shape.T, shape.H, shape.E, shape.K, shape.F, x_dtype=torch.bfloat16, w_dtype=wdt)
    h = torch.empty_like(x0)

    def run(steer):
        def step():
            h.copy_(x0)
            for L, v in zip(layers, vs):
                moe.layer(h, L.wr, L.wg, L.wu, L.wd, shape.K, sg=L.sg, su=L.su, sd=L.sd, residual=h, lw=lw, out=h,
                          steer_v=v if steer else None)
        timer = Timer(torch)
        fn = capture(torch, step).replay if use_graph else step
        timer.run(fn, max(1, warmup))
        n = max(2, steps)
        dt, wall = timer.run(fn, n)
        return dt / n * 1e3, n, wall

    ms, n, wall = run(False)
    res = dict(name=name, T=shape.T, layers=Ls, ms_per_step=ms, ms_per_layer=ms / Ls,
               value=shape.T * Ls / (ms / 1e3), unit="tokens/s per MoE layer (48-layer stack)", steps=n,
               warmup=max(1, warmup), wall_s=wall)
    if steered:
        ms_s, _, _ = run(True)
        res.update(steered_layers=steered, ms_per_step_steered=ms_s, steer_cost_frac=ms_s / ms - 1.0)
    if cpu:
        res["cpu_baseline"] = cpu_baseline_stack(torch, layers, shape)
    del layers
    return res


# ------------------------------------------------------------------ CPU baselines (the oracle, one core)
def _bits(torch, t):
    import numpy as np
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _host_weights(torch, d):
    import oracle
    h = lambda t: None if t is None else _bits(torch, t)  # noqa: E731
    return oracle.Weights(d.shape.wdt, h(d.wg), h(d.wu), h(d.wd), h(d.sg), h(d.su), h(d.sd))


def cpu_baseline_verify(torch, synth, layer, budget_s=10.0):
    import oracle
    s = layer.shape
    x, wr = _bits(torch, layer.x), layer.wr.cpu().numpy()
    W = _host_weights(torch, layer)
    reps, t0 = 0, time.perf_counter()
    while True:
        idx, w, _ = oracle.route(x, wr, s.K)
        oracle.permute(idx, s.E)
        oracle.layer_rows(x, idx, w, W)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    return dict(value=round(s.T * reps / el, 3), unit="tokens/s", cores=1, kind="oracle",
                sample=f"the full 5-token verify step (route, permute, 10 experts per token, combine) of weight set 0, "
                       f"repeated {reps} times ({el:.1f} s, single-threaded C, fp64)", **host_info())


def cpu_baseline_prefill(torch, layer, n_rows=12):
    """Routing of all 8192 tokens, the experts and combine of a seeded sample of
    rows; the layer time is extrapolated linearly in the rows (rows are
    independent)."""
    import numpy as np

    import oracle
    s = layer.shape
    x, wr, bias = _bits(torch, layer.x), layer.wr.cpu().numpy(), layer.bias.cpu().numpy()
    W = _host_weights(torch, layer)
    t0 = time.perf_counter()
    idx, w, _ = oracle.route(x, wr, s.K, bias)
    oracle.permute(idx, s.E)
    t_route = time.perf_counter() - t0
    rows = np.random.default_rng(0).choice(s.T, n_rows, replace=False)
    t0 = time.perf_counter()
    oracle.layer_rows(x, idx, w, W, rows=rows)
    t_rows = time.perf_counter() - t0
    t_layer = t_route + t_rows / n_rows * s.T
    return dict(value=round(s.T / t_layer, 4), unit="tokens/s (extrapolated)", cores=1, kind="oracle",
                sample=f"routing and grouping of all {s.T} tokens ({t_route:.1f} s) and the experts + combine of "
                       f"{n_rows} seeded rows ({t_rows:.1f} s), extrapolated to {s.T} rows: {t_layer:.0f} s per "
                       f"layer (single-threaded C, fp64)", **host_info())


def cpu_baseline_freq(lg, rows=65536):
    """The statistic's counting over a sample of one layer's rows."""
    import oracle
    sample = lg[0, :rows].cpu().numpy()[None]
    t0 = time.perf_counter()
    oracle.expert_freq(sample, 10)
    el = time.perf_counter() - t0
    return dict(value=round(rows / el, 1), unit="logit rows/s", cores=1, kind="oracle",
                sample=f"top-10 counting of {rows} rows of layer 0 ({el:.1f} s, single-threaded C)", **host_info())


def cpu_baseline_stack(torch, layers, shape, n_layers=2, n_rows=6):
    """Per-layer oracle time of the stack: routing of all T tokens and the
    experts + combine of the rows (all of them at T = 5, a seeded sample at
    T = 8192, extrapolated), over the first layers."""
    import numpy as np

    import oracle
    x = _bits(torch, layers[0].x)
    rows = np.arange(shape.T) if shape.T <= 8 else np.random.default_rng(0).choice(shape.T, n_rows, replace=False)
    t_total = 0.0
    for L in layers[:n_layers]:
        wr = L.wr.cpu().numpy()
        W = _host_weights(torch, L)
        t0 = time.perf_counter()
        idx, w, _ = oracle.route(x, wr, shape.K)
        oracle.permute(idx, shape.E)
        t_route = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.layer_rows(x, idx, w, W, rows=rows, residual=x)
        t_rows = time.perf_counter() - t0
        t_total += t_route + t_rows / len(rows) * shape.T
    t_layer = t_total / n_layers
    extra = "" if shape.T <= 8 else f", {n_rows} seeded rows per layer extrapolated to {shape.T}"
    return dict(value=round(shape.T / t_layer, 4), unit="tokens/s per MoE layer" + (" (extrapolated)" if extra else ""),
                cores=1, kind="oracle",
                sample=f"{n_layers} layers of the stack on the stack's input rows: routing of all {shape.T} tokens, "
                       f"experts + combine + residual{extra}; {t_layer:.1f} s per layer (single-threaded C, fp64)",
                **host_info())


def strip(r):
    return {k: v for k, v in r.items() if not k.startswith("_")}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workloads", default="verify,prefill,freq,stack,lowbit,peaks")
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of HIP graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the MoE layer is not sharded across GPUs here "
              "(its token rows would shard with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    cpu = not args.no_cpu_baseline

    import torch
    from routed_expert_ffn_amd import moe, synth
    moe.load()
    use_graph = not args.no_graph
    wl = [w.strip() for w in args.workloads.split(",") if w.strip()]
    also = []
    main_res = None
    if "verify" in wl:
        r = bench_layer(torch, moe, synth, synth.VERIFY_BF16, 2, steps, warmup, N_SETS, use_graph,
                        "verify step 5 tok, E512 top-10 bf16", stat_runs=max(200, steps))
        r["roofline"] = layer_roofline(r, "moe_layer (exact logits, routing + grouping + gate/up, down + combine "
                                          "launches)", "verify_step")
        if cpu:
            r["cpu_baseline"] = cpu_baseline_verify(torch, synth, r["_layers"][0])
        r["is_verify_layer"] = True
        log(f"[verify] {r['ms_per_step']*1e3:.1f} us/step, median {r['step_us']['median_us']} us, "
            f"separate calls {r['separate_calls_us']}")
        main_res = strip(r)
        del r
        torch.cuda.empty_cache()
    if "prefill" in wl:
        r = bench_layer(torch, moe, synth, synth.PREFILL_BF16, 3, max(8, steps // 10), 4, 1, use_graph,
                        "prefill chunk 8192 tok, E512 top-10 bf16, Zipf(1.1) router offset", stat_runs=20)
        r["roofline"] = ffn_mfma_roofline(r)
        r["unit"] = "tokens/s"
        r["steps_rule"] = ("--steps / 10 (at least 8) timed steps after 4 warmup steps: a step is ~1 ms, and only the "
                           "headline workload takes --steps and --warmup as given")
        if cpu:
            r["cpu_baseline"] = cpu_baseline_prefill(torch, r["_layers"][0])
        log(f"[prefill] {r['ms_per_step']:.3f} ms/step, separate calls {r['separate_calls_us']}")
        also.append(strip(r))
        del r
        torch.cuda.empty_cache()
    if "freq" in wl:
        r, prof = bench_freq(torch, moe, synth, max(5, steps // 20), 2, use_graph, cpu)
        r["steps_rule"] = "--steps / 20 (at least 5) calls after 2 warmup calls: a call reads 25.8 GB (~4 ms)"
        log(f"[freq] {r['ms_per_step']:.3f} ms/step")
        also.append(r)
        also.append(prof)
        torch.cuda.empty_cache()
    if "copy" in wl:
        r = bench_copy(torch, steps)
        log(f"[copy] {r['ms_per_step']:.3f} ms per 1 GiB copy, {r['value']} GB/s")
        also.append(r)
        torch.cuda.empty_cache()
    if "peaks" in wl:
        also.append(bench_peaks(torch))
    if "stack" in wl:
        for shp, nm in ((synth.STACK_INT4_VERIFY, "pruned 48-layer int4 stack, 5-tok verify"),
                        (synth.STACK_INT4_PREFILL, "pruned 48-layer int4 stack, 8192-tok prefill")):
            r = bench_stack(torch, moe, synth, shp, max(3, steps // 40), 1, use_graph, nm, cpu=cpu)
            r["steps_rule"] = "--steps / 40 (at least 3) steps after 1 warmup step: a step is 48 layers (2-42 ms)"
            log(f"[stack T={shp.T}] {r['ms_per_step']:.3f} ms/step, {r['ms_per_step_steered']:.3f} ms steered")
            also.append(r)
            torch.cuda.empty_cache()
    if "lowbit" in wl:
        # the verify step of the pruned layer with int4, int3 and int2 experts: one
        # layer over 8 rotating weight sets, and the 48-layer stack
        for shp in (synth.STACK_INT4_VERIFY, synth.STACK_INT3_VERIFY, synth.STACK_INT2_VERIFY):
            r = bench_layer(torch, moe, synth, shp, 5, steps, warmup, N_SETS, use_graph,
                            f"verify step 5 tok, E256 top-10, {shp.wdt} experts", stat_runs=max(200, steps))
            r["unit"] = "tokens/s"
            r["roofline"] = layer_roofline(r, "moe_layer", None)
            log(f"[{shp.wdt} verify] {r['ms_per_step']*1e3:.1f} us/step, median {r['step_us']['median_us']} us, "
                f"{r['roofline']['achieved']:.0f} GB/s, separate calls {r['separate_calls_us']}")
            also.append(strip(r))
            del r
            torch.cuda.empty_cache()
            if shp.wdt != "int4":
                r = bench_stack(torch, moe, synth, shp, max(3, steps // 40), 1, use_graph,
                                f"pruned 48-layer {shp.wdt} stack, 5-tok verify", steered=0)
                log(f"[{shp.wdt} stack T={shp.T}] {r['ms_per_step']:.3f} ms/step")
                also.append(r)
                torch.cuda.empty_cache()

    if main_res is None:          # a partial run (e.g. under a profiler): report the first workload
        main_res = also.pop(0) if also else None
        if main_res is None:
            sys.exit("no workload ran")
    is_verify = main_res.get("is_verify_layer", False)
    line = {
        "metric": METRIC,
        "value": round(main_res["value"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": main_res.get("warmup", warmup),
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": main_res["name"], "tokens": main_res.get("T"), "hidden": 2048, "experts": 512,
                   "top_k": 10, "expert_width": 512, "weight_sets_rotated": N_SETS if is_verify else 1,
                   "hip_graph": use_graph, "layer_calls_per_graph": main_res.get("layers_per_graph", 1)},
        "roofline": main_res.get("roofline"),
        "cpu_baseline": main_res.get("cpu_baseline"),
        "step_us": main_res.get("step_us"),
        "separate_calls_us": main_res.get("separate_calls_us"),
        "step_hbm_frac": round(main_res.get("hbm_frac_step", 0.0), 4),
        "touched_experts": main_res.get("touched_experts"),
        "host": host_info(),
        "also": also,
    }
    print(json.dumps(line, default=lambda o: round(o, 4) if isinstance(o, float) else str(o)))


if __name__ == "__main__":
    main()
