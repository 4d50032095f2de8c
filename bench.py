#!/usr/bin/env python3
"""SSD forward throughput on one MI355X, with the dominant kernel's roofline position
and the fp64 oracle timed on the host cores beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mamba2_2p7b]

One step is one ssd_fwd call: one pass of the whole forward (chunk_cumsum -> chunk_state
-> state_passing -> chunk_scan) over one batch of synthetic inputs already resident in
HBM.  The step time comes from the host clock between two device synchronisations around
the K timed steps.  Right after them, K more steps run as the four stage calls with HIP
events between stages on the launch stream, which gives every kernel's average duration.
Before the warmup, a distribution pass times whole ssd_fwd calls one by one (warm, and
cold after flushing the Infinity Cache).  Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/sec on 1 MI355X; MFMA util % and HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="mamba2_2p7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache step times (so that a kernel trace of the run "
                         "holds warm launches only)")
    ap.add_argument("--stat-steps", type=int, default=0,
                    help="ssd_fwd calls in each per-step distribution pass (warm, cold) run "
                         "before the warmup; default max(steps, 200)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="rough budget for the oracle CPU baseline")
    ap.add_argument("--decode", default="", metavar="WORKLOAD",
                    help="instead of the forward, time ssd_decode_step on a decode workload "
                         "(one token per sequence per step) and print its own JSON line")
    ap.add_argument("--block", default="", metavar="BLOCK",
                    help="time the block between the projections (ssd_block_fwd: prologue, "
                         "ssd_fwd, epilogue) on a model-shaped block (block_2p7b, block_130m)")
    ap.add_argument("--varlen", action="store_true",
                    help="time ssd_fwd_varlen on the 2.7B layer's 16384 tokens packed as one row "
                         "of seeded sequence lengths (64 to 4096 steps)")
    ap.add_argument("--bwd", default="", metavar="WORKLOAD",
                    help="instead of the forward, time the backward (ssd_bwd) on a workload and "
                         "print its own JSON line")
    ap.add_argument("--peaks", action="store_true",
                    help="measure practical peaks on this GPU: a 1 GiB device copy (HBM GB/s) "
                         "and a bf16 8192^3 GEMM through torch (MFMA TFLOP/s)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to calibrate the "
                         "HBM byte counters against a known traffic, and exit")
    return ap.parse_args()


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(w, inputs, budget_s):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload:
    whole batch elements when at least one fits the time budget (all of them when the
    whole workload fits), else the first heads (whole groups) of batch element 0.  Every
    sampled (batch, head) sequence runs over the full T.  Tokens/s is scaled to the
    metric's unit: one (batch, head) sequence is 1/H of each of its T tokens."""
    import oracle

    nthreads = host_threads()
    hpg = w.nheads // w.ngroups

    def sample(nb, nh):
        g = (nh + hpg - 1) // hpg
        pick = lambda t, hs: None if t is None else t[:nb, :, :hs].double().numpy()
        init = inputs["init_state"]
        return dict(x=pick(inputs["x"], nh), dt=pick(inputs["dt"], nh),
                    A=inputs["A"][:nh].double().numpy(), B=pick(inputs["B"], g),
                    C=pick(inputs["C"], g), D=inputs["D"][:nh].double().numpy(),
                    init_state=None if init is None else init[:nb, :nh].double().numpy())

    def timed(nb, nh):
        s = sample(nb, nh)
        t0 = time.perf_counter()
        oracle.ssd_ref(**s, nthreads=nthreads)
        return time.perf_counter() - t0

    probe = timed(1, w.nheads)          # one whole batch element
    if probe * 2 <= budget_s:
        nb, nh = max(1, min(w.batch, int(budget_s / max(probe, 1e-3)))), w.nheads
    else:
        nb = 1
        nh = max(hpg, int(w.nheads * budget_s / probe) // hpg * hpg)
        nh = min(nh, w.nheads)
    el = timed(nb, nh)
    # a sample far below the budget (the whole workload, when it is quick) is repeated
    # until the budget is spent, for a steadier time
    reps = max(1, min(50, int(budget_s / max(el, 1e-3))))
    if reps > 1:
        el = sum(timed(nb, nh) for _ in range(reps)) / reps
    used = oracle.threads_used(nb, nh, nthreads)
    tokens = w.seqlen * nb * nh / w.nheads
    # one thread, on the first group's heads of batch element 0 (a few seconds at most)
    nh1 = min(w.nheads, hpg)
    s1 = sample(1, nh1)
    t0 = time.perf_counter()
    oracle.ssd_ref(**s1, nthreads=1)
    el1 = time.perf_counter() - t0
    return {"value": round(tokens / el, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"batch elements 0..{nb - 1} of {w.batch}, heads 0..{nh - 1} of "
                      f"{w.nheads}, full T={w.seqlen} ({nb * nh} fp64 token-recurrence "
                      f"sequences, {el:.2f} s each, mean of {reps} runs)",
            "single_thread_value": round(w.seqlen * nh1 / w.nheads / el1, 1),
            "single_thread_sample": f"batch element 0, heads 0..{nh1 - 1}, {el1:.2f} s",
            "host": host_info()}


def host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "threads_allowed": host_threads()}


def step_stats(torch, fn, steps, flush=None):
    """Per-step GPU times (HIP events on the current stream) of `steps` calls of fn, in us:
    median, p10, p90.  With `flush`, an untimed flush runs before each timed call."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    q = lambda f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]
    return {"median": round(q(0.5), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2)}


def bench_decode(args, w, torch, binding, roofline, generate):
    """Decode steps back to back on one batch of sequences: tokens/s = batch / step time.
    The step is bound by HBM: it reads and writes the fp32 state once."""
    dev = torch.device("cuda:0")
    log(f"[bench decode] {w.describe()}")
    cpu = generate(w)
    x, dt = cpu["x"][:, 0].to(dev), cpu["dt"][:, 0].contiguous().to(dev)
    Bm, Cm = cpu["B"][:, 0].contiguous().to(dev), cpu["C"][:, 0].contiguous().to(dev)
    A, D = cpu["A"].to(dev), cpu["D"].to(dev)
    state = cpu["init_state"].to(dev)
    y = torch.empty_like(x)
    step = lambda: binding.ssd_decode_step(x, dt, A, Bm, Cm, D, state, y=y)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    c = roofline.decode_cost(w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype)
    gbs = c.bytes / (us * 1e-6) / 1e9
    ms_step = elapsed / args.steps * 1e3
    print(json.dumps({
        "metric": "SSD decode-step tokens/sec on 1 MI355X", "value": round(w.batch / (ms_step * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "ngroups": w.ngroups, "input_dtype": w.dtype},
        "roofline": {"bound": "hbm", "kernel": "decode_step", "achieved": round(gbs, 1),
                     "peak": roofline.PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbs / roofline.PEAK_HBM_GBPS, 4), "traffic": None},
        "kernels": {"decode_step": {"avg_us": round(us, 2), "alg_bytes": int(c.bytes)}},
    }), flush=True)


def bench_bwd(args, w, torch, binding, roofline, generate, generate_grads):
    """Whole ssd_bwd calls back to back (the forward intermediates it recomputes
    included): tokens/s = B*T / call time.  The call's kernels are listed with their
    algorithmic bytes and FLOPs; their durations come from a kernel trace."""
    dev = torch.device("cuda:0")
    log(f"[bench bwd] {w.describe()}")
    cpu = generate(w)
    up = generate_grads(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in cpu.items()}
    u = {k: (None if v is None else v.to(dev)) for k, v in up.items()}
    dims = binding.SsdDims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups)
    ws = torch.empty(binding.ssd_bwd_workspace_size(dims, w.chunk_len), dtype=torch.uint8,
                     device=dev)
    out = dict(dx=torch.empty_like(d["x"]), ddt=torch.empty_like(d["dt"]),
               dA=torch.empty_like(d["A"]), dB=torch.empty_like(d["B"]),
               dC=torch.empty_like(d["C"]), dD=torch.empty_like(d["D"]),
               d_init=torch.empty((w.batch, w.nheads, w.dstate, w.headdim), device=dev))
    step = lambda: binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len,
                                   u["dy"], init_state=d["init_state"], d_final=u["d_final"],
                                   out=out, workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # the same gradients from the forward's own intermediates (ssd_bwd_saved), as a
    # training step that has just run ssd_fwd would take them
    fws = torch.empty(binding.ssd_fwd_workspace_size(dims, w.chunk_len), dtype=torch.uint8,
                      device=dev)
    binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len,
                    init_state=d["init_state"], workspace=fws)
    saved = step_stats(torch, lambda: binding.ssd_bwd(
        d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len, u["dy"],
        init_state=d["init_state"], d_final=u["d_final"], out=out, workspace=ws,
        fwd_workspace=fws), args.steps)
    costs = roofline.bwd_costs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                               w.chunk_len, w.dtype, init_state=w.init_state)
    tot_bytes = sum(c.bytes for c in costs)
    tot_flops = sum(c.flops for c in costs)
    gbs = tot_bytes / (us * 1e-6) / 1e9
    ms_step = elapsed / args.steps * 1e3
    print(json.dumps({
        "metric": "SSD bwd tokens/sec on 1 MI355X", "value": round(w.tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                   "ngroups": w.ngroups, "chunk_len": w.chunk_len, "input_dtype": w.dtype,
                   "init_state": w.init_state},
        "roofline": {"bound": "hbm", "kernel": "ssd_bwd (all kernels)", "achieved": round(gbs, 1),
                     "peak": roofline.PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbs / roofline.PEAK_HBM_GBPS, 4), "traffic": None},
        "call_us": round(us, 2),
        "saved_call_us": saved,
        "kernels": {c.name: {"alg_bytes": int(c.bytes), "alg_flops": int(c.flops)} for c in costs},
        "alg_bytes_total": int(tot_bytes), "alg_flops_total": int(tot_flops),
    }), flush=True)

def bench_block(args, w, cfg, torch, binding, roofline, generate_block):
    """Whole ssd_block_fwd calls back to back: tokens/s = B*T / call time.  A staged pass
    makes the same three calls (prologue, ssd_fwd, epilogue) with HIP events between them
    for the block kernels' durations; the roofline is the slower block kernel's (the SSD
    layer's own kernels have theirs in the default run)."""
    dev = torch.device("cuda:0")
    log(f"[bench block] {w.describe()} {cfg}")
    cpu = generate_block(w, cfg)
    d = {k: (None if v is None else v.to(dev)) for k, v in cpu.items()}
    dims = binding.SsdDims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups)
    code = binding.SSD_BF16 if w.dtype == "bf16" else binding.SSD_F32
    ws = torch.empty(binding.ssd_block_fwd_workspace_size(dims, code, w.chunk_len),
                     dtype=torch.uint8, device=dev)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    hp, gn = H * P, G * N
    out = torch.empty((w.batch, w.seqlen, hp), dtype=d["zxbcdt"].dtype, device=dev)
    fin = torch.empty((w.batch, H, N, P), dtype=torch.float32, device=dev)

    def step():
        binding.ssd_block_fwd(d["zxbcdt"], d["conv_w"], d["conv_b"], d["dt_bias"], d["A"],
                              d["D"], w.chunk_len, d["norm_w"], d["norm_b"], cfg.norm_groups,
                              P, N, G, rms=cfg.rms, eps=cfg.eps, init_state=d["init_state"],
                              out=out, final_state=fin, workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref = out.clone()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    config = {"workload": args.block, "batch": w.batch, "seqlen": w.seqlen, "nheads": H,
              "headdim": P, "dstate": N, "ngroups": G, "chunk_len": w.chunk_len,
              "conv_k": cfg.conv_k, "norm_groups": cfg.norm_groups, "rms": cfg.rms,
              "input_dtype": w.dtype}
    head = {
        "metric": "Mamba-2 block (between the projections) tokens/sec on 1 MI355X",
        "value": round(w.tokens / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic", "config": config,
    }
    if binding.ssd_block_fwd_norm_in_scan(dims, code, w.chunk_len, cfg.norm_groups):
        # the gate and the norm run inside the chunk scan: there is no epilogue launch to
        # time apart, so the per-kernel durations come from a kernel trace
        print(json.dumps({**head, "norm_in_scan": True, "roofline": None,
                          "kernels": {"note": "gate and norm inside the chunk scan; per-kernel "
                                              "durations from rocprofv3 --kernel-trace"}}),
              flush=True)
        return
    # staged: the same three calls with events between them
    zx = d["zxbcdt"]
    x = torch.empty((w.batch, w.seqlen, H, P), dtype=zx.dtype, device=dev)
    Bm = torch.empty((w.batch, w.seqlen, G, N), dtype=zx.dtype, device=dev)
    Cm = torch.empty_like(Bm)
    dt = torch.empty((w.batch, w.seqlen, H), dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    fws = torch.empty(binding.ssd_fwd_workspace_size(dims, w.chunk_len), dtype=torch.uint8,
                      device=dev)
    out2 = torch.empty_like(out)
    names = ["block_prologue", "ssd_fwd", "block_epilogue"]
    per = {n: 0.0 for n in names}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for ev in evs:  # back to back, one synchronisation at the end
        ev[0].record()
        binding.ssd_block_prologue(zx[:, :, hp:2 * hp + 2 * gn], d["conv_w"], d["conv_b"],
                                   zx[:, :, 2 * hp + 2 * gn:], d["dt_bias"], H, P, N, G,
                                   x=x, B=Bm, C=Cm, dt=dt)
        ev[1].record()
        binding.ssd_fwd(x, dt, d["A"], Bm, Cm, d["D"], w.chunk_len, init_state=d["init_state"],
                        y=y, final_state=fin, workspace=fws)
        ev[2].record()
        binding.ssd_block_epilogue(y, zx[:, :, :hp], d["norm_w"], d["norm_b"], cfg.norm_groups,
                                   rms=cfg.rms, eps=cfg.eps, dstate=N, ngroups=G, out=out2)
        ev[3].record()
    torch.cuda.synchronize()
    for ev in evs:
        for i, n in enumerate(names):
            per[n] += ev[i].elapsed_time(ev[i + 1]) / args.steps
    if not torch.equal(out2, ref):
        log("[bench block] WARNING: staged calls and ssd_block_fwd differ")
    costs = {c.name: c for c in roofline.block_costs(w.batch, w.seqlen, H, P, N, G, cfg.conv_k,
                                                     w.dtype, norm_bias=not cfg.rms)}
    kernels = {}
    for n in names:
        kernels[n] = {"avg_us": round(per[n] * 1e3, 2)}
        if n in costs:
            t = per[n] * 1e-3
            gbs = costs[n].bytes / t / 1e9
            kernels[n].update(alg_bytes=int(costs[n].bytes), alg_flops=int(costs[n].flops),
                              hbm_GBps=round(gbs, 1),
                              hbm_frac=round(gbs / roofline.PEAK_HBM_GBPS, 4))
    dom = max(costs, key=lambda n: per[n])
    print(json.dumps({
        **head, "norm_in_scan": False,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["hbm_GBps"],
                     "peak": roofline.PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": kernels[dom]["hbm_frac"], "traffic": None},
        "kernels": kernels,
    }), flush=True)


def bench_varlen(args, torch, binding, generate, Workload):
    """ssd_fwd_varlen calls back to back on one packed row: tokens/s = T / call time, next
    to ssd_fwd on the same tokens as one unbroken sequence."""
    import numpy as np
    dev = torch.device("cuda:0")
    T = 16384
    rng = np.random.default_rng(11)
    cuts = [0]
    while cuts[-1] < T:
        cuts.append(min(T, cuts[-1] + int(rng.integers(64, 4097))))
    w = Workload("packed_2p7b", 1, T, 80, 64, 128, 1, 256)
    log(f"[bench varlen] {w.describe()} {len(cuts) - 1} sequences")
    d = {k: (None if v is None else v.to(dev)) for k, v in generate(w).items()}
    cu = torch.tensor(cuts, dtype=torch.int32, device=dev)
    dims = binding.SsdDims(1, T, w.nheads, w.headdim, w.dstate, w.ngroups)
    ws = torch.empty(binding.ssd_fwd_varlen_workspace_size(dims, 256), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(d["x"])
    fins = torch.empty((len(cuts) - 1, w.nheads, w.dstate, w.headdim), device=dev)
    # the sequence starts are checked once here; the timed calls skip that host copy
    binding.ssd_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256, cu, y=y,
                           final_states=fins, workspace=ws)
    step = lambda: binding.ssd_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256,
                                          cu, y=y, final_states=fins, workspace=ws,
                                          check_cu_seqlens=False)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    fws = torch.empty(binding.ssd_fwd_workspace_size(dims, 256), dtype=torch.uint8, device=dev)
    one = step_stats(torch, lambda: binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"],
                                                    d["D"], 256, y=y, workspace=fws),
                     args.steps)
    print(json.dumps({
        "metric": "SSD fwd (packed variable-length row) tokens/sec on 1 MI355X",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seqlen": T, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "chunk_len": 256, "sequences": len(cuts) - 1,
                   "final_states": True},
        "ssd_fwd_same_tokens_us": one}), flush=True)


def measure_peaks(torch):
    """Practical peaks next to the spec ones: HBM bandwidth from a 1 GiB device-to-device
    copy (read + write bytes over time), MFMA throughput from a bf16 GEMM (hipBLASLt)."""
    from mamba_ssd_chunked_03_amd import roofline
    dev = torch.device("cuda:0")
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy = step_stats(torch, lambda: dst.copy_(src), 20)
    m = 8192
    a = torch.randn((m, m), device=dev).to(torch.bfloat16)
    b = torch.randn((m, m), device=dev).to(torch.bfloat16)
    for _ in range(3):
        a @ b
    gemm = step_stats(torch, lambda: a @ b, 20)
    print(json.dumps({
        "hbm_copy_GBps": round(2 * 4 * n / (copy["median"] * 1e-6) / 1e9, 1),
        "hbm_spec_GBps": roofline.PEAK_HBM_GBPS,
        "bf16_gemm_TFLOPs": round(2 * m ** 3 / (gemm["median"] * 1e-6) / 1e12, 1),
        "bf16_spec_TFLOPs": roofline.PEAK_MFMA_TFLOPS["bf16"],
        "copy_us": copy, "gemm_us": gemm}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: libssd has no multi-GPU path (several GPUs would "
              "each run the same kernels on their own batch elements, heads or groups). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.peaks:
        return measure_peaks(torch)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_MiB": args.copy_calibration,
                          "read_bytes_per_copy": 4 * n, "write_bytes_per_copy": 4 * n}))
        return
    from mamba_ssd_chunked_03_amd import binding, roofline, traffic
    from mamba_ssd_chunked_03_amd.workloads import (BLOCKS, DECODE, WORKLOADS, Workload,
                                                    generate, generate_block, generate_grads)
    if args.varlen:
        return bench_varlen(args, torch, binding, generate, Workload)
    if args.block:
        w, cfg = BLOCKS[args.block]
        return bench_block(args, w, cfg, torch, binding, roofline, generate_block)
    if args.decode:
        return bench_decode(args, DECODE[args.decode], torch, binding, roofline, generate)
    if args.bwd:
        return bench_bwd(args, WORKLOADS[args.bwd], torch, binding, roofline, generate,
                         generate_grads)

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] {w.describe()}: generating inputs")
    cpu_inputs = generate(w)
    d_in = {k: (None if v is None else v.to(dev)) for k, v in cpu_inputs.items()}
    dims = binding.SsdDims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups)
    Q = w.chunk_len
    ws = torch.empty(binding.ssd_fwd_workspace_size(dims, Q), dtype=torch.uint8, device=dev)
    y = torch.empty_like(d_in["x"])
    fin = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device=dev)

    gram_n = binding.ssd_chunk_gram_size(dims, d_in["x"].dtype, Q)

    def fwd():
        binding.ssd_fwd(d_in["x"], d_in["dt"], d_in["A"], d_in["B"], d_in["C"], d_in["D"], Q,
                        init_state=d_in["init_state"], y=y, final_state=fin, workspace=ws)

    # the four stage calls ssd_fwd makes, on its workspace, marshalled once; run with a HIP
    # event between stages (on torch's current stream, the launch stream) they give every
    # kernel's duration
    calls = binding.fwd_stage_calls(d_in["x"], d_in["dt"], d_in["A"], d_in["B"], d_in["C"],
                                    d_in["D"], Q, d_in["init_state"], y, fin, ws)
    names = [n for n, _ in calls]

    def step(ev=None):
        for i, (_, call) in enumerate(calls):
            if ev is not None:
                ev[i].record()
            call()
        if ev is not None:
            ev[len(calls)].record()

    # Per-step time distribution of whole ssd_fwd calls (HIP events per call): cold (the
    # 256 MB Infinity Cache flushed by an untimed 1 GiB write before each call), then warm
    # (back to back).  It runs first, so the GPU has been busy for a while when the timed
    # steps begin.
    nstat = args.stat_steps if args.stat_steps > 0 else max(args.steps, 200)
    log(f"[bench] per-step times: {nstat} cold, {nstat} warm ssd_fwd calls")
    fwd()
    torch.cuda.synchronize()
    y_ref, fin_ref = y.clone(), fin.clone()
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    # cold first: the warm calls then run right before the warm-up and timed steps, so those
    # start from the steady back-to-back state rather than from the flushes' aftermath
    step_us = {"steps": nstat}
    if not args.no_cold:
        step_us["cold"] = step_stats(torch, fwd, nstat, flush=lambda: scratch.fill_(1.0))
    step_us["warm"] = step_stats(torch, fwd, nstat)
    del scratch

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    # the timed steps: whole ssd_fwd calls, back to back
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Right after, the same number of steps as the four stage calls with a HIP event between
    # stages: every kernel's average duration.  (An event between two kernels keeps the next
    # from starting while the last workgroups of the previous drain, so the staged steps run
    # a little longer than the ssd_fwd steps above; the durations are each kernel's own.)
    ev_steps = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
                for _ in range(args.steps)]
    for k in range(args.steps):
        step(ev_steps[k])
    torch.cuda.synchronize()
    if not (torch.equal(y, y_ref) and torch.equal(fin, fin_ref)):
        log("[bench] WARNING: the stage calls and ssd_fwd differ")
    if not torch.isfinite(y.float()).all():
        log("[bench] WARNING: non-finite output")

    per = {n: 0.0 for n in names}
    for ev in ev_steps:
        for i, n in enumerate(names):
            per[n] += ev[i].elapsed_time(ev[i + 1]) / args.steps   # ms
    costs = {c.name: c for c in roofline.kernel_costs(
        w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, Q, w.dtype,
        init_state=w.init_state, final_state=True, gram_bytes=gram_n)}
    kernels = {}
    for n in names:
        t = per[n] * 1e-3
        c = costs[n]
        gbs = c.bytes / t / 1e9
        tfl = c.flops / t / 1e12
        kernels[n] = {"avg_us": round(per[n] * 1e3, 2), "alg_bytes": int(c.bytes),
                      "alg_flops": int(c.flops), "hbm_GBps": round(gbs, 1),
                      "hbm_frac": round(gbs / roofline.PEAK_HBM_GBPS, 4),
                      "mfma_TFLOPs": round(tfl, 2),
                      "mfma_frac": round(tfl / roofline.PEAK_MFMA_TFLOPS["bf16"], 4)}
    # measured HBM bytes per launch, where recorded for the kernels as they are now built
    rec = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                       f"hbm_traffic_{w.name}.md")
    sqrec = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                         "sq_counters_2p7b.md")
    for n in names:
        kernels[n]["hbm_traffic_bytes"] = traffic.current_traffic(rec, n)
        if w.name == "mamba2_2p7b":  # the counter record is of this workload
            busy = traffic.current_mfma_busy(sqrec, n)
            if busy is not None:
                kernels[n]["mfma_busy_counter"] = busy
    dom = max(names, key=lambda n: per[n])
    dk = kernels[dom]
    roof = {"bound": "hbm", "kernel": dom, "achieved": dk["hbm_GBps"],
            "peak": roofline.PEAK_HBM_GBPS, "unit": "GB/s", "frac": dk["hbm_frac"],
            "traffic": dk["hbm_traffic_bytes"]}

    ms_step = elapsed / args.steps * 1e3
    tokens_per_s = w.tokens * args.steps / elapsed
    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                   "ngroups": w.ngroups, "chunk_len": Q, "input_dtype": w.dtype,
                   "init_state": w.init_state, "parallelism": "single_gpu"},
        "roofline": roof,
        "kernels": kernels,
        "step_us": step_us,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        result["cpu_baseline"] = cpu_baseline(w, cpu_inputs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
