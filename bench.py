"""Benchmark: one REINFORCE Zero learner step (logprobs + IS loss + gradients)
per step on the Qwen3-4B tool-use shape, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--mode learner|sample|diag|mx|ceiling] [--lora-rank R]

A step is one rz_reinforce_zero_fwd_bwd call over the whole synthetic batch
(inputs already resident in HBM).  Prints ONE JSON line with the throughput
in valid tokens/s, the fraction of bf16 MFMA peak on the algorithmic
6 H V FLOP per valid token, the roofline of the dominant kernel (its
launches timed live with HIP events on the call's stream), and the float64
oracle timed on a bounded sample on the host cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s fused logprob+IS-loss fwd/bwd (Qwen3-4B shape); % MFMA peak"
METRIC_LORA = ("tokens/s fused logprob+IS-loss fwd/bwd, rank-{r} LoRA on a frozen "
               "head (Qwen3-4B shape); % MFMA peak")
LORA_SCALE = 0.5
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA
HBM_GBS = 8000.0
GEMM_KERNELS = ("fwd_logits_gemm", "bwd_dh_gemm", "bwd_dw_gemm")

# Bytes per launch past L2 from two rocprofv3 counter runs of this script
# (FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0, the factors a plain 1 GiB copy
# reads on the same counters; FETCH_SIZE counts every L2 miss, including
# those the memory-side cache serves), averaged over the launches of one
# step: the learner GEMMs at the Qwen3-4B tool-use shape (profiles/
# gemm_traffic_qwen3_4b_tool.md), the gradient-norm kernel of --mode diag
# (profiles/run_diagnostics_qwen3_4b_step.md) and the MXFP4 expansion of
# --mode mx (profiles/mx_dequant_qwen3_4b_head.md).  Valid only for the
# kernel sources they were taken from.
COUNTER_TRAFFIC = {
    "workload": "qwen3_4b_tool",
    "sources_sha256": "50de99dde003ec4db27f97eb7aab2075a95d7f1944e6ddd4dfb3375af9d5861b",
    # per timed launch: a GEMM with its last-round K pieces and their sum
    "bytes_per_launch": {"fwd_logits_gemm": 26095798992,
                         "bwd_dh_gemm": 24031489230,
                         "bwd_dw_gemm": 27943645919,
                         "grad_norm": 2291958011,
                         "mx_dequant_mxfp4": 984643114},
}


# Matrix-core busy share (SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' cycles)
# and clock (GRBM_GUI_ACTIVE per XCD over the launch time) of the learner
# GEMMs, from the counter run of profiles/mfma_utilisation_qwen3_4b_tool.md,
# over the launches that hold rows; same validity rule as COUNTER_TRAFFIC.
COUNTER_MFMA = {
    "fwd_logits_gemm": {"mfma_busy": 0.605, "clock_ghz": 1.819},
    "bwd_dh_gemm": {"mfma_busy": 0.674, "clock_ghz": 1.717},
    "bwd_dw_gemm": {"mfma_busy": 0.636, "clock_ghz": 1.762},
}


def counter_mfma(key, workload="qwen3_4b_tool"):
    """Counter busy share and clock of `key`, or None once the kernels changed."""
    if (workload != COUNTER_TRAFFIC["workload"]
            or kernel_sources_sha256() != COUNTER_TRAFFIC["sources_sha256"]):
        return None
    return COUNTER_MFMA.get(key)


def counter_traffic(key, workload="qwen3_4b_tool"):
    """Counter bytes per launch of `key`, or None once the kernels changed."""
    if (workload != COUNTER_TRAFFIC["workload"]
            or kernel_sources_sha256() != COUNTER_TRAFFIC["sources_sha256"]):
        return None
    return COUNTER_TRAFFIC["bytes_per_launch"].get(key)


def kernel_sources_sha256():
    """Fingerprint of the HIP sources; counter figures taken from an older
    build of the kernels no longer describe them."""
    import hashlib
    d = os.path.join(ROOT, "invariant_token_logprobs_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def behaviour_logprobs(torch, hidden, head, tokens, rows=2048):
    """Stand-in rollout policy (plain torch fp32 on the GPU) that places
    log mu near log pi; it is input preparation, never timed or compared."""
    Wf = head.float().t().contiguous()
    out = torch.empty(hidden.shape[0], dtype=torch.float32, device=hidden.device)
    for r0 in range(0, hidden.shape[0], rows):
        r1 = min(hidden.shape[0], r0 + rows)
        lp = torch.log_softmax(hidden[r0:r1].float() @ Wf, dim=1)
        out[r0:r1] = lp.gather(1, tokens[r0:r1].long()[:, None])[:, 0]
    del Wf
    return out


def cpu_baseline(b, logmu, max_valid, lora=None):
    """The float64 oracle, as it stands, on the first responses of the same
    workload up to `max_valid` valid rows at the full H and V (with a LoRA
    adapter (A, B, scale) on the head when `lora` is given)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    valid = np.flatnonzero(b.mask != 0)
    n_keep = int(valid[max_valid - 1]) + 1 if len(valid) > max_valid else b.N
    cu = b.cu_rows.astype(np.int64)
    nb = int(np.searchsorted(cu, n_keep, side="left"))
    cu_s = cu[: nb + 1].copy()
    cu_s[nb] = n_keep
    hidden = O.to_f64(b.hidden[:n_keep], b.dtype)
    head = O.to_f64(b.lm_head, b.dtype)
    t0 = time.perf_counter()
    if lora is None:
        out = O.reinforce_zero_fwd_bwd(hidden, head, b.tokens[:n_keep],
                                       logmu[:n_keep].astype(np.float64),
                                       b.mask[:n_keep], cu_s, b.rewards[:nb],
                                       b.group_ids[:nb])
    else:
        A, B, sc = lora
        out = O.reinforce_zero_fwd_bwd_lora(
            hidden, head, O.to_f64(A, b.dtype), O.to_f64(B, b.dtype), sc,
            b.tokens[:n_keep], logmu[:n_keep].astype(np.float64),
            b.mask[:n_keep], cu_s, b.rewards[:nb], b.group_ids[:nb], b.dtype)
    dt = time.perf_counter() - t0
    nv = int(np.count_nonzero(b.mask[:n_keep]))
    assert np.isfinite(out["loss"])
    res = {"value": nv / dt, "unit": "tokens/s", "cores": blas_threads or cores,
           "kind": "oracle",
           "sample": (f"first {nb} responses, {nv} valid of {n_keep} rows of "
                      f"{b.name} at full H={b.H}, V={b.V}; float64 NumPy "
                      f"fwd+loss+bwd, {dt:.1f} s on {cores} host cores "
                      f"(BLAS threads {blas_threads})")}
    if lora is None:
        res["tiny"] = tiny_cpu_baseline()
    return res


def tiny_cpu_baseline():
    """The float64 oracle on the whole Tiny workload (8 responses, fp32,
    H=256, V=1024): valid tokens per second of one fwd+loss+bwd pass."""
    import oracle as O
    from invariant_token_logprobs_amd import synth
    t = synth.make_workload("tiny")
    h64, W64 = O.to_f64(t.hidden, t.dtype), O.to_f64(t.lm_head, t.dtype)
    logpi, _ = O.token_logprobs(h64, W64, t.tokens)
    logmu = synth.make_logmu(logpi, t.sigma, t.noise_seed).astype(np.float64)
    t0 = time.perf_counter()
    out = O.reinforce_zero_fwd_bwd(h64, W64, t.tokens, logmu, t.mask, t.cu_rows,
                                   t.rewards, t.group_ids)
    dt = time.perf_counter() - t0
    assert np.isfinite(out["loss"])
    return {"value": round(t.n_valid / dt, 1), "unit": "tokens/s",
            "sample": f"tiny: all {t.n_valid} valid rows, H={t.H}, V={t.V}, {dt * 1e3:.1f} ms"}


def copy_calibration(torch, dev):
    """One plain 1 GiB device copy, so a counter run can scale its byte
    counters by what they read for a known transfer."""
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    log("copy calibration: 1 GiB read + 1 GiB written by one copy kernel")
    del x, y


def timed_pass(torch, rz, call, steps):
    """The kernels' own HIP-event times over `steps` more calls, with the
    library's kernel timer on.  The timer records an event pair around
    every launch, which costs about 5 us per launch on the stream; the
    sub-millisecond modes therefore time their calls with it off and take
    the per-kernel split from this second pass of the same calls."""
    torch.cuda.synchronize()
    rz.timing_enable(True)
    rz.timing_read(reset=True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    kt = rz.timing_read(reset=True)
    rz.timing_enable(False)
    return kt


def bench_sample(args, torch, rz, synth, dev):
    """The rollout-side draw at decode size: rz_sample_tokens on
    --sample-rows live rows at the Qwen3-4B head (H 2560, V 151936, bf16)."""
    H, V, M = 2560, 151936, args.sample_rows
    hid, _ = synth.random_rows(M, H, V, "bf16", 3001)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x.view(np.int16))).view(
        torch.bfloat16).to(dev)
    hidden = up(hid)
    ids = torch.arange(M, dtype=torch.int64, device=dev)
    ws = rz.Workspace()
    seed = 0x5EED
    fmt = args.head
    if fmt == "bf16":
        head = synth.random_lm_head(V, H, "bf16", 3002)
        W = up(head)
        w_bytes = 2.0 * V * H
        draw = lambda: rz.sample_tokens(hidden, W, ids, seed, workspace=ws)
    else:
        codes_np, scales_np = synth.random_mx_head(V, H, fmt, 3002)
        codes = torch.from_numpy(codes_np).to(dev)
        scales = torch.from_numpy(scales_np).to(dev)
        w_bytes = float(codes_np.nbytes + scales_np.nbytes)
        draw = lambda: rz.sample_tokens_mx(hidden, codes, scales, fmt, ids, seed,
                                           workspace=ws)
    for _ in range(args.warmup):
        draw()
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for _ in range(args.steps):
        tok, logmu = draw()
    torch.cuda.synchronize()
    te = time.perf_counter()
    ms = (te - ts) * 1e3 / args.steps
    kt = timed_pass(torch, rz, draw, args.steps)
    assert bool(torch.isfinite(logmu).all()), "non-finite record"
    fast = fast_baseline(torch, hidden, W if fmt == "bf16" else
                         rz.dequantize_head(codes, scales, fmt), args) \
        if args.fast_baseline else None
    gemm_ms, launches = kt["fwd_sample_gemm"]
    avg = gemm_ms / launches
    flop = 2.0 * M * H * V
    achieved = flop / (avg * 1e-3) / 1e12
    kms = {k: v[0] / args.steps for k, v in kt.items() if v[1]}
    log("per-call kernel ms: " + ", ".join(f"{k}={v:.3f}" for k, v in
                                           sorted(kms.items(), key=lambda x: -x[1])))
    # 2 M H V flops against 2 V H bytes of W: M flops per W byte; below the
    # chip's balance point (2.5 PFLOP/s over 8 TB/s) W's read bounds the GEMM
    if M < PEAK_TFLOPS["bf16"] * 1e12 / (HBM_GBS * 1e9):
        w_gbs = w_bytes / (avg * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "fwd_sample_gemm",
                    "achieved": round(w_gbs, 1), "peak": HBM_GBS, "unit": "GB/s",
                    "frac": round(w_gbs / HBM_GBS, 4), "traffic": None,
                    "avg_launch_ms": round(avg, 4),
                    "mfma_TFLOPs": round(achieved, 2)}
    else:
        roofline = {"bound": "mfma", "kernel": "fwd_sample_gemm",
                    "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                    "traffic": None, "avg_launch_ms": round(avg, 4),
                    "w_read_TBps": round(w_bytes / (avg * 1e-3) / 1e12, 3)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        n_cpu = 16
        t0 = time.perf_counter()
        W64 = (O.to_f64(head, "bf16") if fmt == "bf16"
               else O.dequantize_head(codes_np, scales_np, fmt))
        O.sample_tokens(O.to_f64(hid[:n_cpu], "bf16"), W64, np.arange(n_cpu), seed,
                        row_chunk=n_cpu)
        dt = time.perf_counter() - t0
        cpu = {"value": n_cpu / dt, "unit": "tokens/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"first {n_cpu} rows at full H={H}, V={V}; float64 NumPy "
                         f"logits + Philox noise + draw + record, {dt:.1f} s "
                         "(includes decoding W to float64)"}
    line = {
        "metric": ("sampled tokens/s (rollout draw + recorded logprob, Qwen3-4B head"
                   + (")" if fmt == "bf16" else f", {fmt} weights)")),
        "value": round(M * args.steps / (te - ts), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rollout_draw_qwen3_4b_head" + ("" if fmt == "bf16" else f"_{fmt}"),
                   "hidden": H, "vocab": V, "rows": M, "head": fmt},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fast_baseline": (None if fast is None else
                          dict(fast, aligned_over_fast=round(ms / fast["ms_per_call"], 3))),
        "kernel_ms_per_step": {k: round(v, 4) for k, v in kms.items()},
    }
    print(json.dumps(line), flush=True)


def fast_baseline(torch, hidden, W, args):
    """The unaligned draw the pages compare against: the vendor GEMM
    (torch.mm on bf16, hipBLASLt), an fp32 log-softmax and a Gumbel-max draw
    with torch's own generator -- fast, but neither batch-invariant nor
    reproducible against the learner.  Timed per call like the aligned path
    (W^T is made contiguous once, outside the timed region)."""
    WT = W.t().contiguous()
    gen = torch.Generator(device=hidden.device)
    gen.manual_seed(7)

    def call():
        z = torch.mm(hidden, WT).float()
        lp = torch.log_softmax(z, dim=-1)
        u = torch.rand(z.shape, generator=gen, device=z.device)
        tok = torch.argmax(z - torch.log(-torch.log(u)), dim=-1)
        return tok, lp.gather(1, tok[:, None])[:, 0]

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del WT
    return {"ms_per_call": round(ms, 4),
            "what": "torch.mm (hipBLASLt, bf16) + fp32 log_softmax + Gumbel-max "
                    "draw with torch.rand; not batch-invariant"}


def fast_learner_step(torch, hidden, head, tokens, logmu, mask, cu_rows, rewards,
                      group_ids, chunk=16384):
    """The learner step the unaligned way, for comparison: per chunk of
    valid rows, torch.mm (hipBLASLt, bf16) for the logits, the dHidden and the
    dW products, fp32 logits and log-softmax, the same unclipped IS loss's
    dL/dz, and dW accumulated in fp32.  Not batch-invariant; W^T is made
    contiguous once per step."""
    dev = hidden.device
    valid = torch.nonzero(mask, as_tuple=True)[0]
    B = rewards.shape[0]
    lengths = (cu_rows[1:] - cu_rows[:-1]).long()
    resp = torch.repeat_interleave(torch.arange(B, device=dev), lengths)
    T = torch.zeros(B, device=dev).index_add_(0, resp, mask.float())
    G = int(group_ids.max().item()) + 1
    gsum = torch.zeros(G, device=dev).index_add_(0, group_ids.long(), rewards)
    gcnt = torch.zeros(G, device=dev).index_add_(0, group_ids.long(), torch.ones_like(rewards))
    A = rewards - (gsum / gcnt)[group_ids.long()]
    fac = (A / (B * T.clamp(min=1)))[resp]                   # A_i / (B T_i) per row
    WT = head.t().contiguous()
    dW = torch.zeros(head.shape, dtype=torch.float32, device=dev)
    d_hidden = torch.zeros(hidden.shape, dtype=torch.float32, device=dev)
    loss = torch.zeros((), device=dev)
    for c0 in range(0, valid.numel(), chunk):
        rows = valid[c0:c0 + chunk]
        h = hidden[rows]
        z = torch.mm(h, WT).float()
        lp = torch.log_softmax(z, dim=-1)
        tok = tokens[rows].long()
        lpt = lp.gather(1, tok[:, None])[:, 0]
        w = torch.exp(lpt - logmu[rows])
        coef = fac[rows] * w                                   # dL/dlog pi = -coef
        loss = loss - (coef).sum()
        g = torch.exp(lp) * coef[:, None]                      # coef (softmax - onehot)
        g[torch.arange(rows.numel(), device=dev), tok] -= coef
        gb = g.to(hidden.dtype)
        d_hidden[rows] = torch.mm(gb, head).float()
        dW += torch.mm(gb.t().contiguous(), h).float()
        del z, lp, g, gb
    return loss, d_hidden, dW


def bench_diag(args, torch, rz, synth, dev):
    """Run-level diagnostics over one learner step's outputs at the step's
    shape: rz_grad_norms over dL/dhidden [N, H] and dL/dW [V, H] (fp32),
    rz_response_diagnostics and rz_diagnostics over the N rows, and the
    tracker's per-step record.  Inputs are seeded synthetic values of those
    shapes (the step's own outputs are not needed to time a reduction)."""
    wl = synth.WORKLOADS[args.workload]
    _, lengths, mask_np, _, _ = synth.workload_layout(args.workload)
    H, V = wl.H, wl.V
    N, B = int(lengths.sum()), len(lengths)
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    g = torch.Generator(device=dev)
    g.manual_seed(4001)
    dh = torch.randn((N, H), generator=g, device=dev) * 1e-4
    dw = torch.randn((V, H), generator=g, device=dev) * 1e-6
    rng = np.random.default_rng(4002)
    lp_np = -rng.exponential(2.0, size=N).astype(np.float32)
    lm_np = (lp_np + rng.normal(0.0, wl.sigma, size=N)).astype(np.float32)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    logpi, logmu, mask, cu = up(lp_np), up(lm_np), up(mask_np), up(cu_np)
    ws = rz.Workspace()
    norms = torch.empty(2, dtype=torch.float32, device=dev)
    diag = torch.empty(2, dtype=torch.float32, device=dev)
    tracker = rz.RunTracker(dev, capacity=args.steps + args.warmup + 1)

    def step():
        rz.grad_norms(dh, dw, workspace=ws, out=norms)
        d3, kl = rz.response_diagnostics(logpi, logmu, mask, cu)
        rz.diagnostics(logpi, logmu, mask, workspace=ws, out=diag)
        tracker.record(diag, norms[1:])
        return d3, kl

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for _ in range(args.steps):
        d3, kl = step()
    torch.cuda.synchronize()
    te = time.perf_counter()
    summary = tracker.summary()
    kt = timed_pass(torch, rz, step, args.steps)
    assert np.isfinite(summary["grad_norm_max"]), "non-finite norm"
    if args.copy_calibration:
        copy_calibration(torch, dev)
    ms = (te - ts) * 1e3 / args.steps
    tot_ms, launches = kt["grad_norm"]
    grad_bytes = 4.0 * (N * H + V * H)          # each gradient read once
    per_launch = grad_bytes * args.steps / launches
    achieved = per_launch / (tot_ms / launches * 1e-3) / 1e9
    kms = {k: v[0] / args.steps for k, v in kt.items() if v[1]}
    log("per-pass kernel ms: " + ", ".join(f"{k}={v:.4f}" for k, v in
                                           sorted(kms.items(), key=lambda x: -x[1])))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        h_dh = dh.cpu().numpy()
        h_dw = dw.cpu().numpy()
        t0 = time.perf_counter()
        O.grad_norms(h_dh, h_dw)
        O.response_diagnostics(lp_np, lm_np, mask_np, cu_np)
        O.diagnostics(lp_np, lm_np, mask_np)
        dt = time.perf_counter() - t0
        cpu = {"value": round(1.0 / dt, 4), "unit": "passes/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"one whole pass (N={N}, B={B}, H={H}, V={V}): float64 "
                         f"NumPy norms + per-response and step D3/KL, {dt:.2f} s "
                         "(host copies excluded)"}
    line = {
        "metric": "run-level diagnostic passes/s (gradient norms + per-response "
                  "and step D3/KL + tracker record, Qwen3-4B step shape)",
        "value": round(args.steps / (te - ts), 2), "unit": "passes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"run_diagnostics_{args.workload}", "hidden": H,
                   "vocab": V, "rows": N, "responses": B},
        "roofline": {"bound": "hbm", "kernel": "grad_norm",
                     "achieved": round(achieved, 1), "peak": HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_GBS, 4),
                     "traffic": counter_traffic("grad_norm", args.workload),
                     "avg_launch_ms": round(tot_ms / launches, 4),
                     "launches_per_step": launches // args.steps},
        "cpu_baseline": cpu,
        "kernel_ms_per_step": {k: round(v, 4) for k, v in kms.items()},
    }
    print(json.dumps(line), flush=True)


def bench_ceiling(args, torch, rz, dev):
    """The matrix cores' own ceiling on this part (rz_calibrate_mfma): the
    learner GEMMs' MFMA, four waves per CU with a wave's 128 x 128 block of
    accumulators (the four-wave form of the tile), no global traffic; operands from registers or from LDS
    (the GEMM's read volume), random-looking or zero values.  Each variant
    runs args.warmup untimed launches and args.steps timed ones of about
    30 ms, back to back on one stream."""
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(ncu * 256, dtype=torch.float32, device=dev)
    iters = 16384
    stream = torch.cuda.current_stream()
    res = {}
    for lds in (0, 1):
        for data in (1, 0):
            key = f"{'lds' if lds else 'registers'}_{'random' if data else 'zero'}"
            for _ in range(args.warmup):
                rz.calibrate_mfma(data, lds, ncu, iters, sink)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            flop = 0.0
            for _ in range(args.steps):
                flop += rz.calibrate_mfma(data, lds, ncu, iters, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            tf = flop / (ms * 1e-3) / 1e12
            res[key] = {"TFLOP/s": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4),
                        "ms_per_launch": round(ms / args.steps, 3)}
            log(f"{key}: {tf:.1f} TFLOP/s = {tf / PEAK_TFLOPS['bf16']:.3f} of peak "
                f"({ms / args.steps:.2f} ms per launch)")
    line = {"metric": "bf16 MFMA ceiling (no global traffic), TFLOP/s",
            "mode": "ceiling", "unit": "TFLOP/s", "peak": PEAK_TFLOPS["bf16"],
            "workgroups": ncu, "iters": iters, "steps": args.steps,
            "warmup": args.warmup, "variants": res}
    print(json.dumps(line), flush=True)


def bench_mx(args, torch, rz, synth, dev):
    """The release-precision head: rz_dequantize_head expanding the Qwen3-4B
    head (V 151936, H 2560) from --mx-format storage to bf16."""
    H, V, fmt = 2560, 151936, args.mx_format
    t0 = time.time()
    codes_np, scales_np = synth.random_mx_head(V, H, fmt, 5001)
    log(f"{fmt} head drawn ({time.time() - t0:.1f}s)")
    codes = torch.from_numpy(codes_np).to(dev)
    scales = torch.from_numpy(scales_np).to(dev)
    W = torch.empty((V, H), dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    run = lambda: rz.dequantize_head(codes, scales, fmt, err_flag=err, out=W)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    te = time.perf_counter()
    kt = timed_pass(torch, rz, run, args.steps)
    assert int(err.cpu()[0]) == 0, "invalid block scales in the synthetic head"
    tot_ms, launches = kt["mx_dequant"]
    avg = tot_ms / launches
    nbytes = codes_np.nbytes + scales_np.nbytes + 2.0 * V * H
    achieved = nbytes / (avg * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(torch, dev)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        rows = 16384
        t0 = time.perf_counter()
        O.dequantize_head(codes_np[:rows], scales_np[:rows], fmt)
        dt = time.perf_counter() - t0
        cpu = {"value": round(rows / V / dt, 4), "unit": "heads/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"first {rows} of {V} rows at H={H}; float64 NumPy "
                         f"decode, {dt:.2f} s, scaled to the whole head"}
    line = {
        "metric": f"MX head expansions/s ({fmt} -> bf16, Qwen3-4B head)",
        "value": round(args.steps / (te - ts), 2), "unit": "heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((te - ts) * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"mx_dequant_{fmt}_qwen3_4b_head", "hidden": H,
                   "vocab": V, "format": fmt},
        "roofline": {"bound": "hbm", "kernel": "mx_dequant",
                     "achieved": round(achieved, 1), "peak": HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_GBS, 4),
                     "traffic": counter_traffic(f"mx_dequant_{fmt}"), "avg_launch_ms": round(avg, 4),
                     "bytes_per_launch": int(nbytes)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_4b_tool")
    ap.add_argument("--cpu-valid", type=int, default=3072,
                    help="valid rows in the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("learner", "sample", "diag", "mx", "ceiling"),
                    default="learner",
                    help="learner: the fused fwd/bwd step (the headline); "
                         "sample: the rollout-side draw + record at decode size; "
                         "diag: the run-level diagnostics over a step's outputs; "
                         "mx: expanding an MX-format head to bf16")
    ap.add_argument("--fast-baseline", action="store_true",
                    help="also time the unaligned vendor path: the draw "
                         "(--mode sample) or the learner step (torch.mm, fp32 "
                         "log_softmax)")
    ap.add_argument("--head", choices=("bf16", "mxfp4", "mxfp8"), default="bf16",
                    help="--mode sample: the head's storage (MX heads run "
                         "rz_sample_tokens_mx)")
    ap.add_argument("--lora-rank", type=int, default=0,
                    help="learner mode: a LoRA adapter of this rank (1..64) "
                         "on the frozen head (rz_reinforce_zero_fwd_bwd_lora)")
    ap.add_argument("--mx-format", choices=("mxfp4", "mxfp8"), default="mxfp4",
                    help="element format of the head in --mode mx")
    ap.add_argument("--sample-rows", type=int, default=1024,
                    help="live rows of the rollout batch in --mode sample")
    ap.add_argument("--operand-data", choices=("random", "zero"), default="random",
                    help="learner mode: 'zero' runs the same step with all-zero "
                         "hidden states and head (same kernels, launches and "
                         "addresses; only the values the matrix cores see differ), "
                         "to show what the data costs in power; not a headline figure")
    ap.add_argument("--tokens", choices=("uniform", "zipf"), default="uniform",
                    help="learner mode: the sampled tokens' law (zipf: Zipf(1.1) "
                         "over the vocabulary, the most frequent token on ~8%% "
                         "of the rows)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device "
                         "copy so a counter run can scale its byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_token_logprobs_amd as rz
    from invariant_token_logprobs_amd import synth

    dev = torch.device("cuda:0")
    if args.mode == "sample":
        return bench_sample(args, torch, rz, synth, dev)
    if args.mode == "diag":
        return bench_diag(args, torch, rz, synth, dev)
    if args.mode == "mx":
        return bench_mx(args, torch, rz, synth, dev)
    if args.mode == "ceiling":
        return bench_ceiling(args, torch, rz, dev)
    t0 = time.time()
    b = synth.make_workload(args.workload, tokens=args.tokens)
    log(f"workload {b.name}: N={b.N} B={b.B} valid={b.n_valid} H={b.H} V={b.V} "
        f"({time.time() - t0:.1f}s to draw)")

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if bf16 else x))
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)

    isbf = b.dtype == "bf16"
    hidden, head = up(b.hidden, isbf), up(b.lm_head, isbf)
    zero_ops = args.operand_data == "zero"
    if zero_ops:
        hidden.zero_()
        head.zero_()
    tokens = up(b.tokens)
    r = args.lora_rank
    lora = None
    if r:
        A_np, B_np = synth.random_lora(r, b.H, b.V, b.dtype, 6001)
        lora = (A_np, B_np, LORA_SCALE)
        A_d, B_d = up(A_np, isbf), up(B_np, isbf)
        # stand-in behaviour policy on the merged head W + s B A (torch fp32)
        w_eff = head.float() + LORA_SCALE * (B_d.float() @ A_d.float())
        mu_ref = behaviour_logprobs(torch, hidden, w_eff, tokens)
        del w_eff
    else:
        mu_ref = behaviour_logprobs(torch, hidden, head, tokens)
    logmu = synth.make_logmu(mu_ref.cpu().numpy(), b.sigma, b.noise_seed)
    del mu_ref
    torch.cuda.empty_cache()
    args_dev = [hidden, head, tokens, up(logmu), up(b.mask), up(b.cu_rows),
                up(b.rewards), up(b.group_ids)]
    ws = rz.Workspace()
    outs = {}
    if r:
        def step():
            outs.update(rz.reinforce_zero_fwd_bwd_lora(
                hidden, head, A_d, B_d, LORA_SCALE, *args_dev[2:], workspace=ws))
    else:
        step = lambda: rz.reinforce_zero_fwd_bwd(*args_dev, workspace=ws, outputs=outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    rz.timing_enable(True)
    rz.timing_read(reset=True)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ts = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    te = time.perf_counter()
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    kt = rz.timing_read(reset=True)
    rz.timing_enable(False)
    loss = float(outs["loss"].cpu()[0])
    assert np.isfinite(loss), "non-finite loss"

    ms = (te - ts) * 1e3 / args.steps
    nv = b.n_valid
    value = nv * args.steps / (te - ts)
    # algorithmic FLOP per valid token: forward, dHidden and dW GEMMs 2HV
    # each; with an adapter of rank r the first two are 2(H + r)V, the head's
    # gradient is dB (2rV) and u, dL/dA and the chain rule to h add 6Hr
    flop_tok = (6.0 * b.H * b.V if not r else
                4.0 * (b.H + r) * b.V + 2.0 * r * b.V + 6.0 * b.H * r)
    flop_alg = flop_tok * nv
    peak = PEAK_TFLOPS[b.dtype]
    mfma_frac = flop_alg / (ms * 1e-3) / (peak * 1e12)

    # dominant kernel and its roofline (per-launch average, live HIP events)
    kms = {k: v[0] / args.steps for k, v in kt.items() if v[1]}
    dom = max(GEMM_KERNELS, key=lambda k: kt[k][0])
    tot_ms, launches = kt[dom]
    avg_ms = tot_ms / launches
    gemm_k = b.H if not r else (b.H + r if dom != "bwd_dw_gemm" else r)
    flop_per_launch = 2.0 * gemm_k * b.V * nv * args.steps / launches
    achieved = flop_per_launch / (avg_ms * 1e-3) / 1e12
    traffic = counter_traffic(dom, b.name) if not r else None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic,
                "traffic_unit": "bytes per launch past L2 (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "avg_launch_ms": round(avg_ms, 4),
                "launches_per_step": launches // args.steps,
                "counters": counter_mfma(dom, b.name) if not r else None}
    log("per-step kernel ms: " + ", ".join(f"{k}={v:.2f}" for k, v in
                                            sorted(kms.items(), key=lambda x: -x[1])))

    if args.copy_calibration:
        copy_calibration(torch, dev)

    fast = None
    if args.fast_baseline and not r:
        log("timing the unaligned vendor-GEMM learner step ...")
        fargs = [hidden, head, tokens] + args_dev[3:]
        floss = float(fast_learner_step(torch, *fargs)[0].item())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fast_learner_step(torch, *fargs)
        torch.cuda.synchronize()
        fms = (time.perf_counter() - t0) * 1e3 / args.steps
        torch.cuda.empty_cache()
        fast = {"ms_per_step": round(fms, 2), "aligned_over_fast": round(ms / fms, 3),
                "loss": floss,
                "what": "per 16384 valid rows: torch.mm (hipBLASLt, bf16) logits, dHidden "
                        "and dW, fp32 log_softmax and dL/dz, dW accumulated in fp32; not "
                        "batch-invariant"}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample ...")
        cpu = cpu_baseline(b, logmu, args.cpu_valid, lora)

    line = {
        "metric": METRIC if not r else METRIC_LORA.format(r=r),
        "value": round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": b.dtype,
        "data": ("synthetic" if not zero_ops else
                 "synthetic, zero-valued hidden states and head (power check, "
                 "not a headline figure)"),
        "config": {"workload": b.name, "hidden": b.H, "vocab": b.V,
                   "responses": b.B, "rows": b.N, "valid_tokens": nv,
                   "masked_frac": round(1 - nv / b.N, 4), "lag_sigma": b.sigma,
                   "tokens": args.tokens,
                   **({"lora_rank": r, "lora_scale": LORA_SCALE} if r else {})},
        "rows_per_s": round(b.N * args.steps / (te - ts), 1),
        "step_ms_median": round(float(np.median(step_ms)), 3),
        "step_ms_min": round(float(np.min(step_ms)), 3),
        "mfma_peak_frac_algorithmic": round(mfma_frac, 4),
        "algorithmic_flop_per_valid_token": flop_tok,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fast_baseline": fast,
        "kernel_ms_per_step": {k: round(v, 3) for k, v in kms.items()},
        "loss": loss,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
