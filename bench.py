"""Benchmark of the fused chunked sparse-KL loss head on one MI355X.

One step = one forward call (teacher preparation, chunked fused GEMM with the
online log-sum-exp and gather, sparse-KL reduction, loss) plus one backward
call (teacher preparation, per chunk: logit recompute forming G, dH = G W;
per pair of chunks dW = / += G^T H), writing a fresh dW each step.  Inputs are the
32K-token large-vocabulary workload (T=32768, d=2880, V=201088, K=100, bf16,
5% of positions masked), generated with the seeded recipe of
chunked_sparse_kl_amd.synth and resident in device memory before timing.

Prints ONE JSON line on stdout.  Progress goes to stderr.
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
METRIC = "fused chunked KL fwd+bwd tokens/s & TFLOP/s (% bf16 MFMA peak); peak GiB"
BF16_PEAK_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X published dense fp32 matrix rate
HBM_PEAK_GBS = 8000.0
WORKLOAD = 4                # 32K tokens, d=2880, V=201088, K=100


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_traffic(kernel: str, workload: str = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and on `workload` (a workload name
    followed by the chunk, as the record states it; otherwise None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if workload is not None and rec.get("workload") != workload:
        return None
    # the kernel source, and (where the record names it) the host code that
    # decides how many rows one launch covers, must be the ones measured
    for f, h in ((rec["source_file"], rec["source_sha256"]),
                 (rec.get("driver_file"), rec.get("driver_sha256"))):
        if f is None:
            continue
        src = open(os.path.join(ROOT, "chunked_sparse_kl_amd", "csrc", f), "rb").read()
        if hashlib.sha256(src).hexdigest() != h:
            return None
    return rec["hbm_bytes_per_launch"]


def host_cpus() -> tuple:
    """(CPUs this process may run on, threads the oracle is given): the
    affinity set, capped by OMP_NUM_THREADS when the host sets a share."""
    cpus = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(cpus, int(omp)) if omp.isdigit() and int(omp) > 0 else cpus
    return cpus, threads


def blas_threads() -> int:
    """Threads of the host BLAS the oracle's matrix products run on now."""
    from threadpoolctl import threadpool_info
    return max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
               default=1)


def timed_oracle(fn):
    """Runs fn() with the host BLAS on the threads host_cpus() grants; returns
    (result, seconds, threads used, CPUs visible)."""
    from threadpoolctl import threadpool_limits
    cpus, threads = host_cpus()
    with threadpool_limits(limits=threads, user_api="blas"):
        used = blas_threads()
        t0 = time.perf_counter()
        out = fn()
        dt = time.perf_counter() - t0
    return out, dt, used, cpus


def cpu_baseline(inp: dict, rows: int, seed: int = 3) -> dict:
    """The CPU fp64 oracle (numpy, oracle/kl_oracle.py), as it stands, on a
    seeded subset of rows (forward and backward of those rows), on the host's
    cores."""
    from oracle import kl_oracle as O
    n = inp["H"].shape[0]
    S = np.sort(np.random.default_rng(seed).choice(n, size=rows, replace=False))
    mask = inp["mask"].numpy()

    def run():
        f = O.forward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, rows=S)
        b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, rows=S)
        return f, b

    (f, b), dt, used, cpus = timed_oracle(run)
    assert np.isfinite(f["loss"]) and np.isfinite(b["dW"]).all()
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "host_cpus": int(cpus),
            "sample": f"numpy fp64 oracle, BLAS on {used} threads of {cpus} visible CPUs; "
                      f"{rows} seeded rows of the same workload, forward + backward, {dt:.1f} s wall"}


def make_step(kd, H, W, idx, logp, mask, plan, ws, dW, grad):
    """One timed step: the forward call, then the backward call on the same
    workspace, overwriting dW (accumulate=False: every element written, none
    read).  Returns a function giving (loss, dH) of one step."""
    def step():
        fw = kd.kd_fused_chunked_kl_fwd(H, W, idx, logp, mask, workspace=ws, row_kl=False, plan=plan)
        dH, _ = kd.kd_fused_chunked_kl_bwd(H, W, idx, logp, mask, fw["lse"], grad, workspace=ws,
                                           dW=dW, plan=plan, accumulate=False)
        return fw["loss"], dH
    return step


def roofline_of(stats: list, kernel_traffic_fn, mfma_peak: float = None) -> dict:
    """Roofline record of the kernel with the largest summed time; contractions
    are priced against the MFMA peak of their dtype (bf16 unless given)."""
    peak = BF16_PEAK_TFLOPS if mfma_peak is None else mfma_peak
    dom = max(stats, key=lambda s: s["total_ms"])
    avg_ms = dom["total_ms"] / dom["launches"]
    if dom["flops"] > 0:
        achieved = dom["flops"] / dom["launches"] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        achieved = dom["bytes"] / dom["launches"] / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = kernel_traffic_fn(dom["name"])
    roof["kernel"] = dom["name"]
    roof["avg_launch_ms"] = round(avg_ms, 4)
    return roof


def topk_builder_main(args) -> int:
    """Times the teacher top-K cache builder on the 32K-token head shape used as
    a synthetic teacher (T=32768, d=2880, V=201088, K=100): one build of the
    whole cache per step, inputs resident in device memory."""
    import torch
    import chunked_sparse_kl_amd as kd
    from chunked_sparse_kl_amd import synth

    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[WORKLOAD]
    log(f"generating inputs: {w.name} (as teacher)")
    inp = synth.make_inputs(WORKLOAD)
    Ht, Wt = inp["H"].to(dev), inp["W"].to(dev)
    T, d, V, K = w.T, w.d, w.V, w.K
    plan = kd.kd_teacher_topk_plan(kd.KD_BF16, T, d, V, K, args.chunk)
    log(f"plan: {plan}")
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        idx, logp = kd.kd_teacher_topk(Ht, Wt, K, workspace=ws, plan=plan)
        log(f"warmup {i + 1}/{args.warmup}")
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        idx, logp = kd.kd_teacher_topk(Ht, Wt, K, workspace=ws, plan=plan)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kd.kd_profile_enable(False)
    stats = kd.kd_profile_read()
    ms = elapsed / args.steps * 1e3
    tflops = 4.0 * T * d * V / (ms * 1e-3) / 1e12
    for s in sorted(stats, key=lambda s: -s["total_ms"]):
        log(f"  {s['name']:16s} launches={s['launches']:4d} total={s['total_ms']:9.3f} ms")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import topk_cache_oracle as TO
        rows = np.sort(np.random.default_rng(3).choice(T, size=args.cpu_rows_topk, replace=False))
        ref, dt, used, cpus = timed_oracle(lambda: TO.build_cache(inp["H"], inp["W"], K, rows=rows))
        assert (ref["logp"] <= 0).all()
        cpu = {"value": rows.size / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
               "host_cpus": int(cpus),
               "sample": f"numpy fp64 cache-builder oracle, BLAS on {used} threads of {cpus} visible "
                         f"CPUs; {rows.size} seeded rows of the same shape, {dt:.1f} s wall"}
        log(f"cpu baseline: {cpu}")
    out = {
        "metric": "teacher top-K cache build tokens/s", "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"teacher top-K cache T={T} d={d} V={V} K={K}", "T": T, "d": d,
                   "V": V, "K": K, "chunk": plan["chunk"], "cap": plan["cap"],
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 1), "pct_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
        "kernels": {s["name"]: {"launches": s["launches"], "total_ms": round(s["total_ms"], 3)}
                    for s in stats},
        "roofline": roofline_of(stats, kernel_traffic), "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def memory_sweep_main(args) -> int:
    """Peak device memory and time of one fwd+bwd against T at d=3072,
    V=128256, K=100 (the long-context workload's shapes; values are random
    device tensors: memory and time do not depend on them), with the planner
    choosing the chunk, for the fused path and, with --variants, the two
    comparison variants (dense KL, forward-chunked KL).  A variant that fails
    to allocate at some T is recorded there and not run at larger T.  Fits
    the fused path's peak = a + b*T by least squares over the sizes at the
    planner's largest chunk."""
    import torch
    import chunked_sparse_kl_amd as kd

    dev = torch.device("cuda", 0)
    d, V, K = 3072, 128256, 100
    Ts = [int(t) for t in args.sweep_tokens.split(",")]
    variants = args.variants.split(",")
    calls = {"fused": (kd.kd_fused_chunked_kl_fwd, kd.kd_fused_chunked_kl_bwd),
             "forward_chunked": (kd.kd_forward_chunked_kl_fwd, kd.kd_forward_chunked_kl_bwd),
             "dense": (kd.kd_dense_kl_fwd, kd.kd_dense_kl_bwd)}
    g = torch.Generator(device=dev).manual_seed(5)
    W = (torch.randn(V, d, device=dev, generator=g) * d ** -0.5).to(torch.bfloat16)
    total = torch.cuda.get_device_properties(dev).total_memory
    pts = {v: [] for v in variants}
    failed_at = {v: None for v in variants}

    def one_step(var, H, idx, logp, dW):
        fwd, bwd = calls[var]
        if var == "fused":
            fw = fwd(H, W, idx, logp, None, row_kl=False)
            bwd(H, W, idx, logp, None, fw["lse"], plan=fw["plan"], dW=dW, accumulate=False)
        else:
            fw = fwd(H, W, idx, logp, None, row_kl=False)
            bwd(H, W, idx, logp, None, fw["lse"], fw["grid"], plan=fw["plan"], dW=dW, accumulate=False)
        return fw

    for T in Ts:
        H = torch.randn(T, d, device=dev, generator=g).to(torch.bfloat16)
        idx = torch.randint(0, V, (T, K), device=dev, dtype=torch.int32, generator=g)
        logp = torch.randn(T, K, device=dev, generator=g)
        for var in variants:
            if failed_at[var] is not None:
                continue
            dW = torch.empty((V, d), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats(dev)
            try:
                fw = one_step(var, H, idx, logp, dW)
                torch.cuda.synchronize()
                peak = torch.cuda.max_memory_allocated(dev)
                loss_ok = bool(torch.isfinite(fw["loss"]).item())
                chunk = fw["plan"]["chunk"]
                del fw
                t0 = time.perf_counter()
                for _ in range(args.sweep_steps):
                    fw = one_step(var, H, idx, logp, dW)
                    del fw
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) / args.sweep_steps * 1e3
                pts[var].append({"T": T, "peak_gib": round(peak / 2**30, 4), "ms_per_step": round(ms, 2),
                                 "chunk": chunk, "loss_finite": loss_ok})
                log(f"{var:16s} T={T}: peak {peak / 2**30:.3f} GiB, {ms:.1f} ms/step, chunk {chunk}")
            except torch.cuda.OutOfMemoryError as e:
                failed_at[var] = T
                pts[var].append({"T": T, "out_of_memory": True,
                                 "message": str(e).splitlines()[0][:200]})
                log(f"{var:16s} T={T}: out of device memory")
            finally:
                fw = None
                del dW
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
        del H, idx, logp
        torch.cuda.empty_cache()
    out = {"metric": "peak device memory and time vs tokens (fwd+bwd)", "d": d, "V": V, "K": K,
           "device_memory_gib": round(total / 2**30, 2), "variants": pts,
           "first_T_out_of_memory": failed_at,
           "full_logits_fp32_gib_at_256k": round(262144 * V * 4 / 2**30, 1)}
    fused = [p for p in pts.get("fused", []) if "peak_gib" in p]
    if len(fused) >= 2:
        # the planner's chunk grows with T up to its maximum; from there on the
        # workspace is fixed and peak memory is a + b*T
        cmax = max(p["chunk"] for p in fused)
        fit_pts = [p for p in fused if p["chunk"] == cmax]
        if len(fit_pts) >= 2:
            t = np.array([p["T"] for p in fit_pts], dtype=np.float64)
            y = np.array([p["peak_gib"] for p in fit_pts]) * 2**30
            b, a = np.polyfit(t, y, 1)
            resid = y - (a + b * t)
            out["fused_fit"] = {"over_T": [p["T"] for p in fit_pts], "chunk": cmax,
                                "a_gib": round(a / 2**30, 4), "b_bytes_per_token": round(b, 1),
                                "max_abs_residual_gib": round(float(np.abs(resid).max()) / 2**30, 5)}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--workload", type=int, default=WORKLOAD, choices=sorted((1, 2, 3, 4, 5)),
                    help="1 tiny fp32, 2 toy-head 4K, 3 packed 8K, 4 head-32K (the headline), 5 long 256K")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="rows of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times), to scale HBM byte counters")
    ap.add_argument("--topk-builder", action="store_true",
                    help="time the teacher top-K cache builder instead of the loss step")
    ap.add_argument("--cpu-rows-topk", type=int, default=512, help="rows of the builder's oracle sample")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="peak device memory and time of fwd+bwd against T (4K .. 256K tokens)")
    ap.add_argument("--variants", default="fused",
                    help="memory sweep: comma-separated of fused, forward_chunked, dense")
    ap.add_argument("--sweep-tokens", default="4096,8192,16384,32768,65536,131072,262144",
                    help="memory sweep: the token counts")
    ap.add_argument("--sweep-steps", type=int, default=2, help="memory sweep: timed steps per point")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 3}), flush=True)
        return 0
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the loss head is measured on a single MI355X; "
              "--gpus must be 1", file=sys.stderr)
        return 2
    if args.topk_builder:
        return topk_builder_main(args)
    if args.memory_sweep:
        return memory_sweep_main(args)

    import torch
    import chunked_sparse_kl_amd as kd
    from chunked_sparse_kl_amd import synth

    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[args.workload]
    log(f"generating inputs: {w.name}")
    inp = synth.make_inputs(args.workload)
    H, W = inp["H"].to(dev), inp["W"].to(dev)
    idx, logp, mask = inp["idx"].to(dev), inp["logp"].to(dev), inp["mask"].to(dev)
    T, d, V, K = w.T, w.d, w.V, w.K
    dtype = kd.KD_BF16 if w.dtype == "bf16" else kd.KD_F32
    plan = kd.kd_plan_query(dtype, T, d, V, K, args.chunk if args.chunk else w.chunk)
    log(f"plan: {plan}")
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    grad = torch.ones(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    step = make_step(kd, H, W, idx, logp, mask, plan, ws, dW, grad)

    for i in range(args.warmup):
        loss, _ = step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} loss={loss.item():.6f}")
    torch.cuda.reset_peak_memory_stats(dev)
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        loss, dH = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kd.kd_profile_enable(False)
    stats = kd.kd_profile_read()
    peak_gib = torch.cuda.max_memory_allocated(dev) / 2**30
    loss_v = loss.item()
    log(f"timed {args.steps} steps in {elapsed:.3f} s, loss={loss_v:.6f}")

    ms = elapsed / args.steps * 1e3
    tokens_s = T * args.steps / elapsed
    flop_step = 8.0 * T * d * V
    tflops = flop_step / (ms * 1e-3) / 1e12
    kernels = sorted(stats, key=lambda s: -s["total_ms"])
    for s in kernels:
        log(f"  {s['name']:16s} launches={s['launches']:4d} total={s['total_ms']:9.3f} ms "
            f"avg={s['total_ms'] / s['launches']:8.3f} ms "
            f"{(s['flops'] / (s['total_ms'] * 1e-3) / 1e12) if s['flops'] else 0:8.1f} TFLOP/s")
    run_name = f"{w.name} chunk {plan['chunk']}"
    roof = roofline_of(stats, lambda k: kernel_traffic(k, run_name),
                       BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows} rows")
        cpu = cpu_baseline(inp, args.cpu_rows)
        log(f"cpu baseline: {cpu}")

    props = torch.cuda.get_device_properties(dev)
    out = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "d": d, "V": V, "K": K, "mask": w.mask,
                   "chunk": plan["chunk"], "n_chunks": plan["n_chunks"],
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 1), "pct_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
        "peak_gib": round(peak_gib, 3), "loss": loss_v,
        "device": {"name": props.name, "compute_units": props.multi_processor_count},
        "kernels": {s["name"]: {"launches": s["launches"], "total_ms": round(s["total_ms"], 3)}
                    for s in kernels},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
