"""Throughput of the W8A8 DiT block forward on one MI355X.

A step is one h3k_block_forward call (AdaLN modulation, fused LN + modulate + int8
quantiser, W8A8 QKV GEMM with RoPE and head-major scatter, bf16 flash attention, O
quantiser, W8A8 out-projection with gated residual, second LN + quantiser, W8A8 MLP-up
with GELU, g quantiser, W8A8 MLP-down with gated residual) on one batch of synthetic
input already resident in HBM. Default workload: one block at d=5120, 40 heads x 128,
MLP 20480, L=16384 tokens (4x64x64 grid).

Prints one JSON line. Per-kernel durations come from HIP events recorded by the library
on the stream each kernel runs on, inside the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"int8": 5000.0, "bf16": 2500.0, "fp32": 157.3}  # dense TOP/s or TFLOP/s, MI355X
HBM_GBS = 8000.0


def kernel_work(wl, L):
    """Algorithmic work per launch: ('ops', n, dtype) for matrix-core kernels,
    ('bytes', n) for bandwidth-bound ones."""
    d, F, dc = wl.d, wl.d_ff, wl.d_cond
    return {
        "gemm_qkv": ("ops", 2.0 * L * 3 * d * d, "int8"),
        "gemm_o": ("ops", 2.0 * L * d * d, "int8"),
        "gemm_up": ("ops", 2.0 * L * F * d, "int8"),
        "gemm_down": ("ops", 2.0 * L * d * F, "int8"),
        "attention": ("ops", 4.0 * L * L * d, "bf16"),
        # read bf16 x, write int8 codes + fp32 scale per token
        "ln_quant": ("bytes", L * (3.0 * d + 4)),
        "rowquant_o": ("bytes", L * (3.0 * d + 4)),
        "rowquant_g": ("bytes", L * (3.0 * F + 4)),
        "adaln": ("bytes", 6.0 * d * dc * 2),
    }


def cpu_baseline(wl, x, c, bw, n_rows: int):
    """The oracle timed on the host: QKV for all tokens (attention needs every key) plus the
    rest of the block for n_rows sampled tokens; cost per token = prefix/L + rest/n_rows."""
    import numpy as np

    import oracle as O

    def np64(t):
        return t.detach().float().cpu().numpy().astype(np.float64)

    w = {"w_ada": np64(bw.w_ada)}
    for k in ("qkv", "o", "up", "down"):
        w["q_" + k] = getattr(bw, "w_" + k).cpu().numpy()
        w["s_" + k] = getattr(bw, "s_" + k).cpu().numpy()
    xn = np64(x)
    cn = np64(c)
    rows = np.linspace(0, wl.L - 1, n_rows).astype(np.int64)
    kw = dict(n_heads=wl.n_heads, head_dim=wl.head_dim, grid=wl.grid)
    t0 = time.perf_counter()
    O.block_forward(xn, cn, w, rows=np.zeros(0, np.int64), **kw)
    t1 = time.perf_counter()
    O.block_forward(xn, cn, w, rows=rows, **kw)
    t2 = time.perf_counter()
    prefix = t1 - t0
    rest = max((t2 - t1) - prefix, 1e-9)
    per_token = prefix / wl.L + rest / n_rows
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": (f"{wl.name}: LN+quant+QKV+RoPE for all {wl.L} tokens ({prefix:.1f} s), then "
                       f"attention, out-proj and MLP for {n_rows} evenly spaced tokens "
                       f"({rest:.1f} s); tokens/s = 1 / (prefix/{wl.L} + rest/{n_rows})"),
            "seconds": t2 - t0}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="block_l16384")
    ap.add_argument("--variant", default="w8a8", choices=["w8a8", "bf16gemm", "fp32"])
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 50-block stack and L=65536 measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB on the device twice (counter calibration) and exit")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "h3k runs on one GPU; --gpus must be 1 (the sharded design is described, not implemented)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import synth_inputs as S
    from video_diffusion_transformer_03_amd import h3k

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 2}))
        return
    wl = S.WORKLOADS[args.workload]
    flags = {"w8a8": 0, "bf16gemm": h3k.F_BF16_GEMM, "fp32": h3k.F_FP32_DEBUG}[args.variant]

    wb = S.block_weights_bf16(wl, 0, device="cuda")
    bw = h3k.quantize_block(wb, keep_bf16=(args.variant == "bf16gemm"))
    if args.variant != "bf16gemm":
        del wb
    xdt = torch.float32 if args.variant == "fp32" else torch.bfloat16
    x = S.activations(wl, device="cuda").to(xdt)
    c = S.conditioning(wl, device="cuda")
    dims = h3k.dims_of(wl)
    L = wl.L
    ws = h3k.alloc_workspace(h3k.workspace_bytes(dims, L, flags))
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        h3k.block_forward(x, c, bw, dims, flags, ws, out)
    torch.cuda.synchronize()

    h3k.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h3k.block_forward(x, c, bw, dims, flags, ws, out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = h3k.profile_read()
    h3k.profile_enable(False)

    ms_step = (t1 - t0) * 1e3 / args.steps
    value = L * args.steps / (t1 - t0)

    work = kernel_work(wl, L)
    copy_gbps = device_copy_gbps(torch)
    kernels = {}
    for name, (n, tot) in prof.items():
        if n == 0:
            continue
        avg = tot / n
        ent = {"launches_per_step": n / args.steps, "avg_ms": round(avg, 5),
               "ms_per_step": round(tot / args.steps, 5)}
        if name in work and args.variant == "w8a8":
            wk = work[name]
            if wk[0] == "ops":
                rate = wk[1] / (avg * 1e-3) / 1e12
                ent.update(achieved=round(rate, 2), peak=PEAK[wk[2]],
                           unit="TOP/s" if wk[2] == "int8" else "TFLOP/s",
                           frac=round(rate / PEAK[wk[2]], 4))
            else:
                rate = wk[1] / (avg * 1e-3) / 1e9
                ent.update(achieved=round(rate, 1), peak=HBM_GBS, unit="GB/s",
                           frac=round(rate / HBM_GBS, 4), frac_of_copy=round(rate / copy_gbps, 4))
        kernels[name] = ent

    label = {"w8a8": "W8A8", "bf16gemm": "BF16", "fp32": "int8 GEMM + fp32"}[args.variant]
    result = {
        # the headline workload's metric name; other workloads and variants say what ran
        "metric": f"DiT block tokens/s ({label}, d={wl.d}, L={L}) + % of peak int8/bf16 MFMA",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"w8a8": "int8 GEMM + bf16 attention", "bf16gemm": "bf16",
                  "fp32": "int8 GEMM + f32"}[args.variant],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random-init)",
        "config": {"workload": wl.name, "d": wl.d, "n_heads": wl.n_heads, "head_dim": wl.head_dim,
                   "d_ff": wl.d_ff, "d_cond": wl.d_cond, "L": L, "grid": list(wl.grid),
                   "variant": args.variant},
    }
    if args.variant == "w8a8":
        gemm_names = ["gemm_qkv", "gemm_o", "gemm_up", "gemm_down"]
        gemm_ops = sum(work[k][1] for k in gemm_names)
        gemm_ms = sum(kernels[k]["ms_per_step"] for k in gemm_names if k in kernels)
        attn_ms = kernels.get("attention", {}).get("ms_per_step", float("nan"))
        result["gemm_int8_frac"] = round(gemm_ops / (gemm_ms * 1e-3) / 1e12 / PEAK["int8"], 4)
        result["attention_bf16_frac"] = round(work["attention"][1] / (attn_ms * 1e-3) / 1e12 / PEAK["bf16"], 4)
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        dk = kernels[dom]
        traffic = measured_traffic(args.traffic, wl.name, dom)
        result["roofline"] = {"kernel": dom, "bound": "mfma" if work[dom][0] == "ops" else "hbm",
                              "achieved": dk.get("achieved"), "peak": dk.get("peak"),
                              "unit": dk.get("unit"), "frac": dk.get("frac"), "traffic": traffic}
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "hbm_gib": round(props.total_memory / 2**30, 1)}
    result["device_copy_GBps"] = round(copy_gbps, 1)
    result["kernels"] = kernels
    if not args.no_extras and args.variant == "w8a8" and args.workload == "block_l16384":
        del ws, out
        torch.cuda.empty_cache()
        result["extras"] = extras(S, h3k, torch)
    if not args.no_cpu_baseline and args.variant == "w8a8":
        result["cpu_baseline"] = cpu_baseline(wl, x, c, bw, args.cpu_rows)
    print(json.dumps(result))


def measured_traffic(path, workload, kernel):
    """HBM bytes per launch of `kernel` from the counter summary (FETCH_SIZE + WRITE_SIZE,
    each scaled by its copy-calibration factor), or None when there is no summary for this
    workload or the kernel's source changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    try:
        tr = json.load(open(path))
    except ValueError:
        return None
    if tr.get("workload") != workload:
        return None
    key = {"attention": "attn_v2_kernel"}.get(kernel)
    if key is None:
        return None
    import hashlib
    here = os.path.join(ROOT, "video_diffusion_transformer_03_amd", "csrc")
    for name, ent in tr.get("kernels", {}).items():
        if key in name:
            src = ent["source"]
            h = hashlib.sha256(open(os.path.join(here, src), "rb").read()).hexdigest()[:16]
            if tr.get("sources", {}).get(src) != h:
                return None
            return round(ent["read_bytes"] + ent["write_bytes"])
    return None


def device_copy_gbps(torch, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Bandwidth of a plain device-to-device copy (bytes read plus bytes written per second):
    the practical ceiling beside the nominal 8 TB/s for kernels that stream HBM."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    return 2 * nbytes / dt / 1e9


def _time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def extras(S, h3k, torch):
    """Measurements beside the headline line:
      - the 50-block stack at L=16384: ms per denoising step without and with horizontal
        token pairing in blocks [10, 40), eager and replayed as a recorded HIP graph, and a
        sweep of pairing ranges with the relative L2 distance of the stack output from the
        unpaired stack's;
      - the precision series at L=16384 (BF16 GEMMs, int8 MLP, int8 MLP + QKV, W8A8);
      - block time against sequence length (L = 4096 .. 65536) with a least-squares fit
        t = a L + b L^2, and one block at L=65536 with its attention fraction."""
    import dataclasses

    out = {}
    wl = S.WORKLOADS["stack50_l16384"]
    blocks = []
    for b in range(wl.n_blocks):
        wb = S.block_weights_bf16(wl, b, device="cuda")
        blocks.append(h3k.quantize_block(wb))
        del wb
    x = S.activations(wl, device="cuda")
    c = S.conditioning(wl, device="cuda")
    dims = h3k.dims_of(wl)
    res, sweep, ref = {}, {}, None
    for tr in [(0, 0), wl.tr_range, (5, 45), (15, 35), (20, 30), (0, 50)]:
        ws = h3k.alloc_workspace(h3k.stack_workspace_bytes(dims, wl.L, *tr))
        y = torch.empty_like(x)
        t = _time_steps(torch, lambda: h3k.stack_forward(x, c, blocks, dims, tr[0], tr[1], 0, ws, y), 2, 1)
        if tr in ((0, 0), tuple(wl.tr_range)):
            g = h3k.stack_graph(x, c, blocks, dims, tr[0], tr[1], 0, ws, y)
            tg = _time_steps(torch, g.launch, 2, 1)
            res["graph_" + ("token_reduction" if tr[1] > tr[0] else "full")] = round(tg * 1e3, 2)
            del g
        if tr == (0, 0):
            ref = y.float().clone()
            res["full"] = round(t * 1e3, 2)
        else:
            yf = y.float()
            dist = float((yf - ref).norm() / ref.norm())
            if tr == tuple(wl.tr_range):
                res["token_reduction"] = round(t * 1e3, 2)
            sweep[f"[{tr[0]},{tr[1]})"] = {"ms": round(t * 1e3, 2), "rel_l2_vs_full": round(dist, 5)}
        del ws, y
    out["stack50_l16384_ms_per_denoise_step"] = res
    out["stack50_token_reduction_sweep"] = sweep
    # whole denoising loops (h3k_denoise) with the pages' speed/quality controls: the
    # aggressive pass count, and the default column of their table (20 passes, reuse 2,
    # core reuse 4, 45 blocks, token pairing on)
    loops = {}
    for name, kw in [("steps4", dict(steps=4, reuse=1, core_reuse=1, layers=50, tr=(0, 0))),
                     ("steps20_reuse2_core4_layers45_tr", dict(steps=20, reuse=2, core_reuse=4,
                                                               layers=45, tr=(10, 40)))]:
        ws = h3k.alloc_workspace(h3k.denoise_workspace_bytes(dims, wl.L, *kw["tr"]))
        xs = x.clone()
        run = lambda: h3k.denoise(xs, c, blocks, dims, kw["steps"], kw["reuse"], kw["core_reuse"],  # noqa: E731
                                  kw["layers"], kw["tr"][0], kw["tr"][1], 0, ws)
        t = _time_steps(torch, run, 1, 1)
        loops[name] = {"s": round(t, 3), "stack_evaluations": len([
            f for f, k in enumerate(k for k in range(kw["steps"]) if k % kw["reuse"] == 0 or k == kw["steps"] - 1)
            if f % kw["core_reuse"] == 0 or k == kw["steps"] - 1])}
        del ws, xs
    out["denoise_l16384"] = loops
    del blocks, ref
    torch.cuda.empty_cache()

    # precision series (one block, L=16384)
    wl = S.WORKLOADS["block_l16384"]
    bw = h3k.quantize_block(S.block_weights_bf16(wl, 0, device="cuda"), keep_bf16=True)
    x = S.activations(wl, device="cuda")
    c = S.conditioning(wl, device="cuda")
    dims = h3k.dims_of(wl)
    series = {}
    for name, flags in [("bf16", h3k.F_BF16_GEMM), ("int8_mlp", h3k.F_BF16_QKV | h3k.F_BF16_OUT),
                        ("int8_mlp_qkv", h3k.F_BF16_OUT), ("w8a8", 0)]:
        ws = h3k.alloc_workspace(h3k.workspace_bytes(dims, wl.L, flags))
        y = torch.empty_like(x)
        t = _time_steps(torch, lambda: h3k.block_forward(x, c, bw, dims, flags, ws, y), 5, 2)
        series[name] = round(t * 1e3, 3)
        del ws, y
    out["precision_series_l16384_ms"] = series
    del bw
    torch.cuda.empty_cache()

    # sequence-length scaling (one W8A8 block)
    base = S.WORKLOADS["block_l16384"]
    grids = {4096: (4, 32, 32), 8192: (4, 32, 64), 16384: (4, 64, 64), 32768: (8, 64, 64),
             65536: (16, 64, 64)}
    scaling, l65536 = {}, None
    for L, grid in grids.items():
        wl = dataclasses.replace(base, name=f"block_l{L}", grid=grid)
        bw = h3k.quantize_block(S.block_weights_bf16(wl, 0, device="cuda"))
        x = S.activations(wl, device="cuda")
        c = S.conditioning(wl, device="cuda")
        dims = h3k.dims_of(wl)
        ws = h3k.alloc_workspace(h3k.workspace_bytes(dims, L, 0))
        y = torch.empty_like(x)
        h3k.profile_enable(True)
        t = _time_steps(torch, lambda: h3k.block_forward(x, c, bw, dims, 0, ws, y), 3, 1)
        prof = h3k.profile_read()
        h3k.profile_enable(False)
        n, tot = prof["attention"]
        attn_ms = tot / n
        frac = 4.0 * L * L * wl.d / (attn_ms * 1e-3) / 1e12 / PEAK["bf16"]
        scaling[str(L)] = {"ms": round(t * 1e3, 3), "attention_ms": round(attn_ms, 3),
                           "attention_bf16_frac": round(frac, 4)}
        if L == 65536:
            l65536 = {"ms_per_step": round(t * 1e3, 3), "tokens_per_s": round(L / t, 1),
                      "attention_ms": round(attn_ms, 3), "attention_bf16_frac": round(frac, 4)}
        del bw, x, ws, y
        torch.cuda.empty_cache()
    Ls = [float(k) for k in scaling]
    ts = [scaling[k]["ms"] for k in scaling]
    # least squares for t = a L + b L^2 (normal equations of the two-column design)
    s11 = sum(v * v for v in Ls)
    s12 = sum(v ** 3 for v in Ls)
    s22 = sum(v ** 4 for v in Ls)
    r1 = sum(v * t for v, t in zip(Ls, ts))
    r2 = sum(v * v * t for v, t in zip(Ls, ts))
    det = s11 * s22 - s12 * s12
    a = (r1 * s22 - r2 * s12) / det
    b = (s11 * r2 - s12 * r1) / det
    out["sequence_scaling_ms"] = {"points": scaling, "fit": {"a_ms_per_token": a, "b_ms_per_token2": b,
                                  "quadratic_share_at_16384": round(b * 16384 ** 2 / (a * 16384 + b * 16384 ** 2), 4)}}
    out["block_l65536"] = l65536
    return out


if __name__ == "__main__":
    main()
