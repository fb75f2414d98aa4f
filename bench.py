"""Throughput of the W8A8 DiT block forward on one MI355X.

A step is one h3k_block_forward call (AdaLN modulation, fused LN + modulate + int8
quantiser, W8A8 QKV GEMM with RoPE and head-major scatter, flash attention on fp16
matrix-core operands, O quantiser, W8A8 out-projection with gated residual, second LN + quantiser, W8A8 MLP-up
with GELU, g quantiser, W8A8 MLP-down with gated residual) on one batch of synthetic
input already resident in HBM. Default workload: one block at d=5120, 40 heads x 128,
MLP 20480, L=16384 tokens (4x64x64 grid).

Prints one JSON line. The headline time is an uninstrumented loop of block calls; the
per-kernel durations come from a second, profiled loop of the same calls, in which the
library records HIP events on the stream each kernel runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# dense TOP/s or TFLOP/s, MI355X (fp16 and bf16 matrix cores have the same dense peak)
PEAK = {"int8": 5000.0, "bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
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
        "attention": ("ops", 4.0 * L * L * d, "fp16"),
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
    cores = _cores()
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
            "seconds": t2 - t0, "prefix_per_token_s": prefix / wl.L, "rest_per_token_s": rest / n_rows}


def log(msg: str) -> None:
    """Progress on stderr (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def _oracle_w(bw):
    import numpy as np
    w = {"w_ada": bw.w_ada.detach().float().cpu().numpy().astype(np.float64)}
    for k in ("qkv", "o", "up", "down"):
        w["q_" + k] = getattr(bw, "w_" + k).cpu().numpy()
        w["s_" + k] = getattr(bw, "s_" + k).cpu().numpy()
    return w


def attention_row_seconds(L, H, Dh, rows=8, seed=5):
    """Host seconds the oracle's attention takes per query row at L keys (random values:
    its cost depends on the shapes only)."""
    import numpy as np

    import oracle as O
    g = np.random.default_rng(seed)
    q = g.standard_normal((L, H, Dh))
    k = g.standard_normal((L, H, Dh))
    v = g.standard_normal((L, H, Dh))
    t0 = time.perf_counter()
    O.attention(q, k, v, np.arange(rows))
    return (time.perf_counter() - t0) / rows


def cpu_baselines(S, h3k, torch, head_cpu, bw_head):
    """The oracle on the host for the other workloads, each bounded to a few seconds:
      - tiny (2 blocks, d = 256, L = 512): the whole stack, median of 3, on all the threads
        and on one (the per-core figure);
      - block_l4096: the headline's sampling on its own activations (8 outlier channels);
        the d = 5120 weights are the headline's (the oracle's cost depends on the shapes);
      - block_l65536 and the 50-block stack at L = 16384 (with and without pairing in blocks
        [10, 40)): extrapolated from the headline sample's per-token costs and the oracle's
        attention timed per query row at each key count (attention per row grows with L;
        the rest is per token)."""
    import numpy as np

    import oracle as O
    out = {}
    cores = _cores()
    # tiny: full stack
    wl = S.WORKLOADS["tiny"]
    blocks = [h3k.quantize_block({k: v.cuda() for k, v in S.block_weights_bf16(wl, b).items()})
              for b in range(wl.n_blocks)]
    ow = [_oracle_w(b) for b in blocks]
    x = S.activations(wl).float().numpy().astype(np.float64)
    c = S.conditioning(wl).numpy().astype(np.float64)
    kw = dict(n_heads=wl.n_heads, head_dim=wl.head_dim, grid=wl.grid)

    def run_tiny():
        t0 = time.perf_counter()
        O.stack_forward(x, c, ow, **kw)
        return time.perf_counter() - t0
    ts = sorted(run_tiny() for _ in range(3))
    ent = {"value": round(wl.L / ts[1], 1), "unit": "tokens/s (2-block stack)", "cores": cores,
           "kind": "oracle", "sample": "whole 2-block stack, median of 3"}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = sorted(run_tiny() for _ in range(3))[1]
        ent["one_thread"] = {"value": round(wl.L / t1, 1), "cores": 1}
    except Exception:
        pass
    out["tiny"] = ent
    # block_l4096 on its own activations
    wl4 = S.WORKLOADS["block_l4096"]
    x4 = S.activations(wl4, device="cuda")
    c4 = S.conditioning(wl4, device="cuda")
    r4 = cpu_baseline(wl4, x4, c4, bw_head, 512)
    out["block_l4096"] = {k: r4[k] for k in ("value", "unit", "cores", "kind", "sample")}
    # extrapolations from the headline sample
    wl2 = S.WORKLOADS["block_l16384"]
    pre, rest = head_cpu["prefix_per_token_s"], head_cpu["rest_per_token_s"]
    a16 = attention_row_seconds(wl2.L, wl2.n_heads, wl2.head_dim)
    a8 = attention_row_seconds(wl2.L // 2, wl2.n_heads, wl2.head_dim)
    a64 = attention_row_seconds(4 * wl2.L, wl2.n_heads, wl2.head_dim, rows=4)
    rest_na = max(rest - a16, 0.0)  # per-token work other than attention

    def block_s(L, a_row):
        return L * (pre + rest_na + a_row)
    out["block_l65536"] = {"value": round(65536 / block_s(65536, a64), 2), "unit": "tokens/s",
                           "cores": cores, "kind": "oracle (extrapolated)",
                           "sample": ("per-token costs of the block_l16384 sample with the attention per "
                                      f"row timed at 65536 keys ({a64:.3f} s per row)")}
    full = 50 * block_s(wl2.L, a16)
    paired = 20 * block_s(wl2.L, a16) + 30 * block_s(wl2.L // 2, a8)
    out["stack50_l16384"] = {"value": round(full, 1), "unit": "s per denoising step (50 blocks)",
                             "token_reduction_value": round(paired, 1), "cores": cores,
                             "kind": "oracle (extrapolated)",
                             "sample": ("50 x the block_l16384 per-token costs; with pairing, 30 blocks at "
                                        f"8192 tokens (attention per row {a8:.4f} s at 8192 keys, "
                                        f"{a16:.4f} s at 16384)")}
    return out


def weight_bytes(wl):
    """Bytes of one block's weights in each variant of the precision series (the pages
    report the model's DiT weights going from 36.4 GiB in BF16 to 19.8 GiB with int8): the
    AdaLN linear layer stays bf16; a W8A8 projection holds int8 codes and fp32 scales, a
    bf16 one its bf16 matrix."""
    d, F, dc = wl.d, wl.d_ff, wl.d_cond
    proj = {"qkv": (3 * d, d), "o": (d, d), "up": (F, d), "down": (d, F)}
    int8_of = {"bf16": (), "int8_mlp": ("up", "down"), "int8_mlp_qkv": ("qkv", "up", "down"),
               "w8a8": ("qkv", "o", "up", "down")}
    out = {}
    for name, i8 in int8_of.items():
        b = 6 * d * dc * 2
        for k, (n, kk) in proj.items():
            b += n * kk + 4 * n if k in i8 else 2 * n * kk
        out[name] = {"per_block_GiB": round(b / 2**30, 4), "per_50_blocks_GiB": round(50 * b / 2**30, 2)}
    return out


def clock_under_load(torch, fn, n=12, cycles=int(6e7)):
    """Shader clock (MHz) sustained while n calls of fn run: a one-wave spin kernel
    (torch.cuda._sleep, which waits for `cycles` ticks of the shader clock counter) runs on
    a side stream of default priority alongside them, timed with events on that stream;
    cycles / elapsed is the mean engine clock over the spin. None where unavailable. (The
    SMI clock reading, sampled instead, proved unreliable: it read anything from 166 to
    2095 MHz under the same load.)"""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    try:
        with torch.cuda.stream(side):
            e0.record(side)
            torch.cuda._sleep(cycles)
            e1.record(side)
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
    except (AttributeError, RuntimeError):
        return None
    return round(cycles / (ms * 1e-3) / 1e6, 1) if ms > 0 else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="block_l16384")
    ap.add_argument("--variant", default="w8a8", choices=["w8a8", "w8a8_attn_bf16", "bf16gemm", "fp32"])
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 50-block stack and L=65536 measurements")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the engine clock under load (profiled runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB on the device twice (counter calibration) and exit")
    ap.add_argument("--stack-step", action="store_true",
                    help="time the 50-block stack step (L=16384, token pairing in the middle blocks) "
                         "instead of one block: warm-up, plain and event-timed loops as for a block "
                         "(for profiling the whole step); prints its own JSON line")
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
    if args.stack_step:
        stack_step(args, S, h3k, torch)
        return
    wl = S.WORKLOADS[args.workload]
    flags = {"w8a8": 0, "w8a8_attn_bf16": h3k.F_ATTN_BF16, "bf16gemm": h3k.F_BF16_GEMM,
             "fp32": h3k.F_FP32_DEBUG}[args.variant]
    int8 = args.variant in ("w8a8", "w8a8_attn_bf16")

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

    log(f"{wl.name} {args.variant}: {args.warmup} warm-up and {args.steps} timed steps")
    for _ in range(args.warmup):
        h3k.block_forward(x, c, bw, dims, flags, ws, out)
    torch.cuda.synchronize()

    # the headline: an uninstrumented loop
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h3k.block_forward(x, c, bw, dims, flags, ws, out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-kernel durations: the same loop with the library's event records
    h3k.profile_enable(True)
    for _ in range(args.steps):
        h3k.block_forward(x, c, bw, dims, flags, ws, out)
    torch.cuda.synchronize()
    prof = h3k.profile_read()
    h3k.profile_enable(False)

    ms_step = (t1 - t0) * 1e3 / args.steps
    value = L * args.steps / (t1 - t0)
    # the same step with bf16 attention operands, reported beside the fp16 default (which
    # stores Q, K, V, P and O as fp16 at the same bytes and instruction rate)
    bf16_attn = None
    if args.variant == "w8a8" and not args.no_extras:
        fb = flags | h3k.F_ATTN_BF16
        wsb = h3k.alloc_workspace(h3k.workspace_bytes(dims, L, fb))
        tb = _time_steps(torch, lambda: h3k.block_forward(x, c, bw, dims, fb, wsb, out), args.steps,
                         args.warmup)
        h3k.profile_enable(True)
        for _ in range(args.steps):
            h3k.block_forward(x, c, bw, dims, fb, wsb, out)
        torch.cuda.synchronize()
        pb = h3k.profile_read()
        h3k.profile_enable(False)
        na, ta = pb["attention"]
        wk = kernel_work(wl, L)["attention"][1]
        bf16_attn = {"ms_per_step": round(tb * 1e3, 4), "value": round(L / tb, 1),
                     "attention_ms": round(ta / na, 5),
                     "attention_frac": round(wk / (ta / na * 1e-3) / 1e12 / PEAK["bf16"], 4)}
        del wsb
    sclk = None if args.no_clock else clock_under_load(
        torch, lambda: h3k.block_forward(x, c, bw, dims, flags, ws, out))

    work = kernel_work(wl, L)
    copy_gbps = device_copy_gbps(torch)
    kernels = {}
    for name, (n, tot) in prof.items():
        if n == 0:
            continue
        avg = tot / n
        ent = {"launches_per_step": n / args.steps, "avg_ms": round(avg, 5),
               "ms_per_step": round(tot / args.steps, 5)}
        if name in work and int8:
            wk = work[name]
            if wk[0] == "ops":
                rate = wk[1] / (avg * 1e-3) / 1e12
                ent.update(achieved=round(rate, 2), peak=PEAK[wk[2]],
                           unit="TOP/s" if wk[2] == "int8" else "TFLOP/s",
                           frac=round(rate / PEAK[wk[2]], 4))
            else:
                rate = wk[1] / (avg * 1e-3) / 1e9
                ent.update(achieved=round(rate, 1), peak=HBM_GBS, unit="GB/s",
                           frac=round(rate / HBM_GBS, 4), vs_torch_copy=round(rate / copy_gbps, 4))
        kernels[name] = ent

    label = {"w8a8": "W8A8", "w8a8_attn_bf16": "W8A8, bf16 attention", "bf16gemm": "BF16",
             "fp32": "int8 GEMM + fp32"}[args.variant]
    result = {
        # the headline workload's metric name; other workloads and variants say what ran
        "metric": f"DiT block tokens/s ({label}, d={wl.d}, L={L}) + % of peak int8/bf16 MFMA",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"w8a8": "int8 GEMM + fp16 attention", "w8a8_attn_bf16": "int8 GEMM + bf16 attention",
                  "bf16gemm": "bf16", "fp32": "int8 GEMM + f32"}[args.variant],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random-init)",
        "config": {"workload": wl.name, "d": wl.d, "n_heads": wl.n_heads, "head_dim": wl.head_dim,
                   "d_ff": wl.d_ff, "d_cond": wl.d_cond, "L": L, "grid": list(wl.grid),
                   "variant": args.variant},
    }
    if int8:
        gemm_names = ["gemm_qkv", "gemm_o", "gemm_up", "gemm_down"]
        gemm_ops = sum(work[k][1] for k in gemm_names)
        gemm_ms = sum(kernels[k]["ms_per_step"] for k in gemm_names if k in kernels)
        attn_ms = kernels.get("attention", {}).get("ms_per_step", float("nan"))
        result["gemm_int8_frac"] = round(gemm_ops / (gemm_ms * 1e-3) / 1e12 / PEAK["int8"], 4)
        # against the dense 16-bit matrix-core peak (the same 2.5 PFLOP/s for fp16 and bf16)
        result["attention_frac"] = round(work["attention"][1] / (attn_ms * 1e-3) / 1e12 / PEAK["fp16"], 4)
        result["attention_operands"] = "bf16" if flags & h3k.F_ATTN_BF16 else "fp16"
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        dk = kernels[dom]
        traffic = measured_traffic(args.traffic, wl.name, dom)
        result["roofline"] = {"kernel": dom, "bound": "mfma" if work[dom][0] == "ops" else "hbm",
                              "achieved": dk.get("achieved"), "peak": dk.get("peak"),
                              "unit": dk.get("unit"), "frac": dk.get("frac"), "traffic": traffic}
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "hbm_gib": round(props.total_memory / 2**30, 1),
                        "max_clock_mhz": round(getattr(props, "clock_rate", 0) / 1000.0, 1) or None,
                        "clock_under_load_mhz": sclk,
                        "clock_method": "shader-clock spin kernel beside the block loop (cycles / time)"}
    if int8 and sclk:
        # the dense peaks recomputed at the clock observed under this load: CUs x clock x
        # 8192 int8 ops (4096 16-bit flops) per clock per CU
        cu = props.multi_processor_count
        pk8 = cu * sclk * 1e6 * 8192 / 1e12
        pk16 = cu * sclk * 1e6 * 4096 / 1e12
        gemm_ops = sum(work[k][1] for k in ("gemm_qkv", "gemm_o", "gemm_up", "gemm_down"))
        gemm_ms = sum(kernels[k]["ms_per_step"] for k in ("gemm_qkv", "gemm_o", "gemm_up", "gemm_down"))
        result["at_observed_clock"] = {
            "clock_mhz": sclk, "peak_int8_TOPs": round(pk8, 1), "peak_16bit_TFLOPs": round(pk16, 1),
            "gemm_int8_frac": round(gemm_ops / (gemm_ms * 1e-3) / 1e12 / pk8, 4),
            "attention_frac": round(work["attention"][1] / (kernels["attention"]["ms_per_step"] * 1e-3) / 1e12 / pk16, 4)}
    # a plain torch device copy, for comparison (not a ceiling: the row kernels beat it)
    if bf16_attn is not None:
        result["with_bf16_attention"] = bf16_attn
    result["torch_copy_GBps"] = round(copy_gbps, 1)
    result["kernels"] = kernels
    if not args.no_extras and args.variant == "w8a8" and args.workload == "block_l16384":
        del ws, out
        torch.cuda.empty_cache()
        log("extras: 50-block stack, precision series, sequence scaling")
        result["extras"] = extras(S, h3k, torch)
    result["weight_bytes"] = weight_bytes(wl)
    if not args.no_cpu_baseline and args.variant == "w8a8":
        log("oracle on the host (cpu_baseline)")
        cb = cpu_baseline(wl, x, c, bw, args.cpu_rows)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                     "cpu_model", "seconds")}
        if args.workload == "block_l16384" and not args.no_extras:
            log("oracle on the host: other workloads")
            result["cpu_baselines_other_workloads"] = cpu_baselines(S, h3k, torch, cb, bw)
    print(json.dumps(result))


def stack_step(args, S, h3k, torch):
    """The 50-block W8A8 stack at L=16384 with horizontal token pairing in its middle
    blocks, run as `warmup` untimed steps, `steps` timed steps and `steps` steps with the
    library's event records (the loop structure of the block measurement, so one profile
    summary reads both)."""
    wl = S.WORKLOADS["stack50_l16384"]
    tr = tuple(wl.tr_range)
    blocks = []
    for b in range(wl.n_blocks):
        wb = S.block_weights_bf16(wl, b, device="cuda")
        blocks.append(h3k.quantize_block(wb, rowmajor=False))
        del wb
    x = S.activations(wl, device="cuda")
    c = S.conditioning(wl, device="cuda")
    dims = h3k.dims_of(wl)
    ws = h3k.alloc_workspace(h3k.stack_workspace_bytes(dims, wl.L, *tr))
    y = torch.empty_like(x)
    step = lambda: h3k.stack_forward(x, c, blocks, dims, tr[0], tr[1], 0, ws, y)  # noqa: E731
    log(f"stack step {wl.name} pairing {tr}: {args.warmup} warm-up and {args.steps} timed steps")
    t = _time_steps(torch, step, args.steps, args.warmup)
    h3k.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = h3k.profile_read()
    h3k.profile_enable(False)
    kern = {k: {"launches_per_step": n / args.steps, "ms_per_step": round(tt / args.steps, 3)}
            for k, (n, tt) in prof.items() if n}
    print(json.dumps({"metric": f"ms per denoising step ({wl.n_blocks} W8A8 blocks, L={wl.L}, "
                                f"token pairing in blocks [{tr[0]},{tr[1]}))",
                      "value": round(t * 1e3, 2), "unit": "ms", "steps": args.steps,
                      "warmup": args.warmup, "higher_is_better": False, "kernels": kern}))


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


def _median_time(torch, fn, n, warmup=1):
    """Median over n separately synchronised calls (seconds)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2]


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
        blocks.append(h3k.quantize_block(wb, rowmajor=False))
        del wb
    x = S.activations(wl, device="cuda")
    c = S.conditioning(wl, device="cuda")
    dims = h3k.dims_of(wl)
    res, sweep, ref = {}, {}, None
    for tr in [(0, 0), wl.tr_range, (5, 45), (15, 35), (20, 30), (0, 50)]:
        log(f"stack step, pairing {tr}")
        ws = h3k.alloc_workspace(h3k.stack_workspace_bytes(dims, wl.L, *tr))
        y = torch.empty_like(x)
        nmed = 5 if tr in ((0, 0), tuple(wl.tr_range)) else 3
        t = _median_time(torch, lambda: h3k.stack_forward(x, c, blocks, dims, tr[0], tr[1], 0, ws, y), nmed)
        if tr in ((0, 0), tuple(wl.tr_range)):
            g = h3k.stack_graph(x, c, blocks, dims, tr[0], tr[1], 0, ws, y)
            tg = _median_time(torch, g.launch, 5)
            res["graph_" + ("token_reduction" if tr[1] > tr[0] else "full")] = round(tg * 1e3, 2)
            del g
        if tr == tuple(wl.tr_range):
            # one profiled step: per-kernel time of the whole step, and token pairing's bandwidth
            h3k.profile_enable(True)
            h3k.stack_forward(x, c, blocks, dims, tr[0], tr[1], 0, ws, y)
            torch.cuda.synchronize()
            prof = h3k.profile_read()
            h3k.profile_enable(False)
            step = {k: {"launches": n, "ms": round(tt, 3)} for k, (n, tt) in prof.items() if n}
            npair = wl.L // 2  # paired tokens
            for k, rd, wr in (("token_pair", 4 * wl.d, 4 * wl.d), ("token_unpair", 8 * wl.d, 4 * wl.d)):
                if k in step:
                    gbs = npair * (rd + wr) / (step[k]["ms"] * 1e-3) / 1e9
                    step[k].update(bytes=npair * (rd + wr), GBps=round(gbs, 1), frac_of_8TBps=round(gbs / HBM_GBS, 4))
            out["stack50_l16384_token_reduction_kernels"] = step
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

    log("precision series")
    # precision series (one block, L=16384)
    wl = S.WORKLOADS["block_l16384"]
    bw = h3k.quantize_block(S.block_weights_bf16(wl, 0, device="cuda"), keep_bf16=True)
    x = S.activations(wl, device="cuda")
    c = S.conditioning(wl, device="cuda")
    dims = h3k.dims_of(wl)
    series = {}
    for name, flags in [("bf16", h3k.F_BF16_GEMM), ("int8_mlp", h3k.F_BF16_QKV | h3k.F_BF16_OUT),
                        ("int8_mlp_qkv", h3k.F_BF16_OUT), ("w8a8", 0), ("w8a8_attn_bf16", h3k.F_ATTN_BF16)]:
        ws = h3k.alloc_workspace(h3k.workspace_bytes(dims, wl.L, flags))
        y = torch.empty_like(x)
        t = _median_time(torch, lambda: h3k.block_forward(x, c, bw, dims, flags, ws, y), 5, 2)
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
        log(f"sequence scaling L={L}")
        wl = dataclasses.replace(base, name=f"block_l{L}", grid=grid)
        bw = h3k.quantize_block(S.block_weights_bf16(wl, 0, device="cuda"), rowmajor=False)
        x = S.activations(wl, device="cuda")
        c = S.conditioning(wl, device="cuda")
        dims = h3k.dims_of(wl)
        ws = h3k.alloc_workspace(h3k.workspace_bytes(dims, L, 0))
        y = torch.empty_like(x)
        t = _median_time(torch, lambda: h3k.block_forward(x, c, bw, dims, 0, ws, y), 3, 1)
        h3k.profile_enable(True)
        _time_steps(torch, lambda: h3k.block_forward(x, c, bw, dims, 0, ws, y), 2, 0)
        prof = h3k.profile_read()
        h3k.profile_enable(False)
        n, tot = prof["attention"]
        attn_ms = tot / n
        frac = 4.0 * L * L * wl.d / (attn_ms * 1e-3) / 1e12 / PEAK["fp16"]
        scaling[str(L)] = {"ms": round(t * 1e3, 3), "attention_ms": round(attn_ms, 3),
                           "attention_frac": round(frac, 4)}
        if L == 65536:
            l65536 = {"ms_per_step": round(t * 1e3, 3), "tokens_per_s": round(L / t, 1),
                      "attention_ms": round(attn_ms, 3), "attention_frac": round(frac, 4)}
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
