"""Benchmark: stabilised BF16 attention forward + backward on one MI355X.

One step = one forward (fa_fwd) and one backward (fa_bwd) over a fixed synthetic batch already
resident in HBM.  Default workload: the LLaMA-7B-shaped attention layer (B=1, H=32, N=8192,
d=128, causal, scale 1/sqrt(128)), tie-conditional stabilised shift (stable_flag=1, beta=1.25).

Throughput uses the FlashAttention flop convention: forward 4*B*H*N^2*d (halved when causal),
backward 2.5x the forward.  Per-kernel durations are measured with HIP events on the stream the
kernels are launched on.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd & fwd+bwd (bf16, % MFMA peak), N=8192 d=128 causal"
# MI355X published peaks: dense bf16 (and fp16) MFMA and HBM3E bandwidth.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4, help="workload id (1-5)")
    ap.add_argument("--mode", type=int, default=1, help="stable_flag: 0, 1 or 2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8pv", action="store_true",
                    help="also time the FP8 P^V forward (fa_fwd_fp8pv on the same bf16 inputs); off by "
                         "default: with its V pre-pass it runs a few percent slower than the bf16 forward")
    ap.add_argument("--no-fp8pv", action="store_true", help=argparse.SUPPRESS)  # the default now
    ap.add_argument("--no-f16", action="store_true",
                    help="skip the fp16 leg (the same workload with fp16 inputs, reported beside "
                         "the bf16 headline)")
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (to scale HBM "
                         "traffic counters against a transfer of known size)")
    return ap.parse_args()


# Kernel -> the sources that define it.  HBM traffic figures recorded under profiles/ carry the
# digest of these files at the time the counters were taken; a figure whose digest no longer
# matches describes an older kernel and is not reported.
KERNEL_SOURCES = {
    "fwd": ("fa_fwd.hip", "fa_common.hpp", "fa_launch.hpp"),
    "delta": ("fa_bwd.hip", "fa_common.hpp", "fa_launch.hpp"),
    "dkdv": ("fa_bwd.hip", "fa_common.hpp", "fa_launch.hpp"),
    "dq": ("fa_bwd.hip", "fa_common.hpp", "fa_launch.hpp"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama7b_N8192_d128_causal.md")


def sources_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "precision_numerical_stability_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch from the counter summary, if it was taken on the current sources."""
    import re
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    digest = sources_digest(kernel)
    for m in re.finditer(r"^\|\s*(\w+)\s*\|\s*([0-9a-f]{16})\s*\|[^|]*\|[^|]*\|\s*([0-9.]+)\s*\|", text, re.M):
        if m.group(1) == kernel and m.group(2) == digest:
            return float(m.group(3)) * 1e6
    return None


def time_events(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters  # ms


def cpu_baseline(cfg, t, mode, gpu, budget_s=15.0):
    """The fp64 oracle, as it stands, on whole heads of the workload (forward + backward), head
    after head until about budget_s seconds of host time have been spent (at least one head).
    The heads it computes also serve as the parity check of the timed step's own outputs (`gpu`:
    host copies of o, lse, dq, dk, dv taken right after the timed region, plus the repeat counts
    and the shift from one diagnostics call): the worst errors against the oracle are reported
    beside the timing."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing or no BLAS pool reported
        threads = os.cpu_count() or 1
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    done = 0
    worst = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0, "m": 0.0}
    rows_differ = 0
    rows = 0
    t0 = time.perf_counter()
    t_oracle = 0.0
    for b, h in heads:
        x = {k: v[b, h].to(torch.float64).numpy() for k, v in t.items()}
        t1 = time.perf_counter()
        fr = oracle.forward(x["q"], x["k"], x["v"], cfg.causal, cfg.scale, 1.25, mode)
        br = oracle.backward(x["q"], x["k"], x["v"], x["do"], cfg.causal, cfg.scale, o=fr.o, lse=fr.lse)
        t_oracle += time.perf_counter() - t1
        assert np.isfinite(fr.o).all()
        # O: worst excess over the 1e-2 + 1e-2 |ref| bar, in units of the bar (<= 1 passes)
        o_g = gpu["o"][b, h]
        worst["o"] = max(worst["o"], float(np.max(np.abs(o_g - fr.o) / (1e-2 + 1e-2 * np.abs(fr.o)))))
        worst["lse"] = max(worst["lse"], float(np.max(np.abs(gpu["lse"][b, h] - fr.lse))))
        for key, ref in (("dq", br.dq), ("dk", br.dk), ("dv", br.dv)):
            worst[key] = max(worst[key], float(np.max(np.abs(gpu[key][b, h] - ref)) / np.abs(ref).max()))
        # Repeat counts are decided on the kernel's fp32 dot products; on inputs whose dot products
        # are not exact in fp32 a near-tie can round into a tie (or out of one), so the rows whose
        # counts differ are reported, and the shift is compared where the counts agree.
        same = gpu["dup"][b, h] == fr.rs
        rows_differ += int((~same).sum())
        rows += same.size
        rel = np.abs(gpu["m"][b, h] - fr.m) / np.maximum(np.abs(fr.m), 1e-30)
        worst["m"] = max(worst["m"], float(rel[same].max(initial=0.0)))
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    flops = 3.5 * fwd_flops(1, done, cfg.N, cfg.d, cfg.causal)
    parity = {"heads_checked": done,
              "o_max_err_over_bar": worst["o"], "lse_max_abs_err": worst["lse"],
              "dq_max_err_rel_max": worst["dq"], "dk_max_err_rel_max": worst["dk"],
              "dv_max_err_rel_max": worst["dv"],
              "dupcnt_rows_checked": rows, "dupcnt_rows_differing": rows_differ,
              "shift_m_max_rel_err_where_counts_agree": worst["m"],
              "pass": bool(worst["o"] <= 1.0 and worst["lse"] <= 1e-3 and
                           max(worst["dq"], worst["dk"], worst["dv"]) <= 3e-2)}
    return {"value": flops / t_oracle / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads (b, h in order from 0, 0), forward+backward, "
                      f"fp64 numpy on {threads} BLAS threads, {t_oracle:.1f} s of oracle time",
            "parity_of_timed_step": parity}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the attention heads of "
              "this workload shard across GPUs without communication, so the figure that matters "
              "is the one-GPU kernel on its share of the heads (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import precision_numerical_stability_amd as fa
    from inputs import CONFIGS, make_inputs, tensor_digest

    cfg = CONFIGS[args.config]
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    t = make_inputs(cfg)
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    causal, scale, mode = cfg.causal, cfg.scale, args.mode

    def run_fwd(m=mode):
        fa.fa_fwd(q, k, v, o, lse, causal, scale, 1.25, m, stream=stream)

    def run_stage(stages):
        return lambda: fa.fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, delta, causal, scale,
                                    stages=stages, stream=stream)

    def step(m=mode):
        run_fwd(m)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, causal, scale, stream=stream)

    # Per-kernel durations first (separate loops, same stream; they also bring the GPU to its
    # steady clock before the step is timed).  "dq" is the dQ kernel as the full backward runs it
    # (delta formed in its prologue); "delta" is the standalone delta stage, whose O and dO reads
    # may partly hit the last-level cache when run back to back.
    it = args.kernel_iters
    for _ in range(3):
        step()
    ms_fwd_mode = {str(m): time_events(lambda m=m: run_fwd(m), it, stream) for m in (0, 1, 2)}
    ms_fwd = ms_fwd_mode[str(mode)]
    ms_delta = time_events(run_stage(fa.FA_BWD_DELTA), it, stream)
    ms_dkdv = time_events(run_stage(fa.FA_BWD_DKDV), it, stream)
    ms_dq = time_events(run_stage(fa.FA_BWD_DELTA | fa.FA_BWD_DQ), it, stream)

    # The step: W untimed warm-up steps, then exactly K timed steps.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    # The timed step's own outputs, for the parity check against the oracle (cpu_baseline leg).
    gpu_out = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.float().cpu().numpy(),
               "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
    assert all(np.isfinite(x).all() for x in gpu_out.values())
    # Repeat counts and the rule's shift of the same forward (one diagnostics call, untimed).
    dup_t = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    msh_t = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o_d = torch.empty_like(q)
    lse_d = torch.empty_like(lse)
    fa.fa_fwd_diag(q, k, v, o_d, lse_d, dup_t, None, None, None, msh_t, int(causal), scale, 1.25, mode,
                   stream=stream)
    torch.cuda.synchronize()
    gpu_out["dup"] = dup_t.cpu().numpy()
    gpu_out["m"] = msh_t.cpu().numpy()
    del dup_t, msh_t, o_d, lse_d

    # The whole step in the other stabilised mode (the backward does not depend on the mode).
    other = 2 if mode != 2 else 1
    for _ in range(args.warmup):
        step(other)
    ms_step_other = time_events(lambda: step(other), args.steps, stream)
    run_fwd()
    # Device-to-device copy rate, the attainable HBM figure the delta stage is set against.
    csrc_t = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    cdst_t = torch.empty_like(csrc_t)
    cdst_t.copy_(csrc_t)
    ms_copy = time_events(lambda: cdst_t.copy_(csrc_t), 5, stream)
    copy_gbs = 2 * csrc_t.numel() * 4 / (ms_copy * 1e-3) / 1e9
    del csrc_t, cdst_t
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ff = fwd_flops(B, H, N, d, causal)
    total = 3.5 * ff

    # FP8 P^V leg: the forward with its P^ V product in E4M3 (V quantised per 128-key block by the
    # library's pre-pass, which runs inside the timed call), on the same bf16 inputs.
    fp8pv = None
    if args.fp8pv and not args.no_fp8pv:
        ws8 = torch.empty(fa.fa_fwd_fp8pv_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        o8 = torch.empty_like(q)

        def fwd8():
            fa.fa_fwd_fp8pv(q, k, v, o8, lse, None, None, None, None, ws8, int(causal), scale, 1.25,
                            mode, stream=stream)

        for _ in range(args.warmup):
            fwd8()
        ms8 = time_events(fwd8, it, stream)
        ms_bf = time_events(run_fwd, it, stream)  # the bf16 forward in the same stretch
        torch.cuda.synchronize()
        assert torch.isfinite(o8.float()).all()
        fp8pv = {"fwd_ms": ms8, "fwd_TFLOP/s": ff / (ms8 * 1e-3) / 1e12,
                 "fwd_frac_bf16_peak": ff / (ms8 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "bf16_fwd_ms_same_stretch": ms_bf,
                 "max_abs_diff_to_bf16_O": float((o8.float() - o.float()).abs().max())}
        del ws8, o8
        run_fwd()  # restore this mode's lse

    # fp16 leg: the same draws rounded to fp16 (fa_fwd_elem / fa_bwd_elem), whole step and
    # forward alone, after the bf16 measurements.
    f16 = None
    if not args.no_f16:
        del g, q, k, v, do
        t16 = make_inputs(cfg, dtype=torch.float16)
        h = {k_: v_.to(dev) for k_, v_ in t16.items()}
        o16 = torch.empty_like(h["q"])
        dq16, dk16, dv16 = (torch.empty_like(h["q"]) for _ in range(3))

        def fwd16():
            fa.fa_fwd_elem(h["q"], h["k"], h["v"], o16, lse, None, None, None, None, int(causal),
                           scale, 1.25, mode, stream=stream)

        def step16():
            fwd16()
            fa.fa_bwd_elem(h["q"], h["k"], h["v"], o16, lse, h["do"], dq16, dk16, dv16, delta,
                           int(causal), scale, stream=stream)

        for _ in range(args.warmup):
            step16()
        torch.cuda.synchronize()
        ms16 = time_events(step16, args.steps, stream)
        ms16_fwd = time_events(fwd16, it, stream)
        torch.cuda.synchronize()
        assert torch.isfinite(o16.float()).all() and torch.isfinite(dq16.float()).all()
        f16 = {"ms_per_step": ms16, "fwdbwd_TFLOP/s": total / (ms16 * 1e-3) / 1e12,
               "fwdbwd_frac_f16_peak": total / (ms16 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "fwd_ms": ms16_fwd, "fwd_TFLOP/s": ff / (ms16_fwd * 1e-3) / 1e12,
               "fwd_frac_f16_peak": ff / (ms16_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del h, o16, dq16, dk16, dv16
    value = total / (ms_step * 1e-3) / 1e12
    fwd_tf = ff / (ms_fwd * 1e-3) / 1e12
    pairs = B * H * (N * (N + 1) // 2 if causal else N * N)
    # Algorithmic work per kernel: forward 4d flop per visible pair (two contractions); the dK/dV
    # kernel 8d (S recompute, dP, dV, dK); the dQ kernel 2d (dQ; its S and dP recomputes are
    # extra work); delta reads O and dO and writes one fp32 per row.
    alg = {
        "fwd": ("mfma", ff, ms_fwd),
        "dkdv": ("mfma", 2.0 * ff, ms_dkdv),
        "dq": ("mfma", 0.5 * ff, ms_dq),
        "delta": ("hbm", 2.0 * B * H * N * d * 2 + B * H * N * 4, ms_delta),
    }
    ms_by_kernel = {"fwd": ms_fwd, "delta": ms_delta, "dkdv": ms_dkdv, "dq": ms_dq}
    dom = max(ms_by_kernel, key=ms_by_kernel.get)
    bound, work, ms = alg[dom]
    if bound == "mfma":
        achieved = work / (ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": recorded_traffic(dom)}
    else:
        achieved = work / (ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": recorded_traffic(dom)}
    kernels = {}
    for name, (bnd, work_k, ms_k) in alg.items():
        if bnd == "mfma":
            tf = work_k / (ms_k * 1e-3) / 1e12
            kernels[name] = {"ms": ms_k, "TFLOP/s": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS}
        else:
            gbs = work_k / (ms_k * 1e-3) / 1e9
            kernels[name] = {"ms": ms_k, "GB/s": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                             "frac_measured_copy": gbs / copy_gbs, "cache_inclusive": True}
    kernels["dq"]["note"] = "delta formed in the dQ kernel, as in the full backward"
    fwd_modes = {m: {"ms": t_, "TFLOP/s": ff / (t_ * 1e-3) / 1e12,
                     "frac_bf16_peak": ff / (t_ * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
                 for m, t_ in ms_fwd_mode.items()}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} attention layer", "B": B, "H": H, "N": N, "d": d,
                   "causal": causal, "scale": scale, "stable_flag": mode, "beta": 1.25,
                   "seed": cfg.seed, "q_sha256": tensor_digest(t["q"])[:16]},
        "fwd_tflops": fwd_tf,
        "fwd_frac_peak": fwd_tf / PEAK_BF16_TFLOPS,
        "fwdbwd_tflops": value,
        "fwdbwd_frac_peak": value / PEAK_BF16_TFLOPS,
        "fwd_by_stable_flag": fwd_modes,
        "fwdbwd_by_stable_flag": {
            str(mode): {"ms": ms_step, "TFLOP/s": value, "frac_bf16_peak": value / PEAK_BF16_TFLOPS},
            str(other): {"ms": ms_step_other, "TFLOP/s": total / (ms_step_other * 1e-3) / 1e12,
                         "frac_bf16_peak": total / (ms_step_other * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}},
        "d2d_copy_GB/s": copy_gbs,
        "exact_causal_pairs": pairs,
        "kernels": kernels,
        "roofline": roof,
    }
    if f16 is not None:
        out["f16"] = f16
    if fp8pv is not None:
        out["fp8pv"] = fp8pv
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, t, mode, gpu_out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
