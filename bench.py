"""Benchmark: WaterSIC layer quantization on one MI355X.

One step = the whole hot path on one layer whose inputs already sit in HBM:
    Sigma = X^T X / N  ->  Sigma = U^T U  ->  waterfilled SIC at the target rate (every pass of
    the rate controller)  ->  entropy of the codes  ->  distortion tr(E Sigma E^T).
Default workload: the attention-projection layer (W 4096 x 4096 bf16, X 8192 x 4096 bf16,
2 bits per weight). Metric: quantized weights per second (Gparams/s).

Prints one JSON line. `roofline` is taken for the kernel family with the largest share of the
step (found in the warm-up), from HIP events around its launches on the library's stream in the
last step of the timed region (no other launch carries events); `phases_ms` splits the step at the call
boundaries and `value_from_U` is the rate of the part that starts from U in HBM (waterfill +
entropy + distortion). `cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAKS = {
    "hbm": (8000.0, "GB/s"),
    "mfma_f64": (78.6, "TFLOP/s"),
    "mfma_f32": (157.3, "TFLOP/s"),
    "mfma_bf16": (2500.0, "TFLOP/s"),
    "mfma_i8": (5000.0, "TOP/s"),
    "valu_f64": (78.6, "TFLOP/s"),
}
# kernel family -> (bound, peak key, work unit scale to the peak's unit)
FAMILIES = {
    "gemm_trail_i8": ("mfma", "mfma_i8", 1e-12),
    "gemm_trail": ("mfma", "mfma_f64", 1e-12),
    "gemm_y": ("mfma", "mfma_f64", 1e-12),
    "gemm_chol": ("mfma", "mfma_f64", 1e-12),
    "chol_step": ("mfma", "mfma_f64", 1e-12),
    "potrf_panel": ("alu", "valu_f64", 1e-12),
    "gemm_dist": ("mfma", "mfma_f64", 1e-12),
    "syrk_bf16": ("mfma", "mfma_bf16", 1e-12),
    "sic_leaf": ("hbm", "hbm", 1e-9),
    "hist": ("hbm", "hbm", 1e-9),
    "dist_resid": ("hbm", "hbm", 1e-9),
    "logits_bf16": ("mfma", "mfma_bf16", 1e-12),
    "curvature": ("hbm", "hbm", 1e-9),
}


# algorithmic work per launch, as the library counts it for each family
WORK_UNITS = {
    "sic_leaf": "bytes: weights in (2 B bf16 / 4 B f32) + int32 codes out, per weight of the launch's "
                "columns; the design's intermediates (Y, G, residuals, int8 codes) are not counted",
    "hist": "bytes: 4 per int32 code read",
    "dist_resid": "bytes: 4 per fp32 residual read",
    "gemm_trail_i8": "int8 ops: 2 M N K per digit plane, 5 planes",
    "gemm_y": "fp64 flops: n_out n_in (n_in + 1) (triangular U)",
    "syrk_bf16": "flops: N n_in (n_in + 1) (upper triangle)",
    "chol_step": "fp64 flops of the step's update and panel",
}


def measured_traffic(family: str, workload: str):
    """HBM bytes per launch of `family` from the committed counter summary (rocprofv3
    FETCH_SIZE + WRITE_SIZE scaled by a plain copy), or None when there is none for this
    workload or the kernel's source has changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))["families"][family]
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (KeyError, OSError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="attn_4096")
    ap.add_argument("--target", type=float, default=2.0)
    ap.add_argument("--mode", default="auto", choices=["auto", "secant", "bisect"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=32)
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event timing")
    ap.add_argument("--softwater", action="store_true",
                    help="class-aware grids of a softmax head: class curvatures from the calibration "
                         "inputs, then waterfilling on c / (sqrt(lambda_k) U_jj) and the KL estimate")
    ap.add_argument("--rate-mode", default="pooled", choices=["pooled", "columns"],
                    help="rate held to the target: pooled code entropy, or the mean per-column entropy "
                         "(then the gap to the Gaussian limit is reported)")
    ap.add_argument("--coder-lane-symbols", type=int, default=1024,
                    help="codes per rANS stream for the entropy-coder measurement (0: skip it)")
    ap.add_argument("--smoothing", type=float, default=0.05,
                    help="weight of the uniform distribution mixed into the calibration softmax")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration records (every workload and target)")
    ap.add_argument("--configs-budget-s", type=float, default=360.0,
                    help="wall-clock budget of the whole run after which remaining configurations are skipped")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run one device-to-device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale the counters of
    the other kernels to bytes."""
    import torch

    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n}), flush=True)


def _blas_threads():
    """Threads the host BLAS actually runs with (what the oracle's numpy calls use)."""
    try:
        from threadpoolctl import threadpool_info

        n = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(layer, target, sample_rows):
    """The oracle as it stands, on the host's cores: full covariance and factorization of the
    layer's calibration data, one full SIC pass over every row of W at the oracle's own grid
    scale (its high-rate start), and the pass count of the oracle's search (bracketing +
    geometric bisection) taken from its run on `sample_rows` rows. The whole-layer time is
    covariance + Cholesky + passes x one full pass."""
    import numpy as np

    import oracle

    affinity = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    sigma = oracle.covariance(layer.x_chunks)
    t1 = time.perf_counter()
    L, info = oracle.cholesky_lower(sigma)
    t2 = time.perf_counter()
    c0 = oracle.initial_scale(layer.w, L, target)
    oracle.sic_quantize(layer.w, L, c0)
    t3 = time.perf_counter()
    rows = np.linspace(0, layer.n_out - 1, sample_rows).astype(np.int64)
    wf = oracle.waterfill(layer.w[rows], L, target)
    t4 = time.perf_counter()
    passes = len(wf["trace"])
    t_cov, t_chol, t_pass = t1 - t0, t2 - t1, t3 - t2
    t_full = t_cov + t_chol + passes * t_pass
    return {
        "value": layer.n_out * layer.n_in / t_full / 1e9,
        "unit": "Gparams/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": (f"measured: covariance ({t_cov:.2f} s) and Cholesky ({t_chol:.2f} s) of {layer.n_rows}x{layer.n_in}, "
                   f"one SIC pass over all {layer.n_out} rows ({t_pass:.2f} s); the oracle's search needs {passes} "
                   f"passes (its run on {sample_rows} rows, {t4 - t3:.2f} s), so the whole layer is "
                   f"{t_cov:.2f} + {t_chol:.2f} + {passes} x {t_pass:.2f} = {t_full:.1f} s"),
        "seconds": round(t4 - t0, 2),
        "affinity_cores": affinity,
    }


def cpu_baseline_softwater(layer, target, sample_rows, smoothing, curv_rows=64):
    """The SoftWater oracle on the host: full covariance and factorization, class curvatures on
    `curv_rows` calibration rows (scaled to all rows), the waterfill search on `sample_rows`
    classes (scaled to all classes)."""
    import numpy as np

    from oracle import softwater as sw
    from oracle import watersic as ws

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = _blas_threads()
    ctx = None
    try:
        t0 = time.perf_counter()
        sigma = ws.covariance(layer.x_chunks)
        t1 = time.perf_counter()
        L, info = ws.cholesky_lower(sigma)
        t2 = time.perf_counter()
        X0 = np.asarray(layer.x_chunks[0][:curv_rows], dtype=np.float64)
        lam = sw.softmax_curvature([X0], layer.w, smoothing)
        t3 = time.perf_counter()
        rows = np.linspace(0, layer.n_out - 1, sample_rows).astype(np.int64)
        wf = sw.waterfill(layer.w[rows], L, lam[rows], target)
        t4 = time.perf_counter()
    finally:
        if ctx is not None:
            ctx.unregister() if hasattr(ctx, "unregister") else None
    t_cov, t_chol, t_curv, t_wf = t1 - t0, t2 - t1, t3 - t2, t4 - t3
    t_full = t_cov + t_chol + t_curv * (layer.n_rows / curv_rows) + t_wf * (layer.n_out / sample_rows)
    return {
        "value": layer.n_out * layer.n_in / t_full / 1e9,
        "unit": "Gparams/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"full covariance ({t_cov:.2f} s) and Cholesky ({t_chol:.2f} s) of {layer.n_rows}x{layer.n_in}; "
                   f"class curvatures on {curv_rows} of {layer.n_rows} calibration rows ({t_curv:.2f} s, scaled "
                   f"by {layer.n_rows / curv_rows:.0f}); waterfill on {sample_rows} of {layer.n_out} classes "
                   f"({t_wf:.2f} s, {len(wf['trace'])} passes, scaled by {layer.n_out / sample_rows:.0f})"),
        "seconds": round(t_cov + t_chol + t_curv + t_wf, 2),
    }


# Per-configuration records of the default run: every named workload and target, the LM head
# also with SoftWater grids, and the large down-projection also with dead-feature removal and the
# LMMSE rescale. (workload, target, variant)
CONFIG_CASES = [
    ("ar1_256", 2.0, None),
    ("attn_4096", 1.0, None),
    ("attn_4096", 3.0, None),
    ("attn_4096", 4.0, None),
    ("mlp_up_11008x4096", 2.0, None),
    ("lmhead_32000x4096", 1.5, None),
    ("lmhead_32000x4096", 3.0, None),
    ("lmhead_32000x4096", 1.5, "softwater"),
    ("mlp_down_8192x28672", 2.0, None),
    ("mlp_down_8192x28672", 2.0, "dead_features+lmmse"),
]


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2] if len(xs) % 2 else 0.5 * (xs[len(xs) // 2 - 1] + xs[len(xs) // 2])


def run_case(L, torch, layer, W, X, target, variant, reps, smoothing=0.05, tau=1e-6):
    """One configuration, timed like the headline step (inputs in HBM; covariance -> Cholesky ->
    waterfill -> entropy -> distortion), `reps` timed steps after one warm-up; returns the
    median step time, the part from U on, passes and results."""
    dev = W.device
    n_out, n_in, n_rows = layer.n_out, layer.n_in, layer.n_rows
    sigma = torch.empty((n_in, n_in), dtype=torch.float64, device=dev)
    sw = variant == "softwater"
    fix = variant == "dead_features+lmmse"
    ws_cov = L.workspace(L.OP_COVARIANCE, 1, n_in, dev)
    ws_ent = L.workspace(L.OP_ENTROPY, n_out, n_in, dev)
    lam = torch.empty(n_out, dtype=torch.float64, device=dev) if sw else None
    ws_curv = L.workspace(L.OP_CURVATURE, max(int(c.shape[0]) for c in X), n_out, dev) if sw else None
    extra = {}

    def step(ev):
        ev[0].record()
        for i, c in enumerate(X):
            L.covariance(c, sigma, alpha=1.0 / n_rows, beta=0.0 if i == 0 else 1.0, ws=ws_cov)
        if fix:
            # dead features: columns with Sigma_ii <= tau max Sigma_jj are taken out before the
            # factorization and get code 0
            idx, pos, n_live = L.live_features(sigma, tau)
            Wq, Sq = L.gather_features(W, idx, n_live, sigma)
        else:
            Wq, Sq, n_live = W, sigma, n_in
        U, _ = L.cholesky(Sq)
        if sw:
            for i, c in enumerate(X):
                L.softmax_curvature(c, W, smoothing, lam, alpha=1.0 / n_rows, beta=0.0 if i == 0 else 1.0,
                                    ws=ws_curv)
        ev[1].record()
        if sw:
            wf = L.softwater_waterfill(Wq, U, lam, target)
            h, _ = L.entropy(wf["codes"], ws=ws_ent)
            D, _ = L.softwater_distortion(wf["codes"], U, wf["c"], lam, wf["resid"])
        else:
            wf = L.waterfill(Wq, U, target)
            h, _ = L.entropy(wf["codes"], ws=ws_ent)
            D, _ = L.distortion(Wq, wf["codes"], U, wf["c"], resid=wf["resid"])
        if fix:
            q_full = L.scatter_codes(wf["codes"], pos, n_in)
            gamma, d_before, d_after = L.lmmse_scale(Wq, U, wf["resid"])
            extra.update(n_live=n_live, n_dead=n_in - n_live, tau=tau, D_before_lmmse=d_before,
                         D_after_lmmse=d_after, gamma_min=float(gamma.min()), gamma_max=float(gamma.max()))
            del q_full
        ev[2].record()
        return wf, h, D

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    step(ev)  # warm-up
    torch.cuda.synchronize()
    times, from_u = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        wf, h, D = step(ev)
        torch.cuda.synchronize()
        times.append(1e3 * (time.perf_counter() - t0))
        from_u.append(ev[1].elapsed_time(ev[2]))
    ms, ms_u = _median(times), _median(from_u)
    rec = {"workload": layer.name, "target_bits": target, "variant": variant, "n_out": n_out, "n_in": n_in,
           "calib_rows": n_rows, "reps": reps, "ms_per_step": round(ms, 3),
           "ms_steps": [round(t, 3) for t in times], "gparams_s": round(n_out * n_in / (ms * 1e-3) / 1e9, 4),
           "ms_from_U": round(ms_u, 3), "gparams_s_from_U": round(n_out * n_in / (ms_u * 1e-3) / 1e9, 4),
           "passes": wf["passes"], "c": wf["c"], "rate": wf["rate"], "entropy": h, "D": D}
    rec.update(extra)
    return rec


def config_records(args, L, torch, headline_layer, headline_W, headline_X, t_start, budget_s):
    """Every case of CONFIG_CASES except the headline one, within a wall-clock budget."""
    from rate_allocated_weight_amd import workloads

    dev = torch.device("cuda:0")
    out = []
    cur = (None, None, None, None)
    for name, target, variant in CONFIG_CASES:
        if name == args.workload and target == args.target and variant is None:
            continue
        if time.perf_counter() - t_start > budget_s:
            out.append({"workload": name, "target_bits": target, "variant": variant,
                        "skipped": f"wall-clock budget of {budget_s:.0f} s reached"})
            continue
        try:
            if cur[0] != name:
                cur = (None, None, None, None)
                torch.cuda.empty_cache()
                if name == headline_layer.name:
                    cur = (name, headline_layer, headline_W, headline_X)
                else:
                    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
                    lay = workloads.named_workload(name)
                    if lay.dtype == "bf16":
                        Wd = L.bf16_from_bits(lay.w_bits, dev)
                        Xd = [L.bf16_from_bits(b, dev) for b in lay.x_bits_chunks]
                    else:
                        Wd = torch.from_numpy(lay.w).to(dev)
                        Xd = [torch.from_numpy(c).to(dev) for c in lay.x_chunks]
                    cur = (name, lay, Wd, Xd)
            reps = 2 if cur[1].n_in > 8192 else 3
            print(f"[bench] case {name} R={target} {variant or ''}", file=sys.stderr, flush=True)
            out.append(run_case(L, torch, cur[1], cur[2], cur[3], target, variant, reps,
                                smoothing=args.smoothing))
        except Exception as e:  # a failing case is reported, it does not take the line down
            out.append({"workload": name, "target_bits": target, "variant": variant, "error": str(e)})
    return out


def main():
    t_start = time.perf_counter()
    args = parse()
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(rows of W would shard across GPUs with U replicated; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rate_allocated_weight_amd import _lib as L
    from rate_allocated_weight_amd import workloads

    dev = torch.device("cuda:0")
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    layer = workloads.named_workload(args.workload)
    if layer.dtype == "bf16":
        W = L.bf16_from_bits(layer.w_bits, dev)
        X = [L.bf16_from_bits(b, dev) for b in layer.x_bits_chunks]
    else:
        W = torch.from_numpy(layer.w).to(dev)
        X = [torch.from_numpy(c).to(dev) for c in layer.x_chunks]
    n_out, n_in = layer.n_out, layer.n_in
    n_rows = layer.n_rows

    # buffers allocated once
    sigma = torch.empty((n_in, n_in), dtype=torch.float64, device=dev)
    codes = torch.empty((n_out, n_in), dtype=torch.int32, device=dev)
    resid = torch.empty((n_out, n_in), dtype=torch.float32, device=dev)
    ws_cov = L.workspace(L.OP_COVARIANCE, 1, n_in, dev)
    ws_chol = L.workspace(L.OP_CHOLESKY, 1, n_in, dev)
    ws_wf = L.workspace(L.OP_WATERFILL, n_out, n_in, dev)
    ws_ent = L.workspace(L.OP_ENTROPY_COLUMNS if args.rate_mode == "columns" else L.OP_ENTROPY, n_out, n_in, dev)
    ws_dist = L.workspace(L.OP_DISTORTION, n_out, n_in, dev)
    sw = args.softwater
    if sw:
        ws_wf = L.workspace(L.OP_SOFTWATER, n_out, n_in, dev)
        ws_dist = L.workspace(L.OP_SOFTWATER_DIST, n_out, n_in, dev)
        ws_curv = L.workspace(L.OP_CURVATURE, max(int(c.shape[0]) for c in X), n_out, dev)
        lam = torch.empty(n_out, dtype=torch.float64, device=dev)

    # phase boundaries on the library's stream (the current torch stream)
    phase_names = ("covariance", "cholesky", "curvature", "waterfill", "entropy+distortion")
    phase_ms = {k: 0.0 for k in phase_names}
    phase_events = []

    def step(record=False):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)] if record else None
        if record:
            ev[0].record()
        for i, c in enumerate(X):
            L.covariance(c, sigma, alpha=1.0 / n_rows, beta=0.0 if i == 0 else 1.0, ws=ws_cov)
        if record:
            ev[1].record()
        U, _ = L.cholesky(sigma, ws=ws_chol)
        if record:
            ev[2].record()
        if sw:
            for i, c in enumerate(X):
                L.softmax_curvature(c, W, args.smoothing, lam, alpha=1.0 / n_rows, beta=0.0 if i == 0 else 1.0,
                                    ws=ws_curv)
        if record:
            ev[3].record()
        if sw:
            wf = L.softwater_waterfill(W, U, lam, args.target, mode=args.mode, codes=codes, resid=resid,
                                       ws=ws_wf)
        else:
            wf = L.waterfill(W, U, args.target, mode=args.mode, codes=codes, resid=resid, ws=ws_wf,
                             rate_mode=args.rate_mode)
        if record:
            ev[4].record()
        if sw:
            h, _ = L.entropy(wf["codes"], ws=ws_ent)
            D, _ = L.softwater_distortion(wf["codes"], U, wf["c"], lam, wf["resid"], ws=ws_dist)
        elif args.rate_mode == "columns":
            h = L.entropy_columns(codes, ws=ws_ent)
            D, _ = L.distortion(W, codes, U, wf["c"], resid=resid, ws=ws_dist)
        else:
            h, _ = L.entropy(codes, ws=ws_ent)
            D, _ = L.distortion(W, codes, U, wf["c"], resid=resid, ws=ws_dist)
        if record:
            ev[5].record()
            phase_events.append(ev)
        return wf, h, D

    # warm-up; with profiling on, it also finds the kernel family with the largest share, the
    # only one whose launches carry events in the timed region
    dom = None
    if not args.no_profile:
        L.profile_select(None)
        L.profile_reset()
        L.profile_enable(True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def dominant():
        cand = [(k, L.profile_read(k)["ms"]) for k in L.profile_names() if k in FAMILIES]
        return max(cand, key=lambda kv: kv[1])[0] if cand else None

    # every family's rate against its own peak, from the warm-up step (all families evented)
    families = {}
    if not args.no_profile and args.warmup > 0:
        for name in L.profile_names():
            if name not in FAMILIES:
                continue
            p = L.profile_read(name)
            bound, peak_key, scale = FAMILIES[name]
            peak, unit = PEAKS[peak_key]
            ach = p["work"] * scale / max(1e-12, p["ms"] * 1e-3)
            families[name] = {"ms_per_step": round(p["ms"] / args.warmup, 4), "launches": p["launches"],
                              "achieved": round(ach, 3), "peak": peak, "unit": unit,
                              "frac": round(ach / peak, 4)}
    trailing = None
    if "gemm_trail_i8" in families:
        # the interference (trailing update) runs as an exact int8 digit-plane product: its own
        # rate is against the int8 peak; beside it, how long the algorithmic product (2 M N K
        # flops, one fifth of its int8 ops) would take at the fp32 MFMA peak, over its time
        f = families["gemm_trail_i8"]
        tf = f["achieved"] / 5.0
        trailing = {"kernel": "gemm_trail_i8", "achieved_int8_tops": f["achieved"],
                    "peak_int8_tops": PEAKS["mfma_i8"][0], "frac_of_int8_peak": f["frac"],
                    "algorithmic_tflops": round(tf, 2),
                    "fp32_peak_time_over_measured": round(tf / PEAKS["mfma_f32"][0], 4),
                    "note": "GEMM part only (above the 512-column super-blocks; the product inside the "
                            "super-block launches is part of sic_leaf). fp32_peak_time_over_measured > 1: "
                            "the product finishes faster than an fp32 GEMM at peak could"}

    if not args.no_profile:
        L.profile_enable(False)
        if args.warmup > 0:
            dom = dominant()
        L.profile_reset()
        L.profile_select([dom] if dom else None)  # no warm-up: every family is timed
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    results = []
    for i in range(args.steps):
        # the dominant family's launches carry their events in the last timed step only: an
        # evented launch costs a few microseconds more, which would otherwise weigh on every step
        if not args.no_profile and i == args.steps - 1:
            L.profile_enable(True)
        results.append(step(record=True))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not args.no_profile:
        L.profile_enable(False)
        L.profile_select(None)
    elapsed = t1 - t0
    ms_per_step = 1e3 * elapsed / args.steps
    wf, h, D = results[-1]
    it_gap = None
    if args.rate_mode == "columns" and not sw:
        # after the timed region: the high-rate Gaussian limit at this distortion (the factor U of
        # the last step is still in sigma)
        rg, var = L.gaussian_rate(W, sigma, D)
        it_gap = {"rate_columns": wf["rate"], "gaussian_rate": rg, "gap_bits": wf["rate"] - rg,
                  "uniform_scalar_gap_bits": 0.5 * math.log2(2 * math.pi * math.e / 12),
                  "var_w": var, "theta": D / (n_out * n_in),
                  "note": "Gaussian model of the rows with the weights' variance, high-rate form of "
                          "reverse waterfilling (exact while theta is below var * min eig Sigma)"}
    for ev in phase_events:
        for k, name in enumerate(phase_names):
            phase_ms[name] += ev[k].elapsed_time(ev[k + 1]) / args.steps
    ms_from_u = phase_ms["curvature"] + phase_ms["waterfill"] + phase_ms["entropy+distortion"]

    # the codes of the last step through the entropy coder (after the timed region): the rate the
    # coder actually writes against the empirical entropy, and its encode / decode times
    coder = None
    if args.coder_lane_symbols > 0:
        try:
            cc = (wf["codes"] if sw else codes).contiguous()
            n = cc.numel()
            Ls = args.coder_lane_symbols
            ws_enc = L.workspace(L.OP_RANS_ENC, Ls, n, dev)
            ws_dec = L.workspace(L.OP_RANS_DEC, 1, n_in, dev)
            cap = int(L.lib().wsic_rans_bound(n, Ls))
            blob = torch.empty(cap, dtype=torch.uint8, device=dev)
            back = torch.empty_like(cc)
            w16 = torch.empty((n_out, n_in), dtype=torch.bfloat16, device=dev)

            def timed(fn, reps=5):
                fn()
                torch.cuda.synchronize()
                t = time.perf_counter()
                for _ in range(reps):
                    r = fn()
                torch.cuda.synchronize()
                return r, 1e3 * (time.perf_counter() - t) / reps

            (_, nb), t_enc = timed(lambda: L.rans_encode(cc, Ls, out=blob, ws=ws_enc))
            _, t_dec = timed(lambda: L.rans_decode(blob, nb, n, out=back, ws=ws_dec))
            t_dq = None
            if not sw:  # (the class-aware grids of SoftWater need their row scales: not timed here)
                _, t_dq = timed(lambda: L.rans_decode_dequant(blob, nb, n_out, n_in, sigma, wf["c"], out=w16,
                                                              ws=ws_dec))
            ok = bool(torch.equal(back, cc))
            coder = {"lane_symbols": Ls, "bytes": nb, "bits_per_code": 8.0 * nb / n, "entropy_bits": wf["rate"],
                     "excess_bits": 8.0 * nb / n - wf["rate"], "lossless": ok, "encode_ms": round(t_enc, 4),
                     "decode_ms": round(t_dec, 4),
                     "decode_to_bf16_ms": round(t_dq, 4) if t_dq is not None else None,
                     "decode_codes_GBps": round(4.0 * n / (t_dec * 1e-3) / 1e9, 2),
                     "decode_bf16_GBps": round(2.0 * n / (t_dq * 1e-3) / 1e9, 2) if t_dq is not None else None,
                     "note": "API calls timed with host clocks (each reads the container header back first)"}
            if not sw and args.rate_mode == "columns":
                coder["entropy_bits"] = None  # the step's rate is per column; the coder uses one table
        except Exception as e:  # the measurement never takes the benchmark down
            coder = {"error": str(e)}

    kernels = {}
    roofline = None
    if not args.no_profile:
        if dom is None:
            dom = dominant()
        for name in L.profile_names():
            p = L.profile_read(name)
            kernels[name] = {"launches": p["launches"], "ms": round(p["ms"], 4),
                             "avg_us": round(1e3 * p["ms"] / max(1, p["launches"]), 3), "work": p["work"]}
        if dom in kernels:
            v = kernels[dom]
            bound, peak_key, scale = FAMILIES[dom]
            peak, unit = PEAKS[peak_key]
            achieved = v["work"] * scale / (v["ms"] * 1e-3)
            traffic = measured_traffic(dom, args.workload)
            roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                        "frac": round(achieved / peak, 4),
                        "traffic": round(traffic) if traffic is not None else None,
                        "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                        "work_per_launch": v["work"] / max(1, v["launches"]),
                        "work_unit": WORK_UNITS.get(dom, ""),
                        "traffic_over_algorithmic": (round(traffic / (v["work"] / max(1, v["launches"])), 3)
                                                     if traffic is not None and bound == "hbm" else None),
                        "avg_launch_us": v["avg_us"], "launches": v["launches"],
                        # the events cover one timed step
                        "share_of_step": round(v["ms"] / ms_per_step, 4)}

    if sw:
        metric = (f"Gparams/s SoftWater class-aware waterfill+SIC ({n_out}x{n_in} softmax head, "
                  f"{args.target:g} bit/param); % MFMA/HBM roofline")
        step_name = "covariance+cholesky+class curvatures+class-aware waterfill+entropy+KL distortion"
    else:
        metric = "Gparams/s waterfill+SIC quantize (4096x4096, 2 bit/param); % MFMA/HBM roofline"
        step_name = "covariance+cholesky+waterfill+entropy+distortion"
    if not sw:
        phase_ms.pop("curvature")
    out = {
        "metric": metric,
        "value": round(n_out * n_in * args.steps / elapsed / 1e9, 6),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_out": n_out, "n_in": n_in, "calib_rows": n_rows,
                   "w_dtype": layer.dtype, "target_bits": args.target, "controller": args.mode,
                   "step": step_name, **({"smoothing": args.smoothing} if sw else {})},
        "result": {"c": wf["c"], "rate": wf["rate"], "entropy": h, "passes": wf["passes"], "D": D},
        "phases_ms": {k: round(v, 4) for k, v in phase_ms.items()},
        "value_from_U": round(n_out * n_in / (ms_from_u * 1e-3) / 1e9, 6),
        "roofline": roofline,
        "kernels": kernels,
        "families_warmup": families,
        "trailing_update": trailing,
        "entropy_coder": coder,
    }
    if it_gap is not None:
        out["it_gap"] = it_gap
        out["config"]["rate_mode"] = "columns"
    if not args.no_configs and not sw and args.rate_mode == "pooled":
        del codes, resid, ws_wf, ws_ent, ws_dist
        out["configs"] = config_records(args, L, torch, layer, W, X, t_start, args.configs_budget_s)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = (cpu_baseline_softwater(layer, args.target, args.cpu_sample_rows, args.smoothing)
                               if sw else cpu_baseline(layer, args.target, args.cpu_sample_rows))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
