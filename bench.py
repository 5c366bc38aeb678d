"""Throughput of the mapper apply step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]

A step is one kvmap_apply over the whole cache: de-rotation of the selected source key
layers, then the map GEMM for K and V of every target layer with bias and target RoPE
fused.  Inputs are synthetic, seeded, and resident in HBM before timing starts.  Prints
one JSON line (rank 0).

value      mapped tokens/s: T tokens of the cache (K and V, all target layers) per step
roofline   the map GEMM launch: algorithmic FLOP (2*T*F*N per target layer, K and V) over its
           average duration from HIP events recorded on the apply's stream, against the
           bf16 dense MFMA peak; traffic from the committed rocprofv3 counter summary if it
           was taken on the current kernel source
cpu_baseline  the fp64 oracle on a bounded sample of the same workload, on the host cores
recode     kvmap_recode (identity map: RoPE re-encode, one rotation per pair) of the workload's
           whole source key cache, timed with HIP events; GB/s against the 8 TB/s HBM peak
fit        the fit side on its own workload (262,144 calibration tokens, p 8192, q 1024, batches of
           4096): one kvmap_gram call per batch (shift, hi/lo split, co-moments, Chan merge), 64
           calls timed with HIP events on its stream after at least 0.3 s of warm-up calls; one
           ridge solve of the merged state on the host and one on the device (fp64, W written in
           bf16 output-major)
short      kvmap_apply on the first T tokens (T = 1 .. 8192) with the workload's maps: ms against the
           larger of the HBM roofline (W and the rows) and the matrix-core roofline
fit_driver the complete fit (layer selection, then the maps) at the 14B->32B model shape over
           --fit-seqs seeded calibration sequences of 4096 tokens: wall seconds per pass
library_gemm  context for the roofline: the vendor BLAS (torch.matmul, hipBLASLt on ROCm) on the
           plain GEMMs of the same shape and data -- the first target layer's gathered,
           de-rotated feature rows [T][F] times each of the 2 x L_tgt maps, bf16 in and out with
           fp32 accumulation, no gather, bias or RoPE -- timed with HIP events, against the same
           bf16 dense peak
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mapped tokens/s (K+V, all target layers) at 14B→32B shape; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12     # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0
PEAK_FP32_MFMA_TFLOPS = 157.3                    # dense fp32 matrix peak
PEAK_FP16_TFLOPS = PEAK_BF16_TFLOPS              # dense fp16 matrix peak (same as bf16)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "map_bf16_traffic.json")
DEROPE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "derope_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def traffic_entry(cfg_name, path=TRAFFIC_FILE, kernel="map_bf16_kernel"):
    """HBM bytes per launch of a kernel from its committed counter summary, if that summary was
    taken on the kernel's current code and this workload; else None."""
    from cross_model_kv_amd.profiling import KERNEL_SOURCES, kernel_fingerprint
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel") != kernel or t.get("kernel_code_fingerprint") != kernel_fingerprint(KERNEL_SOURCES[kernel])
            or t.get("workload") != cfg_name):
        return None
    return t.get("hbm_bytes_per_launch")


def host_cpu() -> dict:
    """The host's CPU model and logical CPU count, reported beside the oracle's timing."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count()}


def cpu_baseline(cfg, inp, budget_s=12.0):
    """Time the fp64 oracle on whole target layers over the first `rows` tokens until the budget
    is spent; scale to mapped tokens/s of the full workload (all target layers)."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    rows = np.arange(min(cfg.T, 2048))
    rows_t = torch.as_tensor(rows, device="cuda:0")
    f = lambda t: t.float().cpu().double().numpy()
    sel = inp["layer_sel"]
    done_layers, spent = 0, 0.0
    for t in range(cfg.L_tgt):
        need = [int(s) for s in sel[t]]
        sk = {s: f(inp["src_k"][s][:, rows_t, :]) for s in need}
        sv = {s: f(inp["src_v"][s][:, rows_t, :]) for s in need}
        Wk, Wv = {t: f(inp["W_k"][t])}, {t: f(inp["W_v"][t])}
        bk, bv = {t: f(inp["b_k"][t])}, {t: f(inp["b_v"][t])}
        t0 = time.perf_counter()
        oracle.apply_rows(sk, sv, sel, Wk, bk, Wv, bv, cfg.theta_src, cfg.theta_tgt, cfg.pos0 + rows,
                          targets=[t])
        spent += time.perf_counter() - t0
        done_layers += 1
        if spent >= budget_s:
            break
    # tokens of the full cache (all target layers) per second
    per_token_all_layers = spent / (len(rows) * done_layers) * cfg.L_tgt
    return {"value": 1.0 / per_token_all_layers, "unit": "tokens/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{done_layers} of {cfg.L_tgt} target layers (K and V) x {len(rows)} tokens, fp64 numpy "
                      f"oracle, {spent:.1f} s; scaled to all target layers", **host_cpu()}


def recode_leg(K, ctx, cfg, src, iters=10, warmup=2):
    """kvmap_recode of the whole source key cache [L_src][H][T][d] into a fresh buffer."""
    import torch
    out = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        ctx.recode(src, cfg.theta_src, cfg.theta_tgt, out=out, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        ctx.recode(src, cfg.theta_src, cfg.theta_tgt, out=out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 2 * src.numel() * src.element_size()
    del out
    log(f"recode: {ms:.3f} ms for {nbytes / 1e9:.2f} GB")
    return {"workload": f"{cfg.name} source keys [{cfg.L_src}][{cfg.H}][{cfg.T}][{cfg.d}] {cfg.dtype}, "
                        f"theta {cfg.theta_src:g} -> {cfg.theta_tgt:g}",
            "ms": ms, "bytes": nbytes, "GBps": nbytes / (ms / 1e3) / 1e9,
            "frac_hbm": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS}


def short_leg(K, ctx, cfg, inp, lengths=(1, 16, 64, 128, 256, 512, 1024, 2048, 4096, 8192), iters=20, warmup=3):
    """Short and middle caches (the short-prefix regime): kvmap_apply of the workload's first T
    tokens for a range of T, with all of the workload's maps.  The roofline is the larger of the
    HBM time (W, 2 x L_tgt x N x F bf16, + the gathered source rows + the written target rows
    over 8 TB/s) and the matrix-core time (2 T F N per target layer, K and V, at the bf16 dense
    peak): HBM bounds the apply up to a few hundred tokens, the matrix cores beyond.  Caches of
    up to 128 tokens take the persistent short-cache kernel."""
    import torch
    stream = torch.cuda.current_stream()
    w_bytes = 2 * cfg.L_tgt * cfg.N * cfg.F * 2
    rows = []
    for T in lengths:
        sk = inp["src_k"][:, :, :T, :].contiguous()
        sv = inp["src_v"][:, :, :T, :].contiguous()
        ok_ = torch.empty((cfg.L_tgt, cfg.H, T, cfg.d), dtype=sk.dtype, device=sk.device)
        ov_ = torch.empty_like(ok_)

        def run():
            ctx.apply(sk, sv, inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"], inp["b_v"], cfg.theta_src,
                      cfg.theta_tgt, pos0_src=cfg.pos0, out_k=ok_, out_v=ov_, stream=stream)

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        x_bytes = 2 * cfg.L_tgt * cfg.k * cfg.H * T * cfg.d * 2   # gathered per target layer, K and V
        o_bytes = 2 * cfg.L_tgt * cfg.H * T * cfg.d * 2
        roof_ms = (w_bytes + x_bytes + o_bytes) / (PEAK_HBM_GBPS * 1e9) * 1e3
        mfma_ms = 2.0 * 2 * cfg.L_tgt * T * cfg.F * cfg.N / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        bound = max(roof_ms, mfma_ms)
        rows.append({"T": T, "ms": ms, "W_GBps": w_bytes / (ms / 1e3) / 1e9, "hbm_roofline_ms": roof_ms,
                     "mfma_roofline_ms": mfma_ms, "bound": "hbm" if roof_ms >= mfma_ms else "mfma",
                     "frac_hbm": roof_ms / ms, "frac_roofline": bound / ms,
                     "kernel": "map_bf16_small" if T <= 128 else "map_bf16"})
        log(f"short T={T}: {ms:.3f} ms ({w_bytes / (ms / 1e3) / 1e12:.2f} TB/s of W; HBM roofline {roof_ms:.3f} ms, "
            f"matrix-core roofline {mfma_ms:.3f} ms: {bound / ms * 100:.0f} % of the larger)")
        del sk, sv, ok_, ov_
    return {"workload": f"{cfg.name} maps (W {w_bytes / 1e9:.2f} GB bf16) on the first T tokens of the cache; "
                        f"roofline = max(HBM, matrix cores)",
            "lengths": rows}


def library_gemm_leg(cfg, inp, passes=3):
    """The vendor library on the plain GEMMs of the apply's shape (see the module docstring)."""
    import torch
    stream = torch.cuda.current_stream()
    sel = [int(s) for s in inp["layer_sel"][0]]
    # X[p][(j H + h) d + e] = src_k[sel[j]][h][p][e] (keys as the apply gathers them; the
    # de-rotation changes no statistics that matter to the timing)
    X = inp["src_k"][sel].permute(2, 0, 1, 3).reshape(cfg.T, cfg.F).contiguous()
    maps = [inp[w][t].t().contiguous() for t in range(cfg.L_tgt) for w in ("W_k", "W_v")]  # [F][N] each
    out = torch.empty((cfg.T, cfg.N), dtype=X.dtype, device=X.device)

    def one_pass():
        for Wt in maps:
            torch.matmul(X, Wt, out=out)

    one_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(passes):
        one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / passes
    tflops = cfg.flops / (ms / 1e3) / 1e12
    log(f"library GEMM (torch.matmul) on the same shape: {ms:.3f} ms per pass of {len(maps)} GEMMs, "
        f"{tflops:.0f} TFLOP/s = {tflops / PEAK_BF16_TFLOPS * 100:.1f} % of the bf16 dense peak")
    del X, maps, out
    return {"what": f"torch.matmul [T {cfg.T}][F {cfg.F}] x [F][N {cfg.N}], bf16, {2 * cfg.L_tgt} maps per pass",
            "ms": ms, "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS}


def fit_cpu_baseline(C, X, Y, budget_s=10.0):
    """The fp64 oracle's streamed statistics (two-pass per batch, Chan merge) on the first
    rows of one resident batch until the budget is spent; tokens/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    rows = 1024
    xs = X[:rows].float().cpu().double().numpy()
    ys = Y[:rows].float().cpu().double().numpy()
    st, done, spent = oracle.stats_empty(C.p, C.q), 0, 0.0
    while spent < budget_s:
        t0 = time.perf_counter()
        st = oracle.chan_merge(st, oracle.stats_two_pass(xs, ys))
        spent += time.perf_counter() - t0
        done += rows
    return {"value": done / spent, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{done // rows} batches of {rows} tokens (p {C.p}, q {C.q}), fp64 numpy two-pass "
                      f"statistics + Chan merge, {spent:.1f} s"}


def fit_leg(K, batches_timed=64, warmup_s=0.3, cpu=True):
    """Time kvmap_gram on the fit-statistics workload: a few distinct batches resident in HBM,
    cycled, after calls for at least warmup_s seconds (the GPU has idled while the batches were
    generated on the host, and the first tens of milliseconds of calls run slower); then one host
    ridge solve of the merged state and one on the device."""
    import torch
    from synth.device import fit_inputs
    from synth.workloads import FIT_STATS_CONFIG as C
    dev = "cuda:0"
    resident = [(X, Y) for _, X, Y in fit_inputs(C, range(4), dev)]
    ctx = K.Context(0)
    st = ctx.gram_state(C.p, C.q)
    stream = torch.cuda.current_stream()
    ctx.gram_reset(st, stream)
    t_w, n_w = time.perf_counter(), 0
    while n_w < 16 or time.perf_counter() - t_w < warmup_s:
        for _ in range(16):
            X, Y = resident[n_w % len(resident)]
            ctx.gram(st, X, Y, stream)
            n_w += 1
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(batches_timed):
        X, Y = resident[i % len(resident)]
        ctx.gram(st, X, Y, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / batches_timed
    nb, p, q = C.batch, C.p, C.q
    flops = 2.0 * nb * (p * (p + 1) / 2 + p * q)      # upper triangle of X^T X, all of X^T Y
    in_bytes = nb * (p + q) * 2
    t0 = time.perf_counter()
    W, b = ctx.ridge_solve(st, C.lam, stream)
    ridge_s = time.perf_counter() - t0
    ctx.ridge_solve_device(st, C.lam, dtype=torch.bfloat16, stream=stream)  # first call sizes the scratch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.ridge_solve_device(st, C.lam, dtype=torch.bfloat16, stream=stream)
    ridge_dev_s = time.perf_counter() - t0
    ctx.close()
    log(f"fit: {ms:.3f} ms per batch of {nb}; ridge solve {ridge_s:.2f} s on the host, "
        f"{ridge_dev_s * 1e3:.1f} ms on the device")
    base = fit_cpu_baseline(C, *resident[0]) if cpu else None
    return {"cpu_baseline": base, "workload": f"{C.name}: p {p}, q {q}, batches of {nb}, bf16", "ms_per_batch": ms,
            "tokens_per_s": nb / (ms / 1e3), "ms_per_fit_pass": ms * C.n_batches,
            "algorithmic_tflops": flops / (ms / 1e3) / 1e12, "flop_per_batch": flops,
            "input_GBps": in_bytes / (ms / 1e3) / 1e9, "ridge_solve_s": ridge_s,
            "ridge_solve_device_s": ridge_dev_s,
            "ridge_device_fp64_tflops": (p ** 3 / 3 + 2 * p * p * q) / ridge_dev_s / 1e12,
            "ridge_flop": p ** 3 / 3 + 2 * p * p * q}


def fit_driver_cpu_baseline(n_tok, L_src, L_tgt, H, d, k, lam, budget_s=30.0):
    """The oracle's fit on a bounded sample: one selection unit (single-source ridge + in-sample
    R^2 of one (target, source) pair, K or V) and one map unit (ridge of k*H*d features to H*d
    outputs) on n_tok seeded tokens, extrapolated to the whole fit (2 L_src L_tgt selection units,
    2 L_tgt map units); calibration tokens/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    rng = np.random.default_rng(77)
    N, F = H * d, k * H * d
    n = min(n_tok, 4096)
    Y = rng.standard_normal((n, N))
    t0 = time.perf_counter()
    X = rng.standard_normal((n, N))
    W, b = oracle.ridge(oracle.stats_two_pass(X, Y), lam)
    Yh = X @ W + b
    _ = [oracle.r2_pooled(Y[:, h * d:(h + 1) * d], Yh[:, h * d:(h + 1) * d]) for h in range(H)]
    t_sel = time.perf_counter() - t0
    X = rng.standard_normal((n, F))
    t0 = time.perf_counter()
    oracle.ridge(oracle.stats_two_pass(X, Y), lam)
    t_map = time.perf_counter() - t0
    # statistics scale with the tokens, the solves do not: scale the whole unit (a lower bound)
    total = (2 * L_src * L_tgt * t_sel + 2 * L_tgt * t_map) * (n_tok / n)
    return {"value": n_tok / total, "unit": "calibration tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"1 selection unit ({t_sel:.2f} s) and 1 map unit ({t_map:.2f} s) on {n} tokens, fp64 numpy, "
                      f"extrapolated to {2 * L_src * L_tgt} + {2 * L_tgt} units over {n_tok} tokens: {total:.0f} s"}


def fit_driver_leg(K, n_seqs=8, T=4096, cpu=True):
    """The complete two-stage fit (kvmap_fit_*) at the 14B->32B model shape: 40 source and 64
    target layers, H 8, d 128, k 8, lambda 0.01, over n_seqs seeded bf16 calibration sequences
    of T tokens resident in HBM.  Stage 1 scores all 2560 (target, source) pairs for K and V;
    stage 2 fits and solves 128 maps of 8192 x 1024.  Wall time per pass from the pass callbacks
    (each kvmap_fit_next_pass returns after the solves of the pass it closes).  At this shape the
    fit runs in one pass (the full source Gram; the maps gathered from it)."""
    import torch
    L_src, L_tgt, H, d, k, lam = 40, 64, 8, 128, 8, 0.01
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(20261202)

    def cache(L):
        scale = torch.exp(0.5 * torch.randn((L, H, 1, d), generator=g, device=dev))  # LogNormal(0, 0.5) channels
        return (torch.randn((L, H, T, d), generator=g, device=dev) * scale).to(torch.bfloat16)

    seqs = [(cache(L_src), cache(L_src), cache(L_tgt), cache(L_tgt), 0) for _ in range(n_seqs)]
    torch.cuda.synchronize()
    ctx = K.Context(0)
    stamps = []

    def on_pass(stage, t0, t1, i, n):
        torch.cuda.synchronize()
        stamps.append((time.perf_counter(), stage))
        log(f"fit driver: pass {i}/{n} stage {stage} targets [{t0}, {t1})")

    t_start = time.perf_counter()
    res = ctx.fit(lambda: seqs, L_src=L_src, L_tgt=L_tgt, H=H, d=d, k=k, theta_src=1.0e6, theta_tgt=1.0e6, lam=lam,
                  on_pass=on_pass)
    torch.cuda.synchronize()
    total = time.perf_counter() - t_start
    ctx.close()
    # stamps[i] opens pass i (its stage); the last one marks the end of the last pass, which
    # includes that pass's solves (in one-pass mode: the selection and all maps)
    pass_s = [stamps[i + 1][0] - stamps[i][0] for i in range(len(stamps) - 1)]
    stages = [stamps[i][1] for i in range(len(stamps) - 1)]
    n_tok = n_seqs * T
    del seqs, res
    torch.cuda.empty_cache()
    log(f"fit driver: {total:.2f} s in {len(pass_s)} pass(es) {['%.2f' % x for x in pass_s]} over {n_tok} "
        f"calibration tokens")
    base = fit_driver_cpu_baseline(n_tok, L_src, L_tgt, H, d, k, lam) if cpu else None
    return {"workload": f"qwen3-14b-to-32b fit: L {L_src}->{L_tgt}, H {H}, d {d}, k {k}, {n_seqs} x {T} bf16 "
                        f"calibration tokens, lambda {lam}",
            "seconds": total, "passes": len(pass_s), "pass_stages": stages, "pass_s": pass_s,
            "calibration_tokens": n_tok,
            "calibration_tokens_per_s": n_tok / total, "cpu_baseline": base}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fit", action="store_true", help="skip the fit-side measurement")
    ap.add_argument("--no-recode", action="store_true", help="skip the RoPE-recode measurement")
    ap.add_argument("--no-fit-driver", action="store_true", help="skip the end-to-end fit measurement")
    ap.add_argument("--no-short", action="store_true", help="skip the short-cache measurement")
    ap.add_argument("--no-library-gemm", action="store_true",
                    help="skip the vendor-library GEMM of the same shape (roofline context)")
    ap.add_argument("--fit-seqs", type=int, default=8, help="calibration sequences of 4096 tokens for the fit driver")
    ap.add_argument("--fit-driver-only", action="store_true",
                    help="run only the end-to-end fit measurement and print its object as the JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (the reference dispatch for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the apply shards by target layer or by tokens with no "
              "exchange between GPUs; runs on several GPUs are not measured here",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from cross_model_kv_amd import kvmap as K
    from synth.device import apply_inputs
    from synth.workloads import APPLY_CONFIGS

    if args.fit_driver_only:
        print(json.dumps(fit_driver_leg(K, n_seqs=args.fit_seqs, cpu=not args.no_cpu_baseline)), flush=True)
        return

    cfg = APPLY_CONFIGS[args.config]
    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: {a.numel() * 2} bytes read, {b.numel() * 2} bytes written")
        del a, b
    log(f"generating {cfg.name}: L {cfg.L_src}->{cfg.L_tgt} H={cfg.H} d={cfg.d} k={cfg.k} T={cfg.T}")
    t0 = time.time()
    inp = apply_inputs(cfg, "cuda:0", progress=lambda a, b: log(f"  inputs {a}/{b}") if a % 256 == 0 else None)
    log(f"inputs resident in {time.time() - t0:.1f} s")
    ctx = K.Context(0)
    ctx.reserve(cfg.L_src, cfg.L_tgt, cfg.H, cfg.d, cfg.k, cfg.T, K.BF16 if cfg.dtype == "bf16" else K.F32)
    out_k = torch.empty((cfg.L_tgt, cfg.H, cfg.T, cfg.d), dtype=inp["src_k"].dtype, device="cuda:0")
    out_v = torch.empty_like(out_k)
    stream = torch.cuda.current_stream()

    def step(flags=K.FLAG_TIMING):
        ctx.apply(inp["src_k"], inp["src_v"], inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"], inp["b_v"],
                  cfg.theta_src, cfg.theta_tgt, pos0_src=cfg.pos0, out_k=out_k, out_v=out_v, stream=stream,
                  flags=flags)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup}: kernels {ctx.last_timings()} ms")

    # The timed steps are queued back to back with no host wait between them: one HIP event
    # before each step on the stream, and the library's own per-launch events (it keeps the
    # last 128 timed applies), all read after the closing synchronisation.
    if args.steps > 128:
        raise SystemExit("--steps is at most 128 (the library holds the events of 128 timed applies)")
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        evs[i].record(stream)
        step()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = total_ms / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    kern = [ctx.timings(args.steps - 1 - i) for i in range(args.steps)]
    derope_ms = [x[1] for x in kern]
    gemm_ms = [x[2] for x in kern]
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (median {ms_median:.3f}), gemm "
        f"{sum(gemm_ms) / len(gemm_ms):.3f} ms (median {sorted(gemm_ms)[len(gemm_ms) // 2]:.3f}), "
        f"derope {sum(derope_ms) / len(derope_ms):.3f} ms")

    gemm_avg_s = sum(gemm_ms) / len(gemm_ms) / 1e3
    derope_avg_s = sum(derope_ms) / len(derope_ms) / 1e3
    achieved = cfg.flops / gemm_avg_s / 1e12
    n_used = len({int(s) for row in inp["layer_sel"] for s in row})
    derope_bytes = 2 * n_used * cfg.H * cfg.T * cfg.d * (2 if cfg.dtype == "bf16" else 4)
    traffic = traffic_entry(cfg.name)
    result = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian caches with LogNormal channel scales, random-init maps)",
        "config": {"workload": f"{cfg.name} apply", "L_src": cfg.L_src, "L_tgt": cfg.L_tgt, "H_kv": cfg.H,
                   "head_dim": cfg.d, "k": cfg.k, "T": cfg.T, "F": cfg.F, "N": cfg.N,
                   "theta_src": cfg.theta_src, "theta_tgt": cfg.theta_tgt},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "map_bf16_kernel", "kernel_ms": gemm_avg_s * 1e3,
                     "kernel_ms_median": sorted(gemm_ms)[len(gemm_ms) // 2]},
        "derope": {"ms": derope_avg_s * 1e3, "bytes": derope_bytes,
                   "GBps": derope_bytes / derope_avg_s / 1e9, "frac_hbm": derope_bytes / derope_avg_s / 1e9 / PEAK_HBM_GBPS,
                   "traffic": traffic_entry(cfg.name, DEROPE_TRAFFIC_FILE, "derope_kernel")},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline(cfg, inp)
    if not args.no_recode:
        result["recode"] = recode_leg(K, ctx, cfg, inp["src_k"])
    if not args.no_short:
        result["short"] = short_leg(K, ctx, cfg, inp)
    ctx.close()
    if not args.no_library_gemm and cfg.dtype == "bf16":
        result["library_gemm"] = library_gemm_leg(cfg, inp)
    if not args.no_fit:
        del inp, out_k, out_v
        torch.cuda.empty_cache()
        result["fit"] = fit_leg(K, cpu=not args.no_cpu_baseline)
    if not args.no_fit_driver:
        torch.cuda.empty_cache()
        result["fit_driver"] = fit_driver_leg(K, n_seqs=args.fit_seqs, cpu=not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
