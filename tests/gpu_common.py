"""Shared helpers of the GPU parity tests: tolerance checks against the fp64 oracle."""

import numpy as np

import oracle

# Acceptance bars (bf16 caches: per (target layer, head, K|V) block; fp32: max relative error).
BF16_REL_FRO = 5e-3
BF16_MAX_ABS = 3e-2
F32_MAX_REL = 1e-5
# Where |ref| >= 8 one bf16 step is 0.0625, so rounding alone can exceed 3e-2; those elements
# are held to a relative bound instead (one bf16 ulp = 2^-7 relative) and counted.
BF16_BIG = 8.0
BF16_BIG_REL = 2.0 ** -7


def to_f64(t) -> np.ndarray:
    """Device/host tensor (bf16 or fp32) -> float64 numpy, exactly."""
    return t.float().cpu().double().numpy()


def check_block(got: np.ndarray, ref: np.ndarray, dtype: str, where: str, report: list):
    """Compare one [R][d] block; append failures to report; return metrics."""
    m = oracle.block_metrics(got, ref)
    if dtype == "f32":
        if m["max_rel"] > F32_MAX_REL:
            report.append(f"{where}: max rel {m['max_rel']:.3e} > {F32_MAX_REL}")
        return m
    if m["rel_fro"] > BF16_REL_FRO:
        report.append(f"{where}: rel Frobenius {m['rel_fro']:.3e} > {BF16_REL_FRO}")
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    big = np.abs(ref) >= BF16_BIG
    small_err = float(err[~big].max()) if (~big).any() else 0.0
    if small_err > BF16_MAX_ABS:
        report.append(f"{where}: max abs {small_err:.3e} > {BF16_MAX_ABS}")
    if big.any():
        rel = float((err[big] / np.abs(ref[big])).max())
        m["n_big"] = int(big.sum())
        if rel > BF16_BIG_REL:
            report.append(f"{where}: |ref|>=8 rel err {rel:.3e} > {BF16_BIG_REL}")
    m["max_abs_small"] = small_err
    return m


def compare(out_k, out_v, ref: dict, dtype: str, rows=None):
    """out_k/out_v: numpy [L_tgt][H][T][d] (or the sampled rows); ref: t -> (K, V) [H][R][d]."""
    report, worst = [], dict(rel_fro=0.0, max_abs=0.0, max_rel=0.0)
    for t, (rk, rv) in ref.items():
        for kv, got, r in (("K", out_k, rk), ("V", out_v, rv)):
            g = got[t] if rows is None else got[t][:, rows, :]
            for h in range(r.shape[0]):
                m = check_block(g[h], r[h], dtype, f"t={t} h={h} {kv}", report)
                for key in worst:
                    worst[key] = max(worst[key], m[key])
    return report, worst
