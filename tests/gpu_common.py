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
    m["n_big"] = int(big.sum())
    m["big_max_abs"] = float(err[big].max()) if big.any() else 0.0
    m["big_max_rel"] = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    if m["big_max_rel"] > BF16_BIG_REL:
        report.append(f"{where}: |ref|>=8 rel err {m['big_max_rel']:.3e} > {BF16_BIG_REL}")
    m["max_abs_small"] = small_err
    return m


class Tally:
    """Worst fields over the compared blocks, and the elements with |ref| >= 8 (held to one bf16
    step relative instead of the 3e-2 absolute bar): how many, the blocks they sit in, and their
    largest absolute and relative errors, so the relaxation is reported, not hidden."""

    def __init__(self):
        self.worst = dict(rel_fro=0.0, max_abs=0.0, max_rel=0.0)
        self.n_blocks = 0
        self.n_big = 0
        self.big_blocks = []
        self.big_max_abs = 0.0
        self.big_max_rel = 0.0

    def add(self, m, where):
        self.n_blocks += 1
        for key in self.worst:
            self.worst[key] = max(self.worst[key], m[key])
        if m.get("n_big"):
            self.n_big += m["n_big"]
            self.big_blocks.append((where, m["n_big"], m["big_max_abs"]))
            self.big_max_abs = max(self.big_max_abs, m["big_max_abs"])
            self.big_max_rel = max(self.big_max_rel, m["big_max_rel"])

    def merge(self, other):
        self.n_blocks += other.n_blocks
        for key in self.worst:
            self.worst[key] = max(self.worst[key], other.worst[key])
        self.n_big += other.n_big
        self.big_blocks += other.big_blocks
        self.big_max_abs = max(self.big_max_abs, other.big_max_abs)
        self.big_max_rel = max(self.big_max_rel, other.big_max_rel)

    def summary(self) -> str:
        s = (f"{self.n_blocks} blocks: worst rel_fro {self.worst['rel_fro']:.3e} max_abs "
             f"{self.worst['max_abs']:.3e} max_rel {self.worst['max_rel']:.3e}; |ref|>=8: {self.n_big} elements "
             f"in {len(self.big_blocks)} blocks")
        if self.n_big:
            s += (f", max abs err {self.big_max_abs:.3e}, max rel err {self.big_max_rel:.3e} "
                  f"(blocks: {', '.join(f'{w} x{n} {e:.3e}' for w, n, e in self.big_blocks[:8])}"
                  f"{' ...' if len(self.big_blocks) > 8 else ''})")
        return s


def compare(out_k, out_v, ref: dict, dtype: str, rows=None, tally: Tally | None = None):
    """out_k/out_v: numpy [L_tgt][H][T][d] (or the sampled rows); ref: t -> (K, V) [H][R][d].
    Returns (failures, worst fields); the blocks are also added to `tally` when given."""
    report, tl = [], Tally()
    for t, (rk, rv) in ref.items():
        for kv, got, r in (("K", out_k, rk), ("V", out_v, rv)):
            g = got[t] if rows is None else got[t][:, rows, :]
            for h in range(r.shape[0]):
                where = f"t={t} h={h} {kv}"
                tl.add(check_block(g[h], r[h], dtype, where, report), where)
    if tally is not None:
        tally.merge(tl)
    if dtype != "f32":
        print(f"[compare] {tl.summary()}", flush=True)
    return report, tl.worst
