"""Workload shapes and seeded draws for the cross-model KV mapper.

Shapes follow the model pairs the pages quote: a tiny fp32 pair, a Qwen3
0.6B->1.7B-shaped pair, the Qwen3 14B->32B headline pair (Heo et al., as
summarised on the reactapp.top article, section on the headline numbers), a
Llama-3.1 8B->70B-shaped pair, and one target layer's fit-side statistics
stream.

Conventions
-----------
* Every draw comes from ``numpy.random.default_rng([2026, config_id, stream, *chunk])``
  so any chunk (one source layer and head, one target layer's map, one
  calibration batch) can be regenerated on its own, on any host.
* ``N(mu, v)`` in the workload descriptions names a variance ``v``; only the
  fit-check noise "N(0, 1e-3)" is a standard deviation (see the reading of the
  KVBridge README's holdout R^2 values in the design notes).
* Stored caches are drawn directly in the stored (rotated) frame.  For the
  unscaled N(0,1) pair this is the same distribution as rotating N(0,1)
  content, because a rotation maps an isotropic Gaussian pair to itself; for the
  channel-scaled pairs it only changes which frame carries the scales, which
  matters to neither throughput nor parity.  The fit check, where the frame
  matters, receives raw content and the tests rotate it with the oracle.
* bf16 values are produced by round-to-nearest-even from float32.

Streams: 0 layer_sel, 1 K values, 2 V values, 3 K channel scales, 4 V channel
scales, 5 W_K, 6 b_K, 7 W_V, 8 b_V, 10 fit X means, 11 fit X scales,
12 fit hidden-map columns, 13 fit hidden-map weights, 14 fit hidden bias,
15 fit Y noise, 20.. fit-check draws.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

SEED_ROOT = 2026


# ---------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ---------------------------------------------------------------------------

def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) with round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exactly equal float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, *[int(k) for k in key]])


# ---------------------------------------------------------------------------
# Apply workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class ApplyConfig:
    cid: int                 # seed id
    name: str
    L_src: int
    L_tgt: int
    H: int                   # KV heads (matched between source and target)
    d: int                   # head dim
    T: int                   # tokens in the cache
    k: int                   # selected source layers per target layer
    theta_src: float
    theta_tgt: float
    dtype: str               # "bf16" | "f32"
    chan_sigma: float        # LogNormal(0, chan_sigma) channel scales; 0 = none
    b_var: float = 0.1
    pos0: int = 0

    @property
    def F(self) -> int:      # feature width of one row
        return self.k * self.H * self.d

    @property
    def N(self) -> int:      # per-layer output width
        return self.H * self.d

    @property
    def flops(self) -> float:  # X.W for K and V over all target layers
        return 2.0 * self.T * self.F * self.N * 2 * self.L_tgt

    def replace(self, **kw) -> "ApplyConfig":
        return dataclasses.replace(self, **kw)


APPLY_CONFIGS = {
    1: ApplyConfig(1, "tiny-fp32", 4, 6, 2, 64, 256, 2, 1.0e4, 5.0e5, "f32", 0.0),
    2: ApplyConfig(2, "qwen3-0.6b-to-1.7b", 28, 28, 8, 128, 4096, 4, 1.0e6, 1.0e6, "bf16", 0.5),
    3: ApplyConfig(3, "qwen3-14b-to-32b", 40, 64, 8, 128, 32768, 8, 1.0e6, 1.0e6, "bf16", 0.5),
    4: ApplyConfig(4, "llama3.1-8b-to-70b", 32, 80, 8, 128, 16384, 8, 5.0e5, 5.0e5, "bf16", 0.5),
}


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage dtype; bf16 returns uint16 bit patterns."""
    if dtype == "bf16":
        return bf16_round_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def layer_sel(cfg: ApplyConfig) -> np.ndarray:
    """int32 [L_tgt][k]: a seeded distinct k-subset of source layers per target layer, ascending."""
    rng = _rng(cfg.cid, 0)
    out = np.empty((cfg.L_tgt, cfg.k), dtype=np.int32)
    for t in range(cfg.L_tgt):
        out[t] = np.sort(rng.choice(cfg.L_src, cfg.k, replace=False))
    return out


def _chan_scales(cfg: ApplyConfig, which: str, layer: int) -> np.ndarray:
    stream = 3 if which == "k" else 4
    if cfg.chan_sigma == 0.0:
        return np.ones((cfg.H, cfg.d), dtype=np.float32)
    z = _rng(cfg.cid, stream, layer).standard_normal((cfg.H, cfg.d), dtype=np.float32)
    return np.exp(np.float32(cfg.chan_sigma) * z).astype(np.float32)


def src_head(cfg: ApplyConfig, which: str, layer: int, head: int) -> np.ndarray:
    """One stored source head [T][d] in the storage dtype (bf16 -> uint16 bits)."""
    stream = 1 if which == "k" else 2
    z = _rng(cfg.cid, stream, layer, head).standard_normal((cfg.T, cfg.d), dtype=np.float32)
    z *= _chan_scales(cfg, which, layer)[head][None, :]
    return _store(z, cfg.dtype)


def src_layer(cfg: ApplyConfig, which: str, layer: int) -> np.ndarray:
    """One stored source layer [H][T][d] in the storage dtype."""
    return np.stack([src_head(cfg, which, layer, h) for h in range(cfg.H)])


def w_layer(cfg: ApplyConfig, which: str, t: int) -> np.ndarray:
    """Target layer t's map, output-major [N][F] (row n holds output column n's weights), ~N(0, 1/F)."""
    stream = 5 if which == "k" else 7
    z = _rng(cfg.cid, stream, t).standard_normal((cfg.N, cfg.F), dtype=np.float32)
    z *= np.float32(1.0 / np.sqrt(cfg.F))
    return _store(z, cfg.dtype)


def b_layer(cfg: ApplyConfig, which: str, t: int) -> np.ndarray:
    """Target layer t's bias [N], ~N(0, b_var)."""
    stream = 6 if which == "k" else 8
    z = _rng(cfg.cid, stream, t).standard_normal(cfg.N, dtype=np.float32)
    z *= np.float32(np.sqrt(cfg.b_var))
    return _store(z, cfg.dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values exactly to float64."""
    return bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Fit-side statistics workload
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class FitStatsConfig:
    cid: int
    name: str
    p: int              # feature width (k * H * d)
    q: int              # target width (H * d)
    n_tokens: int
    batch: int
    mean_mu: float      # per-channel mean offset ~ N(mean_mu, 1)
    chan_sigma: float   # per-channel LogNormal(0, chan_sigma) scale
    nnz: int            # nonzeros per column of the hidden sparse map
    noise_sd: float
    lam: float
    dtype: str = "bf16"

    @property
    def n_batches(self) -> int:
        return -(-self.n_tokens // self.batch)

    def replace(self, **kw) -> "FitStatsConfig":
        return dataclasses.replace(self, **kw)


FIT_STATS_CONFIG = FitStatsConfig(5, "qwen3-14b-to-32b-fit-stats", 8192, 1024, 262144, 4096,
                                  5.0, 0.5, 8, 1e-2, 0.01)


def _fit_channels(cfg: FitStatsConfig):
    mu = (cfg.mean_mu + _rng(cfg.cid, 10).standard_normal(cfg.p)).astype(np.float32)
    sc = np.exp(cfg.chan_sigma * _rng(cfg.cid, 11).standard_normal(cfg.p)).astype(np.float32)
    r = _rng(cfg.cid, 12)
    cols = np.stack([np.sort(r.choice(cfg.p, cfg.nnz, replace=False)) for _ in range(cfg.q)])
    wts = (_rng(cfg.cid, 13).standard_normal((cfg.q, cfg.nnz)) / np.sqrt(cfg.nnz)).astype(np.float32)
    bias = (np.sqrt(0.1) * _rng(cfg.cid, 14).standard_normal(cfg.q)).astype(np.float32)
    return mu, sc, cols, wts, bias


def fit_batch(cfg: FitStatsConfig, b: int):
    """Batch b of the calibration stream: (X [rows][p], Y [rows][q]) in the storage dtype.

    X = mu + s * z per channel (mu ~ N(mean_mu, 1), s ~ LogNormal(0, chan_sigma)).
    Y column j = sum_r w[j, r] * (X - mu)[:, cols[j, r]] + bias[j] + noise: a sparse
    hidden affine map, so the cross-moment has structure and the solve is checkable.
    """
    rows = min(cfg.batch, cfg.n_tokens - b * cfg.batch)
    mu, sc, cols, wts, bias = _fit_channels(cfg)
    z = _rng(cfg.cid, 1, b).standard_normal((rows, cfg.p), dtype=np.float32)
    x = mu[None, :] + sc[None, :] * z
    xs = _store(x, cfg.dtype)
    xv = bf16_bits_to_f32(xs) if cfg.dtype == "bf16" else xs
    xc = xv - mu[None, :]
    y = np.einsum("rjk,jk->rj", xc[:, cols], wts, dtype=np.float32) + bias[None, :]
    y += np.float32(cfg.noise_sd) * _rng(cfg.cid, 15, b).standard_normal((rows, cfg.q), dtype=np.float32)
    return xs, _store(y, cfg.dtype)


def fit_hidden_map(cfg: FitStatsConfig):
    """The hidden sparse map as dense logical [p][q] weights and [q] bias (float64),
    expressed against raw X (so the bias absorbs -mu . W)."""
    mu, _, cols, wts, bias = _fit_channels(cfg)
    W = np.zeros((cfg.p, cfg.q))
    for j in range(cfg.q):
        W[cols[j], j] = wts[j]
    return W, bias.astype(np.float64) - mu.astype(np.float64) @ W


# ---------------------------------------------------------------------------
# Fit-check draws (hidden cross-layer affine map between two synthetic models)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class FitCheckConfig:
    cid: int
    L_src: int
    L_tgt: int
    H: int
    d: int
    k: int
    T: int
    n_calib: int                  # calibration sequences at positions 0..T-1
    holdout_pos0: tuple           # first positions of the holdout sequences
    theta_src: float
    theta_tgt: float
    noise_sd: float
    lam: float
    b_var: float = 0.1

    @property
    def F(self) -> int:
        return self.k * self.H * self.d

    @property
    def N(self) -> int:
        return self.H * self.d

    def replace(self, **kw) -> "FitCheckConfig":
        return dataclasses.replace(self, **kw)


# Tiny fp32 pair's fit check: 8 x 256 = 2048 calibration tokens, holdout at 0 and 2048.
FITCHECK = FitCheckConfig(1, 4, 6, 2, 64, 2, 256, 8, (0, 2048), 1.0e4, 5.0e5, 1e-3, 0.01)


def fitcheck_draws(cfg: FitCheckConfig) -> dict:
    """Raw draws for the fit check (float64, content frame, nothing combined).

    Returns dict with
      true_sel  int32 [L_tgt][k]           hidden source layers per target layer (ascending)
      src_k/src_v [n_seq][L_src][H][T][d]  source content (un-rotated) for every sequence
      Wk/Wv    [L_tgt][N][F]               hidden maps, output-major
      bk/bv    [L_tgt][N]                  hidden biases
      noise_k/noise_v [n_seq][L_tgt][H][T][d]
      pos0     [n_seq]                     first position of each sequence
    Sequences 0..n_calib-1 are calibration; the rest are holdout.
    """
    c = cfg
    r = _rng(c.cid, 20)
    true_sel = np.stack([np.sort(r.choice(c.L_src, c.k, replace=False)) for _ in range(c.L_tgt)]).astype(np.int32)
    pos0 = [0] * c.n_calib + list(c.holdout_pos0)
    n_seq = len(pos0)

    def content(stream, s):
        return np.stack([_rng(c.cid, stream, s, l).standard_normal((c.H, c.T, c.d)) for l in range(c.L_src)])

    def noise(stream, s):
        return c.noise_sd * np.stack([_rng(c.cid, stream, s, t).standard_normal((c.H, c.T, c.d))
                                      for t in range(c.L_tgt)])

    return dict(
        true_sel=true_sel,
        pos0=np.array(pos0, dtype=np.int64),
        src_k=np.stack([content(21, s) for s in range(n_seq)]),
        src_v=np.stack([content(22, s) for s in range(n_seq)]),
        Wk=np.stack([_rng(c.cid, 23, t).standard_normal((c.N, c.F)) / np.sqrt(c.F) for t in range(c.L_tgt)]),
        Wv=np.stack([_rng(c.cid, 24, t).standard_normal((c.N, c.F)) / np.sqrt(c.F) for t in range(c.L_tgt)]),
        bk=np.stack([np.sqrt(c.b_var) * _rng(c.cid, 25, t).standard_normal(c.N) for t in range(c.L_tgt)]),
        bv=np.stack([np.sqrt(c.b_var) * _rng(c.cid, 26, t).standard_normal(c.N) for t in range(c.L_tgt)]),
        noise_k=np.stack([noise(27, s) for s in range(n_seq)]),
        noise_v=np.stack([noise(28, s) for s in range(n_seq)]),
    )
