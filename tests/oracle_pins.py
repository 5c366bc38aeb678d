"""Checks that pin the fp64 oracle to facts other than itself.

Each pin raises AssertionError on failure.  They are collected as tests by
test_oracle_pins.py and re-run against deliberately broken copies of the
oracle by test_oracle_mutations.py, which requires every planted mistake to
trip at least one pin.
"""

import cmath
import json
import math
import os

import numpy as np

import oracle
from synth.workloads import APPLY_CONFIGS, FITCHECK, bf16_bits_to_f64, bf16_round_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Rotation
# ---------------------------------------------------------------------------

def pin_rope_frequencies():
    """f_0 = 1 and f_1 = theta^(-2/d): for theta = 1e4, d = 64 that is 10^(-1/8)."""
    f = oracle.inv_freq(1.0e4, 64)
    assert f[0] == 1.0
    assert abs(f[1] - 10.0 ** (-0.125)) < 1e-15
    assert abs(f[1] - 0.7498942093324559) < 1e-15
    # geometric: every ratio is theta^(-2/d); last entry theta^(-(d-2)/d)
    assert np.allclose(f[1:] / f[:-1], 10.0 ** (-0.125), rtol=0, atol=1e-14)
    assert abs(f[-1] - 1.0e4 ** (-62 / 64)) < 1e-18


def pin_rope_matches_complex_rotation():
    """rope() multiplies each pair z = x_i + i x_{i+d/2} by exp(i p f_i) (half-split RoPE)."""
    rng = np.random.default_rng(7)
    d, T, theta = 16, 5, 500.0
    x = rng.standard_normal((T, d))
    pos = np.array([0, 1, 7, 1000, 32767])
    got = oracle.rope(x, pos, theta)
    for t in range(T):
        for i in range(d // 2):
            z = complex(x[t, i], x[t, i + d // 2]) * cmath.exp(1j * pos[t] * theta ** (-(i / (d / 2))))
            assert abs(got[t, i] - z.real) < 1e-12 and abs(got[t, i + d // 2] - z.imag) < 1e-12


def pin_rope_with_model_frequencies():
    """A model's own frequency list (here scaled, uneven frequencies such as a long-context
    model emits) rotates each pair z = x_i + i x_{i+d/2} by exp(i p f_i); the list
    theta^(-2i/d) is the base-theta rotation; strip inverts rope for any list."""
    rng = np.random.default_rng(17)
    d, T = 16, 4
    f = np.sort(rng.uniform(0.0, 1.0, d // 2))[::-1] * np.array([1, 1, 1, 0.5, 0.25, 0.125, 0.1, 0.0])
    x = rng.standard_normal((T, d))
    pos = np.array([0, 5, 999, 32767])
    got = oracle.rope(x, pos, f)
    for t in range(T):
        for i in range(d // 2):
            z = complex(x[t, i], x[t, i + d // 2]) * cmath.exp(1j * pos[t] * f[i])
            assert abs(got[t, i] - z.real) < 1e-11 and abs(got[t, i + d // 2] - z.imag) < 1e-11
    base_list = [1.0e4 ** (-2.0 * i / d) for i in range(d // 2)]
    assert np.max(np.abs(oracle.rope(x, pos, base_list) - oracle.rope(x, pos, 1.0e4))) < 1e-12
    assert np.max(np.abs(oracle.strip_rope(oracle.rope(x, pos, f), pos, f) - x)) < 1e-13


def pin_strip_inverts_rope():
    """strip(rope(x)) = x at equal bases (to fp64 rounding), for positions up to 32K."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64, 128))
    pos = np.concatenate([np.arange(32), 32736 + np.arange(32)])
    for theta in (1.0e4, 5.0e5, 1.0e6):
        y = oracle.strip_rope(oracle.rope(x, pos, theta), pos, theta)
        assert np.max(np.abs(y - x)) < 1e-13
        y = oracle.rope(oracle.strip_rope(x, pos, theta), pos, theta)
        assert np.max(np.abs(y - x)) < 1e-13


def pin_rope_identity_at_zero_and_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 4, 64))
    y = oracle.rope(x, np.zeros(4, dtype=np.int64), 1.0e4)
    assert np.array_equal(y, x)
    pos = np.array([3, 99, 4095, 32767])
    y = oracle.rope(x, pos, 1.0e6)
    h = 32
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2, rtol=1e-13, atol=1e-13)


def pin_recode_single_rotation():
    """Strip at theta_s then rotate at theta_t = one rotation by p (f_t,i - f_s,i) per pair
    (VeloxQuant-MLX "Cross-Model KV Transfer", section "Metal kernel")."""
    rng = np.random.default_rng(3)
    d, T = 64, 6
    ts, tt = 1.0e4, 1.0e6
    x = rng.standard_normal((T, d))
    pos = np.array([0, 1, 2, 511, 8191, 32767])
    got = oracle.rope(oracle.strip_rope(x, pos, ts), pos, tt)
    for t in range(T):
        for i in range(d // 2):
            diff = tt ** (-(2.0 * i) / d) - ts ** (-(2.0 * i) / d)
            z = complex(x[t, i], x[t, i + d // 2]) * cmath.exp(1j * pos[t] * diff)
            assert abs(got[t, i] - z.real) < 1e-11 and abs(got[t, i + d // 2] - z.imag) < 1e-11


# ---------------------------------------------------------------------------
# Apply
# ---------------------------------------------------------------------------

def _identity_case(theta_s, theta_t, d=64, H=2, T=40, L=3):
    rng = np.random.default_rng(4)
    src_k = rng.standard_normal((L, H, T, d))
    src_v = rng.standard_normal((L, H, T, d))
    N = H * d
    sel = np.array([[2], [0], [1], [2]])
    I = np.eye(N)
    W = np.stack([I] * len(sel))
    b = np.zeros((len(sel), N))
    out = oracle.apply(src_k, src_v, sel, W, b, W, b, theta_s, theta_t)
    return src_k, src_v, sel, out


def pin_identity_map_copies_cache():
    """k = 1, W = I, b = 0 at equal bases copies the selected source layer."""
    src_k, src_v, sel, out = _identity_case(1.0e6, 1.0e6)
    for t, (kh, vh) in out.items():
        assert np.max(np.abs(kh - src_k[sel[t][0]])) < 1e-12
        assert np.array_equal(vh, src_v[sel[t][0]])


def pin_identity_map_recodes_keys():
    """k = 1, W = I, b = 0 at different bases: keys rotate by p (f_t - f_s); values copy."""
    ts, tt, d = 1.0e4, 5.0e5, 64
    src_k, src_v, sel, out = _identity_case(ts, tt, d=d)
    T = src_k.shape[2]
    for t, (kh, vh) in out.items():
        x = src_k[sel[t][0]]
        for p in (0, 1, 17, T - 1):
            for i in (0, 1, 5, d // 2 - 1):
                diff = tt ** (-(2.0 * i) / d) - ts ** (-(2.0 * i) / d)
                for h in range(x.shape[0]):
                    z = complex(x[h, p, i], x[h, p, i + d // 2]) * cmath.exp(1j * p * diff)
                    assert abs(kh[h, p, i] - z.real) < 1e-11
                    assert abs(kh[h, p, i + d // 2] - z.imag) < 1e-11
        assert np.array_equal(vh, src_v[sel[t][0]])


def brute_force_apply(src_k, src_v, sel, Wk, bk, Wv, bv, ts, tt, pos0=0):
    """Element-by-element map with math.cos/sin, written from the definitions:
    row feature (j, h, e) = stripped key of selected layer j, head h, dim e;
    output (h_t, e_t) = sum_f feature_f * W[h_t*d + e_t][f] + b; keys re-rotated."""
    L_t, k = len(sel), len(sel[0])
    H, T, d = len(src_k[0]), len(src_k[0][0]), len(src_k[0][0][0])
    half = d // 2
    outk = [[[[0.0] * d for _ in range(T)] for _ in range(H)] for _ in range(L_t)]
    outv = [[[[0.0] * d for _ in range(T)] for _ in range(H)] for _ in range(L_t)]
    for t in range(L_t):
        for p in range(T):
            pos = pos0 + p
            fk, fv = [], []
            for j in range(k):
                s = sel[t][j]
                for h in range(H):
                    for e in range(d):
                        i = e % half
                        a = pos * ts ** (-2.0 * i / d)
                        lo, hi = src_k[s][h][p][i], src_k[s][h][p][i + half]
                        # inverse rotation by a: (lo, hi) -> (lo c + hi s, hi c - lo s)
                        fk.append(lo * math.cos(a) + hi * math.sin(a) if e < half
                                  else hi * math.cos(a) - lo * math.sin(a))
                        fv.append(src_v[s][h][p][e])
            for ht in range(H):
                yk, yv = [0.0] * d, [0.0] * d
                for e in range(d):
                    n = ht * d + e
                    yk[e] = sum(fk[f] * Wk[t][n][f] for f in range(len(fk))) + bk[t][n]
                    yv[e] = sum(fv[f] * Wv[t][n][f] for f in range(len(fv))) + bv[t][n]
                for e in range(d):
                    i = e % half
                    a = pos * tt ** (-2.0 * i / d)
                    lo, hi = yk[i], yk[i + half]
                    outk[t][ht][p][e] = (lo * math.cos(a) - hi * math.sin(a) if e < half
                                         else hi * math.cos(a) + lo * math.sin(a))
                    outv[t][ht][p][e] = yv[e]
    return np.array(outk), np.array(outv)


def _tiny_apply_case(seed=5):
    rng = np.random.default_rng(seed)
    L_s, L_t, H, d, T, k = 3, 2, 2, 4, 3, 2
    F, N = k * H * d, H * d
    src_k = rng.standard_normal((L_s, H, T, d))
    src_v = rng.standard_normal((L_s, H, T, d))
    sel = np.array([[2, 0], [1, 2]])
    Wk = rng.standard_normal((L_t, N, F)); Wv = rng.standard_normal((L_t, N, F))
    bk = rng.standard_normal((L_t, N)); bv = rng.standard_normal((L_t, N))
    return src_k, src_v, sel, Wk, bk, Wv, bv


def pin_apply_brute_force():
    """Vectorised oracle == element-by-element loops on a tiny case (N != F, k = 2, unsorted sel)."""
    case = _tiny_apply_case()
    ts, tt, pos0 = 10.0, 1000.0, 5
    bk, bv = brute_force_apply(*case, ts, tt, pos0)
    out = oracle.apply(*case, ts, tt, pos0_src=pos0)
    for t in range(len(case[2])):
        assert np.max(np.abs(out[t][0] - bk[t])) < 1e-12
        assert np.max(np.abs(out[t][1] - bv[t])) < 1e-12


def pin_apply_rows_and_content_space():
    """Sampled rows equal the full map; and keys mapped at shifted positions are the
    same content (the fit is position-free: VeloxQuant-MLX "The mapping" item 3)."""
    rng = np.random.default_rng(6)
    L_s, H, d, T, k = 4, 2, 8, 10, 2
    F, N = k * H * d, H * d
    content = rng.standard_normal((L_s, H, T, d))
    src_v = rng.standard_normal((L_s, H, T, d))
    sel = np.array([[0, 3], [1, 2], [3, 1]])
    L_t = len(sel)
    Wk = rng.standard_normal((L_t, N, F)); Wv = rng.standard_normal((L_t, N, F))
    bk = rng.standard_normal((L_t, N)); bv = rng.standard_normal((L_t, N))
    ts, tt = 100.0, 3000.0
    outs = {}
    for P in (0, 777):
        stored = oracle.rope(content, P + np.arange(T), ts)
        full = oracle.apply(stored, src_v, sel, Wk, bk, Wv, bv, ts, tt, pos0_src=P)
        rows = np.array([9, 0, 4])
        part = oracle.apply_rows(stored[:, :, rows], src_v[:, :, rows], sel, Wk, bk, Wv, bv, ts, tt,
                                 P + rows)
        for t in range(L_t):
            assert np.max(np.abs(part[t][0] - full[t][0][:, rows])) < 1e-12
            assert np.array_equal(part[t][1], full[t][1][:, rows])
        outs[P] = {t: oracle.strip_rope(full[t][0], P + np.arange(T), tt) for t in range(L_t)}
    for t in range(L_t):
        assert np.max(np.abs(outs[0][t] - outs[777][t])) < 1e-11


def pin_planner_shape_arithmetic():
    """Parameter and statistics sizes the KVBridge planner prints for Qwen3 14B->32B, k = 8,
    follow from F = k*H*d cross-head features and N = H*d outputs per target layer."""
    g = _golden("kvbridge_planner.json")
    c = APPLY_CONFIGS[3]
    params = c.L_tgt * 2 * (c.F * c.N + c.N)
    assert params == g["mapper_params"]
    assert round(params * 4 / 2 ** 30, 4) == g["mapper_gib_fp32"]
    stats = (2 * c.F * c.F + 2 * c.F * c.N) * 4 / 2 ** 30
    assert round(stats, 2) == g["fit_stats_gib_per_one_layer_block"]


# ---------------------------------------------------------------------------
# Statistics
# ---------------------------------------------------------------------------

def _bf16_exact(rng, shape, loc=0.0, scale=1.0):
    x = (loc + scale * rng.standard_normal(shape)).astype(np.float32)
    return bf16_bits_to_f64(bf16_round_bits(x))


def pin_stats_exact_rational():
    """Two-pass fp64 statistics equal exact rational arithmetic on tiny bf16 inputs."""
    rng = np.random.default_rng(8)
    X = _bf16_exact(rng, (9, 4), loc=5.0)
    Y = _bf16_exact(rng, (9, 3), loc=-2.0)
    ex = oracle.stats_exact(X, Y)
    st = oracle.stats_two_pass(X, Y)
    assert st["n"] == ex["n"]
    for key in ("mx", "my"):
        assert np.allclose(st[key], [float(v) for v in ex[key]], rtol=1e-15, atol=1e-15)
    for key in ("Mxx", "Mxy"):
        ref = np.array([[float(v) for v in row] for row in ex[key]])
        assert np.max(np.abs(st[key] - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))
    ref = np.array([float(v) for v in ex["ssy"]])
    assert np.max(np.abs(st["ssy"] - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


def pin_chan_streaming_equals_two_pass():
    """Chan/Welford merging of batches of any sizes (1, empty, ragged) in any order equals
    one two-pass over the whole sample; merging an empty state is the identity."""
    rng = np.random.default_rng(9)
    X = _bf16_exact(rng, (301, 6), loc=5.0, scale=0.7)
    Y = _bf16_exact(rng, (301, 4), loc=1.0)
    ref = oracle.stats_two_pass(X, Y)
    for cuts in ([0, 1, 2, 100, 300, 301], [0, 150, 150, 301], [0, 301], [0, 7, 64, 200, 299, 301]):
        parts = [(X[a:b], Y[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
        for order in (parts, parts[::-1]):
            st = oracle.stats_streamed(order)
            assert st["n"] == ref["n"]
            for key in ("mx", "my", "Mxx", "Mxy", "ssy"):
                assert np.allclose(st[key], ref[key], rtol=1e-12, atol=1e-10)
    e = oracle.stats_empty(6, 4)
    m = oracle.chan_merge(ref, e)
    assert all(np.array_equal(m[k], ref[k]) for k in ("mx", "my", "Mxx", "Mxy", "ssy"))
    m = oracle.chan_merge(e, ref)
    assert all(np.array_equal(m[k], ref[k]) for k in ("mx", "my", "Mxx", "Mxy", "ssy"))


# ---------------------------------------------------------------------------
# Ridge
# ---------------------------------------------------------------------------

def pin_ridge_limits():
    """lambda -> 0 gives least squares with an intercept (numpy.linalg.lstsq); lambda > 0
    equals least squares on the centred data stacked over sqrt(lambda) I; residuals of the
    intercept fit sum to zero."""
    rng = np.random.default_rng(10)
    n, p, q = 200, 12, 5
    X = rng.standard_normal((n, p)) + 3.0
    Y = rng.standard_normal((n, q)) - 1.0
    st = oracle.stats_two_pass(X, Y)
    W0, b0 = oracle.ridge(st, 1e-12)
    A = np.hstack([X, np.ones((n, 1))])
    sol = np.linalg.lstsq(A, Y, rcond=None)[0]
    assert np.allclose(W0, sol[:p], rtol=1e-8, atol=1e-9)
    assert np.allclose(b0, sol[p], rtol=1e-8, atol=1e-9)
    lam = 3.7
    W, b = oracle.ridge(st, lam)
    Xc, Yc = X - X.mean(0), Y - Y.mean(0)
    Aug = np.vstack([Xc, math.sqrt(lam) * np.eye(p)])
    Yaug = np.vstack([Yc, np.zeros((p, q))])
    Wl = np.linalg.lstsq(Aug, Yaug, rcond=None)[0]
    assert np.allclose(W, Wl, rtol=1e-10, atol=1e-12)
    res = Y - (X @ W + b)
    assert np.max(np.abs(res.sum(axis=0))) < 1e-9


def pin_ridge_recovers_hidden_map():
    """Noise-free affine data: ridge at lambda = 0.01 recovers W to O(lambda / n)."""
    rng = np.random.default_rng(11)
    n, p, q = 4000, 10, 3
    X = rng.standard_normal((n, p)) + 5.0
    Wt = rng.standard_normal((p, q))
    bt = rng.standard_normal(q)
    Y = X @ Wt + bt
    W, b = oracle.ridge(oracle.stats_two_pass(X, Y), 0.01)
    assert np.max(np.abs(W - Wt)) < 1e-4
    assert np.max(np.abs(b - bt)) < 1e-3


def pin_r2_textbook():
    """r2_pooled of an ordinary least-squares fit with intercept of one column on one regressor
    is the squared Pearson correlation (numpy.corrcoef); predicting the column means gives 0,
    an exact prediction 1; pooling two columns weights each by its total sum of squares."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal(500) * 2.0 + 1.0
    y = 0.3 * x + rng.standard_normal(500) - 4.0
    slope, icept = np.polyfit(x, y, 1)
    r2 = oracle.r2_pooled(y[:, None], (slope * x + icept)[:, None])
    assert abs(r2 - np.corrcoef(x, y)[0, 1] ** 2) < 1e-12
    Y = np.stack([y, 10.0 * rng.standard_normal(500) + 7.0], axis=1)
    assert abs(oracle.r2_pooled(Y, np.broadcast_to(Y.mean(0), Y.shape))) < 1e-15
    assert oracle.r2_pooled(Y, Y) == 1.0
    # column 0 fitted as above, column 1 by its mean: pooled R^2 = (r2 * tss0) / (tss0 + tss1)
    yhat = np.stack([slope * x + icept, np.full(500, Y[:, 1].mean())], axis=1)
    t0, t1 = np.var(Y[:, 0]) * 500, np.var(Y[:, 1]) * 500
    assert abs(oracle.r2_pooled(Y, yhat) - r2 * t0 / (t0 + t1)) < 1e-12


# ---------------------------------------------------------------------------
# Selection + full fit (KVBridge README "Thirty-second proof" and "Local evidence")
# ---------------------------------------------------------------------------

def run_fitcheck(cfg):
    """Fit the oracle mapper from calibration cache pairs; return (fit, pairs, holdout R^2 [seq][t][kv][h])."""
    from fitcheck_data import build_pairs
    pr = build_pairs(cfg)
    nc = pr["n_calib"]
    fit = oracle.fit_mapper(pr["src_k"][:nc], pr["src_v"][:nc], pr["tgt_k"][:nc], pr["tgt_v"][:nc],
                            pr["pos"][:nc], cfg.theta_src, cfg.theta_tgt, cfg.k, cfg.lam)
    r2 = []
    for s in range(nc, len(pr["pos"])):
        P = int(pr["pos"][s][0])
        out = oracle.apply(pr["src_k"][s], pr["src_v"][s], fit["layer_sel"], fit["W_k"], fit["b_k"],
                           fit["W_v"], fit["b_v"], cfg.theta_src, cfg.theta_tgt, pos0_src=P)
        per_t = []
        for t in range(cfg.L_tgt):
            kh = oracle.strip_rope(out[t][0], pr["pos"][s], cfg.theta_tgt)
            per_t.append([oracle.holdout_r2(pr["tgt_k_content"][s, t], kh),
                          oracle.holdout_r2(pr["tgt_v"][s, t], out[t][1])])
        r2.append(per_t)
    return fit, pr, np.array(r2)


def pin_fitcheck_recovers_hidden_map(cfg=FITCHECK):
    fit, pr, r2 = run_fitcheck(cfg)
    assert np.array_equal(fit["layer_sel"], pr["draws"]["true_sel"])
    assert r2.min() > 0.99999, r2.min()
    # noise is sigma = 1e-3 on unit-variance outputs: 1 - R^2 must be of order 1e-6
    assert 1e-7 < 1.0 - r2.mean() < 1e-5, r2.mean()


# ---------------------------------------------------------------------------
# Layer-selection score (KVBridge README "What ships": every source layer is scored alone by
# the R^2 of its ridge map, averaged over target heads; the k best become the features)
# ---------------------------------------------------------------------------

def _walsh(n):
    """Sylvester-Hadamard matrix of order n (a power of 2): its columns are +-1 Walsh functions,
    mutually orthogonal with squared norm n; every column but the first sums to zero."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def _walsh_selection_case():
    """Content caches whose scores follow by hand.  T = 16 tokens, H = 2 heads of d = 2.  Source
    layer s (K and V alike) holds Walsh columns w[1 + 4s .. 4 + 4s] (s = 0, 1, 2); layer 3 is a
    copy of layer 2.  One target layer:
      K head 0: (3 w1 + w13, w2)    K head 1: (w5, w14)
      V head 0: (w9, w15)           V head 1: (w11, w12)
    The columns are orthogonal and centred, so at lambda -> 0 a map explains exactly the energy of
    the target columns that lie in the source layer's span.  Per-head pooled R^2, averaged over
    heads and then over {K, V}:
      s0: K (10/11 + 0)/2 = 5/11, V 0      -> 5/22
      s1: K (0 + 1/2)/2 = 1/4,    V 0      -> 1/8
      s2: K 0, V (1/2 + 1)/2 = 3/4          -> 3/8   (= s3, an exact tie)"""
    w = _walsh(16)
    T, H, d = 16, 2, 2
    src = np.zeros((1, 4, H, T, d))
    for s in range(3):
        for h in range(H):
            for e in range(d):
                src[0, s, h, :, e] = w[:, 1 + 4 * s + 2 * h + e]
    src[0, 3] = src[0, 2]
    tk = np.zeros((1, 1, H, T, d))
    tv = np.zeros((1, 1, H, T, d))
    tk[0, 0, 0, :, 0] = 3 * w[:, 1] + w[:, 13]
    tk[0, 0, 0, :, 1] = w[:, 2]
    tk[0, 0, 1, :, 0] = w[:, 5]
    tk[0, 0, 1, :, 1] = w[:, 14]
    tv[0, 0, 0, :, 0] = w[:, 9]
    tv[0, 0, 0, :, 1] = w[:, 15]
    tv[0, 0, 1, :, 0] = w[:, 11]
    tv[0, 0, 1, :, 1] = w[:, 12]
    return src, tk, tv


def pin_selection_scores_by_hand():
    """The selection score is the per-head pooled R^2 averaged over target heads and over {K, V}
    (a K-only score, R^2 pooled over a whole layer or averaged per column give other numbers and
    other choices); an exact tie goes to the lower source index; each row is kept ascending."""
    src, tk, tv = _walsh_selection_case()
    sel, scores = oracle.select_layers(src, src.copy(), tk, tv, 1, 1e-9)
    want = np.array([[5 / 22, 1 / 8, 3 / 8, 3 / 8]])
    assert np.max(np.abs(scores - want)) < 1e-8, scores
    assert scores[0, 2] == scores[0, 3]
    assert sel.tolist() == [[2]]
    sel, _ = oracle.select_layers(src, src.copy(), tk, tv, 2, 1e-9)
    assert sel.tolist() == [[2, 3]]
    sel, _ = oracle.select_layers(src, src.copy(), tk, tv, 3, 1e-9)
    assert sel.tolist() == [[0, 2, 3]]


# ---------------------------------------------------------------------------
# Comparison fields of one (layer, head, K/V) block (voidwest.dev "Before Mapping KV Caches,
# Make Them Measurable", "measurement before mapping": cosine, MSE and max abs error per block)
# ---------------------------------------------------------------------------

def pin_block_metrics_hand_values():
    """Fields worked out by hand on tiny blocks.  Relative errors divide by the reference (never
    by the value compared), the MSE is a mean over elements, and the cosine keeps its sign."""
    m = oracle.block_metrics(np.array([[3.0, 4.0], [0.0, 1.0]]), np.array([[3.0, 4.0], [0.0, 0.0]]))
    assert m["rel_fro"] == 1.0 / 5.0       # |diff| 1 over |ref| 5
    assert m["max_abs"] == 1.0
    assert m["max_rel"] == 1.0 / 4.0       # over max |ref| = 4
    assert abs(m["cosine"] - 5.0 / math.sqrt(26.0)) < 1e-15  # 25 / (sqrt(26) * 5)
    assert m["mse"] == 1.0 / 4.0           # one unit error over 4 elements
    ref = np.array([1.0, -2.0, 2.0])
    m = oracle.block_metrics(2.0 * ref, ref)  # the error is ref itself
    assert m["rel_fro"] == 1.0 and m["max_abs"] == 2.0 and m["max_rel"] == 1.0
    assert abs(m["cosine"] - 1.0) < 1e-15 and abs(m["mse"] - 3.0) < 1e-15
    m = oracle.block_metrics(-ref, ref)
    assert abs(m["cosine"] + 1.0) < 1e-15 and abs(m["rel_fro"] - 2.0) < 1e-15
    m = oracle.block_metrics(np.array([0.0, 10.0]), np.array([0.0, 1.0]))
    assert m["rel_fro"] == 9.0 and m["max_rel"] == 9.0 and m["max_abs"] == 9.0


ALL_PINS = [
    pin_rope_frequencies, pin_rope_matches_complex_rotation, pin_rope_with_model_frequencies,
    pin_strip_inverts_rope,
    pin_rope_identity_at_zero_and_norm, pin_recode_single_rotation, pin_identity_map_copies_cache,
    pin_identity_map_recodes_keys, pin_apply_brute_force, pin_apply_rows_and_content_space,
    pin_planner_shape_arithmetic, pin_stats_exact_rational, pin_chan_streaming_equals_two_pass,
    pin_ridge_limits, pin_ridge_recovers_hidden_map, pin_r2_textbook, pin_block_metrics_hand_values,
    pin_selection_scores_by_hand, pin_fitcheck_recovers_hidden_map,
]
