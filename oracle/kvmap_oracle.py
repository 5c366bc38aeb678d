"""Plain, slow, float64 reference for what the mapper computes.

TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and by the bench's
CPU-baseline leg, never by the library.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [KVB]  KVBridge README (github souvikDevloper/kvbridge): "What ships",
         "System design", the fitting section headed "Loading", "Local evidence".
  [VQ]   VeloxQuant-MLX, "Cross-Model KV Transfer -- Reuse One Model's Prefill in
         Another": "The mapping", "Configuration", "Metal kernel", "The honesty crux".
  [RA]   reactapp.top, "KV-Cache zwischen Qwen3-Modellen uebertragen statt neu zu
         prefillen": section "Eine lineare Bruecke reicht" (ridge demo, calibration,
         position stripping).
  [VW]   voidwest.dev, "Before Mapping KV Caches, Make Them Measurable": "what
         became first-class" (cache order [layer][kv_head][position][dim]),
         "measurement before mapping" (per layer/head K/V metrics).

Readings of points the pages leave open (each is listed in the design notes):
  * RoPE is the half-split form: pair (i, i + d/2) rotates by a = p * theta^(-2i/d),
    i < d/2.  The frequency formula on the VQ "Metal kernel" section is garbled;
    this is the standard reading, and the half-split layout is the one VQ's
    "honesty crux" item 7 accepts (it refuses the interleaved one).
  * Feature order in a row: selected rank j (order of layer_sel[t]), then source
    head, then dim.  Output column n = h * d + e.  The map is stored output-major
    [N][F]; the oracle's logical map is its transpose [F][N].
  * Bias is added in content space before the target rotation; values are never
    rotated ([VQ] "The mapping").
  * Statistics are unnormalised centered co-moments; lambda is added to the
    unnormalised centered Gram; the intercept is not penalised ([RA] ridge demo,
    [KVB] fitting section).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "inv_freq", "model_freqs", "angles", "rope", "strip_rope", "feature_rows", "affine",
    "apply_layer", "apply", "apply_rows",
    "stats_empty", "stats_two_pass", "chan_merge", "stats_streamed", "stats_exact",
    "ridge", "r2_pooled", "select_layers", "fit_mapper", "holdout_r2",
    "block_metrics",
]


# ---------------------------------------------------------------------------
# Rotary position encoding ([KVB] "What ships": exact inverse/forward RoPE;
# [VQ] "The mapping": strip_rope before the map, target rope after)
# ---------------------------------------------------------------------------

def inv_freq(theta: float, d: int) -> np.ndarray:
    """Per-pair frequency f_i = theta^(-2i/d), i = 0 .. d/2-1, in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def model_freqs(theta, d: int) -> np.ndarray:
    """A model's rotary frequencies: theta^(-2i/d) for a base theta, or theta itself when it is
    the list of d/2 frequencies the model emits ([KVB] "What ships": exact inverse/forward RoPE
    from each model's own factors)."""
    if np.ndim(theta) == 0:
        return inv_freq(float(theta), d)
    f = np.asarray(theta, dtype=np.float64).reshape(-1)
    if f.shape[0] != d // 2:
        raise ValueError(f"{f.shape[0]} frequencies for head dim {d}")
    return f


def angles(pos: np.ndarray, theta, d: int) -> np.ndarray:
    """a[t, i] = pos[t] * f_i in float64, shape [len(pos)][d/2]; theta is a base or a
    frequency list (model_freqs)."""
    return np.asarray(pos, dtype=np.float64)[:, None] * model_freqs(theta, d)[None, :]


def _rotate(x: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Rotate each pair (x[..., i], x[..., i + d/2]) of x [..., T, d] by angle a [T][d/2]."""
    h = x.shape[-1] // 2
    lo, hi = x[..., :h], x[..., h:]
    c, s = np.cos(a), np.sin(a)
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope(x: np.ndarray, pos: np.ndarray, theta) -> np.ndarray:
    """Apply half-split RoPE at positions pos to x [..., T, d] (float64); theta is the base or
    the model's frequency list."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate(x, angles(pos, theta, x.shape[-1]))


def strip_rope(x: np.ndarray, pos: np.ndarray, theta) -> np.ndarray:
    """Exact inverse of rope(): rotate every pair by the negative angle."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate(x, -angles(pos, theta, x.shape[-1]))


# ---------------------------------------------------------------------------
# Feature rows and the affine map ([KVB] "What ships": cross-head features,
# per-target-head K/V ridge maps; [RA] map_cache = x @ w + b, with x the
# concatenated features of all selected source layers)
# ---------------------------------------------------------------------------

def feature_rows(layers) -> np.ndarray:
    """Concatenate k content layers, each [H][T][d], into rows X [T][k*H*d].

    Column (j*H + h)*d + e of row t holds layers[j][h][t][e].
    """
    cols = []
    for lay in layers:
        lay = np.asarray(lay, dtype=np.float64)
        for h in range(lay.shape[0]):
            cols.append(lay[h])                       # [T][d]
    return np.concatenate(cols, axis=1)


def affine(X: np.ndarray, W_out_major: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Y = X . W + b, with W given output-major [N][F] (logical W is its transpose)."""
    W = np.asarray(W_out_major, dtype=np.float64).T   # logical [F][N]
    return np.asarray(X, dtype=np.float64) @ W + np.asarray(b, dtype=np.float64)[None, :]


def _heads(Y: np.ndarray, H: int) -> np.ndarray:
    """[T][H*d] -> [H][T][d] (output column n = h*d + e)."""
    T, N = Y.shape
    return Y.reshape(T, H, N // H).transpose(1, 0, 2)


def apply_layer(src_k_sel, src_v_sel, Wk, bk, Wv, bv, pos, theta_src, theta_tgt):
    """Map one target layer.

    src_k_sel / src_v_sel: the k selected stored source layers, each [H][T][d],
    in layer_sel order.  Keys: strip the source rotation, build rows, map, add
    bias, apply the target rotation.  Values: rows, map, bias.
    Returns (K_hat, V_hat), each [H][T][d] float64.
    """
    H = np.asarray(src_k_sel[0]).shape[0]
    xk = feature_rows([strip_rope(l, pos, theta_src) for l in src_k_sel])
    xv = feature_rows(src_v_sel)
    k_hat = rope(_heads(affine(xk, Wk, bk), H), pos, theta_tgt)
    v_hat = _heads(affine(xv, Wv, bv), H)
    return k_hat, v_hat


def apply(src_k, src_v, layer_sel, W_k, b_k, W_v, b_v, theta_src, theta_tgt,
          pos0_src=0, pos0_tgt=None, targets=None):
    """Map a whole cache.

    src_k, src_v: stored source cache [L_src][H][T][d]
    layer_sel   : int [L_tgt][k]
    W_k, W_v    : [L_tgt][N][F] output-major;  b_k, b_v: [L_tgt][N]
    Source keys sit at positions pos0_src + t, target keys at pos0_tgt + t
    (pos0_tgt defaults to pos0_src).  Returns dict t -> (K_hat, V_hat).
    """
    if pos0_tgt is None:
        pos0_tgt = pos0_src
    T = np.asarray(src_k[0]).shape[1]
    return apply_rows(src_k, src_v, layer_sel, W_k, b_k, W_v, b_v, theta_src, theta_tgt,
                      pos0_src + np.arange(T), pos0_tgt + np.arange(T), targets)


def apply_rows(src_k, src_v, layer_sel, W_k, b_k, W_v, b_v, theta_src, theta_tgt,
               pos_src, pos_tgt=None, targets=None):
    """Map the token rows whose source positions are pos_src (and target positions pos_tgt).

    src_k[s] / src_v[s] hold those rows of source layer s, [H][R][d] (any indexable of
    layers, e.g. a dict holding only the selected layers).  Every output row depends only
    on the same row of the source cache and on its positions, so a sampled subset of rows
    is mapped exactly as in the full cache.  Returns dict t -> (K_hat [H][R][d], V_hat).
    """
    pos_src = np.asarray(pos_src, dtype=np.int64)
    pos_tgt = pos_src if pos_tgt is None else np.asarray(pos_tgt, dtype=np.int64)
    targets = range(len(layer_sel)) if targets is None else targets
    out = {}
    for t in targets:
        sel = [int(s) for s in layer_sel[t]]
        ks = [np.asarray(src_k[s], dtype=np.float64) for s in sel]
        vs = [np.asarray(src_v[s], dtype=np.float64) for s in sel]
        H = ks[0].shape[0]
        xk = feature_rows([strip_rope(l, pos_src, theta_src) for l in ks])
        xv = feature_rows(vs)
        k_hat = rope(_heads(affine(xk, W_k[t], b_k[t]), H), pos_tgt, theta_tgt)
        v_hat = _heads(affine(xv, W_v[t], b_v[t]), H)
        out[t] = (k_hat, v_hat)
    return out


# ---------------------------------------------------------------------------
# Centered sufficient statistics ([KVB] fitting section: only centered
# statistics are kept, merged batchwise with Chan/Welford updates)
# ---------------------------------------------------------------------------

def stats_empty(p: int, q: int) -> dict:
    return dict(n=0, mx=np.zeros(p), my=np.zeros(q), Mxx=np.zeros((p, p)), Mxy=np.zeros((p, q)),
                ssy=np.zeros(q))


def stats_two_pass(X: np.ndarray, Y: np.ndarray) -> dict:
    """Textbook two-pass statistics: means, then unnormalised centered co-moments.

    ssy is the per-column centered sum of squares of y (the diagonal of the y-y co-moments):
    the total sum of squares that an R^2 of a fitted map divides by ([KVB] "What ships":
    layers are ranked by R^2).
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    n = X.shape[0]
    if n == 0:
        return stats_empty(X.shape[1], Y.shape[1])
    mx, my = X.mean(axis=0), Y.mean(axis=0)
    Xc, Yc = X - mx, Y - my
    return dict(n=n, mx=mx, my=my, Mxx=Xc.T @ Xc, Mxy=Xc.T @ Yc, ssy=np.sum(Yc * Yc, axis=0))


def chan_merge(a: dict, b: dict) -> dict:
    """Combine two statistics of disjoint samples (Chan, Golub & LeVeque pairwise update).

    n = na + nb, delta = mean_b - mean_a, mean = mean_a + delta * nb / n,
    M = Ma + Mb + (na * nb / n) * delta_x delta_y^T (ssy likewise, with delta_y squared).
    An empty side is the identity.
    """
    na, nb = a["n"], b["n"]
    if nb == 0:
        return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in a.items()}
    if na == 0:
        return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in b.items()}
    n = na + nb
    dx, dy = b["mx"] - a["mx"], b["my"] - a["my"]
    f = na * nb / n
    return dict(n=n,
                mx=a["mx"] + dx * (nb / n),
                my=a["my"] + dy * (nb / n),
                Mxx=a["Mxx"] + b["Mxx"] + f * np.outer(dx, dx),
                Mxy=a["Mxy"] + b["Mxy"] + f * np.outer(dx, dy),
                ssy=a["ssy"] + b["ssy"] + f * dy * dy)


def stats_streamed(batches) -> dict:
    """Per-batch two-pass statistics folded left-to-right with chan_merge()."""
    st = None
    for X, Y in batches:
        b = stats_two_pass(X, Y)
        st = b if st is None else chan_merge(st, b)
    return st


def stats_exact(X, Y) -> dict:
    """Exact rational statistics (fractions.Fraction) for tiny inputs; values as Fractions."""
    Xf = [[Fraction(float(v)) for v in row] for row in np.asarray(X, dtype=np.float64)]
    Yf = [[Fraction(float(v)) for v in row] for row in np.asarray(Y, dtype=np.float64)]
    n = len(Xf)
    p, q = len(Xf[0]), len(Yf[0])
    mx = [sum(r[i] for r in Xf) / n for i in range(p)]
    my = [sum(r[j] for r in Yf) / n for j in range(q)]
    Mxx = [[sum((r[i] - mx[i]) * (r[j] - mx[j]) for r in Xf) for j in range(p)] for i in range(p)]
    Mxy = [[sum((rx[i] - mx[i]) * (ry[j] - my[j]) for rx, ry in zip(Xf, Yf)) for j in range(q)]
           for i in range(p)]
    ssy = [sum((ry[j] - my[j]) ** 2 for ry in Yf) for j in range(q)]
    return dict(n=n, mx=mx, my=my, Mxx=Mxx, Mxy=Mxy, ssy=ssy)


# ---------------------------------------------------------------------------
# Ridge ([KVB] fitting section: W = (X^T X + lambda I)^-1 X^T Y, b = Ybar - Xbar W;
# [RA] ridge demo: centre x and y, solve with lambda = 0.01, intercept from means;
# [VQ] "The mapping": the fit runs on centered data, which leaves the intercept unpenalised)
# ---------------------------------------------------------------------------

def ridge(st: dict, lam: float):
    """Closed-form ridge from centered statistics. Returns logical W [p][q] and b [q]."""
    p = st["Mxx"].shape[0]
    A = st["Mxx"] + lam * np.eye(p)
    W = np.linalg.solve(A, st["Mxy"])
    b = st["my"] - st["mx"] @ W
    return W, b


def r2_pooled(y: np.ndarray, yhat: np.ndarray) -> float:
    """Pooled R^2 over all columns: 1 - sum (y - yhat)^2 / sum (y - colmean(y))^2."""
    y = np.asarray(y, dtype=np.float64)
    yhat = np.asarray(yhat, dtype=np.float64)
    rss = np.sum((y - yhat) ** 2)
    tss = np.sum((y - y.mean(axis=0, keepdims=True)) ** 2)
    return 1.0 - rss / tss


# ---------------------------------------------------------------------------
# Layer selection and the full fit ([KVB] "What ships": each source layer scored alone by R^2
# averaged over target heads, the best k concatenated as features; [VQ] "The mapping" item 1)
# ---------------------------------------------------------------------------

def _rows_of_layer(layer_seq) -> np.ndarray:
    """Stack one layer over sequences: [n_seq][H][T][d] -> rows [n_seq*T][H*d]."""
    return np.concatenate([feature_rows([lay]) for lay in layer_seq], axis=0)


def select_layers(src_k_c, src_v_c, tgt_k_c, tgt_v_c, k: int, lam: float):
    """Top-k source layers per target layer.

    Inputs are content-frame caches [n_seq][L][H][T][d].  For every (target t,
    source s) a ridge map from source layer s (all H*d features) to target layer
    t (all H*d outputs) is fitted for K and for V; its in-sample R^2 is pooled over
    each target head's d outputs, then averaged over heads and over {K, V}.
    The k best scores win; ties go to the lower source index.  Rows ascend.
    Returns (layer_sel [L_tgt][k] int32, scores [L_tgt][L_src]).
    """
    L_src, H, d = src_k_c.shape[1], src_k_c.shape[2], src_k_c.shape[4]
    L_tgt = tgt_k_c.shape[1]
    scores = np.zeros((L_tgt, L_src))
    for t in range(L_tgt):
        yk = _rows_of_layer(tgt_k_c[:, t])
        yv = _rows_of_layer(tgt_v_c[:, t])
        for s in range(L_src):
            per = []
            for xs, ys in ((_rows_of_layer(src_k_c[:, s]), yk), (_rows_of_layer(src_v_c[:, s]), yv)):
                W, b = ridge(stats_two_pass(xs, ys), lam)
                yhat = xs @ W + b
                per += [r2_pooled(ys[:, h * d:(h + 1) * d], yhat[:, h * d:(h + 1) * d]) for h in range(H)]
            scores[t, s] = np.mean(per)
    sel = np.empty((L_tgt, k), dtype=np.int32)
    for t in range(L_tgt):
        order = sorted(range(L_src), key=lambda s: (-scores[t, s], s))
        sel[t] = np.sort(order[:k])
    return sel, scores


def fit_mapper(src_k, src_v, tgt_k, tgt_v, pos, theta_src, theta_tgt, k, lam, layer_sel=None):
    """Fit the mapper from stored cache pairs over the same tokens.

    src_k/src_v: [n_seq][L_src][H][T][d] stored (keys rotated by the source model);
    tgt_k/tgt_v: [n_seq][L_tgt][H][T][d] stored (keys rotated by the target model);
    pos: [n_seq][T] positions.  Keys are moved to content space with each model's
    own rotation before any statistics ([VQ] "The mapping" item 3).
    Returns dict(layer_sel, W_k, b_k, W_v, b_v) with maps output-major [L_tgt][N][F].
    """
    n_seq = src_k.shape[0]
    sk = np.stack([strip_rope(src_k[i], pos[i], theta_src) for i in range(n_seq)])
    tk = np.stack([strip_rope(tgt_k[i], pos[i], theta_tgt) for i in range(n_seq)])
    sv = np.asarray(src_v, dtype=np.float64)
    tv = np.asarray(tgt_v, dtype=np.float64)
    if layer_sel is None:
        layer_sel, _ = select_layers(sk, sv, tk, tv, k, lam)
    L_tgt = tk.shape[1]
    Wk, bk, Wv, bv = [], [], [], []
    for t in range(L_tgt):
        sel = [int(s) for s in layer_sel[t]]
        xk = np.concatenate([feature_rows([sk[i, s] for s in sel]) for i in range(n_seq)], axis=0)
        xv = np.concatenate([feature_rows([sv[i, s] for s in sel]) for i in range(n_seq)], axis=0)
        yk = _rows_of_layer(tk[:, t])
        yv = _rows_of_layer(tv[:, t])
        W, b = ridge(stats_two_pass(xk, yk), lam)
        Wk.append(W.T); bk.append(b)
        W, b = ridge(stats_two_pass(xv, yv), lam)
        Wv.append(W.T); bv.append(b)
    return dict(layer_sel=np.asarray(layer_sel, dtype=np.int32), W_k=np.stack(Wk), b_k=np.stack(bk),
                W_v=np.stack(Wv), b_v=np.stack(bv))


def holdout_r2(true_c: np.ndarray, pred_c: np.ndarray) -> np.ndarray:
    """Per-head pooled R^2 of content-frame predictions; inputs [H][T][d] -> [H]."""
    return np.array([r2_pooled(true_c[h], pred_c[h]) for h in range(true_c.shape[0])])


# ---------------------------------------------------------------------------
# Per-(layer, head, K/V) comparison fields ([VW] "measurement before mapping":
# cosine, MSE, R^2, max abs error per layer and head)
# ---------------------------------------------------------------------------

def block_metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    """Comparison of one [T][d] block: got (widened exactly) against ref (float64)."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    diff = g - r
    nr = np.linalg.norm(r)
    return dict(
        rel_fro=float(np.linalg.norm(diff) / nr) if nr > 0 else float(np.linalg.norm(diff)),
        max_abs=float(np.max(np.abs(diff))) if diff.size else 0.0,
        max_rel=float(np.max(np.abs(diff)) / np.max(np.abs(r))) if diff.size and np.max(np.abs(r)) > 0 else 0.0,
        cosine=float(g @ r / (np.linalg.norm(g) * nr)) if nr > 0 and np.linalg.norm(g) > 0 else 1.0,
        mse=float(np.mean(diff ** 2)) if diff.size else 0.0,
    )
