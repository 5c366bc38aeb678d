"""Plant plausible mistakes in the oracle (on the CPU) and require the pins to catch each one."""

import numpy as np
import pytest

import oracle
import oracle.kvmap_oracle as K
import oracle_pins as P

_ORIG = {"chan_merge": K.chan_merge}


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(K, name, fn)
    monkeypatch.setattr(oracle, name, fn, raising=False)


def _rotate_wrong_sign(x, a):
    h = x.shape[-1] // 2
    lo, hi = x[..., :h], x[..., h:]
    c, s = np.cos(a), np.sin(a)
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)


def _rotate_interleaved(x, a):
    lo, hi = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(a), np.sin(a)
    out = np.empty_like(x)
    out[..., 0::2] = lo * c - hi * s
    out[..., 1::2] = hi * c + lo * s
    return out


def _inv_freq_wrong(theta, d):
    return np.power(np.float64(theta), -np.arange(d // 2, dtype=np.float64) / d)


def _features_head_major(layers):
    layers = [np.asarray(l, dtype=np.float64) for l in layers]
    return np.concatenate([layers[j][h] for h in range(layers[0].shape[0]) for j in range(len(layers))], axis=1)


def _affine_no_transpose(X, W, b):
    W = np.asarray(W, dtype=np.float64)
    return np.asarray(X, dtype=np.float64) @ W.reshape(W.shape[1], W.shape[0]) + np.asarray(b)[None, :]


def _affine_drop_bias(X, W, b):
    return np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def _heads_interleaved(Y, H):
    T, N = Y.shape
    return Y.reshape(T, N // H, H).transpose(2, 0, 1)


def _merge_no_cross_term(a, b):
    na, nb = a["n"], b["n"]
    if nb == 0 or na == 0:
        return dict(b if na == 0 else a)
    n = na + nb
    dx, dy = b["mx"] - a["mx"], b["my"] - a["my"]
    return dict(n=n, mx=a["mx"] + dx * nb / n, my=a["my"] + dy * nb / n,
                Mxx=a["Mxx"] + b["Mxx"], Mxy=a["Mxy"] + b["Mxy"])


def _merge_wrong_weight(a, b):
    na, nb = a["n"], b["n"]
    if nb == 0 or na == 0:
        return dict(b if na == 0 else a)
    n = na + nb
    dx, dy = b["mx"] - a["mx"], b["my"] - a["my"]
    f = na * nb / n
    return dict(n=n, mx=a["mx"] + dx * na / n, my=a["my"] + dy * na / n,
                Mxx=a["Mxx"] + b["Mxx"] + f * np.outer(dx, dx), Mxy=a["Mxy"] + b["Mxy"] + f * np.outer(dx, dy))


def _merge_ssy_no_cross_term(a, b):
    m = _ORIG["chan_merge"](a, b)
    if a["n"] and b["n"]:
        m["ssy"] = a["ssy"] + b["ssy"]
    return m


def _r2_uncentered_total(y, yhat):
    y = np.asarray(y, dtype=np.float64)
    return 1.0 - np.sum((y - yhat) ** 2) / np.sum(y ** 2)


def _ridge_wrong_intercept(st, lam):
    W = np.linalg.solve(st["Mxx"] + lam * np.eye(st["Mxx"].shape[0]), st["Mxy"])
    return W, st["my"] + st["mx"] @ W


def _ridge_penalise_scaled(st, lam):
    p = st["Mxx"].shape[0]
    W = np.linalg.solve(st["Mxx"] + lam * st["n"] * np.eye(p), st["Mxy"])
    return W, st["my"] - st["mx"] @ W


def _two_pass_uncentered(X, Y):
    X = np.asarray(X, dtype=np.float64); Y = np.asarray(Y, dtype=np.float64)
    n = X.shape[0]
    if n == 0:
        return K.stats_empty(X.shape[1], Y.shape[1])
    return dict(n=n, mx=X.mean(0), my=Y.mean(0), Mxx=X.T @ X, Mxy=X.T @ Y)


def _strip_same_direction(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    return K._rotate(x, K.angles(pos, theta, x.shape[-1]))


def _select_variant(score, tie_to_higher=False, ascending=True):
    """select_layers with one step changed: score(per-(K|V) list of (ys, yhat, H, d)) -> number."""
    def sel_fn(src_k_c, src_v_c, tgt_k_c, tgt_v_c, k, lam):
        L_src, H, d = src_k_c.shape[1], src_k_c.shape[2], src_k_c.shape[4]
        L_tgt = tgt_k_c.shape[1]
        scores = np.zeros((L_tgt, L_src))
        for t in range(L_tgt):
            yk, yv = K._rows_of_layer(tgt_k_c[:, t]), K._rows_of_layer(tgt_v_c[:, t])
            for s in range(L_src):
                fits = []
                for xs, ys in ((K._rows_of_layer(src_k_c[:, s]), yk), (K._rows_of_layer(src_v_c[:, s]), yv)):
                    W, b = K.ridge(K.stats_two_pass(xs, ys), lam)
                    fits.append((ys, xs @ W + b))
                scores[t, s] = score(fits, H, d)
        sel = np.empty((L_tgt, k), dtype=np.int32)
        for t in range(L_tgt):
            key = (lambda s: (-scores[t, s], -s)) if tie_to_higher else (lambda s: (-scores[t, s], s))
            top = sorted(range(L_src), key=key)[:k]
            sel[t] = np.sort(top) if ascending else top
        return sel, scores
    return sel_fn


def _heads_r2(ys, yh, H, d):
    return [K.r2_pooled(ys[:, h * d:(h + 1) * d], yh[:, h * d:(h + 1) * d]) for h in range(H)]


_score_mean = lambda fits, H, d: np.mean([r for ys, yh in fits for r in _heads_r2(ys, yh, H, d)])
_score_k_only = lambda fits, H, d: np.mean(_heads_r2(fits[0][0], fits[0][1], H, d))
_score_layer_pooled = lambda fits, H, d: np.mean([K.r2_pooled(ys, yh) for ys, yh in fits])
_score_per_column = lambda fits, H, d: np.mean([K.r2_pooled(ys[:, c:c + 1], yh[:, c:c + 1])
                                                for ys, yh in fits for c in range(ys.shape[1])])


def _metrics_variant(rel_by_got=False, max_rel_by_got=False, mse_sum=False, cos_abs=False):
    def fn(got, ref):
        g = np.asarray(got, dtype=np.float64).ravel()
        r = np.asarray(ref, dtype=np.float64).ravel()
        diff = g - r
        nr, ng = np.linalg.norm(r), np.linalg.norm(g)
        cos = g @ r / (ng * nr)
        return dict(rel_fro=float(np.linalg.norm(diff) / (ng if rel_by_got else nr)),
                    max_abs=float(np.max(np.abs(diff))),
                    max_rel=float(np.max(np.abs(diff)) / np.max(np.abs(g if max_rel_by_got else r))),
                    cosine=float(abs(cos) if cos_abs else cos),
                    mse=float(np.sum(diff ** 2) if mse_sum else np.mean(diff ** 2)))
    return fn


MUTANTS = {
    "rotation-sign": ("_rotate", _rotate_wrong_sign),
    "rotation-interleaved-pairs": ("_rotate", _rotate_interleaved),
    "frequency-exponent": ("inv_freq", _inv_freq_wrong),
    "feature-order-head-major": ("feature_rows", _features_head_major),
    "map-not-transposed": ("affine", _affine_no_transpose),
    "bias-dropped": ("affine", _affine_drop_bias),
    "head-split-interleaved": ("_heads", _heads_interleaved),
    "chan-missing-cross-term": ("chan_merge", _merge_no_cross_term),
    "chan-wrong-mean-weight": ("chan_merge", _merge_wrong_weight),
    "chan-ssy-missing-cross-term": ("chan_merge", _merge_ssy_no_cross_term),
    "r2-total-not-centered": ("r2_pooled", _r2_uncentered_total),
    "ridge-intercept-sign": ("ridge", _ridge_wrong_intercept),
    "ridge-lambda-times-n": ("ridge", _ridge_penalise_scaled),
    "stats-not-centered": ("stats_two_pass", _two_pass_uncentered),
    "strip-not-inverse": ("strip_rope", _strip_same_direction),
    "select-k-only-score": ("select_layers", _select_variant(_score_k_only)),
    "select-r2-pooled-over-layer": ("select_layers", _select_variant(_score_layer_pooled)),
    "select-r2-per-column-mean": ("select_layers", _select_variant(_score_per_column)),
    "select-tie-to-higher-index": ("select_layers", _select_variant(_score_mean, tie_to_higher=True)),
    "select-rows-not-ascending": ("select_layers", _select_variant(_score_mean, ascending=False)),
    "metrics-rel-fro-over-got": ("block_metrics", _metrics_variant(rel_by_got=True)),
    "metrics-max-rel-over-got": ("block_metrics", _metrics_variant(max_rel_by_got=True)),
    "metrics-mse-summed": ("block_metrics", _metrics_variant(mse_sum=True)),
    "metrics-cosine-unsigned": ("block_metrics", _metrics_variant(cos_abs=True)),
}


def test_select_variant_scaffold_is_faithful():
    """The scaffold the selection mutants are built on, with the unchanged score, passes the pins
    (so each mutant differs from the oracle only in the step it names)."""
    import pytest as _pt
    mp = _pt.MonkeyPatch()
    try:
        _patch(mp, "select_layers", _select_variant(_score_mean))
        P.pin_selection_scores_by_hand()
        _patch(mp, "block_metrics", _metrics_variant())
        P.pin_block_metrics_hand_values()
    finally:
        mp.undo()


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    _patch(monkeypatch, name, fn)
    caught = None
    for pin in P.ALL_PINS:  # cheapest pins first; the end-to-end fit check comes last
        try:
            pin()
        except Exception as e:  # AssertionError or a shape error both expose the mistake
            caught = (pin.__name__, type(e).__name__)
            break
    assert caught, f"no pin caught mutant {mutant}"
