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
}


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
