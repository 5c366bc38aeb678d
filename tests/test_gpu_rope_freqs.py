"""Models that emit their own rotary frequencies (kvmap_rope.inv_freq) instead of a base theta,
on the GPU against the oracle (which takes the same frequency lists): apply, recode, cache rows
and the fit driver; plus refusals and the table cache keyed by the list.

The lists are a long-context style rescaling of theta^(-2i/d): the slow pairs divided by 8, the
fast ones kept, a smooth ramp between (any non-negative finite list is accepted).
Bounds are those of the theta path (tests/gpu_common.py bars; recode and rows as in their own
tests).
"""

import numpy as np
import pytest

import oracle
from gpu_common import compare
from synth.workloads import FITCHECK, bf16_bits_to_f64, bf16_round_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    from cross_model_kv_amd import kvmap as K
    return K


@pytest.fixture(scope="module")
def ctx(K):
    c = K.Context(0)
    yield c
    c.close()


def scaled_freqs(theta, d, factor=8.0, lo=1.0, hi=4.0, orig_len=8192):
    """theta^(-2i/d) with wavelengths above orig_len / lo divided by `factor`, those below
    orig_len / hi kept, and a linear ramp in between."""
    f = np.power(float(theta), -2.0 * np.arange(d // 2) / d)
    wl = 2.0 * np.pi / f
    out = f.copy()
    slow = wl > orig_len / lo
    out[slow] = f[slow] / factor
    mid = (~slow) & (wl >= orig_len / hi)
    s = (orig_len / wl[mid] - lo) / (hi - lo)
    out[mid] = (1.0 - s) * f[mid] / factor + s * f[mid]
    return out


def _stored(a, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f64(bf16_round_bits(np.asarray(a, dtype=np.float32)))
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_apply_with_model_frequencies(ctx, dtype):
    """Source keys roped with a rescaled list, target with a plain base (and the reverse in a
    second call, which must not hit the first call's tables)."""
    rng = np.random.default_rng([5, 1 if dtype == "bf16" else 2])
    L_src, L_tgt, H, d, T, k = 3, 2, 2, 128, 300, 2
    N, F = H * d, k * H * d
    fs = scaled_freqs(5.0e5, d)
    sel = np.array([[2, 0], [1, 2]], dtype=np.int32)
    src_k = _stored(rng.standard_normal((L_src, H, T, d)), dtype)
    src_v = _stored(rng.standard_normal((L_src, H, T, d)), dtype)
    Wk = _stored(rng.standard_normal((L_tgt, N, F)) / np.sqrt(F), dtype)
    Wv = _stored(rng.standard_normal((L_tgt, N, F)) / np.sqrt(F), dtype)
    bk = _stored(np.sqrt(0.1) * rng.standard_normal((L_tgt, N)), dtype)
    bv = _stored(np.sqrt(0.1) * rng.standard_normal((L_tgt, N)), dtype)
    dv = [_dev(a, dtype) for a in (src_k, src_v, Wk, bk, Wv, bv)]
    for (ts, fl_s), (tt, fl_t) in (((None, fs), (1.0e6, None)), ((1.0e6, None), (None, fs))):
        ok_, ov_ = ctx.apply(dv[0], dv[1], sel, *dv[2:], ts, tt, pos0_src=17, inv_freq_src=fl_s,
                             inv_freq_tgt=fl_t)
        torch.cuda.synchronize()
        ref = oracle.apply(src_k, src_v, sel, Wk, bk, Wv, bv, fl_s if fl_s is not None else ts,
                           fl_t if fl_t is not None else tt, pos0_src=17)
        rep, worst = compare(ok_.float().cpu().double().numpy(), ov_.float().cpu().double().numpy(), ref, dtype)
        print(f"[freqs] apply {dtype} src {'list' if fl_s is not None else 'theta'}: {worst}", flush=True)
        assert not rep, rep[:5]


def test_recode_and_rows_with_model_frequencies(ctx):
    rng = np.random.default_rng(9)
    d, T = 128, 257
    fs, ft = scaled_freqs(1.0e4, d, factor=4.0), scaled_freqs(5.0e5, d, factor=16.0)
    x = _stored(rng.standard_normal((3, T, d)) * 2.0, "f32")
    out = ctx.recode(_dev(x, "f32"), None, None, pos0_src=40, pos0_tgt=40, inv_freq_src=fs, inv_freq_tgt=ft)
    torch.cuda.synchronize()
    pos = 40 + np.arange(T)
    ref = oracle.rope(oracle.strip_rope(x, pos, fs), pos, ft)
    pair = np.sqrt(ref[..., : d // 2] ** 2 + ref[..., d // 2:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    err = np.abs(out.double().cpu().numpy() - ref)
    print(f"[freqs] recode: worst err/bound {np.max(err / (1e-6 * pair + 1e-30)):.3f}", flush=True)
    assert np.all(err <= 1e-6 * pair + 1e-30)
    cache = _stored(rng.standard_normal((2, 4, T, d)), "f32")
    rows = ctx.cache_rows(_dev(cache, "f32"), [1, 0], pos0=3, inv_freq=fs)
    torch.cuda.synchronize()
    pos = 3 + np.arange(T)
    ref = oracle.feature_rows([oracle.strip_rope(cache[l], pos, fs) for l in (1, 0)])
    r3 = ref.reshape(T, -1, d)
    pair = np.sqrt(r3[..., : d // 2] ** 2 + r3[..., d // 2:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1).reshape(T, -1)
    assert np.all(np.abs(rows.double().cpu().numpy() - ref) <= 1e-6 * pair + 1e-30)


def test_fit_with_model_frequencies(ctx):
    """The fit check with both models' keys roped by their own lists: the fit strips them with
    the same lists, selects the hidden layers and matches the oracle's maps."""
    from fitcheck_data import build_pairs
    fs, ft = scaled_freqs(1.0e4, 64, factor=4.0), scaled_freqs(5.0e5, 64, factor=8.0)
    cfg = FITCHECK.replace(theta_src=fs, theta_tgt=ft, holdout_pos0=())
    pr = build_pairs(cfg)
    nc = pr["n_calib"]
    seqs = [tuple(_dev(pr[n][i], "f32") for n in ("src_k", "src_v", "tgt_k", "tgt_v")) + (int(pr["pos"][i][0]),)
            for i in range(nc)]
    res = ctx.fit(lambda: seqs, L_src=cfg.L_src, L_tgt=cfg.L_tgt, H=cfg.H, d=cfg.d, k=cfg.k, theta_src=None,
                  theta_tgt=None, lam=cfg.lam, inv_freq_src=fs, inv_freq_tgt=ft)
    torch.cuda.synchronize()
    st = {n: _stored(pr[n][:nc], "f32") for n in ("src_k", "src_v", "tgt_k", "tgt_v")}
    ref = oracle.fit_mapper(st["src_k"], st["src_v"], st["tgt_k"], st["tgt_v"], pr["pos"][:nc], fs, ft, cfg.k,
                            cfg.lam)
    assert np.array_equal(res["layer_sel"].cpu().numpy(), ref["layer_sel"])
    assert np.array_equal(ref["layer_sel"], pr["draws"]["true_sel"])
    worst = 0.0
    for n in ("W_k", "b_k", "W_v", "b_v"):
        g, r = res[n].double().cpu().numpy(), ref[n]
        worst = max(worst, max(np.linalg.norm(g[t] - r[t]) / np.linalg.norm(r[t]) for t in range(cfg.L_tgt)))
    print(f"[freqs] fit: worst map rel err {worst:.2e}", flush=True)
    assert worst <= 2e-4


def test_frequency_list_refusals(ctx, K):
    x = torch.zeros((2, 16, 64), device="cuda")
    out = torch.full_like(x, 7.0)
    bad = np.full(32, 0.5)
    for v in (-1.0, float("nan"), float("inf")):
        bad[5] = v
        with pytest.raises(K.KvmapError) as e:
            ctx.recode(x, None, 1.0e6, out=out, inv_freq_src=bad)
        assert e.value.status == K.ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
