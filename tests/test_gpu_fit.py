"""Fit side beyond the statistics, on the GPU against the fp64 oracle: token rows
(kvmap_cache_rows), the kept total sum of squares (ss_y), the in-sample R^2 of a ridge fit
(kvmap_ridge_r2) and the end-to-end two-stage fit (kvmap_fit_*: selection, then maps).

Tolerances
  * rows: fp32 without RoPE and bf16 without RoPE are copies (bit-exact); with the strip,
    the fp32 rotation carries ~1e-6 of the pair's norm and bf16 rows are that rotation
    rounded once to nearest (at most 2^-8 of |r|).
  * ss_y: the fp32 statistics bar, 1e-5 relative (like M_xx, M_xy).
  * R^2: the statistics are fp32 with relative error <= 1e-5; R^2 = 1 - RSS/TSS with
    RSS = TSS - w.m - lambda |w|^2 moves by at most ~(1 + 2 kappa) x 1e-5 of TSS, kappa of
    M_xx + lambda I <= ~5 for the shapes here (n >= 4p): 1e-4 absolute.
  * maps, fp32 caches: W = (M_xx + lambda I)^-1 M_xy moves by <= kappa x (2e-5) relative:
    2e-4 relative Frobenius per (target layer, K/V).
  * maps, bf16 caches: the bf16 bar of the apply, 5e-3 relative Frobenius per (layer, K/V);
    scores 1e-3 absolute (the de-rotated rows are rounded to bf16 before the statistics).
"""

import numpy as np
import pytest

import oracle
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


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def _as_stored(a, dtype):
    """What a cache holds after upload, widened exactly to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bf16_round_bits(np.asarray(a, dtype=np.float32)))
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


# ---------------------------------------------------------------------------
# kvmap_cache_rows
# ---------------------------------------------------------------------------

ROW_CASES = [
    # L, H, T, d, dtype, layers, theta (None: no strip), pos0
    (5, 3, 77, 128, "bf16", [4, 0, 2], 1.0e6, 0),
    (3, 2, 300, 64, "f32", [1], 1.0e4, 1000),
    (4, 8, 129, 128, "bf16", [3, 1], None, 0),
    (2, 4, 33, 64, "f32", [0, 1], None, 0),
]


def _random_row_cases(n=12):
    """Seeded random gathers: 1-8 layers of 1-8 heads, 1-599 tokens, d 64 or 128, one to four
    distinct layers in any order, with or without the strip, position offsets up to 1e5."""
    rng = np.random.default_rng([2026, 706])
    out = []
    for _ in range(n):
        L, H = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        layers = [int(v) for v in rng.permutation(L)[: int(rng.integers(1, min(L, 4) + 1))]]
        theta = None if rng.random() < 0.3 else float(rng.choice([1.0e4, 5.0e5, 1.0e6]))
        out.append((L, H, int(rng.integers(1, 600)), int(rng.choice([64, 128])),
                    "f32" if rng.random() < 0.4 else "bf16", layers, theta, int(rng.choice([0, int(rng.integers(1, 100_000))]))))
    return out


ROW_CASES = ROW_CASES + _random_row_cases()


@pytest.mark.parametrize("L,H,T,d,dtype,layers,theta,pos0", ROW_CASES)
def test_cache_rows_matches_oracle(ctx, L, H, T, d, dtype, layers, theta, pos0):
    rng = np.random.default_rng([77, L, H, T, d])
    cache = _as_stored(rng.standard_normal((L, H, T, d)) * 1.5, dtype)
    got = ctx.cache_rows(_dev(cache, dtype), layers, theta=theta, pos0=pos0)
    torch.cuda.synchronize()
    g = got.float().cpu().double().numpy()
    pos = pos0 + np.arange(T)
    content = [oracle.strip_rope(cache[l], pos, theta) if theta is not None else cache[l] for l in layers]
    ref = oracle.feature_rows(content)
    where = f"rows L {L} H {H} T {T} d {d} {dtype} layers {layers} theta {theta}"
    if theta is None:
        assert np.array_equal(g, ref), where
        return
    # pair norms in the row layout: column (j*H + h)*d + e pairs with e +- d/2
    r3 = ref.reshape(T, -1, d)
    pair = np.sqrt(r3[..., : d // 2] ** 2 + r3[..., d // 2:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1).reshape(T, -1)
    bound = (2.0 ** -8 if dtype == "bf16" else 0.0) * np.abs(ref) + 1e-6 * pair + 1e-30
    worst = float(np.max(np.abs(g - ref) / bound))
    print(f"[rows] {where}: worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0, where


# ---------------------------------------------------------------------------
# ss_y and kvmap_ridge_r2
# ---------------------------------------------------------------------------

def _xy(n, p, q, seed, offset=5.0, signal=0.7):
    """Rows with per-column offsets and a partial linear dependence of y on x."""
    rng = np.random.default_rng([91, seed])
    X = rng.standard_normal((n, p)) * rng.uniform(0.5, 2.0, p) + offset * rng.standard_normal(p)
    A = rng.standard_normal((p, q)) / np.sqrt(p)
    Y = signal * (X - X.mean(0)) @ A + rng.standard_normal((n, q)) + rng.standard_normal(q)
    return X, Y


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ss_y_streamed_and_merged(ctx, dtype):
    """ss_y over ragged batches, a call larger than one bf16 sub-batch and a merge of two states
    equals the oracle's two-pass column sums of squares; a state without ss_y merged with one
    that keeps it is refused."""
    from cross_model_kv_amd import kvmap as K
    X, Y = _xy(17000 + 900, 64, 36, seed=1)
    X, Y = _as_stored(X, dtype), _as_stored(Y, dtype)
    a = ctx.gram_state(64, 36, keep_ss_y=True)
    b = ctx.gram_state(64, 36, keep_ss_y=True)
    ctx.gram_reset(a)
    ctx.gram_reset(b)
    cuts = [0, 1, 700, 17700, 17900]
    for i, (r0, r1) in enumerate(zip(cuts[:-1], cuts[1:])):
        ctx.gram(a if i < 3 else b, _dev(X[r0:r1], dtype), _dev(Y[r0:r1], dtype))
    ctx.gram_merge(a, b)
    torch.cuda.synchronize()
    ref = oracle.stats_two_pass(X, Y)
    got = a.ss_y.double().cpu().numpy()
    r = _rel(got, ref["ssy"])
    print(f"[ss_y] {dtype}: rel {r:.2e}", flush=True)
    assert r <= 1e-5
    c = ctx.gram_state(64, 36)
    ctx.gram_reset(c)
    with pytest.raises(K.KvmapError) as e:
        ctx.gram_merge(c, a)
    assert e.value.status == K.ERR_INVALID_ARGUMENT


def _random_r2_cases(n=8):
    """Seeded random R^2 calls: p a multiple of 4 up to 600, groups of 4-128 columns (a multiple of
    4), 1-6 groups, n = 4p + up to 500 rows, lambda 0.01, 1 or 50, bf16 or fp32."""
    rng = np.random.default_rng([2026, 707])
    out = []
    for _ in range(n):
        p = 4 * int(rng.integers(1, 151))
        group = 4 * int(rng.integers(1, 33))
        out.append((4 * p + int(rng.integers(1, 500)), p, group * int(rng.integers(1, 7)), group,
                    float(rng.choice([0.01, 1.0, 50.0])), "f32" if rng.random() < 0.4 else "bf16"))
    return out


@pytest.mark.parametrize("n,p,q,group,lam,dtype", [
    (3000, 128, 256, 64, 0.01, "f32"),
    (4096, 520, 136, 68, 0.01, "bf16"),
    (2500, 64, 192, 192, 50.0, "f32"),
] + _random_r2_cases())
def test_ridge_r2_matches_oracle(ctx, n, p, q, group, lam, dtype):
    """Pooled in-sample R^2 per group of y columns from the statistics, against the oracle's R^2
    of the fitted predictions (oracle.ridge on two-pass statistics, then r2_pooled)."""
    X, Y = _xy(n, p, q, seed=p + q)
    X, Y = _as_stored(X, dtype), _as_stored(Y, dtype)
    st = ctx.gram_state(p, q, keep_ss_y=True)
    ctx.gram_reset(st)
    for r0 in range(0, n, 1500):
        ctx.gram(st, _dev(X[r0:r0 + 1500], dtype), _dev(Y[r0:r0 + 1500], dtype))
    got = ctx.ridge_r2(st, lam, group).cpu().numpy()
    W, b = oracle.ridge(oracle.stats_two_pass(X, Y), lam)
    Yh = X @ W + b
    ref = np.array([oracle.r2_pooled(Y[:, g * group:(g + 1) * group], Yh[:, g * group:(g + 1) * group])
                    for g in range(q // group)])
    err = np.max(np.abs(got - ref))
    print(f"[r2] n {n} p {p} q {q} group {group} lambda {lam} {dtype}: R^2 {ref.min():.4f}..{ref.max():.4f}, "
          f"max |err| {err:.2e}", flush=True)
    assert err <= 1e-4


def test_ridge_r2_refusals(ctx, K):
    st = ctx.gram_state(64, 128)  # no ss_y
    ctx.gram_reset(st)
    with pytest.raises(K.KvmapError) as e:
        ctx.ridge_r2(st, 0.01, 64)
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    st = ctx.gram_state(64, 128, keep_ss_y=True)
    ctx.gram_reset(st)
    with pytest.raises(K.KvmapError) as e:
        ctx.ridge_r2(st, 0.01, 48)  # 48 does not divide 128
    assert e.value.status == K.ERR_SHAPE


# ---------------------------------------------------------------------------
# End-to-end fit (kvmap_fit_*)
# ---------------------------------------------------------------------------

def _pairs(cfg, dtype):
    """Calibration pairs of the fit check as stored (bf16-rounded when dtype is bf16), the
    device tensors of each calibration sequence, and the content-frame caches the oracle
    selects on."""
    from fitcheck_data import build_pairs
    pr = build_pairs(cfg)
    nc = pr["n_calib"]
    st = {k: _as_stored(pr[k][:nc], dtype) for k in ("src_k", "src_v", "tgt_k", "tgt_v")}
    seqs = [(_dev(st["src_k"][i], dtype), _dev(st["src_v"][i], dtype), _dev(st["tgt_k"][i], dtype),
             _dev(st["tgt_v"][i], dtype), int(pr["pos"][i][0])) for i in range(nc)]
    return pr, st, seqs


def _oracle_fit(cfg, pr, st, layer_sel=None):
    nc = pr["n_calib"]
    pos = pr["pos"][:nc]
    fit = oracle.fit_mapper(st["src_k"], st["src_v"], st["tgt_k"], st["tgt_v"], pos, cfg.theta_src, cfg.theta_tgt,
                            cfg.k, cfg.lam, layer_sel=layer_sel)
    return fit


def _oracle_scores(cfg, pr, st, targets):
    nc = pr["n_calib"]
    pos = pr["pos"][:nc]
    sk = np.stack([oracle.strip_rope(st["src_k"][i], pos[i], cfg.theta_src) for i in range(nc)])
    tk = np.stack([oracle.strip_rope(st["tgt_k"][i][targets], pos[i], cfg.theta_tgt) for i in range(nc)])
    _, scores = oracle.select_layers(sk, st["src_v"], tk, st["tgt_v"][:, targets], cfg.k, cfg.lam)
    return scores


def _run_fit(ctx, cfg, seqs, **kw):
    res = ctx.fit(lambda: seqs, L_src=cfg.L_src, L_tgt=cfg.L_tgt, H=cfg.H, d=cfg.d, k=cfg.k,
                  theta_src=cfg.theta_src, theta_tgt=cfg.theta_tgt, lam=cfg.lam, **kw)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None and v.dtype != torch.bfloat16 else
                (v.float().cpu().numpy() if v is not None else None)) for k, v in res.items()}


def _check_maps(got, ref, bound, where):
    worst = 0.0
    for t in range(ref["W_k"].shape[0]):
        for kv in ("k", "v"):
            rw = _rel(got[f"W_{kv}"][t].astype(np.float64), ref[f"W_{kv}"][t])
            rb = _rel(got[f"b_{kv}"][t].astype(np.float64), ref[f"b_{kv}"][t])
            worst = max(worst, rw, rb)
    print(f"[fit] {where}: worst map rel err {worst:.2e}", flush=True)
    assert worst <= bound, where


def test_fit_fitcheck_matches_oracle(ctx, K):
    """The tiny pair's fit check (fp32, 8 x 256 calibration tokens) end to end on the GPU:
    selection equal to the oracle's (and to the hidden layers), scores and maps within the
    fp32 bounds, holdout R^2 > 0.99999 through the GPU apply; a blocked run (selection blocks
    of 4 and map blocks of 4 target layers: ragged last blocks) and a run with the selection
    given agree with it."""
    cfg = FITCHECK
    pr, st, seqs = _pairs(cfg, "f32")
    got = _run_fit(ctx, cfg, seqs)
    ref = _oracle_fit(cfg, pr, st)
    assert np.array_equal(got["layer_sel"], ref["layer_sel"])
    assert np.array_equal(got["layer_sel"], pr["draws"]["true_sel"])
    ref_scores = _oracle_scores(cfg, pr, st, list(range(cfg.L_tgt)))
    serr = np.max(np.abs(got["scores"] - ref_scores))
    print(f"[fit] fitcheck scores: max |err| {serr:.2e}", flush=True)
    assert serr <= 1e-4
    _check_maps(got, ref, 2e-4, "fitcheck f32")
    # holdout through the GPU apply
    sel = got["layer_sel"]
    for s in range(pr["n_calib"], len(pr["pos"])):
        P = int(pr["pos"][s][0])
        ok_, ov_ = ctx.apply(_dev(pr["src_k"][s], "f32"), _dev(pr["src_v"][s], "f32"), sel,
                             *(torch.from_numpy(got[n]).cuda() for n in ("W_k", "b_k", "W_v", "b_v")),
                             cfg.theta_src, cfg.theta_tgt, pos0_src=P)
        torch.cuda.synchronize()
        gk, gv = ok_.double().cpu().numpy(), ov_.double().cpu().numpy()
        for t in range(cfg.L_tgt):
            kc = oracle.strip_rope(gk[t], pr["pos"][s], cfg.theta_tgt)
            r2 = np.concatenate([oracle.holdout_r2(pr["tgt_k_content"][s, t], kc),
                                 oracle.holdout_r2(pr["tgt_v"][s, t], gv[t])])
            assert r2.min() > 0.99999, (s, t, r2)
    # The default run is the one-pass mode (maps gathered from the full source Gram); the same
    # fit in two passes (forced, or by blocks of target layers) and from a given selection
    # computes every co-moment from the same products, so it agrees to fp32 rounding of the
    # merges; blocked and unblocked two-pass runs are bit-identical.
    two = _run_fit(ctx, cfg, seqs, two_pass=True)
    blocked = _run_fit(ctx, cfg, seqs, select_block=4, map_block=4)
    given = _run_fit(ctx, cfg, seqs, layer_sel=torch.from_numpy(got["layer_sel"]), map_block=5)
    assert given["scores"] is None
    for run in (two, blocked):
        assert np.array_equal(run["layer_sel"], got["layer_sel"])
        assert np.max(np.abs(run["scores"] - got["scores"])) <= 1e-9
    for n in ("W_k", "b_k", "W_v", "b_v"):
        assert np.array_equal(blocked[n], two[n]), n
        assert np.array_equal(given[n], two[n]), n
        rel = max(np.linalg.norm(two[n][t] - got[n][t]) / np.linalg.norm(got[n][t]) for t in range(cfg.L_tgt))
        print(f"[fit] one pass vs two passes {n}: rel {rel:.2e}", flush=True)
        assert rel <= 1e-5, n


def test_fit_bf16_matches_oracle(ctx):
    """bf16 caches (H = 4, d = 128, 6 source and 4 target layers, k = 2, 4 x 1024 calibration
    tokens at theta 1e6 -> 5e5): selection equal, scores and maps within the bf16 bounds;
    maps written in fp32 and in bf16 from the same statistics (the latter the fp32 maps
    rounded once)."""
    cfg = FITCHECK.replace(cid=11, L_src=6, L_tgt=4, H=4, d=128, k=2, T=1024, n_calib=4, holdout_pos0=(),
                           theta_src=1.0e6, theta_tgt=5.0e5, noise_sd=1e-2)
    pr, st, seqs = _pairs(cfg, "bf16")
    got = _run_fit(ctx, cfg, seqs, out_dtype=torch.float32)
    ref = _oracle_fit(cfg, pr, st)
    assert np.array_equal(got["layer_sel"], ref["layer_sel"])
    ref_scores = _oracle_scores(cfg, pr, st, list(range(cfg.L_tgt)))
    serr = np.max(np.abs(got["scores"] - ref_scores))
    print(f"[fit] bf16 scores: max |err| {serr:.2e}", flush=True)
    assert serr <= 1e-3
    _check_maps(got, ref, 5e-3, "bf16 caches, fp32 maps")
    # the same fit (given selection: same statistics) with maps written in fp32 and in bf16
    sel_t = torch.from_numpy(got["layer_sel"])
    g32 = _run_fit(ctx, cfg, seqs, out_dtype=torch.float32, layer_sel=sel_t)
    gb = _run_fit(ctx, cfg, seqs, out_dtype=torch.bfloat16, layer_sel=sel_t)
    for n in ("W_k", "b_k", "W_v", "b_v"):
        w32 = g32[n].astype(np.float64)
        assert np.all(np.abs(gb[n] - w32) <= 2.0 ** -8 * np.abs(w32) + 1e-30), n


def _random_fit_configs(n=6):
    """Seeded random small fits: 2-8 source and 1-6 target layers, k 1-3, 1-4 heads, d 64 or 128,
    256 or 512 tokens per sequence and enough sequences for n >= 4 p, fp32 or bf16 caches."""
    rng = np.random.default_rng([2026, 703])
    thetas = [1.0e4, 5.0e5, 1.0e6]
    out = []
    for i in range(n):
        L_src = int(rng.integers(2, 9))
        k = int(rng.integers(1, min(3, L_src) + 1))
        H = int(rng.integers(1, 5))
        d = int(rng.choice([64, 128]))
        T = int(rng.choice([256, 512]))
        dtype = "f32" if rng.random() < 0.5 else "bf16"
        n_calib = max(2, -(-4 * k * H * d // T))
        cfg = FITCHECK.replace(cid=600 + i, L_src=L_src, L_tgt=int(rng.integers(1, 7)), H=H, d=d, k=k, T=T,
                               n_calib=n_calib, holdout_pos0=(), theta_src=float(rng.choice(thetas)),
                               theta_tgt=float(rng.choice(thetas)), noise_sd=1e-3 if dtype == "f32" else 1e-2)
        out.append((cfg, dtype))
    return out


@pytest.mark.parametrize("cfg,dtype", _random_fit_configs(),
                         ids=lambda v: f"L{v.L_src}-{v.L_tgt}-k{v.k}-H{v.H}-d{v.d}-T{v.T}x{v.n_calib}"
                         if hasattr(v, "L_src") else str(v))
def test_fit_random_shapes(ctx, cfg, dtype):
    """Selection equal to the oracle's and to the hidden layers; scores and maps within the
    fp32 or bf16 bounds above."""
    pr, st, seqs = _pairs(cfg, dtype)
    got = _run_fit(ctx, cfg, seqs, out_dtype=torch.float32)
    ref = _oracle_fit(cfg, pr, st)
    assert np.array_equal(got["layer_sel"], ref["layer_sel"])
    assert np.array_equal(got["layer_sel"], pr["draws"]["true_sel"])
    ref_scores = _oracle_scores(cfg, pr, st, list(range(cfg.L_tgt)))
    serr = np.max(np.abs(got["scores"] - ref_scores))
    print(f"[fit] random {cfg.cid} {dtype}: scores max |err| {serr:.2e}", flush=True)
    assert serr <= (1e-4 if dtype == "f32" else 1e-3)
    _check_maps(got, ref, 2e-4 if dtype == "f32" else 5e-3, f"random {cfg.cid} {dtype}")
    # the blocked two-pass mode with random block sizes: the same selection and scores; maps
    # from statistics merged in another order, each within the 1e-5 statistics bar, so within
    # the kappa x 2e-5 = 2e-4 bound above (n = 4 p here: less well conditioned than the fit check)
    rng = np.random.default_rng([2026, 709, cfg.cid])
    two = _run_fit(ctx, cfg, seqs, out_dtype=torch.float32, two_pass=True,
                   select_block=int(rng.integers(1, cfg.L_tgt + 1)), map_block=int(rng.integers(1, cfg.L_tgt + 1)))
    assert np.array_equal(two["layer_sel"], got["layer_sel"])
    assert np.max(np.abs(two["scores"] - got["scores"])) <= 1e-6
    for n in ("W_k", "b_k", "W_v", "b_v"):
        rel = max(np.linalg.norm(two[n][t] - got[n][t]) / np.linalg.norm(got[n][t]) for t in range(cfg.L_tgt))
        assert rel <= 2e-4, (n, rel)


def test_fit_selection_full_target_width(ctx):
    """Stage-1 states at the 14B->32B width: 64 target layers of H = 8, d = 128 in one block
    (q = 65536 outputs per state), 2 source layers, k = 1, bf16, 2048 tokens.  Every target
    layer selects its hidden source; scores of sampled target layers (first, middle, last)
    against the oracle."""
    cfg = FITCHECK.replace(cid=12, L_src=2, L_tgt=64, H=8, d=128, k=1, T=1024, n_calib=2, holdout_pos0=(),
                           theta_src=1.0e6, theta_tgt=1.0e6, noise_sd=1e-2)
    pr, st, seqs = _pairs(cfg, "bf16")
    got = _run_fit(ctx, cfg, seqs, out_dtype=torch.bfloat16)
    assert np.array_equal(got["layer_sel"], pr["draws"]["true_sel"])
    targets = [0, 31, 63]
    ref_scores = _oracle_scores(cfg, pr, st, targets)
    serr = np.max(np.abs(got["scores"][targets] - ref_scores))
    print(f"[fit] full-width selection: scores {ref_scores.ravel()}, max |err| {serr:.2e}", flush=True)
    assert serr <= 1e-3


def test_fit_refusals(ctx, K):
    cfg = FITCHECK
    pr, st, seqs = _pairs(cfg, "f32")
    base = dict(L_src=cfg.L_src, L_tgt=cfg.L_tgt, H=cfg.H, d=cfg.d, k=cfg.k, theta_src=cfg.theta_src,
                theta_tgt=cfg.theta_tgt, lam=cfg.lam)
    for bad, status in ((dict(k=5), K.ERR_SHAPE), (dict(d=96), K.ERR_UNSUPPORTED), (dict(lam=-1.0), K.ERR_INVALID_ARGUMENT),
                        (dict(select_block=300), K.ERR_SHAPE)):
        kw = {**base, **bad}
        with pytest.raises(K.KvmapError) as e:
            ctx.fit(lambda: seqs, **kw)
        assert e.value.status == status, bad
    sel = torch.tensor([[0, 0]] * cfg.L_tgt, dtype=torch.int32)
    with pytest.raises(K.KvmapError) as e:
        ctx.fit(lambda: seqs, layer_sel=sel, **base)
    assert e.value.status == K.ERR_SHAPE
    # a pass that sees fewer tokens than the first (two passes: the one-pass mode has no second)
    calls = []

    def shrinking():
        calls.append(1)
        return seqs if len(calls) == 1 else seqs[:-1]

    with pytest.raises(K.KvmapError) as e:
        ctx.fit(shrinking, two_pass=True, **base)
    assert e.value.status == K.ERR_SHAPE
    assert len(calls) == 2


def test_ridge_batches_equal_single_solves(ctx, K):
    """kvmap_ridge_solve_device_batch / kvmap_ridge_r2_batch over 18 states (two batches: at most
    16 systems share the kernels) give bit for bit the single-system results; a state that is not
    positive definite is named in the refusal."""
    states = []
    for i in range(18):
        X, Y = _xy(300 + 7 * i, 72, 24, seed=100 + i)
        st = ctx.gram_state(72, 24, keep_ss_y=True)
        ctx.gram_reset(st)
        ctx.gram(st, _dev(X, "f32"), _dev(Y, "f32"))
        states.append(st)
    outs = ctx.ridge_solve_device_batch(states, 0.01, dtype=torch.float32)
    r2s = ctx.ridge_r2_batch(states, 0.01, 8)
    for st, (W, b), r2 in zip(states, outs, r2s):
        W1, b1 = ctx.ridge_solve_device(st, 0.01, dtype=torch.float32)
        assert torch.equal(W, W1) and torch.equal(b, b1)
        assert torch.equal(r2, ctx.ridge_r2(st, 0.01, 8))
    empty = ctx.gram_state(72, 24, keep_ss_y=True)
    ctx.gram_reset(empty)
    with pytest.raises(K.KvmapError) as e:
        ctx.ridge_solve_device_batch(states[:3] + [empty], 0.0)
    assert e.value.status == K.ERR_NOT_SPD and "system 3" in str(e.value)


def test_fit_two_source_groups(ctx):
    """130 source layers of H 2 x d 64 exceed one selection state's 128 row layers: two groups
    of source layers (128 + 2), so the fit runs in two passes (block-diagonal selection states,
    then per-target statistics).  Selection and maps against the oracle at the fp32 bounds."""
    cfg = FITCHECK.replace(cid=13, L_src=130, L_tgt=3, holdout_pos0=())
    pr, st, seqs = _pairs(cfg, "f32")
    passes = []
    res = ctx.fit(lambda: seqs, L_src=cfg.L_src, L_tgt=cfg.L_tgt, H=cfg.H, d=cfg.d, k=cfg.k,
                  theta_src=cfg.theta_src, theta_tgt=cfg.theta_tgt, lam=cfg.lam,
                  on_pass=lambda *a: passes.append(a))
    torch.cuda.synchronize()
    assert [p_[0] for p_ in passes] == [1, 2, 0], passes
    ref = _oracle_fit(cfg, pr, st)
    assert np.array_equal(res["layer_sel"].cpu().numpy(), ref["layer_sel"])
    assert np.array_equal(ref["layer_sel"], pr["draws"]["true_sel"])
    ref_scores = _oracle_scores(cfg, pr, st, list(range(cfg.L_tgt)))
    serr = np.max(np.abs(res["scores"].cpu().numpy() - ref_scores))
    got = {n: res[n].cpu().numpy() for n in ("W_k", "b_k", "W_v", "b_v")}
    print(f"[fit] two source groups: scores max |err| {serr:.2e}", flush=True)
    assert serr <= 1e-4
    _check_maps(got, ref, 2e-4, "two source groups")
