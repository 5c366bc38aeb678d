"""kvmap_gram / kvmap_gram_merge / kvmap_ridge_solve on the GPU against the fp64 oracle."""

import numpy as np
import pytest

import oracle
from synth.device import fit_inputs, host_to_tensor
from synth.workloads import FIT_STATS_CONFIG, FITCHECK, bf16_bits_to_f64, fit_batch, fit_hidden_map

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GRAM_REL = 1e-5


@pytest.fixture(scope="module")
def ctx():
    from cross_model_kv_amd import kvmap as K
    c = K.Context(0)
    yield c
    c.close()


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def _check_state(st, ref, where):
    torch.cuda.synchronize()
    assert st.n == ref["n"], where
    f = lambda t: t.double().cpu().numpy()
    r_xx, r_xy = _rel(f(st.M_xx), ref["Mxx"]), _rel(f(st.M_xy), ref["Mxy"])
    mx = np.max(np.abs(f(st.mean_x) - ref["mx"])) / np.max(np.abs(ref["mx"]))
    my = np.max(np.abs(f(st.mean_y) - ref["my"])) / np.max(np.abs(ref["my"]))
    print(f"[gram] {where}: rel M_xx {r_xx:.2e}  M_xy {r_xy:.2e}  mean_x {mx:.2e}  mean_y {my:.2e}", flush=True)
    assert r_xx <= GRAM_REL and r_xy <= GRAM_REL and mx <= GRAM_REL and my <= GRAM_REL, where
    # both triangles are stored
    Mxx = f(st.M_xx)
    assert np.array_equal(Mxx, Mxx.T) or np.max(np.abs(Mxx - Mxx.T)) <= 1e-6 * np.max(np.abs(Mxx))


SMALL = FIT_STATS_CONFIG.replace(cid=401, p=520, q=68, n_tokens=2000, batch=700)


def _batches(cfg, sizes, dtype="bf16"):
    """Batches of the given row counts cut from the seeded stream (bf16 or widened to fp32)."""
    xs, ys = [], []
    b = 0
    while sum(len(x) for x in xs) < sum(sizes):
        x, y = fit_batch(cfg, b)
        xs.append(bf16_bits_to_f64(x)); ys.append(bf16_bits_to_f64(y))
        b += 1
    X, Y = np.concatenate(xs), np.concatenate(ys)
    out, r = [], 0
    for n in sizes:
        out.append((X[r:r + n], Y[r:r + n]))
        r += n
    return out


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).cuda()
    return torch.from_numpy(a.astype(np.float32)).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gram_ragged_batches(ctx, dtype):
    """Batches of 700, 1, 37 and 1262 rows (p = 520, q = 68: not tile multiples), mean offset ~5."""
    parts = _batches(SMALL, [700, 1, 37, 1262])
    st = ctx.gram_state(SMALL.p, SMALL.q)
    ctx.gram_reset(st)
    for X, Y in parts:
        ctx.gram(st, _dev(X, dtype), _dev(Y, dtype))
    ref = oracle.stats_two_pass(np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    _check_state(st, ref, f"ragged {dtype}")


def _random_stats_configs(n=16):
    """Seeded random statistics calls: p and q (multiples of 4, not of the 256-wide tiles), one to
    four batches of 1 to 900 rows, bf16 or fp32, with or without ss_y."""
    rng = np.random.default_rng([2026, 701])
    out = []
    for i in range(n):
        p = 4 * int(rng.integers(1, 201))
        q = 4 * int(rng.integers(1, 101))
        sizes = [int(v) for v in rng.integers(1, 901, int(rng.integers(1, 5)))]
        dtype = "f32" if rng.random() < 0.3 else "bf16"
        out.append((i, p, q, sizes, dtype, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("i,p,q,sizes,dtype,ssy", _random_stats_configs())
def test_gram_random_shapes(ctx, i, p, q, sizes, dtype, ssy):
    """Every element of the state (and ss_y when kept) against the oracle's two-pass statistics."""
    cfg = FIT_STATS_CONFIG.replace(cid=500 + i, p=p, q=q, n_tokens=sum(sizes), batch=1024)
    parts = _batches(cfg, sizes)
    st = ctx.gram_state(p, q, keep_ss_y=ssy)
    ctx.gram_reset(st)
    for X, Y in parts:
        ctx.gram(st, _dev(X, dtype), _dev(Y, dtype))
    ref = oracle.stats_two_pass(np.concatenate([v[0] for v in parts]), np.concatenate([v[1] for v in parts]))
    _check_state(st, ref, f"random {i}: p {p} q {q} batches {sizes} {dtype}")
    if ssy:
        r = _rel(st.ss_y.double().cpu().numpy(), ref["ssy"])
        assert r <= GRAM_REL, f"ss_y {r:.2e}"


def test_gram_wide_state_every_element(ctx):
    """p = 6144, q = 1024 (396 co-moment tiles, more than one wave of the compute units), bf16
    batches of 1000, 300 and 1000 rows: the first shifted by its own column means, the merging
    ones by the running mean; every element against the oracle's two-pass statistics."""
    cfg = FIT_STATS_CONFIG.replace(cid=402, p=6144, q=1024, n_tokens=2300, batch=1000)
    parts = _batches(cfg, [1000, 300, 1000])
    st = ctx.gram_state(cfg.p, cfg.q)
    ctx.gram_reset(st)
    for X, Y in parts:
        ctx.gram(st, _dev(X, "bf16"), _dev(Y, "bf16"))
    ref = oracle.stats_two_pass(np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    _check_state(st, ref, "wide state")


def test_gram_call_larger_than_sub_batch(ctx):
    """One call of 16384 + 1000 + 3 rows (the library merges it in sub-batches of at most
    16384 rows), p = 264, q = 36 (q not a multiple of 8), bf16."""
    cfg = FIT_STATS_CONFIG.replace(cid=402, p=264, q=36, n_tokens=17387, batch=4096)
    (X, Y), = _batches(cfg, [17387])
    st = ctx.gram_state(cfg.p, cfg.q)
    ctx.gram_reset(st)
    ctx.gram(st, _dev(X, "bf16"), _dev(Y, "bf16"))
    _check_state(st, oracle.stats_two_pass(X, Y), "one call over sub-batches")


def test_gram_merge_and_resume(ctx):
    """Two states over disjoint halves merged = one state over the stream; an empty state merges
    as the identity; a state is a checkpoint (continue streaming after a merge)."""
    parts = _batches(SMALL, [500, 400, 300, 800])
    a, b, e = ctx.gram_state(SMALL.p, SMALL.q), ctx.gram_state(SMALL.p, SMALL.q), ctx.gram_state(SMALL.p, SMALL.q)
    for s in (a, b, e):
        ctx.gram_reset(s)
    ctx.gram(a, _dev(parts[0][0], "bf16"), _dev(parts[0][1], "bf16"))
    ctx.gram(b, _dev(parts[1][0], "bf16"), _dev(parts[1][1], "bf16"))
    ctx.gram(b, _dev(parts[2][0], "bf16"), _dev(parts[2][1], "bf16"))
    ctx.gram_merge(a, b)
    ctx.gram_merge(a, e)
    ctx.gram(a, _dev(parts[3][0], "bf16"), _dev(parts[3][1], "bf16"))
    ref = oracle.stats_two_pass(np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    _check_state(a, ref, "merge+resume")
    # merging into an empty state copies
    ctx.gram_merge(e, a)
    _check_state(e, ref, "merge into empty")


def test_fitcheck_on_gpu(ctx):
    """The tiny pair's fit check with GPU statistics and the library's ridge solve: maps that
    match the oracle's fit, and holdout R^2 > 0.99999 through the GPU apply."""
    from fitcheck_data import build_pairs
    cfg = FITCHECK
    pr = build_pairs(cfg)
    nc = pr["n_calib"]
    fit = oracle.fit_mapper(pr["src_k"][:nc], pr["src_v"][:nc], pr["tgt_k"][:nc], pr["tgt_v"][:nc],
                            pr["pos"][:nc], cfg.theta_src, cfg.theta_tgt, cfg.k, cfg.lam)
    sel = fit["layer_sel"]
    assert np.array_equal(sel, pr["draws"]["true_sel"])
    sk = np.stack([oracle.strip_rope(pr["src_k"][i], pr["pos"][i], cfg.theta_src) for i in range(nc)])
    tk = np.stack([oracle.strip_rope(pr["tgt_k"][i], pr["pos"][i], cfg.theta_tgt) for i in range(nc)])
    Wk = np.zeros((cfg.L_tgt, cfg.N, cfg.F), np.float32); Wv = np.zeros_like(Wk)
    bk = np.zeros((cfg.L_tgt, cfg.N), np.float32); bv = np.zeros_like(bk)
    for t in range(cfg.L_tgt):
        for src, tgt, W, b, ref_W in ((sk, tk, Wk, bk, fit["W_k"]), (pr["src_v"][:nc], pr["tgt_v"][:nc], Wv, bv, fit["W_v"])):
            X = np.concatenate([oracle.feature_rows([src[i, s] for s in sel[t]]) for i in range(nc)])
            Y = np.concatenate([oracle.feature_rows([tgt[i, t]]) for i in range(nc)])
            st = ctx.gram_state(cfg.F, cfg.N)
            ctx.gram_reset(st)
            for r in range(0, len(X), 512):
                ctx.gram(st, _dev(X[r:r + 512], "f32"), _dev(Y[r:r + 512], "f32"))
            W[t], b[t] = ctx.ridge_solve(st, cfg.lam)
            assert np.max(np.abs(W[t] - ref_W[t])) < 1e-3
    # holdout through the GPU apply (fp32 path)
    from cross_model_kv_amd import kvmap as K
    for s in range(nc, len(pr["pos"])):
        P = int(pr["pos"][s][0])
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        ok_, ov_ = ctx.apply(dev(pr["src_k"][s]), dev(pr["src_v"][s]), sel, dev(Wk), dev(bk), dev(Wv), dev(bv),
                             cfg.theta_src, cfg.theta_tgt, pos0_src=P)
        torch.cuda.synchronize()
        gk, gv = ok_.double().cpu().numpy(), ov_.double().cpu().numpy()
        for t in range(cfg.L_tgt):
            kc = oracle.strip_rope(gk[t], pr["pos"][s], cfg.theta_tgt)
            r2 = np.concatenate([oracle.holdout_r2(pr["tgt_k_content"][s, t], kc),
                                 oracle.holdout_r2(pr["tgt_v"][s, t], gv[t])])
            assert r2.min() > 0.99999, (s, t, r2)
    assert K.version() == 100


def test_fit_stats_full_size(ctx):
    """The fit-statistics stream at the 14B->32B shape: 262,144 tokens in batches of 4096,
    p = 8192, q = 1024, per-channel offsets ~N(5, 1).  Sampled 96 x 96 blocks of M_xx and
    96 x 64 of M_xy against the oracle's two-pass statistics of those columns; then the host
    ridge solve recovers the hidden sparse map."""
    cfg = FIT_STATS_CONFIG
    rng = np.random.default_rng(5)
    cx = np.sort(rng.choice(cfg.p, 96, replace=False))
    cy = np.sort(rng.choice(cfg.q, 64, replace=False))
    st = ctx.gram_state(cfg.p, cfg.q)
    ctx.gram_reset(st)
    hx, hy = [], []
    for b, X, Y in fit_inputs(cfg, range(cfg.n_batches)):
        ctx.gram(st, X, Y)
        hx.append(X[:, torch.as_tensor(cx, device=X.device)].double().cpu().numpy())
        hy.append(Y[:, torch.as_tensor(cy, device=Y.device)].double().cpu().numpy())
        if b % 16 == 0:
            print(f"[gram] batch {b}/{cfg.n_batches}", flush=True)
    torch.cuda.synchronize()
    ref = oracle.stats_two_pass(np.concatenate(hx), np.concatenate(hy))
    f = lambda t: t.double().cpu().numpy()
    Mxx = f(st.M_xx)[np.ix_(cx, cx)]
    Mxy = f(st.M_xy)[np.ix_(cx, cy)]
    r_xx, r_xy = _rel(Mxx, ref["Mxx"]), _rel(Mxy, ref["Mxy"])
    mx = np.max(np.abs(f(st.mean_x)[cx] - ref["mx"])) / np.max(np.abs(ref["mx"]))
    print(f"[gram] full size sampled: rel M_xx {r_xx:.2e} M_xy {r_xy:.2e} mean_x {mx:.2e}", flush=True)
    assert st.n == cfg.n_tokens
    assert r_xx <= GRAM_REL and r_xy <= GRAM_REL and mx <= GRAM_REL
    W, b = ctx.ridge_solve(st, cfg.lam)
    Wt, bt = fit_hidden_map(cfg)
    err = np.max(np.abs(W.T - Wt))
    print(f"[gram] ridge vs hidden map: max |W - W*| {err:.2e}", flush=True)
    assert err < 2e-3
    # the same solve on the device (fp64), fp32 and bf16 outputs
    Wd, bd = ctx.ridge_solve_device(st, cfg.lam, dtype=torch.float32)
    Wd, bd = Wd.double().cpu().numpy(), bd.double().cpu().numpy()
    rw, rb = _rel(Wd, W.astype(np.float64)), _rel(bd, b.astype(np.float64))
    errd = np.max(np.abs(Wd.T - Wt))
    print(f"[gram] device ridge vs host: rel W {rw:.2e} b {rb:.2e}; vs hidden map {errd:.2e}", flush=True)
    assert rw <= 1e-5 and rb <= 1e-5 and errd < 2e-3
    Wb, bb = ctx.ridge_solve_device(st, cfg.lam, dtype=torch.bfloat16)
    Wb = Wb.double().cpu().numpy()
    assert np.all(np.abs(Wb - W) <= 2.0 ** -8 * (1 + 1e-5) * np.abs(W) + 1e-30)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gram_largest_state(ctx, dtype):
    """The largest state the boundary accepts, p = q = 65,536 (M_xx and M_xy 17.2 GB each, element
    offsets past 2^32), with ss_y: batches of 300, 77 and 1 rows drawn on the device with
    per-column offsets ~N(5, 1), so the first goes into the empty state and the others merge.
    Sampled 96 x 96 of M_xx (both triangles), 96 x 64 of M_xy, the means and ss_y (first and last
    columns included) against the oracle's two-pass statistics of those columns."""
    from cross_model_kv_amd import kvmap as K
    p = q = 65536
    g = torch.Generator(device="cuda:0").manual_seed(2026604)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ox = 5.0 + torch.randn(p, generator=g, device="cuda:0")
    oy = 5.0 + torch.randn(q, generator=g, device="cuda:0")
    rng = np.random.default_rng([2026, 605])
    cx = np.unique(np.concatenate([[0, p - 1], rng.choice(p, 94, replace=False)]))
    cy = np.unique(np.concatenate([[0, q - 1], rng.choice(q, 62, replace=False)]))
    cx_t, cy_t = torch.as_tensor(cx, device="cuda:0"), torch.as_tensor(cy, device="cuda:0")
    st = ctx.gram_state(p, q, keep_ss_y=True)
    ctx.gram_reset(st)
    hx, hy = [], []
    for n_b in (300, 77, 1):
        X = (torch.randn((n_b, p), generator=g, device="cuda:0") + ox).to(dt)
        Y = (torch.randn((n_b, q), generator=g, device="cuda:0") + oy).to(dt)
        ctx.gram(st, X, Y)
        hx.append(X[:, cx_t].double().cpu().numpy())
        hy.append(Y[:, cy_t].double().cpu().numpy())
    torch.cuda.synchronize()
    ref = oracle.stats_two_pass(np.concatenate(hx), np.concatenate(hy))
    f = lambda t: t.double().cpu().numpy()
    Mxx = f(st.M_xx[cx_t][:, cx_t])
    Mxy = f(st.M_xy[cx_t][:, cy_t])
    r_xx, r_xy = _rel(Mxx, ref["Mxx"]), _rel(Mxy, ref["Mxy"])
    mx = np.max(np.abs(f(st.mean_x[cx_t]) - ref["mx"])) / np.max(np.abs(ref["mx"]))
    my = np.max(np.abs(f(st.mean_y[cy_t]) - ref["my"])) / np.max(np.abs(ref["my"]))
    r_ss = _rel(f(st.ss_y[cy_t]), ref["ssy"])
    print(f"[gram] largest state {dtype}: rel M_xx {r_xx:.2e} M_xy {r_xy:.2e} mean_x {mx:.2e} mean_y {my:.2e} "
          f"ss_y {r_ss:.2e}", flush=True)
    assert st.n == 378
    assert max(r_xx, r_xy, mx, my, r_ss) <= GRAM_REL
    assert np.max(np.abs(Mxx - Mxx.T)) <= 1e-6 * np.max(np.abs(Mxx))
    del st
    torch.cuda.empty_cache()


def test_ridge_device_largest_state(ctx):
    """kvmap_ridge_solve_device on the largest state the boundary accepts in p (65,536; q 256):
    the fp64 system alone is 34 GB and its element offsets pass 2^32.  The state comes from 2,048
    device-drawn rows (y a noisy multiple of the first q features).  With 2,048 rows M_xx has a
    63,000-dimensional null space, and the fp32 state's error (at most 1e-2 per entry, but about 13
    in spectral norm, measured against fp64 statistics of the same rows) leaves M_xx + lambda I
    indefinite for lambda below about 12.5: at lambda = 0.01 the solve refuses it with
    KVMAP_ERR_NOT_SPD (checked here), and it runs at lambda = 100.  No host solve finishes at this
    size, so W is checked by a property that holds at any size: the residual (M_xx + lambda I) W
    - M_xy, formed in fp64 from the state, relative to ||M_xx + lambda I|| ||W||, within a few
    fp32 roundings of W; and b = mean_y - mean_x W."""
    from cross_model_kv_amd import kvmap as K
    p, q, lam = 65536, 256, 100.0
    g = torch.Generator(device="cuda:0").manual_seed(2026606)
    st = ctx.gram_state(p, q)
    ctx.gram_reset(st)
    for n_b in (1024, 1024):
        X = (torch.randn((n_b, p), generator=g, device="cuda:0") + 1.0).to(torch.bfloat16)
        Y = (0.5 * X[:, :q].float() + 0.1 * torch.randn((n_b, q), generator=g, device="cuda:0")).to(torch.bfloat16)
        ctx.gram(st, X, Y)
    del X, Y
    with pytest.raises(K.KvmapError) as e:
        ctx.ridge_solve_device(st, 0.01, dtype=torch.float32)
    assert e.value.status == K.ERR_NOT_SPD
    W, b = ctx.ridge_solve_device(st, lam, dtype=torch.float32)  # W output-major [q][p]
    torch.cuda.synchronize()
    A = st.M_xx.double()
    A.diagonal().add_(lam)
    Wt = W.double().t().contiguous()
    res = float((A @ Wt - st.M_xy.double()).norm() / (A.norm() * Wt.norm()))
    b_ref = st.mean_y.double() - st.mean_x.double() @ Wt
    rb = float((b.double() - b_ref).norm() / b_ref.norm())
    print(f"[gram] device ridge, largest state: relative residual {res:.2e}, b {rb:.2e}", flush=True)
    assert res <= 1e-6 and rb <= 1e-5
    del A, Wt, st
    torch.cuda.empty_cache()


def test_ridge_solve_device_matches_oracle(ctx):
    """kvmap_ridge_solve_device on a GPU-built state (p = 520, q = 68: padded to multiples of
    128 inside, 10 blocks of 64 in 3 panels, so the 128-tile updates of the trailing matrix and
    of the right-hand sides run on partial panels), against the oracle's fp64 ridge on the same
    (fp32) statistics and against the host solver; lambda = 0.01 and a larger lambda."""
    from cross_model_kv_amd import kvmap as K
    parts = _batches(SMALL, [700, 1300])
    st = ctx.gram_state(SMALL.p, SMALL.q)
    ctx.gram_reset(st)
    for X, Y in parts:
        ctx.gram(st, _dev(X, "bf16"), _dev(Y, "bf16"))
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    stats = dict(n=st.n, mx=f(st.mean_x), my=f(st.mean_y), Mxx=np.triu(f(st.M_xx)) + np.triu(f(st.M_xx), 1).T,
                 Mxy=f(st.M_xy))
    for lam in (0.01, 3.0):
        Wr, br = oracle.ridge(stats, lam)  # W [p][q], b [q]
        Wd, bd = ctx.ridge_solve_device(st, lam, dtype=torch.float32)
        Wh, bh = ctx.ridge_solve(st, lam)
        rw, rb = _rel(f(Wd).T, Wr), _rel(f(bd), br)
        rh = _rel(f(Wd), Wh.astype(np.float64))
        print(f"[ridge] device lambda {lam}: rel W {rw:.2e} b {rb:.2e}; vs host {rh:.2e}", flush=True)
        assert rw <= 1e-5 and rb <= 1e-5 and rh <= 1e-5


def _random_ridge_cases(n=10):
    """Seeded random device solves: p (multiple of 4, up to 1200: one to 19 blocks of 64), q (up to
    400), n >= 4 p rows of bf16 or fp32 batches, lambda 0.01 or 3."""
    rng = np.random.default_rng([2026, 704])
    out = []
    for i in range(n):
        p = 4 * int(rng.integers(1, 301))
        q = 4 * int(rng.integers(1, 101))
        out.append((i, p, q, max(4 * p, 64), "f32" if rng.random() < 0.3 else "bf16", float(rng.choice([0.01, 3.0]))))
    # the smallest states and block edges: one padded 128-tile, exactly one and just past one
    # 64-wide block, q past one 128-tile
    for j, (p, q) in enumerate([(4, 4), (8, 4), (60, 12), (64, 64), (68, 132)]):
        out.append((n + j, p, q, max(4 * p, 64), "bf16" if j % 2 else "f32", 0.01))
    return out


@pytest.mark.parametrize("i,p,q,n,dtype,lam", _random_ridge_cases())
def test_ridge_device_random_shapes(ctx, i, p, q, n, dtype, lam):
    """W and b of the device solve against the oracle's fp64 ridge of the same fp32 statistics."""
    cfg = FIT_STATS_CONFIG.replace(cid=520 + i, p=p, q=q, n_tokens=n, batch=1024,
                                   nnz=min(FIT_STATS_CONFIG.nnz, p // 2))  # the hidden map's nonzeros per column
    st = ctx.gram_state(p, q)
    ctx.gram_reset(st)
    for X, Y in _batches(cfg, [n]):
        ctx.gram(st, _dev(X, dtype), _dev(Y, dtype))
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    stats = dict(n=st.n, mx=f(st.mean_x), my=f(st.mean_y), Mxx=np.triu(f(st.M_xx)) + np.triu(f(st.M_xx), 1).T,
                 Mxy=f(st.M_xy))
    Wr, br = oracle.ridge(stats, lam)
    Wd, bd = ctx.ridge_solve_device(st, lam, dtype=torch.float32)
    rw, rb = _rel(f(Wd).T, Wr), _rel(f(bd), br)
    print(f"[ridge] random {i}: p {p} q {q} n {n} {dtype} lambda {lam}: rel W {rw:.2e} b {rb:.2e}", flush=True)
    assert rw <= 1e-5 and rb <= 1e-5


def test_ridge_solve_device_not_spd(ctx):
    """An empty state with lambda = 0 has a zero pivot: KVMAP_ERR_NOT_SPD."""
    from cross_model_kv_amd import kvmap as K
    st = ctx.gram_state(64, 8)
    ctx.gram_reset(st)
    with pytest.raises(K.KvmapError) as e:
        ctx.ridge_solve_device(st, 0.0)
    assert e.value.status == K.ERR_NOT_SPD


# positions of a planted bad entry: each 16-wide sub-block of the first 64-wide diagonal block,
# the first row of the second block, a later block, and the last row (second panel of 4 blocks)
_BAD_AT = [0, 5, 17, 40, 63, 64, 130, 299]


@pytest.mark.parametrize("kind", ["negative", "zero", "nan", "inf", "nan-off-diagonal"])
def test_ridge_device_refuses_bad_pivots(ctx, kind):
    """The diagonal factor flags a system whose pivot is not positive and finite, wherever it
    falls: M_xx + lambda I with a negative, zero (M_xx_jj = -lambda and row j zero), NaN or +inf
    diagonal entry, or a NaN off the diagonal (row j, column j / 2), at positions in every
    16-wide sub-block of a 64-wide diagonal block, in later blocks and in the second panel
    (p 300: 6 blocks): KVMAP_ERR_NOT_SPD.  The state restored, the solve gives its result again
    (lambda 0.5, exact in fp32, so that the zero case is an exact zero pivot)."""
    from cross_model_kv_amd import kvmap as K
    p, q, lam = 300, 16, 0.5
    rng = np.random.default_rng(2026)
    X = rng.standard_normal((900, p))
    Y = X[:, :q] * 0.5 + 0.1 * rng.standard_normal((900, q))
    st = ctx.gram_state(p, q)
    ctx.gram_reset(st)
    ctx.gram(st, _dev(X, "f32"), _dev(Y, "f32"))
    W0, b0 = ctx.ridge_solve_device(st, lam, dtype=torch.float32)
    for j in _BAD_AT:
        saved = st.M_xx.clone()
        if kind == "negative":
            st.M_xx[j, j] = -1e4
        elif kind == "zero":
            st.M_xx[j, :] = 0.0
            st.M_xx[:, j] = 0.0
            st.M_xx[j, j] = -lam
        elif kind == "nan":
            st.M_xx[j, j] = float("nan")
        elif kind == "inf":
            st.M_xx[j, j] = float("inf")
        else:
            m = j // 2 if j else 1
            st.M_xx[j, m] = float("nan")
            st.M_xx[m, j] = float("nan")
        print(f"[ridge] bad pivot {kind} at {j}", flush=True)
        with pytest.raises(K.KvmapError) as e:
            ctx.ridge_solve_device(st, lam, dtype=torch.float32)
        assert e.value.status == K.ERR_NOT_SPD, (kind, j)
        st.M_xx.copy_(saved)
    W1, b1 = ctx.ridge_solve_device(st, lam, dtype=torch.float32)
    assert torch.equal(W0, W1) and torch.equal(b0, b1)


@pytest.mark.parametrize("dtype,bd", [("bf16", 64), ("bf16", 256), ("f32", 64), ("f32", 128)])
def test_gram_block_diagonal_state(ctx, dtype, bd):
    """A state that keeps M_xx only on its diagonal blocks (xx_block): each block equals the
    oracle's M_xx block of the full two-pass statistics, M_xy, the means and ss_y are those of
    the full state; a merge of two blocked states too.  p = 512 in blocks of 64 (not a tile
    multiple: tiles reach past a block and are masked) or of 128 / 256."""
    cfg = FIT_STATS_CONFIG.replace(cid=403, p=512, q=72, n_tokens=1500, batch=700)
    parts = _batches(cfg, [700, 800])
    a = ctx.gram_state(cfg.p, cfg.q, keep_ss_y=True, xx_block=bd)
    b = ctx.gram_state(cfg.p, cfg.q, keep_ss_y=True, xx_block=bd)
    ctx.gram_reset(a)
    ctx.gram_reset(b)
    ctx.gram(a, _dev(parts[0][0], dtype), _dev(parts[0][1], dtype))
    ctx.gram(b, _dev(parts[1][0], dtype), _dev(parts[1][1], dtype))
    ctx.gram_merge(a, b)
    torch.cuda.synchronize()
    ref = oracle.stats_two_pass(np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    f = lambda t: t.double().cpu().numpy()
    Mxx = f(a.M_xx)
    assert Mxx.shape == (cfg.p // bd, bd, bd)
    worst = 0.0
    for g in range(cfg.p // bd):
        blk = ref["Mxx"][g * bd:(g + 1) * bd, g * bd:(g + 1) * bd]
        worst = max(worst, _rel(Mxx[g], blk))
    r_xy = _rel(f(a.M_xy), ref["Mxy"])
    r_ss = _rel(f(a.ss_y), ref["ssy"])
    print(f"[gram] blocked {dtype} bd {bd}: worst block rel {worst:.2e}, M_xy {r_xy:.2e}, ss_y {r_ss:.2e}", flush=True)
    assert worst <= GRAM_REL and r_xy <= GRAM_REL and r_ss <= GRAM_REL
    assert np.max(np.abs(f(a.mean_x) - ref["mx"])) <= GRAM_REL * np.max(np.abs(ref["mx"]))


def _random_merge_cases(n=10):
    """Seeded random merges: 2-4 states of 1-2 batches each (1-500 rows), full or block-diagonal
    M_xx (blocks of 4-256 features, a multiple of 4), bf16 or fp32, all merged into the first."""
    rng = np.random.default_rng([2026, 708])
    out = []
    for i in range(n):
        bd = 0 if rng.random() < 0.4 else 4 * int(rng.integers(1, 65))
        p = (bd * int(rng.integers(1, 9))) if bd else 4 * int(rng.integers(1, 151))
        q = 4 * int(rng.integers(1, 41))
        states = [[int(v) for v in rng.integers(1, 501, int(rng.integers(1, 3)))] for _ in range(int(rng.integers(2, 5)))]
        out.append((i, p, q, bd, states, "f32" if rng.random() < 0.3 else "bf16"))
    return out


@pytest.mark.parametrize("i,p,q,bd,states,dtype", _random_merge_cases())
def test_gram_random_merges(ctx, i, p, q, bd, states, dtype):
    """The merged state equals the oracle's two-pass statistics of all the rows: M_xx (or its
    diagonal blocks), M_xy, the means, ss_y and n."""
    sizes = [n for s_ in states for n in s_]
    cfg = FIT_STATS_CONFIG.replace(cid=540 + i, p=p, q=q, n_tokens=sum(sizes), batch=1024,
                                   nnz=min(FIT_STATS_CONFIG.nnz, p // 2))
    parts = _batches(cfg, sizes)
    sts, k = [], 0
    for s_ in states:
        st = ctx.gram_state(p, q, keep_ss_y=True, xx_block=bd)
        ctx.gram_reset(st)
        for _ in s_:
            ctx.gram(st, _dev(parts[k][0], dtype), _dev(parts[k][1], dtype))
            k += 1
        sts.append(st)
    for st in sts[1:]:
        ctx.gram_merge(sts[0], st)
    torch.cuda.synchronize()
    a = sts[0]
    ref = oracle.stats_two_pass(np.concatenate([v[0] for v in parts]), np.concatenate([v[1] for v in parts]))
    f = lambda t: t.double().cpu().numpy()
    assert a.n == sum(sizes)
    if bd:
        Mxx = f(a.M_xx)
        r_xx = max(_rel(Mxx[g], ref["Mxx"][g * bd:(g + 1) * bd, g * bd:(g + 1) * bd]) for g in range(p // bd))
    else:
        r_xx = _rel(f(a.M_xx), ref["Mxx"])
    r_xy, r_ss = _rel(f(a.M_xy), ref["Mxy"]), _rel(f(a.ss_y), ref["ssy"])
    mx = np.max(np.abs(f(a.mean_x) - ref["mx"])) / np.max(np.abs(ref["mx"]))
    my = np.max(np.abs(f(a.mean_y) - ref["my"])) / np.max(np.abs(ref["my"]))
    print(f"[gram] random merge {i}: p {p} q {q} bd {bd} states {states} {dtype}: M_xx {r_xx:.2e} "
          f"M_xy {r_xy:.2e} ss_y {r_ss:.2e}", flush=True)
    assert max(r_xx, r_xy, r_ss, mx, my) <= GRAM_REL


def test_gram_merge_refuses_overlapping_states(ctx):
    """A merge whose source shares memory with its destination is refused before any device
    work, and the destination is left as it was."""
    from cross_model_kv_amd import kvmap as K
    (X, Y), = _batches(SMALL, [300])
    a = ctx.gram_state(SMALL.p, SMALL.q)
    ctx.gram_reset(a)
    ctx.gram(a, _dev(X, "bf16"), _dev(Y, "bf16"))
    b = ctx.gram_state(SMALL.p, SMALL.q)
    ctx.gram_reset(b)
    ctx.gram(b, _dev(X, "bf16"), _dev(Y, "bf16"))
    torch.cuda.synchronize()
    before = a.M_xx.clone()
    b.c.M_xy = a.M_xx.data_ptr() + 4096  # b's cross-moments over a's Gram
    with pytest.raises(K.KvmapError) as e:
        ctx.gram_merge(a, b)
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    with pytest.raises(K.KvmapError):
        ctx.gram_merge(a, a)
    torch.cuda.synchronize()
    assert torch.equal(a.M_xx, before) and a.n == 300


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gram_smallest_state(ctx, dtype):
    """p = q = 4 (the smallest state: one partial tile each way), batches of 1, 5 and 33 rows
    with the fit-statistics offsets, against the oracle on every element."""
    cfg = FIT_STATS_CONFIG.replace(cid=403, p=4, q=4, n_tokens=64, batch=64, nnz=2)
    parts = _batches(cfg, [1, 5, 33])
    st = ctx.gram_state(cfg.p, cfg.q)
    ctx.gram_reset(st)
    for X, Y in parts:
        ctx.gram(st, _dev(X, dtype), _dev(Y, dtype))
    ref = oracle.stats_two_pass(np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    _check_state(st, ref, f"smallest {dtype}")
