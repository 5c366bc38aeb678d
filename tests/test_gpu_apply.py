"""kvmap_apply on the GPU against the fp64 oracle, element by element.

Small configurations are compared in full; the full-size Qwen3 14B->32B and
Llama-3.1 8B->70B shapes are compared on sampled token rows (each output row depends
only on its own source row and position, so a sampled row is exact) and via the
determinism property that holds at any size.
"""

import numpy as np
import pytest

import oracle
from gpu_common import Tally, compare, to_f64
from synth.device import apply_inputs, device_apply_inputs
from synth.workloads import APPLY_CONFIGS, ApplyConfig, b_layer, layer_sel, src_layer, to_f64 as s2f, w_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ctx():
    from cross_model_kv_amd import kvmap as K
    c = K.Context(0)
    yield c
    c.close()


def _run(ctx, cfg, inp, **kw):
    print(f"[apply] {cfg.name} T={cfg.T} L={cfg.L_src}->{cfg.L_tgt} H={cfg.H} d={cfg.d} k={cfg.k} {cfg.dtype}",
          flush=True)
    out = ctx.apply(inp["src_k"], inp["src_v"], inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"],
                    inp["b_v"], cfg.theta_src, cfg.theta_tgt, pos0_src=cfg.pos0, **kw)
    torch.cuda.synchronize()
    return out


def _host(cfg):
    """Full host copies (float64) of a small configuration's inputs, drawn independently of the GPU."""
    f = lambda a: s2f(a, cfg.dtype)
    return dict(
        src_k=np.stack([f(src_layer(cfg, "k", l)) for l in range(cfg.L_src)]),
        src_v=np.stack([f(src_layer(cfg, "v", l)) for l in range(cfg.L_src)]),
        W_k=np.stack([f(w_layer(cfg, "k", t)) for t in range(cfg.L_tgt)]),
        W_v=np.stack([f(w_layer(cfg, "v", t)) for t in range(cfg.L_tgt)]),
        b_k=np.stack([f(b_layer(cfg, "k", t)) for t in range(cfg.L_tgt)]),
        b_v=np.stack([f(b_layer(cfg, "v", t)) for t in range(cfg.L_tgt)]),
        layer_sel=layer_sel(cfg),
    )


def _full_check(ctx, cfg, targets=None):
    inp = apply_inputs(cfg, "cuda:0")
    ok_, ov_ = _run(ctx, cfg, inp)
    h = _host(cfg)
    ref = oracle.apply(h["src_k"], h["src_v"], h["layer_sel"], h["W_k"], h["b_k"], h["W_v"], h["b_v"],
                       cfg.theta_src, cfg.theta_tgt, pos0_src=cfg.pos0, targets=targets)
    report, worst = compare(to_f64(ok_), to_f64(ov_), ref, cfg.dtype)
    print(f"[apply] worst {worst}", flush=True)
    assert not report, "\n".join(report[:20])
    return inp, ok_, ov_


def test_tiny_fp32_pair(ctx):
    """The tiny fp32 pair (4 -> 6 layers, H=2, d=64, T=256, k=2), every element."""
    _full_check(ctx, APPLY_CONFIGS[1])


EDGE = [
    # ragged token tail, 1.5 feature tiles (H=3), L_tgt > L_src
    ApplyConfig(201, "ragged-T300-H3", 5, 7, 3, 128, 300, 2, 1.0e4, 1.0e6, "bf16", 0.5),
    # head dim 64 in bf16, a single token, k = 3
    ApplyConfig(202, "d64-T1", 4, 3, 2, 64, 1, 3, 1.0e4, 5.0e5, "bf16", 0.5),
    # continuation offset: positions start at 1000, different bases, k = 1
    ApplyConfig(203, "pos0-1000-k1", 3, 2, 2, 128, 257, 1, 1.0e4, 5.0e5, "bf16", 0.5, pos0=1000),
    # fp32 with d = 128 and a ragged tail
    ApplyConfig(204, "fp32-d128-T70", 3, 2, 2, 128, 70, 2, 1.0e6, 1.0e6, "f32", 0.5),
    # one head, d = 64 (N = 64: a partial feature tile), many K-steps (k*H*d = 320)
    ApplyConfig(205, "H1-d64-k5", 6, 2, 1, 64, 513, 5, 1.0e4, 1.0e4, "bf16", 0.5),
    # several token blocks and heads, small enough for the full oracle
    ApplyConfig(206, "bf16-T1100-H8", 6, 3, 8, 128, 1100, 2, 1.0e6, 1.0e6, "bf16", 0.5),
    # every source layer selected (k = L_src), one token past the short-cache limit
    ApplyConfig(207, "k-all-T129", 3, 2, 2, 128, 129, 3, 1.0e4, 1.0e6, "bf16", 0.5),
    # the short-cache kernel at its limit with k = L_src and head dim 64
    ApplyConfig(208, "short-T128-k-all-d64", 4, 3, 2, 64, 128, 4, 1.0e4, 5.0e5, "bf16", 0.5),
    # positions from one million: large angles, different bases
    ApplyConfig(209, "pos0-1M", 3, 2, 2, 128, 300, 2, 1.0e4, 1.0e6, "bf16", 0.5, pos0=1_000_000),
    # fp32 with a single token and every layer selected
    ApplyConfig(210, "fp32-T1-k-all", 2, 3, 1, 64, 1, 2, 1.0e4, 5.0e5, "f32", 0.0),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_edge_cases(ctx, cfg):
    _full_check(ctx, cfg)


def _random_configs(n=24):
    """Seeded random small shapes: layer counts, heads, head dim, k, cache length on both sides
    of the short-cache limit, bases, position offsets, channel scales and dtype."""
    rng = np.random.default_rng([2026, 700])
    out = []
    for i in range(n):
        L_src = int(rng.integers(1, 10))
        k = int(rng.integers(1, min(L_src, 6) + 1))
        H = int(rng.integers(1, 6))
        d = int(rng.choice([64, 128]))
        T = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 700))]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        thetas = [1.0e4, 5.0e5, 1.0e6]
        out.append(ApplyConfig(300 + i, f"rand{i}-L{L_src}-{k}-H{H}-d{d}-T{T}-{dtype}", L_src,
                               int(rng.integers(1, 7)), H, d, T, k, float(rng.choice(thetas)),
                               float(rng.choice(thetas)), dtype, float(rng.choice([0.0, 0.5])),
                               pos0=int(rng.choice([0, int(rng.integers(1, 100_000))]))))
    return out


@pytest.mark.parametrize("cfg", _random_configs(), ids=lambda c: c.name)
def test_random_shapes(ctx, cfg):
    """Every element against the oracle, for each seeded random shape."""
    _full_check(ctx, cfg)


def test_qwen3_small_pair_full_layers(ctx):
    """Qwen3 0.6B -> 1.7B shape (28 -> 28, H=8, d=128, T=4096, k=4): every element of every
    target layer, K and V, against the oracle (in groups of 4 target layers); the outputs are
    filled with NaN before the apply, so an element it never wrote fails."""
    cfg = APPLY_CONFIGS[2]
    inp = apply_inputs(cfg, "cuda:0")
    ok_ = torch.full((cfg.L_tgt, cfg.H, cfg.T, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    ov_ = torch.full_like(ok_, float("nan"))
    _run(ctx, cfg, inp, out_k=ok_, out_v=ov_)
    assert bool(torch.isfinite(ok_).all()) and bool(torch.isfinite(ov_).all())
    tally = Tally()
    for t0 in range(0, cfg.L_tgt, 4):
        _check_sampled(cfg, inp, ok_, ov_, targets=list(range(t0, min(cfg.L_tgt, t0 + 4))), rows=np.arange(cfg.T),
                       tally=tally)
    print(f"[apply] {cfg.name} every element: {tally.summary()}", flush=True)


def _check_sampled(cfg, inp, ok_, ov_, targets, rows, tally=None):
    rows_t = torch.as_tensor(rows, device="cuda:0")
    sel = inp["layer_sel"]
    need = sorted({int(s) for t in targets for s in sel[t]})
    sk = {s: to_f64(inp["src_k"][s][:, rows_t, :]) for s in need}
    sv = {s: to_f64(inp["src_v"][s][:, rows_t, :]) for s in need}
    Wk = {t: to_f64(inp["W_k"][t]) for t in targets}
    Wv = {t: to_f64(inp["W_v"][t]) for t in targets}
    bk = {t: to_f64(inp["b_k"][t]) for t in targets}
    bv = {t: to_f64(inp["b_v"][t]) for t in targets}
    ref = oracle.apply_rows(sk, sv, sel, Wk, bk, Wv, bv, cfg.theta_src, cfg.theta_tgt, cfg.pos0 + rows,
                            targets=targets)
    gk = {t: to_f64(ok_[t][:, rows_t, :]) for t in targets}
    gv = {t: to_f64(ov_[t][:, rows_t, :]) for t in targets}
    report, worst = compare(gk, gv, ref, cfg.dtype, tally=tally)
    print(f"[apply] sampled {len(rows)} rows x {len(targets)} layers: worst {worst}", flush=True)
    assert not report, "\n".join(report[:20])


def test_identity_map_copies_values_bit_exact(ctx):
    """k = 1, W = I, b = 0, equal bases: values come back bit-exact; keys (stripped, rounded to
    bf16 and re-rotated) within one bf16 step of each pair's norm."""
    cfg = ApplyConfig(210, "identity", 3, 3, 2, 128, 333, 1, 1.0e6, 1.0e6, "bf16", 0.5)
    inp = apply_inputs(cfg, "cuda:0")
    N = cfg.N
    eye = torch.eye(N, dtype=torch.bfloat16, device="cuda:0")
    for t in range(cfg.L_tgt):
        inp["W_k"][t].copy_(eye)
        inp["W_v"][t].copy_(eye)
    inp["b_k"].zero_()
    inp["b_v"].zero_()
    ok_, ov_ = _run(ctx, cfg, inp)
    for t in range(cfg.L_tgt):
        s = int(inp["layer_sel"][t][0])
        assert torch.equal(ov_[t], inp["src_v"][s])
        x = inp["src_k"][s].float()
        err = (ok_[t].float() - x).abs()
        half = cfg.d // 2
        pair = torch.sqrt(x[..., :half] ** 2 + x[..., half:] ** 2).repeat(1, 1, 2)
        # the de-rotated key is stored in bf16 before rotating back: one bf16 step of the pair norm
        assert float((err / pair.clamp_min(1e-6)).max()) <= 2.0 ** -7


def test_deterministic_and_stream_ordered(ctx):
    """Two applies give bit-identical outputs (no atomics in the apply path); a second call on a
    side stream is ordered by that stream."""
    cfg = EDGE[0]
    inp = apply_inputs(cfg, "cuda:0")
    a = _run(ctx, cfg, inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = ctx.apply(inp["src_k"], inp["src_v"], inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"],
                      inp["b_v"], cfg.theta_src, cfg.theta_tgt, stream=s)
    s.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_check_finite_flag_and_refusal_leaves_outputs(ctx):
    from cross_model_kv_amd import kvmap as K
    cfg = EDGE[0]
    inp = apply_inputs(cfg, "cuda:0")
    ok_, ov_ = _run(ctx, cfg, inp, flags=K.FLAG_CHECK_FINITE)
    inp["src_v"][:, 0, 5, 3] = float("nan")
    with pytest.raises(K.KvmapError) as e:
        _run(ctx, cfg, inp, out_k=ok_, out_v=ov_, flags=K.FLAG_CHECK_FINITE)
    assert e.value.status == K.ERR_NONFINITE
    # a refused call (duplicate selection) touches nothing
    before = ok_.clone()
    bad = inp["layer_sel"].copy()
    bad[0, 1] = bad[0, 0]
    with pytest.raises(K.KvmapError) as e:
        ctx.apply(inp["src_k"], inp["src_v"], bad, inp["W_k"], inp["b_k"], inp["W_v"], inp["b_v"],
                  cfg.theta_src, cfg.theta_tgt, out_k=ok_, out_v=ov_)
    assert e.value.status == K.ERR_SHAPE
    torch.cuda.synchronize()
    assert torch.equal(before, ok_)


def _block_rows(T, block=256, seed=0):
    """One row from every 256-token block (the map GEMM's token tile), at a seeded offset inside
    the block, plus the first and the last row of the cache."""
    rng = np.random.default_rng([2026, 77, seed])
    rows = [b + int(rng.integers(0, min(block, T - b))) for b in range(0, T, block)]
    return np.unique(np.array(rows + [0, T - 1]))


@pytest.mark.parametrize("cid", [3, 4])
def test_full_size_sampled(ctx, cid):
    """The full Qwen3 14B->32B (T=32768) and Llama-3.1 8B->70B (T=16384) shapes, in the launch
    configuration the bench times.
      * Coverage: the outputs are filled with NaN before the apply, and afterwards no element of
        either cache may be non-finite, so every output tile was written.
      * Every target layer, K and V, every head, on one row of every 256-token block plus the
        first and last rows: each (target layer, K|V, token block, feature tile) tile of the GEMM
        is checked against the oracle on at least one row.
      * Windows of 24 consecutive rows at the start, middle and end of four target layers.
      * Every element of the first and the last target layer, K and V (the first and the last
        (t, K|V) pairs of the tile walk), checked in chunks of 4096 rows.
      * A second apply gives bit-identical outputs.
    The elements with |ref| >= 8 are counted and their errors printed per block."""
    cfg = APPLY_CONFIGS[cid]
    print(f"[apply] generating {cfg.name}", flush=True)
    inp = apply_inputs(cfg, "cuda:0")
    shape = (cfg.L_tgt, cfg.H, cfg.T, cfg.d)
    ok_ = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    ov_ = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    _run(ctx, cfg, inp, out_k=ok_, out_v=ov_)
    assert bool(torch.isfinite(ok_).all()) and bool(torch.isfinite(ov_).all()), "an output tile was not written"
    T = cfg.T
    tally = Tally()
    rows = _block_rows(T, seed=cid)
    print(f"[apply] {len(rows)} rows (one per token block) x all {cfg.L_tgt} target layers", flush=True)
    for t0 in range(0, cfg.L_tgt, 8):
        _check_sampled(cfg, inp, ok_, ov_, list(range(t0, min(t0 + 8, cfg.L_tgt))), rows, tally)
    rows = np.unique(np.concatenate([np.arange(0, 24), np.arange(T // 2 - 12, T // 2 + 12), np.arange(T - 24, T)]))
    targets = [0, cfg.L_tgt // 3, (2 * cfg.L_tgt) // 3, cfg.L_tgt - 1]
    _check_sampled(cfg, inp, ok_, ov_, targets, rows, tally)
    for t in (0, cfg.L_tgt - 1):
        for r0 in range(0, T, 4096):
            _check_sampled(cfg, inp, ok_, ov_, [t], np.arange(r0, min(r0 + 4096, T)), tally)
    print(f"[apply] {cfg.name} total: {tally.summary()}", flush=True)
    # determinism at full size
    ok2, ov2 = _run(ctx, cfg, inp)
    assert torch.equal(ok_, ok2) and torch.equal(ov_, ov2)


def test_largest_cache(ctx):
    """The largest cache the boundary accepts at head dim 128: T = 2^24 - 1 tokens, one layer and
    one head (k = 1), so T * d sits just under the 2^31 limit, the 32-bit byte offsets of the
    gathered rows reach their top, the last token block is ragged (255 tokens) and the RoPE
    positions run to 1.7e7.  Inputs are drawn on the device.  Every output element is written
    (NaN prefill); one row of every 256-token block, the first 256 and the last 300 rows are
    checked against the oracle."""
    cfg = ApplyConfig(231, "max-T", 1, 1, 1, 128, (1 << 24) - 1, 1, 1.0e4, 1.0e6, "bf16", 0.0)
    assert cfg.T * cfg.d < 2 ** 31 <= (cfg.T + 1) * cfg.d
    print(f"[apply] generating {cfg.name} on the device", flush=True)
    inp = device_apply_inputs(cfg)
    shape = (cfg.L_tgt, cfg.H, cfg.T, cfg.d)
    ok_ = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    ov_ = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    _run(ctx, cfg, inp, out_k=ok_, out_v=ov_)
    assert bool(torch.isfinite(ok_).all()) and bool(torch.isfinite(ov_).all()), "an output tile was not written"
    rows = np.unique(np.concatenate([_block_rows(cfg.T, seed=231), np.arange(256), np.arange(cfg.T - 300, cfg.T)]))
    tally = Tally()
    _check_sampled(cfg, inp, ok_, ov_, [0], rows, tally)
    print(f"[apply] {cfg.name} total: {tally.summary()}", flush=True)
    del inp, ok_, ov_
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [300, 100])
def test_largest_map(ctx, T):
    """The largest map the boundary accepts at d 128 and k 64: H = 45 heads, so N * F =
    5760 * 368,640 = 2,123,366,400 sits just under 2^31 (4.25 GB per map) and the 32-bit byte
    offsets of the map rows reach their top.  T = 300 runs the tiled kernel (a ragged second
    token block, a half-filled last feature tile), T = 100 the short-cache kernel.  Inputs are
    drawn on the device.  Every output element is written (NaN prefill); six rows of heads 0, 1,
    22 and 44, K and V, are checked against the oracle, which maps those heads' rows of W."""
    cfg = ApplyConfig(232, f"max-map-T{T}", 64, 1, 45, 128, T, 64, 1.0e4, 1.0e6, "bf16", 0.0)
    assert cfg.N * cfg.F < 2 ** 31 <= (cfg.N + cfg.d) * (cfg.F + cfg.k * cfg.d)
    print(f"[apply] generating {cfg.name} on the device", flush=True)
    inp = device_apply_inputs(cfg)
    shape = (cfg.L_tgt, cfg.H, cfg.T, cfg.d)
    ok_ = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    ov_ = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    _run(ctx, cfg, inp, out_k=ok_, out_v=ov_)
    assert bool(torch.isfinite(ok_).all()) and bool(torch.isfinite(ov_).all()), "an output tile was not written"
    rows = np.array(sorted({0, 1, T // 3, T // 2 + 1, T - 2, T - 1}))
    heads = [0, 1, 22, 44]
    rows_t = torch.as_tensor(rows, device="cuda:0")
    sel = [int(s) for s in inp["layer_sel"][0]]
    pos = cfg.pos0 + rows
    xk = oracle.feature_rows([oracle.strip_rope(to_f64(inp["src_k"][s][:, rows_t, :]), pos, cfg.theta_src) for s in sel])
    xv = oracle.feature_rows([to_f64(inp["src_v"][s][:, rows_t, :]) for s in sel])
    n_idx = torch.as_tensor(np.concatenate([np.arange(h * cfg.d, (h + 1) * cfg.d) for h in heads]), device="cuda:0")
    R, nh = len(rows), len(heads)
    heads_of = lambda y: y.reshape(R, nh, cfg.d).transpose(1, 0, 2)  # [R][nh*d] -> [nh][R][d]
    yk = oracle.affine(xk, to_f64(inp["W_k"][0][n_idx]), to_f64(inp["b_k"][0][n_idx]))
    yv = oracle.affine(xv, to_f64(inp["W_v"][0][n_idx]), to_f64(inp["b_v"][0][n_idx]))
    ref = {0: (oracle.rope(heads_of(yk), pos, cfg.theta_tgt), heads_of(yv))}
    h_t = torch.as_tensor(heads, device="cuda:0")
    gk = {0: to_f64(ok_[0][h_t][:, rows_t, :])}
    gv = {0: to_f64(ov_[0][h_t][:, rows_t, :])}
    tally = Tally()
    report, worst = compare(gk, gv, ref, cfg.dtype, tally=tally)
    print(f"[apply] {cfg.name}: {R} rows x heads {heads}: worst {worst}; {tally.summary()}", flush=True)
    assert not report, "\n".join(report[:20])
    del inp, ok_, ov_
    torch.cuda.empty_cache()


def test_alternating_selections_queue_without_host_wait(ctx):
    """Applies with selections the context has not seen are queued behind 30 ms of other work on
    the same stream: the host returns while that work is still running (the selection goes up
    through pinned staging with an asynchronous copy, not a stream synchronisation), and each
    queued apply gives the outputs of the same apply run alone."""
    cfg = EDGE[5]
    inp = apply_inputs(cfg, "cuda:0")
    sels = [np.array([[0, 5], [1, 4], [2, 3]], np.int32), np.array([[5, 0], [3, 1], [4, 2]], np.int32),
            np.array([[1, 2], [0, 3], [5, 4]], np.int32)]
    args = lambda sel: (inp["src_k"], inp["src_v"], sel, inp["W_k"], inp["b_k"], inp["W_v"], inp["b_v"],
                        cfg.theta_src, cfg.theta_tgt)
    alone = []
    for sel in sels:  # warms the tables and the workspace too
        alone.append(ctx.apply(*args(sel)))
        torch.cuda.synchronize()
    # the module's earlier tests filled the context's slots with other selections; these three
    # must be uploaded again after 8 others have pushed them out
    rng = np.random.default_rng([2026, 78])
    others = set()
    while len(others) < 8:
        cand = tuple(int(v) for v in rng.permutation(6))
        if all(cand != tuple(s.ravel()) for s in sels):
            others.add(cand)
    for o in sorted(others):
        ctx.apply(*args(np.array(o, np.int32).reshape(3, 2)))
    torch.cuda.synchronize()
    a = torch.randn(8192, 8192, device="cuda:0", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for _ in range(50):
        a = a @ a.T.contiguous() * 1e-4  # ~30 ms of queued work ahead of the applies
    queued = [ctx.apply(*args(sel)) for sel in (sels[0], sels[1], sels[2], sels[0])]
    still_busy = not stream.query()
    torch.cuda.synchronize()
    assert still_busy, "the host waited for the stream inside kvmap_apply"
    for (gk, gv), (rk, rv) in zip(queued, alone + alone[:1]):
        assert torch.equal(gk, rk) and torch.equal(gv, rv)


# ---- short caches (T <= 128: the persistent short-cache kernel; a separate reduce when the
# K reduction is split or the tile holds 16 or 32 tokens) ---

SHORT = [
    # 1.5 feature tiles (H=3), 64 tokens: exactly one 64-token tile, L_tgt > L_src
    ApplyConfig(221, "short-T64-H3", 5, 7, 3, 128, 64, 2, 1.0e4, 1.0e6, "bf16", 0.5),
    # d = 64, ragged 37 tokens, continuation offset, k = 3
    ApplyConfig(222, "short-d64-T37-pos0", 4, 3, 2, 64, 37, 3, 1.0e6, 5.0e5, "bf16", 0.5, pos0=1000),
    # 256 tokens (past the short path: the long-cache kernel), H = 8
    ApplyConfig(223, "short-T256-H8", 4, 2, 8, 128, 256, 2, 1.0e6, 1.0e6, "bf16", 0.5),
    # ragged 100 tokens in one 128-token tile (the 3-stage ring, 2 token blocks per wave)
    ApplyConfig(228, "short-T100-H3", 5, 7, 3, 128, 100, 2, 1.0e4, 1.0e6, "bf16", 0.5, pos0=33),
    # exactly 128 tokens, head dim 64, k = 3
    ApplyConfig(229, "short-T128-d64", 4, 5, 2, 64, 128, 3, 1.0e6, 5.0e5, "bf16", 0.5),
    # 128-token tiles with 4 splits and 5 work items per workgroup (as short-many-items-T16)
    ApplyConfig(230, "short-many-items-T100", 3, 80, 4, 128, 100, 1, 1.0e4, 1.0e6, "bf16", 0.5),
    # one head of d = 64 (N = 64, a partial feature tile), k = 5 (320 features: 5 K-steps)
    ApplyConfig(224, "short-H1-d64-k5-T129", 6, 2, 1, 64, 129, 5, 1.0e4, 1.0e4, "bf16", 0.5),
    # 320 tiles (80 target layers x K/V x 2 feature tiles) on a 256-CU device: the K reduction
    # is split 4 ways and every workgroup streams 5 work items (tiles of different target
    # layers, K/V and splits) through one ring
    ApplyConfig(226, "short-many-items-T16", 3, 80, 4, 128, 16, 1, 1.0e4, 1.0e6, "bf16", 0.5),
    # head dim 64, 3 selected layers, T = 5: 12 splits of one K-step each, so consecutive
    # items of a workgroup read different (selected layer, head) slabs
    ApplyConfig(227, "short-many-items-k3-T5", 4, 48, 4, 64, 5, 3, 1.0e6, 5.0e5, "bf16", 0.5, pos0=7),
    # Unsplit K reductions at 64- and 128-token tiles, where the short-cache kernel adds the bias,
    # rotates the keys and writes bf16 itself (no reduce kernel), on a 256-CU device:
    # 256 tiles (64 target layers x K/V x 2 feature tiles, the second half past N = 384), ragged
    # 100 tokens in a 128-token tile
    ApplyConfig(233, "short-fused-T100-H3", 6, 64, 3, 128, 100, 2, 1.0e4, 1.0e6, "bf16", 0.5, pos0=5),
    # the same at head dim 64 (N = 320: the second feature tile holds one head), ragged 50
    # tokens in a 64-token tile
    ApplyConfig(234, "short-fused-d64-T50-H5", 5, 64, 5, 64, 50, 2, 1.0e6, 5.0e5, "bf16", 0.5),
    # a single K-step (k = 1, one head of 64): one head in the first wave of the tile, the rest
    # of the tile past N
    ApplyConfig(235, "short-fused-one-kstep-T40", 2, 3, 1, 64, 40, 1, 1.0e4, 1.0e4, "bf16", 0.5, pos0=3),
]


@pytest.mark.parametrize("cfg", SHORT, ids=lambda c: c.name)
def test_short_caches(ctx, cfg):
    _full_check(ctx, cfg)


@pytest.mark.parametrize("T", [1, 16, 64, 128])
def test_short_cache_full_layer_shape(ctx, T):
    """The Qwen3 14B->32B layer shape (L 40->64, H 8, d 128, k 8) at T = 1, 16, 64 and 128, where
    every workgroup streams two whole tiles through its ring: every row of sampled target
    layers against the oracle, and bit-identical outputs on a second call (the partial sums
    are added in a fixed order)."""
    cfg = APPLY_CONFIGS[3].replace(cid=225, name=f"qwen3-14b-to-32b-T{T}", T=T)
    inp = apply_inputs(cfg, "cuda:0")
    ok_, ov_ = _run(ctx, cfg, inp)
    targets = [0, 21, 42, 63]
    _check_sampled(cfg, inp, ok_, ov_, targets, np.arange(cfg.T))
    ok2, ov2 = _run(ctx, cfg, inp)
    assert torch.equal(ok_, ok2) and torch.equal(ov_, ov2)


def test_aliasing_refused_and_outputs_untouched(ctx):
    """An output that overlaps an input (here the first target layers written over the source
    cache) or the other output is refused before any device work; nothing is written."""
    from cross_model_kv_amd import kvmap as K
    cfg = EDGE[5]  # 6 source layers, 3 target layers: a [3][H][T][d] view of the source fits
    inp = apply_inputs(cfg, "cuda:0")
    src_before = inp["src_k"].clone()
    args = (inp["src_k"], inp["src_v"], inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"], inp["b_v"],
            cfg.theta_src, cfg.theta_tgt)
    ov = torch.empty((cfg.L_tgt, cfg.H, cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(K.KvmapError) as e:
        ctx.apply(*args, out_k=inp["src_k"][: cfg.L_tgt], out_v=ov)
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    ok_ = torch.empty_like(ov)
    with pytest.raises(K.KvmapError) as e:
        ctx.apply(*args, out_k=ok_, out_v=ok_)
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.equal(inp["src_k"], src_before)


def test_timing_ring():
    """kvmap_last_timings / kvmap_timings: nothing held before a timed apply; the RoPE-table
    time is reported only by the apply that built the tables; untimed applies do not enter the
    ring; the ring holds the last 128 timed applies and refuses older ones; every duration read
    back is finite and non-negative, the kernels' positive."""
    from cross_model_kv_amd import kvmap as K
    cfg = EDGE[0]  # ragged T, bf16: de-rotation and the long-cache GEMM
    inp = apply_inputs(cfg, "cuda:0")
    c = K.Context(0)
    try:
        with pytest.raises(K.KvmapError):
            c.last_timings()
        with pytest.raises(K.KvmapError):
            c.timings(0)
        _run(c, cfg, inp, flags=K.FLAG_TIMING)
        first = c.last_timings()
        _run(c, cfg, inp)  # untimed: not recorded
        _run(c, cfg, inp, flags=K.FLAG_TIMING)
        second = c.last_timings()
        print(f"[timing] first {first}, second {second}", flush=True)
        assert first[0] > 0 and second[0] == 0.0  # tables built once, then cached
        for t in (first, second):
            assert all(np.isfinite(v) and v >= 0 for v in t) and t[1] > 0 and t[2] > 0
        assert c.timings(0) == second and c.timings(1) == first
        with pytest.raises(K.KvmapError):
            c.timings(2)
        with pytest.raises(K.KvmapError):
            c.timings(-1)
        for _ in range(130):
            c.apply(inp["src_k"], inp["src_v"], inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"], inp["b_v"],
                    cfg.theta_src, cfg.theta_tgt, pos0_src=cfg.pos0, flags=K.FLAG_TIMING)
        torch.cuda.synchronize()
        assert c.timings(127)[2] > 0
        with pytest.raises(K.KvmapError):
            c.timings(128)
    finally:
        c.close()


def test_two_contexts_two_threads():
    """Two contexts driven from two host threads at once, each on its own stream, with different
    shapes: every output equals the same apply run alone (contexts share no state)."""
    import threading
    from cross_model_kv_amd import kvmap as K
    cfgs = (EDGE[5], EDGE[0])
    inps = [apply_inputs(c, "cuda:0") for c in cfgs]
    ref = []
    for c, inp in zip(cfgs, inps):
        cx = K.Context(0)
        ref.append(_run(cx, c, inp))
        cx.close()
    ctxs = [K.Context(0) for _ in cfgs]
    streams = [torch.cuda.Stream() for _ in cfgs]
    outs = [[None] * 4 for _ in cfgs]
    errors = []

    def worker(w):
        try:
            c, inp = cfgs[w], inps[w]
            for it in range(4):
                ok_ = torch.empty((c.L_tgt, c.H, c.T, c.d), dtype=torch.bfloat16, device="cuda:0")
                ov_ = torch.empty_like(ok_)
                ctxs[w].apply(inp["src_k"], inp["src_v"], inp["layer_sel"], inp["W_k"], inp["b_k"], inp["W_v"],
                              inp["b_v"], c.theta_src, c.theta_tgt, pos0_src=c.pos0, out_k=ok_, out_v=ov_,
                              stream=streams[w])
                outs[w][it] = (ok_, ov_)
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(w,)) for w in range(len(cfgs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for c in ctxs:
        c.close()
    assert not errors, errors
    for w in range(len(cfgs)):
        for ok_, ov_ in outs[w]:
            assert torch.equal(ok_, ref[w][0]) and torch.equal(ov_, ref[w][1])
