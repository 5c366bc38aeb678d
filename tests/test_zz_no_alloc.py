"""kvmap_gram_noalloc (statistics through the library's static device scratch, for callers that
cannot allocate) against kvmap_gram through the C ABI: two calls in a row on one state, the
second smaller, at a shape where every batch fits one static sub-batch (bit-identical) and at
the 14B->32B fit-statistics shape, where a 4096-row batch is merged in static sub-batches
(within the 1e-5 Gram bar of kvmap_gram's state).  Plus the refusal of a state too wide for the
static scratch, which leaves the state untouched."""

import numpy as np
import pytest

from synth.workloads import FIT_STATS_CONFIG, bf16_bits_to_f64, fit_batch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GRAM_REL = 1e-5


@pytest.fixture(scope="module")
def ctx():
    from cross_model_kv_amd import kvmap as K
    c = K.Context(0)
    yield c
    c.close()


def _rows(cfg, n, first_batch=0):
    xs, ys, b = [], [], first_batch
    while sum(len(x) for x in xs) < n:
        x, y = fit_batch(cfg, b)
        xs.append(bf16_bits_to_f64(x)); ys.append(bf16_bits_to_f64(y))
        b += 1
    return np.concatenate(xs)[:n], np.concatenate(ys)[:n]


def _dev(a, dtype):
    t = torch.from_numpy(a.astype(np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def _pair(ctx, p, q):
    from cross_model_kv_amd import kvmap as K
    a = K.GramState(p, q, "cuda:0", keep_ss_y=True)
    b = K.GramState(p, q, "cuda:0", keep_ss_y=True)
    ctx.gram_reset(a)
    ctx.gram_reset(b)
    return a, b


def _fields(st):
    return {k: getattr(st, k) for k in ("mean_x", "mean_y", "M_xx", "M_xy", "ss_y")}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_gram_bit_for_bit(ctx, dtype):
    """p 520, q 68: calls of 1262 then 37 rows, each within one static sub-batch, give the
    same state bits as kvmap_gram."""
    cfg = FIT_STATS_CONFIG.replace(cid=421, p=520, q=68, n_tokens=2000, batch=700)
    X, Y = _rows(cfg, 1299)
    a, b = _pair(ctx, cfg.p, cfg.q)
    for r0, r1 in ((0, 1262), (1262, 1299)):
        print(f"[noalloc] {dtype} p={cfg.p} q={cfg.q} rows {r0}..{r1}", flush=True)
        x, y = _dev(X[r0:r1], dtype), _dev(Y[r0:r1], dtype)
        ctx.gram(a, x, y)
        ctx.gram_noalloc(b, x, y)
        torch.cuda.synchronize()
        assert a.n == b.n == r1
        fa, fb = _fields(a), _fields(b)
        for k in fa:
            assert torch.equal(fa[k], fb[k]), k


def _random_cases(n=8):
    """Seeded random shapes small enough that every call fits one static sub-batch: p and q
    multiples of 4 (p + q at most 2,400), two calls of 1-900 rows, the second smaller."""
    rng = np.random.default_rng([2026, 710])
    out = []
    for i in range(n):
        p, q = 4 * int(rng.integers(1, 401)), 4 * int(rng.integers(1, 201))
        r1 = int(rng.integers(2, 901))
        out.append((i, p, q, r1, int(rng.integers(1, r1)), "f32" if rng.random() < 0.3 else "bf16"))
    return out


@pytest.mark.parametrize("i,p,q,r1,r2,dtype", _random_cases())
def test_noalloc_random_shapes_bit_for_bit(ctx, i, p, q, r1, r2, dtype):
    """Two calls in a row, the second smaller, give the same state bits as kvmap_gram."""
    cfg = FIT_STATS_CONFIG.replace(cid=560 + i, p=p, q=q, n_tokens=r1 + r2, batch=1024,
                                   nnz=min(FIT_STATS_CONFIG.nnz, p // 2))
    X, Y = _rows(cfg, r1 + r2)
    a, b = _pair(ctx, p, q)
    for s0, s1 in ((0, r1), (r1, r1 + r2)):
        print(f"[noalloc] random {i}: {dtype} p={p} q={q} rows {s0}..{s1}", flush=True)
        x, y = _dev(X[s0:s1], dtype), _dev(Y[s0:s1], dtype)
        ctx.gram(a, x, y)
        ctx.gram_noalloc(b, x, y)
        torch.cuda.synchronize()
        assert a.n == b.n == s1
        fa, fb = _fields(a), _fields(b)
        for k in fa:
            assert torch.equal(fa[k], fb[k]), k


def test_noalloc_sub_batches_at_fit_shape(ctx):
    """p 8192, q 1024 (the 14B->32B fit statistics), bf16: a 4096-row call (three static
    sub-batches of at most 1664 rows), then a 1000-row call (one), against kvmap_gram's state
    after each call: n exact, M_xx / M_xy / ss_y within 1e-5 relative Frobenius, means within
    1e-5 of their largest magnitude."""
    cfg = FIT_STATS_CONFIG
    a, b = _pair(ctx, cfg.p, cfg.q)
    X, Y = _rows(cfg, 5096)
    for r0, r1 in ((0, 4096), (4096, 5096)):
        print(f"[noalloc] bf16 p={cfg.p} q={cfg.q} rows {r0}..{r1}", flush=True)
        x, y = _dev(X[r0:r1], "bf16"), _dev(Y[r0:r1], "bf16")
        ctx.gram(a, x, y)
        ctx.gram_noalloc(b, x, y)
        torch.cuda.synchronize()
        assert a.n == b.n == r1
        fa, fb = _fields(a), _fields(b)
        for k in ("M_xx", "M_xy", "ss_y"):
            ra, rb = fa[k].double(), fb[k].double()
            rel = float(torch.linalg.norm(rb - ra) / torch.linalg.norm(ra))
            print(f"[noalloc]   {k}: rel Frobenius {rel:.2e}", flush=True)
            assert rel <= GRAM_REL, k
        for k in ("mean_x", "mean_y"):
            ra, rb = fa[k].double(), fb[k].double()
            rel = float((rb - ra).abs().max() / ra.abs().max())
            assert rel <= GRAM_REL, k


def test_noalloc_refuses_state_too_wide(ctx):
    """p 65536 + q 40000 needs more than the 64 MiB static scratch: UNSUPPORTED, state untouched."""
    from cross_model_kv_amd import kvmap as K
    st = K.GramState(65536, 40000, "cuda:0", xx_block=64)
    ctx.gram_reset(st)
    x = torch.zeros((64, 65536), dtype=torch.bfloat16, device="cuda:0")
    y = torch.zeros((64, 40000), dtype=torch.bfloat16, device="cuda:0")
    before = st.mean_x.clone()
    with pytest.raises(K.KvmapError) as e:
        ctx.gram_noalloc(st, x, y)
    assert e.value.status == K.ERR_UNSUPPORTED
    assert st.n == 0 and torch.equal(before, st.mean_x)
    del st
    torch.cuda.empty_cache()
