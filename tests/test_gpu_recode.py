"""kvmap_recode (identity-map RoPE re-encode) on the GPU against the fp64 oracle.

The oracle side strips the source RoPE and applies the target RoPE as two rotations
(oracle.strip_rope, oracle.rope); the kernel does one rotation per pair by the angle
difference from an fp64-built table.  Bound per element: the bf16 result is the fp32
rotation rounded once to nearest (8 significant bits: at most 2^-8 of |r|, the unit
roundoff), plus the fp32 rotation's own error, taken as 1e-6 of the pair's norm; fp32
results carry only the latter.
"""

import numpy as np
import pytest

import oracle

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


def _src(rows, T, d, dtype, seed):
    x = np.random.default_rng([2026, 601, seed]).standard_normal((rows, T, d)).astype(np.float32) * 2.0
    t = torch.from_numpy(x)
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def _ref(x64, pos_s, pos_t, ts, tt):
    return oracle.rope(oracle.strip_rope(x64, pos_s, ts), pos_t, tt)


def _check(got, ref, dtype, where):
    g = got.float().cpu().double().numpy()
    d = ref.shape[-1]
    pair = np.sqrt(ref[..., : d // 2] ** 2 + ref[..., d // 2:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    bound = (2.0 ** -8 if dtype == "bf16" else 0.0) * np.abs(ref) + 1e-6 * pair + 1e-30
    err = np.abs(g - ref)
    worst = float(np.max(err / bound))
    print(f"[recode] {where}: max err {err.max():.3e}, worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0, where


CASES = [
    # rows, T, d, dtype, theta_s, theta_t, pos0_s, pos0_t
    (5, 300, 128, "bf16", 1.0e4, 1.0e6, 0, 0),
    (3, 70, 64, "bf16", 1.0e6, 5.0e5, 1000, 1000),
    (2, 1, 128, "f32", 1.0e4, 1.0e6, 37, 37),
    (4, 257, 64, "f32", 5.0e5, 1.0e6, 0, 12),
    (6, 4099, 128, "bf16", 1.0e4, 1.0e6, 28000, 28000),
]


@pytest.mark.parametrize("rows,T,d,dtype,ts,tt,ps,pt", CASES)
def test_recode_matches_oracle(ctx, rows, T, d, dtype, ts, tt, ps, pt):
    x = _src(rows, T, d, dtype, seed=rows * 7 + d)
    out = ctx.recode(x, ts, tt, pos0_src=ps, pos0_tgt=pt)
    torch.cuda.synchronize()
    x64 = x.float().cpu().double().numpy()
    ref = _ref(x64, ps + np.arange(T), pt + np.arange(T), ts, tt)
    _check(out, ref, dtype, f"rows {rows} T {T} d {d} {dtype} {ts:g}->{tt:g} pos0 {ps}->{pt}")


def _random_recode_cases(n=16):
    rng = np.random.default_rng([2026, 702])
    thetas = [1.0e4, 5.0e5, 1.0e6]
    out = []
    for i in range(n):
        out.append((int(rng.integers(1, 7)), int(rng.integers(1, 3000)), int(rng.choice([64, 128])),
                    "f32" if rng.random() < 0.3 else "bf16", float(rng.choice(thetas)), float(rng.choice(thetas)),
                    int(rng.choice([0, int(rng.integers(1, 200_000))])), int(rng.choice([0, int(rng.integers(1, 200_000))]))))
    return out


@pytest.mark.parametrize("rows,T,d,dtype,ts,tt,ps,pt", _random_recode_cases())
def test_recode_random_cases(ctx, rows, T, d, dtype, ts, tt, ps, pt):
    """Seeded random rows, lengths, head dims, dtypes, bases and position offsets; every element."""
    x = _src(rows, T, d, dtype, seed=rows * 31 + T)
    out = ctx.recode(x, ts, tt, pos0_src=ps, pos0_tgt=pt)
    torch.cuda.synchronize()
    x64 = x.float().cpu().double().numpy()
    ref = _ref(x64, ps + np.arange(T), pt + np.arange(T), ts, tt)
    _check(out, ref, dtype, f"rows {rows} T {T} d {d} {dtype} {ts:g}->{tt:g} pos0 {ps}->{pt}")


def test_recode_largest_cache(ctx):
    """One row of T = 2^24 - 1 tokens at d 128 (T * d just under 2^31, positions to 1.7e7 from
    pos0 1000), drawn on the device; 3 tokens of every 4096 and the last 300 are checked."""
    T, d = (1 << 24) - 1, 128
    g = torch.Generator(device="cuda:0").manual_seed(2026602)
    x = (torch.randn((1, T, d), generator=g, device="cuda:0") * 2.0).to(torch.bfloat16)
    out = ctx.recode(x, 1.0e4, 1.0e6, pos0_src=1000, pos0_tgt=1000)
    torch.cuda.synchronize()
    rng = np.random.default_rng([2026, 603])
    toks = np.unique(np.concatenate([rng.integers(0, T, 3 * (T // 4096)), np.arange(T - 300, T)]))
    idx = torch.as_tensor(toks, device="cuda:0")
    x64 = x[:, idx, :].float().cpu().double().numpy()
    ref = _ref(x64, 1000 + toks, 1000 + toks, 1.0e4, 1.0e6)
    _check(out[:, idx, :], ref, "bf16", f"T {T} d {d} bf16, {len(toks)} sampled tokens")
    del x, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_recode_equal_bases_is_a_copy(ctx, dtype):
    """theta and pos0 equal on both sides: the angle difference is exactly 0 in fp64, so the
    output must equal the input bit for bit."""
    x = _src(3, 129, 128, dtype, seed=5)
    out = ctx.recode(x, 1.0e6, 1.0e6, pos0_src=77, pos0_tgt=77)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if dtype == "bf16" else torch.int32),
                       x.view(torch.int16 if dtype == "bf16" else torch.int32))


def test_recode_refusals_leave_output(ctx, K):
    x = _src(2, 16, 128, "bf16", seed=9)
    out = torch.full_like(x, 3.0)
    before = out.clone()
    with pytest.raises(K.KvmapError) as e:
        ctx.recode(x, 1e4, 1e6, out=out, style_src=1)
    assert e.value.status == K.ERR_UNSUPPORTED
    with pytest.raises(K.KvmapError) as e:
        ctx.recode(x, -1.0, 1e6, out=out)
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    with pytest.raises(K.KvmapError) as e:
        ctx.recode(x, 1e4, 1e6, out=x)  # in place is an overlap
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    y = _src(2, 16, 96, "bf16", seed=9)
    with pytest.raises(K.KvmapError) as e:
        ctx.recode(y, 1e4, 1e6)
    assert e.value.status == K.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(out, before)


def test_recode_full_size_sampled(ctx):
    """The 14B source key cache shape: 40 layers x 8 heads = 320 rows, T = 32768, d = 128,
    bf16, theta 1e6 -> 5e5; sampled rows and tokens (first, last, ragged middle) against the
    oracle."""
    rows, T, d = 320, 32768, 128
    gen = torch.Generator(device="cuda").manual_seed(20260611)
    x = (torch.randn((rows, T, d), generator=gen, device="cuda") * 2.0).to(torch.bfloat16)
    out = ctx.recode(x, 1.0e6, 5.0e5)
    torch.cuda.synchronize()
    rsel = np.array([0, 1, 159, 318, 319])
    tsel = np.concatenate([np.arange(0, 40), np.arange(16380, 16420), np.arange(T - 40, T)])
    xs = x[torch.as_tensor(rsel)][:, torch.as_tensor(tsel)].float().cpu().double().numpy()
    gs = out[torch.as_tensor(rsel)][:, torch.as_tensor(tsel)]
    ref = _ref(xs, tsel, tsel, 1.0e6, 5.0e5)
    _check(gs, ref, "bf16", "full size sampled")
