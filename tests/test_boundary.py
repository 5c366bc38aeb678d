"""The C-ABI boundary on the CPU: the library loads, exports every declared entry point,
validates arguments on the host, and its host ridge solve matches the oracle."""

import os
import re

import numpy as np
import pytest

import oracle
from cross_model_kv_amd import kvmap as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvmap.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvmap_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = K.lib()
    names = _declared()
    assert "kvmap_apply" in names and "kvmap_gram" in names and len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert K.version() == 100
    assert K.status_string(K.OK) == "KVMAP_OK"
    assert K.status_string(K.ERR_NOT_SPD) == "KVMAP_ERR_NOT_SPD"
    assert K.status_string(99) == "KVMAP_ERR_UNKNOWN"


def test_create_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(K.KvmapError) as e:
        K.Context(0)
    assert e.value.status == K.ERR_DEVICE


GOOD = dict(L_src=6, L_tgt=4, H=2, d=128, k=3, T=100, dtype=K.BF16, theta_src=1e4, theta_tgt=5e5)


def _sel(L_t=4, k=3):
    return np.array([[0, 2, 5], [1, 3, 4], [5, 4, 3], [0, 1, 2]][:L_t], dtype=np.int32)[:, :k]


def _validate(**over):
    args = dict(GOOD)
    sel = over.pop("layer_sel", _sel())
    args.update(over)
    return K.validate_apply(args["L_src"], args["L_tgt"], args["H"], args["d"], args["k"], args["T"],
                            args["dtype"], sel, args["theta_src"], args["theta_tgt"],
                            args.get("pos0_src", 0), args.get("pos0_tgt", 0),
                            args.get("style_src", 0), args.get("style_tgt", 0),
                            args.get("inv_freq_src"), args.get("inv_freq_tgt"))


def test_validate_accepts_good_call():
    assert _validate() == K.OK
    assert _validate(d=64) == K.OK
    assert _validate(dtype=K.F32, T=1) == K.OK
    assert _validate(pos0_src=2048, pos0_tgt=2048) == K.OK


@pytest.mark.parametrize("over,status", [
    (dict(k=7, layer_sel=np.zeros((4, 7), np.int32)), K.ERR_SHAPE),              # k > L_src
    (dict(layer_sel=np.array([[0, 0, 1]] * 4, np.int32)), K.ERR_SHAPE),          # duplicate in a row
    (dict(layer_sel=np.array([[0, 1, 6]] * 4, np.int32)), K.ERR_SHAPE),          # out of range
    (dict(layer_sel=np.array([[0, 1, -1]] * 4, np.int32)), K.ERR_SHAPE),         # negative
    (dict(d=127), K.ERR_SHAPE),                                                  # odd head dim
    (dict(d=96), K.ERR_UNSUPPORTED),                                             # not built
    (dict(style_src=K.ROPE_INTERLEAVED), K.ERR_UNSUPPORTED),                     # traditional RoPE
    (dict(style_tgt=K.ROPE_INTERLEAVED), K.ERR_UNSUPPORTED),
    (dict(theta_src=0.0), K.ERR_INVALID_ARGUMENT),
    (dict(theta_tgt=float("nan")), K.ERR_INVALID_ARGUMENT),
    (dict(pos0_src=-1), K.ERR_INVALID_ARGUMENT),
    (dict(pos0_tgt=2 ** 31), K.ERR_INVALID_ARGUMENT),
    (dict(T=0), K.ERR_SHAPE),
    (dict(H=0), K.ERR_SHAPE),
    (dict(dtype=7), K.ERR_UNSUPPORTED),
])
def test_validate_refusals(over, status):
    assert _validate(**over) == status
    assert K.last_error() != ""


def _buffers(dtype=K.BF16, **over):
    """Addresses of a well-placed apply call at GOOD's shape (L 6 -> 4, H 2, d 128, k 3, T 100):
    every buffer in its own region, 16-byte aligned.  Nothing is ever read at them."""
    es = 2 if dtype == K.BF16 else 4
    H, d, T, k, Ls, Lt = GOOD["H"], GOOD["d"], GOOD["T"], GOOD["k"], GOOD["L_src"], GOOD["L_tgt"]
    N = H * d
    sizes = dict(src_k=Ls * H * T * d * es, src_v=Ls * H * T * d * es, W_k=Lt * N * N * k * es, b_k=Lt * N * es,
                 W_v=Lt * N * N * k * es, b_v=Lt * N * es, tgt_k=Lt * H * T * d * es, tgt_v=Lt * H * T * d * es)
    addr, base = {}, 1 << 40
    for name, n in sizes.items():
        addr[name] = base
        base += (n + 4095) // 4096 * 4096
    addr.update(over)
    return addr, sizes


def _validate_buffers(dtype=K.BF16, **over):
    a, _ = _buffers(dtype, **over)
    return K.validate_apply_buffers(GOOD["L_src"], GOOD["L_tgt"], GOOD["H"], GOOD["d"], GOOD["k"], GOOD["T"],
                                    dtype, a["src_k"], a["src_v"], a["W_k"], a["b_k"], a["W_v"], a["b_v"],
                                    a["tgt_k"], a["tgt_v"])


def test_validate_buffers_accepts_disjoint_aligned():
    assert _validate_buffers() == K.OK
    assert _validate_buffers(K.F32) == K.OK


def test_validate_buffers_refusals():
    """kvmap_apply's own buffer checks, run before any device work: NULL, misaligned, an output
    over an input (anywhere inside it, or straddling its end), the two outputs overlapping."""
    a, sz = _buffers()
    assert _validate_buffers(src_k=0) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_v=0) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(W_k=a["W_k"] + 8) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_k=a["src_k"]) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_k=a["src_v"] + sz["src_v"] - 16) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_v=a["W_v"] + 4096) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_v=a["b_k"]) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_v=a["tgt_k"] + sz["tgt_k"] - 16) == K.ERR_INVALID_ARGUMENT
    assert _validate_buffers(tgt_v=a["tgt_k"]) == K.ERR_INVALID_ARGUMENT
    assert K.last_error() != ""
    # exactly adjacent ranges do not overlap
    assert _validate_buffers(tgt_v=a["tgt_k"] + sz["tgt_k"]) == K.OK


def test_validate_frequency_lists():
    """A model's own frequency list replaces theta (which is then not read); entries must be
    finite and >= 0 (0: a pair that never turns)."""
    f = np.power(1.0e4, -2.0 * np.arange(64) / 128)
    assert _validate(theta_src=0.0, inv_freq_src=f) == K.OK
    assert _validate(theta_tgt=float("nan"), inv_freq_tgt=np.zeros(64)) == K.OK
    for bad in (-1e-3, float("nan"), float("inf")):
        g = f.copy()
        g[17] = bad
        assert _validate(inv_freq_src=g) == K.ERR_INVALID_ARGUMENT
        assert "inv_freq[17]" in K.last_error()


def test_fit_and_ridge_refuse_null_handles():
    """Host-side refusals of the fit driver and device ridge entry points (no GPU needed)."""
    L = K.lib()
    import ctypes
    h = ctypes.c_void_p()
    cfg = K.FitConfigC()
    assert L.kvmap_fit_create(None, ctypes.byref(cfg), ctypes.byref(h)) == K.ERR_INVALID_ARGUMENT
    assert h.value is None
    info = K.FitPassC()
    assert L.kvmap_fit_next_pass(None, ctypes.byref(info), None) == K.ERR_INVALID_ARGUMENT
    assert L.kvmap_fit_add(None, None, None, None, None, 16, 0, None) == K.ERR_INVALID_ARGUMENT
    assert L.kvmap_fit_destroy(None) == K.OK
    st = K.GramStateC()
    assert L.kvmap_ridge_r2(None, ctypes.byref(st), 0.01, 64, None, None) == K.ERR_INVALID_ARGUMENT
    assert L.kvmap_ridge_solve_device(None, ctypes.byref(st), 0.01, None, None, K.F32, None) == \
        K.ERR_INVALID_ARGUMENT


def test_validate_accepts_repeats_across_rows():
    # a source layer may feed several target layers; only repeats within a row are refused
    assert _validate(layer_sel=np.array([[0, 1, 2]] * 4, np.int32)) == K.OK


def _random_stats(p, q, n, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, p)) * rng.lognormal(0, 0.5, p) + rng.normal(5, 1, p)
    Y = X[:, :q] @ rng.standard_normal((q, q)) + rng.standard_normal((n, q))
    return oracle.stats_two_pass(X, Y)


def _random_host_ridge_cases(n=8):
    rng = np.random.default_rng([2026, 705])
    out = []
    for _ in range(n):
        p = int(rng.integers(1, 400))
        out.append((p, int(rng.integers(1, min(p, 60) + 1)), int(4 * p + rng.integers(1, 200))))
    return out


@pytest.mark.parametrize("p,q,n", [(8, 4, 50), (64, 16, 500), (300, 40, 1000), (389, 37, 1200)]
                         + _random_host_ridge_cases())
def test_ridge_solve_host_matches_oracle(p, q, n):
    st = _random_stats(p, q, n, seed=p)
    lam = 0.01
    f32 = {k: (v.astype(np.float32) if isinstance(v, np.ndarray) else v) for k, v in st.items()}
    W, b = K.ridge_solve_host(f32["mx"], f32["my"], np.triu(f32["Mxx"]), f32["Mxy"], lam, n_threads=4)
    # the oracle solves the same fp32-rounded statistics in fp64
    ref = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in f32.items()}
    Wr, br = oracle.ridge(ref, lam)
    assert W.shape == (q, p)
    assert np.max(np.abs(W.T - Wr)) <= 1e-5 * max(1.0, np.max(np.abs(Wr)))
    assert np.max(np.abs(b - br)) <= 1e-5 * max(1.0, np.max(np.abs(br)))


def test_ridge_solve_host_thread_count_and_lower_triangle():
    # p = 3 * 128 + 5 and q = 4 * 8 + 5: ragged panel, ragged 6 x 8 register blocks on both sides.
    # The tiles do not depend on the thread count and each is summed by one thread, so any
    # thread count gives the same bits; only M_xx's upper triangle is read, so NaN below the
    # diagonal changes nothing.
    p, q, n = 389, 37, 1200
    st = _random_stats(p, q, n, seed=7)
    f32 = {k: (v.astype(np.float32) if isinstance(v, np.ndarray) else v) for k, v in st.items()}
    Mxx = np.triu(f32["Mxx"])
    W1, b1 = K.ridge_solve_host(f32["mx"], f32["my"], Mxx, f32["Mxy"], 0.01, n_threads=1)
    Mxx_nan = Mxx.copy()
    Mxx_nan[np.tril_indices(p, -1)] = np.nan
    for nt in (2, 3, 8):
        W, b = K.ridge_solve_host(f32["mx"], f32["my"], Mxx_nan, f32["Mxy"], 0.01, n_threads=nt)
        assert np.array_equal(W, W1) and np.array_equal(b, b1), nt


def test_ridge_solve_host_refusals():
    p, q = 6, 2
    mx, my = np.zeros(p, np.float32), np.zeros(q, np.float32)
    Mxy = np.ones((p, q), np.float32)
    with pytest.raises(K.KvmapError) as e:
        K.ridge_solve_host(mx, my, -np.eye(p, dtype=np.float32), Mxy, 0.0)
    assert e.value.status == K.ERR_NOT_SPD
    with pytest.raises(K.KvmapError) as e:
        K.ridge_solve_host(mx, my, np.eye(p, dtype=np.float32), Mxy, -1.0)
    assert e.value.status == K.ERR_INVALID_ARGUMENT
    # rank-deficient Gram with lambda = 0 is refused, lambda > 0 makes it solvable
    Z = np.zeros((p, p), np.float32)
    with pytest.raises(K.KvmapError):
        K.ridge_solve_host(mx, my, Z, Mxy, 0.0)
    W, b = K.ridge_solve_host(mx, my, Z, Mxy, 0.5)
    assert np.allclose(W, 2.0)


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so, before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_reserve_checks_dims_before_anything():
    """kvmap_reserve refuses a zeroed or unsupported kvmap_dims with a status code (it used to
    reach the short-cache plan's arithmetic), before it looks at the context."""
    import ctypes
    L = K.lib()
    zero = K.Dims(0, 0, 0, 0, 0, 0, 0)
    assert L.kvmap_reserve(None, ctypes.byref(zero)) == K.ERR_SHAPE
    d32 = K.Dims(1, 1, 1, 32, 1, 16, K.BF16)  # head dim 32: not built
    assert L.kvmap_reserve(None, ctypes.byref(d32)) == K.ERR_UNSUPPORTED
    neg = K.Dims(4, 4, -2, 128, 2, 64, K.BF16)
    assert L.kvmap_reserve(None, ctypes.byref(neg)) == K.ERR_SHAPE
    bad_dtype = K.Dims(4, 4, 2, 128, 2, 64, 7)
    assert L.kvmap_reserve(None, ctypes.byref(bad_dtype)) == K.ERR_UNSUPPORTED
    assert L.kvmap_reserve(None, None) == K.ERR_INVALID_ARGUMENT
    good = K.Dims(4, 4, 2, 128, 2, 64, K.BF16)
    assert L.kvmap_reserve(None, ctypes.byref(good)) == K.ERR_INVALID_ARGUMENT  # then the NULL ctx


def test_timings_refuse_without_context():
    """kvmap_timings / kvmap_last_timings refuse a NULL context (and a short output array)
    before touching the device."""
    import ctypes
    buf = (ctypes.c_float * 3)()
    assert K.lib().kvmap_timings(None, 0, buf, 3) == K.ERR_INVALID_ARGUMENT
    assert K.lib().kvmap_last_timings(None, buf, 3) == K.ERR_INVALID_ARGUMENT
    assert K.lib().kvmap_timings(None, 0, buf, 2) == K.ERR_INVALID_ARGUMENT


def _gram_addrs(p=520, q=68, n_b=700, dtype=K.BF16, xx_block=0, ss_y=True):
    """Addresses of a state and a batch laid out apart, 16-byte aligned (never read)."""
    es = 2 if dtype == K.BF16 else 4
    sizes = dict(mean_x=p * 4, mean_y=q * 4, M_xx=p * (xx_block or p) * 4, M_xy=p * q * 4, ss_y=q * 4,
                 X=n_b * p * es, Y=n_b * q * es)
    addr, base = {}, 1 << 41
    for k_, n in sizes.items():
        addr[k_] = base
        base += (n + 4095) // 4096 * 4096
    if not ss_y:
        addr["ss_y"] = 0
    return addr, sizes


def _vg(p=520, q=68, n_b=700, dtype=K.BF16, xx_block=0, n=0, **over):
    a, _ = _gram_addrs(p, q, n_b, dtype, xx_block)
    a.update(over)
    return K.validate_gram(p, q, n, a["mean_x"], a["mean_y"], a["M_xx"], a["M_xy"], a["ss_y"], xx_block,
                           a["X"], a["Y"], n_b, dtype)


def test_validate_gram_accepts_and_refuses():
    """kvmap_validate_gram: the statistics calls' host checks, before any device work."""
    a, sz = _gram_addrs()
    assert _vg() == K.OK
    assert _vg(dtype=K.F32) == K.OK
    assert _vg(xx_block=104) == K.OK
    assert _vg(n_b=0, X=0, Y=0) == K.OK                            # an empty batch is a no-op
    assert _vg(dtype=7) == K.ERR_UNSUPPORTED
    assert _vg(n_b=-1) == K.ERR_SHAPE
    assert _vg(p=522) == K.ERR_SHAPE                                # not a multiple of 4
    assert _vg(xx_block=12) == K.ERR_SHAPE                          # does not divide p
    assert _vg(n=-5) == K.ERR_SHAPE
    assert _vg(X=0) == K.ERR_INVALID_ARGUMENT
    assert _vg(M_xy=0) == K.ERR_INVALID_ARGUMENT
    assert _vg(Y=a["Y"] + 8) == K.ERR_INVALID_ARGUMENT             # misaligned
    assert _vg(X=a["M_xx"]) == K.ERR_INVALID_ARGUMENT              # the batch over the state
    assert _vg(Y=a["M_xy"] + sz["M_xy"] - 16) == K.ERR_INVALID_ARGUMENT
    assert _vg(X=a["mean_y"] - 16) == K.ERR_INVALID_ARGUMENT
    assert _vg(Y=a["ss_y"]) == K.ERR_INVALID_ARGUMENT
    assert K.last_error() != ""
    # adjacent, not overlapping
    assert _vg(Y=a["ss_y"] + sz["ss_y"]) == K.OK
