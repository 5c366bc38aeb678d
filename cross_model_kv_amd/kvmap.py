"""Python binding of libkvmap (ctypes).  Argument marshalling only: every step of the
mapping runs in the library's HIP kernels; torch supplies device memory and streams.

The names follow include/kvmap.h: ``Context.apply`` is ``kvmap_apply``, ``Context.gram``
is ``kvmap_gram`` and so on.  If the library has not been built the import of this module
succeeds but the first call raises ``KvmapError`` (there is no fallback of any kind).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libkvmap.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_SHAPE = 2
ERR_UNSUPPORTED = 3
ERR_NONFINITE = 4
ERR_NOT_SPD = 5
ERR_DEVICE = 6
ERR_OUT_OF_MEMORY = 7

BF16 = 0
F32 = 1
ROPE_HALF_SPLIT = 0
ROPE_INTERLEAVED = 1
FLAG_CHECK_FINITE = 0x1
FLAG_TIMING = 0x2


class KvmapError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status) if _lib else status}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [("L_src", ctypes.c_int32), ("L_tgt", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k", ctypes.c_int32), ("T", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


class Rope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("pos0", ctypes.c_int64), ("style", ctypes.c_int32),
                ("inv_freq", ctypes.c_void_p)]


def _rope(theta, pos0, style, inv_freq, keep: list) -> Rope:
    """A kvmap_rope; inv_freq (host sequence of head_dim/2 frequencies, or None) is kept alive in
    `keep` for the duration of the call."""
    ptr = None
    if inv_freq is not None:
        a = np.ascontiguousarray(np.asarray(inv_freq, dtype=np.float64).reshape(-1))
        keep.append(a)
        ptr = a.ctypes.data
    return Rope(float(theta if theta is not None else 0.0), int(pos0), int(style), ptr)


class GramStateC(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("p", ctypes.c_int32), ("q", ctypes.c_int32),
                ("mean_x", ctypes.c_void_p), ("mean_y", ctypes.c_void_p),
                ("M_xx", ctypes.c_void_p), ("M_xy", ctypes.c_void_p), ("ss_y", ctypes.c_void_p),
                ("xx_block", ctypes.c_int32)]


class FitConfigC(ctypes.Structure):
    _fields_ = [("L_src", ctypes.c_int32), ("L_tgt", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("select_block", ctypes.c_int32), ("map_block", ctypes.c_int32),
                ("given_sel", ctypes.c_int32), ("two_pass", ctypes.c_int32), ("theta_src", ctypes.c_double),
                ("theta_tgt", ctypes.c_double),
                ("lambda_", ctypes.c_double), ("layer_sel", ctypes.c_void_p), ("scores", ctypes.c_void_p),
                ("W_k", ctypes.c_void_p), ("b_k", ctypes.c_void_p), ("W_v", ctypes.c_void_p),
                ("b_v", ctypes.c_void_p), ("inv_freq_src", ctypes.c_void_p), ("inv_freq_tgt", ctypes.c_void_p)]


class FitPassC(ctypes.Structure):
    _fields_ = [("stage", ctypes.c_int32), ("t_begin", ctypes.c_int32), ("t_end", ctypes.c_int32),
                ("pass_", ctypes.c_int32), ("passes", ctypes.c_int32)]


_lib = None

_SIGS = {
    "kvmap_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvmap_last_error": (ctypes.c_char_p, []),
    "kvmap_version": (ctypes.c_int, []),
    "kvmap_create": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]),
    "kvmap_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "kvmap_reserve": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Dims)]),
    "kvmap_validate_apply_buffers": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 8),
    "kvmap_validate_gram": (ctypes.c_int, [ctypes.POINTER(GramStateC), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int32]),
    "kvmap_validate_apply": (ctypes.c_int, [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.POINTER(Rope),
                                            ctypes.POINTER(Rope)]),
    "kvmap_apply": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.POINTER(Rope), ctypes.POINTER(Rope),
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32]),
    "kvmap_last_timings": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int]),
    "kvmap_timings": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_int]),
    "kvmap_recode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Rope), ctypes.POINTER(Rope),
                                    ctypes.c_void_p]),
    "kvmap_cache_rows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.POINTER(Rope), ctypes.c_void_p, ctypes.c_void_p]),
    "kvmap_gram_reset": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(GramStateC), ctypes.c_void_p]),
    "kvmap_gram": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.POINTER(GramStateC), ctypes.c_void_p]),
    "kvmap_gram_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.POINTER(GramStateC), ctypes.c_void_p]),
    "kvmap_gram_merge": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(GramStateC), ctypes.POINTER(GramStateC),
                                        ctypes.c_void_p]),
    "kvmap_ridge_solve_host": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int]),
    "kvmap_ridge_solve": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(GramStateC), ctypes.c_double,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvmap_ridge_solve_device": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(GramStateC), ctypes.c_double,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "kvmap_ridge_r2": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(GramStateC), ctypes.c_double, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "kvmap_ridge_solve_device_batch": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.POINTER(GramStateC)),
                                                      ctypes.c_int32, ctypes.c_double, ctypes.POINTER(ctypes.c_void_p),
                                                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_void_p]),
    "kvmap_ridge_r2_batch": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.POINTER(GramStateC)), ctypes.c_int32,
                                            ctypes.c_double, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.c_void_p]),
    "kvmap_fit_create": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(FitConfigC), ctypes.POINTER(ctypes.c_void_p)]),
    "kvmap_fit_next_pass": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(FitPassC), ctypes.c_void_p]),
    "kvmap_fit_add": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "kvmap_fit_destroy": (ctypes.c_int, [ctypes.c_void_p]),
}


def lib():
    """Load libkvmap.so (built in-tree). Raises KvmapError if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvmapError(ERR_DEVICE, "load", f"{LIB_PATH} is not built; run "
                             "`python -m cross_model_kv_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvmap_status_string(status).decode()


def last_error() -> str:
    return lib().kvmap_last_error().decode()


def version() -> int:
    return lib().kvmap_version()


def _check(status: int, where: str):
    if status != OK:
        raise KvmapError(status, where, last_error())


def _dims(L_src, L_tgt, H, d, k, T, dtype) -> Dims:
    return Dims(int(L_src), int(L_tgt), int(H), int(d), int(k), int(T), int(dtype))


def _sel_array(layer_sel) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(layer_sel.cpu() if hasattr(layer_sel, "cpu") else layer_sel),
                             dtype=np.int32)
    if a.ndim != 2:
        raise ValueError("layer_sel must be [L_tgt][k]")
    return a


def validate_apply(L_src, L_tgt, H, d, k, T, dtype, layer_sel, theta_src, theta_tgt,
                   pos0_src=0, pos0_tgt=0, style_src=ROPE_HALF_SPLIT, style_tgt=ROPE_HALF_SPLIT,
                   inv_freq_src=None, inv_freq_tgt=None) -> int:
    """kvmap_validate_apply; returns the status code (host only, needs no GPU)."""
    sel = _sel_array(layer_sel)
    dm = _dims(L_src, L_tgt, H, d, k, T, dtype)
    keep = []
    rs = _rope(theta_src, pos0_src, style_src, inv_freq_src, keep)
    rt = _rope(theta_tgt, pos0_tgt, style_tgt, inv_freq_tgt, keep)
    return lib().kvmap_validate_apply(ctypes.byref(dm), sel.ctypes.data, ctypes.byref(rs), ctypes.byref(rt))


def validate_apply_buffers(L_src, L_tgt, H, d, k, T, dtype, src_k, src_v, W_k, b_k, W_v, b_v,
                           tgt_k, tgt_v) -> int:
    """kvmap_validate_apply_buffers on buffer addresses given as integers (nothing is read);
    returns the status code (host only, needs no GPU)."""
    dm = _dims(L_src, L_tgt, H, d, k, T, dtype)
    addrs = [ctypes.c_void_p(int(a)) if a else None for a in (src_k, src_v, W_k, b_k, W_v, b_v, tgt_k, tgt_v)]
    return lib().kvmap_validate_apply_buffers(ctypes.byref(dm), *addrs)


def validate_gram(p, q, n, mean_x, mean_y, M_xx, M_xy, ss_y, xx_block, X, Y, n_b, dtype) -> int:
    """kvmap_validate_gram on a state and batch given as addresses (integers; nothing is read);
    returns the status code (host only, needs no GPU)."""
    st = GramStateC(int(n), int(p), int(q), mean_x or None, mean_y or None, M_xx or None, M_xy or None,
                    ss_y or None, int(xx_block))
    return lib().kvmap_validate_gram(ctypes.byref(st), X or None, Y or None, int(n_b), int(dtype))


def ridge_solve_host(mean_x, mean_y, M_xx, M_xy, lam: float, n_threads: int = 0):
    """kvmap_ridge_solve_host on host arrays; returns (W [q][p] output-major, b [q]) float32."""
    mx = np.ascontiguousarray(mean_x, dtype=np.float32)
    my = np.ascontiguousarray(mean_y, dtype=np.float32)
    Mxx = np.ascontiguousarray(M_xx, dtype=np.float32)
    Mxy = np.ascontiguousarray(M_xy, dtype=np.float32)
    p, q = mx.shape[0], my.shape[0]
    if Mxx.shape != (p, p) or Mxy.shape != (p, q):
        raise ValueError("shape mismatch")
    W = np.empty((q, p), dtype=np.float32)
    b = np.empty(q, dtype=np.float32)
    _check(lib().kvmap_ridge_solve_host(p, q, mx.ctypes.data, my.ctypes.data, Mxx.ctypes.data, Mxy.ctypes.data,
                                        float(lam), W.ctypes.data, b.ctypes.data, int(n_threads)),
           "kvmap_ridge_solve_host")
    return W, b


# ---------------------------------------------------------------------------------------
# device side (torch tensors for memory, torch streams)
# ---------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream_handle(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _chain(first, rest):
    yield from first
    yield from rest


class GramState:
    """Device-resident centered statistics (n, mean_x, mean_y, M_xx, M_xy and, with
    keep_ss_y, the per-column centered sum of squares ss_y) of kvmap_gram."""

    def __init__(self, p: int, q: int, device, keep_ss_y: bool = False, xx_block: int = 0):
        torch = _torch()
        self.p, self.q, self.device = int(p), int(q), torch.device(device)
        self.xx_block = int(xx_block)
        kw = dict(dtype=torch.float32, device=self.device)
        self.mean_x = torch.zeros(p, **kw)
        self.mean_y = torch.zeros(q, **kw)
        # blocked: [p / b][b][b] diagonal blocks only
        self.M_xx = (torch.zeros(p // self.xx_block, self.xx_block, self.xx_block, **kw) if self.xx_block
                     else torch.zeros(p, p, **kw))
        self.M_xy = torch.zeros(p, q, **kw)
        self.ss_y = torch.zeros(q, **kw) if keep_ss_y else None
        self.c = GramStateC(0, self.p, self.q, self.mean_x.data_ptr(), self.mean_y.data_ptr(),
                            self.M_xx.data_ptr(), self.M_xy.data_ptr(),
                            self.ss_y.data_ptr() if keep_ss_y else None, self.xx_block)

    @property
    def n(self) -> int:
        return int(self.c.n)


class Context:
    """A libkvmap context on one HIP device (kvmap_create / kvmap_destroy)."""

    def __init__(self, device: int = 0):
        self.device = int(device)
        h = ctypes.c_void_p()
        _check(lib().kvmap_create(ctypes.byref(h), self.device), "kvmap_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().kvmap_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---- apply ---------------------------------------------------------------------
    def reserve(self, L_src, L_tgt, H, d, k, T, dtype=BF16):
        dm = _dims(L_src, L_tgt, H, d, k, T, dtype)
        _check(lib().kvmap_reserve(self._h, ctypes.byref(dm)), "kvmap_reserve")

    def apply(self, src_k, src_v, layer_sel, W_k, b_k, W_v, b_v, theta_src: float, theta_tgt: float,
              pos0_src: int = 0, pos0_tgt: int | None = None, out_k=None, out_v=None, stream=None,
              flags: int = 0, style_src: int = ROPE_HALF_SPLIT, style_tgt: int = ROPE_HALF_SPLIT,
              inv_freq_src=None, inv_freq_tgt=None):
        """kvmap_apply.  src_k/src_v [L_src][H][T][d], W_k/W_v [L_tgt][N][F] (output-major),
        b_k/b_v [L_tgt][N] device tensors of one dtype (bf16 or fp32); layer_sel host
        int [L_tgt][k].  inv_freq_src/tgt: optional host [d/2] rotary frequencies of each model
        (instead of theta).  Returns (tgt_k, tgt_v) [L_tgt][H][T][d] (allocated if not given)."""
        torch = _torch()
        sel = _sel_array(layer_sel)
        L_src, H, T, d = src_k.shape
        L_tgt, k = sel.shape
        dt = _dtype_code(src_k)
        for name, t in (("src_v", src_v), ("W_k", W_k), ("b_k", b_k), ("W_v", W_v), ("b_v", b_v)):
            if t.dtype != src_k.dtype:
                raise TypeError(f"{name} dtype {t.dtype} differs from src_k {src_k.dtype}")
        N, F = H * d, k * H * d
        if tuple(src_v.shape) != tuple(src_k.shape):
            raise ValueError("src_v shape differs from src_k")
        if tuple(W_k.shape) != (L_tgt, N, F) or tuple(W_v.shape) != (L_tgt, N, F):
            raise ValueError(f"W must be [L_tgt={L_tgt}][N={N}][F={F}]")
        if tuple(b_k.shape) != (L_tgt, N) or tuple(b_v.shape) != (L_tgt, N):
            raise ValueError(f"b must be [L_tgt={L_tgt}][N={N}]")
        if out_k is None:
            out_k = torch.empty((L_tgt, H, T, d), dtype=src_k.dtype, device=src_k.device)
        if out_v is None:
            out_v = torch.empty((L_tgt, H, T, d), dtype=src_k.dtype, device=src_k.device)
        for name, t in (("out_k", out_k), ("out_v", out_v)):
            if tuple(t.shape) != (L_tgt, H, T, d) or t.dtype != src_k.dtype:
                raise ValueError(f"{name} must be [L_tgt][H][T][d] of the input dtype")
        dm = _dims(L_src, L_tgt, H, d, k, T, dt)
        keep = []
        rs = _rope(theta_src, pos0_src, style_src, inv_freq_src, keep)
        rt = _rope(theta_tgt, pos0_src if pos0_tgt is None else pos0_tgt, style_tgt, inv_freq_tgt, keep)
        st = lib().kvmap_apply(self._h, ctypes.byref(dm), _dev_ptr(src_k, "src_k"), _dev_ptr(src_v, "src_v"),
                               sel.ctypes.data, _dev_ptr(W_k, "W_k"), _dev_ptr(b_k, "b_k"),
                               _dev_ptr(W_v, "W_v"), _dev_ptr(b_v, "b_v"), ctypes.byref(rs), ctypes.byref(rt),
                               _dev_ptr(out_k, "out_k"), _dev_ptr(out_v, "out_v"),
                               _stream_handle(stream, src_k.device), int(flags))
        _check(st, "kvmap_apply")
        return out_k, out_v

    def last_timings(self):
        """(rope_table_ms, derope_ms, map_gemm_ms) of the last FLAG_TIMING apply."""
        ms = (ctypes.c_float * 3)()
        _check(lib().kvmap_last_timings(self._h, ms, 3), "kvmap_last_timings")
        return float(ms[0]), float(ms[1]), float(ms[2])

    def timings(self, back: int):
        """(rope_table_ms, derope_ms, map_gemm_ms) of the FLAG_TIMING apply `back` calls before the
        last one (0 = the last; the context holds 128)."""
        ms = (ctypes.c_float * 3)()
        _check(lib().kvmap_timings(self._h, int(back), ms, 3), "kvmap_timings")
        return float(ms[0]), float(ms[1]), float(ms[2])

    def recode(self, src, theta_src: float, theta_tgt: float, pos0_src: int = 0, pos0_tgt: int | None = None,
               out=None, stream=None, style_src: int = ROPE_HALF_SPLIT, style_tgt: int = ROPE_HALF_SPLIT,
               inv_freq_src=None, inv_freq_tgt=None):
        """kvmap_recode: re-encode keys src [..., T, d] (device, bf16 or fp32; leading dims
        are the rows) from RoPE (theta_src, pos0_src) to (theta_tgt, pos0_tgt) (or the given
        frequency lists).  Returns out (allocated if not given), of src's shape and dtype."""
        torch = _torch()
        if src.dim() < 2:
            raise ValueError("src must be [..., T, d]")
        T, d = int(src.shape[-2]), int(src.shape[-1])
        rows = int(src.numel() // max(1, T * d))
        if out is None:
            out = torch.empty_like(src)
        if tuple(out.shape) != tuple(src.shape) or out.dtype != src.dtype:
            raise ValueError("out must match src's shape and dtype")
        keep = []
        rs = _rope(theta_src, pos0_src, style_src, inv_freq_src, keep)
        rt = _rope(theta_tgt, pos0_src if pos0_tgt is None else pos0_tgt, style_tgt, inv_freq_tgt, keep)
        _check(lib().kvmap_recode(self._h, rows, T, d, _dtype_code(src), _dev_ptr(src, "src"), _dev_ptr(out, "out"),
                                  ctypes.byref(rs), ctypes.byref(rt), _stream_handle(stream, src.device)),
               "kvmap_recode")
        return out

    # ---- fit-side statistics ---------------------------------------------------------
    def cache_rows(self, cache, layers, theta: float | None = None, pos0: int = 0, out=None, stream=None,
                   style: int = ROPE_HALF_SPLIT, inv_freq=None):
        """kvmap_cache_rows: rows [T][len(layers) * H * d] of the layers of cache [L][H][T][d]
        (device, bf16 or fp32), RoPE stripped at (theta or inv_freq, pos0) unless both are None."""
        torch = _torch()
        L, H, T, d = (int(x) for x in cache.shape)
        lay = np.ascontiguousarray(np.asarray(layers, dtype=np.int32).reshape(-1))
        width = len(lay) * H * d
        if out is None:
            out = torch.empty((T, width), dtype=cache.dtype, device=cache.device)
        if tuple(out.shape) != (T, width) or out.dtype != cache.dtype:
            raise ValueError(f"out must be [T={T}][{width}] of the cache dtype")
        keep = []
        rope = (None if theta is None and inv_freq is None
                else ctypes.byref(_rope(theta, pos0, style, inv_freq, keep)))
        _check(lib().kvmap_cache_rows(self._h, _dev_ptr(cache, "cache"), L, H, T, d, _dtype_code(cache),
                                      lay.ctypes.data, len(lay), rope, _dev_ptr(out, "out"),
                                      _stream_handle(stream, cache.device)), "kvmap_cache_rows")
        return out

    def gram_state(self, p: int, q: int, keep_ss_y: bool = False, xx_block: int = 0) -> GramState:
        return GramState(p, q, f"cuda:{self.device}", keep_ss_y, xx_block)

    def gram_reset(self, st: GramState, stream=None):
        _check(lib().kvmap_gram_reset(self._h, ctypes.byref(st.c), _stream_handle(stream, st.device)),
               "kvmap_gram_reset")

    def gram(self, st: GramState, X, Y, stream=None):
        """kvmap_gram: merge the batch X [n_b][p], Y [n_b][q] (device, bf16 or fp32) into st."""
        if X.dim() != 2 or Y.dim() != 2 or X.shape[0] != Y.shape[0]:
            raise ValueError("X [n_b][p] and Y [n_b][q] must share n_b")
        if X.shape[1] != st.p or Y.shape[1] != st.q:
            raise ValueError("batch width does not match the state")
        if X.dtype != Y.dtype:
            raise TypeError("X and Y dtypes differ")
        _check(lib().kvmap_gram(self._h, _dev_ptr(X, "X"), _dev_ptr(Y, "Y"), int(X.shape[0]), _dtype_code(X),
                                ctypes.byref(st.c), _stream_handle(stream, st.device)), "kvmap_gram")

    def gram_noalloc(self, st: GramState, X, Y, stream=None):
        """kvmap_gram_noalloc: kvmap_gram through the library's static device scratch (no
        allocation by the library; batches are merged in sub-batches that fit it)."""
        if X.dim() != 2 or Y.dim() != 2 or X.shape[0] != Y.shape[0]:
            raise ValueError("X [n_b][p] and Y [n_b][q] must share n_b")
        if X.shape[1] != st.p or Y.shape[1] != st.q:
            raise ValueError("batch width does not match the state")
        if X.dtype != Y.dtype:
            raise TypeError("X and Y dtypes differ")
        _check(lib().kvmap_gram_noalloc(self._h, _dev_ptr(X, "X"), _dev_ptr(Y, "Y"), int(X.shape[0]),
                                        _dtype_code(X), ctypes.byref(st.c), _stream_handle(stream, st.device)),
               "kvmap_gram_noalloc")

    def gram_merge(self, dst: GramState, src: GramState, stream=None):
        _check(lib().kvmap_gram_merge(self._h, ctypes.byref(dst.c), ctypes.byref(src.c),
                                      _stream_handle(stream, dst.device)), "kvmap_gram_merge")

    def ridge_solve_device(self, st: GramState, lam: float, W_out=None, b_out=None, dtype=None, stream=None):
        """kvmap_ridge_solve_device: (W [q][p] output-major, b [q]) device tensors in bf16 or fp32
        (allocated if not given; dtype defaults to that of W_out, else fp32)."""
        torch = _torch()
        if dtype is None:
            dtype = W_out.dtype if W_out is not None else torch.float32
        if W_out is None:
            W_out = torch.empty((st.q, st.p), dtype=dtype, device=st.device)
        if b_out is None:
            b_out = torch.empty((st.q,), dtype=dtype, device=st.device)
        if tuple(W_out.shape) != (st.q, st.p) or tuple(b_out.shape) != (st.q,):
            raise ValueError("W_out must be [q][p] and b_out [q]")
        if W_out.dtype != dtype or b_out.dtype != dtype:
            raise TypeError("W_out and b_out must share the dtype")
        _check(lib().kvmap_ridge_solve_device(self._h, ctypes.byref(st.c), float(lam), _dev_ptr(W_out, "W_out"),
                                              _dev_ptr(b_out, "b_out"), _dtype_code(W_out),
                                              _stream_handle(stream, st.device)), "kvmap_ridge_solve_device")
        return W_out, b_out

    def ridge_r2(self, st: GramState, lam: float, group: int, out=None, stream=None):
        """kvmap_ridge_r2: in-sample R^2 of the ridge fit of st, pooled over groups of `group`
        y columns -> device float64 [q / group].  The state must keep ss_y."""
        torch = _torch()
        if out is None:  # a group that does not divide q is the library's to refuse
            out = torch.empty((max(1, st.q // max(1, int(group))),), dtype=torch.float64, device=st.device)
        elif out.dtype != torch.float64 or out.numel() * int(group) != st.q:
            raise ValueError("out must be float64 [q / group]")
        _check(lib().kvmap_ridge_r2(self._h, ctypes.byref(st.c), float(lam), int(group), _dev_ptr(out, "out"),
                                    _stream_handle(stream, st.device)), "kvmap_ridge_r2")
        return out

    def ridge_solve_device_batch(self, states, lam: float, dtype=None, stream=None):
        """kvmap_ridge_solve_device_batch: [(W [q][p] output-major, b [q])] for states of one (p, q),
        solved together on the device (dtype: bf16 or fp32, default fp32)."""
        torch = _torch()
        dtype = dtype if dtype is not None else torch.float32
        n = len(states)
        outs = [(torch.empty((st.q, st.p), dtype=dtype, device=st.device),
                 torch.empty((st.q,), dtype=dtype, device=st.device)) for st in states]
        sp = (ctypes.POINTER(GramStateC) * n)(*[ctypes.pointer(st.c) for st in states])
        Wp = (ctypes.c_void_p * n)(*[w.data_ptr() for w, _ in outs])
        bp = (ctypes.c_void_p * n)(*[b.data_ptr() for _, b in outs])
        code = BF16 if dtype == torch.bfloat16 else F32
        _check(lib().kvmap_ridge_solve_device_batch(self._h, sp, n, float(lam), Wp, bp, code,
                                                    _stream_handle(stream, states[0].device)),
               "kvmap_ridge_solve_device_batch")
        return outs

    def ridge_r2_batch(self, states, lam: float, group: int, stream=None):
        """kvmap_ridge_r2_batch: [R^2 per group of y columns, device float64 [q / group]] per state."""
        torch = _torch()
        n = len(states)
        outs = [torch.empty((max(1, st.q // max(1, int(group))),), dtype=torch.float64, device=st.device)
                for st in states]
        sp = (ctypes.POINTER(GramStateC) * n)(*[ctypes.pointer(st.c) for st in states])
        op = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
        _check(lib().kvmap_ridge_r2_batch(self._h, sp, n, float(lam), int(group), op,
                                          _stream_handle(stream, states[0].device)), "kvmap_ridge_r2_batch")
        return outs

    def fit(self, calibration, *, L_src: int, L_tgt: int, H: int, d: int, k: int, theta_src: float,
            theta_tgt: float, lam: float, out_dtype=None, layer_sel=None, select_block: int = 0,
            map_block: int = 0, stream=None, on_pass=None, inv_freq_src=None, inv_freq_tgt=None,
            two_pass: bool = False) -> dict:
        """kvmap_fit_*: the two-stage fit (selection, then maps) over re-iterable calibration data.

        `calibration` is a callable returning an iterable of (src_k, src_v, tgt_k, tgt_v, pos0):
        device caches [L_src][H][T][d] and [L_tgt][H][T][d] of one sequence (keys stored rotated)
        and its first position; it is called once per pass and must yield the same sequences
        each time.  layer_sel (device int32 [L_tgt][k]) skips the selection stage.
        Returns dict(layer_sel, scores (None with a given layer_sel), W_k, b_k, W_v, b_v); the maps
        are output-major [L_tgt][H*d][k*H*d] in out_dtype (default: the caches' dtype).
        on_pass(stage, t_begin, t_end, pass_index, passes) is called after each
        kvmap_fit_next_pass (which returns once the previous pass is solved).
        inv_freq_src/tgt: optional host [d/2] rotary frequencies of each model."""
        torch = _torch()
        dev = torch.device(f"cuda:{self.device}")
        N, F = H * d, k * H * d
        given = layer_sel is not None
        if given:
            layer_sel = layer_sel.to(device=dev, dtype=torch.int32).contiguous()
            if tuple(layer_sel.shape) != (L_tgt, k):
                raise ValueError(f"layer_sel must be [{L_tgt}][{k}]")
            scores = None
        else:
            layer_sel = torch.empty((L_tgt, k), dtype=torch.int32, device=dev)
            scores = torch.empty((L_tgt, L_src), dtype=torch.float64, device=dev)
        maps = {}
        dtype_in = None
        h = ctypes.c_void_p()
        try:
            info = FitPassC()
            first = True
            while True:
                if first:
                    # the caches' dtype fixes the config: peek at the first sequence
                    it = iter(calibration())
                    seq = next(it, None)
                    if seq is None:
                        raise ValueError("calibration yields no sequence")
                    dtype_in = seq[0].dtype
                    odt = out_dtype if out_dtype is not None else dtype_in
                    for name, shape in (("W_k", (L_tgt, N, F)), ("b_k", (L_tgt, N)), ("W_v", (L_tgt, N, F)),
                                        ("b_v", (L_tgt, N))):
                        maps[name] = torch.empty(shape, dtype=odt, device=dev)
                    fq = [None if f is None else np.ascontiguousarray(np.asarray(f, dtype=np.float64).reshape(-1))
                          for f in (inv_freq_src, inv_freq_tgt)]
                    cfg = FitConfigC(int(L_src), int(L_tgt), int(H), int(d), int(k), _dtype_code(seq[0]),
                                     _dtype_code(maps["W_k"]), int(select_block), int(map_block), int(given),
                                     int(bool(two_pass)),
                                     float(theta_src if theta_src is not None else 0.0),
                                     float(theta_tgt if theta_tgt is not None else 0.0), float(lam),
                                     layer_sel.data_ptr(), scores.data_ptr() if scores is not None else None,
                                     *(maps[n].data_ptr() for n in ("W_k", "b_k", "W_v", "b_v")),
                                     *(None if f is None else f.ctypes.data for f in fq))
                    _check(lib().kvmap_fit_create(self._h, ctypes.byref(cfg), ctypes.byref(h)), "kvmap_fit_create")
                sh = _stream_handle(stream, dev)
                _check(lib().kvmap_fit_next_pass(h, ctypes.byref(info), sh), "kvmap_fit_next_pass")
                if on_pass is not None:
                    on_pass(info.stage, info.t_begin, info.t_end, info.pass_, info.passes)
                if info.stage == 0:
                    break
                # the first pass continues the peeked iterator; each later pass asks for a new one
                seqs, it = ([seq], it) if first else ([], iter(calibration()))
                first = False
                for seq in _chain(seqs, it):
                    sk, sv, tk, tv, pos0 = seq
                    if (tuple(sk.shape) != (L_src, H, sk.shape[2], d) or tuple(sv.shape) != tuple(sk.shape)
                            or tuple(tk.shape) != (L_tgt, H, sk.shape[2], d) or tuple(tv.shape) != tuple(tk.shape)):
                        raise ValueError("calibration caches must be [L_src][H][T][d] / [L_tgt][H][T][d]")
                    if any(t.dtype != dtype_in for t in (sk, sv, tk, tv)):
                        raise TypeError("calibration caches must share one dtype")
                    _check(lib().kvmap_fit_add(h, _dev_ptr(sk, "src_k"), _dev_ptr(sv, "src_v"), _dev_ptr(tk, "tgt_k"),
                                               _dev_ptr(tv, "tgt_v"), int(sk.shape[2]), int(pos0), sh),
                           "kvmap_fit_add")
        finally:
            if h.value:
                lib().kvmap_fit_destroy(h)
        return dict(layer_sel=layer_sel, scores=scores, **maps)

    def ridge_solve(self, st: GramState, lam: float, stream=None):
        """kvmap_ridge_solve: (W [q][p] output-major float32, b [q]) on the host."""
        W = np.empty((st.q, st.p), dtype=np.float32)
        b = np.empty(st.q, dtype=np.float32)
        _check(lib().kvmap_ridge_solve(self._h, ctypes.byref(st.c), float(lam), W.ctypes.data, b.ctypes.data,
                                       _stream_handle(stream, st.device)), "kvmap_ridge_solve")
        return W, b
