"""Upload seeded workloads to a GPU (torch tensors), generating chunks on host threads.

Only draws and copies happen here.  Every value of apply_inputs and fit_inputs equals what
synth.workloads returns for the same chunk, so the oracle can regenerate any part of the input on
the host; device_apply_inputs draws on the device instead (shapes too large for the host), and
its checks read back the input rows they use.
"""

from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from .workloads import ApplyConfig, FitStatsConfig, b_layer, fit_batch, layer_sel, src_head, w_layer


def _torch():
    import torch
    return torch


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 4))


def host_to_tensor(a: np.ndarray, dtype: str):
    """Storage array (uint16 bf16 bits or float32) -> CPU torch tensor of the storage dtype."""
    torch = _torch()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def torch_dtype(dtype: str):
    torch = _torch()
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def apply_inputs(cfg: ApplyConfig, device="cuda:0", progress=None) -> dict:
    """All inputs of one apply call on `device`:
    src_k, src_v [L_src][H][T][d]; W_k, W_v [L_tgt][N][F]; b_k, b_v [L_tgt][N]; layer_sel (numpy)."""
    torch = _torch()
    dt = torch_dtype(cfg.dtype)
    out = dict(
        layer_sel=layer_sel(cfg),
        src_k=torch.empty((cfg.L_src, cfg.H, cfg.T, cfg.d), dtype=dt, device=device),
        src_v=torch.empty((cfg.L_src, cfg.H, cfg.T, cfg.d), dtype=dt, device=device),
        W_k=torch.empty((cfg.L_tgt, cfg.N, cfg.F), dtype=dt, device=device),
        W_v=torch.empty((cfg.L_tgt, cfg.N, cfg.F), dtype=dt, device=device),
        b_k=torch.empty((cfg.L_tgt, cfg.N), dtype=dt, device=device),
        b_v=torch.empty((cfg.L_tgt, cfg.N), dtype=dt, device=device),
    )
    jobs = []
    for which in ("k", "v"):
        for l in range(cfg.L_src):
            for h in range(cfg.H):
                jobs.append((f"src_{which}", (l, h), lambda w=which, l=l, h=h: src_head(cfg, w, l, h)))
        for t in range(cfg.L_tgt):
            jobs.append((f"W_{which}", (t,), lambda w=which, t=t: w_layer(cfg, w, t)))
            jobs.append((f"b_{which}", (t,), lambda w=which, t=t: b_layer(cfg, w, t)))
    done = 0
    with cf.ThreadPoolExecutor(_threads()) as ex:
        futs = {ex.submit(fn): (name, idx) for name, idx, fn in jobs}
        for f in cf.as_completed(futs):
            name, idx = futs[f]
            out[name][idx].copy_(host_to_tensor(f.result(), cfg.dtype))
            done += 1
            if progress and done % 64 == 0:
                progress(done, len(jobs))
    torch.cuda.synchronize(device)
    return out


def device_apply_inputs(cfg: ApplyConfig, device="cuda:0") -> dict:
    """The inputs of one apply call drawn on `device` with torch's seeded generator, for caches
    too large to draw on the host (the largest accepted shapes): src_k, src_v ~ N(0, 1); W_k, W_v
    ~ N(0, 1/F); b_k, b_v ~ N(0, b_var); layer_sel as synth.workloads draws it.  These values do
    not match synth.workloads: whoever checks them reads back the rows it needs."""
    torch = _torch()
    g = torch.Generator(device=device).manual_seed(20260000 + cfg.cid)
    dt = torch_dtype(cfg.dtype)

    def normal(shape, std):
        t = torch.empty(shape, dtype=dt, device=device)
        flat = t.view(-1)
        step = 1 << 28  # a 1 GiB float32 temporary at most
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            flat[i:i + n].copy_(torch.randn(n, generator=g, device=device, dtype=torch.float32) * std)
        return t

    out = dict(layer_sel=layer_sel(cfg))
    for w in ("k", "v"):
        out[f"src_{w}"] = normal((cfg.L_src, cfg.H, cfg.T, cfg.d), 1.0)
        out[f"W_{w}"] = normal((cfg.L_tgt, cfg.N, cfg.F), cfg.F ** -0.5)
        out[f"b_{w}"] = normal((cfg.L_tgt, cfg.N), cfg.b_var ** 0.5)
    if torch.device(device).type == "cuda":
        torch.cuda.synchronize(device)
    return out


def fit_inputs(cfg: FitStatsConfig, batches, device="cuda:0", window: int = 4):
    """Yield (b, X, Y) device tensors for the given batch indices, generating up to
    `window` batches ahead on host threads."""
    batches = list(batches)
    with cf.ThreadPoolExecutor(min(window, _threads())) as ex:
        pending = [ex.submit(fit_batch, cfg, b) for b in batches[:window]]
        for i, b in enumerate(batches):
            xs, ys = pending[i].result()
            pending[i] = None
            if i + window < len(batches):
                pending.append(ex.submit(fit_batch, cfg, batches[i + window]))
            yield b, host_to_tensor(xs, cfg.dtype).to(device), host_to_tensor(ys, cfg.dtype).to(device)
