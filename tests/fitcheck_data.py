"""Assemble fit-check cache pairs from raw seeded draws, using the oracle's arithmetic.

The hidden map is the data-generating process of the KVBridge README's synthetic
demo ("Thirty-second proof"): a source and a target model of one family that differ in
layer count and RoPE base, an affine map across layers hidden in the data, cache pairs
over the same tokens, and holdout sequences the fit never sees.
"""

import numpy as np

import oracle
from synth.workloads import fitcheck_draws


def build_pairs(cfg):
    """Returns dict with stored caches for every sequence plus the raw draws.

    src_k/src_v: [n_seq][L_src][H][T][d]  (keys rotated by the source model)
    tgt_k/tgt_v: [n_seq][L_tgt][H][T][d]  (keys rotated by the target model)
    tgt_k_content: [n_seq][L_tgt][H][T][d]
    pos: [n_seq][T]
    """
    dr = fitcheck_draws(cfg)
    n_seq = len(dr["pos0"])
    pos = np.stack([dr["pos0"][s] + np.arange(cfg.T) for s in range(n_seq)])
    src_k = np.stack([oracle.rope(dr["src_k"][s], pos[s], cfg.theta_src) for s in range(n_seq)])
    src_v = dr["src_v"]
    tk_c = np.empty((n_seq, cfg.L_tgt, cfg.H, cfg.T, cfg.d))
    tv = np.empty_like(tk_c)
    for s in range(n_seq):
        for t in range(cfg.L_tgt):
            sel = dr["true_sel"][t]
            xk = oracle.feature_rows([dr["src_k"][s][l] for l in sel])
            xv = oracle.feature_rows([dr["src_v"][s][l] for l in sel])
            yk = oracle.affine(xk, dr["Wk"][t], dr["bk"][t])
            yv = oracle.affine(xv, dr["Wv"][t], dr["bv"][t])
            tk_c[s, t] = yk.reshape(cfg.T, cfg.H, cfg.d).transpose(1, 0, 2) + dr["noise_k"][s, t]
            tv[s, t] = yv.reshape(cfg.T, cfg.H, cfg.d).transpose(1, 0, 2) + dr["noise_v"][s, t]
    tgt_k = np.stack([oracle.rope(tk_c[s], pos[s], cfg.theta_tgt) for s in range(n_seq)])
    return dict(draws=dr, pos=pos, src_k=src_k, src_v=src_v, tgt_k=tgt_k, tgt_v=tv,
                tgt_k_content=tk_c, n_calib=cfg.n_calib)
