"""Comparison rules between the GPU library and the CPU oracle.

  * index scores: |g - o| <= 1e-3 * max(|o|, 1e-3 * max_row |o|) at visible positions
    (the row floor guards cancellation: head weights are signed), identical -inf
    pattern elsewhere (only where the library materialises it);
  * top-k on identical scores: identical output (both resolve equal scores towards the
    smaller position and list positions in ascending order);
  * top-k after scoring on both sides: same cardinality min(k, n), unique, visible,
    ascending, -1 tail; positions in the symmetric difference of the two sets must
    have oracle scores within 1e-3 (relative, same row floor) of the oracle's k-th
    largest score tau;
  * attention outputs: |g - o| <= 2e-2 (bf16 inputs/outputs) or 1e-4 (fp32), lse
    within 1e-3 (bf16) or 1e-5 (fp32) absolute, compared on the same indices;
  * indexer preparation: scales within 2e-6 relative; every FP8 code decodes to the
    oracle's nearest e4m3fn value of its pre-rounding value y, except that where y lies
    within 2e-3 of the midpoint between two e4m3fn values (the fp32 rotation's error
    bound, in units of y) the other neighbour is accepted too.
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 1e-3
ATTN_ATOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_ATOL = {"bf16": 1e-3, "f32": 1e-5}


def _n_visible(L, T, t, compress):
    """rows visible to query row t: positions 0..pos, or with compressed entries
    (compress = m > 1) the entries e < (pos + 1) / m"""
    return (int(L) - T + t + 1) // compress


def check_scores(gpu: np.ndarray, orc: np.ndarray, lens, T: int, full_mask: bool = True, rows=None,
                 compress: int = 1):
    """gpu/orc: [R, Lmax] rows (b,t) given by `rows` (list of (b, t)) or all of [B,T,Lmax]."""
    if rows is None:
        B = gpu.shape[0]
        rows = [(b, t) for b in range(B) for t in range(T)]
        gpu = gpu.reshape(B * T, -1)
        orc = orc.reshape(B * T, -1)
    worst = 0.0
    for r, (b, t) in enumerate(rows):
        n = _n_visible(lens[b], T, t, compress)
        if full_mask:
            assert np.all(np.isneginf(gpu[r, n:])), f"row {(b, t)}: invisible score not -inf"
        if n == 0:
            continue
        g, o = gpu[r, :n].astype(np.float64), orc[r, :n].astype(np.float64)
        assert np.all(np.isfinite(g)), f"row {(b, t)}: non-finite GPU score at a visible position"
        floor = 1e-3 * np.abs(o).max()
        tol = SCORE_RTOL * np.maximum(np.abs(o), floor)
        err = np.abs(g - o)
        bad = np.flatnonzero(err > tol)
        assert bad.size == 0, (f"row {(b, t)}: {bad.size} scores off, first at s={bad[0]}: "
                               f"gpu={g[bad[0]]} oracle={o[bad[0]]}")
        worst = max(worst, float((err / np.maximum(tol, 1e-300)).max()) * SCORE_RTOL)
    return worst


def check_topk(gpu_idx: np.ndarray, orc_scores: np.ndarray, orc_idx: np.ndarray, lens, T: int,
               k: int, rows=None, compress: int = 1):
    """gpu_idx/orc_idx: [R, k]; orc_scores: [R, Lmax]; rows: list of (b, t)."""
    if rows is None:
        B = gpu_idx.shape[0]
        rows = [(b, t) for b in range(B) for t in range(T)]
        gpu_idx = gpu_idx.reshape(B * T, k)
        orc_idx = orc_idx.reshape(B * T, k)
        orc_scores = orc_scores.reshape(B * T, -1)
    swaps = 0
    for r, (b, t) in enumerate(rows):
        n = _n_visible(lens[b], T, t, compress)
        kk = min(k, n)
        g = gpu_idx[r]
        assert np.all(g[kk:] == -1), f"row {(b, t)}: tail is not -1"
        gv = g[:kk]
        assert np.all(gv >= 0) and np.all(gv < n), f"row {(b, t)}: index out of the visible range"
        assert np.all(np.diff(gv) > 0), f"row {(b, t)}: not strictly ascending / duplicates"
        ov = orc_idx[r, :kk]
        diff = np.setxor1d(gv, ov)
        if diff.size:
            sc = orc_scores[r, :n].astype(np.float64)
            tau = np.sort(sc)[::-1][kk - 1]
            floor = 1e-3 * np.abs(sc).max()
            tol = SCORE_RTOL * max(abs(tau), floor)
            off = diff[np.abs(sc[diff] - tau) > tol]
            assert off.size == 0, (f"row {(b, t)}: selection differs beyond the tie band at "
                                   f"{off[:5]} (scores {sc[off[:5]]}, tau {tau})")
            swaps += diff.size // 2
    return swaps


def check_attention(out_g, lse_g, out_o, lse_o, dtype: str):
    out_g = np.asarray(out_g, np.float64)
    err = np.abs(out_g - out_o)
    assert np.all(np.isfinite(out_g)), "non-finite attention output"
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= ATTN_ATOL[dtype], f"attention max abs err {err.max()} at {i}"
    if lse_g is not None:
        lse_g = np.asarray(lse_g, np.float64)
        fin = np.isfinite(lse_o)
        assert np.array_equal(fin, np.isfinite(lse_g)), "lse -inf pattern differs"
        if fin.any():
            lerr = np.abs(lse_g[fin] - lse_o[fin])
            assert lerr.max() <= LSE_ATOL[dtype], f"lse max abs err {lerr.max()}"
    return float(err.max())


PREP_SCALE_RTOL = 2e-6
PREP_MID_TOL = 2e-3


def _e4m3_decode(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def check_prep(codes_g, scale_g, y_o, scale_o):
    """GPU codes/scales of the indexer preparation against the oracle's pre-rounding
    values y_o (x / scale in float64) and scales; returns the number of codes that took
    the other neighbour at a midpoint."""
    scale_g = np.asarray(scale_g, np.float64)
    rel = np.abs(scale_g - scale_o) / scale_o
    assert rel.max() <= PREP_SCALE_RTOL, f"prep scale rel err {rel.max()}"
    grid = _e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))          # 0 .. 448 ascending
    y = np.clip(np.asarray(y_o, np.float64), -448.0, 448.0)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(grid, a), 1, len(grid) - 1)
    lo_v, hi_v = grid[hi - 1], grid[hi]
    mid = (lo_v + hi_v) / 2
    # nearest, ties to the even code (codes of lo_v and hi_v are hi - 1 and hi)
    near = np.where(a < mid, lo_v, np.where(a > mid, hi_v, np.where((hi - 1) % 2 == 0, lo_v, hi_v)))
    other = np.where(near == lo_v, hi_v, lo_v)
    dec = np.abs(_e4m3_decode(codes_g))
    sign_ok = (dec == 0) | (np.signbit(_e4m3_decode(codes_g)) == np.signbit(y)) | (near == 0)
    exact = dec == near
    at_mid = (np.abs(a - mid) <= PREP_MID_TOL) & (dec == other)
    ok = (exact | at_mid) & sign_ok
    bad = np.flatnonzero(~ok.ravel())
    assert bad.size == 0, (f"prep codes: {bad.size} mismatches, first at flat {bad[:5]}: "
                           f"y={y.ravel()[bad[:5]]} gpu={dec.ravel()[bad[:5]]} want={near.ravel()[bad[:5]]}")
    return int(np.count_nonzero(at_mid & ~exact))
