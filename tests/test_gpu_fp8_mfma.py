"""Precision of the two matrix-core forms of the indexer contraction (needs an MI355X).

The per-head dot products q_j . k_s of the score box ("dsa-indexer.excalidraw") are run on
the gfx950 FP8 instruction and on the bf16 form over exactly widened codes, through the
library's diagnostic entry point, and compared with exact sums; both are then carried
through the rest of the score (per-head ReLU, head weights and scales, sum over heads) and
checked against the score tolerance of the parity tests.  The index kernels use the bf16
form: this test measures why -- the FP8 form's error is reported and must exceed that
tolerance somewhere in the sample, while the bf16 form must stay within fp32 rounding.
Inputs: the seeded indexer codes of a two-sequence, 2048-key slice of the V3.2-size
decode workload (64 heads x 128)."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import dsa_synth as S
from parity import SCORE_RTOL

pytestmark = pytest.mark.gpu


def _decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_fp8_and_bf16_matrix_core_dots():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import deepseek_dsa_indexer_amd as D
    D.load()
    cfg = dataclasses.replace(S.CONFIGS["decode_v32"], name="fp8dots", B=2, Lmax=2048, seed=901)
    c = S.make_case(cfg)
    B, H, L, Dd = cfg.B, cfg.H_I, cfg.Lmax, cfg.D_I
    qc = c["q_i"].reshape(B, H, Dd)
    kc = c["k_i"].reshape(B, L, Dd)
    # every (b, h, s) pair: row p = (b H + h) L + s
    a = np.repeat(qc[:, :, None, :], L, axis=2).reshape(-1, Dd)
    b = np.repeat(kc[:, None, :, :], H, axis=1).reshape(-1, Dd)
    ga = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    gb = torch.from_numpy(np.ascontiguousarray(b)).cuda()
    d8, db = D.diag_fp8_mfma_dots(ga, gb)
    torch.cuda.synchronize()
    d8 = d8.double().cpu().numpy().reshape(B, H, L)
    db = db.double().cpu().numpy().reshape(B, H, L)
    qv, kv = _decode(qc), _decode(kc)
    exact = np.einsum("bhd,bld->bhl", qv, kv)
    absum = np.einsum("bhd,bld->bhl", np.abs(qv), np.abs(kv))
    rel8 = np.abs(d8 - exact) / np.maximum(absum, 1e-300)
    relb = np.abs(db - exact) / np.maximum(absum, 1e-300)
    # exact products, fp32 accumulation of 128 of them: at most 128 units of 2^-24
    assert relb.max() <= 128 * 2.0 ** -24, f"bf16 form: error {relb.max():.3e} of sum|q k|"

    # the rest of the score: sum_h w_h q_scale_h relu(d_h), times the key scale and sm_scale
    wq = (c["w"].reshape(B, H) * c["q_scale"].reshape(B, H)).astype(np.float64)
    ks = c["k_scale"].reshape(B, L).astype(np.float64)

    def score(d):
        return np.einsum("bh,bhl->bl", wq, np.maximum(d, 0.0)) * ks * cfg.sm_scale_i

    so, s8, sb = score(exact), score(d8), score(db)

    def violations(g):
        floor = 1e-3 * np.abs(so).max(axis=1, keepdims=True)
        tol = SCORE_RTOL * np.maximum(np.abs(so), floor)
        return int(np.count_nonzero(np.abs(g - so) > tol)), float((np.abs(g - so) / tol).max())

    nb, wb = violations(sb)
    n8, w8 = violations(s8)
    print(f"\n[fp8 dots] {rel8.size} dots: FP8 form max error {rel8.max():.3e}, median "
          f"{np.median(rel8):.3e} of sum|q k|; bf16 form max {relb.max():.3e}", flush=True)
    print(f"[fp8 dots] {so.size} scores: FP8 form {n8} outside the score tolerance "
          f"(worst {w8:.2f}x it), bf16 form {nb} (worst {wb:.3f}x)", flush=True)
    sys.stdout.flush()
    assert nb == 0, "bf16 form: scores outside the tolerance"
    assert n8 > 0, ("FP8 form: every score within the tolerance -- the reason the index kernels "
                    "widen to bf16 no longer holds on this device")
