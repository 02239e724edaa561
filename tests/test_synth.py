"""The seeded input generator: storage formats, determinism, poisoning, subsets."""
import numpy as np
import pytest
import torch

import dsa_synth as S


def _nearest_even_e4m3(y):
    """Brute force: nearest finite e4m3fn value, ties to the even code."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ok = np.isfinite(vals)
    codes, vals = codes[ok], vals[ok]
    out = np.empty(y.shape, np.uint8)
    for i, x in enumerate(y.ravel()):
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        cand = codes[best]
        if len(cand) > 1:
            # drop -0 if +0 is also a candidate (same value): prefer the sign of x
            even = cand[(cand & 1) == 0]
            cand = even if len(even) else cand
            if len(cand) > 1:
                cand = cand[(cand >> 7) == (1 if x < 0 else 0)]
        out.ravel()[i] = cand[0]
    return out


def test_quantizer_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 128)).astype(np.float32) * 3
    codes, scale = S.quantize_e4m3fn(x, 128)
    assert scale.shape == (64, 1)
    y = np.clip(x / scale, -448, 448)
    np.testing.assert_array_equal(codes, _nearest_even_e4m3(y))
    # the block maximum maps to +-448 exactly
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.allclose(np.abs(vals).max(axis=1), 448.0)


def test_case_shapes_poison_and_subset():
    cfg = S.CONFIGS["tiny"]
    case = S.make_case(cfg)
    assert case["q_i"].shape == (1, 64, 4, 32) and case["k_i"].shape == (1, 64, 32)
    assert case["q"].dtype == np.float32 and case["latent"].shape == (1, 64, 80)
    again = S.make_case(cfg)
    for key in ("q_i", "k_i", "w", "q", "latent"):
        np.testing.assert_array_equal(case[key], again[key])


def test_ragged_lengths_and_poison():
    cfg = S.CONFIGS["decode_ragged"]
    lens = S.lengths(cfg)
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 65536
    small = S.Config(**{**cfg.__dict__, "B": 3, "Lmax": 4096, "lens": "ragged:1000:3000"})
    case = S.make_case(small)
    for b in range(3):
        L = int(case["lens"][b])
        assert np.all(case["k_i"][b, L:] == S.POISON_K_CODE)
        assert np.all(case["k_scale"][b, L:] == S.POISON_VALUE)
        lat = torch.from_numpy(case["latent"][b, L:].view(np.int16)).view(torch.bfloat16).float()
        assert torch.all(lat == torch.tensor(S.POISON_VALUE).bfloat16().float())
    sub = S.make_case(small, seqs=[2])
    np.testing.assert_array_equal(sub["k_i"][0], case["k_i"][2])
    np.testing.assert_array_equal(sub["latent"][0], case["latent"][2])


def test_fp8_latent_rows():
    """656-byte rows: codes and scales from the blockwise quantizer of the same float32
    draws as the bf16 cache, bf16 rope bytes equal to the bf16 cache's, poison beyond len."""
    import dataclasses
    cfg = dataclasses.replace(S.CONFIGS["decode_ragged"], B=2, Lmax=96, lens="ragged:40:96")
    a = S.make_case(cfg, latent_form="fp8")
    b = S.make_case(cfg)
    lat8, lat16 = a["latent"], b["latent"]
    assert lat8.dtype == np.uint8 and lat8.shape == (2, 96, S.FP8_LATENT_ROW_BYTES)
    np.testing.assert_array_equal(a["q"], b["q"])
    for j, L in enumerate(a["lens"]):
        L = int(L)
        x = np.random.default_rng([cfg.seed, 4, j]).standard_normal((L, 576), dtype=np.float32)
        codes, scales = S.quantize_e4m3fn(x[:, :512], 128)
        np.testing.assert_array_equal(lat8[j, :L, :512], codes)
        np.testing.assert_array_equal(lat8[j, :L, 512:528].view(np.float32), scales)
        np.testing.assert_array_equal(lat8[j, :L, 528:].view(np.uint16), lat16[j, :L, 512:])
        assert (lat8[j, L:, :512] == S.POISON_K_CODE).all()
        assert (lat8[j, L:, 512:528].view(np.float32) == S.POISON_VALUE).all()
    with pytest.raises(AssertionError):
        S.make_case(S.CONFIGS["tiny"], latent_form="fp8")
