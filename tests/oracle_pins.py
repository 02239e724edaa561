"""Pins of the CPU reference against facts that do not come from the reference itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError on a
mismatch.  They are collected by ``test_oracle_pins.py`` and re-run by
``test_oracle_mutations.py`` against deliberately broken builds of the oracle, to
show that a plausible mistake (a dropped term, a wrong sign or index, a transposed
operand) fails at least one of them.

What pins what:
  * e4m3fn decoding        -> torch's float8_e4m3fn decoding of all 256 codes;
  * index scores           -> closed forms (all products positive: the score is a
                              plain matrix product, computed by torch.matmul; all
                              products negative: exactly zero; one head positive),
                              the causal pattern, and invariances (head order,
                              column order, scale linearity);
  * top-k                  -> torch.topk / numpy's stable argsort, cardinality and
                              ordering invariants;
  * sparse attention       -> torch's scaled_dot_product_attention with a boolean
                              mask of the selected and visible keys (k >= n is
                              plain dense causal attention), k = 1, equal values;
  * MHA prefill            -> the same library routine per head, and the pages'
                              dense "scores + index mask + causal mask" form;
  * layer step             -> with k >= len the result is dense attention whatever
                              the indexer does; a planted dominant key is picked;
  * indexer preparation    -> the e4m3fn encoder against torch's float8 cast (all
                              midpoints, ties, signed zeros), rope against complex
                              multiplication and the rotation against scipy's Hadamard
                              matrix (recovered through the returned scales), a
                              quantisation closed form, the cache append placement;
  * compressed entries     -> the V4 visualiser's tiny configuration (16 positions,
                              compress rate 4, top-2): warm-up rows of -1 sentinels,
                              then one, two, three, four available entries; scores,
                              top-k and attention under compression equal the
                              uncompressed ones restricted to the available entries;
  * FP8 latent rows        -> torch's float8_e4m3fn and bfloat16 decoding at the
                              656-byte layout (512 codes, 4 fp32 block scales, 64
                              bf16 rope values), and attention over such rows ==
                              SDPA over the torch-decoded rows.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def _fp8_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _rand_codes(rng, shape, positive=False, negative=False):
    # finite e4m3fn codes: exclude 0x7F / 0xFF (NaN)
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)   # 0x00..0x7E, all >= 0
    if negative:
        c = c | 0x80
    elif not positive:
        c = c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)
    return c


def _nonzero_pos_codes(rng, shape):
    # strictly positive normal codes 0x08..0x7E (values 2^-6 .. 448)
    return rng.integers(0x08, 0x7F, size=shape).astype(np.uint8)


# ----------------------------------------------------------------------------- codec

def pin_e4m3fn_codec(o):
    codes = np.arange(256, dtype=np.uint8)
    ref = _fp8_values(codes)
    got = np.array([o.e4m3fn_value(int(c)) for c in codes])
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got)), "NaN codes differ"
    assert set(np.flatnonzero(nan_ref)) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], got[~nan_ref]), "finite e4m3fn values differ"
    assert o.e4m3fn_value(0x7E) == 448.0 and o.e4m3fn_value(0x01) == 2.0 ** -9


def pin_bf16_codec(o):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=512).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([o.bf16_value(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], got[fin])


# ----------------------------------------------------------------------------- index scores

def _idx_case(rng, B, T, H, D, Lmax, lens, qpos=False, kpos=False, qneg=False):
    q = _nonzero_pos_codes(rng, (B, T, H, D)) if qpos else _rand_codes(rng, (B, T, H, D), negative=qneg)
    k = _nonzero_pos_codes(rng, (B, Lmax, D)) if kpos else _rand_codes(rng, (B, Lmax, D))
    qs = rng.uniform(0.5, 2.0, (B, T, H)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2.0, (B, Lmax)).astype(np.float32)
    return q, qs, w, k, ks, np.asarray(lens, np.int32)


def pin_index_scores_positive_closed_form(o):
    """All q and k codes positive -> every product is positive, ReLU is the identity and
    the score is k_scale[s] * ((w*q_scale*sm) @ Q) . K[s]: one matrix product."""
    rng = np.random.default_rng(21)
    B, T, H, D, Lmax = 2, 3, 5, 32, 40
    lens = [40, 37]
    q, qs, w, k, ks, lens = _idx_case(rng, B, T, H, D, Lmax, lens, qpos=True, kpos=True)
    sm = D ** -0.5
    got = o.index_scores(q, qs, w, k, ks, lens, sm)
    Q = torch.from_numpy(_fp8_values(q))
    K = torch.from_numpy(_fp8_values(k))
    wf = torch.from_numpy(w.astype(np.float64) * qs.astype(np.float64) * sm)
    for b in range(B):
        for t in range(T):
            pos = int(lens[b]) - T + t
            u = wf[b, t] @ Q[b, t]                        # [D]
            ref = torch.matmul(K[b, : pos + 1], u) * torch.from_numpy(ks[b, : pos + 1].astype(np.float64))
            np.testing.assert_allclose(got[b, t, : pos + 1], ref.numpy(), rtol=2e-7, atol=0)
            assert np.all(np.isneginf(got[b, t, pos + 1:]))


def pin_index_scores_relu_zero(o):
    """All q codes negative, all k codes positive -> every product < 0 -> score exactly 0."""
    rng = np.random.default_rng(22)
    q, qs, w, k, ks, lens = _idx_case(rng, 1, 1, 4, 32, 16, [16], qneg=True, kpos=True)
    q = q | 0x80
    q[q == 0x80] = 0x88          # no negative zero: strictly negative values
    got = o.index_scores(q, qs, w, k, ks, lens, 1.0)
    assert np.all(got == 0.0)


def pin_index_scores_one_head(o):
    """Head 0 has positive products and a NEGATIVE weight; heads 1.. have negative
    products.  ReLU then weight: the score is w0*qs0*sm*dot0*ks (negative)."""
    rng = np.random.default_rng(23)
    H, D, L = 4, 32, 24
    q = np.empty((1, 1, H, D), np.uint8)
    q[0, 0, 0] = _nonzero_pos_codes(rng, D)
    q[0, 0, 1:] = _nonzero_pos_codes(rng, (H - 1, D)) | 0x80
    k = _nonzero_pos_codes(rng, (1, L, D))
    qs = rng.uniform(0.5, 2.0, (1, 1, H)).astype(np.float32)
    w = -np.abs(rng.standard_normal((1, 1, H))).astype(np.float32) - 0.1
    ks = rng.uniform(0.5, 2.0, (1, L)).astype(np.float32)
    sm = 0.25
    got = o.index_scores(q, qs, w, k, ks, np.array([L], np.int32), sm)
    K = torch.from_numpy(_fp8_values(k[0]))
    dot0 = torch.matmul(K, torch.from_numpy(_fp8_values(q[0, 0, 0])))
    ref = float(w[0, 0, 0]) * float(qs[0, 0, 0]) * sm * dot0.numpy() * ks[0].astype(np.float64)
    assert np.all(ref < 0)
    np.testing.assert_allclose(got[0, 0], ref, rtol=2e-7)


def pin_index_scores_relu_per_head_mixed_signs(o):
    """The ReLU of the score box acts on each head's whole dot product, not on the single
    products: two heads whose products have mixed signs, values worked out by hand.
      head 0: q = [2, -1],  head 1: q = [1, -3]   (other columns 0)
      key 0 = [ 1,  1]: dots ( 1, -2) -> ReLU ( 1, 0)
      key 1 = [ 1,  2]: dots ( 0, -5) -> ( 0, 0)
      key 2 = [ 2,  1]: dots ( 3, -1) -> ( 3, 0)
      key 3 = [-1, -1]: dots (-1,  2) -> ( 0, 2)
    With w = [0.5, -0.25], q_scale = [1, 2], sm = 1 and key scales 1 the folded weights
    are [0.5, -0.5], so the scores are exactly [0.5, 0, 1.5, -1].  Clipping each product
    at zero instead would give [0.5, 0.5, 1.5, -1]; no ReLU at all [1.5, 2.5, 2, -1.5]."""
    one, two, three = 0x38, 0x40, 0x44          # e4m3fn codes of 1, 2, 3
    neg = 0x80
    D = 32
    q = np.zeros((1, 1, 2, D), np.uint8)
    q[0, 0, 0, :2] = [two, one | neg]
    q[0, 0, 1, :2] = [one, three | neg]
    k = np.zeros((1, 4, D), np.uint8)
    k[0, 0, :2] = [one, one]
    k[0, 1, :2] = [one, two]
    k[0, 2, :2] = [two, one]
    k[0, 3, :2] = [one | neg, one | neg]
    qs = np.array([[[1.0, 2.0]]], np.float32)
    w = np.array([[[0.5, -0.25]]], np.float32)
    ks = np.ones((1, 4), np.float32)
    got = o.index_scores(q, qs, w, k, ks, np.array([4], np.int32), 1.0)
    np.testing.assert_array_equal(got[0, 0], np.array([0.5, 0.0, 1.5, -1.0], np.float32))


def pin_index_scores_invariances(o):
    """Mixed signs: permuting heads (with their weights) or permuting the d columns of q and
    k together leaves the scores unchanged; doubling k_scale doubles them; the visible
    pattern is s <= len - T + t."""
    rng = np.random.default_rng(24)
    B, T, H, D, Lmax = 2, 4, 6, 64, 30
    q, qs, w, k, ks, lens = _idx_case(rng, B, T, H, D, Lmax, [30, 19])
    sm = D ** -0.5
    base = o.index_scores(q, qs, w, k, ks, lens, sm)
    perm_h = rng.permutation(H)
    g = o.index_scores(q[:, :, perm_h], qs[:, :, perm_h], w[:, :, perm_h], k, ks, lens, sm)
    np.testing.assert_allclose(g, base, rtol=1e-6, atol=1e-30)
    perm_d = rng.permutation(D)
    g = o.index_scores(q[..., perm_d], qs, w, k[..., perm_d], ks, lens, sm)
    np.testing.assert_array_equal(g, base)
    g = o.index_scores(q, qs, w, k, ks * 2, lens, sm)
    np.testing.assert_array_equal(g, base * 2)
    for b in range(B):
        for t in range(T):
            pos = int(lens[b]) - T + t
            assert np.all(np.isfinite(base[b, t, : pos + 1]))
            assert np.all(np.isneginf(base[b, t, pos + 1:]))
    # a non-trivial mix of positive and zero contributions
    assert np.any(base[np.isfinite(base)] > 0) and np.any(base[np.isfinite(base)] < 0)


# ----------------------------------------------------------------------------- top-k

def pin_topk_library(o):
    """Distinct scores: the chosen set equals torch.topk's; order ascending; -1 tail."""
    rng = np.random.default_rng(31)
    B, T, Lmax, k = 3, 5, 50, 12
    lens = np.array([50, 20, 9], np.int32)
    scores = rng.standard_normal((B, T, Lmax)).astype(np.float32)
    for b in range(B):
        for t in range(T):
            scores[b, t, int(lens[b]) - T + t + 1:] = -np.inf
    idx = o.topk(scores, lens, k)
    for b in range(B):
        for t in range(T):
            n = int(lens[b]) - T + t + 1
            kk = min(k, n)
            ref = torch.topk(torch.from_numpy(scores[b, t, :n]), kk).indices.numpy()
            row = idx[b, t]
            assert set(row[:kk].tolist()) == set(ref.tolist())
            assert np.all(np.diff(row[:kk]) > 0)
            assert np.all(row[kk:] == -1)
            assert row[:kk].max() <= n - 1


def pin_topk_ties(o):
    """Heavy ties: the chosen set is the first k of a stable descending sort (equal scores
    keep the smaller position); every chosen score >= every unchosen visible score."""
    rng = np.random.default_rng(32)
    B, T, Lmax, k = 2, 3, 64, 10
    lens = np.array([64, 40], np.int32)
    scores = rng.integers(-3, 4, size=(B, T, Lmax)).astype(np.float32)
    idx = o.topk(scores, lens, k)
    for b in range(B):
        for t in range(T):
            n = int(lens[b]) - T + t + 1
            order = np.argsort(-scores[b, t, :n], kind="stable")[:k]
            assert sorted(idx[b, t, :k].tolist()) == sorted(order.tolist())
            chosen = scores[b, t, idx[b, t, :k]]
            rest = np.delete(scores[b, t, :n], idx[b, t, :k])
            assert chosen.min() >= rest.max()


def pin_topk_short_rows(o):
    """n <= k: every visible position is returned, padded with -1."""
    scores = np.random.default_rng(33).standard_normal((1, 4, 8)).astype(np.float32)
    lens = np.array([6], np.int32)
    idx = o.topk(scores, lens, 8)
    for t in range(4):
        n = 6 - 4 + t + 1
        assert idx[0, t, :n].tolist() == list(range(n))
        assert np.all(idx[0, t, n:] == -1)


# ----------------------------------------------------------------------------- attention

def _sdpa_rows(q, keys, vals, mask, scale):
    """torch SDPA in float64: q [H,E], keys [S,E], vals [S,Ev], mask [S] bool."""
    out = F.scaled_dot_product_attention(q[None], keys[None], vals[None],
                                         attn_mask=mask[None, None, :].expand(1, q.shape[0], -1),
                                         scale=scale)
    return out[0]


def pin_latent_attention_library(o):
    """Sparse latent attention == SDPA over a boolean mask of the selected and visible
    positions (with k >= n this is plain dense causal attention)."""
    rng = np.random.default_rng(41)
    B, T, H, Dv, Dr, Lmax = 2, 3, 4, 24, 8, 40
    lens = np.array([40, 21], np.int32)
    q = rng.standard_normal((B, T, H, Dv + Dr))
    lat = rng.standard_normal((B, Lmax, Dv + Dr))
    sm = (Dv + Dr) ** -0.5
    for k in (7, 64):
        idx = np.full((B, T, k), -1, np.int32)
        for b in range(B):
            for t in range(T):
                n = int(lens[b]) - T + t + 1
                m = min(k, n)
                idx[b, t, :m] = rng.choice(n, size=m, replace=False)
        if k == 7:
            # one selected slot per row points past the row's position: it must be ignored
            for b in range(B):
                for t in range(T):
                    pos = int(lens[b]) - T + t
                    idx[b, t, -1] = rng.integers(pos + 1, Lmax) if pos + 1 < Lmax else -1
        out, lse = o.sparse_mla_decode(q, lat, idx, lens, Dv, sm)
        for b in range(B):
            for t in range(T):
                pos = int(lens[b]) - T + t
                mask = torch.zeros(Lmax, dtype=torch.bool)
                sel = idx[b, t][(idx[b, t] >= 0) & (idx[b, t] <= pos)]
                mask[torch.from_numpy(sel.astype(np.int64))] = True
                C = torch.from_numpy(lat[b])
                ref = _sdpa_rows(torch.from_numpy(q[b, t]), C, C[:, :Dv], mask, sm)
                np.testing.assert_allclose(out[b, t], ref.numpy(), rtol=1e-10, atol=1e-12)
                logits = torch.from_numpy(q[b, t]) @ C[mask].T * sm
                np.testing.assert_allclose(lse[b, t], torch.logsumexp(logits, -1).numpy(), rtol=1e-12)


def pin_latent_attention_special(o):
    """k = 1 -> the selected value row exactly; all value rows equal -> that row."""
    rng = np.random.default_rng(42)
    H, Dv, Dr, L = 3, 16, 4, 12
    q = rng.standard_normal((1, 1, H, Dv + Dr))
    lat = rng.standard_normal((1, L, Dv + Dr))
    idx = np.array([[[5]]], np.int32)
    out, lse = o.sparse_mla_decode(q, lat, idx, np.array([L], np.int32), Dv, 0.3)
    for h in range(H):
        np.testing.assert_array_equal(out[0, 0, h], lat[0, 5, :Dv])
        np.testing.assert_allclose(lse[0, 0, h], 0.3 * q[0, 0, h] @ lat[0, 5], rtol=1e-13)
    lat2 = lat.copy()
    lat2[0, :, :Dv] = lat[0, 0, :Dv]
    idx = np.array([[[0, 3, 7, -1]]], np.int32)
    out, _ = o.sparse_mla_decode(q, lat2, idx, np.array([L], np.int32), Dv, 0.3)
    for h in range(H):
        np.testing.assert_allclose(out[0, 0, h], lat[0, 0, :Dv], rtol=1e-13)


def pin_mha_prefill_library(o):
    """Per head, sparse MHA == SDPA with mask = selected & (s <= t); the pages' dense
    index-mask form agrees."""
    rng = np.random.default_rng(43)
    B, T, H, Dqk, Dv, k = 1, 12, 3, 20, 10, 5
    q = rng.standard_normal((B, T, H, Dqk))
    kk = rng.standard_normal((B, T, H, Dqk))
    v = rng.standard_normal((B, T, H, Dv))
    idx = np.full((B, T, k), -1, np.int32)
    for t in range(T):
        m = min(k, T)
        idx[0, t, :m] = rng.choice(T, size=m, replace=False)   # may include s > t
    idx[0, 0, 0] = 0                                            # every row sees >= 1 key
    for t in range(1, T):
        if not np.any((idx[0, t] >= 0) & (idx[0, t] <= t)):
            idx[0, t, 0] = t
    sm = Dqk ** -0.5
    out, lse = o.sparse_mha_prefill(q, kk, v, idx, sm)
    out_d, lse_d = o.sparse_mha_prefill_dense(q, kk, v, idx, sm)
    rows = [(0, 11), (0, 0), (0, 5)]
    out_r, lse_r = o.sparse_mha_prefill_rows(q, kk, v, idx, sm, rows)
    for i, (b, t) in enumerate(rows):
        np.testing.assert_array_equal(out_r[i], out[b, t])
        np.testing.assert_array_equal(lse_r[i], lse[b, t])
    np.testing.assert_allclose(out, out_d, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_d, rtol=1e-12)
    for t in range(T):
        mask = torch.zeros(T, dtype=torch.bool)
        sel = idx[0, t][(idx[0, t] >= 0) & (idx[0, t] <= t)]
        mask[torch.from_numpy(sel.astype(np.int64))] = True
        for h in range(H):
            ref = _sdpa_rows(torch.from_numpy(q[0, t, h][None]), torch.from_numpy(kk[0, :, h]),
                             torch.from_numpy(v[0, :, h]), mask, sm)
            np.testing.assert_allclose(out[0, t, h], ref[0].numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- layer step

def pin_layer_step_dense_limit(o):
    """k >= len: the selection keeps every visible key, so the step is dense causal
    attention (SDPA with is_causal-style mask) whatever the index scores are."""
    rng = np.random.default_rng(51)
    B, T, H_I, D_I, Lmax = 1, 16, 4, 32, 16
    H, Dv, Dr = 2, 16, 8
    q_i = _rand_codes(rng, (B, T, H_I, D_I))
    k_i = _rand_codes(rng, (B, Lmax, D_I))
    qs = np.ones((B, T, H_I), np.float32)
    w = rng.standard_normal((B, T, H_I)).astype(np.float32)
    ks = np.ones((B, Lmax), np.float32)
    lens = np.array([Lmax], np.int32)
    q = rng.standard_normal((B, T, H, Dv + Dr))
    lat = rng.standard_normal((B, Lmax, Dv + Dr))
    sm = 0.2
    out, lse, idx = o.layer_step_latent(q_i, qs, w, k_i, ks, lens, D_I ** -0.5, 16, q, lat, Dv, sm)
    C = torch.from_numpy(lat[0])
    for t in range(T):
        mask = torch.arange(Lmax) <= t
        ref = _sdpa_rows(torch.from_numpy(q[0, t]), C, C[:, :Dv], mask, sm)
        np.testing.assert_allclose(out[0, t], ref.numpy(), rtol=1e-10, atol=1e-12)


def pin_layer_step_planted_key(o):
    """k = 1 with one key whose index score dominates: the output is that key's value
    row for every head (decode, T = 1)."""
    rng = np.random.default_rng(52)
    H_I, D_I, L = 4, 32, 20
    H, Dv, Dr = 3, 16, 8
    q_i = _nonzero_pos_codes(rng, (1, 1, H_I, D_I))
    q_i[..., :] = 0x38                                   # 1.0 everywhere
    k_i = _rand_codes(rng, (1, L, D_I))
    k_i[0, :] = k_i[0, :] | 0x80                         # all keys negative ...
    k_i[0, 13] = 0x40                                    # ... except key 13 (= 2.0)
    qs = np.ones((1, 1, H_I), np.float32)
    w = np.ones((1, 1, H_I), np.float32)
    ks = np.ones((1, L), np.float32)
    q = rng.standard_normal((1, 1, H, Dv + Dr))
    lat = rng.standard_normal((1, L, Dv + Dr))
    out, lse, idx = o.layer_step_latent(q_i, qs, w, k_i, ks, np.array([L], np.int32),
                                        D_I ** -0.5, 1, q, lat, Dv, 0.1)
    assert idx[0, 0, 0] == 13
    for h in range(H):
        np.testing.assert_array_equal(out[0, 0, h], lat[0, 13, :Dv])


def pin_layer_step_mha_dense_limit(o):
    """MHA form with k >= T equals per-head dense causal attention (SDPA is_causal)."""
    rng = np.random.default_rng(53)
    B, T, H_I, D_I, H, Dqk, Dv = 1, 10, 4, 32, 2, 12, 6
    q_i = _rand_codes(rng, (B, T, H_I, D_I))
    k_i = _rand_codes(rng, (B, T, D_I))
    qs = np.ones((B, T, H_I), np.float32)
    w = rng.standard_normal((B, T, H_I)).astype(np.float32)
    ks = np.ones((B, T), np.float32)
    q = rng.standard_normal((B, T, H, Dqk))
    kk = rng.standard_normal((B, T, H, Dqk))
    v = rng.standard_normal((B, T, H, Dv))
    out, lse, idx = o.layer_step_mha(q_i, qs, w, k_i, ks, D_I ** -0.5, T, q, kk, v, 0.3)
    qt = torch.from_numpy(q[0]).transpose(0, 1)      # [H,T,D]
    kt = torch.from_numpy(kk[0]).transpose(0, 1)
    vt = torch.from_numpy(v[0]).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.3).transpose(0, 1)
    np.testing.assert_allclose(out[0], ref.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- FP8 latent rows

def _fp8_latent_rows(rng, n):
    """n random 656-byte rows: finite codes, fp32 scales over a wide range, finite bf16
    rope values.  Returns (rows u8 [n,656], torch-decoded float64 [n,576])."""
    codes = _rand_codes(rng, (n, 512))
    scales = (2.0 ** rng.uniform(-12, 6, size=(n, 4))).astype(np.float32)
    rope = torch.from_numpy(rng.standard_normal((n, 64)).astype(np.float32)).to(torch.bfloat16)
    rows = np.concatenate([codes, scales.view(np.uint8).reshape(n, 16),
                           rope.view(torch.int16).numpy().view(np.uint8).reshape(n, 128)], axis=1)
    ref = np.concatenate([_fp8_values(codes) * np.repeat(scales.astype(np.float64), 128, axis=1),
                          rope.double().numpy()], axis=1)
    return rows, ref


def pin_latent_fp8_decode_library(o):
    """The 656-byte row (the diagram's per-token latent figure) decodes, column by column,
    to torch's e4m3fn value times the scale of its 128-column block, then torch's bf16
    rope values."""
    assert 512 + 4 * 4 + 64 * 2 == 656 == o.FP8_LATENT_ROW_BYTES
    rows, ref = _fp8_latent_rows(np.random.default_rng(71), 6)
    got = o.latent_fp8_decode(rows)
    np.testing.assert_array_equal(got, ref)


def pin_latent_fp8_attention_library(o):
    """Sparse latent attention over FP8 rows with bf16 queries == SDPA in float64 over the
    torch-decoded rows (keys: all 576 columns, values: the first 512)."""
    rng = np.random.default_rng(72)
    B, T, H, Lmax, k = 2, 2, 3, 20, 6
    lens = np.array([20, 13], np.int32)
    rows, ref = _fp8_latent_rows(rng, B * Lmax)
    rows, ref = rows.reshape(B, Lmax, 656), ref.reshape(B, Lmax, 576)
    qf = torch.from_numpy(rng.standard_normal((B, T, H, 576)).astype(np.float32)).to(torch.bfloat16)
    q_bits = qf.view(torch.int16).numpy().view(np.uint16)
    sm = 192.0 ** -0.5
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = int(lens[b]) - T + t + 1
            idx[b, t, :k - 1] = rng.choice(n, size=k - 1, replace=False)
            idx[b, t, k - 1] = min(n, Lmax - 1) if n < Lmax else -1   # past pos: ignored
    out, lse = o.sparse_mla_decode(q_bits, rows, idx, lens, 512, sm)
    for b in range(B):
        for t in range(T):
            pos = int(lens[b]) - T + t
            mask = torch.zeros(Lmax, dtype=torch.bool)
            sel = idx[b, t][(idx[b, t] >= 0) & (idx[b, t] <= pos)]
            mask[torch.from_numpy(sel.astype(np.int64))] = True
            C = torch.from_numpy(ref[b])
            qd = qf[b, t].double()
            want = _sdpa_rows(qd, C, C[:, :512], mask, sm)
            np.testing.assert_allclose(out[b, t], want.numpy(), rtol=1e-9, atol=1e-12)
            logits = qd @ C[mask].T * sm
            np.testing.assert_allclose(lse[b, t], torch.logsumexp(logits, -1).numpy(), rtol=1e-12)


# ----------------------------------------------------------------------------- compressed entries

def pin_compressed_entries_v4_tiny(o):
    """The V4 mask visualiser's tiny configuration: 16 query positions, compress rate 4,
    top-2 over the compressed entries.  Positions 0..2 have no entry yet (all slots -1,
    the warm-up sentinel); positions 3..6 have exactly entry 0; 7..10 entries 0 and 1
    (both kept); 11..14 three entries, 15 four (two kept).  Scores of unavailable
    entries are -inf."""
    rng = np.random.default_rng(91)
    S_, m, k, H, D = 16, 4, 2, 2, 32
    L_e = S_ // m
    qc = _rand_codes(rng, (1, S_, H, D))
    kc = _rand_codes(rng, (1, L_e, D))
    qs = rng.uniform(0.5, 2, (1, S_, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2, (1, L_e)).astype(np.float32)
    w = rng.standard_normal((1, S_, H)).astype(np.float32)
    lens = np.array([S_], np.int32)
    sc = o.index_scores(qc, qs, w, kc, ks, lens, 0.2, compress=m)
    idx = o.topk(sc, lens, k, compress=m)
    avail = [0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 4]
    for t in range(S_):
        n = avail[t]
        assert np.all(np.isfinite(sc[0, t, :n])) and np.all(sc[0, t, n:] == -np.inf), t
        got = idx[0, t]
        assert np.all(got[min(n, k):] == -1) and np.all(got[:min(n, k)] >= 0), (t, got)
        assert set(got[:min(n, k)]) <= set(range(n))
    assert [list(idx[0, t]) for t in (0, 2, 3, 6, 7, 10)] == [[-1, -1], [-1, -1], [0, -1], [0, -1],
                                                             [0, 1], [0, 1]]


def pin_compressed_entries_restriction(o):
    """Under compression m the scores, top-k and attention are the uncompressed ones
    restricted to the entries a row may see (e < (pos + 1) / m), over a cache of
    entries, for several query rows per sequence and ragged lengths."""
    rng = np.random.default_rng(92)
    B, T, H, D, m, k = 2, 5, 3, 32, 3, 4
    lens = np.array([40, 17], np.int32)
    Lmax = 40 // m + 1
    qc = _rand_codes(rng, (B, T, H, D))
    kc = _rand_codes(rng, (B, Lmax, D))
    qs = rng.uniform(0.5, 2, (B, T, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2, (B, Lmax)).astype(np.float32)
    w = rng.standard_normal((B, T, H)).astype(np.float32)
    sc_m = o.index_scores(qc, qs, w, kc, ks, lens, 0.3, compress=m)
    # uncompressed reference over the same Lmax entries: a call whose rows all see the
    # whole entry cache (len = Lmax, one row per call) gives every entry's score
    for b in range(B):
        for t in range(T):
            n = (int(lens[b]) - T + t + 1) // m
            full = o.index_scores(qc[b:b + 1, t:t + 1], qs[b:b + 1, t:t + 1], w[b:b + 1, t:t + 1],
                                  kc[b:b + 1], ks[b:b + 1], np.array([Lmax], np.int32), 0.3)
            np.testing.assert_array_equal(sc_m[b, t, :n], full[0, 0, :n])
            assert np.all(sc_m[b, t, n:] == -np.inf)
    idx_m = o.topk(sc_m, lens, k, compress=m)
    for b in range(B):
        for t in range(T):
            n = (int(lens[b]) - T + t + 1) // m
            order = np.argsort(-sc_m[b, t, :n].astype(np.float64), kind="stable")[:k]
            assert list(idx_m[b, t, :min(n, k)]) == sorted(order.tolist())
            assert np.all(idx_m[b, t, min(n, k):] == -1)
    # attention: the slots of unavailable entries are ignored
    q = rng.standard_normal((B, T, H, 24))
    lat = rng.standard_normal((B, Lmax, 24))
    idx = np.stack([np.stack([rng.permutation(Lmax)[:6] for _ in range(T)]) for _ in range(B)]).astype(np.int32)
    out_m, lse_m = o.sparse_mla_decode(q, lat, idx, lens, 16, 0.2, compress=m)
    idx_r = idx.copy()
    for b in range(B):
        for t in range(T):
            n = (int(lens[b]) - T + t + 1) // m
            idx_r[b, t][idx_r[b, t] >= n] = -1
    for b in range(B):
        for t in range(T):
            # one uncompressed row with len = Lmax sees every entry of the cache
            o1, l1 = o.sparse_mla_decode(q[b:b + 1, t:t + 1], lat[b:b + 1], idx_r[b:b + 1, t:t + 1],
                                         np.array([Lmax], np.int32), 16, 0.2)
            np.testing.assert_allclose(out_m[b, t], o1[0, 0], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse_m[b, t], l1[0, 0], rtol=1e-12)


# ----------------------------------------------------------------------------- indexer preparation

def _e4m3_grid():
    v = _fp8_values(np.arange(0, 0x7F, dtype=np.uint8))     # 0 .. 448, ascending
    return v


def pin_e4m3fn_encode_library(o):
    """Encoder == torch's float8_e4m3fn cast on every representable value, every midpoint
    (ties to even), points just off the midpoints, signed zeros and random values."""
    g = _e4m3_grid()
    mids = (g[:-1] + g[1:]) / 2
    rng = np.random.default_rng(81)
    xs = np.concatenate([g, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                         rng.uniform(-448, 448, 4000), rng.uniform(-0.02, 0.02, 2000)])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    xs = xs[np.abs(xs) <= 448]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([o.e4m3fn_encode(float(x)) for x in xs], np.uint8)
    bad = np.flatnonzero(ref != got)
    assert bad.size == 0, f"e4m3fn encode differs at {xs[bad[:5]]}: {got[bad[:5]]} vs {ref[bad[:5]]}"
    assert o.e4m3fn_encode(-0.0) == 0x80 and o.e4m3fn_encode(0.0) == 0x00


def _rope_angles(P, R, base=10000.0):
    j = np.arange(R // 2)
    theta = np.arange(P)[:, None] * base ** (-2.0 * j[None, :] / R)
    return theta, np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


def pin_indexer_prep_rope_and_rotation(o):
    """The pre-rounding values times their scale, rotated back with scipy's Hadamard
    matrix (its own inverse once normalised), equal the inputs rotated by complex
    multiplication: (x_j + i x_{j+R/2}) e^{i theta_j} for the rope pairs, x unchanged
    beyond R."""
    import scipy.linalg
    rng = np.random.default_rng(82)
    B, T, H, D, R, P, Lmax = 2, 3, 2, 32, 8, 40, 40
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, D))
    theta, cs, sn = _rope_angles(P, R)
    start = np.array([5, 30], np.int32)
    r = o.indexer_prep(q, k, cs, sn, start, R, np.zeros((B, Lmax, D), np.uint8),
                       np.zeros((B, Lmax), np.float32))
    Hm = scipy.linalg.hadamard(D) / np.sqrt(D)
    for b in range(B):
        for t in range(T):
            pos = start[b] + t
            e = np.cos(theta[pos]).astype(np.float32) + 1j * np.sin(theta[pos]).astype(np.float32)
            for x, y, sc in [(q[b, t, h], r["q_y"][b, t, h], r["q_scale"][b, t, h]) for h in range(H)] + \
                            [(k[b, t], r["k_y"][b, t], r["k_scale64"][b, t])]:
                want = x.copy()
                z = (x[:R // 2] + 1j * x[R // 2:R]) * e
                want[:R // 2], want[R // 2:R] = z.real, z.imag
                np.testing.assert_allclose(Hm @ (y * sc), want, rtol=1e-10, atol=1e-12)


def pin_indexer_prep_quant_closed_form(o):
    """No rotation angle (cos 1, sin 0) and a row equal to a scaled column of the
    Hadamard matrix: after the rotation the row is one spike, so its code is +-448 and
    every other value decodes to 0; the scale is |spike| / 448."""
    import scipy.linalg
    D, R = 32, 8
    Hm = scipy.linalg.hadamard(D)
    cs = np.ones((4, R // 2), np.float32)
    sn = np.zeros((4, R // 2), np.float32)
    q = np.stack([3.0 * Hm[:, 5] / np.sqrt(D), -0.5 * Hm[:, 17] / np.sqrt(D)])[None, None]
    k = (2.0 * Hm[:, 0] / np.sqrt(D))[None, None]
    r = o.indexer_prep(q, k, cs, sn, np.array([1], np.int32), R, np.zeros((1, 4, D), np.uint8),
                       np.zeros((1, 4), np.float32))
    for codes, spike, val, sc in [(r["q_fp8"][0, 0, 0], 5, 448.0, r["q_scale"][0, 0, 0]),
                                  (r["q_fp8"][0, 0, 1], 17, -448.0, r["q_scale"][0, 0, 1]),
                                  (r["k_cache"][0, 1], 0, 448.0, r["k_scale64"][0, 0])]:
        dec = _fp8_values(codes)
        assert dec[spike] == val and np.all(dec[np.arange(D) != spike] == 0.0)
    np.testing.assert_allclose(r["q_scale"][0, 0], [3.0 / 448, 0.5 / 448], rtol=1e-14)
    np.testing.assert_allclose(r["k_scale64"][0, 0], 2.0 / 448, rtol=1e-14)


def pin_indexer_prep_quant_bound_and_append(o):
    """Every code is the nearest e4m3fn value of its pre-rounding value (decoded error at
    most half a step of the e4m3 grid there), the largest magnitude of each row maps to
    +-448, and the keys land in exactly rows start..start+T-1 of the cache."""
    rng = np.random.default_rng(83)
    B, T, H, D, R, P, Lmax = 3, 4, 3, 64, 16, 60, 50
    q = rng.standard_normal((B, T, H, D)) * rng.uniform(0.01, 10, (B, T, H, 1))
    k = rng.standard_t(3, (B, T, D))
    _, cs, sn = _rope_angles(P, R)
    start = np.array([0, 17, Lmax - T], np.int32)
    kc0 = rng.integers(0, 256, (B, Lmax, D)).astype(np.uint8)
    ks0 = rng.standard_normal((B, Lmax)).astype(np.float32)
    r = o.indexer_prep(q, k, cs, sn, start, R, kc0, ks0)
    g = _e4m3_grid()
    for codes, y in [(r["q_fp8"].reshape(-1, D), r["q_y"].reshape(-1, D)),
                     (np.concatenate([r["k_cache"][b, start[b]:start[b] + T] for b in range(B)]),
                      r["k_y"].reshape(-1, D))]:
        dec = _fp8_values(codes)
        idx = np.clip(np.searchsorted(g, np.abs(y)), 1, len(g) - 1)
        step = g[idx] - g[idx - 1]
        assert np.all(np.abs(dec - y) <= step / 2 + 1e-12)
        am = np.argmax(np.abs(y), axis=1)
        assert np.all(np.abs(dec[np.arange(len(am)), am]) == 448.0)
    for b in range(B):
        keep = np.ones(Lmax, bool)
        keep[start[b]:start[b] + T] = False
        assert np.array_equal(r["k_cache"][b, keep], kc0[b, keep])
        assert np.array_equal(r["k_scale"][b, keep], ks0[b, keep])
        np.testing.assert_allclose(r["k_scale"][b, start[b]:start[b] + T], r["k_scale64"][b], rtol=1e-7)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
