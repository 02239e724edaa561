"""GPU library vs CPU oracle, element by element, on seeded inputs (needs an MI355X).

Sizes are chosen so that the oracle finishes in seconds while the kernels still run
several tiles, ragged tails, padded heads/columns, causal rows and short rows."""
import dataclasses
import sys
import zlib

import numpy as np
import pytest
import torch

import dsa_synth as S
from parity import check_attention, check_prep, check_scores, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import deepseek_dsa_indexer_amd as D
    D.load()
    return D


def _small(base: str, **kw) -> S.Config:
    return dataclasses.replace(S.CONFIGS[base], **kw)


def _dev(case):
    return S.to_device(case, "cuda")


def _np_out(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------- indexer preparation

PREP_CASES = [
    ("decode_small", _small("decode_v32", name="pds", B=3, Lmax=300, seed=301)),
    ("ragged_t3_student", _small("decode_ragged", name="prs", B=4, T=3, Lmax=2000,
                                 lens="ragged:3:2000", seed=302)),
    ("tiny_f32_d32", _small("tiny")),
    ("d64_rope16", _small("decode_v32", name="pd64", B=2, T=2, Lmax=90, H_I=16, D_I=64,
                          rope_i=16, seed=303)),
    ("no_rope", _small("decode_v32", name="pnr", B=2, Lmax=64, rope_i=0, seed=304)),
]


@pytest.mark.parametrize("name,cfg", PREP_CASES, ids=[c[0] for c in PREP_CASES])
def test_indexer_prep(dsa, orc, name, cfg):
    _say(f"[indexer_prep] {name}")
    c = S.make_prep_case(cfg)
    d = _dev(c)
    R = cfg.rope_i
    q_fp8, q_scale = dsa.indexer_prep(d["q"], d["k"], d["cos"], d["sin"], d["start"], R,
                                      d["k_cache"], d["k_scale"])
    torch.cuda.synchronize()
    r = orc.indexer_prep(c["q"], c["k"], c["cos"], c["sin"], c["start"], R, c["k_cache"],
                         c["k_scale"])
    swaps = check_prep(q_fp8.cpu().numpy(), q_scale.cpu().numpy(), r["q_y"], r["q_scale"])
    kc, ks = d["k_cache"].cpu().numpy(), d["k_scale"].cpu().numpy()
    st, T = c["start"], cfg.T
    rows = np.stack([kc[b, st[b]:st[b] + T] for b in range(len(st))])
    scales = np.stack([ks[b, st[b]:st[b] + T] for b in range(len(st))])
    swaps += check_prep(rows, scales, r["k_y"], r["k_scale64"])
    for b in range(len(st)):
        keep = np.ones(cfg.Lmax, bool)
        keep[st[b]:st[b] + T] = False
        assert np.array_equal(kc[b, keep], c["k_cache"][b, keep]), "cache rows outside the new tokens changed"
        assert np.array_equal(ks[b, keep], c["k_scale"][b, keep])
    _say(f"[indexer_prep] {name}: {swaps} codes took the other neighbour at a midpoint")


# ----------------------------------------------------------------------------- index scores

INDEX_CASES = [
    ("tiny", _small("tiny")),
    ("decode_ragged_small", _small("decode_ragged", name="drs", B=3, Lmax=1100,
                                   lens="ragged:37:1100", seed=105)),
    ("decode_normal_small", _small("decode_v32", name="dns", B=2, Lmax=777, seed=102)),
    # more than 64 sequences: the block-wide block numbering (64 or fewer: one wave's)
    ("decode_many_seqs", _small("decode_ragged", name="dms", B=80, Lmax=600, lens="ragged:30:600",
                                seed=107)),
    ("prefill_small", _small("prefill_chunk", name="ps", T=70, Lmax=300, lens="ragged:70:300",
                             B=2, H_I=48, D_I=64, seed=104)),
    # long decode rows: the LDS-streamed decode kernel (four or more chunks per wave),
    # with padded heads and columns and ragged lengths
    ("decode_long_rows", _small("decode_ragged", name="dlr", B=2, Lmax=270000,
                                lens="ragged:100000:270000", H_I=48, D_I=64, H=4, Dv=16, Dr=16,
                                seed=106)),
]


@pytest.mark.parametrize("name,cfg", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_index_scores(dsa, orc, name, cfg):
    _say(f"[index_scores] {name}")
    c = S.make_case(cfg)
    d = _dev(c)
    got = dsa.index_scores(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                           cfg.sm_scale_i)
    torch.cuda.synchronize()
    ref = orc.index_scores(c["q_i"], c["q_scale"], c["w"], c["k_i"], c["k_scale"], c["lens"],
                           cfg.sm_scale_i)
    check_scores(got.cpu().numpy(), ref, c["lens"], cfg.T)


# ----------------------------------------------------------------------------- top-k

def _scores_case(kind, B, T, Lmax, lens, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        sc = rng.standard_normal((B, T, Lmax)).astype(np.float32)
    elif kind == "ties":
        sc = rng.integers(-20, 21, size=(B, T, Lmax)).astype(np.float32) * 0.25
    elif kind == "heavy":
        x = rng.standard_t(3, size=(B, T, Lmax)).astype(np.float32)
        # keep 8 mantissa bits so that exact ties appear in the tail
        sc = (x.view(np.uint32) & np.uint32(0xFFFF8000)).view(np.float32)
    else:   # signed zeros and a constant row
        sc = np.where(rng.random((B, T, Lmax)) < 0.5, np.float32(0.0), np.float32(-0.0))
    return sc, np.asarray(lens, np.int32)


TOPK_CASES = [
    ("normal_decode", "normal", 4, 1, 8192, [8192, 3000, 2049, 100], 2048),
    ("ties_decode", "ties", 3, 1, 5000, [5000, 4097, 2500], 2048),
    ("heavy_long", "heavy", 2, 1, 40000, [40000, 17001], 2048),
    # rows beyond 16384 positions: chunk-local candidates, then a merge
    ("ties_long", "ties", 2, 1, 70000, [70000, 16500], 2048),
    ("zeros_long", "zeros", 1, 1, 30000, [30000], 2048),
    ("causal_long_odd_k", "normal", 1, 3, 20000, [20000], 3001),
    ("big_k_long", "heavy", 2, 1, 20000, [20000, 9000], 8000),
    # nine rows of unequal length (chunk boundaries, rows needing no selection)
    ("ragged_long_rows", "heavy", 9, 1, 50000,
     [50000, 1000, 16384, 16385, 32768, 2049, 2048, 40001, 24000], 2048),
    # 70 sequences of up to 17000 positions: two-stage, chunks numbered block-wide
    ("many_long_rows", "heavy", 70, 1, 17000, [17000 - 97 * i for i in range(70)], 2048),
    ("zeros", "zeros", 2, 1, 3000, [3000, 2100], 2048),
    ("causal_rows", "normal", 2, 37, 1001, [1001, 37], 64),
    ("k1", "ties", 2, 3, 500, [500, 300], 1),
    ("k_gt_n", "normal", 2, 2, 64, [64, 10], 100),
]


@pytest.mark.parametrize("name,kind,B,T,Lmax,lens,k", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_exact(dsa, orc, name, kind, B, T, Lmax, lens, k):
    _say(f"[topk] {name}")
    sc, lens = _scores_case(kind, B, T, Lmax, lens, seed=zlib.crc32(name.encode()) % 1000)
    got = dsa.topk(torch.from_numpy(sc).cuda(), torch.from_numpy(lens).cuda(), k)
    torch.cuda.synchronize()
    ref = orc.topk(sc, lens, k)
    np.testing.assert_array_equal(got.cpu().numpy(), ref)


def test_topk_deterministic(dsa):
    sc, lens = _scores_case("ties", 4, 1, 9000, [9000] * 4, seed=3)
    s, l = torch.from_numpy(sc).cuda(), torch.from_numpy(lens).cuda()
    a = dsa.topk(s, l, 2048)
    b = dsa.topk(s, l, 2048)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------- sparse attention

def _random_idx(rng, B, T, k, lens, invisible=False):
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = int(lens[b]) - T + t + 1
            m = min(k, n)
            idx[b, t, :m] = np.sort(rng.choice(n, size=m, replace=False))
            if invisible and m < k and n < int(lens[b]):
                idx[b, t, m] = rng.integers(n, int(lens[b]))      # must be ignored
    return idx


MLA_CASES = [
    # name, B, T, Lmax, lens, k, H
    ("decode_k2048", 2, 1, 3000, [3000, 1500], 2048, 128),
    ("decode_ragged_k", 3, 1, 700, [700, 650, 90], 100, 128),
    ("two_rows_causal", 1, 2, 2100, [2100], 2048, 128),
    ("heads64", 2, 1, 900, [900, 513], 512, 64),
    ("many_rows_nosplit", 260, 1, 160, [160] * 260, 64, 128),
]


@pytest.mark.parametrize("name,B,T,Lmax,lens,k,H", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_sparse_mla_decode_mfma(dsa, orc, name, B, T, Lmax, lens, k, H):
    _say(f"[sparse_mla_decode bf16] {name}")
    rng = np.random.default_rng(zlib.crc32(name.encode()) % 10000)
    lens = np.asarray(lens, np.int32)
    q = S.to_bf16_bits(rng.standard_normal((B, T, H, 576), dtype=np.float32))
    lat = S.to_bf16_bits(rng.standard_normal((B, Lmax, 576), dtype=np.float32))
    idx = _random_idx(rng, B, T, k, lens, invisible=True)
    sm = 192 ** -0.5
    tq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    tl = torch.from_numpy(lat.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_decode(tq, tl, torch.from_numpy(idx).cuda(),
                                     torch.from_numpy(lens).cuda(), 512, sm)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mla_decode(q, lat, idx, lens, 512, sm)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


# (B, k): two rows run the 32x32x16 kernels (sparse_mla_decode32*.hip); forty rows are more
# workgroups than one wave of 256 and run mla_decode_mfma_kernel (sparse_attn.hip)
# (B, k, slot of the late boosted key): the slot lies in the second or a later tile of its
# split under either plan (4 tiles of 32 slots per split for B = 2; 3 per split for B = 40)
SPREAD_SHAPES = [(2, 2048, 200), (40, 512, 250)]


@pytest.mark.parametrize("B,k,late", SPREAD_SHAPES, ids=[f"B{b}" for b, _, _ in SPREAD_SHAPES])
def test_sparse_mla_decode_logit_spread(dsa, orc, B, k, late):
    """Logits far above the rest of a split: in row 0 one key selected late in a split
    scores about 100 (log2 units) above everything before it for head 5 (the split is
    then recomputed from its true maximum); in row 1 such a key comes first, so every
    later probability of head 9 underflows relative to it.  The boost sits in the rope
    columns, so the outputs keep the magnitude of ordinary value rows."""
    _say(f"[sparse_mla_decode bf16] logit spread, B={B} k={k}")
    rng = np.random.default_rng(11)
    T, H, Lmax = 1, 128, 3000
    lens = np.full(B, 3000, np.int32)
    qf = rng.standard_normal((B, T, H, 576), dtype=np.float32)
    latf = rng.standard_normal((B, Lmax, 576), dtype=np.float32)
    idx = _random_idx(rng, B, T, k, lens, invisible=False)
    qf = (S.to_bf16_bits(qf).astype(np.uint32) << 16).view(np.float32)   # bf16 values
    latf[0, idx[0, 0, late], 512:] = 16.0 * qf[0, 0, 5, 512:]     # exact in bf16
    latf[1, idx[1, 0, 3], 512:] = 16.0 * qf[1, 0, 9, 512:]
    q = S.to_bf16_bits(qf)
    lat = S.to_bf16_bits(latf)
    sm = 192 ** -0.5
    tq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    tl = torch.from_numpy(lat.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_decode(tq, tl, torch.from_numpy(idx).cuda(),
                                     torch.from_numpy(lens).cuda(), 512, sm)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mla_decode(q, lat, idx, lens, 512, sm)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


@pytest.mark.parametrize("B,k,late", SPREAD_SHAPES, ids=[f"B{b}" for b, _, _ in SPREAD_SHAPES])
def test_sparse_mla_decode_fp8_logit_spread(dsa, orc, B, k, late):
    """FP8 latent rows with logits far above the rest of a split: one selected row's bf16
    rope columns are 16x the query's rope part of one head, so its logit lies about 100
    log2 units above the others -- late in a split in row 0 (the split is recomputed from
    its true maximum, with FP8 gathers and block-scaled numerators), first in row 1."""
    _say(f"[sparse_mla_decode fp8 latent] logit spread, B={B} k={k}")
    rng = np.random.default_rng(12)
    T, H, Lmax = 1, 128, 3000
    lens = np.full(B, 3000, np.int32)
    qf = rng.standard_normal((B, T, H, 576), dtype=np.float32)
    qf = (S.to_bf16_bits(qf).astype(np.uint32) << 16).view(np.float32)   # bf16 values
    x = rng.standard_normal((B, Lmax, 576), dtype=np.float32)
    f = np.exp2(rng.uniform(-5, 0, size=(B, Lmax, 4))).astype(np.float32)
    x[..., :512] *= np.repeat(f, 128, axis=-1)
    idx = _random_idx(rng, B, T, k, lens, invisible=False)
    x[0, idx[0, 0, late], 512:] = 16.0 * qf[0, 0, 5, 512:]     # exact in bf16
    x[1, idx[1, 0, 3], 512:] = 16.0 * qf[1, 0, 9, 512:]
    q = S.to_bf16_bits(qf)
    lat = S.pack_latent_fp8(x)
    sm = 192 ** -0.5
    tq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_decode(tq, torch.from_numpy(lat).cuda(), torch.from_numpy(idx).cuda(),
                                     torch.from_numpy(lens).cuda(), 512, sm)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mla_decode(q, lat, idx, lens, 512, sm)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


def test_sparse_mla_prefill_logit_spread(dsa, orc):
    """MHA prefill with a selected key far above the rest of its row: for row 150 of head
    1, key 130 (third key block) has rope columns 16x the query's, about 100 log2 units
    above the logits of the first key block (the workgroup is recomputed from the true
    maximum); for row 40 of head 0 such a key sits in the first block (key 5), so the
    later numerators of that row underflow relative to it."""
    _say("[sparse_mla_prefill bf16] logit spread")
    rng = np.random.default_rng(13)
    B, T, H, Dqk, Dv, k = 1, 200, 2, 192, 128, 48
    qf = rng.standard_normal((B, T, H, Dqk), dtype=np.float32)
    qf = (S.to_bf16_bits(qf).astype(np.uint32) << 16).view(np.float32)
    kf = rng.standard_normal((B, T, H, Dqk), dtype=np.float32)
    v = S.to_bf16_bits(rng.standard_normal((B, T, H, Dv), dtype=np.float32))
    idx = np.full((B, T, k), -1, np.int32)
    for t in range(T):
        m = min(k, t + 1)
        idx[0, t, :m] = rng.choice(t + 1, size=m, replace=False)
    for t, h, s_key in ((150, 1, 130), (40, 0, 5)):
        row = idx[0, t]
        if s_key not in row:
            row[0] = s_key
        kf[0, s_key, h, 128:] = 16.0 * qf[0, t, h, 128:]
    q = S.to_bf16_bits(qf)
    kk = S.to_bf16_bits(kf)
    tt = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_prefill(tt(q), tt(kk), tt(v), torch.from_numpy(idx).cuda(), Dqk ** -0.5)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mha_prefill(q, kk, v, idx, Dqk ** -0.5)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


def test_sparse_mla_decode_generic_f32(dsa, orc):
    _say("[sparse_mla_decode f32 generic]")
    rng = np.random.default_rng(7)
    B, T, H, Dv, Dr, Lmax, k = 2, 5, 4, 64, 16, 40, 8
    lens = np.array([40, 9], np.int32)
    q = rng.standard_normal((B, T, H, Dv + Dr)).astype(np.float32)
    lat = rng.standard_normal((B, Lmax, Dv + Dr)).astype(np.float32)
    idx = _random_idx(rng, B, T, k, lens, invisible=True)
    out, lse = dsa.sparse_mla_decode(torch.from_numpy(q).cuda(), torch.from_numpy(lat).cuda(),
                                     torch.from_numpy(idx).cuda(), torch.from_numpy(lens).cuda(),
                                     Dv, 0.11)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mla_decode(q, lat, idx, lens, Dv, 0.11)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32")


FP8_MLA_CASES = [
    # name, B, T, Lmax, lens, k, H   (H 64 / 128: matrix cores; other H: vector ALUs)
    ("decode_k2048", 2, 1, 3000, [3000, 1500], 2048, 128),
    ("decode_ragged_k", 3, 1, 700, [700, 650, 90], 100, 128),
    ("two_rows_causal", 1, 2, 2100, [2100], 2048, 128),
    ("heads64", 2, 1, 900, [900, 513], 512, 64),
    ("many_rows_nosplit", 260, 1, 160, [160] * 260, 64, 128),
    ("long_k_16_splits", 1, 1, 17000, [17000], 16384, 128),
    ("heads16_generic", 2, 3, 300, [300, 77], 40, 16),
]


def _fp8_rows(rng, shape):
    """656-byte FP8 latent rows whose 128-column blocks differ in magnitude by up to 32x
    (so that each block's scale matters), values at most about 3 in magnitude."""
    x = rng.standard_normal(shape + (576,), dtype=np.float32)
    f = np.exp2(rng.uniform(-5, 0, size=shape + (4,))).astype(np.float32)
    x[..., :512] *= np.repeat(f, 128, axis=-1)
    return S.pack_latent_fp8(x)


@pytest.mark.parametrize("name,B,T,Lmax,lens,k,H", FP8_MLA_CASES, ids=[c[0] for c in FP8_MLA_CASES])
def test_sparse_mla_decode_fp8_latent(dsa, orc, name, B, T, Lmax, lens, k, H):
    _say(f"[sparse_mla_decode fp8 latent] {name}")
    rng = np.random.default_rng(zlib.crc32(("fp8" + name).encode()) % 10000)
    lens = np.asarray(lens, np.int32)
    q = S.to_bf16_bits(rng.standard_normal((B, T, H, 576), dtype=np.float32))
    lat = _fp8_rows(rng, (B, Lmax))
    idx = _random_idx(rng, B, T, k, lens, invisible=True)
    sm = 192 ** -0.5
    tq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_decode(tq, torch.from_numpy(lat).cuda(), torch.from_numpy(idx).cuda(),
                                     torch.from_numpy(lens).cuda(), 512, sm)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mla_decode(q, lat, idx, lens, 512, sm)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sparse_mla_prefill(dsa, orc, dt):
    _say(f"[sparse_mla_prefill {dt}]")
    rng = np.random.default_rng(9)
    B, T, H, Dqk, Dv, k = 2, 40, 3, 192, 128, 16
    mk = (lambda a: S.to_bf16_bits(a)) if dt == "bf16" else (lambda a: a)
    q = mk(rng.standard_normal((B, T, H, Dqk), dtype=np.float32))
    kk = mk(rng.standard_normal((B, T, H, Dqk), dtype=np.float32))
    v = mk(rng.standard_normal((B, T, H, Dv), dtype=np.float32))
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            m = min(k, T)
            idx[b, t, :m] = rng.choice(T, size=m, replace=False)   # includes s > t: ignored
    def tt(a):
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    out, lse = dsa.sparse_mla_prefill(tt(q), tt(kk), tt(v), torch.from_numpy(idx).cuda(), 0.07)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mha_prefill(q, kk, v, idx, 0.07)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, dt)


# ----------------------------------------------------------------------------- layer step

LAYER_CASES = [
    ("tiny", _small("tiny")),
    ("decode_small", _small("decode_v32", name="ds", B=3, Lmax=4100, seed=202)),
    ("ragged_small_t3", _small("decode_ragged", name="rs", B=5, T=3, Lmax=6000,
                               lens="ragged:1024:6000", seed=205)),
    # two query rows per sequence beyond 16384 positions: two-stage top-k with several
    # rows per sequence, indexer blocks of two rows
    ("long_t2", _small("decode_long", name="lt2", B=2, T=2, Lmax=40000,
                       lens="ragged:20000:40000", seed=206)),
    # a prefill chunk in the absorbed (latent) form: 256 query rows over their own chunk
    ("prefill_latent_t256", _small("prefill_chunk_latent", name="pl", T=256, Lmax=256, k=64,
                                   seed=209)),
    # rows of 8192 positions with k = 2000: the last tile of the selection is partly unused
    ("k2000_l8192", _small("decode_v32", name="fk", B=2, Lmax=8192, k=2000, lens="ragged:7000:8192",
                           seed=210)),
    # four query rows per sequence on the 32x32x16 attention kernel (eight rows: 16 splits
    # each): causal rows, some with fewer visible positions than k
    ("t4_rows", _small("decode_v32", name="tf", B=2, T=4, Lmax=5000, lens="ragged:1000:5000",
                       seed=216)),
]


FP8_LAYER_CASES = [
    ("decode_small", _small("decode_v32", name="ds8", B=3, Lmax=4100, seed=212)),
    ("ragged_small_t3", _small("decode_ragged", name="rs8", B=5, T=3, Lmax=6000,
                               lens="ragged:1024:6000", seed=215)),
    # four causal query rows per sequence on the 32x32x16 FP8-row kernel (eight rows, 16
    # splits), some rows with fewer visible positions than k
    ("t4_rows", _small("decode_v32", name="tf8", B=2, T=4, Lmax=5000, lens="ragged:1000:5000",
                       seed=218)),
]


def _layer_step_latent(dsa, cfg, c):
    d = _dev(c)
    step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                         cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                         Dv=cfg.Dv, want_idx=True, want_scores=True)
    out, lse = step()
    torch.cuda.synchronize()
    return step, out, lse


@pytest.mark.parametrize("name,cfg", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_step_latent(dsa, orc, name, cfg):
    _say(f"[layer_step latent] {name}")
    c = S.make_case(cfg)
    step, out, lse = _layer_step_latent(dsa, cfg, c)
    ro, rl, ridx, rsc = orc.layer_step_latent(c["q_i"], c["q_scale"], c["w"], c["k_i"],
                                              c["k_scale"], c["lens"], cfg.sm_scale_i, cfg.k,
                                              c["q"], c["latent"], cfg.Dv, cfg.sm_scale,
                                              want_scores=True)
    check_scores(step.scores.cpu().numpy(), rsc, c["lens"], cfg.T)
    gidx = step.idx.cpu().numpy()
    check_topk(gidx, rsc, ridx, c["lens"], cfg.T, cfg.k)
    # attention on the GPU's own selection
    ro2, rl2 = orc.sparse_mla_decode(c["q"], c["latent"], gidx, c["lens"], cfg.Dv, cfg.sm_scale)
    check_attention(_np_out(out), lse.cpu().numpy(), ro2, rl2, cfg.attn_dtype)


@pytest.mark.parametrize("name,cfg", FP8_LAYER_CASES, ids=[c[0] for c in FP8_LAYER_CASES])
def test_layer_step_fp8_latent(dsa, orc, name, cfg):
    _say(f"[layer_step fp8 latent] {name}")
    c = S.make_case(cfg, latent_form="fp8")
    step, out, lse = _layer_step_latent(dsa, cfg, c)
    ro, rl, ridx, rsc = orc.layer_step_latent(c["q_i"], c["q_scale"], c["w"], c["k_i"],
                                              c["k_scale"], c["lens"], cfg.sm_scale_i, cfg.k,
                                              c["q"], c["latent"], cfg.Dv, cfg.sm_scale,
                                              want_scores=True)
    check_scores(step.scores.cpu().numpy(), rsc, c["lens"], cfg.T)
    gidx = step.idx.cpu().numpy()
    check_topk(gidx, rsc, ridx, c["lens"], cfg.T, cfg.k)
    ro2, rl2 = orc.sparse_mla_decode(c["q"], c["latent"], gidx, c["lens"], cfg.Dv, cfg.sm_scale)
    check_attention(_np_out(out), lse.cpu().numpy(), ro2, rl2, "bf16")


COMPRESSED_CASES = [
    # name, config (lens in positions, Lmax in entries), compress rate
    ("prefill_t64_m4", _small("decode_v32", name="cp1", B=1, T=64, Lmax=64, k=8, seed=501), 4),
    ("decode_ragged_m4", _small("decode_ragged", name="cp2", B=5, Lmax=750, lens="ragged:10:3000",
                                k=64, seed=502), 4),
    ("ragged_t3_m2", _small("decode_ragged", name="cp3", B=4, T=3, Lmax=3000,
                            lens="ragged:1024:6000", seed=503), 2),
    # more than 16384 visible entries: the two-stage top-k, two rows per sequence
    ("long_t2_m4", _small("decode_long", name="cp4", B=2, T=2, Lmax=20000,
                          lens="ragged:70000:80000", seed=504), 4),
    # FP8 latent rows: the 32x32x16 FP8 kernel (first) and the 16x16x32 one (second)
    ("prefill_t64_m4_fp8", _small("decode_v32", name="cp5", B=1, T=64, Lmax=64, k=8, seed=505), 4),
    ("ragged_t3_m2_fp8", _small("decode_ragged", name="cp6", B=4, T=3, Lmax=3000,
                                lens="ragged:1024:6000", seed=506), 2),
]


@pytest.mark.parametrize("name,cfg,m", COMPRESSED_CASES, ids=[c[0] for c in COMPRESSED_CASES])
def test_layer_step_compressed_entries(dsa, orc, name, cfg, m):
    """Caches of compressed entries (each standing for m positions): row (b,t) may select
    entry e iff e < (pos + 1) / m; rows with no entry get -1 slots, a zero output and
    lse = -inf."""
    _say(f"[layer_step compressed] {name} m={m}")
    c = S.make_case(cfg, compress=m, latent_form="fp8" if name.endswith("_fp8") else "bf16")
    d = _dev(c)
    step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                         cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                         Dv=cfg.Dv, want_idx=True, want_scores=True, compress_rate=m)
    out, lse = step()
    torch.cuda.synchronize()
    ro, rl, ridx, rsc = orc.layer_step_latent(c["q_i"], c["q_scale"], c["w"], c["k_i"],
                                              c["k_scale"], c["lens"], cfg.sm_scale_i, cfg.k,
                                              c["q"], c["latent"], cfg.Dv, cfg.sm_scale,
                                              want_scores=True, compress=m)
    check_scores(step.scores.cpu().numpy(), rsc, c["lens"], cfg.T, compress=m)
    gidx = step.idx.cpu().numpy()
    check_topk(gidx, rsc, ridx, c["lens"], cfg.T, cfg.k, compress=m)
    ro2, rl2 = orc.sparse_mla_decode(c["q"], c["latent"], gidx, c["lens"], cfg.Dv, cfg.sm_scale,
                                     compress=m)
    check_attention(_np_out(out), lse.cpu().numpy(), ro2, rl2, cfg.attn_dtype)
    if name.startswith("prefill"):
        # the first m - 1 positions have no entry yet: -1 slots, zero rows, lse -inf
        assert np.all(gidx[0, :m - 1] == -1)
        assert np.all(_np_out(out)[0, :m - 1] == 0) and np.all(np.isneginf(lse.cpu().numpy()[0, :m - 1]))


def test_layer_step_mha_small(dsa, orc):
    _say("[layer_step mha] small")
    cfg = _small("prefill_chunk", name="pm", T=96, Lmax=96, H=4, k=24, seed=404)
    c = S.make_case(cfg)
    d = _dev(c)
    step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                         cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, k=d["k"], v=d["v"],
                         want_idx=True, want_scores=True)
    out, lse = step()
    torch.cuda.synchronize()
    rsc = orc.index_scores(c["q_i"], c["q_scale"], c["w"], c["k_i"], c["k_scale"], c["lens"],
                           cfg.sm_scale_i)
    ridx = orc.topk(rsc, c["lens"], cfg.k)
    check_scores(step.scores.cpu().numpy(), rsc, c["lens"], cfg.T)
    gidx = step.idx.cpu().numpy()
    check_topk(gidx, rsc, ridx, c["lens"], cfg.T, cfg.k)
    ro, rl = orc.sparse_mha_prefill(c["q"], c["k"], c["v"], gidx, cfg.sm_scale)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


@pytest.mark.parametrize("B,Lmax,lo,seed", [(3, 20000, 1024, 207), (9, 36000, 700, 208),
                                            (3, 8000, 700, 209),
                                            # four or more key chunks per wave: the
                                            # LDS-streamed decode index kernel
                                            (8, 65536, 30000, 217),
                                            # more than 64 sequences: its block-wide
                                            # numbering over unequal visible ranges
                                            (80, 8192, 1024, 218)])
def test_layer_step_without_intermediates(dsa, orc, B, Lmax, lo, seed):
    """The production configuration (scores and indices kept in the workspace, invisible
    scores never written, key blocks and top-k chunks numbered over the visible range
    only, the top-k candidates of rows beyond 16384 positions sharing the scratch region
    with the attention partials) gives bit-identical results to the configuration that
    exposes the intermediates, which is checked against the oracle.  The shapes cover
    both index kernels (register-staged short streams; LDS-streamed rows of four or more
    chunks per wave, with one wave's or the block's numbering)."""
    _say(f"[layer_step] without intermediates, long ragged rows, B={B} Lmax={Lmax}")
    cfg = _small("decode_ragged", name="ni", B=B, Lmax=Lmax, lens=f"ragged:{lo}:{Lmax}", seed=seed)
    c = S.make_case(cfg)
    d = _dev(c)
    args = (d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"], cfg.sm_scale_i,
            cfg.k, d["q"], cfg.sm_scale)
    full = dsa.LayerStep(*args, latent=d["latent"], Dv=cfg.Dv, want_idx=True, want_scores=True)
    bare = dsa.LayerStep(*args, latent=d["latent"], Dv=cfg.Dv)
    o1, l1 = full()
    o2, l2 = bare()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rsc = orc.index_scores(c["q_i"], c["q_scale"], c["w"], c["k_i"], c["k_scale"], c["lens"],
                           cfg.sm_scale_i)
    ridx = orc.topk(rsc, c["lens"], cfg.k)
    gidx = full.idx.cpu().numpy()
    check_topk(gidx, rsc, ridx, c["lens"], cfg.T, cfg.k)
    ro, rl = orc.sparse_mla_decode(c["q"], c["latent"], gidx, c["lens"], cfg.Dv, cfg.sm_scale)
    check_attention(_np_out(o2), l2.cpu().numpy(), ro, rl, cfg.attn_dtype)


def test_layer_step_deterministic(dsa):
    cfg = _small("decode_v32", name="det", B=4, Lmax=5000, seed=303)
    c = S.make_case(cfg)
    s1, o1, l1 = _layer_step_latent(dsa, cfg, c)
    i1 = s1.idx.clone()
    o1 = o1.clone()
    o2, l2 = s1()
    torch.cuda.synchronize()
    assert torch.equal(i1, s1.idx)
    assert torch.equal(o1, o2)


GRAPH_CASES = [
    ("decode_split", _small("decode_v32", name="graph_decode", B=8, Lmax=9000, lens="ragged:3000:9000",
                            seed=311)),
    ("decode_long_rows", _small("decode_long", name="graph_long", B=2, Lmax=40000, seed=312)),
    ("prefill_mha", _small("prefill_chunk", name="graph_mha", T=300, Lmax=300, H=4, k=64, seed=313)),
]


@pytest.mark.parametrize("name,cfg", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_layer_step_graph_replay(dsa, name, cfg):
    """The whole step captured in one HIP graph, the way the benchmark can replay it: every
    replay, with eager work and synchronisations between replays, reproduces the eager
    step bit for bit (scores, selection, output, lse).  The outputs are overwritten
    before each replay, so a replay that skipped a kernel would be caught."""
    _say(f"[graph] {name}")
    c = S.make_case(cfg)
    d = _dev(c)
    if cfg.form == "latent":
        step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                             cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                             Dv=cfg.Dv, want_idx=True, want_scores=True)
    else:
        step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                             cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, k=d["k"], v=d["v"],
                             want_idx=True, want_scores=True)
    out, lse = step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.scores, step.idx, out, lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        step.scores.fill_(7.0)
        step.idx.fill_(-7)
        step.out.fill_(3.0)
        step.lse.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((step.scores, step.idx, step.out, step.lse), ref,
                                   ("scores", "idx", "out", "lse")):
            assert torch.equal(got, want), f"replay {r}: {what} differs from the eager step"


@pytest.mark.parametrize("sm", [0.0, -0.07])
def test_sparse_mla_prefill_nonpositive_scale(dsa, orc, sm):
    """The matrix-core prefill shape (bf16, qk 192 / v 128) with a zero or negative softmax
    scale: served by the vector-ALU kernel (the matrix-core one scales each block's maximum
    after taking it, which needs a positive scale), still against the oracle."""
    _say(f"[sparse_mla_prefill bf16] scale {sm}")
    rng = np.random.default_rng(41)
    B, T, H, Dqk, Dv, k = 1, 40, 2, 192, 128, 16
    q = S.to_bf16_bits(rng.standard_normal((B, T, H, Dqk), dtype=np.float32))
    kk = S.to_bf16_bits(rng.standard_normal((B, T, H, Dqk), dtype=np.float32))
    v = S.to_bf16_bits(rng.standard_normal((B, T, H, Dv), dtype=np.float32))
    idx = np.full((B, T, k), -1, np.int32)
    for t in range(T):
        m = min(k, t + 1)
        idx[0, t, :m] = rng.choice(t + 1, size=m, replace=False)
    tt = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_prefill(tt(q), tt(kk), tt(v), torch.from_numpy(idx).cuda(), sm)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mha_prefill(q, kk, v, idx, sm)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")


@pytest.mark.parametrize("T,H,k", [(200, 2, 48), (130, 3, 130), (64, 1, 1)])
def test_sparse_mla_prefill_blocks(dsa, orc, T, H, k):
    """Several 128-row query blocks and 64-key blocks, ragged tails, k >= T (dense causal)
    and k = 1."""
    _say(f"[sparse_mla_prefill bf16 blocks] T={T} H={H} k={k}")
    rng = np.random.default_rng(T * 7 + H)
    B, Dqk, Dv = 2, 192, 128
    q = S.to_bf16_bits(rng.standard_normal((B, T, H, Dqk), dtype=np.float32))
    kk = S.to_bf16_bits(rng.standard_normal((B, T, H, Dqk), dtype=np.float32))
    v = S.to_bf16_bits(rng.standard_normal((B, T, H, Dv), dtype=np.float32))
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            m = min(k, t + 1)
            idx[b, t, :m] = rng.choice(t + 1, size=m, replace=False)
    tt = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = dsa.sparse_mla_prefill(tt(q), tt(kk), tt(v), torch.from_numpy(idx).cuda(), Dqk ** -0.5)
    torch.cuda.synchronize()
    ro, rl = orc.sparse_mha_prefill(q, kk, v, idx, Dqk ** -0.5)
    check_attention(_np_out(out), lse.cpu().numpy(), ro, rl, "bf16")
