"""The layer step at the full benchmark shapes (needs an MI355X), checked against the CPU
oracle on sampled rows: the oracle recomputes, for each sampled query row, its complete
index-score row, its top-k and its attention output over the GPU's own selection.

Shapes: V3.2-size decode (B=32, L=8192), long-context decode (B=8, L=131072), ragged
decode (B=64, lengths in [1024, 65536], Student-t(3) indexer inputs), chunked prefill
(T=8192, MHA form, 128 heads, qk 192 / v 128); the V3.2 and ragged decodes also with the
latent cache in its 656-byte FP8 row form.  Cache padding past each length is
poisoned, so any read beyond it fails the comparison."""
import sys

import numpy as np
import pytest
import torch

import dsa_synth as S
from parity import check_attention, check_scores, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import deepseek_dsa_indexer_amd as D
    D.load()
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("name,latent_form", [("decode_v32", "bf16"), ("decode_long", "bf16"),
                                               ("decode_ragged", "bf16"), ("decode_v32", "fp8"),
                                               ("decode_long", "fp8"), ("decode_ragged", "fp8")],
                         ids=["decode_v32", "decode_long", "decode_ragged", "decode_v32-fp8",
                              "decode_long-fp8", "decode_ragged-fp8"])
def test_fullsize_decode(dsa, orc, name, latent_form):
    cfg = S.CONFIGS[name]
    _say(f"[fullsize] {name} ({latent_form} latent): generating inputs")
    c = S.make_case(cfg, latent_form=latent_form)
    d = S.to_device(c, "cuda")
    step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                         cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                         Dv=cfg.Dv, want_idx=True, want_scores=True)
    _say(f"[fullsize] {name}: layer step on the GPU")
    out, lse = step()
    torch.cuda.synchronize()
    lens = c["lens"]
    sample = sorted({0, cfg.B // 2, cfg.B - 1, int(np.argmin(lens)), int(np.argmax(lens))})
    gidx_all = step.idx.cpu().numpy()
    for b in sample:
        _say(f"[fullsize] {name}: oracle on sequence {b} (len {int(lens[b])})")
        sl = slice(b, b + 1)
        rsc = orc.index_scores(c["q_i"][sl], c["q_scale"][sl], c["w"][sl], c["k_i"][sl],
                               c["k_scale"][sl], lens[sl], cfg.sm_scale_i)
        check_scores(step.scores[b:b + 1].cpu().numpy(), rsc, lens[sl], cfg.T)
        ridx = orc.topk(rsc, lens[sl], cfg.k)
        gidx = gidx_all[sl]
        check_topk(gidx, rsc, ridx, lens[sl], cfg.T, cfg.k)
        ro, rl = orc.sparse_mla_decode(c["q"][sl], c["latent"][sl], gidx, lens[sl], cfg.Dv,
                                       cfg.sm_scale)
        check_attention(_np(out[sl]), lse[sl].cpu().numpy(), ro, rl, cfg.attn_dtype)
    _say(f"[fullsize] {name} ({latent_form} latent): done")


def test_fullsize_prefill(dsa, orc):
    cfg = S.CONFIGS["prefill_chunk"]
    _say("[fullsize] prefill_chunk: generating inputs")
    c = S.make_case(cfg)
    d = S.to_device(c, "cuda")
    step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                         cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, k=d["k"], v=d["v"],
                         want_idx=True, want_scores=True)
    _say("[fullsize] prefill_chunk: layer step on the GPU")
    out, lse = step()
    torch.cuda.synchronize()
    T = cfg.T
    rows = [0, 1, 63, 64, 2046, 2047, 2048, 5000, T - 1]
    lens_full = np.array([T], np.int32)
    gidx_all = step.idx.cpu().numpy()
    out_np, lse_np = _np(out), lse.cpu().numpy()
    for t in rows:
        _say(f"[fullsize] prefill_chunk: oracle on row {t}")
        # row t alone: a one-row call whose length is t + 1 sees exactly keys 0..t
        rsc = orc.index_scores(c["q_i"][:, t:t + 1], c["q_scale"][:, t:t + 1], c["w"][:, t:t + 1],
                               c["k_i"], c["k_scale"], np.array([t + 1], np.int32), cfg.sm_scale_i)
        check_scores(step.scores[0, t:t + 1].cpu().numpy(), rsc[0], lens_full, T, rows=[(0, t)])
        ridx = orc.topk(rsc, np.array([t + 1], np.int32), cfg.k)
        check_topk(gidx_all[0, t:t + 1], rsc[0], ridx[0], lens_full, T, cfg.k, rows=[(0, t)])
    ro, rl = orc.sparse_mha_prefill_rows(c["q"], c["k"], c["v"], gidx_all, cfg.sm_scale,
                                         [(0, t) for t in rows])
    check_attention(out_np[0, rows], lse_np[0, rows], ro, rl, "bf16")


def test_fullsize_prefill_latent(dsa, orc):
    """The latent form of the chunked prefill (T=8192 rows of one sequence, top-2048, 128
    heads over 512 + 64 latent rows): the step runs whole on the GPU; sampled rows are
    checked against the oracle, each as a one-row query whose length ends at its own
    position, so the oracle sees exactly that row's causal keys."""
    cfg = S.CONFIGS["prefill_chunk_latent"]
    _say("[fullsize] prefill_chunk_latent: generating inputs")
    c = S.make_case(cfg)
    d = S.to_device(c, "cuda")
    step = dsa.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                         cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                         Dv=cfg.Dv, want_idx=True, want_scores=True)
    _say("[fullsize] prefill_chunk_latent: layer step on the GPU")
    out, lse = step()
    torch.cuda.synchronize()
    T = cfg.T
    assert int(c["lens"][0]) == T
    rows = [0, 1, 2046, 2047, 2048, 4097, 6000, T - 1]
    lens_full = np.array([T], np.int32)
    gidx_all = step.idx.cpu().numpy()
    out_np, lse_np = _np(out), lse.cpu().numpy()
    for t in rows:
        _say(f"[fullsize] prefill_chunk_latent: oracle on row {t}")
        one = np.array([t + 1], np.int32)
        rsc = orc.index_scores(c["q_i"][:, t:t + 1], c["q_scale"][:, t:t + 1], c["w"][:, t:t + 1],
                               c["k_i"], c["k_scale"], one, cfg.sm_scale_i)
        check_scores(step.scores[0, t:t + 1].cpu().numpy(), rsc[0], lens_full, T, rows=[(0, t)])
        ridx = orc.topk(rsc, one, cfg.k)
        gidx = gidx_all[:, t:t + 1]
        check_topk(gidx[0], rsc[0], ridx[0], lens_full, T, cfg.k, rows=[(0, t)])
        ro, rl = orc.sparse_mla_decode(c["q"][:, t:t + 1], c["latent"], gidx, one, cfg.Dv,
                                       cfg.sm_scale)
        check_attention(out_np[:, t:t + 1], lse_np[:, t:t + 1], ro, rl, cfg.attn_dtype)
    _say("[fullsize] prefill_chunk_latent: done")


@pytest.mark.parametrize("name", ["decode_v32", "prefill_chunk"])
def test_fullsize_indexer_prep(dsa, orc, name):
    """The indexer preparation of every new token of the workload (32 decode tokens, or
    the 8192 tokens of the prefill chunk), checked against the oracle on sampled tokens."""
    from parity import check_prep
    cfg = S.CONFIGS[name]
    _say(f"[fullsize] prep {name}: generating inputs")
    c = S.make_prep_case(cfg)
    d = S.to_device(c, "cuda")
    R = cfg.rope_i
    q_fp8, q_scale = dsa.indexer_prep(d["q"], d["k"], d["cos"], d["sin"], d["start"], R,
                                      d["k_cache"], d["k_scale"])
    torch.cuda.synchronize()
    q_fp8, q_scale = q_fp8.cpu().numpy(), q_scale.cpu().numpy()
    kc, ks = d["k_cache"].cpu().numpy(), d["k_scale"].cpu().numpy()
    if cfg.T == 1:
        samples = [(b, 0) for b in range(cfg.B)]
    else:
        samples = [(0, t) for t in (0, 1, 63, 4095, cfg.T - 2, cfg.T - 1)]
    for b, t in samples:
        pos = int(c["start"][b]) + t
        r = orc.indexer_prep(c["q"][b:b + 1, t:t + 1], c["k"][b:b + 1, t:t + 1], c["cos"], c["sin"],
                             np.array([pos], np.int32), R, c["k_cache"][b:b + 1], c["k_scale"][b:b + 1])
        check_prep(q_fp8[b:b + 1, t:t + 1], q_scale[b:b + 1, t:t + 1], r["q_y"], r["q_scale"])
        check_prep(kc[b:b + 1, pos:pos + 1], ks[b:b + 1, pos:pos + 1], r["k_y"], r["k_scale64"])
    # rows of the cache outside the new tokens are untouched
    for b in range(cfg.B):
        keep = np.ones(cfg.Lmax, bool)
        keep[int(c["start"][b]):int(c["start"][b]) + cfg.T] = False
        assert np.array_equal(kc[b, keep], c["k_cache"][b, keep])
    _say(f"[fullsize] prep {name}: done")
