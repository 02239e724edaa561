"""Seeded synthetic inputs for one DSA layer step.

This module only draws random numbers and packs them into the storage formats the
layer step consumes (FP8 e4m3fn codes with one fp32 scale per 128-wide block, bf16 or
fp32 attention tensors, per-sequence lengths).  It holds none of the step's own
arithmetic: both the GPU library and the CPU reference receive its arrays unchanged.

Seeding: every tensor of sequence ``b`` comes from ``numpy.random.default_rng([seed,
tensor_id, b])`` (tensor ids: 0 indexer q, 1 indexer K, 2 head weights, 3 attention
q, 4 latent cache / MHA k, 5 MHA v, 7 / 8 the new tokens' indexer q / k before their
preparation); the lengths come from ``default_rng([seed, 6])``.
Generating a subset of sequences therefore reproduces exactly their slices of the
full batch.  Cache rows at or beyond ``len[b]`` are poisoned (K code 0x7E = 448,
K scale 1e4, latent 1e4) so that any read past the valid length shows up.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

FP8_MAX = 448.0
POISON_K_CODE = 0x7E
POISON_VALUE = 1.0e4


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    form: str            # "latent" (absorbed MQA attention) or "mha" (prefill MHA)
    B: int
    T: int
    Lmax: int
    lens: str            # "full" (= Lmax), or "ragged:lo:hi" (uniform integers, inclusive)
    H_I: int
    D_I: int
    k: int
    H: int
    Dv: int              # value width (latent: 512 / 64; MHA: 128)
    Dr: int              # latent: rope width appended to the key; MHA: unused (0)
    Dqk: int             # MHA only: query/key width (nope 128 + rope 64)
    attn_dtype: str      # "bf16" or "f32"
    dist: str            # "normal" or "student_t3" for the indexer q/k draws
    seed: int
    rope_i: int = 64     # rope columns at the front of each indexer q head / key row

    @property
    def sm_scale_i(self) -> float:
        return self.D_I ** -0.5

    @property
    def sm_scale(self) -> float:
        # MLA softmax scale qk_head_dim^-0.5; the tiny case uses its dotted width.
        if self.name == "tiny":
            return float(self.Dv + self.Dr) ** -0.5
        return 192.0 ** -0.5

    @property
    def Dq(self) -> int:
        return self.Dv + self.Dr if self.form == "latent" else self.Dqk


CONFIGS = {
    "tiny": Config("tiny", "latent", B=1, T=64, Lmax=64, lens="full", H_I=4, D_I=32, k=8,
                   H=4, Dv=64, Dr=16, Dqk=0, attn_dtype="f32", dist="normal", seed=1,
                   rope_i=8),
    "decode_v32": Config("decode_v32", "latent", B=32, T=1, Lmax=8192, lens="full", H_I=64,
                         D_I=128, k=2048, H=128, Dv=512, Dr=64, Dqk=0, attn_dtype="bf16",
                         dist="normal", seed=2),
    "decode_long": Config("decode_long", "latent", B=8, T=1, Lmax=131072, lens="full", H_I=64,
                          D_I=128, k=2048, H=128, Dv=512, Dr=64, Dqk=0, attn_dtype="bf16",
                          dist="normal", seed=3),
    "prefill_chunk": Config("prefill_chunk", "mha", B=1, T=8192, Lmax=8192, lens="full",
                            H_I=64, D_I=128, k=2048, H=128, Dv=128, Dr=0, Dqk=192,
                            attn_dtype="bf16", dist="normal", seed=4),
    "decode_ragged": Config("decode_ragged", "latent", B=64, T=1, Lmax=65536,
                            lens="ragged:1024:65536", H_I=64, D_I=128, k=2048, H=128, Dv=512,
                            Dr=64, Dqk=0, attn_dtype="bf16", dist="student_t3", seed=5),
    # the prefill chunk in the absorbed (latent, MQA) form instead of the MHA form: the
    # same indexer work, attention of 128 heads over the selected 576-wide latent rows
    "prefill_chunk_latent": Config("prefill_chunk_latent", "latent", B=1, T=8192, Lmax=8192,
                                   lens="full", H_I=64, D_I=128, k=2048, H=128, Dv=512, Dr=64,
                                   Dqk=0, attn_dtype="bf16", dist="normal", seed=6),
}


def lengths(cfg: Config) -> np.ndarray:
    if cfg.lens == "full":
        return np.full(cfg.B, cfg.Lmax, np.int32)
    _, lo, hi = cfg.lens.split(":")
    rng = np.random.default_rng([cfg.seed, 6])
    return rng.integers(int(lo), int(hi), size=cfg.B, endpoint=True).astype(np.int32)


def _rng(cfg: Config, tensor_id: int, b: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, tensor_id, b])


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "student_t3":
        return rng.standard_t(3, size=shape).astype(np.float32)
    return rng.standard_normal(shape, dtype=np.float32)


def quantize_e4m3fn(x: np.ndarray, block: int):
    """Blockwise FP8 storage of ``x`` [..., D]: one fp32 scale per ``block`` columns,
    scale = max(amax, 1e-12) / 448, code = e4m3fn(clip(x / scale, +-448)) rounded to
    nearest-even.  Returns (codes uint8 [..., D], scales float32 [..., D // block])."""
    D = x.shape[-1]
    assert D % block == 0
    xb = x.reshape(*x.shape[:-1], D // block, block).astype(np.float32)
    amax = np.abs(xb).max(axis=-1, keepdims=True)
    scale = (np.maximum(amax, np.float32(1e-12)) / np.float32(FP8_MAX)).astype(np.float32)
    y = np.clip(xb / scale, -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy().reshape(x.shape), scale[..., 0]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even) as raw uint16 words."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


FP8_LATENT_ROW_BYTES = 656
FP8_LATENT_DV, FP8_LATENT_DR, FP8_LATENT_BLOCK = 512, 64, 128


def pack_latent_fp8(x: np.ndarray) -> np.ndarray:
    """Store float32 latent rows ``x`` [..., 576] in the 656-byte FP8 form: the 512 latent
    columns as e4m3fn codes (quantize_e4m3fn, one scale per 128 columns), then the four
    fp32 scales, then the 64 rope columns as bf16."""
    assert x.shape[-1] == FP8_LATENT_DV + FP8_LATENT_DR
    lead = x.shape[:-1]
    codes, scales = quantize_e4m3fn(x[..., :FP8_LATENT_DV], FP8_LATENT_BLOCK)
    rope = to_bf16_bits(x[..., FP8_LATENT_DV:])
    out = np.empty(lead + (FP8_LATENT_ROW_BYTES,), np.uint8)
    out[..., :FP8_LATENT_DV] = codes
    out[..., FP8_LATENT_DV:FP8_LATENT_DV + 16] = np.ascontiguousarray(
        scales, dtype=np.float32).view(np.uint8).reshape(lead + (16,))
    out[..., FP8_LATENT_DV + 16:] = np.ascontiguousarray(rope).view(np.uint8).reshape(lead + (128,))
    return out


def make_case(cfg: Config, seqs=None, latent_form: str = "bf16", compress: int = 1) -> dict:
    """All inputs of one layer step as host numpy arrays.

    ``seqs`` restricts the batch to the listed sequence ids (same values as in the
    full batch).  Attention tensors are float32 or bf16 bits (uint16) per
    ``cfg.attn_dtype``.  Keys: q_i, q_scale, w, k_i, k_scale, lens, and either
    (q, latent) or (q, k, v).  ``latent_form="fp8"`` (bf16 latent configurations with
    576-wide rows only) stores the latent cache as 656-byte FP8 rows (pack_latent_fp8)
    drawn from the same float32 values; poisoned rows then hold code 448 with scale
    1e4 and rope 1e4.  ``compress = m > 1`` makes the caches compressed entries, each
    standing for m positions: sequence b (len[b] positions) has len[b] // m valid cache
    rows, and Lmax counts entries."""
    assert latent_form in ("bf16", "fp8")
    fp8_lat = latent_form == "fp8"
    if fp8_lat:
        assert (cfg.form == "latent" and cfg.attn_dtype == "bf16" and cfg.Dv == FP8_LATENT_DV
                and cfg.Dr == FP8_LATENT_DR), "FP8 latent rows need the 512 + 64 bf16 shape"
    all_lens = lengths(cfg)
    seqs = list(range(cfg.B)) if seqs is None else list(seqs)
    nb = len(seqs)
    lens = all_lens[seqs].copy()
    T, Lmax, H_I, D_I = cfg.T, cfg.Lmax, cfg.H_I, cfg.D_I
    block = min(128, D_I)
    nblk = D_I // block
    assert nblk == 1, "one scale per key/head row is what the library consumes"

    q_i = np.empty((nb, T, H_I, D_I), np.uint8)
    q_scale = np.empty((nb, T, H_I), np.float32)
    w = np.empty((nb, T, H_I), np.float32)
    k_i = np.full((nb, Lmax, D_I), POISON_K_CODE, np.uint8)
    k_scale = np.full((nb, Lmax), POISON_VALUE, np.float32)
    bf16 = cfg.attn_dtype == "bf16"
    adt = np.uint16 if bf16 else np.float32
    conv = to_bf16_bits if bf16 else (lambda a: a.astype(np.float32))
    if cfg.form == "latent":
        q = np.empty((nb, T, cfg.H, cfg.Dq), adt)
        if fp8_lat:
            latent = np.empty((nb, Lmax, FP8_LATENT_ROW_BYTES), np.uint8)
            latent[...] = _poison_fp8_row()
        else:
            latent = np.empty((nb, Lmax, cfg.Dq), adt)
            latent[...] = conv(np.full((1,), POISON_VALUE, np.float32))[0]
    else:
        q = np.empty((nb, T, cfg.H, cfg.Dqk), adt)
        kk = np.empty((nb, T, cfg.H, cfg.Dqk), adt)
        v = np.empty((nb, T, cfg.H, cfg.Dv), adt)

    for j, b in enumerate(seqs):
        L = int(lens[j]) // compress                # valid cache rows
        assert L <= Lmax, "the cache must hold every valid row"
        c, s = quantize_e4m3fn(_draw(_rng(cfg, 0, b), (T, H_I, D_I), cfg.dist), block)
        q_i[j], q_scale[j] = c, s[..., 0]
        c, s = quantize_e4m3fn(_draw(_rng(cfg, 1, b), (L, D_I), cfg.dist), block)
        k_i[j, :L], k_scale[j, :L] = c, s[..., 0]
        w[j] = _rng(cfg, 2, b).standard_normal((T, H_I), dtype=np.float32) / np.float32(math.sqrt(H_I))
        if cfg.form == "latent":
            q[j] = conv(_rng(cfg, 3, b).standard_normal((T, cfg.H, cfg.Dq), dtype=np.float32))
            x = _rng(cfg, 4, b).standard_normal((L, cfg.Dq), dtype=np.float32)
            latent[j, :L] = pack_latent_fp8(x) if fp8_lat else conv(x)
        else:
            q[j] = conv(_rng(cfg, 3, b).standard_normal((T, cfg.H, cfg.Dqk), dtype=np.float32))
            kk[j] = conv(_rng(cfg, 4, b).standard_normal((T, cfg.H, cfg.Dqk), dtype=np.float32))
            v[j] = conv(_rng(cfg, 5, b).standard_normal((T, cfg.H, cfg.Dv), dtype=np.float32))

    case = dict(q_i=q_i, q_scale=q_scale, w=w, k_i=k_i, k_scale=k_scale, lens=lens, seqs=seqs)
    if cfg.form == "latent":
        case.update(q=q, latent=latent)
    else:
        case.update(q=q, k=kk, v=v)
    return case


def _poison_fp8_row() -> np.ndarray:
    row = np.empty(FP8_LATENT_ROW_BYTES, np.uint8)
    row[:FP8_LATENT_DV] = POISON_K_CODE
    row[FP8_LATENT_DV:FP8_LATENT_DV + 16] = np.full(4, POISON_VALUE, np.float32).view(np.uint8)
    row[FP8_LATENT_DV + 16:] = np.repeat(
        to_bf16_bits(np.full((1,), POISON_VALUE, np.float32)), FP8_LATENT_DR).view(np.uint8)
    return row


def rope_tables(n_pos: int, rope_dim: int, base: float = 10000.0):
    """cos and sin [n_pos, rope_dim/2] float32 of the rotary angle pos * base^(-2j/rope_dim)
    (a standard frequency schedule; the preparation takes the tables as inputs)."""
    j = np.arange(rope_dim // 2, dtype=np.float64)
    theta = np.arange(n_pos, dtype=np.float64)[:, None] * base ** (-2.0 * j[None, :] / rope_dim)
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


def make_prep_case(cfg: Config, seqs=None) -> dict:
    """Inputs of the indexer preparation for the T new tokens of each sequence (the last T
    positions, start = len - T): q [B,T,H_I,D_I] and k [B,T,D_I] before rope, rotation and
    quantisation (N(0,1), Student-t(3) for the "student_t3" workloads; bf16 bits, or
    float32 for f32 workloads), the rope tables over Lmax positions, and the key cache
    and scales the new keys are appended to (the case's own cache from make_case)."""
    all_lens = lengths(cfg)
    seqs = list(range(cfg.B)) if seqs is None else list(seqs)
    lens = all_lens[seqs].copy()
    T, H_I, D_I = cfg.T, cfg.H_I, cfg.D_I
    # the case's own key cache (same draws as make_case), poisoned past each length
    k_i = np.full((len(seqs), cfg.Lmax, D_I), POISON_K_CODE, np.uint8)
    k_scale = np.full((len(seqs), cfg.Lmax), POISON_VALUE, np.float32)
    for j, b in enumerate(seqs):
        L = int(lens[j])
        c, sc = quantize_e4m3fn(_draw(_rng(cfg, 1, b), (L, D_I), cfg.dist), min(128, D_I))
        k_i[j, :L], k_scale[j, :L] = c, sc[..., 0]
    conv = to_bf16_bits if cfg.attn_dtype == "bf16" else (lambda a: a.astype(np.float32))
    q = np.stack([conv(_draw(_rng(cfg, 7, b), (T, H_I, D_I), cfg.dist)) for b in seqs])
    k = np.stack([conv(_draw(_rng(cfg, 8, b), (T, D_I), cfg.dist)) for b in seqs])
    cos, sin = rope_tables(cfg.Lmax, cfg.rope_i)
    return dict(q=q, k=k, cos=cos, sin=sin, start=(lens - T).astype(np.int32),
                k_cache=k_i, k_scale=k_scale, lens=lens, seqs=seqs)


def to_device(case: dict, device="cuda") -> dict:
    """Copy a case to torch tensors on ``device`` (bf16 words become torch.bfloat16)."""
    out = {}
    for key, a in case.items():
        if key == "seqs":
            out[key] = a
            continue
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        out[key] = t.to(device)
    return out


def visible_keys(cfg: Config, lens: np.ndarray) -> int:
    """Number of (row, key) pairs the indexer scores: sum_b sum_t (pos(b,t) + 1)."""
    T = cfg.T
    return int(sum(int(L) * T - T * (T - 1) // 2 for L in lens))
