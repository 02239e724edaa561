"""CPU reference for one DSA layer step: TEST INFRASTRUCTURE, not the product.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg import
this package.  It wraps ``liboracle.so`` (built from ``dsa_oracle.c`` by
:func:`build`) with ctypes and numpy; every number it returns comes from that plain
C code, written from the pages' definitions (see the header comment of
``dsa_oracle.c`` for the citations).  It shares nothing with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64, FP8_LATENT = 0, 1, 2, 3
FP8_LATENT_ROW_BYTES = 656      # 512 e4m3fn codes + 4 fp32 scales + 64 bf16 rope values
_OK, _ERR_SHAPE, _ERR_INDEX = 0, 1, 2


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (OpenMP over independent query rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.orc_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3fn_value.restype = D
        lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_value.restype = D
        lib.orc_latent_fp8_value.argtypes = [P, I]
        lib.orc_latent_fp8_value.restype = D
        lib.orc_index_scores.argtypes = [P, P, P, P, P, P, I, I, I, I, I, D, I, P]
        lib.orc_topk.argtypes = [P, P, I, I, I, I, I, P]
        lib.orc_sparse_mla_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, D, I, P, P]
        lib.orc_sparse_mha_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, P, P]
        lib.orc_sparse_mha_prefill_dense.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, P, P]
        lib.orc_sparse_mha_prefill_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, P, P, I, P, P]
        lib.orc_layer_step_latent.argtypes = [P, P, P, P, P, P, I, I, I, I, I, D, I,
                                              P, P, I, I, I, I, D, I, P, P, P, P]
        lib.orc_layer_step_mha.argtypes = [P, P, P, P, P, I, I, I, I, D, I,
                                           P, P, P, I, I, I, I, D, P, P, P, P]
        lib.orc_e4m3fn_encode.argtypes = [D]
        lib.orc_e4m3fn_encode.restype = ctypes.c_uint8
        lib.orc_indexer_prep.argtypes = [P, P, I, P, P, I, P, I, I, I, I, I, I,
                                         P, P, P, P, P, P, P]
        lib.orc_indexer_prep.restype = I
        lib.orc_max_threads.argtypes = []
        lib.orc_set_threads.argtypes = [I]
        lib.orc_set_threads.restype = None
        for fn in (lib.orc_index_scores, lib.orc_topk, lib.orc_sparse_mla_decode,
                   lib.orc_sparse_mha_prefill, lib.orc_sparse_mha_prefill_dense,
                   lib.orc_sparse_mha_prefill_rows,
                   lib.orc_layer_step_latent, lib.orc_layer_step_mha, lib.orc_max_threads):
            fn.restype = I
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _attn_array(x):
    """Return (contiguous array, dtype code).  bf16 travels as raw uint16 words; uint8
    arrays whose last axis is 656 bytes are latent rows in the FP8 storage form."""
    if x.dtype == np.uint8 and x.shape[-1] == FP8_LATENT_ROW_BYTES:
        return np.ascontiguousarray(x), FP8_LATENT
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), F32
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), F64
    raise TypeError(f"attention inputs must be float32, float64 or bf16 bits (uint16), got {x.dtype}")


def _check(rc, what):
    if rc != _OK:
        raise OracleError(f"{what}: oracle returned {rc}")


def max_threads() -> int:
    return _load().orc_max_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's following parallel loops."""
    _load().orc_set_threads(int(n))


def e4m3fn_value(code: int) -> float:
    return _load().orc_e4m3fn_value(code)


def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits)


def latent_fp8_value(row, d: int) -> float:
    """Decoded column d of one 656-byte FP8 latent row (uint8 array)."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    assert row.shape == (FP8_LATENT_ROW_BYTES,)
    return _load().orc_latent_fp8_value(row.ctypes.data_as(ctypes.c_void_p), int(d))


def latent_fp8_decode(rows) -> np.ndarray:
    """Decode FP8 latent rows [..., 656] u8 to float64 [..., 576] column by column."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    flat = rows.reshape(-1, FP8_LATENT_ROW_BYTES)
    out = np.empty((flat.shape[0], 576), np.float64)
    lib = _load()
    for i in range(flat.shape[0]):
        p = flat[i].ctypes.data_as(ctypes.c_void_p)
        for d in range(576):
            out[i, d] = lib.orc_latent_fp8_value(p, d)
    return out.reshape(*rows.shape[:-1], 576)


def e4m3fn_encode(y: float) -> int:
    """OCP e4m3fn code of y in [-448, 448] (nearest, ties to even)."""
    return int(_load().orc_e4m3fn_encode(float(y)))


def indexer_prep(q, k, cos, sin, start, rope_dim, k_cache, k_scale):
    """Rope (non-interleaved) + Walsh-Hadamard rotation + blockwise FP8 quantisation of the
    new indexer queries q [B,T,H,D] and keys k [B,T,D] (float32/float64 or bf16 bits), the
    keys appended into copies of k_cache [B,Lmax,D] u8 / k_scale [B,Lmax] f32 at positions
    start[b] + t.  Returns a dict: q_fp8, q_scale (float64), k_cache, k_scale (the updated
    copies), k_scale64, q_y, k_y (values divided by their scale, before rounding)."""
    B, T, H, D = q.shape
    Lmax = k_cache.shape[1]
    qa, dt = _attn_array(q)
    ka, dt2 = _attn_array(k)
    assert dt == dt2 and ka.shape == (B, T, D)
    cos, pc = _c(cos, np.float32)
    sin, ps = _c(sin, np.float32)
    assert cos.shape == sin.shape and cos.shape[1] == rope_dim // 2
    start, pst = _c(start, np.int32)
    kc = np.array(k_cache, dtype=np.uint8, copy=True, order="C")
    ks = np.array(k_scale, dtype=np.float32, copy=True, order="C")
    out = dict(q_fp8=np.empty((B, T, H, D), np.uint8), q_scale=np.empty((B, T, H), np.float64),
               k_scale64=np.empty((B, T), np.float64), q_y=np.empty((B, T, H, D), np.float64),
               k_y=np.empty((B, T, D), np.float64))
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(_load().orc_indexer_prep(vp(qa), vp(ka), dt, pc, ps, cos.shape[0], pst, B, T, H, D,
                                    rope_dim, Lmax, vp(out["q_fp8"]), vp(out["q_scale"]),
                                    vp(kc), vp(ks), vp(out["k_scale64"]), vp(out["q_y"]),
                                    vp(out["k_y"])), "indexer_prep")
    out.update(k_cache=kc, k_scale=ks)
    return out


def index_scores(q_fp8, q_scale, w, k_fp8, k_scale, lens, sm_scale_i, compress=1):
    """scores[B,T,Lmax] f32 = sum_h w*q_scale*sm_scale_i * ReLU(q.k) * k_scale, -inf if invisible
    (compress = m > 1: the cache rows are compressed entries, row (b,t) sees
    e < (len - T + t + 1) / m)."""
    B, T, H, D = q_fp8.shape
    Lmax = k_fp8.shape[1]
    lib = _load()
    q_fp8, pq = _c(q_fp8, np.uint8)
    q_scale, pqs = _c(q_scale, np.float32)
    w, pw = _c(w, np.float32)
    k_fp8, pk = _c(k_fp8, np.uint8)
    k_scale, pks = _c(k_scale, np.float32)
    lens, pl = _c(lens, np.int32)
    out = np.empty((B, T, Lmax), np.float32)
    _check(lib.orc_index_scores(pq, pqs, pw, pk, pks, pl, B, T, H, D, Lmax, float(sm_scale_i),
                                int(compress), out.ctypes.data_as(ctypes.c_void_p)), "index_scores")
    return out


def topk(scores, lens, k, compress=1):
    """idx[B,T,k] i32: the min(k, n) best visible rows ascending, then -1."""
    B, T, Lmax = scores.shape
    lib = _load()
    scores, ps = _c(scores, np.float32)
    lens, pl = _c(lens, np.int32)
    out = np.empty((B, T, k), np.int32)
    _check(lib.orc_topk(ps, pl, B, T, Lmax, k, int(compress), out.ctypes.data_as(ctypes.c_void_p)),
           "topk")
    return out


def sparse_mla_decode(q, latent, idx, lens, Dv, sm_scale, compress=1):
    """Absorbed-form sparse attention.  Returns (out[B,T,H,Dv] f64, lse[B,T,H] f64)."""
    B, T, H, Dq = q.shape
    Lmax = latent.shape[1]
    k = idx.shape[-1]
    lib = _load()
    q, dt = _attn_array(q)
    latent, dt2 = _attn_array(latent)
    if dt2 == FP8_LATENT:
        assert dt == BF16 and Dq == 576 and Dv == 512
        dt = FP8_LATENT
    else:
        assert dt == dt2 and latent.shape[-1] == Dq
    idx, pi = _c(idx, np.int32)
    lens, pl = _c(lens, np.int32)
    out = np.empty((B, T, H, Dv), np.float64)
    lse = np.empty((B, T, H), np.float64)
    _check(lib.orc_sparse_mla_decode(q.ctypes.data_as(ctypes.c_void_p),
                                     latent.ctypes.data_as(ctypes.c_void_p), pi, pl, dt,
                                     B, T, H, Dv, Dq - Dv, Lmax, k, float(sm_scale), int(compress),
                                     out.ctypes.data_as(ctypes.c_void_p),
                                     lse.ctypes.data_as(ctypes.c_void_p)), "sparse_mla_decode")
    return out, lse


def _mha(fn, q, k_, v, idx, sm_scale):
    B, T, H, Dqk = q.shape
    Dv = v.shape[-1]
    topk_ = idx.shape[-1]
    q, dt = _attn_array(q)
    k_, dt2 = _attn_array(k_)
    v, dt3 = _attn_array(v)
    assert dt == dt2 == dt3
    idx, pi = _c(idx, np.int32)
    out = np.empty((B, T, H, Dv), np.float64)
    lse = np.empty((B, T, H), np.float64)
    _check(fn(q.ctypes.data_as(ctypes.c_void_p), k_.ctypes.data_as(ctypes.c_void_p),
              v.ctypes.data_as(ctypes.c_void_p), pi, dt, B, T, H, Dqk, Dv, topk_,
              float(sm_scale), out.ctypes.data_as(ctypes.c_void_p),
              lse.ctypes.data_as(ctypes.c_void_p)), "sparse_mha_prefill")
    return out, lse


def sparse_mha_prefill(q, k_, v, idx, sm_scale):
    """Gather-form sparse MHA over selected and causally visible keys."""
    return _mha(_load().orc_sparse_mha_prefill, q, k_, v, idx, sm_scale)


def sparse_mha_prefill_rows(q, k_, v, idx, sm_scale, rows):
    """Gather-form sparse MHA for the listed query rows [(b, t), ...] only.
    Returns (out[R,H,Dv] f64, lse[R,H] f64)."""
    B, T, H, Dqk = q.shape
    Dv = v.shape[-1]
    topk_ = idx.shape[-1]
    q, dt = _attn_array(q)
    k_, dt2 = _attn_array(k_)
    v, dt3 = _attn_array(v)
    assert dt == dt2 == dt3
    idx, pi = _c(idx, np.int32)
    rb, prb = _c(np.array([r[0] for r in rows]), np.int32)
    rt, prt = _c(np.array([r[1] for r in rows]), np.int32)
    out = np.empty((len(rows), H, Dv), np.float64)
    lse = np.empty((len(rows), H), np.float64)
    _check(_load().orc_sparse_mha_prefill_rows(
        q.ctypes.data_as(ctypes.c_void_p), k_.ctypes.data_as(ctypes.c_void_p),
        v.ctypes.data_as(ctypes.c_void_p), pi, dt, B, T, H, Dqk, Dv, topk_, float(sm_scale),
        prb, prt, len(rows), out.ctypes.data_as(ctypes.c_void_p),
        lse.ctypes.data_as(ctypes.c_void_p)), "sparse_mha_prefill_rows")
    return out, lse


def sparse_mha_prefill_dense(q, k_, v, idx, sm_scale):
    """The same result computed as dense scores + index mask + causal mask."""
    return _mha(_load().orc_sparse_mha_prefill_dense, q, k_, v, idx, sm_scale)


def layer_step_latent(q_fp8, q_scale, w, k_fp8, k_scale, lens, sm_scale_i, k, q, latent, Dv,
                      sm_scale, want_scores=False, compress=1):
    """Index scores -> top-k -> sparse latent attention.  Returns (out, lse, idx[, scores])."""
    B, T, H_I, D_I = q_fp8.shape
    Lmax = k_fp8.shape[1]
    H, Dq = q.shape[2], q.shape[3]
    lib = _load()
    arrs = [_c(q_fp8, np.uint8), _c(q_scale, np.float32), _c(w, np.float32),
            _c(k_fp8, np.uint8), _c(k_scale, np.float32), _c(lens, np.int32)]
    qa, dt = _attn_array(q)
    la, dt2 = _attn_array(latent)
    if dt2 == FP8_LATENT:
        assert dt == BF16 and Dq == 576 and Dv == 512
        dt = FP8_LATENT
    else:
        assert dt == dt2
    out = np.empty((B, T, H, Dv), np.float64)
    lse = np.empty((B, T, H), np.float64)
    idx = np.empty((B, T, k), np.int32)
    scores = np.empty((B, T, Lmax), np.float32) if want_scores else None
    _check(lib.orc_layer_step_latent(*[p for _, p in arrs], B, T, H_I, D_I, Lmax,
                                     float(sm_scale_i), k, qa.ctypes.data_as(ctypes.c_void_p),
                                     la.ctypes.data_as(ctypes.c_void_p), dt, H, Dv, Dq - Dv,
                                     float(sm_scale), int(compress),
                                     out.ctypes.data_as(ctypes.c_void_p),
                                     lse.ctypes.data_as(ctypes.c_void_p),
                                     scores.ctypes.data_as(ctypes.c_void_p) if want_scores else None,
                                     idx.ctypes.data_as(ctypes.c_void_p)), "layer_step_latent")
    return (out, lse, idx, scores) if want_scores else (out, lse, idx)


def layer_step_mha(q_fp8, q_scale, w, k_fp8, k_scale, sm_scale_i, k, q, k_, v, sm_scale):
    """Index scores -> top-k -> sparse MHA prefill (chunk from position 0)."""
    B, T, H_I, D_I = q_fp8.shape
    H, Dqk = q.shape[2], q.shape[3]
    Dv = v.shape[-1]
    lib = _load()
    arrs = [_c(q_fp8, np.uint8), _c(q_scale, np.float32), _c(w, np.float32),
            _c(k_fp8, np.uint8), _c(k_scale, np.float32)]
    qa, dt = _attn_array(q)
    ka, _ = _attn_array(k_)
    va, _ = _attn_array(v)
    out = np.empty((B, T, H, Dv), np.float64)
    lse = np.empty((B, T, H), np.float64)
    idx = np.empty((B, T, k), np.int32)
    _check(lib.orc_layer_step_mha(*[p for _, p in arrs], B, T, H_I, D_I, float(sm_scale_i), k,
                                  qa.ctypes.data_as(ctypes.c_void_p),
                                  ka.ctypes.data_as(ctypes.c_void_p),
                                  va.ctypes.data_as(ctypes.c_void_p), dt, H, Dqk, Dv,
                                  float(sm_scale), out.ctypes.data_as(ctypes.c_void_p),
                                  lse.ctypes.data_as(ctypes.c_void_p), None,
                                  idx.ctypes.data_as(ctypes.c_void_p)), "layer_step_mha")
    return out, lse, idx
