"""The C-ABI library on the host (no GPU needed): it loads, it exports every entry point
that include/dsa.h declares, and its argument validation rejects bad calls before any
work is enqueued (these paths return before touching the device)."""
import ctypes
import os
import re

import pytest

from deepseek_dsa_indexer_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.library_path()):
        pytest.fail("libdsa_amd.so is not built (python -m deepseek_dsa_indexer_amd.build)")
    return N.load()


def test_exports_match_header(lib):
    declared = _declared()
    assert sorted(N.EXPORTED) == declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dsa_version() >= 100


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def test_index_scores_validation(lib):
    p = _fake()
    st = lib.dsa_index_scores(None, p, p, p, p, p, 1, 1, 64, 128, 16, 1.0, p, None)
    assert st == 1 and b"NULL" in lib.dsa_last_error()
    assert lib.dsa_index_scores(p, p, p, p, p, p, 1, 1, 65, 128, 16, 1.0, p, None) == 2
    assert lib.dsa_index_scores(p, p, p, p, p, p, 1, 1, 64, 96, 16, 1.0, p, None) == 2
    assert lib.dsa_index_scores(p, p, p, p, p, p, 1, 17, 64, 128, 16, 1.0, p, None) == 2
    assert lib.dsa_index_scores(p, p, p, p, p, p, 0, 1, 64, 128, 16, 1.0, p, None) == 2
    q = _fake(0x10004)
    assert lib.dsa_index_scores(q, p, p, p, p, p, 1, 1, 64, 128, 16, 1.0, p, None) == 4


def test_diag_fp8_dots_validation(lib):
    p = _fake()
    assert lib.dsa_diag_fp8_mfma_dots(None, p, 16, p, p, None) == 1
    assert lib.dsa_diag_fp8_mfma_dots(p, p, 15, p, p, None) == 2
    assert lib.dsa_diag_fp8_mfma_dots(p, p, 0, p, p, None) == 2
    assert lib.dsa_diag_fp8_mfma_dots(_fake(0x10008), p, 16, p, p, None) == 4


def test_topk_validation(lib):
    p = _fake()
    assert lib.dsa_topk(p, p, 1, 1, 16, 0, p, None, 0, None) == 2
    assert lib.dsa_topk(None, p, 1, 1, 16, 4, p, None, 0, None) == 1
    assert lib.dsa_topk(p, p, 1, 2, 1, 4, p, None, 0, None) == 2
    # rows up to 16384 positions need no workspace; longer rows keep per-chunk candidates
    assert lib.dsa_topk_workspace_bytes(32, 1, 8192, 2048) == 0
    assert lib.dsa_topk_workspace_bytes(4, 1, 16384, 2048) == 0
    need = lib.dsa_topk_workspace_bytes(8, 1, 131072, 2048)
    assert need >= 8 * 131072 // 16384 * 2048 * 8      # keys + positions of every chunk's top-k
    assert lib.dsa_topk_workspace_bytes(8, 1, 131072, 8192) == 0   # k >= chunk: one pass
    st = lib.dsa_topk(p, p, 8, 1, 131072, 2048, p, None, 0, None)
    assert st == 5 and b"workspace" in lib.dsa_last_error()
    st = lib.dsa_topk(p, p, 8, 1, 131072, 2048, p, p, need - 1, None)
    assert st == 5


def test_attention_validation_and_workspace(lib):
    p = _fake()
    # the matrix-core shape needs a workspace once the rows are split
    need = lib.dsa_sparse_mla_decode_workspace_bytes(2, 1, 128, 512, 64, 2048, N.DSA_BF16)
    assert need > 0
    st = lib.dsa_sparse_mla_decode(p, p, p, p, 2, 1, 128, 512, 64, 4096, 2048, 0.1, N.DSA_BF16,
                                   p, None, None, 0, None)
    assert st == 5 and b"workspace" in lib.dsa_last_error()
    st = lib.dsa_sparse_mla_decode(p, p, p, p, 2, 1, 128, 512, 64, 4096, 2048, 0.1, 7, p, None,
                                   None, 0, None)
    assert st == 3
    # rows that fill the GPU keep each row in one workgroup (no partials)
    assert lib.dsa_sparse_mla_decode_workspace_bytes(256, 1, 128, 512, 64, 1024, N.DSA_BF16) == 0
    # beyond 16 splits of 1024 slots the latent shape leaves the matrix-core path: the
    # generic path needs no workspace but must hold all k logits in LDS
    assert lib.dsa_sparse_mla_decode_workspace_bytes(2, 1, 128, 512, 64, 16384, N.DSA_BF16) > 0
    assert lib.dsa_sparse_mla_decode_workspace_bytes(2, 1, 128, 512, 64, 16385, N.DSA_BF16) == 0
    st = lib.dsa_sparse_mla_decode(p, p, p, p, 2, 1, 128, 512, 64, 1 << 16, 20000, 0.1,
                                   N.DSA_BF16, p, None, None, 0, None)
    assert st == 2 and b"too large" in lib.dsa_last_error()
    # generic (f32) path: logits of all k slots must fit in LDS
    st = lib.dsa_sparse_mla_prefill(p, p, p, p, 1, 8, 2, 192, 128, 1 << 15, 0.1, N.DSA_F32, p,
                                    None, None, 0, None)
    assert st == 2
    # matrix-core (bf16 192/128) path: needs the selection-mask workspace
    assert lib.dsa_sparse_mla_prefill_workspace_bytes(1, 8192, 128, 192, 128, 2048, N.DSA_BF16) >= 8192 * 256 * 4
    st = lib.dsa_sparse_mla_prefill(p, p, p, p, 1, 8, 2, 192, 128, 1 << 15, 0.1, N.DSA_BF16, p,
                                    None, None, 0, None)
    assert st == 5


def test_layer_step_validation(lib):
    a = N.LayerArgs()
    assert lib.dsa_layer_step(None, None, 0, None) == 1
    assert lib.dsa_layer_step(ctypes.byref(a), None, 0, None) == 1
    p = 0x10000
    a.q_fp8 = a.q_scale = a.w = a.k_fp8 = a.k_scale = a.len = p
    a.B, a.T, a.H_I, a.d_I, a.Lmax, a.topk = 32, 1, 64, 128, 8192, 2048
    a.form, a.dtype = N.DSA_ATTN_LATENT, N.DSA_BF16
    a.q = a.latent = a.out = p
    a.H, a.Dv, a.Dr = 128, 512, 64
    need = lib.dsa_layer_step_workspace_bytes(ctypes.byref(a))
    assert need >= 32 * 8192 * 4 + 32 * 2048 * 4
    assert lib.dsa_layer_step(ctypes.byref(a), None, 0, None) == 5
    assert lib.dsa_layer_step(ctypes.byref(a), ctypes.c_void_p(p + 16), need, None) == 4
    # compressed entries: T may exceed the entry capacity Lmax; negative rates are rejected
    a.compress_rate = -1
    assert lib.dsa_layer_step(ctypes.byref(a), ctypes.c_void_p(p), need, None) == 2
    a.compress_rate = 4
    a.T, a.Lmax = 64, 16
    need_c = lib.dsa_layer_step_workspace_bytes(ctypes.byref(a))
    assert lib.dsa_layer_step(ctypes.byref(a), None, 0, None) == 5      # validation passed
    a.T, a.Lmax = 1, 8192
    a.form = N.DSA_ATTN_MHA
    a.k = a.v = p
    a.Dqk = 192
    assert lib.dsa_layer_step(ctypes.byref(a), ctypes.c_void_p(p), need, None) == 2  # MHA + compression
    assert b"latent form" in lib.dsa_last_error()
    a.compress_rate = 0
    assert need_c > 0
    assert lib.dsa_layer_step(ctypes.byref(a), ctypes.c_void_p(p), need, None) == 2  # Lmax != T


def test_layer_step_noalloc_validation(lib):
    """The allocation-free entry point rejects, before touching the device, any shape
    whose workspace exceeds its fixed scratch (a T=8192 prefill chunk's scores), and
    validates like dsa_layer_step otherwise."""
    a = N.LayerArgs()
    assert lib.dsa_layer_step_noalloc(None, None) == 1
    p = 0x10000
    a.q_fp8 = a.q_scale = a.w = a.k_fp8 = a.k_scale = a.len = p
    a.B, a.T, a.H_I, a.d_I, a.Lmax, a.topk = 1, 8192, 64, 128, 8192, 2048
    a.form, a.dtype = N.DSA_ATTN_MHA, N.DSA_BF16
    a.q = a.k = a.v = a.out = p
    a.H, a.Dv, a.Dqk = 128, 128, 192
    assert lib.dsa_layer_step_workspace_bytes(ctypes.byref(a)) > N.NOALLOC_SCRATCH_BYTES
    assert lib.dsa_layer_step_noalloc(ctypes.byref(a), None) == 5
    assert b"scratch" in lib.dsa_last_error()
    # the largest decode workload (64 sequences of up to 65536 positions) fits
    a.B, a.T, a.Lmax = 64, 1, 65536
    a.form, a.latent, a.Dv, a.Dr, a.Dqk = N.DSA_ATTN_LATENT, p, 512, 64, 0
    assert lib.dsa_layer_step_workspace_bytes(ctypes.byref(a)) <= N.NOALLOC_SCRATCH_BYTES


def test_fp8_latent_validation(lib):
    """FP8 latent rows: the latent form only, at the storage form's 512 + 64 widths; the
    matrix-core shape takes the same split workspace as bf16 rows."""
    p = _fake()
    F8 = N.DSA_FP8_LATENT
    assert F8 == 2
    assert (lib.dsa_sparse_mla_decode_workspace_bytes(2, 1, 128, 512, 64, 2048, F8) ==
            lib.dsa_sparse_mla_decode_workspace_bytes(2, 1, 128, 512, 64, 2048, N.DSA_BF16))
    st = lib.dsa_sparse_mla_decode(p, p, p, p, 2, 1, 128, 256, 64, 4096, 2048, 0.1, F8, p, None,
                                   None, 0, None)
    assert st == 3 and b"FP8" in lib.dsa_last_error()
    st = lib.dsa_sparse_mla_decode(p, p, p, p, 2, 1, 128, 512, 64, 4096, 2048, 0.1, F8, p, None,
                                   None, 0, None)
    assert st == 5
    # any head count runs on the vector-ALU path (no workspace)
    assert lib.dsa_sparse_mla_decode_workspace_bytes(2, 1, 16, 512, 64, 2048, F8) == 0
    # the MHA prefill form has no FP8 variant
    st = lib.dsa_sparse_mla_prefill(p, p, p, p, 1, 8, 2, 192, 128, 64, 0.1, F8, p, None, None, 0,
                                    None)
    assert st == 3


def test_indexer_prep_validation(lib):
    p = _fake()
    args = lambda **kw: [kw.get("q", p), p, kw.get("dt", N.DSA_BF16), p, p, kw.get("P", 100), p,
                         kw.get("B", 2), kw.get("T", 1), kw.get("H", 64), kw.get("D", 128),
                         kw.get("R", 64), kw.get("Lmax", 100), p, p, p, p, None]
    assert lib.dsa_indexer_prep(*args(q=None)) == 1
    assert lib.dsa_indexer_prep(*args(dt=N.DSA_FP8_LATENT)) == 3
    assert lib.dsa_indexer_prep(*args(D=96)) == 2
    assert lib.dsa_indexer_prep(*args(H=65)) == 2
    assert lib.dsa_indexer_prep(*args(R=62)) == 2 and b"rope_dim" in lib.dsa_last_error()
    assert lib.dsa_indexer_prep(*args(R=48)) == 2
    assert lib.dsa_indexer_prep(*args(R=132)) == 2
    assert lib.dsa_indexer_prep(*args(T=101)) == 2
    assert lib.dsa_indexer_prep(*args(q=_fake(0x10008))) == 4
    # no rope: the tables may be NULL (validation passes through to the alignment checks)
    a = args(R=0)
    a[3] = a[4] = None
    a[0] = _fake(0x10008)
    assert lib.dsa_indexer_prep(*a) == 4
