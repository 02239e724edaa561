"""ctypes binding of libdsa_amd.so (the C ABI declared in include/dsa.h).

Argument marshalling only: shapes are read off the torch tensors, pointers and the
current HIP stream are passed through, and workspaces are allocated as torch tensors
(the library itself never allocates).  Every computation happens in the library's
kernels; there is no fallback of any kind, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_amd.so")

DSA_OK = 0
DSA_F32, DSA_BF16, DSA_FP8_LATENT = 0, 1, 2
FP8_LATENT_ROW_BYTES = 656     # 512 e4m3fn codes, four fp32 block scales, 64 bf16 rope values
DSA_ATTN_LATENT, DSA_ATTN_MHA = 0, 1
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_DTYPE",
                4: "DSA_ERR_ALIGN", 5: "DSA_ERR_WORKSPACE", 6: "DSA_ERR_HIP"}

EXPORTED = ["dsa_last_error", "dsa_version", "dsa_indexer_prep", "dsa_index_scores",
            "dsa_topk_workspace_bytes",
            "dsa_topk", "dsa_sparse_mla_decode_workspace_bytes", "dsa_sparse_mla_decode",
            "dsa_sparse_mla_prefill_workspace_bytes", "dsa_sparse_mla_prefill",
            "dsa_layer_step_workspace_bytes", "dsa_layer_step", "dsa_layer_step_noalloc",
            "dsa_profile_begin", "dsa_profile_end", "dsa_diag_fp8_mfma_dots"]
NOALLOC_SCRATCH_BYTES = 64 << 20     # DSA_NOALLOC_SCRATCH_BYTES
PHASES = ("index_scores", "topk", "attention", "combine")


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class LayerArgs(ctypes.Structure):
    """Mirror of ``dsa_layer_args``."""
    _fields_ = [
        ("q_fp8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("k_fp8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("len", ctypes.c_void_p),
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H_I", ctypes.c_int), ("d_I", ctypes.c_int),
        ("Lmax", ctypes.c_int), ("topk", ctypes.c_int), ("sm_scale_I", ctypes.c_float),
        ("form", ctypes.c_int), ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p), ("latent", ctypes.c_void_p), ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("H", ctypes.c_int), ("Dv", ctypes.c_int), ("Dr", ctypes.c_int), ("Dqk", ctypes.c_int),
        ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("idx_out", ctypes.c_void_p), ("scores_out", ctypes.c_void_p),
        ("compress_rate", ctypes.c_int),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libdsa_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m deepseek_dsa_indexer_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_version.restype = I
    lib.dsa_version.argtypes = []
    lib.dsa_indexer_prep.argtypes = [P, P, I, P, P, I, P, I, I, I, I, I, I, P, P, P, P, P]
    lib.dsa_index_scores.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, P, P]
    lib.dsa_topk_workspace_bytes.argtypes = [I, I, I, I]
    lib.dsa_topk_workspace_bytes.restype = Z
    lib.dsa_topk.argtypes = [P, P, I, I, I, I, P, P, Z, P]
    lib.dsa_sparse_mla_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.dsa_sparse_mla_decode_workspace_bytes.restype = Z
    lib.dsa_sparse_mla_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, I, P, P, P, Z, P]
    lib.dsa_sparse_mla_prefill_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.dsa_sparse_mla_prefill_workspace_bytes.restype = Z
    lib.dsa_sparse_mla_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, Z, P]
    lib.dsa_layer_step_workspace_bytes.argtypes = [ctypes.POINTER(LayerArgs)]
    lib.dsa_layer_step_workspace_bytes.restype = Z
    lib.dsa_layer_step.argtypes = [ctypes.POINTER(LayerArgs), P, Z, P]
    lib.dsa_layer_step_noalloc.argtypes = [ctypes.POINTER(LayerArgs), P]
    lib.dsa_profile_begin.argtypes = [I]
    lib.dsa_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I)]
    lib.dsa_diag_fp8_mfma_dots.argtypes = [P, P, I, P, P, P]
    for fn in ("dsa_indexer_prep", "dsa_index_scores", "dsa_topk", "dsa_sparse_mla_decode",
               "dsa_sparse_mla_prefill",
               "dsa_layer_step", "dsa_layer_step_noalloc", "dsa_profile_begin", "dsa_profile_end",
               "dsa_diag_fp8_mfma_dots"):
        getattr(lib, fn).restype = I
    _lib = lib
    return lib


def _check(status: int):
    if status != DSA_OK:
        raise DSAError(status, load().dsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fp8(t, name):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _need(t, torch.uint8, name)
    return t


def _attn_dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"attention tensors must be bf16 or f32, got {t.dtype}")


def _latent_dtype(q, latent) -> int:
    """dtype code of a latent-form call: uint8 rows of 656 bytes are the FP8 storage form
    (bf16 queries), otherwise latent has q's dtype."""
    if latent.dtype == torch.uint8 and latent.shape[-1] == FP8_LATENT_ROW_BYTES:
        if q.dtype != torch.bfloat16:
            raise TypeError("FP8 latent rows take bf16 queries")
        _need(latent, torch.uint8, "latent")
        return DSA_FP8_LATENT
    _need(latent, q.dtype, "latent")
    return _attn_dtype(q)


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def indexer_prep(q, k, rope_cos, rope_sin, start, rope_dim, k_cache, k_scale, q_fp8=None,
                 q_scale=None):
    """Rope + rotation + FP8 quantisation of the new tokens' indexer queries q [B,T,H,D]
    and keys k [B,T,D] (bf16 or f32); the key codes and scales are written into
    k_cache [B,Lmax,D] / k_scale [B,Lmax] at positions start[b] + t.  Returns
    (q_fp8 [B,T,H,D] u8, q_scale [B,T,H] f32)."""
    dt = _attn_dtype(q)
    _need(q, q.dtype, "q")
    _need(k, q.dtype, "k")
    _need(start, torch.int32, "start")
    k_cache = _fp8(k_cache, "k_cache")
    _need(k_scale, torch.float32, "k_scale")
    if rope_dim:
        _need(rope_cos, torch.float32, "rope_cos")
        _need(rope_sin, torch.float32, "rope_sin")
        P = rope_cos.shape[0]
    else:
        P = k_cache.shape[1]
    B, T, H, D = q.shape
    Lmax = k_cache.shape[1]
    if q_fp8 is None:
        q_fp8 = torch.empty((B, T, H, D), dtype=torch.uint8, device=q.device)
    if q_scale is None:
        q_scale = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    _check(load().dsa_indexer_prep(_ptr(q), _ptr(k), dt, _ptr(rope_cos) if rope_dim else None,
                                   _ptr(rope_sin) if rope_dim else None, P, _ptr(start), B, T, H,
                                   D, int(rope_dim), Lmax, _ptr(q_fp8), _ptr(q_scale),
                                   _ptr(k_cache), _ptr(k_scale), _stream(q.device)))
    return q_fp8, q_scale


def index_scores(q_fp8, q_scale, w, k_fp8, k_scale, lens, sm_scale_i, scores=None):
    """scores[B,T,Lmax] f32 of the lightning indexer (-inf where not visible)."""
    q_fp8 = _fp8(q_fp8, "q_fp8")
    k_fp8 = _fp8(k_fp8, "k_fp8")
    B, T, H, D = q_fp8.shape
    Lmax = k_fp8.shape[1]
    for t, n in ((q_scale, "q_scale"), (w, "w"), (k_scale, "k_scale")):
        _need(t, torch.float32, n)
    _need(lens, torch.int32, "lens")
    if scores is None:
        scores = torch.empty((B, T, Lmax), dtype=torch.float32, device=q_fp8.device)
    _check(load().dsa_index_scores(_ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8),
                                   _ptr(k_scale), _ptr(lens), B, T, H, D, Lmax,
                                   float(sm_scale_i), _ptr(scores), _stream(q_fp8.device)))
    return scores


def topk(scores, lens, k, idx=None):
    """idx[B,T,k] i32: the selected positions in ascending order, then -1."""
    _need(scores, torch.float32, "scores")
    _need(lens, torch.int32, "lens")
    B, T, Lmax = scores.shape
    lib = load()
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    ws_bytes = lib.dsa_topk_workspace_bytes(B, T, Lmax, k)
    ws = _workspace(ws_bytes, scores.device)
    _check(lib.dsa_topk(_ptr(scores), _ptr(lens), B, T, Lmax, k, _ptr(idx), _ptr(ws), ws_bytes,
                        _stream(scores.device)))
    return idx


def sparse_mla_decode(q, latent, idx, lens, Dv, sm_scale, out=None, lse=None, want_lse=True):
    """Absorbed-form sparse attention; returns (out[B,T,H,Dv], lse[B,T,H] or None)."""
    _need(q, q.dtype, "q")
    dt = _latent_dtype(q, latent)
    _need(idx, torch.int32, "idx")
    _need(lens, torch.int32, "lens")
    B, T, H, Dq = q.shape
    Lmax = latent.shape[1]
    k = idx.shape[-1]
    lib = load()
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    ws_bytes = lib.dsa_sparse_mla_decode_workspace_bytes(B, T, H, Dv, Dq - Dv, k, dt)
    ws = _workspace(ws_bytes, q.device)
    _check(lib.dsa_sparse_mla_decode(_ptr(q), _ptr(latent), _ptr(idx), _ptr(lens), B, T, H, Dv,
                                     Dq - Dv, Lmax, k, float(sm_scale), dt, _ptr(out), _ptr(lse),
                                     _ptr(ws), ws_bytes, _stream(q.device)))
    return out, lse


def sparse_mla_prefill(q, k, v, idx, sm_scale, out=None, lse=None, want_lse=True):
    """MHA-form sparse attention over a chunk starting at position 0."""
    dt = _attn_dtype(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, q.dtype, n)
    _need(idx, torch.int32, "idx")
    B, T, H, Dqk = q.shape
    Dv = v.shape[-1]
    topk_ = idx.shape[-1]
    lib = load()
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    ws_bytes = lib.dsa_sparse_mla_prefill_workspace_bytes(B, T, H, Dqk, Dv, topk_, dt)
    ws = _workspace(ws_bytes, q.device)
    _check(lib.dsa_sparse_mla_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), B, T, H, Dqk, Dv,
                                      topk_, float(sm_scale), dt, _ptr(out), _ptr(lse), _ptr(ws),
                                      ws_bytes, _stream(q.device)))
    return out, lse


def profile_begin(max_steps: int):
    """Start HIP-event timing of the phases of every following layer step."""
    _check(load().dsa_profile_begin(int(max_steps)))


def profile_end() -> dict:
    """Stop timing; returns {phase: (total_ms, count)} for the recorded steps."""
    ms = (ctypes.c_double * 4)()
    cnt = (ctypes.c_int * 4)()
    _check(load().dsa_profile_end(ms, cnt))
    return {name: (ms[i], cnt[i]) for i, name in enumerate(PHASES)}


def diag_fp8_mfma_dots(a, b):
    """Diagnostic: dot products of the 128-code FP8 rows a[p] . b[p] (uint8 [n,128] device
    tensors, n a multiple of 16) on the FP8 and on the bf16 matrix-core forms.
    Returns (out_fp8, out_bf16), float32 [n]."""
    for t, n in ((a, "a"), (b, "b")):
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[1] != 128 or not t.is_contiguous():
            raise ValueError(f"{n}: need a contiguous uint8 [n, 128] tensor")
    if a.shape != b.shape:
        raise ValueError("a and b differ in shape")
    n = a.shape[0]
    out8 = torch.empty(n, dtype=torch.float32, device=a.device)
    outb = torch.empty(n, dtype=torch.float32, device=a.device)
    _check(load().dsa_diag_fp8_mfma_dots(a.data_ptr(), b.data_ptr(), n, out8.data_ptr(),
                                         outb.data_ptr(), _stream(a.device)))
    return out8, outb


class LayerStep:
    """One DSA layer step bound to a fixed set of device tensors.

    Builds the ``dsa_layer_args`` once and owns the workspace, so ``__call__`` is a
    single C call that enqueues the whole step on the current stream."""

    def __init__(self, q_fp8, q_scale, w, k_fp8, k_scale, lens, sm_scale_i, topk, q, sm_scale,
                 latent=None, k=None, v=None, Dv=None, want_lse=True, want_idx=False,
                 want_scores=False, compress_rate=1, workspace=True):
        q_fp8 = _fp8(q_fp8, "q_fp8")
        k_fp8 = _fp8(k_fp8, "k_fp8")
        for t, n in ((q_scale, "q_scale"), (w, "w"), (k_scale, "k_scale")):
            _need(t, torch.float32, n)
        _need(lens, torch.int32, "lens")
        B, T, H_I, D_I = q_fp8.shape
        Lmax = k_fp8.shape[1]
        dt = _attn_dtype(q)
        dev = q.device
        H = q.shape[2]
        a = LayerArgs()
        a.q_fp8, a.q_scale, a.w = q_fp8.data_ptr(), q_scale.data_ptr(), w.data_ptr()
        a.k_fp8, a.k_scale, a.len = k_fp8.data_ptr(), k_scale.data_ptr(), lens.data_ptr()
        a.B, a.T, a.H_I, a.d_I, a.Lmax, a.topk = B, T, H_I, D_I, Lmax, topk
        a.sm_scale_I = float(sm_scale_i)
        a.compress_rate = int(compress_rate)
        a.dtype = dt
        a.q = q.data_ptr()
        a.H = H
        a.sm_scale = float(sm_scale)
        if latent is not None:
            a.dtype = dt = _latent_dtype(q, latent)
            if Dv is None:
                raise ValueError("Dv is required for the latent form")
            a.form = DSA_ATTN_LATENT
            a.latent = latent.data_ptr()
            a.Dv, a.Dr, a.Dqk = Dv, q.shape[3] - Dv, 0
        else:
            _need(k, q.dtype, "k")
            _need(v, q.dtype, "v")
            a.form = DSA_ATTN_MHA
            a.k, a.v = k.data_ptr(), v.data_ptr()
            Dv = v.shape[-1]
            a.Dv, a.Dr, a.Dqk = Dv, 0, q.shape[3]
        self.out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
        self.lse = torch.empty((B, T, H), dtype=torch.float32, device=dev) if want_lse else None
        self.idx = torch.empty((B, T, topk), dtype=torch.int32, device=dev) if want_idx else None
        self.scores = (torch.empty((B, T, Lmax), dtype=torch.float32, device=dev)
                       if want_scores else None)
        a.out = self.out.data_ptr()
        a.lse = self.lse.data_ptr() if want_lse else None
        a.idx_out = self.idx.data_ptr() if want_idx else None
        a.scores_out = self.scores.data_ptr() if want_scores else None
        self.args = a
        self._keep = (q_fp8, q_scale, w, k_fp8, k_scale, lens, q, latent, k, v)
        lib = load()
        self.ws_bytes = lib.dsa_layer_step_workspace_bytes(ctypes.byref(a))
        # 256-byte aligned workspace (torch's caching allocator aligns to 512 bytes);
        # workspace=False: none (for call_noalloc only)
        self.ws = _workspace(self.ws_bytes, dev) if workspace else None
        self._ws_ptr = _ptr(self.ws)
        self.device = dev

    def __call__(self, stream=None):
        s = ctypes.c_void_p(stream) if stream is not None else _stream(self.device)
        _check(load().dsa_layer_step(ctypes.byref(self.args), self._ws_ptr, self.ws_bytes, s))
        return self.out, self.lse

    def call_noalloc(self, stream=None):
        """The same step through dsa_layer_step_noalloc (the library's own per-device
        scratch instead of this object's workspace)."""
        s = ctypes.c_void_p(stream) if stream is not None else _stream(self.device)
        _check(load().dsa_layer_step_noalloc(ctypes.byref(self.args), s))
        return self.out, self.lse
