"""Plant a mistake in the CPU reference (on the CPU, in a private build) and check that
at least one pin of oracle_pins.py fails.  This shows the pins would catch a dropped
term, a wrong sign, a wrong index or a transposed operand in the reference."""
import contextlib
import ctypes
import os
import subprocess

import pytest

from oracle_pins import ALL_PINS

MUTATIONS = [
    ("drop ReLU", "acc += wf * (dot > 0.0 ? dot : 0.0);", "acc += wf * dot;"),
    ("ReLU after weighting", "acc += wf * (dot > 0.0 ? dot : 0.0);",
     "acc += (wf * dot > 0.0 ? wf * dot : 0.0);"),
    ("ReLU per product", "for (int d = 0; d < D; ++d) dot += table[qh[d]] * table[ks[d]];",
     "for (int d = 0; d < D; ++d) { const double p_ = table[qh[d]] * table[ks[d]]; "
     "dot += p_ > 0.0 ? p_ : 0.0; }"),
    ("drop q_scale", "(double)w[row * H + h] * (double)q_scale[row * H + h] * sm_scale",
     "(double)w[row * H + h] * sm_scale"),
    ("drop indexer scale", "(double)w[row * H + h] * (double)q_scale[row * H + h] * sm_scale",
     "(double)w[row * H + h] * (double)q_scale[row * H + h]"),
    ("k_scale indexed by row", "(double)k_scale[(size_t)b * Lmax + s]",
     "(double)k_scale[(size_t)b * Lmax + t]"),
    ("causal off by one", "if (s >= n) { out[s] = -INFINITY; continue; }",
     "if (s >= n - 1) { out[s] = -INFINITY; continue; }"),
    ("query head ignored", "const uint8_t* qh = q + (row * H + h) * D;",
     "const uint8_t* qh = q + (row * H) * D;"),
    ("decode e4m3 bias 8", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("top-k takes smallest", "for (int j = 0; j < kk; ++j) out[j] = v[j].pos;",
     "for (int j = 0; j < kk; ++j) out[j] = v[n - 1 - j].pos;"),
    ("top-k ties prefer larger position", "return (x->pos > y->pos) - (x->pos < y->pos);",
     "return (x->pos < y->pos) - (x->pos > y->pos);"),
    ("top-k drops current position", "const int n = visible_rows(len[b], T, t, m);\n            const int kk",
     "const int n = visible_rows(len[b] - (len[b] > T), T, t, m);\n            const int kk"),
    ("attention scale dropped", "logit[j] = sm_scale * dot;", "logit[j] = dot;"),
    ("latent key drops rope part", "for (int d = 0; d < Dq; ++d)\n", "for (int d = 0; d < Dv; ++d)\n"),
    ("latent value offset", "o[d] += p * C[(size_t)j * Dq + d];",
     "o[d] += p * C[(size_t)j * Dq + Dr + d];"),
    ("fp8 latent scale ignored", "return orc_e4m3fn_value(row[d]) * (double)scale;",
     "return orc_e4m3fn_value(row[d]);"),
    ("fp8 latent scale per 64 columns", "row + ORC_FP8_LATENT_DV + 4 * (d / ORC_FP8_LATENT_BLOCK)",
     "row + ORC_FP8_LATENT_DV + 4 * ((d / 64) & 3)"),
    ("fp8 latent rope read over the scales",
     "4 * (ORC_FP8_LATENT_DV / ORC_FP8_LATENT_BLOCK) +\n                      2 * (d - ORC_FP8_LATENT_DV)",
     "2 * (d - ORC_FP8_LATENT_DV)"),
    ("compressed threshold rounded up", "    return (len - T + t + 1) / m;",
     "    return (len - T + t + m) / m;"),
    ("top-k ignores compression", "const int n = visible_rows(len[b], T, t, m);\n            const int kk",
     "const int n = visible_rows(len[b], T, t, 1);\n            const int kk"),
    ("attention ignores compression", "const int nvis = visible_rows(len[b], T, t, m);",
     "const int nvis = visible_rows(len[b], T, t, 1);"),
    ("prep rope interleaved pairs", "const double a = v[j], b = v[j + R / 2];",
     "const double a = v[2 * j], b = v[2 * j + 1];"),
    ("prep rope sin sign", "v[j] = a * (double)cs[j] - b * (double)sn[j];",
     "v[j] = a * (double)cs[j] + b * (double)sn[j];"),
    ("prep rotation unnormalised", "const double norm = 1.0 / sqrt((double)D);",
     "const double norm = 1.0;"),
    ("prep rotation wrong sign pattern", "__builtin_popcount((unsigned)(i & j))",
     "__builtin_popcount((unsigned)(i | j))"),
    ("prep scale over 240", "const double scale = fmax(amax, 1e-12) / 448.0;",
     "const double scale = fmax(amax, 1e-12) / 240.0;"),
    ("prep ties away from zero", "const int mant = (int)nearbyint((m - 1.0) * 8.0);",
     "const int mant = (int)round((m - 1.0) * 8.0);"),
    ("prep key row off by one", "const size_t kr = (size_t)b * Lmax + pos;",
     "const size_t kr = (size_t)b * Lmax + pos - (pos > 0);"),
    ("fp8 latent queries not bf16", "const int qdt = dtype == ORC_FP8_LATENT ? ORC_BF16 : dtype;",
     "const int qdt = dtype == ORC_FP8_LATENT ? ORC_F32 : dtype;"),
    ("latent ignores visibility", "if (sel[j] >= 0 && sel[j] < nvis) keys[n++] = sel[j];",
     "if (sel[j] >= 0) keys[n++] = sel[j];"),
    ("lse without max", "lse[row * H + h] = m + log(sum);", "lse[row * H + h] = log(sum);"),
    ("MHA ignores causality", "if (sel[j] >= 0 && sel[j] <= t) keys[n++] = sel[j];",
     "if (sel[j] >= 0) keys[n++] = sel[j];"),
    ("MHA key head fixed", "const size_t koff = (((size_t)b * T + keys[j]) * H + h) * (size_t)Dqk;",
     "const size_t koff = (((size_t)b * T + keys[j]) * H + 0) * (size_t)Dqk;"),
    ("MHA value from the query row", "const size_t voff = (((size_t)b * T + keys[j]) * H + h) * (size_t)Dv;",
     "const size_t voff = (((size_t)b * T + t) * H + h) * (size_t)Dv;"),
]


@contextlib.contextmanager
def _variant(orc, path):
    saved = orc._load()
    lib = ctypes.CDLL(path)
    for fn in ("orc_e4m3fn_value", "orc_bf16_value", "orc_latent_fp8_value", "orc_e4m3fn_encode",
               "orc_indexer_prep", "orc_index_scores", "orc_topk",
               "orc_sparse_mla_decode", "orc_sparse_mha_prefill", "orc_sparse_mha_prefill_dense",
               "orc_sparse_mha_prefill_rows",
               "orc_layer_step_latent", "orc_layer_step_mha", "orc_max_threads", "orc_set_threads"):
        getattr(lib, fn).argtypes = getattr(saved, fn).argtypes
        getattr(lib, fn).restype = getattr(saved, fn).restype
    orc._lib = lib
    try:
        yield
    finally:
        orc._lib = saved


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(orc, tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(orc.__file__), "dsa_oracle.c")).read()
    assert old in src, f"mutation anchor missing: {old!r}"
    (tmp_path / "dsa_oracle.h").write_text(
        open(os.path.join(os.path.dirname(orc.__file__), "dsa_oracle.h")).read())
    (tmp_path / "m.c").write_text(src.replace(old, new))
    so = str(tmp_path / "libm.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so,
                    str(tmp_path / "m.c"), "-lm"], check=True)
    failed = []
    with _variant(orc, so):
        for pin in ALL_PINS:
            try:
                pin(orc)
            except Exception:
                failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
