"""dsa_layer_step_noalloc (the entry point for callers that cannot allocate: the
workspace comes from the library's fixed per-device scratch array) against
dsa_layer_step with a caller workspace: identical outputs, on two calls in a row, the
second with a smaller input (the scratch then still holds the first call's values)."""
import dataclasses
import sys

import pytest
import torch

import dsa_synth as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import deepseek_dsa_indexer_amd as D
    D.load()
    return D


def test_noalloc_matches_workspace_entry_point(dsa):
    # 8 ragged rows beyond 16384 positions (two-stage top-k candidates and split attention
    # partials in the scratch), then 3 shorter rows
    for B, Lmax, lo, seed in [(8, 40000, 17000, 611), (3, 4100, 1000, 612)]:
        print(f"[no_alloc] B={B} Lmax={Lmax}", flush=True)
        sys.stdout.flush()
        cfg = dataclasses.replace(S.CONFIGS["decode_ragged"], name="na", B=B, Lmax=Lmax,
                                  lens=f"ragged:{lo}:{Lmax}", seed=seed)
        c = S.make_case(cfg)
        d = S.to_device(c, "cuda")
        args = (d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale)
        ref = dsa.LayerStep(*args, latent=d["latent"], Dv=cfg.Dv)
        o_ref, l_ref = ref()
        torch.cuda.synchronize()
        na = dsa.LayerStep(*args, latent=d["latent"], Dv=cfg.Dv, workspace=False)
        assert na.ws is None and na.ws_bytes <= dsa.NOALLOC_SCRATCH_BYTES
        o, l = na.call_noalloc()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "outputs differ from the workspace entry point"
        assert torch.equal(l, l_ref), "lse differs from the workspace entry point"
