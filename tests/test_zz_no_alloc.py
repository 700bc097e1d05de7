"""fsa_attention_static, the entry point that allocates nothing (GPU).

Its workspace is a static device array inside the library, shared by every
call on a GPU. Checked through the C ABI against fsa_attention (the same
kernels, with a workspace of the caller's) on two calls in a row, the second
with a smaller input, so the second runs on the contents the first left
behind; both against the oracle's bar on sampled rows; and a plan whose
workspace exceeds the array is refused before any launch.
"""
import numpy as np
import pytest
import torch

from frame_aligned_block_amd import fsa
from frame_aligned_block_amd.inputs import CONFIGS, make_inputs

from gpu_util import assert_close, oracle_rows, sample_rows, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU too; every test here is gpu-marked
    pytest.skip("no GPU", allow_module_level=True)


def plan_of(cfg):
    code = fsa.FSA_BF16 if cfg.dtype == "bf16" else fsa.FSA_F32
    return fsa.fsa_plan_create(fsa.make_shape(cfg.B, cfg.H, cfg.F, cfg.T, cfg.d, cfg.window,
                                              cfg.ref_frame, 0, 0, code))


def test_static_workspace_matches_fsa_attention_twice():
    torch.cuda.set_device(0)
    cases = [CONFIGS["small"].with_(H=8), CONFIGS["small"].with_(F=5, T=240, H=2, window=1)]
    for i, cfg in enumerate(cases):
        say("fsa_attention_static call", i, cfg.name, cfg.F, cfg.T, cfg.H)
        Q, K, V = make_inputs(cfg, seed=i, device="cuda")
        plan = plan_of(cfg)
        assert fsa.fsa_workspace_bytes(plan) <= fsa.FSA_STATIC_WS_BYTES
        want = fsa.attention(Q, K, V, cfg.F, cfg.T, cfg.window, cfg.ref_frame)
        O = torch.full_like(Q, float("nan"))
        fsa.fsa_attention_static(plan, Q, K, V, O, cfg.scale, "auto")
        torch.cuda.synchronize()
        assert torch.equal(O, want), f"call {i}"
        rows = sample_rows(cfg, 120, seed=i)
        for h in (0, cfg.H - 1):
            ref = oracle_rows(cfg, Q, K, V, 0, h, rows)
            assert_close(cfg, O[0, h, rows], ref, f"static call {i} head {h}")


def test_static_workspace_refuses_a_plan_that_does_not_fit():
    cfg = CONFIGS["720p"].with_(H=48)                 # about 18 MiB of workspace
    say("fsa_attention_static too large")
    plan = plan_of(cfg)
    assert fsa.fsa_workspace_bytes(plan) > fsa.FSA_STATIC_WS_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fsa.FsaError) as e:
        fsa.fsa_attention_static(plan, x, x, x, x, cfg.scale, "auto")
    assert e.value.status == fsa.FSA_ERR_WORKSPACE
    assert "static workspace" in fsa.fsa_last_error()
