"""Seeded random shapes through the whole path vs the fp64 oracle (GPU).

Each case draws a frame count, frame span (a multiple of 16), window,
reference frame, batch, heads, head width, dtype and route mode from a fixed
seed, runs fsa_bounds and fsa_forward twice, and checks every output row
against the oracle (bf16: max-abs 2e-2, mean-abs 2e-3; fp32: max-abs 1e-5)
and the two launches bit for bit. Cross-attention cases draw a reference-set
size instead of a window. The shapes cover single frames, frames shorter than
one workgroup, spans that leave ragged row units and key chunks, and both
kernels' head widths, in both workgroup geometries of the bf16 kernel.
"""
import os

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as orc
from frame_aligned_block_amd.inputs import CONFIGS, to_f64

from gpu_util import Run, assert_close, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU too; every test here is gpu-marked
    pytest.skip("no GPU", allow_module_level=True)

MODES = ("auto", "online", "auto_frame", "auto_rows")


def draw_case(i: int):
    rng = np.random.default_rng(1000 + i)
    F = int(rng.integers(1, 7))
    T = 16 * int(rng.integers(1, 41))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    cross = rng.random() < 0.25
    cfg = CONFIGS["small"].with_(
        name=f"fuzz{i}", F=F, T=T, d=d, dtype=dtype, B=int(rng.integers(1, 3)),
        H=int(rng.integers(1, 4)), window=0 if cross else int(rng.integers(0, F + 1)),
        ref_frame=0 if cross else int(rng.integers(0, F)),
        M=16 * int(rng.integers(1, 81)) if cross else 0,
        key_sigma=float(rng.choice([1.0, 2.0])))
    mode = str(rng.choice(MODES))
    # bf16: the forward kernel's workgroup geometry (128 or 256 rows)
    row_block = int(rng.choice([128, 256])) if dtype == "bf16" else 0
    return cfg, mode, row_block


# FSA_FUZZ_CASES widens the sweep for a one-off run (the default keeps the
# suite short)
N_CASES = int(os.environ.get("FSA_FUZZ_CASES", "24"))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    cfg, mode, row_block = draw_case(i)
    say("fuzz", i, cfg, mode, row_block)
    run = Run(cfg, seed=i, row_block=row_block).bounds()
    O1 = run.forward(mode)
    O2 = run.forward(mode)
    assert torch.equal(O1, O2), "two launches differ"
    Q, K, V = (to_f64(t) for t in (run.Q, run.K, run.V))
    if cfg.M:
        want = orc.cross_attention(Q, K, V, cfg.scale)
    else:
        want = orc.attention(Q, K, V, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
    mx, mean = assert_close(cfg, O1, want, f"fuzz {i} {mode}")
    print(f"fuzz {i}: F={cfg.F} T={cfg.T} d={cfg.d} {cfg.dtype} B={cfg.B} H={cfg.H} "
          f"w={cfg.window} r={cfg.ref_frame} M={cfg.M} {mode}: max {mx:.3g} mean {mean:.3g}")
