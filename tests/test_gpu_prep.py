"""The producer kernel (fsa_prep) and the bounds after it, vs the fp64
oracle (GPU).

Q, K, V: every bf16 output within the rounding it can carry, elementwise:
2^-9 |want| (rounding of the output) + 2^-9 S (rounding of each folded weight
W*gamma to bf16, S = sum_c |W_oc x_hat_c| over the output's source channels,
two of them for a rotated pair) + 1e-4 (fp32 accumulation and the hardware
sine); and mean-abs within 3e-3 (the two roundings average about 1.8e-3);
the row norms and key mean against the GPU's own bf16 outputs in fp64
(1e-5 relative); the bounds products as for fsa_bounds, flags bit-exact; the
attention fed by the producer against the oracle on the same tensors.
"""
import os

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as orc
from oracle import prep_oracle as prp
from frame_aligned_block_amd import fsa
from frame_aligned_block_amd.inputs import CONFIGS, make_prep_inputs, to_f64

from gpu_util import assert_close, oracle_rows, sample_rows, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU too; every test here is gpu-marked
    pytest.skip("no GPU", allow_module_level=True)


class PrepRun:
    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        self.X, self.W, self.g = (t.cuda() for t in make_prep_inputs(cfg, seed=seed, device="cpu"))
        self.Wp = torch.empty_like(self.W)
        fsa.fsa_prep_pack_weights(self.W, self.g, self.Wp, cfg.H, cfg.d)
        shape = fsa.make_shape(cfg.B, cfg.H, cfg.F, cfg.T, cfg.d, cfg.window, cfg.ref_frame,
                               0, 0, fsa.FSA_BF16)
        self.plan = fsa.fsa_plan_create(shape)
        self.ws = torch.zeros(fsa.fsa_workspace_bytes(self.plan), dtype=torch.uint8,
                              device="cuda")
        qshape = (cfg.B, cfg.H, cfg.N, cfg.d)
        self.Q, self.K, self.V = (torch.full(qshape, float("nan"), dtype=torch.bfloat16,
                                             device="cuda") for _ in range(3))

    def prep(self):
        Hg, Wg = self.cfg.grid
        fsa.fsa_prep(self.plan, Hg, Wg, self.X, self.Wp, self.Q, self.K, self.V, self.ws)
        return self

    def bounds(self):
        fsa.fsa_bounds_after_prep(self.plan, self.K, self.ws, self.cfg.scale)
        torch.cuda.synchronize()
        return self

    def oracle_rows(self, b, rows):
        Hg, Wg = self.cfg.grid
        c = self.cfg
        return prp.prep_rows(to_f64(self.X), to_f64(self.W), self.g.double().cpu().numpy(),
                             c.F, Hg, Wg, c.H, c.d, b, rows)


def check_outputs(run, b, rows, what):
    cfg = run.cfg
    Hg, Wg = cfg.grid
    want = run.oracle_rows(b, rows)
    # S: what the bf16 rounding of the folded weights can move each output by
    xh = prp.rms_norm(to_f64(run.X[b][rows]), run.g.double().cpu().numpy())
    S = np.abs(to_f64(run.W)) @ np.abs(xh).T                  # [3C, n]
    C, d = cfg.H * cfg.d, cfg.d
    for part, (name, got, w) in enumerate(zip("QKV", (run.Q, run.K, run.V), want)):
        g = got[b][:, rows].double().cpu().numpy()
        assert np.isfinite(g).all(), (what, name)
        s = S[part * C:(part + 1) * C].T.reshape(len(rows), cfg.H, d).transpose(1, 0, 2)
        if part < 2:            # a rotated pair mixes its two source channels
            s = np.repeat(s[..., 0::2] + s[..., 1::2], 2, axis=-1)
        err = np.abs(g - w)
        bound = 2.0 ** -9 * (np.abs(w) + s) + 1e-4
        assert np.all(err <= bound), (what, name, float(err.max()), float((err - bound).max()))
        assert err.mean() <= 3e-3, (what, name, float(err.mean()))
        print(f"{what} {name}: max {err.max():.3g} mean {err.mean():.3g} "
              f"(worst err/bound {float((err / bound).max()):.3f})")


def check_stats_and_bounds(run, heads, margin=True):
    """margin: the inputs are drawn to keep each head's statistic at least 5%
    from the threshold, and that is asserted; otherwise the flag is compared
    only where the statistic is more than 1e-4 (relative) from it."""
    cfg = run.cfg
    v = fsa.workspace_views(run.plan, run.ws)
    for b in range(cfg.B):
        for h in heads:
            q = to_f64(run.Q[b, h])
            k = to_f64(run.K[b, h])
            # the producer's row norms and key mean, against its own bf16 outputs
            qn = v["qnorm"][b, h].double().cpu().numpy()
            assert np.allclose(qn, np.linalg.norm(q, axis=1), rtol=1e-5, atol=1e-6), (b, h)
            mu = v["mu"][b, h].double().cpu().numpy()
            assert np.max(np.abs(mu - k.mean(axis=0))) < 1e-5, (b, h)
            want = orc.bounds(q[None, None], k[None, None], cfg.F, cfg.T, cfg.window,
                              cfg.ref_frame, cfg.scale)
            rtol = 1e-5
            assert np.allclose(v["rframe"][b, h].double().cpu().numpy(), want["R"][0, 0], rtol=rtol)
            assert np.allclose(v["rslice"][b, h].double().cpu().numpy(), want["R_S"][0, 0],
                               rtol=rtol)
            assert float(v["stat"][b, h]) == pytest.approx(want["stat"][0, 0], rel=rtol)
            gap = abs(want["stat"][0, 0] - orc.BETA) / orc.BETA
            if margin:
                assert gap > 0.05
            if gap > 1e-4:
                assert int(v["elig"][b, h]) == int(want["elig"][0, 0]), (b, h)
            assert np.array_equal(v["eligf"][b, h].cpu().numpy().astype(bool),
                                  want["elig_frame"][0, 0])
            gb = orc.gap_bounds(q[None, None], k[None, None], cfg.F, cfg.T, cfg.window,
                                cfg.ref_frame, cfg.scale)
            ds = v["dslice"][b, h].double().cpu().numpy()
            assert np.max(np.abs(ds - gb["dslice"][0, 0])) < 1e-4, (b, h)


def test_prep_small_full():
    cfg = CONFIGS["prep-small"]
    say("prep", cfg.name)
    run = PrepRun(cfg).prep().bounds()
    check_outputs(run, 0, np.arange(cfg.N), cfg.name)
    check_stats_and_bounds(run, range(cfg.H))


def test_prep_feeds_the_attention():
    """The producer's outputs, its bounds and the forward kernel in a row,
    against the oracle attention on the same tensors; and the same workspace
    products as fsa_bounds computes from Q and K directly."""
    cfg = CONFIGS["prep-small"]
    say("prep -> attention", cfg.name)
    run = PrepRun(cfg).prep().bounds()
    O = torch.empty_like(run.Q)
    fsa.fsa_forward(run.plan, run.Q, run.K, run.V, O, run.ws, cfg.scale, "auto")
    torch.cuda.synchronize()
    O_rows = torch.empty_like(run.Q)          # the row-block route reads the slice offsets
    fsa.fsa_forward(run.plan, run.Q, run.K, run.V, O_rows, run.ws, cfg.scale, "auto_rows")
    torch.cuda.synchronize()
    for h in range(cfg.H):
        rows = sample_rows(cfg, 200, seed=h)
        want = oracle_rows(cfg, run.Q, run.K, run.V, 0, h, rows)
        assert_close(cfg, O[0, h, rows], want, f"prep->attention head {h}")
        assert_close(cfg, O_rows[0, h, rows], want, f"prep->attention auto_rows head {h}")
    ws2 = torch.zeros_like(run.ws)
    fsa.fsa_bounds(run.plan, run.Q, run.K, ws2, cfg.scale)
    torch.cuda.synchronize()
    a = fsa.workspace_views(run.plan, run.ws)
    c = fsa.workspace_views(run.plan, ws2)
    assert torch.equal(a["qnorm"], c["qnorm"]) or \
        float((a["qnorm"] - c["qnorm"]).abs().max()) < 1e-5
    for k in ("mu", "rframe", "rslice", "stat", "statf"):
        assert torch.allclose(a[k], c[k], rtol=1e-5, atol=1e-6), k
    # slice mean minus mu: the two routes take mu from different sum orders
    assert float((a["dslice"] - c["dslice"]).abs().max()) < 1e-5
    for k in ("elig", "eligf"):
        assert torch.equal(a[k], c[k]), k


def test_prep_720p_sampled():
    """The SR layer that feeds the 720p attention (C = 3072), in the launch
    configuration the benchmark times: sampled tokens of every frame against
    the oracle, and the statistics of three heads."""
    cfg = CONFIGS["720p-prep"]
    say("prep", cfg.name)
    run = PrepRun(cfg).prep().bounds()
    rows = sample_rows(cfg, 120, seed=7)
    check_outputs(run, 0, rows, cfg.name)
    check_stats_and_bounds(run, [0, 11, 23])


PREP_EDGE = [
    # name, F, Hg, Wg, H, B
    ("one-head", 3, 4, 12, 1, 1),          # T = 48, N = 144: a 16-token tail tile
    ("tiny-frames", 5, 4, 4, 2, 1),        # T = 16: many frames per tile
    ("batch-2", 2, 8, 10, 2, 2),           # N = 160 per batch
    ("exact-tiles", 2, 8, 16, 3, 1),       # N = 256: no tail
]


@pytest.mark.parametrize("case", PREP_EDGE, ids=[c[0] for c in PREP_EDGE])
def test_prep_edge_shapes(case):
    name, F, Hg, Wg, H, B = case
    cfg = CONFIGS["prep-small"].with_(name=name, F=F, T=Hg * Wg, H=H, B=B, grid=(Hg, Wg),
                                      window=1)
    say("prep edge", case)
    run = PrepRun(cfg).prep().bounds()
    for b in range(B):
        check_outputs(run, b, np.arange(cfg.N), f"{name} b{b}")
    check_stats_and_bounds(run, range(H))


def test_prep_is_deterministic():
    cfg = CONFIGS["prep-small"]
    say("prep determinism")
    a = PrepRun(cfg).prep().bounds()
    b = PrepRun(cfg).prep().bounds()
    for x, y in ((a.Q, b.Q), (a.K, b.K), (a.V, b.V), (a.ws, b.ws)):
        assert torch.equal(x, y)


def draw_prep_case(i: int):
    """Seeded random producer shape: T = Hg * Wg a multiple of 16."""
    rng = np.random.default_rng(2000 + i)
    while True:
        Hg, Wg = int(rng.integers(1, 13)), int(rng.integers(1, 33))
        if (Hg * Wg) % 16 == 0 and Hg * Wg <= 320:
            break
    F = int(rng.integers(1, 6))
    return dict(F=F, Hg=Hg, Wg=Wg, H=int(rng.integers(1, 5)), B=int(rng.integers(1, 3)),
                window=int(rng.integers(1, 3)), ref=int(rng.integers(0, F)))


# FSA_PREP_FUZZ_CASES widens the sweep for a one-off run
N_PREP_CASES = int(os.environ.get("FSA_PREP_FUZZ_CASES", "8"))


@pytest.mark.parametrize("i", range(N_PREP_CASES))
def test_prep_random_shapes(i):
    """Random grids, frame counts, head counts (an odd head count leaves a
    workgroup's second head empty), batches, windows and reference frames:
    every output within its rounding bound, and the statistics and flags as
    for fsa_bounds."""
    c = draw_prep_case(i)
    cfg = CONFIGS["prep-small"].with_(name=f"prep-fuzz{i}", F=c["F"], T=c["Hg"] * c["Wg"],
                                      H=c["H"], B=c["B"], grid=(c["Hg"], c["Wg"]),
                                      window=c["window"], ref_frame=c["ref"])
    say("prep fuzz", i, c)
    run = PrepRun(cfg, seed=i).prep().bounds()
    for b in range(cfg.B):
        check_outputs(run, b, np.arange(cfg.N), f"prep fuzz {i} b{b}")
    check_stats_and_bounds(run, range(cfg.H), margin=False)
