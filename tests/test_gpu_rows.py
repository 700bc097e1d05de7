"""Route per block of query rows (FSA_MODE_AUTO_ROWS) vs the fp64 oracle (GPU).

A row's gap bound G_i = B_i - scale q_i.(mean key of its slice - mu) bounds
how far the fixed max lies above its true max (oracle: gap_bounds). Under
AUTO_ROWS each workgroup of the bf16 kernel (a block of 256 or 128
consecutive rows of one frame, fsa_plan_row_block; both geometries are
tested) takes the fixed max iff all its rows have G_i <= 64; the fp32
kernel decides row by row. Checks: the slice offsets the bounds write
(dslice) against the oracle; every block whose oracle gap bound is clear of
the limit by 0.1% is bit-identical to FIXED_ONLY (below) or ONLINE_ONLY
(above); outputs meet the usual bar against the oracle (bf16 max-abs 2e-2,
mean-abs 2e-3; fp32 max-abs 1e-5).
"""
import numpy as np
import pytest
import torch

from oracle import fsa_oracle as orc
from frame_aligned_block_amd import fsa
from frame_aligned_block_amd.inputs import CONFIGS, to_f64

from gpu_util import Run, assert_close, oracle_cross_rows, oracle_rows, sample_rows, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU too; every test here is gpu-marked
    pytest.skip("no GPU", allow_module_level=True)

ROW_BLOCKS = (128, 256)  # rows per workgroup of the bf16 kernel: 4 or 8 waves of 32 rows
CLEAR = 1e-3           # relative distance from the limit below which a block is not judged


def row_blocks(T: int, F: int, size: int):
    """(frame, first row, end row) of every row block, frame by frame."""
    for f in range(F):
        for b0 in range(0, T, size):
            yield f, f * T + b0, f * T + min(b0 + size, T)


def check_blocks(cfg, gap, O_rows, O_fix, O_onl, h, size):
    """Each block clear of the limit is bit-identical to the route its oracle
    gap bound picks. Returns (fixed blocks, online blocks)."""
    n_fix = n_onl = 0
    for f, a, e in row_blocks(cfg.T, cfg.F, size):
        g = gap[a:e].max()
        if g < orc.GAP_LIMIT * (1 - CLEAR):
            assert torch.equal(O_rows[0, h, a:e], O_fix[0, h, a:e]), (h, f, a, g)
            n_fix += 1
        elif g > orc.GAP_LIMIT * (1 + CLEAR):
            assert torch.equal(O_rows[0, h, a:e], O_onl[0, h, a:e]), (h, f, a, g)
            n_onl += 1
    return n_fix, n_onl


def test_slice_offsets_parity():
    """dslice (mean key of each frame's slice minus mu) against the oracle."""
    cfg = CONFIGS["loose-rows-small"]
    say("slice offsets", cfg.name)
    run = Run(cfg).bounds()
    torch.cuda.synchronize()
    ds = run.views()["dslice"]
    for h in range(cfg.H):
        q = to_f64(run.Q[0, h])[None, None]
        k = to_f64(run.K[0, h])[None, None]
        want = orc.gap_bounds(q, k, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
        got = ds[0, h].double().cpu().numpy()
        assert np.max(np.abs(got - want["dslice"][0, 0])) < 1e-4, h


@pytest.mark.parametrize("row_block", ROW_BLOCKS)
def test_auto_rows_small(row_block):
    """The looser small workload: the per-head and per-frame checks send every
    head online; AUTO_ROWS keeps the blocks outside each frame's hot band on
    the fixed max, bit-identically to FIXED_ONLY, and the blocks of the band
    online, bit-identically to ONLINE_ONLY; every row meets the bar."""
    cfg = CONFIGS["loose-rows-small"]
    say("auto_rows", cfg.name, row_block)
    run = Run(cfg, row_block=row_block).bounds()
    assert run.row_block == row_block
    torch.cuda.synchronize()
    v = run.views()
    assert not v["elig"].any() and not v["eligf"].any()
    O_rows = run.forward("auto_rows")
    O_fix = run.forward("fixed")
    O_onl = run.forward("online")
    tot_fix = tot_onl = 0
    for h in range(cfg.H):
        q = to_f64(run.Q[0, h])[None, None]
        k = to_f64(run.K[0, h])[None, None]
        gap = orc.gap_bounds(q, k, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)["gap"][0, 0]
        n_fix, n_onl = check_blocks(cfg, gap, O_rows, O_fix, O_onl, h, run.row_block)
        tot_fix += n_fix
        tot_onl += n_onl
        want = oracle_rows(cfg, run.Q, run.K, run.V, 0, h, np.arange(cfg.N))
        mx, mean = assert_close(cfg, O_rows[0, h], want, f"auto_rows head {h}")
        print(f"auto_rows h{h}: {n_fix} fixed / {n_onl} online blocks, max {mx:.3g} mean {mean:.3g}")
    assert tot_fix > 0 and tot_onl > 0


@pytest.mark.parametrize("row_block", ROW_BLOCKS)
def test_auto_rows_720p_shape_sampled(row_block):
    """The 720p-shaped looser workload (128-row blocks: the launch
    configuration the benchmark times; and 256-row blocks): decisions of two
    heads block by block, sampled rows against the oracle."""
    cfg = CONFIGS["loose-rows"]
    say("auto_rows", cfg.name, row_block)
    run = Run(cfg, row_block=row_block).bounds()
    O_rows = run.forward("auto_rows")
    O_fix = run.forward("fixed")
    O_onl = run.forward("online")
    for h in (0, 17):
        q = to_f64(run.Q[0, h])[None, None]
        k = to_f64(run.K[0, h])[None, None]
        gap = orc.gap_bounds(q, k, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)["gap"][0, 0]
        n_fix, n_onl = check_blocks(cfg, gap, O_rows, O_fix, O_onl, h, run.row_block)
        assert n_fix > 0.8 * (n_fix + n_onl), (h, n_fix, n_onl)
        rows = sample_rows(cfg, 200, seed=h)
        want = oracle_rows(cfg, run.Q, run.K, run.V, 0, h, rows)
        mx, mean = assert_close(cfg, O_rows[0, h, rows], want, f"auto_rows 720p head {h}")
        print(f"auto_rows 720p h{h}: {n_fix} fixed / {n_onl} online, max {mx:.3g} mean {mean:.3g}")


@pytest.mark.parametrize("row_block", ROW_BLOCKS)
def test_auto_rows_stress_keeps_the_loose_head_online(row_block):
    """On a stress-like workload the loose head's rows all have gap bounds far
    beyond the limit (its outlier keys are in every slice): every block of it
    is online; the other heads are fixed throughout."""
    cfg = CONFIGS["stress"].with_(F=6, T=720, H=3, loose_period=3, loose_phase=1)
    say("auto_rows stress-like", cfg.name, row_block)
    run = Run(cfg, row_block=row_block).bounds()
    O_rows = run.forward("auto_rows")
    O_fix = run.forward("fixed")
    O_onl = run.forward("online")
    for h in range(cfg.H):
        q = to_f64(run.Q[0, h])[None, None]
        k = to_f64(run.K[0, h])[None, None]
        gap = orc.gap_bounds(q, k, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)["gap"][0, 0]
        n_fix, n_onl = check_blocks(cfg, gap, O_rows, O_fix, O_onl, h, run.row_block)
        nblk = cfg.F * ((cfg.T + run.row_block - 1) // run.row_block)
        assert (n_onl if cfg.is_loose(h) else n_fix) == nblk, (h, n_fix, n_onl)
        rows = sample_rows(cfg, 100, seed=h)
        want = oracle_rows(cfg, run.Q, run.K, run.V, 0, h, rows)
        assert_close(cfg, O_rows[0, h, rows], want, f"auto_rows stress-like head {h}")


def test_auto_rows_fp32_row_by_row():
    """fp32 kernel: one row per thread, so the route is per row: rows clear of
    the limit match FIXED_ONLY or ONLINE_ONLY bit for bit, and the whole output
    meets the fp32 bar."""
    cfg = CONFIGS["tiny"].with_(shared_mean=True, key_sigma=3.0, hot_rows=8, hot_scale=3.0)
    say("auto_rows fp32", cfg.name)
    run = Run(cfg).bounds()
    O_rows = run.forward("auto_rows")
    O_fix = run.forward("fixed")
    O_onl = run.forward("online")
    Q, K, V = (to_f64(t) for t in (run.Q, run.K, run.V))
    want = orc.attention(Q, K, V, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
    assert_close(cfg, O_rows, want, "auto_rows fp32")
    g = orc.gap_bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)["gap"]
    n_fix = n_onl = 0
    for h in range(cfg.H):
        for i in range(cfg.N):
            if g[0, h, i] < orc.GAP_LIMIT * (1 - CLEAR):
                assert torch.equal(O_rows[0, h, i], O_fix[0, h, i]), (h, i)
                n_fix += 1
            elif g[0, h, i] > orc.GAP_LIMIT * (1 + CLEAR):
                assert torch.equal(O_rows[0, h, i], O_onl[0, h, i]), (h, i)
                n_onl += 1
    assert n_fix > 0 and n_onl > 0, (n_fix, n_onl)


def test_auto_rows_cross():
    """Cross-attention: the slice is the whole reference set, so the gap bound
    is the row's bound; the loose head (a x20 reference key) goes online
    block by block, the others stay fixed; outputs meet the bar."""
    cfg = CONFIGS["xref-small"]
    say("auto_rows cross", cfg.name)
    run = Run(cfg).bounds()
    torch.cuda.synchronize()
    ds = run.views()["dslice"]
    assert float(ds.abs().max()) < 1e-4         # the set's mean minus its own mean
    O_rows = run.forward("auto_rows")
    O_fix = run.forward("fixed")
    O_onl = run.forward("online")
    for h in range(cfg.H):
        q = to_f64(run.Q[0, h])[None, None]
        k = to_f64(run.K[0, h])[None, None]
        gap = orc.cross_bounds(q, k, cfg.F, cfg.T, cfg.scale)["gap"][0, 0]
        n_fix, n_onl = check_blocks(cfg, gap, O_rows, O_fix, O_onl, h, run.row_block)
        if cfg.is_loose(h):
            assert n_fix == 0 and n_onl > 0, h
        rows = sample_rows(cfg, 150, seed=h)
        want = oracle_cross_rows(cfg, run.Q, run.K, run.V, 0, h, rows)
        assert_close(cfg, O_rows[0, h, rows], want, f"auto_rows cross head {h}")


@pytest.mark.parametrize("row_block", ROW_BLOCKS)
@pytest.mark.parametrize("name,kw", [
    ("d64", dict(d=64)),
    ("batch-2", dict(B=2)),
    ("short-frames", dict(T=144, hot_rows=16)),   # frames shorter than one block
])
def test_auto_rows_edge_shapes(name, kw, row_block):
    """AUTO_ROWS on other shapes: d = 64, two batches, frames shorter than
    one block, in both workgroup geometries. Blocks clear of the limit match
    FIXED_ONLY or ONLINE_ONLY bit for bit; all rows meet the bar."""
    cfg = CONFIGS["loose-rows-small"].with_(**kw)
    say("auto_rows edge", name, row_block)
    run = Run(cfg, row_block=row_block).bounds()
    block = run.row_block
    O_rows = run.forward("auto_rows")
    O_fix = run.forward("fixed")
    O_onl = run.forward("online")
    n_fix = n_onl = 0
    for b in range(cfg.B):
        for h in range(cfg.H):
            q = to_f64(run.Q[b, h])[None, None]
            k = to_f64(run.K[b, h])[None, None]
            gap = orc.gap_bounds(q, k, cfg.F, cfg.T, cfg.window, cfg.ref_frame,
                                 cfg.scale)["gap"][0, 0]
            for f, a, e in row_blocks(cfg.T, cfg.F, block):
                g = gap[a:e].max()
                if g < orc.GAP_LIMIT * (1 - CLEAR):
                    assert torch.equal(O_rows[b, h, a:e], O_fix[b, h, a:e]), (b, h, f, a)
                    n_fix += 1
                elif g > orc.GAP_LIMIT * (1 + CLEAR):
                    assert torch.equal(O_rows[b, h, a:e], O_onl[b, h, a:e]), (b, h, f, a)
                    n_onl += 1
            rows = sample_rows(cfg, 100, seed=h)
            want = oracle_rows(cfg, run.Q, run.K, run.V, b, h, rows)
            assert_close(cfg, O_rows[b, h, rows], want, f"auto_rows {name} b{b} h{h}")
    # a block that covers a whole frame holds that frame's hot rows, so only
    # frames of several blocks can keep some of them on the fixed max
    assert n_onl > 0 and (n_fix > 0 or block >= cfg.T), (n_fix, n_onl)
