"""The library's host plan builder against the oracle's plan, bit for bit (CPU).

The plan is host C++ inside libfsa.so, so these run without a GPU.
"""
import numpy as np
import pytest

from oracle import fsa_oracle as orc
from frame_aligned_block_amd import fsa

CASES = [
    # F, T, window, ref, bq, bk
    (5, 48, 1, 0, 16, 16), (5, 48, 1, 0, 48, 16), (5, 48, 1, 0, 16, 48),
    (7, 32, 1, 3, 16, 32), (6, 48, 0, 5, 48, 48), (4, 16, 3, 2, 16, 16),
    (9, 880, 2, 0, 80, 176), (9, 880, 2, 0, 880, 16), (9, 880, 2, 0, 16, 80),
    (13, 3600, 2, 0, 48, 48), (13, 3600, 2, 0, 144, 240), (9, 8160, 1, 0, 48, 96),
    (13, 3600, 2, 12, 240, 400), (10, 64, 2, 4, 32, 64), (1, 16, 0, 0, 16, 16),
    (3, 32, 0, 1, 32, 16), (8, 16, 1, 7, 16, 16), (8, 16, 1, 5, 16, 16),
]


def plan(F, T, w, r, bq, bk, d=128, dtype=fsa.FSA_BF16, B=1, H=1):
    return fsa.fsa_plan_create(fsa.make_shape(B, H, F, T, d, w, r, bq, bk, dtype))


@pytest.mark.parametrize("F,T,w,r,bq,bk", CASES)
def test_plan_bit_exact_vs_oracle(F, T, w, r, bq, bk):
    got = fsa.fsa_plan_export(plan(F, T, w, r, bq, bk))
    want = orc.plan(F, T, w, r, bq, bk)
    assert got["nnz"] == want["nnz"]
    assert np.array_equal(got["row_ptr"], want["row_ptr"])
    assert np.array_equal(got["col_idx"], want["col_idx"])
    assert np.array_equal(got["qframe"], want["qframe"])
    for qb in range(got["n_qblocks"]):
        runs = [tuple(x) for x in want["runs"][qb]]
        flat = [v for rr in runs for v in rr] + [0] * (4 - 2 * len(runs))
        assert list(got["runs"][qb]) == flat


@pytest.mark.parametrize("F,T,w,r,bq,bk", CASES)
def test_valid_pairs(F, T, w, r, bq, bk):
    assert fsa.fsa_plan_valid_pairs(plan(F, T, w, r, bq, bk)) == orc.valid_pairs_per_head(F, T, w, r)


@pytest.mark.parametrize("T,d,bq", [(3600, 128, 48), (8160, 128, 48), (880, 128, 16),
                                    (48, 64, 48), (880, 64, 16), (64, 128, 64)])
def test_auto_block_sizes(T, d, bq):
    s = fsa.fsa_plan_shape(plan(3, T, 1, 0, 0, 0, d=d))
    assert s.bq == bq
    assert s.bk % 16 == 0 and T % s.bk == 0


def test_workspace_layout_is_aligned_and_disjoint():
    p = plan(13, 3600, 2, 0, 0, 0, H=24)
    lay = fsa.fsa_workspace_layout(p)
    B, H, N, d, F = 1, 24, 13 * 3600, 128, 13
    sizes = {"mu": B * H * d * 4, "qnorm": B * H * N * 4,
             "rframe": B * H * F * 4, "rslice": B * H * F * 4, "stat": B * H * 4, "elig": B * H,
             "statf": B * H * F * 4, "eligf": B * H * F, "dslice": B * H * F * d * 4}
    spans = sorted((lay[k], lay[k] + n) for k, n in sizes.items())
    for (a0, e0), (a1, _) in zip(spans, spans[1:]):
        assert e0 <= a1
    assert all(lay[k] % 256 == 0 for k in sizes)
    assert lay["total"] == fsa.fsa_workspace_bytes(p) >= spans[-1][1]


# ------------------------------------------------------------------ cross-attention plans

CROSS = [
    # F, T, M, bq, bk
    (5, 48, 720, 16, 16), (5, 48, 720, 48, 80), (13, 3600, 3600, 48, 144),
    (4, 880, 720, 80, 48), (1, 16, 16, 16, 16), (9, 8160, 48, 96, 48),
]


def cross_plan(F, T, M, bq, bk, d=128, dtype=fsa.FSA_BF16, B=1, H=1):
    return fsa.fsa_plan_create_cross(fsa.make_shape(B, H, F, T, d, 0, 0, bq, bk, dtype), M)


@pytest.mark.parametrize("F,T,M,bq,bk", CROSS)
def test_cross_plan_bit_exact_vs_oracle(F, T, M, bq, bk):
    p = cross_plan(F, T, M, bq, bk)
    got = fsa.fsa_plan_export(p)
    want = orc.cross_plan(F, T, M, bq, bk)
    # closed form: every tile of the (F*T/bq) x (M/bk) grid is live
    assert got["nnz"] == want["nnz"] == (F * T // bq) * (M // bk)
    assert np.array_equal(got["row_ptr"], want["row_ptr"])
    assert np.array_equal(got["col_idx"], want["col_idx"])
    assert np.array_equal(got["qframe"], want["qframe"])
    # the oracle's key runs, in the library's {start0, end0, start1, end1} form
    runs = np.array([[a, e] + [0, 0] * (2 - len(r)) for r in want["runs"] for a, e in r[:1]])
    assert len(want["runs"]) == got["n_qblocks"] and all(len(r) == 1 for r in want["runs"])
    assert np.array_equal(got["runs"], runs)
    assert fsa.fsa_plan_valid_pairs(p) == F * T * M
    assert fsa.fsa_plan_key_tokens(p) == M


def test_key_tokens_of_self_plan():
    assert fsa.fsa_plan_key_tokens(plan(13, 3600, 2, 0, 0, 0)) == 13 * 3600


def test_cross_auto_block_sizes():
    s = fsa.fsa_plan_shape(cross_plan(13, 3600, 720, 0, 0))
    assert s.bq == 48 and s.bk == 48          # 720 = 16 * 45: 48 is the largest <= 64
    s = fsa.fsa_plan_shape(cross_plan(4, 880, 16, 0, 0))
    assert s.bk == 16


def test_cross_workspace_layout():
    H, F, T, M = 24, 13, 3600, 3600
    p = cross_plan(F, T, M, 0, 0, H=H)
    lay = fsa.fsa_workspace_layout(p)
    # one key radius per head (H floats, padded to 256 bytes); per-frame slice
    # radii as for self-attention
    assert lay["rslice"] - lay["rframe"] == 256
    sizes = {"mu": H * 128 * 4, "qnorm": H * F * T * 4, "rframe": H * 4, "rslice": H * F * 4,
             "stat": H * 4, "elig": H, "statf": H * F * 4, "eligf": H * F,
             "dslice": H * F * 128 * 4}
    spans = sorted((lay[k], lay[k] + n) for k, n in sizes.items())
    for (a0, e0), (a1, _) in zip(spans, spans[1:]):
        assert e0 <= a1
    assert lay["total"] == fsa.fsa_workspace_bytes(p) >= spans[-1][1]
