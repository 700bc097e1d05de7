"""The C ABI without a GPU: exported symbols and synchronous argument errors."""
import os
import re

import pytest

from frame_aligned_block_amd import fsa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    L = fsa.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(fsa.EXPORTS) == names


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    for name in ("FSA_ELIG_BETA", "FSA_GAP_LIMIT", "FSA_SCALED_LIMIT", "FSA_MAX_FRAMES"):
        m = re.search(r"#define\s+%s\s+([0-9.]+)f?\b" % name, text)
        assert m, name
        assert float(getattr(fsa, name)) == float(m.group(1)), name
    m = re.search(r"#define\s+FSA_STATIC_WS_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and fsa.FSA_STATIC_WS_BYTES == int(m.group(1)) << int(m.group(2))


def test_status_strings():
    assert fsa.fsa_status_string(0) == "FSA_OK"
    assert fsa.fsa_status_string(-3) == "FSA_ERR_WORKSPACE"


def shape(**kw):
    base = dict(B=1, H=2, F=5, T=48, d=64, window=1, ref_frame=0, bq=0, bk=0, dtype=fsa.FSA_F32)
    base.update(kw)
    return fsa.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=40), fsa.FSA_ERR_UNSUPPORTED),          # T % 16 != 0
    (dict(d=96), fsa.FSA_ERR_UNSUPPORTED),
    (dict(F=256), fsa.FSA_ERR_UNSUPPORTED),
    (dict(ref_frame=5), fsa.FSA_ERR_INVALID_ARG),
    (dict(ref_frame=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(window=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(B=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(bq=32), fsa.FSA_ERR_INVALID_ARG),         # does not divide 48
    (dict(bk=24), fsa.FSA_ERR_INVALID_ARG),         # not a multiple of 16
    (dict(dtype=7), fsa.FSA_ERR_INVALID_ARG),
    (dict(H=40000, T=3600, F=13, d=128), fsa.FSA_ERR_UNSUPPORTED),   # > 2^31 elements
])
def test_plan_create_errors(kw, status):
    with pytest.raises(fsa.FsaError) as e:
        fsa.fsa_plan_create(shape(**kw))
    assert e.value.status == status
    assert fsa.fsa_last_error()


FAKE = 0x10000   # a 256-aligned address; never dereferenced: calls fail validation first


def test_bounds_and_forward_validate_before_launch():
    p = fsa.fsa_plan_create(shape())
    cases = [
        (lambda: fsa.fsa_bounds(p, None, FAKE, FAKE, 0.125, 0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_bounds(p, FAKE, FAKE, FAKE, 0.0, 0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_bounds(p, FAKE, FAKE, FAKE, float("nan"), 0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_bounds(p, FAKE + 8, FAKE, FAKE, 0.125, 0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_bounds(p, FAKE, FAKE, None, 0.125, 0), fsa.FSA_ERR_WORKSPACE),
        (lambda: fsa.fsa_bounds(p, FAKE, FAKE, FAKE + 16, 0.125, 0), fsa.FSA_ERR_WORKSPACE),
        (lambda: fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE, None, FAKE, 0.125, 0, 0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE, FAKE * 64, FAKE * 128, 0.125, 9, 0),
         fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE, FAKE * 64, FAKE * 128, -1.0, 0, 0),
         fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_forward(p, FAKE, None, FAKE, FAKE * 64, FAKE * 128, 0.125, 0, 0),
         fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE, FAKE * 32, FAKE * 128, 0.125, 0, 0),
         fsa.FSA_ERR_INVALID_ARG),     # O == K
        # O aliasing Q / the workspace
        (lambda: fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE * 64, FAKE + 256, FAKE * 128, 0.125, 0, 0),
         fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE * 64, FAKE * 128, FAKE * 128, 0.125, 0, 0),
         fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_copy_eligibility(p, None, 0), fsa.FSA_ERR_WORKSPACE),
        (lambda: fsa.fsa_copy_eligibility(p, FAKE + 16, 0), fsa.FSA_ERR_WORKSPACE),
        (lambda: fsa._check(fsa.lib().fsa_copy_eligibility(p, FAKE, None, None)),
         fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa._check(fsa.lib().fsa_copy_eligibility(None, FAKE, FAKE, None)),
         fsa.FSA_ERR_INVALID_ARG),
    ]
    for call, status in cases:
        with pytest.raises(fsa.FsaError) as e:
            call()
        assert e.value.status == status, fsa.fsa_last_error()


def test_attention_validates_before_launch():
    F, T, w, r, B, H, d = 5, 48, 1, 0, 1, 2, 64
    need = fsa.fsa_attention_workspace_bytes(F, T, w, r, B, H, d, fsa.FSA_F32)
    # the row norms and per-part sums, far less than one [B,H,N,d] tensor
    assert B * H * F * T * 4 < need < B * H * F * T * d * 4
    base = [FAKE, FAKE * 64, FAKE * 128, FAKE * 256, F, T, w, r, 0.125, B, H, d, fsa.FSA_F32,
            0, FAKE * 512, need]
    def call(**over):
        args = list(base)
        names = ["Q", "K", "V", "O", "F", "T", "window", "ref_frame", "scale", "B", "H", "d",
                 "dtype", "mode", "ws", "ws_bytes"]
        for k, v in over.items():
            args[names.index(k)] = v
        fsa.fsa_attention(*args, stream=0)
    for over, status in [
        (dict(ws_bytes=need - 1), fsa.FSA_ERR_WORKSPACE),
        (dict(ws=None), fsa.FSA_ERR_WORKSPACE),
        (dict(ws=FAKE * 512 + 64), fsa.FSA_ERR_WORKSPACE),
        (dict(T=40), fsa.FSA_ERR_UNSUPPORTED),
        (dict(d=32), fsa.FSA_ERR_UNSUPPORTED),
        (dict(ref_frame=9), fsa.FSA_ERR_INVALID_ARG),
        (dict(scale=float("inf")), fsa.FSA_ERR_INVALID_ARG),
        (dict(mode=5), fsa.FSA_ERR_INVALID_ARG),
        (dict(mode=-1), fsa.FSA_ERR_INVALID_ARG),
        (dict(O=FAKE * 64), fsa.FSA_ERR_INVALID_ARG),        # O == K
        (dict(V=None), fsa.FSA_ERR_INVALID_ARG),
    ]:
        with pytest.raises(fsa.FsaError) as e:
            call(**over)
        assert e.value.status == status, (over, fsa.fsa_last_error())
    fsa.fsa_cache_clear()


@pytest.mark.parametrize("kw,M,status", [
    (dict(), 0, fsa.FSA_ERR_INVALID_ARG),
    (dict(), -16, fsa.FSA_ERR_INVALID_ARG),
    (dict(), 40, fsa.FSA_ERR_UNSUPPORTED),           # M % 16 != 0
    (dict(window=1), 64, fsa.FSA_ERR_INVALID_ARG),    # no window in cross-attention
    (dict(ref_frame=1), 64, fsa.FSA_ERR_INVALID_ARG),
    (dict(bk=32), 48, fsa.FSA_ERR_INVALID_ARG),       # 32 does not divide M = 48
    (dict(bk=32), 96, None),                          # 32 divides M = 96, though not T = 48
    (dict(T=40), 64, fsa.FSA_ERR_UNSUPPORTED),
    (dict(H=2000, d=128), 1 << 20, fsa.FSA_ERR_UNSUPPORTED),   # > 2^31 key elements
])
def test_cross_plan_create_errors(kw, M, status):
    base = dict(window=0)
    base.update(kw)
    if status is None:
        p = fsa.fsa_plan_create_cross(shape(**base), M)
        assert fsa.fsa_plan_shape(p).bk == kw["bk"]
        return
    with pytest.raises(fsa.FsaError) as e:
        fsa.fsa_plan_create_cross(shape(**base), M)
    assert e.value.status == status
    assert fsa.fsa_last_error()


def test_cross_attention_validates_before_launch():
    F, T, M, B, H, d = 5, 48, 720, 1, 2, 64
    need = fsa.fsa_cross_attention_workspace_bytes(F, T, M, B, H, d, fsa.FSA_F32)
    assert B * H * F * T * 4 < need < B * H * F * T * d * 4
    names = ["Q", "Kr", "Vr", "O", "F", "T", "M", "scale", "B", "H", "d", "dtype", "mode",
             "ws", "ws_bytes"]
    base = [FAKE, FAKE * 64, FAKE * 128, FAKE * 256, F, T, M, 0.125, B, H, d, fsa.FSA_F32, 0,
            FAKE * 512, need]

    def call(**over):
        args = list(base)
        for k, v in over.items():
            args[names.index(k)] = v
        fsa.fsa_cross_attention(*args, stream=0)
    kv = B * H * M * d * 4
    for over, status in [
        (dict(ws_bytes=need - 1), fsa.FSA_ERR_WORKSPACE),
        (dict(ws=None), fsa.FSA_ERR_WORKSPACE),
        (dict(M=0), fsa.FSA_ERR_INVALID_ARG),
        (dict(M=24), fsa.FSA_ERR_UNSUPPORTED),
        (dict(T=40), fsa.FSA_ERR_UNSUPPORTED),
        (dict(scale=0.0), fsa.FSA_ERR_INVALID_ARG),
        (dict(mode=7), fsa.FSA_ERR_INVALID_ARG),
        (dict(Vr=None), fsa.FSA_ERR_INVALID_ARG),
        (dict(O=FAKE * 64 + kv - 256), fsa.FSA_ERR_INVALID_ARG),   # O overlaps the end of Kr
    ]:
        with pytest.raises(fsa.FsaError) as e:
            call(**over)
        assert e.value.status == status, (over, fsa.fsa_last_error())
    with pytest.raises(fsa.FsaError):
        fsa.fsa_cross_attention_workspace_bytes(F, T, 0, B, H, d, fsa.FSA_F32)
    fsa.fsa_cache_clear()


def test_prep_validates_before_launch():
    F, T, H, d = 3, 48, 2, 128
    p = fsa.fsa_plan_create(fsa.make_shape(1, H, F, T, d, 1, 0, 0, 0, fsa.FSA_BF16))
    nb = 1 * H * F * T * d * 2
    wb = fsa.fsa_prep_weight_bytes(H, d)
    assert wb == 3 * (H * d) ** 2 * 2
    X, Wp, Q, K, V, ws = (FAKE * (1 << i) for i in range(6, 12))
    ok = dict(grid_h=4, grid_w=12, X=X, Wp=Wp, Q=Q, K=K, V=V, ws=ws)

    def call(plan=p, **over):
        a = dict(ok)
        a.update(over)
        fsa.fsa_prep(plan, a["grid_h"], a["grid_w"], a["X"], a["Wp"], a["Q"], a["K"], a["V"],
                     a["ws"], stream=0)
    cross = fsa.fsa_plan_create_cross(fsa.make_shape(1, H, F, T, d, 0, 0, 0, 0, fsa.FSA_BF16), 64)
    d64 = fsa.fsa_plan_create(fsa.make_shape(1, H, F, T, 64, 1, 0, 0, 0, fsa.FSA_BF16))
    for over, status in [
        (dict(grid_w=10), fsa.FSA_ERR_INVALID_ARG),          # 4 x 10 != 48
        (dict(X=None), fsa.FSA_ERR_INVALID_ARG),
        (dict(Q=Q + 8), fsa.FSA_ERR_INVALID_ARG),             # misaligned
        (dict(K=Q + nb // 2), fsa.FSA_ERR_INVALID_ARG),       # K overlaps Q
        (dict(V=X), fsa.FSA_ERR_INVALID_ARG),                 # V overlaps X
        (dict(ws=None), fsa.FSA_ERR_WORKSPACE),
        (dict(plan=cross), fsa.FSA_ERR_UNSUPPORTED),
        (dict(plan=d64), fsa.FSA_ERR_UNSUPPORTED),
    ]:
        with pytest.raises(fsa.FsaError) as e:
            call(**over)
        assert e.value.status == status, (over, fsa.fsa_last_error())
    for fn, status in [
        (lambda: fsa.fsa_bounds_after_prep(p, None, ws, 0.1, stream=0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_bounds_after_prep(p, K, ws, 0.0, stream=0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_bounds_after_prep(p, K, ws + 16, 0.1, stream=0), fsa.FSA_ERR_WORKSPACE),
        (lambda: fsa.fsa_bounds_after_prep(cross, K, ws, 0.1, stream=0), fsa.FSA_ERR_UNSUPPORTED),
        (lambda: fsa.fsa_prep_pack_weights(None, FAKE, Wp, H, d, stream=0), fsa.FSA_ERR_INVALID_ARG),
        (lambda: fsa.fsa_prep_pack_weights(X, FAKE, Wp, H, 64, stream=0), fsa.FSA_ERR_UNSUPPORTED),
        (lambda: fsa.fsa_prep_pack_weights(X, FAKE, X + 64, H, d, stream=0), fsa.FSA_ERR_INVALID_ARG),
    ]:
        with pytest.raises(fsa.FsaError) as e:
            fn()
        assert e.value.status == status, fsa.fsa_last_error()


def test_row_block_choice_and_override():
    """The bf16 forward kernel's row block: the plan's own choice, both
    geometries on request, and rejected values; fp32 plans compute a row per
    thread."""
    # 4 waves (128 rows) for every shape; 8 waves (256 rows) on request
    for T in (880, 16, 3600, 8160):
        q = fsa.fsa_plan_create(shape(dtype=fsa.FSA_BF16, d=128, T=T, F=9, H=16, window=2))
        assert fsa.fsa_plan_row_block(q) == 128, T
    p = fsa.fsa_plan_create(shape(dtype=fsa.FSA_BF16, d=128, T=3600, F=13, H=24, window=2))
    assert fsa.fsa_plan_row_block(p) == 128
    fsa.fsa_plan_set_row_block(p, 256)
    assert fsa.fsa_plan_row_block(p) == 256
    fsa.fsa_plan_set_row_block(p, 0)
    assert fsa.fsa_plan_row_block(p) == 128
    for bad in (64, 192, 512, -1):
        with pytest.raises(fsa.FsaError) as e:
            fsa.fsa_plan_set_row_block(p, bad)
        assert e.value.status == fsa.FSA_ERR_INVALID_ARG
    # the tile list does not depend on the kernel's geometry
    before = fsa.fsa_plan_export(p)
    fsa.fsa_plan_set_row_block(p, 256)
    after = fsa.fsa_plan_export(p)
    assert all((before[k] == after[k]).all() for k in ("row_ptr", "col_idx", "qframe", "runs"))
    q = fsa.fsa_plan_create(shape())                 # fp32
    assert fsa.fsa_plan_row_block(q) == 1
    fsa.fsa_plan_set_row_block(q, 0)
    with pytest.raises(fsa.FsaError):
        fsa.fsa_plan_set_row_block(q, 128)
    assert fsa.lib().fsa_plan_row_block(None) == -1


def test_attention_rejects_bad_out_and_workspace():
    """fsa.attention / fsa.cross_attention check a caller-supplied output and
    workspace before anything reaches the C ABI (which cannot see sizes)."""
    import torch
    q = torch.zeros(1, 2, 5 * 48, 64)        # CPU tensors: rejected before any launch
    with pytest.raises(ValueError):
        fsa._check_out_ws(torch.zeros(1, 2, 5 * 48, 32), None, q, 1024)   # wrong shape
    with pytest.raises(ValueError):
        fsa._check_out_ws(torch.zeros_like(q), None, q, 1024)              # not on a GPU
    with pytest.raises(ValueError):
        fsa._check_out_ws(None, torch.zeros(8, dtype=torch.uint8), q, 1024)   # not on a GPU
    fsa._check_out_ws(None, None, q, 1024)                                 # nothing given


def test_attention_rejects_bad_inputs():
    """Inputs must be contiguous CUDA tensors of the stated shapes, one dtype
    and one device; CPU tensors, a wrong shape, dtype or layout are rejected
    before anything reaches the C ABI."""
    import torch
    q = torch.zeros(1, 2, 5 * 48, 64)
    with pytest.raises(ValueError):
        fsa._check_inputs(((q, q.shape),), q, "cpu")                        # not on a GPU
    with pytest.raises(ValueError):
        fsa.attention(q, q, q, F=5, T=48, window=1, ref_frame=0)           # through the wrapper
    with pytest.raises(ValueError):
        fsa.cross_attention(q, q[:, :, :48], q[:, :, :48], F=5, T=48)
    with pytest.raises(ValueError):
        fsa.attention(q, q, q, F=4, T=48, window=1, ref_frame=0)           # N != F*T


def test_record_pmax_flag_validation():
    """FSA_MODE_RECORD_PMAX combines with any route of a bf16 plan; an fp32
    plan rejects it, and unknown mode bits are rejected, before any launch."""
    p = fsa.fsa_plan_create(shape())                  # fp32
    with pytest.raises(fsa.FsaError) as e:
        fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE * 64, FAKE * 96, FAKE * 128, 0.125,
                        fsa.FSA_MODE_AUTO | fsa.FSA_MODE_RECORD_PMAX, 0)
    assert e.value.status == fsa.FSA_ERR_UNSUPPORTED
    for bad in (fsa.FSA_MODE_AUTO | 0x200, 5 | fsa.FSA_MODE_RECORD_PMAX):
        with pytest.raises(fsa.FsaError) as e:
            fsa.fsa_forward(p, FAKE, FAKE * 32, FAKE * 64, FAKE * 96, FAKE * 128, 0.125, bad, 0)
        assert e.value.status == fsa.FSA_ERR_INVALID_ARG
    lay = fsa.fsa_workspace_layout(p)
    assert lay["pmax"] % 256 == 0 and lay["pmax"] + 4 <= lay["total"]
