"""ctypes binding of libfsa (include/fsa.h): argument marshalling only.

Every function here has the name of the C entry point it calls and passes
plain pointers and sizes through; all computation happens in the library's
HIP kernels (or, for the plan, its host C++). Tensors are torch tensors on
the GPU, used only as device memory; the stream is torch's current HIP
stream unless one is given.

There is no fallback: if libfsa.so is missing the import of the library
raises, and every call that fails in the library raises FsaError with the
library's own error text.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# FSA_LIBRARY names another build of the same library (the sanitizer build of
# the host code the CPU tests load); the default is the in-tree libfsa.so.
LIB_PATH = os.environ.get("FSA_LIBRARY") or os.path.join(_HERE, "libfsa.so")

FSA_OK = 0
FSA_ERR_INVALID_ARG = -1
FSA_ERR_UNSUPPORTED = -2
FSA_ERR_WORKSPACE = -3
FSA_ERR_HIP = -4
FSA_ERR_NOMEM = -5

FSA_BF16 = 0
FSA_F32 = 1

FSA_MODE_AUTO = 0
FSA_MODE_ONLINE_ONLY = 1
FSA_MODE_FIXED_ONLY = 2
FSA_MODE_AUTO_FRAME = 3
FSA_MODE_AUTO_ROWS = 4
FSA_MODE_RECORD_PMAX = 0x100
MODES = {"auto": FSA_MODE_AUTO, "online": FSA_MODE_ONLINE_ONLY, "fixed": FSA_MODE_FIXED_ONLY,
         "auto_frame": FSA_MODE_AUTO_FRAME, "auto_rows": FSA_MODE_AUTO_ROWS}

FSA_ELIG_BETA = 32.0
FSA_GAP_LIMIT = 64.0
FSA_SCALED_LIMIT = 32.0
FSA_MAX_FRAMES = 255
FSA_STATIC_WS_BYTES = 16 << 20

# Every symbol include/fsa.h declares.
EXPORTS = (
    "fsa_plan_create", "fsa_plan_create_cross", "fsa_plan_destroy", "fsa_plan_shape",
    "fsa_plan_export", "fsa_plan_valid_pairs", "fsa_plan_key_tokens", "fsa_plan_row_block",
    "fsa_plan_set_row_block", "fsa_workspace_bytes",
    "fsa_workspace_layout", "fsa_bounds", "fsa_forward", "fsa_copy_eligibility",
    "fsa_attention", "fsa_attention_workspace_bytes", "fsa_attention_static", "fsa_cross_attention",
    "fsa_cross_attention_workspace_bytes", "fsa_prep_weight_bytes", "fsa_prep_pack_weights",
    "fsa_prep", "fsa_bounds_after_prep",
    "fsa_cache_clear", "fsa_status_string", "fsa_last_error",
)


class fsa_shape(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("B", "H", "F", "T", "d", "window", "ref_frame",
                                        "bq", "bk", "dtype")]


class fsa_ws_layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("mu", "qnorm", "rframe", "rslice", "stat",
                                         "elig", "statf", "eligf", "dslice", "pmax", "total")]


class FsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfsa.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    L.fsa_plan_create.argtypes = [POINTER(fsa_shape), POINTER(P)]
    L.fsa_plan_create.restype = c_int32
    L.fsa_plan_create_cross.argtypes = [POINTER(fsa_shape), c_int32, POINTER(P)]
    L.fsa_plan_create_cross.restype = c_int32
    L.fsa_plan_destroy.argtypes = [P]
    L.fsa_plan_destroy.restype = None
    L.fsa_plan_shape.argtypes = [P, POINTER(fsa_shape)]
    L.fsa_plan_shape.restype = c_int32
    L.fsa_plan_export.argtypes = [P, P, P, P, P, POINTER(c_int32), POINTER(c_int64)]
    L.fsa_plan_export.restype = c_int32
    L.fsa_plan_valid_pairs.argtypes = [P]
    L.fsa_plan_valid_pairs.restype = c_int64
    L.fsa_plan_key_tokens.argtypes = [P]
    L.fsa_plan_key_tokens.restype = c_int64
    L.fsa_plan_row_block.argtypes = [P]
    L.fsa_plan_row_block.restype = c_int32
    L.fsa_plan_set_row_block.argtypes = [P, c_int32]
    L.fsa_plan_set_row_block.restype = c_int32
    L.fsa_workspace_bytes.argtypes = [P]
    L.fsa_workspace_bytes.restype = c_size_t
    L.fsa_workspace_layout.argtypes = [P, POINTER(fsa_ws_layout)]
    L.fsa_workspace_layout.restype = c_int32
    L.fsa_bounds.argtypes = [P, P, P, P, c_float, P]
    L.fsa_bounds.restype = c_int32
    L.fsa_forward.argtypes = [P, P, P, P, P, P, c_float, c_int32, P]
    L.fsa_forward.restype = c_int32
    L.fsa_copy_eligibility.argtypes = [P, P, P, P]
    L.fsa_copy_eligibility.restype = c_int32
    L.fsa_attention.argtypes = [P, P, P, P, c_int32, c_int32, c_int32, c_int32, c_float,
                                c_int32, c_int32, c_int32, c_int32, c_int32, P, c_size_t, P]
    L.fsa_attention.restype = c_int32
    L.fsa_attention_static.argtypes = [P, P, P, P, P, c_float, c_int32, P]
    L.fsa_attention_static.restype = c_int32
    L.fsa_attention_workspace_bytes.argtypes = [c_int32] * 8
    L.fsa_attention_workspace_bytes.restype = c_size_t
    L.fsa_cross_attention.argtypes = [P, P, P, P, c_int32, c_int32, c_int32, c_float, c_int32,
                                      c_int32, c_int32, c_int32, c_int32, P, c_size_t, P]
    L.fsa_cross_attention.restype = c_int32
    L.fsa_cross_attention_workspace_bytes.argtypes = [c_int32] * 7
    L.fsa_cross_attention_workspace_bytes.restype = c_size_t
    L.fsa_prep_weight_bytes.argtypes = [c_int32, c_int32]
    L.fsa_prep_weight_bytes.restype = c_size_t
    L.fsa_prep_pack_weights.argtypes = [P, P, P, c_int32, c_int32, P]
    L.fsa_prep_pack_weights.restype = c_int32
    L.fsa_prep.argtypes = [P, c_int32, c_int32, P, P, P, P, P, P, P]
    L.fsa_prep.restype = c_int32
    L.fsa_bounds_after_prep.argtypes = [P, P, P, c_float, P]
    L.fsa_bounds_after_prep.restype = c_int32
    L.fsa_cache_clear.argtypes = []
    L.fsa_cache_clear.restype = None
    L.fsa_status_string.argtypes = [c_int32]
    L.fsa_status_string.restype = c_char_p
    L.fsa_last_error.argtypes = []
    L.fsa_last_error.restype = c_char_p
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().fsa_status_string(status).decode()
    except Exception:   # noqa: BLE001 - naming only
        return str(status)


def _check(status: int) -> None:
    if status != FSA_OK:
        raise FsaError(status, fsa_last_error())


def fsa_status_string(status: int) -> str:
    return lib().fsa_status_string(status).decode()


def fsa_last_error() -> str:
    return lib().fsa_last_error().decode()


def _ptr(t) -> int | None:
    """Device (or host) address of a tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ plan

class Plan:
    """Owns an fsa_plan handle (host memory). M: reference tokens of a cross
    plan, 0 for self-attention."""

    def __init__(self, handle: int, M: int = 0):
        self.handle = handle
        self.M = M

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.fsa_plan_destroy(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return c_void_p(self.handle)


def make_shape(B, H, F, T, d, window, ref_frame, bq=0, bk=0, dtype=FSA_BF16) -> fsa_shape:
    return fsa_shape(B, H, F, T, d, window, ref_frame, bq, bk, dtype)


def fsa_plan_create(shape: fsa_shape) -> Plan:
    h = c_void_p()
    _check(lib().fsa_plan_create(ctypes.byref(shape), ctypes.byref(h)))
    return Plan(h.value)


def fsa_plan_create_cross(shape: fsa_shape, M: int) -> Plan:
    h = c_void_p()
    _check(lib().fsa_plan_create_cross(ctypes.byref(shape), int(M), ctypes.byref(h)))
    return Plan(h.value, int(M))


def fsa_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        lib().fsa_plan_destroy(plan.handle)
        plan.handle = None


def fsa_plan_shape(plan: Plan) -> fsa_shape:
    s = fsa_shape()
    _check(lib().fsa_plan_shape(plan, ctypes.byref(s)))
    return s


def fsa_plan_export(plan: Plan) -> dict:
    """The tile list as numpy int32 arrays (row_ptr, col_idx, qframe, runs)."""
    L = lib()
    nq = c_int32()
    nnz = c_int64()
    _check(L.fsa_plan_export(plan, None, None, None, None, ctypes.byref(nq), ctypes.byref(nnz)))
    row_ptr = np.zeros(nq.value + 1, np.int32)
    col_idx = np.zeros(nnz.value, np.int32)
    qframe = np.zeros(nq.value, np.int32)
    runs = np.zeros((nq.value, 4), np.int32)
    _check(L.fsa_plan_export(plan, row_ptr.ctypes.data, col_idx.ctypes.data,
                             qframe.ctypes.data, runs.ctypes.data, None, None))
    return {"row_ptr": row_ptr, "col_idx": col_idx, "qframe": qframe, "runs": runs,
            "n_qblocks": nq.value, "nnz": nnz.value}


def fsa_plan_valid_pairs(plan: Plan) -> int:
    return int(lib().fsa_plan_valid_pairs(plan))


def fsa_plan_key_tokens(plan: Plan) -> int:
    return int(lib().fsa_plan_key_tokens(plan))


def fsa_plan_row_block(plan: Plan) -> int:
    return int(lib().fsa_plan_row_block(plan))


def fsa_plan_set_row_block(plan: Plan, rows: int) -> None:
    _check(lib().fsa_plan_set_row_block(plan, int(rows)))


def fsa_workspace_bytes(plan: Plan) -> int:
    return int(lib().fsa_workspace_bytes(plan))


def fsa_workspace_layout(plan: Plan) -> dict:
    w = fsa_ws_layout()
    _check(lib().fsa_workspace_layout(plan, ctypes.byref(w)))
    return {n: int(getattr(w, n)) for n, _ in fsa_ws_layout._fields_}


# ------------------------------------------------------------------ launches

def fsa_bounds(plan: Plan, Q, K, ws, scale: float, stream=None) -> None:
    _check(lib().fsa_bounds(plan, _ptr(Q), _ptr(K), _ptr(ws), float(scale), _stream(stream)))


def fsa_forward(plan: Plan, Q, K, V, O, ws, scale: float, mode=FSA_MODE_AUTO,
                stream=None) -> None:
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().fsa_forward(plan, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(ws), float(scale),
                             mode, _stream(stream)))


def fsa_copy_eligibility(plan: Plan, ws, stream=None):
    """The B*H eligibility flags fsa_bounds wrote into ws, as a uint8 numpy
    array of shape (B, H); synchronizes the stream."""
    shape = fsa_plan_shape(plan)
    out = np.zeros((shape.B, shape.H), dtype=np.uint8)
    _check(lib().fsa_copy_eligibility(plan, _ptr(ws), out.ctypes.data, _stream(stream)))
    return out


def fsa_attention(Q, K, V, O, F, T, window, ref_frame, scale, B, H, d, dtype, mode, ws,
                  ws_bytes, stream=None) -> None:
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().fsa_attention(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), F, T, window, ref_frame,
                               float(scale), B, H, d, dtype, mode, _ptr(ws), int(ws_bytes),
                               _stream(stream)))


def fsa_attention_static(plan: Plan, Q, K, V, O, scale: float, mode=FSA_MODE_AUTO,
                         stream=None) -> None:
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().fsa_attention_static(plan, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), float(scale),
                                      mode, _stream(stream)))


def fsa_attention_workspace_bytes(F, T, window, ref_frame, B, H, d, dtype) -> int:
    n = int(lib().fsa_attention_workspace_bytes(F, T, window, ref_frame, B, H, d, dtype))
    if n == 0:
        raise FsaError(FSA_ERR_INVALID_ARG, fsa_last_error())
    return n


def fsa_cross_attention(Q, Kr, Vr, O, F, T, M, scale, B, H, d, dtype, mode, ws, ws_bytes,
                        stream=None) -> None:
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().fsa_cross_attention(_ptr(Q), _ptr(Kr), _ptr(Vr), _ptr(O), F, T, M, float(scale),
                                     B, H, d, dtype, mode, _ptr(ws), int(ws_bytes),
                                     _stream(stream)))


def fsa_cross_attention_workspace_bytes(F, T, M, B, H, d, dtype) -> int:
    n = int(lib().fsa_cross_attention_workspace_bytes(F, T, M, B, H, d, dtype))
    if n == 0:
        raise FsaError(FSA_ERR_INVALID_ARG, fsa_last_error())
    return n


def fsa_prep_weight_bytes(H: int, d: int) -> int:
    return int(lib().fsa_prep_weight_bytes(H, d))


def fsa_prep_pack_weights(W, gamma, Wp, H: int, d: int, stream=None) -> None:
    _check(lib().fsa_prep_pack_weights(_ptr(W), _ptr(gamma), _ptr(Wp), H, d, _stream(stream)))


def fsa_prep(plan: Plan, grid_h: int, grid_w: int, X, Wp, Q, K, V, ws, stream=None) -> None:
    _check(lib().fsa_prep(plan, grid_h, grid_w, _ptr(X), _ptr(Wp), _ptr(Q), _ptr(K), _ptr(V),
                          _ptr(ws), _stream(stream)))


def fsa_bounds_after_prep(plan: Plan, K, ws, scale: float, stream=None) -> None:
    _check(lib().fsa_bounds_after_prep(plan, _ptr(K), _ptr(ws), float(scale), _stream(stream)))


def fsa_cache_clear() -> None:
    lib().fsa_cache_clear()


# ------------------------------------------------------------------ torch helpers

def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FSA_BF16
    if t.dtype == torch.float32:
        return FSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_inputs(pairs, like, what: str) -> None:
    """Each (tensor, shape) of pairs: a contiguous CUDA tensor of that shape,
    with like's dtype, on like's device (the kernels take one device's
    pointers)."""
    for t, shp in pairs:
        if not t.is_cuda or t.device != like.device or not t.is_contiguous() \
                or tuple(t.shape) != tuple(shp) or t.dtype != like.dtype:
            raise ValueError(what)


def _check_out_ws(out, ws, like, need: int) -> None:
    """The C ABI cannot see buffer sizes: reject an output or workspace that
    the kernels would overrun or misread."""
    if out is not None:
        if not out.is_cuda or out.device != like.device or not out.is_contiguous() \
                or tuple(out.shape) != tuple(like.shape) or out.dtype != like.dtype:
            raise ValueError(f"out must be a contiguous CUDA tensor of shape {tuple(like.shape)} "
                             f"and dtype {like.dtype} on {like.device}")
    if ws is not None:
        if not ws.is_cuda or ws.device != like.device or not ws.is_contiguous() \
                or ws.numel() * ws.element_size() < need:
            raise ValueError(f"ws must be a contiguous CUDA tensor of at least {need} bytes on "
                             f"{like.device}")


def attention(q, k, v, F: int, T: int, window: int, ref_frame: int, scale: float | None = None,
              mode="auto", out=None, ws=None):
    """O = frame-aligned windowed attention of [B, H, F*T, d] CUDA tensors.

    Calls fsa_attention on torch's current stream; allocates O and the
    workspace with torch unless given.
    """
    import torch
    B, H, N, d = q.shape
    if N != F * T:
        raise ValueError(f"N={N} != F*T={F * T}")
    _check_inputs(((q, q.shape), (k, q.shape), (v, q.shape)), q,
                  "q, k, v must be contiguous CUDA tensors of one shape, dtype and device")
    if scale is None:
        scale = d ** -0.5
    code = dtype_code(q)
    need = fsa_attention_workspace_bytes(F, T, window, ref_frame, B, H, d, code)
    _check_out_ws(out, ws, q, need)
    with torch.cuda.device(q.device):           # launch on q's device and its current stream
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty_like(q)
        fsa_attention(q, k, v, out, F, T, window, ref_frame, scale, B, H, d, code, mode, ws,
                      ws.numel() * ws.element_size())
    return out


def cross_attention(q, kr, vr, F: int, T: int, scale: float | None = None, mode="auto",
                    out=None, ws=None):
    """O [B, H, F*T, d]: every query row of q attends to all M reference
    tokens of kr, vr [B, H, M, d] (CUDA tensors). Calls fsa_cross_attention on
    torch's current stream; allocates O and the workspace with torch unless
    given."""
    import torch
    B, H, N, d = q.shape
    M = kr.shape[2]
    if N != F * T:
        raise ValueError(f"N={N} != F*T={F * T}")
    _check_inputs(((q, q.shape), (kr, (B, H, M, d)), (vr, (B, H, M, d))), q,
                  "q [B,H,F*T,d], kr and vr [B,H,M,d] must be contiguous CUDA tensors of "
                  "one dtype and device")
    if scale is None:
        scale = d ** -0.5
    code = dtype_code(q)
    need = fsa_cross_attention_workspace_bytes(F, T, M, B, H, d, code)
    _check_out_ws(out, ws, q, need)
    with torch.cuda.device(q.device):           # launch on q's device and its current stream
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty_like(q)
        fsa_cross_attention(q, kr, vr, out, F, T, M, scale, B, H, d, code, mode, ws,
                            ws.numel() * ws.element_size())
    return out


def workspace_views(plan: Plan, ws):
    """Typed torch views of the bound products inside a workspace tensor."""
    import torch
    s = fsa_plan_shape(plan)
    lay = fsa_workspace_layout(plan)
    BH, N = s.B * s.H, s.F * s.T
    KF = 1 if plan.M else s.F             # a cross plan has one key frame

    def view(off, n, dt, sz, shape):
        return ws[off:off + n * sz].view(dt).view(*shape)

    return {
        "mu": view(lay["mu"], BH * s.d, torch.float32, 4, (s.B, s.H, s.d)),
        "qnorm": view(lay["qnorm"], BH * N, torch.float32, 4, (s.B, s.H, N)),
        "rframe": view(lay["rframe"], BH * KF, torch.float32, 4, (s.B, s.H, KF)),
        "rslice": view(lay["rslice"], BH * s.F, torch.float32, 4, (s.B, s.H, s.F)),
        "stat": view(lay["stat"], BH, torch.float32, 4, (s.B, s.H)),
        "elig": view(lay["elig"], BH, torch.uint8, 1, (s.B, s.H)),
        "statf": view(lay["statf"], BH * s.F, torch.float32, 4, (s.B, s.H, s.F)),
        "eligf": view(lay["eligf"], BH * s.F, torch.uint8, 1, (s.B, s.H, s.F)),
        "dslice": view(lay["dslice"], BH * s.F * s.d, torch.float32, 4, (s.B, s.H, s.F, s.d)),
        "pmax": view(lay["pmax"], 1, torch.float32, 4, (1,)),
    }
