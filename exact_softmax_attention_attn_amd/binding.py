"""ctypes binding of libattn.so: argument marshalling only.

Every function here has the name of the C entry point it calls (declared in
``include/attn.h``) and takes torch tensors laid out [B, N, H, d] (float32 or
bfloat16) plus L / workspace [B, H, N] float32, all on one HIP device.  The
work is enqueued on ``torch.cuda.current_stream()``.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch  # imported before the library so that one HIP runtime is mapped

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_MASK_BLOCK = 128
ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

_SIGNATURES = {
    "attn_fwd_lse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_preprocess": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "attn_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_fwd_lse_masked": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_masked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                             _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_dkdv_masked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I,
                                  _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_dq_masked": (_I, [_P, _P, _P, _P, _P, _P, _P, _I,
                                _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_bwd_bwd": (_I, [_P] * 14 + [_I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_bwd_masked": (_I, [_P] * 15 + [_I] * 6 + [_F, _I, _P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.attn_status_string(status).decode()
        if status == ATTN_ERR_HIP:
            msg += ": " + lib.attn_last_error().decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python exact_softmax_attention_attn_amd/build_lib.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_bnhd(*ts: torch.Tensor):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("expected [B, N, H, d] tensors")
    for t in ts:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("Q, K, V, O, dO and outputs must share shape, dtype and device")
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("tensors must be contiguous HIP device tensors")


def _check_rows(t: torch.Tensor, B: int, H: int, N: int, device, lead=()):
    shape = tuple(lead) + (B, H, N)
    if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"expected a contiguous float32 {shape} tensor on {device}")


def _mask_arg(mask: torch.Tensor, B: int, H: int, N: int, device):
    """A block mask tensor -> (pointer, mask_heads).  uint8 or bool, contiguous,
    [nb, nb] (shared by every (b, h)) or [B, H, nb, nb], nb = ceil(N / 128)."""
    nb = (N + ATTN_MASK_BLOCK - 1) // ATTN_MASK_BLOCK
    if mask.dtype not in (torch.uint8, torch.bool) or not mask.is_contiguous() \
            or mask.device != device:
        raise ValueError(f"mask must be a contiguous uint8 or bool tensor on {device}")
    if tuple(mask.shape) == (nb, nb):
        return ctypes.c_void_p(mask.data_ptr()), 1
    if tuple(mask.shape) == (B, H, nb, nb):
        return ctypes.c_void_p(mask.data_ptr()), B * H
    raise ValueError(f"mask must be [{nb}, {nb}] or [{B}, {H}, {nb}, {nb}]")


def new_workspace(B: int, H: int, N: int, device) -> torch.Tensor:
    """Workspace for attn_bwd: [2, B, H, N] float32 (-D, then -L * log2(e))."""
    return torch.empty((2, B, H, N), dtype=torch.float32, device=device)


def _call(name: str, *args):
    st = getattr(load(), name)(*args)
    if st != ATTN_OK:
        raise AttnError(st, name)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_workspace_bytes(B, H, N, d))


def attn_fwd_lse(q, k, v, causal: bool = True, scale: float | None = None, o=None, lse=None):
    """O [B, N, H, d] and L [B, H, N] float32 (natural log of the row normaliser)."""
    _check_bnhd(q, k, v)
    B, N, H, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_bnhd(q, o)
    _check_rows(lse, B, H, N, q.device)
    with torch.cuda.device(q.device):
        _call("attn_fwd_lse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
              int(bool(causal)), scale, _dtype_code(q), _stream(q.device))
    return o, lse


def attn_bwd(q, k, v, o, do, lse, causal: bool = True, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV [B, N, H, d]; workspace ([2, B, H, N] float32) ends up holding -D, -L*log2(e)."""
    _check_bnhd(q, k, v, o, do)
    B, N, H, d = q.shape
    _check_rows(lse, B, H, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_bnhd(q, dq, dk, dv)
    workspace = new_workspace(B, H, N, q.device) if workspace is None else workspace
    _check_rows(workspace, B, H, N, q.device, lead=(2,))
    with torch.cuda.device(q.device):
        _call("attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
              _ptr(dk), _ptr(dv), _ptr(workspace), B, H, N, d, int(bool(causal)), scale,
              _dtype_code(q), _stream(q.device))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal: bool = True,
                     scale: float | None = None):
    """attn_bwd with the library's static per-GPU workspace (the C call
    allocates nothing; outputs are the caller's): dQ, dK, dV."""
    _check_bnhd(q, k, v, o, do, dq, dk, dv)
    B, N, H, d = q.shape
    _check_rows(lse, B, H, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _call("attn_bwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
              _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), scale,
              _dtype_code(q), _stream(q.device))
    return dq, dk, dv


def attn_bwd_preprocess(o, do, lse, workspace):
    _check_bnhd(o, do)
    B, N, H, d = o.shape
    _check_rows(lse, B, H, N, o.device)
    _check_rows(workspace, B, H, N, o.device, lead=(2,))
    with torch.cuda.device(o.device):
        _call("attn_bwd_preprocess", _ptr(o), _ptr(do), _ptr(lse), _ptr(workspace), B, H, N, d,
              _dtype_code(o), _stream(o.device))
    return workspace


def attn_bwd_dkdv(q, k, v, do, workspace, dk, dv, causal: bool = True,
                  scale: float | None = None):
    _check_bnhd(q, k, v, do, dk, dv)
    B, N, H, d = q.shape
    _check_rows(workspace, B, H, N, q.device, lead=(2,))
    scale = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _call("attn_bwd_dkdv", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace),
              _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), scale, _dtype_code(q),
              _stream(q.device))
    return dk, dv


def attn_bwd_dq(q, k, v, do, workspace, dq, causal: bool = True, scale: float | None = None):
    _check_bnhd(q, k, v, do, dq)
    B, N, H, d = q.shape
    _check_rows(workspace, B, H, N, q.device, lead=(2,))
    scale = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _call("attn_bwd_dq", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace),
              _ptr(dq), B, H, N, d, int(bool(causal)), scale, _dtype_code(q), _stream(q.device))
    return dq


def attn_fwd_lse_masked(q, k, v, mask, causal: bool = True, scale: float | None = None,
                        o=None, lse=None):
    """attn_fwd_lse over the pairs a block mask keeps (rows keeping no key: O = 0, L = -inf)."""
    _check_bnhd(q, k, v)
    B, N, H, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_bnhd(q, o)
    _check_rows(lse, B, H, N, q.device)
    mp, mh = _mask_arg(mask, B, H, N, q.device)
    with torch.cuda.device(q.device):
        _call("attn_fwd_lse_masked", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), mp, mh,
              B, H, N, d, int(bool(causal)), scale, _dtype_code(q), _stream(q.device))
    return o, lse


def attn_bwd_masked(q, k, v, o, do, lse, mask, causal: bool = True, scale: float | None = None,
                    dq=None, dk=None, dv=None, workspace=None):
    """attn_bwd over the pairs a block mask keeps; lse from attn_fwd_lse_masked (same mask)."""
    _check_bnhd(q, k, v, o, do)
    B, N, H, d = q.shape
    _check_rows(lse, B, H, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_bnhd(q, dq, dk, dv)
    workspace = new_workspace(B, H, N, q.device) if workspace is None else workspace
    _check_rows(workspace, B, H, N, q.device, lead=(2,))
    mp, mh = _mask_arg(mask, B, H, N, q.device)
    with torch.cuda.device(q.device):
        _call("attn_bwd_masked", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), mp, mh, B, H, N, d,
              int(bool(causal)), scale, _dtype_code(q), _stream(q.device))
    return dq, dk, dv


def attn_bwd_dkdv_masked(q, k, v, do, workspace, dk, dv, mask, causal: bool = True,
                         scale: float | None = None):
    """Stage 2 of attn_bwd_masked: dK, dV (workspace from attn_bwd_preprocess)."""
    _check_bnhd(q, k, v, do, dk, dv)
    B, N, H, d = q.shape
    _check_rows(workspace, B, H, N, q.device, lead=(2,))
    scale = default_scale(d) if scale is None else float(scale)
    mp, mh = _mask_arg(mask, B, H, N, q.device)
    with torch.cuda.device(q.device):
        _call("attn_bwd_dkdv_masked", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace),
              _ptr(dk), _ptr(dv), mp, mh, B, H, N, d, int(bool(causal)), scale, _dtype_code(q),
              _stream(q.device))
    return dk, dv


def attn_bwd_dq_masked(q, k, v, do, workspace, dq, mask, causal: bool = True,
                       scale: float | None = None):
    """Stage 3 of attn_bwd_masked: dQ (workspace from attn_bwd_preprocess)."""
    _check_bnhd(q, k, v, do, dq)
    B, N, H, d = q.shape
    _check_rows(workspace, B, H, N, q.device, lead=(2,))
    scale = default_scale(d) if scale is None else float(scale)
    mp, mh = _mask_arg(mask, B, H, N, q.device)
    with torch.cuda.device(q.device):
        _call("attn_bwd_dq_masked", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace),
              _ptr(dq), mp, mh, B, H, N, d, int(bool(causal)), scale, _dtype_code(q),
              _stream(q.device))
    return dq


def attn_bwd_bwd(q, k, v, o, do, lse, gq, gk, gv, causal: bool = True,
                 scale: float | None = None, hq=None, hk=None, hv=None, hdo=None,
                 workspace=None):
    """Gradients of <gQ,dQ> + <gK,dK> + <gV,dV> w.r.t. Q, K, V, dO: (hQ, hK, hV, hdO).
    workspace: [4, B, H, N] float32 (-D, -L log2(e), r, E)."""
    _check_bnhd(q, k, v, o, do, gq, gk, gv)
    B, N, H, d = q.shape
    _check_rows(lse, B, H, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    hq = torch.empty_like(q) if hq is None else hq
    hk = torch.empty_like(q) if hk is None else hk
    hv = torch.empty_like(q) if hv is None else hv
    hdo = torch.empty_like(q) if hdo is None else hdo
    _check_bnhd(q, hq, hk, hv, hdo)
    if workspace is None:
        workspace = torch.empty((4, B, H, N), dtype=torch.float32, device=q.device)
    _check_rows(workspace, B, H, N, q.device, lead=(4,))
    with torch.cuda.device(q.device):
        _call("attn_bwd_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(gq),
              _ptr(gk), _ptr(gv), _ptr(hq), _ptr(hk), _ptr(hv), _ptr(hdo), _ptr(workspace),
              B, H, N, d, int(bool(causal)), scale, _dtype_code(q), _stream(q.device))
    return hq, hk, hv, hdo


def attn_bwd_bwd_masked(q, k, v, o, do, lse, gq, gk, gv, mask, causal: bool = True,
                        scale: float | None = None, hq=None, hk=None, hv=None, hdo=None,
                        workspace=None):
    """attn_bwd_bwd over the pairs a block mask keeps; lse from attn_fwd_lse_masked
    (same mask).  Returns (hQ, hK, hV, hdO)."""
    _check_bnhd(q, k, v, o, do, gq, gk, gv)
    B, N, H, d = q.shape
    _check_rows(lse, B, H, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    mp, mh = _mask_arg(mask, B, H, N, q.device)
    hq = torch.empty_like(q) if hq is None else hq
    hk = torch.empty_like(q) if hk is None else hk
    hv = torch.empty_like(q) if hv is None else hv
    hdo = torch.empty_like(q) if hdo is None else hdo
    _check_bnhd(q, hq, hk, hv, hdo)
    if workspace is None:
        workspace = torch.empty((4, B, H, N), dtype=torch.float32, device=q.device)
    _check_rows(workspace, B, H, N, q.device, lead=(4,))
    with torch.cuda.device(q.device):
        _call("attn_bwd_bwd_masked", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
              _ptr(gq), _ptr(gk), _ptr(gv), _ptr(hq), _ptr(hk), _ptr(hv), _ptr(hdo),
              _ptr(workspace), mp, mh, B, H, N, d, int(bool(causal)), scale, _dtype_code(q),
              _stream(q.device))
    return hq, hk, hv, hdo
