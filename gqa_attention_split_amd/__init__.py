"""Fused GQA exp-sum-div attention for MI355X (gfx950).

Computes the Mirage GQA tutorial graph ("Mirage: Define GQA Computation
Graph"): O = (E / rowsum(E)) V with E = exp(Q K), Q (B, M, D), K stored
head-dim-major as (B, D, N), V (B, N, D), all fp16, no scale and no max
subtraction. D is 64 (the tutorial graph) or 128 (the tutorial's launch
example, Q (64, 1, 128)).

The functions named ``mga_*`` mirror the C ABI in ``include/mga_gqa.h`` one to
one and only marshal arguments (pointers may be ints or torch tensors; the
stream may be an int handle or a torch stream; strides a sequence of nine
ints). ``gqa_forward`` is the convenience form for torch tensors: it
validates, allocates the output and the workspace with torch, and calls
``mga_gqa_forward`` (contiguous tensors) or ``mga_gqa_forward_strided``
(views, e.g. K as the transpose of a (B, N, D) tensor). Every step of the
computation runs in the HIP kernels; nothing here computes.
"""
from __future__ import annotations

from . import _lib

MGA_OK = 0
MGA_ERR_INVALID_VALUE = 1
MGA_ERR_LAYOUT = 2
MGA_ERR_CONFIG = 3
MGA_ERR_WORKSPACE = 4
MGA_ERR_HIP = 5
MGA_ERR_SCRATCH = 6
NOALLOC_SCRATCH_BYTES = 16 << 20
KEY_BLOCK = 128
HEAD_DIMS = (64, 128)


class GqaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(mga_status_string(status))
        self.status = status


def _ptr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(s) -> int | None:
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


# ------------------------------------------------------ C ABI, 1:1 ----
def mga_status_string(status: int) -> str:
    return _lib.load().mga_status_string(int(status)).decode()


def mga_gqa_choose_splits(B: int, M: int, N: int, D: int) -> int:
    return _lib.load().mga_gqa_choose_splits(B, M, N, D)


def mga_gqa_effective_splits(B: int, M: int, N: int, D: int, splits: int) -> int:
    return _lib.load().mga_gqa_effective_splits(B, M, N, D, splits)


def mga_gqa_workspace_bytes(B: int, M: int, N: int, D: int, splits: int) -> int:
    return _lib.load().mga_gqa_workspace_bytes(B, M, N, D, splits)


def mga_gqa_plan(B: int, M: int, N: int, D: int, splits: int):
    """(status, tile_rows, effective_splits) for a shape."""
    import ctypes
    rows, eff = ctypes.c_int(0), ctypes.c_int(0)
    rc = _lib.load().mga_gqa_plan(B, M, N, D, splits, ctypes.byref(rows), ctypes.byref(eff))
    return rc, rows.value, eff.value


def mga_gqa_check_args(q, k, v, o, B, M, N, D, splits, ws, ws_bytes) -> int:
    return _lib.load().mga_gqa_check_args(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D, splits,
                                          _ptr(ws), ws_bytes)


def mga_gqa_forward(q, k, v, o, B, M, N, D, splits, ws, ws_bytes, stream) -> int:
    return _lib.load().mga_gqa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D, splits,
                                       _ptr(ws), ws_bytes, _stream(stream))


def _strides(st):
    import ctypes
    if st is None:
        return None
    vals = [int(x) for x in st]
    if len(vals) != 9:
        raise ValueError("strides: nine element strides (q_b, q_i, k_b, k_d, k_n, v_b, v_n, o_b, o_i)")
    return ctypes.cast((ctypes.c_int64 * 9)(*vals), ctypes.c_void_p)


def mga_gqa_forward_strided(q, k, v, o, B, M, N, D, strides, splits, ws, ws_bytes, stream) -> int:
    return _lib.load().mga_gqa_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D,
                                               _strides(strides), splits, _ptr(ws), ws_bytes,
                                               _stream(stream))


def mga_gqa_forward_noalloc(q, k, v, o, B, M, N, D, strides, splits, stream) -> int:
    return _lib.load().mga_gqa_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D,
                                               _strides(strides), splits, _stream(stream))


def mga_gqa_check_args_strided(q, k, v, o, B, M, N, D, strides, splits, ws, ws_bytes) -> int:
    return _lib.load().mga_gqa_check_args_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D,
                                                  _strides(strides), splits, _ptr(ws), ws_bytes)


def mga_gqa_qknorm_forward(q, k, v, o, B, M, N, D, eps, strides, splits, ws, ws_bytes, stream) -> int:
    return _lib.load().mga_gqa_qknorm_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D,
                                              float(eps), _strides(strides), splits, _ptr(ws),
                                              ws_bytes, _stream(stream))


def mga_gqa_qknorm_workspace_bytes(B: int, M: int, N: int, D: int, splits: int) -> int:
    return _lib.load().mga_gqa_qknorm_workspace_bytes(B, M, N, D, splits)


def mga_gqa_qknorm_plan(B: int, M: int, N: int, D: int, splits: int):
    """(status, tile_rows, effective_splits) of the QK-normalised path."""
    import ctypes
    rows, eff = ctypes.c_int(0), ctypes.c_int(0)
    rc = _lib.load().mga_gqa_qknorm_plan(B, M, N, D, splits, ctypes.byref(rows), ctypes.byref(eff))
    return rc, rows.value, eff.value


def mga_gqa_qknorm_check_args(q, k, v, o, B, M, N, D, eps, strides, splits, ws, ws_bytes) -> int:
    return _lib.load().mga_gqa_qknorm_check_args(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D,
                                                 float(eps), _strides(strides), splits, _ptr(ws),
                                                 ws_bytes)


def mga_gqa_partial(q, k, v, o, B, M, N, D, splits, ws, ws_bytes, stream) -> int:
    return _lib.load().mga_gqa_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, M, N, D, splits,
                                       _ptr(ws), ws_bytes, _stream(stream))


def mga_gqa_combine(o, B, M, N, D, splits, ws, ws_bytes, stream) -> int:
    return _lib.load().mga_gqa_combine(_ptr(o), B, M, N, D, splits, _ptr(ws), ws_bytes,
                                       _stream(stream))


# ------------------------------------------------- torch convenience ----
def _check_tensors(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != 3:
            raise ValueError(f"{name} must be 3-D")
    B, M, D = q.shape
    if D not in HEAD_DIMS:
        raise ValueError(f"head dim must be one of {HEAD_DIMS}, got {D}")
    if k.shape[0] != B or k.shape[1] != D:
        raise ValueError(f"k must be (B, D, N) = ({B}, {D}, N), got {tuple(k.shape)}")
    N = k.shape[2]
    if tuple(v.shape) != (B, N, D):
        raise ValueError(f"v must be (B, N, D) = ({B}, {N}, {D}), got {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    return B, M, N, D


def workspace_for(B: int, M: int, N: int, D: int, splits: int = 0, device=None, qk_norm=False):
    """A torch uint8 workspace of mga_gqa_workspace_bytes(...) (or, with
    qk_norm, mga_gqa_qknorm_workspace_bytes(...)) bytes, or None."""
    import torch
    nbytes = (mga_gqa_qknorm_workspace_bytes if qk_norm else mga_gqa_workspace_bytes)(B, M, N, D, splits)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gqa_forward(q, k, v, out=None, splits: int = 0, workspace=None, stream=None,
                qk_norm: bool = False, eps: float = 1e-6):
    """O = (exp(QK) / rowsum) V for fp16 GPU tensors q (B,M,D), k (B,D,N), v (B,N,D).

    The tensors may be strided views (the library checks which layouts it
    takes: unit stride along D for q, v and out; k with unit stride along N
    or along D; other strides multiples of 8). ``out`` may be a view too.
    With ``qk_norm`` every query row and key vector is first rms-normalised
    over the head dim (eps inside the root, no weight)."""
    import torch
    B, M, N, D = _check_tensors(q, k, v)
    if out is None:
        out = torch.empty((B, M, D), dtype=torch.float16, device=q.device)
    elif out.dtype != torch.float16 or tuple(out.shape) != (B, M, D) or out.device != q.device:
        raise ValueError(f"out must be a float16 (B, M, {D}) tensor on q's device")
    if workspace is None:
        workspace = workspace_for(B, M, N, D, splits, q.device, qk_norm=qk_norm)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    contiguous = all(t.is_contiguous() for t in (q, k, v, out))
    st = None
    if not contiguous:
        for name, t in (("q", q), ("v", v), ("out", out)):
            if t.stride(2) != 1 and t.shape[2] > 1:
                raise ValueError(f"{name} needs unit stride along the head dim")
        st = (q.stride(0), q.stride(1), k.stride(0), k.stride(1), k.stride(2), v.stride(0),
              v.stride(1), out.stride(0), out.stride(1))
    if qk_norm:
        rc = mga_gqa_qknorm_forward(q, k, v, out, B, M, N, D, eps, st, splits, workspace, ws_bytes,
                                    stream)
    elif contiguous:
        rc = mga_gqa_forward(q, k, v, out, B, M, N, D, splits, workspace, ws_bytes, stream)
    else:
        rc = mga_gqa_forward_strided(q, k, v, out, B, M, N, D, st, splits, workspace, ws_bytes, stream)
    if rc != MGA_OK:
        raise GqaError(rc)
    return out
