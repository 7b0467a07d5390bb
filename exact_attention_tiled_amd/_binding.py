"""ctypes binding of libattn.so (include/attn.h), with the same entry-point names.

Argument marshalling only: torch tensors supply device memory and the current HIP stream;
every step of the computation runs in the library's kernels. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libattn.so")

ATTN_BF16, ATTN_F32 = 0, 1
ATTN_MASK_NONE, ATTN_MASK_CAUSAL_TOP_LEFT, ATTN_MASK_CAUSAL_BOTTOM_RIGHT = 0, 1, 2
ATTN_PATH_AUTO, ATTN_PATH_PREFILL, ATTN_PATH_SPLITK = 0, 1, 2
(ATTN_PROBE_PREFILL, ATTN_PROBE_PREFILL_GENERIC, ATTN_PROBE_SPLITK, ATTN_PROBE_BWD_KV,
 ATTN_PROBE_BWD_Q, ATTN_PROBE_BWD_KV_F32, ATTN_PROBE_BWD_Q_F32) = 0, 1, 2, 3, 4, 5, 6

EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_fwd_workspace_size", "attn_fwd_ex_workspace_size",
           "attn_bwd", "attn_bwd_workspace_size", "attn_fwd_dropout",
           "attn_fwd_dropout_workspace_size", "attn_bwd_dropout", "attn_dropout_probe",
           "attn_mask_probe", "attn_describe_plan", "attn_status_string", "attn_version",
           "attn_fwd_no_workspace", "attn_mask_probe_ex", "attn_check_seqlens")

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
_U64 = ctypes.c_uint64


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def library_path() -> str:
    return LIB_PATH


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libattn.so (built by exact_attention_tiled_amd.build) and declare signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m exact_attention_tiled_amd.build`")
    lib = ctypes.CDLL(p)
    shape10 = [_I] * 10
    lib.attn_fwd.argtypes = [_P, _P, _P, _P, _P] + [_I] * 9 + [_F, _I, _I, _P, _P, _P, _S, _P]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = [_P, _P, _P, _P, _P] + [_I] * 9 + [_F, _I, _I, _I, _I,
                                                                  _P, _P, _P, _S, _P]
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_fwd_no_workspace.argtypes = [_P, _P, _P, _P, _P] + [_I] * 9 + [_F, _I, _I, _P, _P, _P]
    lib.attn_fwd_no_workspace.restype = ctypes.c_int
    lib.attn_fwd_workspace_size.argtypes = [_I] * 11
    lib.attn_fwd_workspace_size.restype = _S
    lib.attn_fwd_ex_workspace_size.argtypes = [_I] * 13
    lib.attn_fwd_ex_workspace_size.restype = _S
    lib.attn_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P] + [_I] * 9 + \
        [_F, _I, _I, _P, _P, _P, _P, _S, _P]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [_I] * 11
    lib.attn_bwd_workspace_size.restype = _S
    lib.attn_fwd_dropout.argtypes = [_P, _P, _P, _P, _P] + [_I] * 9 + [_F, _I, _I, _F, _U64,
                                                                       _P, _P, _P, _P, _S, _P]
    lib.attn_fwd_dropout.restype = ctypes.c_int
    lib.attn_fwd_dropout_workspace_size.argtypes = [_I] * 11
    lib.attn_fwd_dropout_workspace_size.restype = _S
    lib.attn_bwd_dropout.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P] + [_I] * 9 + \
        [_F, _I, _I, _F, _U64, _P, _P, _P, _P, _S, _P]
    lib.attn_bwd_dropout.restype = ctypes.c_int
    lib.attn_dropout_probe.argtypes = [_I] * 6 + [_F, _U64, _P, _P]
    lib.attn_dropout_probe.restype = ctypes.c_int
    lib.attn_check_seqlens.argtypes = [_P, _P] + [_I] * 5 + [_P, _P]
    lib.attn_check_seqlens.restype = ctypes.c_int
    lib.attn_mask_probe.argtypes = [_P, _P] + [_I] * 9 + [_P, _P]
    lib.attn_mask_probe.restype = ctypes.c_int
    lib.attn_mask_probe_ex.argtypes = [_P, _P] + [_I] * 16 + [_P, _P]
    lib.attn_mask_probe_ex.restype = ctypes.c_int
    lib.attn_describe_plan.argtypes = shape10 + [_I, _I, _I, ctypes.c_char_p, _S]
    lib.attn_describe_plan.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


class use_library:
    """Context manager: the binding's calls go to another build of the library (the race-
    exposure build lib/libattn_poison.so, for tests) while it is active."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = load()
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return int(load().attn_version())


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise AttnError(fn, rc, attn_status_string(rc))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(*ts) -> None:
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live in GPU memory")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _shape_args(q, k, cu_q, max_q, max_k):
    return (int(cu_q.shape[0]) - 1, int(q.shape[0]), int(k.shape[0]), int(max_q), int(max_k),
            int(q.shape[1]), int(k.shape[1]), int(q.shape[2]))


def attn_fwd_workspace_size(q, k, cu_q, max_seqlen_q, max_seqlen_k, mask_mode, window=0,
                            path=ATTN_PATH_AUTO, num_splits=0) -> int:
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_q, max_seqlen_q, max_seqlen_k)
    return int(load().attn_fwd_ex_workspace_size(n, tq, tk, mq, mk, hq, hkv, d, _dtype_code(q),
                                                 int(mask_mode), int(window), int(path),
                                                 int(num_splits)))


def attn_describe_plan(q, k, cu_q, max_seqlen_q, max_seqlen_k, mask_mode, window=0,
                       path=ATTN_PATH_AUTO, num_splits=0) -> str:
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_q, max_seqlen_q, max_seqlen_k)
    buf = ctypes.create_string_buffer(512)
    _check("attn_describe_plan",
           load().attn_describe_plan(n, tq, tk, mq, mk, hq, hkv, d, _dtype_code(q),
                                     int(mask_mode), int(window), int(path), int(num_splits),
                                     buf, 512))
    return buf.value.decode()


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
             cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, scale: float,
             mask_mode: int, window: int = 0, *, path: int = ATTN_PATH_AUTO, num_splits: int = 0,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward pass. q [Tq,Hq,d], k/v [Tk,Hkv,d] (bf16 or fp32, contiguous, on the GPU),
    cu_seqlens int32 [B+1] on the GPU. Returns (out [Tq,Hq,d], lse [Hq,Tq] fp32)."""
    _dev(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, workspace)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    need = attn_fwd_workspace_size(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, mask_mode,
                                   window, path, num_splits)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    rc = load().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                            n, tq, tk, mq, mk, hq, hkv, d, _dtype_code(q), float(scale),
                            int(mask_mode), int(window), int(path), int(num_splits), _ptr(out),
                            _ptr(lse), _ptr(workspace), int(workspace.numel()), _stream())
    _check("attn_fwd", rc)
    return out, lse


def attn_fwd_no_workspace(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                          max_seqlen_q: int, max_seqlen_k: int, scale: float, mask_mode: int,
                          window: int = 0, *, out: torch.Tensor, lse: torch.Tensor) -> None:
    """attn_fwd without a workspace: the library's fixed device scratch stands in for it.
    The caller passes the outputs (nothing is allocated here either)."""
    _dev(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    rc = load().attn_fwd_no_workspace(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                      _ptr(cu_seqlens_k), n, tq, tk, mq, mk, hq, hkv, d,
                                      _dtype_code(q), float(scale), int(mask_mode), int(window),
                                      _ptr(out), _ptr(lse), _stream())
    _check("attn_fwd_no_workspace", rc)


def attn_bwd_workspace_size(q, k, cu_q, max_seqlen_q, max_seqlen_k, mask_mode, window=0) -> int:
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_q, max_seqlen_q, max_seqlen_k)
    return int(load().attn_bwd_workspace_size(n, tq, tk, mq, mk, hq, hkv, d, _dtype_code(q),
                                              int(mask_mode), int(window)))


def attn_bwd(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
             scale, mask_mode, window=0, *, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass; returns (dq, dk, dv) with dk, dv summed over each GQA group."""
    _dev(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_workspace_size(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, mask_mode,
                                   window)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    rc = load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                         _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), n, tq, tk, mq, mk, hq, hkv, d,
                         _dtype_code(q), float(scale), int(mask_mode), int(window), _ptr(dq),
                         _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace.numel()), _stream())
    _check("attn_bwd", rc)
    return dq, dk, dv


def attn_fwd_dropout_workspace_size(q, k, cu_q, max_seqlen_q, max_seqlen_k, mask_mode,
                                    window=0) -> int:
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_q, max_seqlen_q, max_seqlen_k)
    return int(load().attn_fwd_dropout_workspace_size(n, tq, tk, mq, mk, hq, hkv, d,
                                                      _dtype_code(q), int(mask_mode),
                                                      int(window)))


def attn_fwd_dropout(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale,
                     mask_mode, window, dropout_p, seed, *, out=None, lse=None, workspace=None,
                     out_residual=None):
    """Forward with dropout on the attention weights (attn_fwd_dropout in include/attn.h):
    returns (out, lse); lse is that of the undropped softmax. A bf16 `out_residual` tensor
    shaped like q receives each output's rounding residual, for attn_bwd_dropout (also at
    dropout_p = 0: the forward and backward of attn_fwd / attn_bwd with D formed from the
    unrounded output)."""
    _dev(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, workspace, out_residual)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    need = int(load().attn_fwd_dropout_workspace_size(n, tq, tk, mq, mk, hq, hkv, d,
                                                      _dtype_code(q), int(mask_mode),
                                                      int(window)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = load().attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), n, tq, tk, mq, mk, hq, hkv, d,
                                 _dtype_code(q), float(scale), int(mask_mode), int(window),
                                 float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out),
                                 _ptr(lse), _ptr(out_residual), _ptr(workspace),
                                 int(workspace.numel()), _stream())
    _check("attn_fwd_dropout", rc)
    return out, lse


def attn_bwd_dropout(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     max_seqlen_k, scale, mask_mode, window, dropout_p, seed, *, dq=None,
                     dk=None, dv=None, workspace=None, out_residual=None):
    """Backward of attn_fwd_dropout with the same dropout_p and seed; returns (dq, dk, dv).
    With the forward's `out_residual` D comes from the unrounded output (and with dropout
    the separate pass that computes D is skipped)."""
    _dev(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace,
         out_residual)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_workspace_size(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, mask_mode,
                                   window)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    n, tq, tk, mq, mk, hq, hkv, d = _shape_args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k)
    rc = load().attn_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(out_residual), _ptr(dout),
                                 _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), n, tq, tk, mq, mk, hq,
                                 hkv, d, _dtype_code(q), float(scale), int(mask_mode),
                                 int(window), float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                 int(workspace.numel()), _stream())
    _check("attn_bwd_dropout", rc)
    return dq, dk, dv


def attn_dropout_probe(seq, head, q0, nq, k0, nk, dropout_p, seed,
                       device="cuda") -> torch.Tensor:
    """uint8 [nq, nk] for element (q0+i, k0+j) of (seq, head): bit 0 = kept by the row form
    of the realisation (forward, dQ kernels), bit 1 = kept by the column form (dK/dV)."""
    keep = torch.empty((nq, nk), dtype=torch.uint8, device=device)
    rc = load().attn_dropout_probe(int(seq), int(head), int(q0), int(nq), int(k0), int(nk),
                                   float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                   _ptr(keep), _stream())
    _check("attn_dropout_probe", rc)
    return keep


SEQLENS_ERRORS = {1: "cu_seqlens_q[0] != 0", 2: "cu_seqlens_q decreases",
                  4: "cu_seqlens_q[-1] != total_q", 8: "a query length exceeds max_seqlen_q",
                  16: "cu_seqlens_k[0] != 0", 32: "cu_seqlens_k decreases",
                  64: "cu_seqlens_k[-1] != total_k", 128: "a key length exceeds max_seqlen_k"}


def attn_check_seqlens(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q,
                       max_seqlen_k) -> int:
    """The attn_seqlens_error bits of the two arrays (0 = well formed), checked on the device;
    synchronises the current stream to read the word."""
    _dev(cu_seqlens_q, cu_seqlens_k)
    word = torch.empty(1, dtype=torch.int32, device=cu_seqlens_q.device)
    rc = load().attn_check_seqlens(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                   int(cu_seqlens_q.shape[0]) - 1, int(total_q), int(total_k),
                                   int(max_seqlen_q), int(max_seqlen_k), _ptr(word), _stream())
    _check("attn_check_seqlens", rc)
    return int(word.item())


def attn_mask_probe(cu_seqlens_q, cu_seqlens_k, total_q, total_k, mask_mode, window, q0, nq,
                    k0, nk) -> torch.Tensor:
    """uint8 [nq, nk]: 1 where the forward kernel lets pair (q0+i, k0+j) into the softmax."""
    _dev(cu_seqlens_q, cu_seqlens_k)
    bits = torch.empty((nq, nk), dtype=torch.uint8, device=cu_seqlens_q.device)
    rc = load().attn_mask_probe(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                int(cu_seqlens_q.shape[0]) - 1, int(total_q), int(total_k),
                                int(mask_mode), int(window), int(q0), int(nq), int(k0), int(nk),
                                _ptr(bits), _stream())
    _check("attn_mask_probe", rc)
    return bits


def attn_mask_probe_ex(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k,
                       num_heads_q, num_heads_kv, mask_mode, window, unit, q0, nq, k0, nk, *,
                       head=0, num_splits=0) -> torch.Tensor:
    """uint8 [nq, nk]: 1 where kernel unit `unit` (ATTN_PROBE_*) lets pair (q0+i, k0+j) into
    its softmax (forward) or gradient sums (backward)."""
    _dev(cu_seqlens_q, cu_seqlens_k)
    bits = torch.empty((nq, nk), dtype=torch.uint8, device=cu_seqlens_q.device)
    rc = load().attn_mask_probe_ex(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                   int(cu_seqlens_q.shape[0]) - 1, int(total_q), int(total_k),
                                   int(max_seqlen_q), int(max_seqlen_k), int(num_heads_q),
                                   int(num_heads_kv), int(mask_mode), int(window), int(unit),
                                   int(head), int(num_splits), int(q0), int(nq), int(k0),
                                   int(nk), _ptr(bits), _stream())
    _check("attn_mask_probe_ex", rc)
    return bits
