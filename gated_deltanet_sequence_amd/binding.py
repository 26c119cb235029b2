"""Thin ctypes binding over libgdn.so (C ABI in include/gdn.h).

Argument marshalling only: every step of the forward pass and of the decode
step runs in the HIP kernels behind the C ABI.  PyTorch provides the device
memory and the stream.  There is no fallback: if the library is missing or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _build

GDN_OK = 0
GDN_ERR_INVALID_ARG = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_ALIGNMENT = 3
GDN_ERR_HIP = 4

GDN_F32 = 0
GDN_BF16 = 1

_DTYPES = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}
_lib = None


class GDNError(RuntimeError):
    """A nonzero return code of the C ABI."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, strerror(code), code))


def load_library(path: str | None = None):
    """Load libgdn.so (building it first only if no build exists at all)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    lib_path = path or _build.LIB
    if not os.path.exists(lib_path):
        _build.build()
    lib = ctypes.CDLL(lib_path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32, p]
    lib.gdn_chunk_fwd.restype = i32
    lib.gla_chunk_fwd.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32, p]
    lib.gla_chunk_fwd.restype = i32
    lib.gdn_scan_fwd.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i32,
                                 p, ctypes.c_size_t, p]
    lib.gdn_scan_fwd.restype = i32
    lib.gdn_scan_fwd_vecgate.argtypes = lib.gdn_scan_fwd.argtypes
    lib.gdn_scan_fwd_vecgate.restype = i32
    for fn in (lib.gdn_recurrent_fwd, lib.gdn_recurrent_fwd_vecgate):
        fn.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i32, p]
        fn.restype = i32
    lib.gdn_chunk_fwd_vecgate.argtypes = lib.gdn_chunk_fwd.argtypes
    lib.gdn_chunk_fwd_vecgate.restype = i32
    lib.gdn_chunk_fwd_vecgate_split.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32,
                                                p, ctypes.c_size_t, p]
    lib.gdn_chunk_fwd_vecgate_split.restype = i32
    lib.gdn_chunk_fwd_vecgate_split_workspace.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.gdn_chunk_fwd_vecgate_split_workspace.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_vecgate_2pass.argtypes = lib.gdn_chunk_fwd_vecgate_split.argtypes
    lib.gdn_chunk_fwd_vecgate_2pass.restype = i32
    lib.gdn_chunk_fwd_vecgate_2pass_workspace.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.gdn_chunk_fwd_vecgate_2pass_workspace.restype = ctypes.c_size_t
    lib.gdn_scan_fwd_workspace.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.gdn_scan_fwd_workspace.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_split.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32,
                                        p, ctypes.c_size_t, p]
    lib.gdn_chunk_fwd_split.restype = i32
    lib.gdn_chunk_fwd_split_noalloc.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32, p]
    lib.gdn_chunk_fwd_split_noalloc.restype = i32
    lib.gdn_chunk_fwd_split_workspace.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.gdn_chunk_fwd_split_workspace.restype = ctypes.c_size_t
    for fn in (lib.gdn_recurrent_step, lib.gdn_recurrent_step_vecgate, lib.gla_recurrent_step):
        fn.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i32, p]
        fn.restype = i32
    lib.gdn_strerror.argtypes = [i32]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().gdn_strerror(int(code)).decode()


def version() -> str:
    return load_library().gdn_version().decode()


def _dev_ptr(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_fwd_args(q, k, v, alpha, beta, initial_state, alpha_per_dim=False):
    if q.dtype not in _DTYPES:
        raise TypeError("q/k/v must be bfloat16 or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    ashape = (B, H, T, dk) if alpha_per_dim else (B, H, T)
    if alpha.dtype != torch.float32 or tuple(alpha.shape) != ashape:
        raise ValueError("alpha must be fp32 %s" % ("[B,H,T,dk]" if alpha_per_dim else "[B,H,T]"))
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, T):
        raise ValueError("beta must be fp32 [B,H,T]")
    if initial_state is not None and (initial_state.dtype != torch.float32 or
                                      tuple(initial_state.shape) != (B, H, dv, dk)):
        raise ValueError("initial_state must be fp32 [B,H,dv,dk]")
    return B, H, T, dk, dv


def gdn_chunk_fwd(q, k, v, alpha, beta, initial_state=None, chunk_size: int = 64, *,
                  o=None, final_state=None, output_final_state: bool = True, stream=None):
    """Chunked forward pass (chunk_size 64, or 32).  q, k [B,H,T,dk], v [B,H,T,dv] (bf16 or fp32);
    alpha, beta [B,H,T] fp32; initial_state [B,H,dv,dk] fp32 or None.

    Returns (o [B,H,T,dv] in the input dtype, final_state [B,H,dv,dk] fp32 or
    None).  ``final_state`` may be passed (and may be ``initial_state`` itself
    for an in-place carry)."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.gdn_chunk_fwd(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                           _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                           _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                           _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                           int(chunk_size), _DTYPES[q.dtype], _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd")
    return o, final_state


def gla_chunk_fwd(q, k, v, alpha, beta, initial_state=None, chunk_size: int = 64, *,
                  o=None, final_state=None, output_final_state: bool = True, stream=None):
    """Gated linear attention without the delta rule,
    S_t = alpha_t S_{t-1} + beta_t v_t k_t^T, o_t = S_t q_t.  Same arguments,
    dtypes, chunk sizes and result as gdn_chunk_fwd."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    rc = load_library().gla_chunk_fwd(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                      _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                      _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                      _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                      int(chunk_size), _DTYPES[q.dtype], _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gla_chunk_fwd")
    return o, final_state


def gdn_scan_fwd_workspace(B, H, T, dk, dv, dtype=torch.bfloat16) -> int:
    """Bytes of workspace gdn_scan_fwd needs."""
    return int(load_library().gdn_scan_fwd_workspace(B, H, T, dk, dv, _DTYPES[dtype]))


def gdn_scan_fwd(q, k, v, alpha, beta, initial_state=None, *, o=None, final_state=None,
                 output_final_state: bool = True, workspace=None, stream=None, _vecgate=False):
    """The same recurrence by the blocked parallel-scan route (fp32 state;
    bf16 or fp32 q/k/v; d 64 or 128).  Same arguments and result as
    gdn_chunk_fwd without the chunk size; the workspace (uint8 GPU tensor) is
    allocated here when not given."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state, alpha_per_dim=_vecgate)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    need = gdn_scan_fwd_workspace(B, H, T, dk, dv, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = load_library().gdn_scan_fwd_vecgate if _vecgate else load_library().gdn_scan_fwd
    rc = fn(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                     _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                     _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                     _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                     _DTYPES[q.dtype], _dev_ptr(workspace, "workspace"), ws_bytes,
                                     _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_scan_fwd_vecgate" if _vecgate else "gdn_scan_fwd")
    return o, final_state


def gdn_recurrent_fwd(q, k, v, alpha, beta, initial_state=None, *, o=None, final_state=None,
                      output_final_state: bool = True, stream=None, _vecgate=False):
    """The forward pass token by token (one launch, the state in registers):
    for many short sequences.  Same arguments and result as gdn_chunk_fwd
    without the chunk size."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state, alpha_per_dim=_vecgate)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    name = "gdn_recurrent_fwd_vecgate" if _vecgate else "gdn_recurrent_fwd"
    rc = getattr(load_library(), name)(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                       _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                       _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                       _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                       _DTYPES[q.dtype], _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, name)
    return o, final_state


def gdn_recurrent_fwd_vecgate(q, k, v, alpha, beta, initial_state=None, **kw):
    """gdn_recurrent_fwd with a per-dimension gate alpha [B,H,T,dk] (fp32)."""
    return gdn_recurrent_fwd(q, k, v, alpha, beta, initial_state, _vecgate=True, **kw)


def gdn_scan_fwd_vecgate(q, k, v, alpha, beta, initial_state=None, **kw):
    """gdn_scan_fwd with a per-dimension gate alpha [B,H,T,dk] (fp32) that
    decays the key columns of the state."""
    return gdn_scan_fwd(q, k, v, alpha, beta, initial_state, _vecgate=True, **kw)


VECGATE_CHUNK = 32


def gdn_chunk_fwd_vecgate(q, k, v, alpha, beta, initial_state=None, chunk_size: int = VECGATE_CHUNK, *,
                          o=None, final_state=None, output_final_state: bool = True, stream=None):
    """Chunked forward pass with a per-dimension gate alpha [B,H,T,dk] (fp32)
    that decays the key columns of the state; bf16 or fp32 q/k/v, 32-token
    chunks."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state, alpha_per_dim=True)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.gdn_chunk_fwd_vecgate(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                   _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                   _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                   _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                   int(chunk_size), _DTYPES[q.dtype], _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_vecgate")
    return o, final_state


def gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, dk, dv, chunk_size: int = VECGATE_CHUNK,
                                          dtype=torch.bfloat16) -> int:
    """Bytes of workspace with which gdn_chunk_fwd_vecgate_2pass uses its largest tile."""
    return int(load_library().gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, dk, dv, int(chunk_size),
                                                                    _DTYPES[dtype]))


def gdn_chunk_fwd_vecgate_2pass(q, k, v, alpha, beta, initial_state=None, chunk_size: int = VECGATE_CHUNK, *,
                                o=None, final_state=None, output_final_state: bool = True,
                                workspace=None, stream=None):
    """gdn_chunk_fwd_vecgate in two passes (the state-independent chunk work
    once per chunk, into workspace records; then the state products per value
    slice).  Same arguments and result (for bf16 up to the order of the
    products' fp32 sums); the workspace (a uint8 GPU tensor) is allocated here
    when not given."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state, alpha_per_dim=True)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, dk, dv, chunk_size, q.dtype)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    rc = lib.gdn_chunk_fwd_vecgate_2pass(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                         _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                         _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                         _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                         int(chunk_size), _DTYPES[q.dtype],
                                         _dev_ptr(workspace, "workspace"), ws_bytes,
                                         _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_vecgate_2pass")
    return o, final_state


def gdn_chunk_fwd_vecgate_split_workspace(B, H, T, dk, dv, chunk_size: int = VECGATE_CHUNK,
                                          dtype=torch.bfloat16) -> int:
    """Bytes of workspace gdn_chunk_fwd_vecgate_split needs on the current device (0: no split)."""
    return int(load_library().gdn_chunk_fwd_vecgate_split_workspace(B, H, T, dk, dv, int(chunk_size),
                                                                    _DTYPES[dtype]))


def gdn_chunk_fwd_vecgate_split(q, k, v, alpha, beta, initial_state=None, chunk_size: int = VECGATE_CHUNK, *,
                                o=None, final_state=None, output_final_state: bool = True,
                                workspace=None, stream=None):
    """gdn_chunk_fwd_vecgate with every sequence split into segments that run
    in parallel (for few, long sequences).  Same arguments and result; the
    workspace (a uint8 GPU tensor) is allocated here when not given."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state, alpha_per_dim=True)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    need = gdn_chunk_fwd_vecgate_split_workspace(B, H, T, dk, dv, chunk_size, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    rc = lib.gdn_chunk_fwd_vecgate_split(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                         _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                         _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                         _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                         int(chunk_size), _DTYPES[q.dtype],
                                         _dev_ptr(workspace, "workspace"), ws_bytes,
                                         _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_vecgate_split")
    return o, final_state


def gdn_chunk_fwd_split_workspace(B, H, T, dk, dv, chunk_size: int = 64, dtype=torch.bfloat16) -> int:
    """Bytes of workspace gdn_chunk_fwd_split needs on the current device (0: no split)."""
    return int(load_library().gdn_chunk_fwd_split_workspace(B, H, T, dk, dv, int(chunk_size),
                                                            _DTYPES[dtype]))


def gdn_chunk_fwd_split(q, k, v, alpha, beta, initial_state=None, chunk_size: int = 64, *,
                        o=None, final_state=None, output_final_state: bool = True,
                        workspace=None, stream=None):
    """gdn_chunk_fwd with every sequence split into segments that run in
    parallel (for few, long sequences).  Same arguments and result; the
    workspace (a uint8 GPU tensor) is allocated here when not given."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    need = gdn_chunk_fwd_split_workspace(B, H, T, dk, dv, chunk_size, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    rc = lib.gdn_chunk_fwd_split(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                 _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                 _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                 _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                 int(chunk_size), _DTYPES[q.dtype],
                                 _dev_ptr(workspace, "workspace"), ws_bytes,
                                 _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_split")
    return o, final_state


def gdn_chunk_fwd_split_noalloc(q, k, v, alpha, beta, initial_state=None, chunk_size: int = 64, *,
                                o=None, final_state=None, output_final_state: bool = True, stream=None):
    """gdn_chunk_fwd_split on the library's static per-GPU scratch instead of a
    workspace (the C entry point allocates nothing; outputs are allocated here
    only when not given).  Calls on one GPU must not overlap in time."""
    B, H, T, dk, dv = _check_fwd_args(q, k, v, alpha, beta, initial_state)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.gdn_chunk_fwd_split_noalloc(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                         _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                         _dev_ptr(initial_state, "initial_state"), _dev_ptr(o, "o"),
                                         _dev_ptr(final_state, "final_state"), B, H, T, dk, dv,
                                         int(chunk_size), _DTYPES[q.dtype], _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_split_noalloc")
    return o, final_state


SPLIT_NOALLOC_SCRATCH_BYTES = 8 << 20


def _step(name, q, k, v, alpha, beta, state, o, stream, vec_gate):
    if q.dtype not in _DTYPES:
        raise TypeError("q/k/v must be bfloat16 or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [N,H,dk] and v [N,H,dv]")
    N, H, dk = q.shape
    dv = v.shape[2]
    a_shape = (N, H, dk) if vec_gate else (N, H)
    if alpha.dtype != torch.float32 or tuple(alpha.shape) != a_shape:
        raise ValueError("alpha must be fp32 [%s]" % ("N,H,dk" if vec_gate else "N,H"))
    if beta.dtype != torch.float32 or tuple(beta.shape) != (N, H):
        raise ValueError("beta must be fp32 [N,H]")
    if state.dtype != torch.float32 or tuple(state.shape) != (N, H, dv, dk):
        raise ValueError("state must be fp32 [N,H,dv,dk]")
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    lib = load_library()
    rc = getattr(lib, name)(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                            _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                            _dev_ptr(state, "state"), _dev_ptr(o, "o"), N, H, dk, dv,
                            _DTYPES[q.dtype], _stream_ptr(stream, q.device))
    if rc != GDN_OK:
        raise GDNError(rc, name)
    return o


def gdn_recurrent_step(q, k, v, alpha, beta, state, *, o=None, stream=None):
    """One decode step.  q, k [N,H,dk], v [N,H,dv] (bf16 or fp32); alpha, beta
    [N,H] fp32; state [N,H,dv,dk] fp32, updated IN PLACE.  Returns o [N,H,dv]."""
    return _step("gdn_recurrent_step", q, k, v, alpha, beta, state, o, stream, vec_gate=False)


def gdn_recurrent_step_vecgate(q, k, v, alpha, beta, state, *, o=None, stream=None):
    """gdn_recurrent_step with a per-dimension gate alpha [N,H,dk] fp32."""
    return _step("gdn_recurrent_step_vecgate", q, k, v, alpha, beta, state, o, stream, vec_gate=True)


def gla_recurrent_step(q, k, v, alpha, beta, state, *, o=None, stream=None):
    """One decode step of gated linear attention (no erase term); arguments as
    gdn_recurrent_step."""
    return _step("gla_recurrent_step", q, k, v, alpha, beta, state, o, stream, vec_gate=False)
