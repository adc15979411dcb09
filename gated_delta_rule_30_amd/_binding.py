"""ctypes binding of libkda.so: argument marshalling only.

Torch supplies device memory and the current stream; every step of the operator runs in
the library's HIP kernels. If the library has not been built the import fails loudly:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "kda.h")

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
# input options of the _ex entry points (KDA_OPT_* in include/kda.h)
OPT_SCALAR_GATE = 1
OPT_GATE_LOGITS = 2
OPT_BETA_LOGITS = 4
OPT_L2NORM_QK = 8
STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERROR_INVALID_VALUE", 2: "KDA_ERROR_NOT_SUPPORTED",
          3: "KDA_ERROR_WORKSPACE_TOO_SMALL", 4: "KDA_ERROR_LAUNCH"}


class KdaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s" % (what, _lib().kda_status_string(status).decode()))
        self.status = status


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkda.so is not built (expected at %s); run "
                              "python -m gated_delta_rule_30_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_chunk_fwd_workspace_size.restype = sz
        lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                      ctypes.c_int, vp, vp, vp, sz, vp]
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                        ctypes.c_int, vp]
        u32 = ctypes.c_uint32
        lib.kda_chunk_fwd_ex.restype = ctypes.c_int
        lib.kda_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                         ctypes.c_int, u32, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                              i32, ctypes.c_int, u32, vp, vp, vp]
        lib.kda_chunk_fwd_scan_workspace_size.restype = sz
        lib.kda_chunk_fwd_scan_workspace_size.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int, i32]
        lib.kda_chunk_fwd_scan.restype = ctypes.c_int
        lib.kda_chunk_fwd_scan.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                           ctypes.c_int, u32, i32, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_scan_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                              ctypes.c_int, u32, i32, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_scan_ex.restype = ctypes.c_int
        lib.kda_chunk_bwd_workspace_size.restype = sz
        lib.kda_chunk_bwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int]
        lib.kda_chunk_bwd_workspace_size_ex.restype = sz
        lib.kda_chunk_bwd_workspace_size_ex.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int,
                                                        ctypes.c_uint32, i64]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                      ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.kda_chunk_bwd_ex.restype = ctypes.c_int
        lib.kda_chunk_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                         ctypes.c_int, ctypes.c_uint32, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_ckpt.restype = ctypes.c_int
        lib.kda_chunk_fwd_ckpt.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                           ctypes.c_int, u32, vp, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_ckpt_interval.restype = i64
        lib.kda_chunk_fwd_ckpt_interval.argtypes = [i32, i64, i32]
        lib.kda_chunk_fwd_ckpt_bytes.restype = sz
        lib.kda_chunk_fwd_ckpt_bytes.argtypes = [i32, i64, i32, i32, i32]
        lib.kda_chunk_bwd_ckpt.restype = ctypes.c_int
        lib.kda_chunk_bwd_ckpt.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                           ctypes.c_int, ctypes.c_uint32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp, sz, vp]
        lib.kda_decode_step_ex.restype = ctypes.c_int
        lib.kda_decode_step_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           ctypes.c_int, u32, vp]
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


def declared_functions():
    """Names of the functions declared in include/kda.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError("q/k/v/log_alpha/beta must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype) -> int:
    code = KDA_DTYPE_BF16 if dtype == torch.bfloat16 else KDA_DTYPE_F32
    return int(_lib().kda_chunk_fwd_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, code))


def bwd_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype, segment_tokens=None,
                       options=0) -> int:
    """Workspace bytes of chunk_bwd with these input options (OPT_* bits): the default
    segments (``segment_tokens`` None), or segments of that many tokens (0: one segment)."""
    code = KDA_DTYPE_BF16 if dtype == torch.bfloat16 else KDA_DTYPE_F32
    seg = -1 if segment_tokens is None else int(segment_tokens)
    return int(_lib().kda_chunk_bwd_workspace_size_ex(num_seqs, total_tokens, num_heads, dk, dv,
                                                      code, int(options), seg))


def ckpt_interval(num_seqs, total_tokens, num_heads) -> int:
    """Chunks of 64 tokens between the checkpoints chunk_fwd keeps for chunk_bwd."""
    return int(_lib().kda_chunk_fwd_ckpt_interval(num_seqs, total_tokens, num_heads))


def ckpt_empty(num_seqs, total_tokens, num_heads, dk, dv, device):
    """An uninitialised fp32 checkpoint buffer for chunk_fwd(checkpoints=...): one [H, K, V]
    state per checkpoint (possibly none)."""
    nb = int(_lib().kda_chunk_fwd_ckpt_bytes(num_seqs, total_tokens, num_heads, dk, dv))
    return torch.empty((nb // (4 * num_heads * dk * dv), num_heads, dk, dv), dtype=torch.float32,
                       device=device)


def chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, num_seqs=None,
              output_final_state=True, o=None, final_state=None, workspace=None, options=0,
              checkpoints=None):
    """kda_chunk_fwd on torch tensors (token-major [T, H, .], see include/kda.h).

    Returns (o [T, H, V] in the input dtype, final_state [N, H, K, V] fp32 or None).
    ``final_state`` may be passed as the same tensor as ``init_state`` (in-place update).
    ``options`` (OPT_* bits) selects kda_chunk_fwd_ex; with OPT_SCALAR_GATE log_alpha is [T, H].
    ``checkpoints`` (a ckpt_empty buffer) selects kda_chunk_fwd_ckpt, which also keeps the
    states chunk_bwd(checkpoints=...) starts its segments from.
    """
    device = q.device
    T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, device)
        N = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != N:
            raise ValueError("num_seqs does not match cu_seqlens")
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gshape = (T, H) if options & OPT_SCALAR_GATE else (T, H, K)
    for name, t, shp in (("q", q, (T, H, K)), ("k", k, (T, H, K)), ("v", v, (T, H, V)),
                         ("log_alpha", log_alpha, gshape), ("beta", beta, (T, H))):
        _check(t, name, shp, dt, device)
    if init_state is not None:
        _check(init_state, "init_state", (N, H, K, V), torch.float32, device)
    if o is None:
        o = torch.empty((T, H, V), dtype=dt, device=device)
    else:
        _check(o, "o", (T, H, V), dt, device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, K, V), dtype=torch.float32, device=device)
    elif final_state is not None:
        _check(final_state, "final_state", (N, H, K, V), torch.float32, device)
    need = int(_lib().kda_chunk_fwd_workspace_size(N, T, H, K, V, code))
    if need == 0:
        raise KdaError(2 if K not in (32, 64, 128, 256) or V not in (32, 64, 128, 256) else 1,
                       "kda_chunk_fwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if checkpoints is not None:
        nb = int(_lib().kda_chunk_fwd_ckpt_bytes(N, T, H, K, V))
        _check(checkpoints, "checkpoints", (nb // (4 * H * K * V), H, K, V), torch.float32, device)
        st = _lib().kda_chunk_fwd_ckpt(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                       _ptr(init_state), _ptr(cu_seqlens), N, T, H, K, V, code,
                                       int(options), _ptr(o), _ptr(final_state),
                                       _ptr(checkpoints) if nb else None, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(device))
        if st != 0:
            raise KdaError(st, "kda_chunk_fwd_ckpt")
        return o, final_state
    st = _lib().kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                 _ptr(init_state), _ptr(cu_seqlens), N, T, H, K, V, code,
                                 int(options), _ptr(o), _ptr(final_state), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(device))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd")
    return o, final_state


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None,
                      num_seqs=None, o=None, final_state=None, options=0):
    """kda_chunk_fwd_noalloc on torch tensors: chunk_fwd without a workspace (the library's
    fixed scratch serves it). final_state is always produced; ``o`` and ``final_state`` may be
    passed preallocated (then nothing is allocated here either). Returns (o, final_state)."""
    device = q.device
    T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, device)
        N = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != N:
            raise ValueError("num_seqs does not match cu_seqlens")
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gshape = (T, H) if options & OPT_SCALAR_GATE else (T, H, K)
    for name, t, shp in (("q", q, (T, H, K)), ("k", k, (T, H, K)), ("v", v, (T, H, V)),
                         ("log_alpha", log_alpha, gshape), ("beta", beta, (T, H))):
        _check(t, name, shp, dt, device)
    if init_state is not None:
        _check(init_state, "init_state", (N, H, K, V), torch.float32, device)
    if o is None:
        o = torch.empty((T, H, V), dtype=dt, device=device)
    else:
        _check(o, "o", (T, H, V), dt, device)
    if final_state is None:
        final_state = torch.empty((N, H, K, V), dtype=torch.float32, device=device)
    else:
        _check(final_state, "final_state", (N, H, K, V), torch.float32, device)
    st = _lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                      _ptr(init_state), _ptr(cu_seqlens), N, T, H, K, V, code,
                                      int(options), _ptr(o), _ptr(final_state), _stream(device))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_noalloc")
    return o, final_state


def chunk_fwd_scan(q, k, v, log_alpha, beta, init_state=None, num_seqs=None, num_groups=8,
                   output_final_state=True, o=None, final_state=None, workspace=None, options=0,
                   cu_seqlens=None):
    """kda_chunk_fwd_scan_ex on torch tensors: sequences packed token-major ([T, H, .]), equal
    lengths (num_seqs of them, default 1) or given by cu_seqlens, each split into num_groups
    groups whose states are combined by a scan (see include/kda.h). Returns (o, final_state) as
    chunk_fwd does."""
    device = q.device
    T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, device)
        N = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != N:
            raise ValueError("num_seqs does not match cu_seqlens")
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gshape = (T, H) if options & OPT_SCALAR_GATE else (T, H, K)
    for name, t, shp in (("q", q, (T, H, K)), ("k", k, (T, H, K)), ("v", v, (T, H, V)),
                         ("log_alpha", log_alpha, gshape), ("beta", beta, (T, H))):
        _check(t, name, shp, dt, device)
    if init_state is not None:
        _check(init_state, "init_state", (N, H, K, V), torch.float32, device)
    if o is None:
        o = torch.empty((T, H, V), dtype=dt, device=device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, K, V), dtype=torch.float32, device=device)
    need = int(_lib().kda_chunk_fwd_scan_workspace_size(N, T, H, K, V, code, int(num_groups)))
    if need == 0:
        raise KdaError(2 if K != V or K not in (32, 64, 128) else 1,
                       "kda_chunk_fwd_scan_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    st = _lib().kda_chunk_fwd_scan_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                      _ptr(init_state), _ptr(cu_seqlens), N, T, H, K, V, code,
                                      int(options), int(num_groups), _ptr(o), _ptr(final_state),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(device))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_scan_ex")
    return o, final_state


def chunk_bwd(q, k, v, log_alpha, beta, d_o, init_state=None, d_final_state=None,
              cu_seqlens=None, num_seqs=None, workspace=None, grads=None, segment_tokens=None,
              options=0, checkpoints=None):
    """kda_chunk_bwd_ex on torch tensors: the gradients of sum(d_o * o) + sum(d_final_state *
    final_state) for chunk_fwd on the same inputs and options (OPT_* bits; with OPT_SCALAR_GATE
    log_alpha and its gradient are [T, H]). d_o [T, H, V] in the input dtype; d_final_state
    [N, H, K, V] fp32 or None (zero). Returns fp32 tensors (dq [T, H, K], dk [T, H, K],
    dv [T, H, V], dlog_alpha, dbeta [T, H], dinit_state [N, H, K, V]). ``grads`` may pass those
    six tensors to be written in place (e.g. under graph capture). Without ``workspace``, one of
    the default size is allocated, or, with ``segment_tokens``, one sized for segments of that
    many tokens (0: one segment). ``checkpoints``, filled by chunk_fwd(checkpoints=...) on the
    same inputs, selects kda_chunk_bwd_ckpt: its segments start from those states instead of a
    pass that forms them again."""
    device = q.device
    T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, device)
        N = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != N:
            raise ValueError("num_seqs does not match cu_seqlens")
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gshape = (T, H) if options & OPT_SCALAR_GATE else (T, H, K)
    for name, t, shp in (("q", q, (T, H, K)), ("k", k, (T, H, K)), ("v", v, (T, H, V)),
                         ("log_alpha", log_alpha, gshape), ("beta", beta, (T, H)),
                         ("d_o", d_o, (T, H, V))):
        _check(t, name, shp, dt, device)
    for name, t in (("init_state", init_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check(t, name, (N, H, K, V), torch.float32, device)
    f32 = dict(dtype=torch.float32, device=device)
    if grads is None:
        dq, dk = (torch.empty((T, H, K), **f32) for _ in range(2))
        dg = torch.empty(gshape, **f32)
        dv = torch.empty((T, H, V), **f32)
        db = torch.empty((T, H), **f32)
        dinit = torch.empty((N, H, K, V), **f32)
    else:
        dq, dk, dv, dg, db, dinit = grads
        for name, t, shp in (("dq", dq, (T, H, K)), ("dk", dk, (T, H, K)), ("dv", dv, (T, H, V)),
                             ("dlog_alpha", dg, gshape), ("dbeta", db, (T, H)),
                             ("dinit_state", dinit, (N, H, K, V))):
            _check(t, name, shp, torch.float32, device)
    if workspace is None:
        need = bwd_workspace_size(N, T, H, K, V, dt, segment_tokens, options)
        if need == 0:
            raise KdaError(2 if K not in (32, 64, 128) or V not in (32, 64, 128) else 1,
                           "kda_chunk_bwd_workspace_size_ex")
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if checkpoints is not None:
        nb = int(_lib().kda_chunk_fwd_ckpt_bytes(N, T, H, K, V))
        _check(checkpoints, "checkpoints", (nb // (4 * H * K * V), H, K, V), torch.float32, device)
        st = _lib().kda_chunk_bwd_ckpt(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                       _ptr(init_state), _ptr(cu_seqlens), N, T, H, K, V, code,
                                       int(options), _ptr(d_o), _ptr(d_final_state),
                                       _ptr(checkpoints) if nb else None, _ptr(dq), _ptr(dk),
                                       _ptr(dv), _ptr(dg), _ptr(db), _ptr(dinit), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(device))
        if st != 0:
            raise KdaError(st, "kda_chunk_bwd_ckpt")
        return dq, dk, dv, dg, db, dinit
    st = _lib().kda_chunk_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                 _ptr(init_state), _ptr(cu_seqlens), N, T, H, K, V, code,
                                 int(options), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(dg), _ptr(db), _ptr(dinit), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(device))
    if st != 0:
        raise KdaError(st, "kda_chunk_bwd_ex")
    return dq, dk, dv, dg, db, dinit


def decode_step(q, k, v, log_alpha, beta, state, o=None, options=0):
    """kda_decode_step on torch tensors: q, k, log_alpha [N, H, K], v [N, H, V], beta [N, H],
    state [N, H, K, V] fp32 updated in place. Returns o [N, H, V] in the input dtype.
    ``options`` (OPT_* bits) selects kda_decode_step_ex; with OPT_SCALAR_GATE log_alpha is
    [N, H]."""
    device = q.device
    N, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    gshape = (N, H) if options & OPT_SCALAR_GATE else (N, H, K)
    for name, t, shp in (("q", q, (N, H, K)), ("k", k, (N, H, K)), ("v", v, (N, H, V)),
                         ("log_alpha", log_alpha, gshape), ("beta", beta, (N, H))):
        _check(t, name, shp, dt, device)
    _check(state, "state", (N, H, K, V), torch.float32, device)
    if o is None:
        o = torch.empty((N, H, V), dtype=dt, device=device)
    else:
        _check(o, "o", (N, H, V), dt, device)
    st = _lib().kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                   _ptr(state), _ptr(o), N, H, K, V, code, int(options),
                                   _stream(device))
    if st != 0:
        raise KdaError(st, "kda_decode_step")
    return o
