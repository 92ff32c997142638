"""Gated DeltaNet (gated delta rule) state recurrence on AMD Instinct MI355X.

A thin ctypes binding over ``libgdn.so`` (C ABI in ``include/gdn.h``).  The
functions carry the C names and do argument marshalling only: they read
pointers, element strides and the current HIP stream off torch tensors and call
the library, which runs every step of the path in its own gfx950 kernels.  There
is no fallback: if ``libgdn.so`` is missing or fails to load, every call raises.
``prepare(entry, ...)`` marshals one call once and returns an object that repeats
it, so that a loop over static buffers pays for the C call alone.

Tensor conventions (all fp32 CUDA tensors unless noted, inner dim contiguous):

* ``state``: ``[B, pitch]`` or ``[B, NV, D, D]``; the row stride is the slot
  pitch in elements.  ``gdn_decode_f16state`` takes a ``torch.float16`` pool.
* ``q``, ``k``: ``[rows, >= NK*D]``; ``v``, ``z``: ``[rows, >= NV*D]``;
  ``alpha``, ``beta``: ``[rows, >= NV]`` -- ``rows = B`` for decode and
  ``B*T`` for the sequence (``[B, T, ...]`` is accepted and viewed as rows).
  Row strides may exceed the width (views into a packed projection row).
* ``norm_weight``: ``[D]``.  Outputs are ``[rows, NV*D]`` (allocated when not
  given), fp32 or bf16.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_OK = 0
GDN_F32 = 0
GDN_BF16 = 1
STATUS_NAMES = {
    0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_STRIDE",
    4: "GDN_ERR_UNSUPPORTED", 5: "GDN_ERR_ALIAS", 6: "GDN_ERR_DTYPE", 7: "GDN_ERR_HIP",
    8: "GDN_ERR_ARG", 9: "GDN_ERR_SCRATCH",
}
EXPORTS = ("gdn_decode", "gdn_decode_norm", "gdn_decode_norm_q", "gdn_decode_f16state",
           "gdn_recurrence_seq", "gdn_recurrence_seq_ws", "gdn_recurrence_seq_noalloc",
           "gdn_seq_workspace_bytes",
           "gdn_decode_verify", "gdn_decode_fused", "gdn_state_f32_to_f16",
           "gdn_state_f16_to_f32", "gdn_status_string", "gdn_last_hip_error")
VERIFY_MAX_TOKENS = 8


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib().gdn_status_string(status).decode()
        if status == 7:
            msg += f" (hipError_t {_lib().gdn_last_hip_error()})"
        super().__init__(f"{what}: {msg}")


_LIB = None


def _lib():
    """Load ``libgdn.so`` (once) and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950)")
    # torch carries its own HIP runtime under the same soname as ROCm's.  With torch
    # loaded first, libgdn.so binds to that runtime, so the library and the tensors
    # and streams it is handed share one runtime.  Loaded the other way round, the
    # process held two HIP runtimes and every launch of the library failed
    # (hipErrorNoDevice).
    _torch()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    lib.gdn_decode.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64,
                               i32, i32, i32, i32, i32, vp]
    norm_sig = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, f32, vp, i32, i64,
                i32, i32, i32, i32, i32, vp]
    lib.gdn_decode_norm.argtypes = norm_sig
    lib.gdn_decode_f16state.argtypes = norm_sig
    lib.gdn_recurrence_seq.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp,
                                       f32, vp, i64, i32, i32, i32, i32, i32, i32, vp]
    lib.gdn_recurrence_seq_ws.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp,
                                          f32, vp, i64, i32, i32, i32, i32, i32, i32, vp, i64, vp]
    lib.gdn_recurrence_seq_noalloc.argtypes = lib.gdn_recurrence_seq.argtypes
    lib.gdn_seq_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.gdn_decode_norm_q.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, f32,
                                      vp, i64, vp, i64, vp, i64, i32, i32, i32, i32, i32, vp]
    lib.gdn_decode_fused.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i32, vp, vp, i64, vp, vp, f32,
                                     vp, i64, vp, f32, vp, i64, i32, i32, i32, i32, i32, vp]
    lib.gdn_decode_verify.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64,
                                      vp, f32, vp, i64, i32, i32, i32, i32, i32, i32, vp]
    lib.gdn_state_f32_to_f16.argtypes = [vp, vp, i64, vp]
    lib.gdn_state_f16_to_f32.argtypes = [vp, vp, i64, vp]
    for name in EXPORTS:
        if name not in ("gdn_status_string", "gdn_last_hip_error", "gdn_seq_workspace_bytes"):
            getattr(lib, name).restype = ctypes.c_int
    lib.gdn_seq_workspace_bytes.restype = i64
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_hip_error.argtypes = []
    lib.gdn_last_hip_error.restype = i32
    _LIB = lib
    return lib


def lib():
    """The raw ctypes handle of ``libgdn.so`` (signatures declared)."""
    return _lib()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


_RAW_STREAM = None


def _stream(t, stream):
    """The HIP stream handle: the caller's, else torch's current stream on the
    tensor's device (the raw-handle query avoids building a Stream object on
    every call)."""
    global _RAW_STREAM
    if stream is not None:
        return int(stream)
    if _RAW_STREAM is None:
        torch = _torch()
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or (
            lambda idx: torch.cuda.current_stream(idx).cuda_stream)
    return int(_RAW_STREAM(t.get_device()))


def _rows(t, rows: int, width: int, name: str, dtype=None):
    """(pointer, row stride in elements) of a ``[rows, >= width]`` row array."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() == 2:   # the common case, with one query of shape and strides
        n, wd = t.shape
        s0, s1 = t.stride()
        if n != rows:
            raise ValueError(f"{name}: expected {rows} rows, got {n}")
        if wd < width:
            raise ValueError(f"{name}: rows of {wd} < {width} elements")
        if wd > 1 and s1 != 1:
            raise ValueError(f"{name}: inner dimension must be contiguous")
        return t.data_ptr(), int(s0 if rows > 1 else max(wd, width)), t
    if t.dim() > 2:
        if t.shape[-1] < 1:
            raise ValueError(f"{name} is empty")
        try:
            t = t.view(rows, -1)
        except RuntimeError as e:
            raise ValueError(f"{name} cannot be viewed as {rows} rows: {e}") from None
    if t.dim() == 1:
        t = t.view(1, -1)
    if t.shape[0] != rows:
        raise ValueError(f"{name}: expected {rows} rows, got {t.shape[0]}")
    if t.shape[1] < width:
        raise ValueError(f"{name}: rows of {t.shape[1]} < {width} elements")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: inner dimension must be contiguous")
    stride = t.stride(0) if rows > 1 else max(t.shape[1], width)
    return t.data_ptr(), int(stride), t


def _state(state, batch: int, slot: int, dtype):
    ptr, pitch, _ = _rows(state if state.dim() <= 2 else state.view(state.shape[0], -1),
                          batch, slot, "state", dtype)
    return ptr, pitch


def _check(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


class _Capture(threading.local):
    active = False
    record = None


_CAPTURE = _Capture()


def _invoke(name: str, args: tuple, keep: tuple = ()):
    """Call the library function ``name`` on marshalled ``args``, or, inside
    ``prepare``, record the call instead (with tensors made here that the call
    needs alive)."""
    if _CAPTURE.active:
        _CAPTURE.record = (name, args, keep)
        return
    _check(getattr(_lib(), name)(*args), name)


class PreparedCall:
    """One entry-point call whose arguments were marshalled once by ``prepare``:
    calling it launches the same library call again (same tensors, shapes,
    strides and stream) and returns what the entry point returned."""

    __slots__ = ("_fn", "_args", "_name", "result", "_keep")

    def __init__(self, fn, args, name, result, keep):
        self._fn, self._args, self._name, self.result, self._keep = fn, args, name, result, keep

    def __call__(self):
        status = self._fn(*self._args)
        if status != GDN_OK:
            raise GdnError(status, self._name)
        return self.result


def prepare(entry, *args, **kwargs) -> PreparedCall:
    """Marshal one call of an entry point of this module once, for a loop that
    repeats it on the same buffers (a serving loop's static inputs, outputs and
    state).  ``entry(*args, **kwargs)`` is checked and marshalled as usual but
    not launched; the returned object launches it, for the cost of the C call
    alone.  The stream is the one the call would have used now (``stream=`` or
    torch's current stream).  The object keeps every tensor the call reads or
    writes alive; the caller must not resize or free them, and new contents of
    the same tensors are simply read by the next launch."""
    if _CAPTURE.active:
        raise RuntimeError("prepare cannot be nested")
    _CAPTURE.active, _CAPTURE.record = True, None
    try:
        result = entry(*args, **kwargs)
        record = _CAPTURE.record
    finally:
        _CAPTURE.active, _CAPTURE.record = False, None
    if record is None:
        raise ValueError(f"{getattr(entry, '__name__', entry)} launches nothing to prepare")
    name, cargs, keep = record
    return PreparedCall(getattr(_lib(), name), cargs, name, result, (args, kwargs, keep))


def _dims(gn_or_none, num_k_heads, num_v_heads, head_dim):
    if head_dim is None:
        if gn_or_none is None:
            raise ValueError("head_dim is required")
        head_dim = gn_or_none.shape[0]
    return int(num_k_heads), int(num_v_heads), int(head_dim)


def _empty_rows(rows: int, width: int, dtype, like):
    return _torch().empty((rows, width), dtype=dtype, device=like.device)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def gdn_decode(state, q, k, v, alpha, beta, out=None, *, num_k_heads: int, num_v_heads: int,
               head_dim: int, stream=None):
    """One token: advance ``state`` (fp32) in place and return the raw output o."""
    torch = _torch()
    B = state.shape[0]
    NK, NV, D = _dims(None, num_k_heads, num_v_heads, head_dim)
    if out is None:
        out = _empty_rows(B, NV * D, torch.float32, state)
    sp, pitch = _state(state, B, NV * D * D, torch.float32)
    qp, qs, _ = _rows(q, B, NK * D, "q", torch.float32)
    kp, ks, _ = _rows(k, B, NK * D, "k", torch.float32)
    if qs != ks:
        raise ValueError("q and k must share one row stride")
    vp_, vs, _ = _rows(v, B, NV * D, "v", torch.float32)
    ap, abs_, _ = _rows(alpha, B, NV, "alpha", torch.float32)
    bp, bs, _ = _rows(beta, B, NV, "beta", torch.float32)
    if abs_ != bs:
        raise ValueError("alpha and beta must share one row stride")
    op, os_, _ = _rows(out, B, NV * D, "out", torch.float32)
    _invoke("gdn_decode", (sp, pitch, qp, kp, qs, vp_, vs, ap, bp, abs_, op, os_, B, NK, NV, D, D,
                           _stream(state, stream)))
    return out


def _norm_call(fn_name, state, state_dtype, q, k, v, alpha, beta, z, norm_weight, eps, out,
               out_dtype, num_k_heads, num_v_heads, head_dim, stream, raw_ok):
    torch = _torch()
    B = state.shape[0]
    NK, NV, D = _dims(norm_weight, num_k_heads, num_v_heads, head_dim)
    if z is None and not raw_ok:
        raise ValueError("z is required")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    code = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}.get(out_dtype)
    if code is None:
        raise TypeError(f"unsupported output dtype {out_dtype}")
    if out is None:
        out = _empty_rows(B, NV * D, out_dtype, state)
    sp, pitch = _state(state, B, NV * D * D, state_dtype)
    qp, qs, _ = _rows(q, B, NK * D, "q", torch.float32)
    kp, ks, _ = _rows(k, B, NK * D, "k", torch.float32)
    if qs != ks:
        raise ValueError("q and k must share one row stride")
    vp_, vs, _ = _rows(v, B, NV * D, "v", torch.float32)
    ap, abs_, _ = _rows(alpha, B, NV, "alpha", torch.float32)
    bp, bs, _ = _rows(beta, B, NV, "beta", torch.float32)
    if abs_ != bs:
        raise ValueError("alpha and beta must share one row stride")
    if z is not None:
        zp, zs, _ = _rows(z, B, NV * D, "z", torch.float32)
        if norm_weight is None or norm_weight.dtype != torch.float32 or norm_weight.numel() < D:
            raise ValueError("norm_weight must be fp32 [D]")
        gp = norm_weight.data_ptr()
    else:
        zp, zs, gp = None, 0, None
    op, os_, _ = _rows(out, B, NV * D, "out", out_dtype)
    _invoke(fn_name, (sp, pitch, qp, kp, qs, vp_, vs, ap, bp, abs_, zp, zs, gp, float(eps), op, code,
                      os_, B, NK, NV, D, D, _stream(state, stream)))
    return out


def gdn_decode_norm(state, q, k, v, alpha, beta, z, norm_weight, eps: float = 1e-6, out=None, *,
                    out_dtype=None, num_k_heads: int, num_v_heads: int,
                    head_dim: Optional[int] = None, stream=None):
    """One token with the fused gated RMS norm; returns y (fp32 or bf16)."""
    return _norm_call("gdn_decode_norm", state, _torch().float32, q, k, v, alpha, beta, z,
                      norm_weight, eps, out, out_dtype, num_k_heads, num_v_heads, head_dim,
                      stream, raw_ok=False)


def gdn_decode_norm_q(state, q, k, v, alpha, beta, z, norm_weight, eps: float = 1e-6, out=None,
                      codes=None, scales=None, *, write_y: bool = True, num_k_heads: int,
                      num_v_heads: int, head_dim: Optional[int] = None, stream=None):
    """One token with the fused gated RMS norm and int8 group quantisation of y.

    Returns ``(y or None, codes int8 [B, NV*D], scales fp32 [B, NV*D/32])``; with
    ``write_y=False`` (and no ``out``) y is not written at all."""
    torch = _torch()
    B = state.shape[0]
    NK, NV, D = _dims(norm_weight, num_k_heads, num_v_heads, head_dim)
    if out is None and write_y:
        out = _empty_rows(B, NV * D, torch.float32, state)
    if codes is None:
        codes = _empty_rows(B, NV * D, torch.int8, state)
    if scales is None:
        scales = _empty_rows(B, max(NV * D // 32, 1), torch.float32, state)
    sp, pitch = _state(state, B, NV * D * D, torch.float32)
    qp, qs, _ = _rows(q, B, NK * D, "q", torch.float32)
    kp, ks, _ = _rows(k, B, NK * D, "k", torch.float32)
    if qs != ks:
        raise ValueError("q and k must share one row stride")
    vp_, vs, _ = _rows(v, B, NV * D, "v", torch.float32)
    ap, abs_, _ = _rows(alpha, B, NV, "alpha", torch.float32)
    bp, bs, _ = _rows(beta, B, NV, "beta", torch.float32)
    if abs_ != bs:
        raise ValueError("alpha and beta must share one row stride")
    zp, zs, _ = _rows(z, B, NV * D, "z", torch.float32)
    if norm_weight is None or norm_weight.dtype != torch.float32:
        raise ValueError("norm_weight must be fp32 [D]")
    if out is not None:
        op, os_, _ = _rows(out, B, NV * D, "out", torch.float32)
    else:
        op, os_ = None, 0
    cp, cs, _ = _rows(codes, B, NV * D, "codes", torch.int8)
    scp, scs, _ = _rows(scales, B, NV * D // 32, "scales", torch.float32)
    _invoke("gdn_decode_norm_q", (sp, pitch, qp, kp, qs, vp_, vs, ap, bp, abs_, zp, zs,
                                  norm_weight.data_ptr(), float(eps), op, os_, cp, cs, scp, scs,
                                  B, NK, NV, D, D, _stream(state, stream)))
    return out, codes, scales


def gdn_decode_f16state(state, q, k, v, alpha, beta, z=None, norm_weight=None, eps: float = 1e-6,
                        out=None, *, out_dtype=None, num_k_heads: int, num_v_heads: int,
                        head_dim: Optional[int] = None, stream=None):
    """One token on a binary16 (``torch.float16``) state pool; y, or raw o if z is None."""
    return _norm_call("gdn_decode_f16state", state, _torch().float16, q, k, v, alpha, beta, z,
                      norm_weight, eps, out, out_dtype, num_k_heads, num_v_heads, head_dim,
                      stream, raw_ok=True)


def _seq_args(state, q, k, v, alpha, beta, z, norm_weight, out, seq_len, num_k_heads, num_v_heads,
              head_dim):
    torch = _torch()
    B = state.shape[0]
    T = int(seq_len)
    NK, NV, D = _dims(norm_weight, num_k_heads, num_v_heads, head_dim)
    rows = B * T
    if out is None:
        out = _empty_rows(rows, NV * D, torch.float32, state)
    sp, pitch = _state(state, B, NV * D * D, torch.float32)
    qp, qs, _ = _rows(q, rows, NK * D, "q", torch.float32)
    kp, ks, _ = _rows(k, rows, NK * D, "k", torch.float32)
    if qs != ks:
        raise ValueError("q and k must share one row stride")
    vp_, vs, _ = _rows(v, rows, NV * D, "v", torch.float32)
    ap, abs_, _ = _rows(alpha, rows, NV, "alpha", torch.float32)
    bp, bs, _ = _rows(beta, rows, NV, "beta", torch.float32)
    if abs_ != bs:
        raise ValueError("alpha and beta must share one row stride")
    if z is not None:
        zp, zs, _ = _rows(z, rows, NV * D, "z", torch.float32)
        if norm_weight is None or norm_weight.dtype != torch.float32:
            raise ValueError("norm_weight must be fp32 [D]")
        gp = norm_weight.data_ptr()
    else:
        zp, zs, gp = None, 0, None
    op, os_, _ = _rows(out, rows, NV * D, "out", torch.float32)
    head = (sp, pitch, qp, kp, qs, vp_, vs, ap, bp, abs_, zp, zs, gp)
    tail = (op, os_, B, T, NK, NV, D, D)
    return out, head, tail


def gdn_recurrence_seq(state, q, k, v, alpha, beta, z=None, norm_weight=None, eps: float = 1e-6,
                       out=None, *, seq_len: int, num_k_heads: int, num_v_heads: int,
                       head_dim: Optional[int] = None, stream=None):
    """``seq_len`` tokens per sequence with the state on chip; returns o (or y) rows."""
    out, head, tail = _seq_args(state, q, k, v, alpha, beta, z, norm_weight, out, seq_len,
                                num_k_heads, num_v_heads, head_dim)
    _invoke("gdn_recurrence_seq", (*head, float(eps), *tail, _stream(state, stream)))
    return out


def gdn_seq_workspace_bytes(batch: int, seq_len: int, num_v_heads: int, head_dim: int) -> int:
    """Bytes of workspace ``gdn_recurrence_seq_ws`` uses for this shape (0: none)."""
    n = int(_lib().gdn_seq_workspace_bytes(int(batch), int(seq_len), int(num_v_heads),
                                           int(head_dim), int(head_dim)))
    if n < 0:
        raise ValueError("invalid sequence shape")
    return n


def gdn_recurrence_seq_ws(state, q, k, v, alpha, beta, z=None, norm_weight=None,
                          eps: float = 1e-6, out=None, workspace=None, *, seq_len: int,
                          num_k_heads: int, num_v_heads: int, head_dim: Optional[int] = None,
                          stream=None):
    """``gdn_recurrence_seq`` with a device workspace (a uint8 tensor of at least
    ``gdn_seq_workspace_bytes`` bytes; allocated here when not given)."""
    torch = _torch()
    out, head, tail = _seq_args(state, q, k, v, alpha, beta, z, norm_weight, out, seq_len,
                                num_k_heads, num_v_heads, head_dim)
    B, T, NV, D = tail[2], tail[3], tail[5], tail[6]
    need = gdn_seq_workspace_bytes(B, T, NV, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=state.device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    _invoke("gdn_recurrence_seq_ws", (*head, float(eps), *tail, workspace.data_ptr(), nbytes,
                                      _stream(state, stream)), keep=(workspace,))
    return out


# bytes of the library's static scratch behind gdn_recurrence_seq_noalloc, per GPU
SEQ_NOALLOC_MAX_BYTES = 64 << 20


def gdn_recurrence_seq_noalloc(state, q, k, v, alpha, beta, z=None, norm_weight=None,
                               eps: float = 1e-6, out=None, *, seq_len: int, num_k_heads: int,
                               num_v_heads: int, head_dim: Optional[int] = None, stream=None):
    """``gdn_recurrence_seq_ws`` with the workspace in the library's static
    scratch (at most ``SEQ_NOALLOC_MAX_BYTES``); calls on one GPU must not
    overlap.  ``out`` is allocated here when not given."""
    out, head, tail = _seq_args(state, q, k, v, alpha, beta, z, norm_weight, out, seq_len,
                                num_k_heads, num_v_heads, head_dim)
    _invoke("gdn_recurrence_seq_noalloc", (*head, float(eps), *tail, _stream(state, stream)))
    return out


def gdn_decode_verify(state, q, k, v, alpha, beta, z=None, norm_weight=None, eps: float = 1e-6,
                      out=None, inter_state=None, *, num_tokens: int, num_k_heads: int,
                      num_v_heads: int, head_dim: Optional[int] = None, stream=None):
    """``num_tokens`` tokens per sequence in one launch; returns ``(out, inter_state)``.

    ``inter_state`` (allocated when not given, fp32 ``[B*(num_tokens-1), pitch]``)
    receives the state after each token but the last, slot ``b*(num_tokens-1)+t``."""
    torch = _torch()
    B = state.shape[0]
    T = int(num_tokens)
    NK, NV, D = _dims(norm_weight, num_k_heads, num_v_heads, head_dim)
    rows = B * T
    if out is None:
        out = _empty_rows(rows, NV * D, torch.float32, state)
    if inter_state is None and T > 1:
        inter_state = torch.empty((B * (T - 1), NV * D * D), dtype=torch.float32, device=state.device)
    sp, pitch = _state(state, B, NV * D * D, torch.float32)
    if T > 1:
        ip, ipitch = _state(inter_state, B * (T - 1), NV * D * D, torch.float32)
    else:
        ip, ipitch = None, 0
    qp, qs, _ = _rows(q, rows, NK * D, "q", torch.float32)
    kp, ks, _ = _rows(k, rows, NK * D, "k", torch.float32)
    if qs != ks:
        raise ValueError("q and k must share one row stride")
    vp_, vs, _ = _rows(v, rows, NV * D, "v", torch.float32)
    ap, abs_, _ = _rows(alpha, rows, NV, "alpha", torch.float32)
    bp, bs, _ = _rows(beta, rows, NV, "beta", torch.float32)
    if abs_ != bs:
        raise ValueError("alpha and beta must share one row stride")
    if z is not None:
        zp, zs, _ = _rows(z, rows, NV * D, "z", torch.float32)
        if norm_weight is None or norm_weight.dtype != torch.float32:
            raise ValueError("norm_weight must be fp32 [D]")
        gp = norm_weight.data_ptr()
    else:
        zp, zs, gp = None, 0, None
    op, os_, _ = _rows(out, rows, NV * D, "out", torch.float32)
    _invoke("gdn_decode_verify", (sp, pitch, ip, ipitch, qp, kp, qs, vp_, vs, ap, bp, abs_, zp, zs,
                                  gp, float(eps), op, os_, B, T, NK, NV, D, D,
                                  _stream(state, stream)))
    return out, inter_state


def gdn_decode_fused(state, conv_state, x, conv_weight, br, ar, dt_bias, decay_rate, z=None,
                     norm_weight=None, eps: float = 1e-6, l2_eps: float = 1e-6, out=None,
                     conv_state_out=None, *, num_k_heads: int, num_v_heads: int,
                     head_dim: Optional[int] = None, stream=None):
    """One token with the input stage fused in front of the step.

    ``x`` holds the projection rows ``[B, >= C]`` (channels q | k | v, before the
    conv), ``conv_state`` the rings ``[B, taps*C]`` (or ``[B, taps, C]``, updated),
    ``conv_weight`` ``[taps, C]``, ``br``/``ar`` ``[B, >= NV]`` and
    ``dt_bias``/``decay_rate`` ``[NV]``.  With ``conv_state_out`` (same shape and
    row stride as ``conv_state``) the new ring goes there and ``conv_state`` is
    only read.  Returns o, or y when ``z`` is given."""
    torch = _torch()
    B = state.shape[0]
    NK, NV, D = _dims(norm_weight, num_k_heads, num_v_heads, head_dim)
    C = (2 * NK + NV) * D
    if conv_weight.dim() != 2 or conv_weight.shape[1] != C or not conv_weight.is_contiguous():
        raise ValueError(f"conv_weight must be contiguous [taps, {C}]")
    taps = conv_weight.shape[0]
    if out is None:
        out = _empty_rows(B, NV * D, torch.float32, state)
    sp, pitch = _state(state, B, NV * D * D, torch.float32)
    rp, rpitch = _state(conv_state, B, taps * C, torch.float32)
    if conv_state_out is not None:
        rop, ropitch = _state(conv_state_out, B, taps * C, torch.float32)
        if B > 1 and ropitch != rpitch:
            raise ValueError("conv_state_out must have conv_state's row stride")
    else:
        rop = None
    xp, xs, _ = _rows(x, B, C, "x", torch.float32)
    bp, bs, _ = _rows(br, B, NV, "br", torch.float32)
    ap, as_, _ = _rows(ar, B, NV, "ar", torch.float32)
    if bs != as_:
        raise ValueError("br and ar must share one row stride")
    for t, n in ((dt_bias, "dt_bias"), (decay_rate, "decay_rate"), (conv_weight, "conv_weight")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous fp32 device tensor")
    if dt_bias.numel() != NV or decay_rate.numel() != NV:
        raise ValueError("dt_bias and decay_rate must hold num_v_heads values")
    if z is not None:
        zp, zs, _ = _rows(z, B, NV * D, "z", torch.float32)
        if norm_weight is None or norm_weight.dtype != torch.float32:
            raise ValueError("norm_weight must be fp32 [D]")
        gp = norm_weight.data_ptr()
    else:
        zp, zs, gp = None, 0, None
    op, os_, _ = _rows(out, B, NV * D, "out", torch.float32)
    _invoke("gdn_decode_fused", (sp, pitch, rp, rpitch, rop, xp, xs, conv_weight.data_ptr(), taps, bp,
                                 ap, bs, dt_bias.data_ptr(), decay_rate.data_ptr(), float(l2_eps),
                                 zp, zs, gp, float(eps), op, os_, B, NK, NV, D, D,
                                 _stream(state, stream)))
    return out


def gdn_state_f32_to_f16(src, dst=None, stream=None):
    """fp32 -> binary16 (RNE) over a whole pool; returns a ``torch.float16`` tensor."""
    torch = _torch()
    if src.dtype != torch.float32 or not src.is_contiguous():
        raise ValueError("src must be a contiguous fp32 tensor")
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.float16, device=src.device)
    if dst.dtype != torch.float16 or not dst.is_contiguous() or dst.numel() != src.numel():
        raise ValueError("dst must be a contiguous float16 tensor of the same size")
    _invoke("gdn_state_f32_to_f16", (src.data_ptr(), dst.data_ptr(), src.numel(), _stream(src, stream)))
    return dst


def gdn_state_f16_to_f32(src, dst=None, stream=None):
    """binary16 -> fp32 (exact) over a whole pool."""
    torch = _torch()
    if src.dtype != torch.float16 or not src.is_contiguous():
        raise ValueError("src must be a contiguous float16 tensor")
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.float32, device=src.device)
    if dst.dtype != torch.float32 or not dst.is_contiguous() or dst.numel() != src.numel():
        raise ValueError("dst must be a contiguous fp32 tensor of the same size")
    _invoke("gdn_state_f16_to_f32", (src.data_ptr(), dst.data_ptr(), src.numel(), _stream(src, stream)))
    return dst
