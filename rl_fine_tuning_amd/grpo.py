"""Thin Python binding of the C ABI in include/grpo.h (ctypes).

Argument marshalling only: tensors are torch device tensors, passed by pointer with
the current HIP stream; every step of the computation runs in the HIP library.  The
binding fails loudly when the library has not been built.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

from .build import LIB_PATH

GRPO_OK = 0
GRPO_BF16, GRPO_F32 = 0, 1
GRPO_AGG = {"seq_mean": 0, "token_mean": 1}
GRPO_STD = {"unbiased": 0, "population": 1}
KERNELS = ["target_logit", "logits_lse", "merge", "probs", "dh_gemm", "dh_reduce", "token_index",
           "loss_finalize", "advantages", "frag_copy", "transpose_w", "probs_kept", "onehot_fix", "ht_copy",
           "dw_gemm", "w_copy", "qt_band"]
KERNEL_ID = {k: i for i, k in enumerate(KERNELS)}


class GrpoShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int64), ("V", ctypes.c_int64),
                ("chunk_tokens", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("logit_scale_multiply", ctypes.c_float),
                ("logit_scale_divide", ctypes.c_float), ("logit_softcapping", ctypes.c_float),
                ("keep_chunk_logits", ctypes.c_int32), ("dh_fp32", ctypes.c_int32)]


class GrpoLossParams(ctypes.Structure):
    _fields_ = [("clip_eps_low", ctypes.c_float), ("clip_eps_high", ctypes.c_float),
                ("beta", ctypes.c_float), ("agg", ctypes.c_int32)]


class GrpoError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().grpo_status_string(status).decode()} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rl_fine_tuning_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                 ctypes.c_size_t)
        sp = ctypes.POINTER(GrpoShape)
        L.grpo_workspace_bytes.argtypes = [sp, i64, ctypes.c_int]
        L.grpo_workspace_bytes.restype = sz
        L.grpo_plan_info.argtypes = [sp, i64, ctypes.c_int, ctypes.POINTER(i64)]
        L.grpo_plan_info.restype = ctypes.c_int
        L.grpo_logp_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.grpo_logp_fwd.restype = ctypes.c_int
        L.grpo_advantages.argtypes = [vp, i64, i64, i32, f32, vp, vp]
        L.grpo_advantages.restype = ctypes.c_int
        L.grpo_loss_fwd_bwd.argtypes = [sp, ctypes.POINTER(GrpoLossParams), vp, vp, vp, vp, i64, vp, vp,
                                        vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.grpo_loss_fwd_bwd.restype = ctypes.c_int
        L.grpo_loss_fwd_bwd_static.argtypes = [sp, ctypes.POINTER(GrpoLossParams), vp, vp, vp, vp, i64, vp, vp,
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.grpo_loss_fwd_bwd_static.restype = ctypes.c_int
        L.grpo_logp_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.grpo_logp_bwd.restype = ctypes.c_int
        L.grpo_ce_loss_fwd_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.grpo_ce_loss_fwd_bwd.restype = ctypes.c_int
        L.grpo_status_string.argtypes = [ctypes.c_int]
        L.grpo_status_string.restype = ctypes.c_char_p
        L.grpo_debug_token_index.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]
        L.grpo_debug_token_index.restype = ctypes.c_int
        L.grpo_timer_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.grpo_timer_create.restype = ctypes.c_int
        L.grpo_timer_destroy.argtypes = [vp]
        L.grpo_timer_destroy.restype = ctypes.c_int
        L.grpo_timer_reset.argtypes = [vp]
        L.grpo_timer_reset.restype = ctypes.c_int
        L.grpo_timer_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                                      ctypes.POINTER(i64)]
        L.grpo_timer_read.restype = ctypes.c_int
        L.grpo_offload_create.argtypes = [ctypes.POINTER(vp)]
        L.grpo_offload_create.restype = ctypes.c_int
        L.grpo_offload_destroy.argtypes = [vp]
        L.grpo_offload_destroy.restype = ctypes.c_int
        L.grpo_logp_fwd_offload.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.grpo_logp_fwd_offload.restype = ctypes.c_int
        L.grpo_logp_bwd_offload.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.grpo_logp_bwd_offload.restype = ctypes.c_int
        L.grpo_version.argtypes = []
        L.grpo_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != GRPO_OK:
        raise GrpoError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Allocations made under this context belong to the call's stream, so the caching
    allocator never hands a buffer the call's kernels still use to work on another stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GRPO_BF16
    if t.dtype == torch.float32:
        return GRPO_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _is_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _dev(t, name: str, device=None, dtype=None, shape=None):
    """Check a tensor argument before its pointer reaches the library: a device tensor on
    `device`, contiguous, of one of the dtypes in `dtype` and of shape `shape` (when given)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise TypeError(f"{name} must be {' or '.join(str(d) for d in allowed)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


_MASK = (torch.uint8, torch.bool)


def _hw(H, W, targets):
    """Shapes of the common inputs: H [T, D] bf16 or fp32, W [V, D] of H's dtype, targets int32 [T]."""
    _dev(H, "H", dtype=(torch.bfloat16, torch.float32))
    if H.dim() != 2:
        raise ValueError(f"H must be [T, D], got shape {tuple(H.shape)}")
    T, D = H.shape
    _dev(W, "W", H.device, H.dtype)
    if W.dim() != 2 or W.shape[1] != D:
        raise ValueError(f"W must be [V, {D}], got shape {tuple(W.shape)}")
    _dev(targets, "targets", H.device, torch.int32, (T,))
    return int(T), int(D), int(W.shape[0])


def make_shape(T, D, V, chunk_tokens, dtype, temperature=1.0, logit_scale_multiply=0.0, logit_scale_divide=0.0,
               logit_softcapping=0.0, keep_chunk_logits=False, dh_fp32=False) -> GrpoShape:
    """0 for a logit argument means 'not used' (see grpo_shape in include/grpo.h)."""
    return GrpoShape(int(T), int(D), int(V), int(chunk_tokens), int(dtype), float(temperature),
                     float(logit_scale_multiply), float(logit_scale_divide), float(logit_softcapping),
                     int(bool(keep_chunk_logits)), int(bool(dh_fp32)))


def _dh_dtype(H, dh_fp32):
    return torch.float32 if dh_fp32 else H.dtype


GRPO_WS_HOST_H = 4


def _bwd_mode(with_backward, with_dW, host_h=False):
    mode = 2 if with_dW else int(bool(with_backward))
    return mode | (GRPO_WS_HOST_H if host_h else 0)


def grpo_workspace_bytes(T, D, V, chunk_tokens, dtype=GRPO_BF16, temperature=1.0, num_seqs=1,
                         with_backward=True, logit_softcapping=0.0, keep_chunk_logits=False,
                         with_dW=False, dh_fp32=False, host_h=False) -> int:
    """host_h: the workspace of grpo_logp_bwd_offload (H in pinned host memory)."""
    shape = make_shape(T, D, V, chunk_tokens, dtype, temperature, logit_softcapping=logit_softcapping,
                       keep_chunk_logits=keep_chunk_logits, dh_fp32=dh_fp32)
    return int(lib().grpo_workspace_bytes(ctypes.byref(shape), int(num_seqs),
                                          _bwd_mode(with_backward, with_dW, host_h)))


def grpo_plan_info(T, D, V, chunk_tokens, dtype=GRPO_BF16, temperature=1.0, num_seqs=1, with_backward=True,
                   logit_softcapping=0.0, keep_chunk_logits=False, with_dW=False, dh_fp32=False,
                   host_h=False) -> dict:
    """The library's workspace layout for a call: which fragment-major copies of W it keeps,
    the tokens per backward slice and the workspace bytes."""
    shape = make_shape(T, D, V, chunk_tokens, dtype, temperature, logit_softcapping=logit_softcapping,
                       keep_chunk_logits=keep_chunk_logits, dh_fp32=dh_fp32)
    info = (ctypes.c_int64 * 4)()
    st = lib().grpo_plan_info(ctypes.byref(shape), int(num_seqs), _bwd_mode(with_backward, with_dW, host_h), info)
    _check(st, "grpo_plan_info")
    return dict(w_transposed_copy=int(info[0]) == 1, w_transposed_bands=int(info[0]) if info[0] >= 2 else 0,
                w_copy=bool(info[1]), backward_slice_tokens=int(info[2]),
                workspace_bytes=int(info[3]))


def _workspace(nbytes, workspace, device):
    """The caller's workspace (a uint8 device tensor of at least nbytes) or a new one."""
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", device, torch.uint8)
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace too small: {workspace.numel()} bytes, the call needs {nbytes}")
    return workspace, workspace.numel()


def _out(t, name, device, dtype, shape):
    """A caller-given output (checked) or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name, device, dtype, shape)
    return t


def _want_dW(dW, V, D, device):
    """dW argument: None/False = not computed, True = allocate, or an fp32 [V, D] tensor."""
    if dW is None or dW is False:
        return None
    if dW is True:
        return torch.empty(V, D, dtype=torch.float32, device=device)
    _dev(dW, "dW", device, torch.float32, (V, D))
    return dW


class Timer:
    """Per-launch event timing of the library's kernels (see grpo_timer_* in grpo.h)."""

    def __init__(self, capacity: int = 8192):
        h = ctypes.c_void_p()
        _check(lib().grpo_timer_create(int(capacity), ctypes.byref(h)), "grpo_timer_create")
        self.handle = h

    def reset(self):
        _check(lib().grpo_timer_reset(self.handle), "grpo_timer_reset")

    def read(self, kernel: str):
        ms, n, dropped = ctypes.c_double(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().grpo_timer_read(self.handle, KERNEL_ID[kernel], ctypes.byref(ms), ctypes.byref(n),
                                     ctypes.byref(dropped)), "grpo_timer_read")
        return ms.value, n.value, dropped.value

    def close(self):
        if self.handle:
            lib().grpo_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def grpo_logp_fwd(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, chunk_tokens: int,
                  temperature: float = 1.0, *, logit_scale_multiply=0.0, logit_scale_divide=0.0,
                  logit_softcapping=0.0, return_lse: bool = False, out=None, lse=None, workspace=None,
                  stream=None, timer: Timer | None = None):
    """logp[t] = log softmax(H[t] W^T / temperature)[targets[t]] (fp32), chunked.  With
    return_lse (or an fp32 [T] `lse` given) also the per-token log-sum-exp."""
    T, D, V = _hw(H, W, targets)
    dev = H.device
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping)
    nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 0))
    with _on(stream):
        ws, wsn = _workspace(nbytes, workspace, dev)
        logp = _out(out, "out", dev, torch.float32, (T,))
        return_lse = return_lse or lse is not None
        lse = _out(lse, "lse", dev, torch.float32, (T,)) if return_lse else None
        st = lib().grpo_logp_fwd(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(logp), _ptr(lse),
                                 _ptr(ws), wsn, _stream(stream), timer.handle if timer else None)
    _check(st, "grpo_logp_fwd")
    return (logp, lse) if return_lse else logp


def grpo_logp_bwd(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor,
                  grad_logp: torch.Tensor, chunk_tokens: int, temperature: float = 1.0, *,
                  logit_scale_multiply=0.0, logit_scale_divide=0.0, logit_softcapping=0.0, dh_fp32=False, dH=None,
                  dW=None, workspace=None, stream=None, timer: Timer | None = None):
    """dH of sum_t grad_logp[t] * logp_t, recomputing each chunk's logits from the forward's lse.
    With dW (an fp32 [V, D] tensor, or True to allocate one) returns (dH, dW).  A caller's
    workspace must hold grpo_workspace_bytes(..., with_dW=bool(dW)) bytes."""
    T, D, V = _hw(H, W, targets)
    dev = H.device
    _dev(lse, "lse", dev, torch.float32, (T,))
    _dev(grad_logp, "grad_logp", dev, torch.float32, (T,))
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping, dh_fp32=dh_fp32)
    with _on(stream):
        dW = _want_dW(dW, V, D, dev)
        nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 2 if dW is not None else 1))
        ws, wsn = _workspace(nbytes, workspace, dev)
        dH = _out(dH, "dH", dev, _dh_dtype(H, dh_fp32), (T, D))
        st = lib().grpo_logp_bwd(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(lse), _ptr(grad_logp),
                                 _ptr(dH), _ptr(dW), _ptr(ws), wsn, _stream(stream), timer.handle if timer else None)
    _check(st, "grpo_logp_bwd")
    return (dH, dW) if dW is not None else dH


class Offload:
    """A host-offload context (grpo_offload_* in grpo.h): a copy stream and its events on the
    current device.  One call at a time."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().grpo_offload_create(ctypes.byref(h)), "grpo_offload_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib().grpo_offload_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _pinned(t, name, dtype, shape):
    """A pinned host tensor (torch.empty(..., pin_memory=True)) of dtype and shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def grpo_logp_fwd_offload(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, chunk_tokens: int,
                          offload: Offload, temperature: float = 1.0, *, H_host=None, logit_scale_multiply=0.0,
                          logit_scale_divide=0.0, logit_softcapping=0.0, out=None, lse=None, workspace=None,
                          stream=None, timer: Timer | None = None):
    """grpo_logp_fwd, and H copied to pinned host memory beside the GEMMs (H_host: a pinned
    tensor like H, or None to allocate one).  Returns (logp, lse, H_host)."""
    T, D, V = _hw(H, W, targets)
    dev = H.device
    if H_host is None:
        H_host = torch.empty((T, D), dtype=H.dtype, pin_memory=True)
    _pinned(H_host, "H_host", H.dtype, (T, D))
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping)
    nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 0))
    with _on(stream):
        ws, wsn = _workspace(nbytes, workspace, dev)
        logp = _out(out, "out", dev, torch.float32, (T,))
        lse = _out(lse, "lse", dev, torch.float32, (T,))
        st = lib().grpo_logp_fwd_offload(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(logp),
                                         _ptr(lse), _ptr(H_host), _ptr(ws), wsn, _stream(stream),
                                         timer.handle if timer else None, offload.handle)
    _check(st, "grpo_logp_fwd_offload")
    return logp, lse, H_host


def grpo_logp_bwd_offload(H_host: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor,
                          grad_logp: torch.Tensor, chunk_tokens: int, offload: Offload, temperature: float = 1.0, *,
                          logit_scale_multiply=0.0, logit_scale_divide=0.0, logit_softcapping=0.0, dh_fp32=False,
                          dH=None, dW=None, workspace=None, stream=None, timer: Timer | None = None):
    """grpo_logp_bwd with H in pinned host memory (H_host [T, D], W's dtype): each chunk's rows
    are brought to the GPU during the previous chunk's work.  Returns dH, or (dH, dW)."""
    _dev(W, "W", dtype=(torch.bfloat16, torch.float32))
    if W.dim() != 2:
        raise ValueError(f"W must be [V, D], got shape {tuple(W.shape)}")
    V, D = int(W.shape[0]), int(W.shape[1])
    if not isinstance(H_host, torch.Tensor) or H_host.dim() != 2 or H_host.shape[1] != D:
        raise ValueError(f"H_host must be a [T, {D}] tensor")
    T = int(H_host.shape[0])
    _pinned(H_host, "H_host", W.dtype, (T, D))
    dev = W.device
    _dev(targets, "targets", dev, torch.int32, (T,))
    _dev(lse, "lse", dev, torch.float32, (T,))
    _dev(grad_logp, "grad_logp", dev, torch.float32, (T,))
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(W), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping, dh_fp32=dh_fp32)
    with _on(stream):
        dW = _want_dW(dW, V, D, dev)
        nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1,
                                                _bwd_mode(True, dW is not None, host_h=True)))
        ws, wsn = _workspace(nbytes, workspace, dev)
        dH = _out(dH, "dH", dev, torch.float32 if dh_fp32 else W.dtype, (T, D))
        st = lib().grpo_logp_bwd_offload(ctypes.byref(shape), _ptr(H_host), _ptr(W), _ptr(targets), _ptr(lse),
                                         _ptr(grad_logp), _ptr(dH), _ptr(dW), _ptr(ws), wsn, _stream(stream),
                                         timer.handle if timer else None, offload.handle)
    _check(st, "grpo_logp_bwd_offload")
    return (dH, dW) if dW is not None else dH


def grpo_ce_loss_fwd_bwd(H, W, targets, chunk_tokens, *, temperature=1.0, logit_scale_multiply=0.0,
                         logit_scale_divide=0.0, logit_softcapping=0.0, keep_chunk_logits=False, dh_fp32=False,
                         mask=None, want_logp=True, want_token_loss=False, loss=None, logp=None, token_loss=None,
                         dH=None, dW=None, workspace=None, stream=None, timer: Timer | None = None):
    """Mean cross-entropy over the unmasked tokens, per-token logp, dL/dH and (with dW: an
    fp32 [V, D] tensor, or True to allocate one) dL/dW.  A caller's workspace must hold
    grpo_workspace_bytes(..., with_dW=bool(dW)) bytes."""
    T, D, V = _hw(H, W, targets)
    dev = H.device
    if mask is not None:
        _dev(mask, "mask", dev, _MASK, (T,))
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping, keep_chunk_logits, dh_fp32)
    with _on(stream):
        dW = _want_dW(dW, V, D, dev)
        nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 2 if dW is not None else 1))
        ws, wsn = _workspace(nbytes, workspace, dev)
        loss = _out(loss, "loss", dev, torch.float64, (1,))
        logp = _out(logp, "logp", dev, torch.float32, (T,)) if want_logp or logp is not None else None
        tl = (_out(token_loss, "token_loss", dev, torch.float32, (T,))
              if want_token_loss or token_loss is not None else None)
        dH = _out(dH, "dH", dev, _dh_dtype(H, dh_fp32), (T, D))
        st = lib().grpo_ce_loss_fwd_bwd(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(mask),
                                        _ptr(loss), _ptr(logp), _ptr(tl), _ptr(dH), _ptr(dW), _ptr(ws), wsn,
                                        _stream(stream), timer.handle if timer else None)
    _check(st, "grpo_ce_loss_fwd_bwd")
    return dict(loss=loss, logp=logp, token_loss=tl, dH=dH, dW=dW)


def grpo_advantages(rewards: torch.Tensor, group_size: int, std_mode: str = "unbiased", eps: float = 1e-4,
                    *, out=None, stream=None) -> torch.Tensor:
    _dev(rewards, "rewards", dtype=torch.float32)
    if rewards.dim() != 1:
        raise ValueError(f"rewards must be [S], got shape {tuple(rewards.shape)}")
    with _on(stream):
        adv = _out(out, "out", rewards.device, torch.float32, tuple(rewards.shape))
        st = lib().grpo_advantages(_ptr(rewards), rewards.numel(), int(group_size), GRPO_STD[std_mode], float(eps),
                                   _ptr(adv), _stream(stream))
    _check(st, "grpo_advantages")
    return adv


def _loss_call(static, H, W, targets, cu_seqlens, old_logp, ref_logp, adv, chunk_tokens, *, temperature,
               logit_scale_multiply, logit_scale_divide, logit_softcapping, keep_chunk_logits, dh_fp32, clip_eps_low,
               clip_eps_high, beta, agg, mask, want_logp, want_token_loss, loss, logp, token_loss, dH, dW,
               workspace, stream, timer):
    T, D, V = _hw(H, W, targets)
    dev = H.device
    cu = torch.as_tensor(cu_seqlens).cpu()
    if cu.dim() != 1 or cu.numel() < 2 or cu.dtype not in (torch.int32, torch.int64):
        raise ValueError("cu_seqlens must be a 1-D integer array of S + 1 offsets")
    cu = cu.to(torch.int32).contiguous()
    S = cu.numel() - 1
    _dev(old_logp, "old_logp", dev, torch.float32, (T,))
    if ref_logp is not None:
        _dev(ref_logp, "ref_logp", dev, torch.float32, (T,))
    _dev(adv, "adv", dev, torch.float32, (S,))
    if mask is not None:
        _dev(mask, "mask", dev, _MASK, (T,))
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping, keep_chunk_logits, dh_fp32)
    params = GrpoLossParams(float(clip_eps_low), float(clip_eps_high), float(beta), GRPO_AGG[agg])
    with _on(stream):
        dW = _want_dW(dW, V, D, dev)
        loss = _out(loss, "loss", dev, torch.float64, (1,))
        logp = _out(logp, "logp", dev, torch.float32, (T,)) if want_logp or logp is not None else None
        tl = (_out(token_loss, "token_loss", dev, torch.float32, (T,))
              if want_token_loss or token_loss is not None else None)
        dH = _out(dH, "dH", dev, _dh_dtype(H, dh_fp32), (T, D))
        args = [ctypes.byref(shape), ctypes.byref(params), _ptr(H), _ptr(W), _ptr(targets),
                ctypes.c_void_p(cu.data_ptr()), S, _ptr(mask), _ptr(old_logp), _ptr(ref_logp), _ptr(adv),
                _ptr(loss), _ptr(logp), _ptr(tl), _ptr(dH), _ptr(dW)]
        if static:
            st = lib().grpo_loss_fwd_bwd_static(*args, _stream(stream), timer.handle if timer else None)
        else:
            nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), S, 2 if dW is not None else 1))
            ws, wsn = _workspace(nbytes, workspace, dev)
            st = lib().grpo_loss_fwd_bwd(*args, _ptr(ws), wsn, _stream(stream), timer.handle if timer else None)
    _check(st, "grpo_loss_fwd_bwd_static" if static else "grpo_loss_fwd_bwd")
    return dict(loss=loss, logp=logp, token_loss=tl, dH=dH, dW=dW)


def grpo_loss_fwd_bwd(H, W, targets, cu_seqlens, old_logp, ref_logp, adv, chunk_tokens, *,
                      temperature=1.0, logit_scale_multiply=0.0, logit_scale_divide=0.0, logit_softcapping=0.0,
                      keep_chunk_logits=False, dh_fp32=False, clip_eps_low=0.2, clip_eps_high=0.2, beta=0.001,
                      agg="seq_mean",
                      mask=None, want_logp=True, want_token_loss=True, loss=None, logp=None, token_loss=None,
                      dH=None, dW=None, workspace=None, stream=None, timer: Timer | None = None):
    """GRPO loss, per-token logp and objective, and dL/dH (and dL/dW with dW: an fp32 [V, D]
    tensor, or True to allocate one).  cu_seqlens is a host int32 array/tensor.  A caller's
    workspace must hold grpo_workspace_bytes(..., num_seqs=S, with_dW=bool(dW)) bytes.
    Outputs (loss fp64 [1], logp and token_loss fp32 [T], dH) may be passed in."""
    return _loss_call(False, H, W, targets, cu_seqlens, old_logp, ref_logp, adv, chunk_tokens,
                      temperature=temperature, logit_scale_multiply=logit_scale_multiply,
                      logit_scale_divide=logit_scale_divide, logit_softcapping=logit_softcapping,
                      keep_chunk_logits=keep_chunk_logits, dh_fp32=dh_fp32, clip_eps_low=clip_eps_low,
                      clip_eps_high=clip_eps_high,
                      beta=beta, agg=agg, mask=mask, want_logp=want_logp, want_token_loss=want_token_loss,
                      loss=loss, logp=logp, token_loss=token_loss, dH=dH, dW=dW, workspace=workspace,
                      stream=stream, timer=timer)


def grpo_loss_fwd_bwd_static(H, W, targets, cu_seqlens, old_logp, ref_logp, adv, chunk_tokens, *,
                             temperature=1.0, logit_scale_multiply=0.0, logit_scale_divide=0.0,
                             logit_softcapping=0.0, keep_chunk_logits=False, dh_fp32=False, clip_eps_low=0.2,
                             clip_eps_high=0.2,
                             beta=0.001, agg="seq_mean", mask=None, want_logp=True, want_token_loss=True,
                             loss=None, logp=None, token_loss=None, dH=None, dW=None, stream=None,
                             timer: Timer | None = None):
    """grpo_loss_fwd_bwd through the library's allocation-free entry point: its static
    per-device scratch (GRPO_STATIC_SCRATCH_BYTES) replaces the workspace, so with every
    output passed in nothing is allocated.  Calls that overlap on one device race."""
    return _loss_call(True, H, W, targets, cu_seqlens, old_logp, ref_logp, adv, chunk_tokens,
                      temperature=temperature, logit_scale_multiply=logit_scale_multiply,
                      logit_scale_divide=logit_scale_divide, logit_softcapping=logit_softcapping,
                      keep_chunk_logits=keep_chunk_logits, dh_fp32=dh_fp32, clip_eps_low=clip_eps_low,
                      clip_eps_high=clip_eps_high,
                      beta=beta, agg=agg, mask=mask, want_logp=want_logp, want_token_loss=want_token_loss,
                      loss=loss, logp=logp, token_loss=token_loss, dH=dH, dW=dW, workspace=None,
                      stream=stream, timer=timer)


GRPO_STATIC_SCRATCH_BYTES = 256 << 20


def grpo_debug_token_index(cu_seqlens, T: int, chunk_tokens: int, device="cuda", stream=None):
    cu = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu().contiguous()
    S = cu.numel() - 1
    with _on(stream):
        out = [torch.empty(T, dtype=torch.int32, device=device) for _ in range(3)]
        ws = torch.empty(max(256, (S + 1) * 4 + 255) // 256 * 256, dtype=torch.uint8, device=device)
        st = lib().grpo_debug_token_index(ctypes.c_void_p(cu.data_ptr()), S, int(T), int(chunk_tokens),
                                          *[_ptr(o) for o in out], _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "grpo_debug_token_index")
    return tuple(out)
