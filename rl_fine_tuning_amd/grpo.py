"""Thin Python binding of the C ABI in include/grpo.h (ctypes).

Argument marshalling only: tensors are torch device tensors, passed by pointer with
the current HIP stream; every step of the computation runs in the HIP library.  The
binding fails loudly when the library has not been built.
"""
from __future__ import annotations

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
                ("keep_chunk_logits", ctypes.c_int32)]


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


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GRPO_BF16
    if t.dtype == torch.float32:
        return GRPO_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_shape(T, D, V, chunk_tokens, dtype, temperature=1.0, logit_scale_multiply=0.0, logit_scale_divide=0.0,
               logit_softcapping=0.0, keep_chunk_logits=False) -> GrpoShape:
    """0 for a logit argument means 'not used' (see grpo_shape in include/grpo.h)."""
    return GrpoShape(int(T), int(D), int(V), int(chunk_tokens), int(dtype), float(temperature),
                     float(logit_scale_multiply), float(logit_scale_divide), float(logit_softcapping),
                     int(bool(keep_chunk_logits)))


def _bwd_mode(with_backward, with_dW):
    return 2 if with_dW else int(bool(with_backward))


def grpo_workspace_bytes(T, D, V, chunk_tokens, dtype=GRPO_BF16, temperature=1.0, num_seqs=1,
                         with_backward=True, logit_softcapping=0.0, keep_chunk_logits=False,
                         with_dW=False) -> int:
    shape = make_shape(T, D, V, chunk_tokens, dtype, temperature, logit_softcapping=logit_softcapping,
                       keep_chunk_logits=keep_chunk_logits)
    return int(lib().grpo_workspace_bytes(ctypes.byref(shape), int(num_seqs), _bwd_mode(with_backward, with_dW)))


def grpo_plan_info(T, D, V, chunk_tokens, dtype=GRPO_BF16, temperature=1.0, num_seqs=1, with_backward=True,
                   logit_softcapping=0.0, keep_chunk_logits=False, with_dW=False) -> dict:
    """The library's workspace layout for a call: which fragment-major copies of W it keeps,
    the tokens per backward slice and the workspace bytes."""
    shape = make_shape(T, D, V, chunk_tokens, dtype, temperature, logit_softcapping=logit_softcapping,
                       keep_chunk_logits=keep_chunk_logits)
    info = (ctypes.c_int64 * 4)()
    st = lib().grpo_plan_info(ctypes.byref(shape), int(num_seqs), _bwd_mode(with_backward, with_dW), info)
    _check(st, "grpo_plan_info")
    return dict(w_transposed_copy=bool(info[0]), w_copy=bool(info[1]), backward_slice_tokens=int(info[2]),
                workspace_bytes=int(info[3]))


def _workspace(nbytes, workspace, device):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() < nbytes:
        raise ValueError("workspace too small")
    return workspace, workspace.numel()


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
                  logit_softcapping=0.0, return_lse: bool = False, out=None, workspace=None,
                  stream=None, timer: Timer | None = None):
    """logp[t] = log softmax(H[t] W^T / temperature)[targets[t]] (fp32), chunked."""
    for t, n in ((H, "H"), (W, "W"), (targets, "targets")):
        _dev(t, n)
    T, D = H.shape
    V = W.shape[0]
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping)
    nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 0))
    ws, wsn = _workspace(nbytes, workspace, H.device)
    logp = out if out is not None else torch.empty(T, dtype=torch.float32, device=H.device)
    lse = torch.empty(T, dtype=torch.float32, device=H.device) if return_lse else None
    st = lib().grpo_logp_fwd(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(logp), _ptr(lse),
                             _ptr(ws), wsn, _stream(stream), timer.handle if timer else None)
    _check(st, "grpo_logp_fwd")
    return (logp, lse) if return_lse else logp


def grpo_logp_bwd(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor,
                  grad_logp: torch.Tensor, chunk_tokens: int, temperature: float = 1.0, *,
                  logit_scale_multiply=0.0, logit_scale_divide=0.0, logit_softcapping=0.0, dH=None,
                  dW=None, workspace=None, stream=None, timer: Timer | None = None):
    """dH of sum_t grad_logp[t] * logp_t, recomputing each chunk's logits from the forward's lse.
    With dW (an fp32 [V, D] tensor, or True to allocate one) returns (dH, dW).  A caller's
    workspace must hold grpo_workspace_bytes(..., with_dW=bool(dW)) bytes."""
    for t, n in ((H, "H"), (W, "W"), (targets, "targets"), (lse, "lse"), (grad_logp, "grad_logp")):
        _dev(t, n)
    T, D = H.shape
    V = W.shape[0]
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping)
    nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 2 if dW is not None and dW is not False else 1))
    ws, wsn = _workspace(nbytes, workspace, H.device)
    if dH is None:
        dH = torch.empty_like(H)
    want_dW = dW is not None and dW is not False
    if dW is True:
        dW = torch.empty(V, D, dtype=torch.float32, device=H.device)
    st = lib().grpo_logp_bwd(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(lse), _ptr(grad_logp),
                             _ptr(dH), _ptr(dW) if want_dW else None, _ptr(ws), wsn, _stream(stream),
                             timer.handle if timer else None)
    _check(st, "grpo_logp_bwd")
    return (dH, dW) if want_dW else dH


def grpo_ce_loss_fwd_bwd(H, W, targets, chunk_tokens, *, temperature=1.0, logit_scale_multiply=0.0,
                         logit_scale_divide=0.0, logit_softcapping=0.0, keep_chunk_logits=False, mask=None,
                         want_logp=True, want_token_loss=False, dH=None, dW=None, workspace=None, stream=None,
                         timer: Timer | None = None):
    """Mean cross-entropy over the unmasked tokens, per-token logp, dL/dH and (with dW: an
    fp32 [V, D] tensor, or True to allocate one) dL/dW.  A caller's workspace must hold
    grpo_workspace_bytes(..., with_dW=bool(dW)) bytes."""
    for t, n in ((H, "H"), (W, "W"), (targets, "targets")):
        _dev(t, n)
    if mask is not None:
        _dev(mask, "mask")
    T, D = H.shape
    V = W.shape[0]
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping, keep_chunk_logits)
    nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), 1, 2 if dW is not None and dW is not False else 1))
    ws, wsn = _workspace(nbytes, workspace, H.device)
    dev = H.device
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    logp = torch.empty(T, dtype=torch.float32, device=dev) if want_logp else None
    tl = torch.empty(T, dtype=torch.float32, device=dev) if want_token_loss else None
    if dH is None:
        dH = torch.empty_like(H)
    if dW is True:
        dW = torch.empty(V, D, dtype=torch.float32, device=dev)
    st = lib().grpo_ce_loss_fwd_bwd(ctypes.byref(shape), _ptr(H), _ptr(W), _ptr(targets), _ptr(mask), _ptr(loss),
                                    _ptr(logp), _ptr(tl), _ptr(dH), _ptr(dW) if dW is not None and dW is not False else None, _ptr(ws),
                                    wsn, _stream(stream), timer.handle if timer else None)
    _check(st, "grpo_ce_loss_fwd_bwd")
    return dict(loss=loss, logp=logp, token_loss=tl, dH=dH, dW=dW)


def grpo_advantages(rewards: torch.Tensor, group_size: int, std_mode: str = "unbiased", eps: float = 1e-4,
                    *, out=None, stream=None) -> torch.Tensor:
    _dev(rewards, "rewards")
    adv = out if out is not None else torch.empty_like(rewards)
    st = lib().grpo_advantages(_ptr(rewards), rewards.numel(), int(group_size), GRPO_STD[std_mode], float(eps),
                               _ptr(adv), _stream(stream))
    _check(st, "grpo_advantages")
    return adv


def grpo_loss_fwd_bwd(H, W, targets, cu_seqlens, old_logp, ref_logp, adv, chunk_tokens, *,
                      temperature=1.0, logit_scale_multiply=0.0, logit_scale_divide=0.0, logit_softcapping=0.0,
                      keep_chunk_logits=False, clip_eps_low=0.2, clip_eps_high=0.2, beta=0.001, agg="seq_mean",
                      mask=None, want_logp=True, want_token_loss=True, dH=None, dW=None, workspace=None,
                      stream=None, timer: Timer | None = None):
    """GRPO loss, per-token logp and objective, and dL/dH (and dL/dW with dW: an fp32 [V, D]
    tensor, or True to allocate one).  cu_seqlens is a host int32 array/tensor.  A caller's
    workspace must hold grpo_workspace_bytes(..., num_seqs=S, with_dW=bool(dW)) bytes."""
    for t, n in ((H, "H"), (W, "W"), (targets, "targets"), (old_logp, "old_logp"), (adv, "adv")):
        _dev(t, n)
    if ref_logp is not None:
        _dev(ref_logp, "ref_logp")
    if mask is not None:
        _dev(mask, "mask")
    cu = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu().contiguous()
    S = cu.numel() - 1
    T, D = H.shape
    V = W.shape[0]
    shape = make_shape(T, D, V, chunk_tokens, _dtype_code(H), temperature, logit_scale_multiply,
                       logit_scale_divide, logit_softcapping, keep_chunk_logits)
    params = GrpoLossParams(float(clip_eps_low), float(clip_eps_high), float(beta), GRPO_AGG[agg])
    nbytes = int(lib().grpo_workspace_bytes(ctypes.byref(shape), S, 2 if dW is not None and dW is not False else 1))
    ws, wsn = _workspace(nbytes, workspace, H.device)
    dev = H.device
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    logp = torch.empty(T, dtype=torch.float32, device=dev) if want_logp else None
    tl = torch.empty(T, dtype=torch.float32, device=dev) if want_token_loss else None
    if dH is None:
        dH = torch.empty_like(H)
    if dW is True:
        dW = torch.empty(V, D, dtype=torch.float32, device=dev)
    st = lib().grpo_loss_fwd_bwd(ctypes.byref(shape), ctypes.byref(params), _ptr(H), _ptr(W), _ptr(targets),
                                 ctypes.c_void_p(cu.data_ptr()), S, _ptr(mask), _ptr(old_logp), _ptr(ref_logp),
                                 _ptr(adv), _ptr(loss), _ptr(logp), _ptr(tl), _ptr(dH),
                                 _ptr(dW) if dW is not None and dW is not False else None, _ptr(ws), wsn, _stream(stream),
                                 timer.handle if timer else None)
    _check(st, "grpo_loss_fwd_bwd")
    return dict(loss=loss, logp=logp, token_loss=tl, dH=dH, dW=dW)


def grpo_debug_token_index(cu_seqlens, T: int, chunk_tokens: int, device="cuda", stream=None):
    cu = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu().contiguous()
    S = cu.numel() - 1
    out = [torch.empty(T, dtype=torch.int32, device=device) for _ in range(3)]
    ws = torch.empty(max(256, (S + 1) * 4 + 255) // 256 * 256, dtype=torch.uint8, device=device)
    st = lib().grpo_debug_token_index(ctypes.c_void_p(cu.data_ptr()), S, int(T), int(chunk_tokens),
                                      *[_ptr(o) for o in out], _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "grpo_debug_token_index")
    return tuple(out)
