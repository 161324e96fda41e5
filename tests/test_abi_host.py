"""Host-side checks of the C ABI: the library loads, exports every function that
include/grpo.h declares, and rejects bad arguments before any HIP call (so these
run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from rl_fine_tuning_amd import grpo as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grpo.h")

FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every case fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(grpo_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 11
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.grpo_version().startswith(b"grpo-mi355x")


def test_status_strings():
    lib = B.lib()
    for s in range(8):
        assert lib.grpo_status_string(s)
    assert lib.grpo_status_string(99) == b"unknown status"


def shape(T=100, D=64, V=512, C=32, dtype=0, tau=1.0):
    return B.make_shape(T, D, V, C, dtype, tau)


def test_workspace_bound_one_chunk_of_logits():
    # extra memory <= one chunk's fp32 logits + O(T + C (V / 256 + D)) per-token state
    for (T, D, V, C, S) in [(110000, 4096, 151936, 8192, 2), (40960, 1536, 151936, 4096, 64),
                            (20480, 4096, 128256, 2048, 4), (380000, 2880, 201088, 8192, 4),
                            (128, 64, 512, 32, 4)]:
        for dt in (0, 1):
            n = B.grpo_workspace_bytes(T, D, V, C, dt, num_seqs=S)
            bound = C * V * 4 + 64 * T + 64 * 2 ** 20 + 8 * C * (V // 256 + 1) + 32 * C * D
            assert 0 < n <= bound, (T, D, V, C, dt, n, bound)
    assert B.grpo_workspace_bytes(0, 64, 512, 32) > 0
    assert B.grpo_workspace_bytes(10, 63, 512, 32) == 0  # D not a multiple of 8 for bf16


def test_plan_layouts():
    # The layout grpo_workspace_bytes sizes: the largest of (both fragment-major copies of W,
    # whole-chunk backward), (both copies, backward in two token slices; not with kept
    # logits), (W^T only), (neither) that stays within one chunk's fp32 logits.
    info = B.grpo_plan_info(110000, 4096, 151936, 8192, num_seqs=2)       # Qwen3-8B-shaped, 110K
    assert info["w_transposed_copy"] and info["w_copy"] and info["backward_slice_tokens"] == 4096
    assert info["workspace_bytes"] == B.grpo_workspace_bytes(110000, 4096, 151936, 8192, num_seqs=2)
    assert info["workspace_bytes"] <= 8192 * 151936 * 4
    # with dW the backward takes whole chunks (a slice would read and write the fp32 dW again)
    info = B.grpo_plan_info(110000, 4096, 151936, 8192, num_seqs=2, with_dW=True)
    assert info["w_transposed_copy"] and not info["w_copy"] and info["backward_slice_tokens"] == 8192
    assert info["workspace_bytes"] <= 8192 * 151936 * 4
    # with kept logits the chunk's matrix is filled whole in the forward: no slices, W^T only
    info = B.grpo_plan_info(110000, 4096, 151936, 8192, num_seqs=2, keep_chunk_logits=True)
    assert info["w_transposed_copy"] and not info["w_copy"] and info["backward_slice_tokens"] == 8192
    info = B.grpo_plan_info(40960, 1536, 151936, 4096, num_seqs=64)       # both copies, whole chunks
    assert info["w_transposed_copy"] and info["w_copy"] and info["backward_slice_tokens"] == 4096
    info = B.grpo_plan_info(20480, 4096, 128256, 2048, num_seqs=4)        # no room for either copy:
    assert not info["w_transposed_copy"] and not info["w_copy"] and info["backward_slice_tokens"] == 2048
    assert info["w_transposed_bands"] == 3 and info["workspace_bytes"] <= 2048 * 128256 * 4  # W^T in 3 bands
    for kw in (dict(with_dW=True), dict(dh_fp32=True)):                    # no bands with dW or fp32 dH,
        assert B.grpo_plan_info(20480, 4096, 128256, 2048, num_seqs=4, **kw)["w_transposed_bands"] == 0
    assert B.grpo_plan_info(20480, 4096, 128256, 1024, num_seqs=4)["w_transposed_bands"] == 0  # nor below 2048
    assert B.grpo_plan_info(2600, 2048, 40000, 2048, num_seqs=2)["w_transposed_bands"] == 2
    info = B.grpo_plan_info(380000, 2880, 201088, 8192, num_seqs=4)
    assert info["w_transposed_copy"] and info["w_copy"] and info["backward_slice_tokens"] == 8192
    # the forward alone keeps the copy of W when it fits; fp32 inputs keep no copies
    info = B.grpo_plan_info(110000, 4096, 151936, 8192, with_backward=False)
    assert info["w_copy"] and not info["w_transposed_copy"] and info["backward_slice_tokens"] == 0
    info = B.grpo_plan_info(4096, 256, 10000, 1024, dtype=1, num_seqs=2)
    assert not info["w_copy"] and not info["w_transposed_copy"] and info["backward_slice_tokens"] == 1024
    for T, D, V, C in [(110000, 4096, 151936, 8192), (1024, 264, 10000, 512), (701, 264, 999, 128)]:
        for keep in (False, True):
            for dW in (False, True):
                i = B.grpo_plan_info(T, D, V, C, num_seqs=2, keep_chunk_logits=keep, with_dW=dW)
                assert i["backward_slice_tokens"] % 256 == 0 and i["backward_slice_tokens"] > 0
                if keep or dW:
                    assert i["backward_slice_tokens"] >= min(T, C)
    with pytest.raises(B.GrpoError):
        B.grpo_plan_info(10, 63, 512, 32)


def test_logp_fwd_validation():
    lib = B.lib()
    s = shape()
    ws = ctypes.c_void_p(1 << 20)
    f = lambda sh, H=FAKE, W=FAKE, y=FAKE, lp=FAKE, wsp=ws, n=1 << 40: lib.grpo_logp_fwd(
        ctypes.byref(sh), H, W, y, lp, None, wsp, n, None, None)
    assert lib.grpo_logp_fwd(None, FAKE, FAKE, FAKE, FAKE, None, ws, 1 << 40, None, None) == 1
    assert f(s, H=None) == 1
    assert f(s, lp=None) == 1
    assert f(shape(tau=0.0)) == 3
    assert f(shape(tau=float("nan"))) == 3
    assert f(shape(tau=-1.0)) == 3
    assert f(shape(D=60)) == 5  # bf16 rows must be 16-byte multiples
    assert f(shape(dtype=7)) == 5
    assert f(shape(C=0)) == 2
    assert f(shape(V=0)) == 2
    assert f(shape(T=-1)) == 2
    assert f(s, H=ctypes.c_void_p((1 << 20) + 2)) == 5  # misaligned
    assert f(s, n=16) == 4
    assert f(s, wsp=None) == 4
    assert f(s, wsp=ctypes.c_void_p((1 << 20) + 16)) == 4  # workspace must be 256-byte aligned
    # T = 0: nothing to do, nothing touched
    assert f(shape(T=0), H=None, y=None, lp=None) == 0


def test_loss_validation():
    lib = B.lib()
    T = 100
    cu = np.array([0, 30, 60, 100], dtype=np.int32)
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    good = B.GrpoLossParams(0.2, 0.2, 0.001, 0)

    def call(sh=None, prm=good, cu_p=cup, S=3, ref=FAKE, ws_bytes=1 << 40, H=FAKE, dH=FAKE, old=FAKE,
             adv=FAKE, loss=FAKE, dW=None):
        sh = sh or shape(T=T)
        return lib.grpo_loss_fwd_bwd(ctypes.byref(sh), ctypes.byref(prm), H, FAKE, FAKE, cu_p, S, None, old,
                                     ref, adv, loss, None, None, dH, dW, FAKE, ws_bytes, None, None)

    assert call(ws_bytes=16) == 4
    assert call(H=None) == 1
    assert call(dH=None) == 1
    assert call(old=None) == 1
    assert call(adv=None) == 1
    assert call(loss=None) == 1
    assert call(ref=None) == 1                                    # beta != 0 needs ref_logp
    assert call(ref=None, prm=B.GrpoLossParams(0.2, 0.2, 0.0, 0), ws_bytes=16) == 4  # beta == 0: ref optional
    assert call(prm=B.GrpoLossParams(1.0, 0.2, 0.001, 0)) == 3    # eps_low must be < 1
    assert call(prm=B.GrpoLossParams(-0.1, 0.2, 0.001, 0)) == 3
    assert call(prm=B.GrpoLossParams(0.2, float("inf"), 0.001, 0)) == 3
    assert call(prm=B.GrpoLossParams(0.2, 0.2, -1.0, 0)) == 3
    assert call(prm=B.GrpoLossParams(0.2, 0.2, 0.001, 5)) == 3
    assert call(cu_p=None) == 1
    assert call(S=0) == 2
    bad = np.array([1, 30, 60, 100], dtype=np.int32)
    assert call(cu_p=bad.ctypes.data_as(ctypes.c_void_p)) == 2     # cu[0] != 0
    bad = np.array([0, 60, 30, 100], dtype=np.int32)
    assert call(cu_p=bad.ctypes.data_as(ctypes.c_void_p)) == 2     # not monotone
    bad = np.array([0, 30, 60, 99], dtype=np.int32)
    assert call(cu_p=bad.ctypes.data_as(ctypes.c_void_p)) == 2     # cu[S] != T
    assert call(sh=shape(T=T, tau=0.0)) == 3
    assert call(dH=ctypes.c_void_p((1 << 20) + 4)) == 5
    assert call(sh=shape(T=T, dtype=1), dW=FAKE) == 5  # dW: bf16 only


def test_advantages_validation():
    lib = B.lib()
    f = lambda S=8, G=4, mode=0, eps=1e-4, r=FAKE, a=FAKE: lib.grpo_advantages(r, S, G, mode, eps, a, None)
    assert f(r=None) == 1
    assert f(a=None) == 1
    assert f(S=7) == 2
    assert f(S=0) == 2
    assert f(G=0) == 2
    assert f(mode=3) == 3
    assert f(eps=-1.0) == 3
    assert f(eps=float("nan")) == 3


def test_debug_index_and_timer_validation():
    lib = B.lib()
    cu = np.array([0, 3, 3, 10], dtype=np.int32)
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    assert lib.grpo_debug_token_index(cup, 3, 11, 4, FAKE, FAKE, FAKE, FAKE, 256, None) == 2
    assert lib.grpo_debug_token_index(cup, 3, 10, 0, FAKE, FAKE, FAKE, FAKE, 256, None) == 2
    assert lib.grpo_debug_token_index(cup, 3, 10, 4, FAKE, FAKE, FAKE, None, 256, None) == 4
    assert lib.grpo_debug_token_index(cup, 3, 10, 4, None, FAKE, FAKE, FAKE, 256, None) == 1
    h = ctypes.c_void_p()
    assert lib.grpo_timer_create(0, ctypes.byref(h)) == 3
    assert lib.grpo_timer_create(4, None) == 1
    assert lib.grpo_timer_read(None, 0, None, None, None) == 1


def test_logp_bwd_validation():
    lib = B.lib()
    ws = ctypes.c_void_p(1 << 20)

    def f(sh=None, H=FAKE, W=FAKE, y=FAKE, lse=FAKE, g=FAKE, dH=FAKE, wsp=ws, n=1 << 40, dW=None):
        sh = sh or shape()
        return lib.grpo_logp_bwd(ctypes.byref(sh), H, W, y, lse, g, dH, dW, wsp, n, None, None)

    assert lib.grpo_logp_bwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, 1 << 40, None, None) == 1
    for k in ("H", "W", "y", "lse", "g", "dH"):
        assert f(**{k: None}) == 1, k
    assert f(shape(tau=0.0)) == 3
    assert f(shape(D=60)) == 5
    assert f(dH=ctypes.c_void_p((1 << 20) + 4)) == 5
    assert f(n=16) == 4
    assert f(wsp=ctypes.c_void_p((1 << 20) + 16)) == 4
    assert f(shape(T=0), H=None, y=None, lse=None, g=None, dH=None) == 0  # nothing to do
    assert f(shape(dtype=1, D=64), dW=FAKE) == 5  # dW: bf16 only
    assert f(dW=ctypes.c_void_p((1 << 20) + 8)) == 5  # dW: 16-byte aligned (its epilogue moves float4s)


def test_ce_loss_validation():
    lib = B.lib()

    def f(sh=None, H=FAKE, W=FAKE, y=FAKE, loss=FAKE, dH=FAKE, n=1 << 40, wsp=FAKE):
        sh = sh or shape()
        return lib.grpo_ce_loss_fwd_bwd(ctypes.byref(sh), H, W, y, None, loss, None, None, dH, None, wsp, n,
                                         None, None)

    for k in ("H", "W", "y", "loss", "dH"):
        assert f(**{k: None}) == 1, k
    assert f(shape(tau=float("inf"))) == 3
    assert f(shape(dtype=3)) == 5
    assert f(n=16) == 4
    assert f(wsp=None) == 4


def test_logit_arguments_validation():
    lib = B.lib()
    ws = ctypes.c_void_p(1 << 20)

    def f(**kw):
        sh = B.make_shape(100, 64, 512, 32, 0, kw.pop("tau", 1.0), **kw)
        return lib.grpo_logp_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, ws, 1 << 40, None, None)

    assert f(logit_scale_multiply=-1.0) == 3
    assert f(logit_scale_divide=float("nan")) == 3
    assert f(logit_softcapping=float("inf")) == 3
    assert f(logit_softcapping=-30.0) == 3
    assert f(logit_scale_multiply=1e30, logit_scale_divide=1e-30) == 3  # scale overflows
    assert f(logit_scale_multiply=1e-30, logit_scale_divide=1e30) == 3  # scale underflows to 0
    sh = B.make_shape(100, 64, 512, 32, 0, 0.7, 2.0, 0.0, 30.0)  # valid: only the small workspace fails
    assert lib.grpo_logp_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, ws, 16, None, None) == 4
    # zeros mean "not used": a zero tail is a valid plain shape (validation passes; the
    # oversized workspace claim is what fails, with status 4)
    sh = B.make_shape(100, 64, 512, 32, 0, 1.0)
    assert lib.grpo_logp_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, ws, 16, None, None) == 4


def test_keep_chunk_logits_validation():
    lib = B.lib()
    ws = ctypes.c_void_p(1 << 20)
    sh = B.make_shape(100, 64, 512, 32, 0, 1.0)
    sh.keep_chunk_logits = 2
    assert lib.grpo_logp_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, ws, 1 << 40, None, None) == 3
    sh = B.make_shape(100, 64, 512, 32, 1, 1.0, keep_chunk_logits=True)  # fp32 inputs: not supported
    assert lib.grpo_logp_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, ws, 1 << 40, None, None) == 5
    # keeping the logits needs no memory beyond the same bound: one chunk's fp32 logits
    for (T, D, V, C) in [(110000, 4096, 151936, 8192), (40960, 1536, 151936, 4096), (380000, 2880, 201088, 8192)]:
        assert 0 < B.grpo_workspace_bytes(T, D, V, C, 0, num_seqs=2, keep_chunk_logits=True) <= C * V * 4


class _FakeLib:
    """Stands in for the library in binding tests: counts compute calls, sizes nothing."""

    def __init__(self):
        self.calls = []

    def grpo_workspace_bytes(self, *a):
        return 1024

    def __getattr__(self, name):
        def call(*a):
            self.calls.append(name)
            return 0
        return call


def test_binding_rejects_bad_arguments_before_the_library(monkeypatch):
    # Every wrapper checks device, contiguity, dtype and shape of each tensor before a
    # pointer reaches the library.  CPU tensors stand in for device tensors here.
    import types
    import torch
    fake = _FakeLib()
    monkeypatch.setattr(B, "lib", lambda: fake)
    monkeypatch.setattr(B, "_is_device", lambda t: True)
    monkeypatch.setattr(B, "_on", lambda s: __import__("contextlib").nullcontext())
    stream = types.SimpleNamespace(cuda_stream=0)
    T, D, V, S = 12, 16, 40, 3
    bf = torch.bfloat16
    good = dict(H=torch.zeros(T, D, dtype=bf), W=torch.zeros(V, D, dtype=bf),
                targets=torch.zeros(T, dtype=torch.int32), cu=np.array([0, 4, 8, 12], np.int32),
                old=torch.zeros(T), ref=torch.zeros(T), adv=torch.zeros(S))

    def loss(**over):
        a = dict(good, **over)
        return B.grpo_loss_fwd_bwd(a["H"], a["W"], a["targets"], a["cu"], a["old"], a["ref"], a["adv"], 4,
                                   stream=stream, **{k: v for k, v in over.items() if k in ("mask", "dH", "dW", "workspace")})

    loss()
    assert fake.calls == ["grpo_loss_fwd_bwd"]
    bad = [
        (dict(targets=torch.zeros(T, dtype=torch.int64)), TypeError),      # torch's default integer type
        (dict(targets=torch.zeros(T + 1, dtype=torch.int32)), ValueError),
        (dict(W=torch.zeros(V, D)), TypeError),                            # W's dtype differs from H's
        (dict(W=torch.zeros(V, D + 8, dtype=bf)), ValueError),
        (dict(H=torch.zeros(T, D, dtype=torch.float16)), TypeError),
        (dict(H=torch.zeros(D, T, dtype=bf).t()), ValueError),             # not contiguous
        (dict(old=torch.zeros(T, dtype=torch.float64)), TypeError),
        (dict(ref=torch.zeros(T - 1)), ValueError),
        (dict(adv=torch.zeros(S + 1)), ValueError),
        (dict(mask=torch.zeros(T, dtype=torch.int32)), TypeError),
        (dict(dH=torch.zeros(T, D)), TypeError),                           # dH takes H's dtype
        (dict(dW=torch.zeros(V, D, dtype=bf)), TypeError),                 # dW is fp32
        (dict(dW=torch.zeros(V + 1, D)), ValueError),
        (dict(workspace=torch.zeros(2048)), TypeError),                    # a uint8 buffer
        (dict(workspace=torch.zeros(16, dtype=torch.uint8)), ValueError),  # too small
        (dict(H=np.zeros((T, D))), TypeError),
    ]
    for over, exc in bad:
        with pytest.raises(exc):
            loss(**over)
    assert fake.calls == ["grpo_loss_fwd_bwd"], "a bad argument reached the library"
    with pytest.raises(TypeError):
        B.grpo_logp_fwd(good["H"], good["W"], torch.zeros(T, dtype=torch.int64), 4, stream=stream)
    with pytest.raises(TypeError):
        B.grpo_logp_bwd(good["H"], good["W"], good["targets"], torch.zeros(T, dtype=torch.float64), good["old"], 4,
                        stream=stream)
    with pytest.raises(ValueError):
        B.grpo_ce_loss_fwd_bwd(good["H"], good["W"], good["targets"], 4, mask=torch.zeros(T + 2, dtype=torch.uint8),
                               stream=stream)
    with pytest.raises(TypeError):
        B.grpo_advantages(torch.zeros(S, dtype=torch.float64), 3, stream=stream)
    with pytest.raises(ValueError):
        B.grpo_loss_fwd_bwd_static(good["H"], good["W"], good["targets"], good["cu"], good["old"], good["ref"],
                                   torch.zeros(S - 1), 4, stream=stream)
    assert fake.calls == ["grpo_loss_fwd_bwd"]


def test_static_entry_rejects_calls_beyond_its_scratch():
    # grpo_loss_fwd_bwd_static refuses, before any HIP call, a call whose workspace would pass
    # the static scratch (256 MiB), and accepts the same shape with a chunk small enough.
    lib = B.lib()
    T = 110000
    cu = np.array([0, 55000, 110000], dtype=np.int32)
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    prm = B.GrpoLossParams(0.2, 0.2, 0.001, 0)
    big = B.make_shape(T, 4096, 151936, 8192, 0)
    assert B.grpo_workspace_bytes(T, 4096, 151936, 8192, num_seqs=2) > B.GRPO_STATIC_SCRATCH_BYTES
    st = lib.grpo_loss_fwd_bwd_static(ctypes.byref(big), ctypes.byref(prm), FAKE, FAKE, FAKE, cup, 2, None, FAKE,
                                      FAKE, FAKE, FAKE, None, None, FAKE, None, None, None)
    assert st == 7 and b"static scratch" in lib.grpo_status_string(st)
    assert B.grpo_workspace_bytes(T, 4096, 151936, 256, num_seqs=2) <= B.GRPO_STATIC_SCRATCH_BYTES
    # host-checkable errors come first, as for grpo_loss_fwd_bwd
    st = lib.grpo_loss_fwd_bwd_static(ctypes.byref(big), ctypes.byref(prm), None, FAKE, FAKE, cup, 2, None, FAKE,
                                      FAKE, FAKE, FAKE, None, None, FAKE, None, None, None)
    assert st == 1


def test_dh_fp32_validation_and_plan():
    lib = B.lib()
    sh = B.make_shape(100, 64, 512, 32, 0)
    sh.dh_fp32 = 2
    assert lib.grpo_workspace_bytes(ctypes.byref(sh), 1, 1) == 0  # 0 or 1 only
    # fp32 dH keeps the probabilities as bf16 hi + lo pairs: the buffer doubles (both halves
    # padded to an even number of 16-entry k steps)
    a = B.grpo_workspace_bytes(1000, 64, 512, 256)
    b = B.grpo_workspace_bytes(1000, 64, 512, 256, dh_fp32=True)
    assert b - a == 256 * 2 * 32 * 16 * 2 - 256 * 32 * 16 * 2
    assert B.grpo_workspace_bytes(1000, 64, 512, 256, dtype=1, dh_fp32=True) == \
        B.grpo_workspace_bytes(1000, 64, 512, 256, dtype=1)  # fp32 inputs: dH is fp32 anyway
    # at the Qwen3-8B shape the doubled buffer fits the one-chunk bound by slicing the backward
    i = B.grpo_plan_info(110000, 4096, 151936, 8192, num_seqs=2, dh_fp32=True)
    assert i["backward_slice_tokens"] == 4096 and i["workspace_bytes"] <= 8192 * 151936 * 4
    assert B.grpo_plan_info(110000, 4096, 151936, 8192, num_seqs=2) == \
        B.grpo_plan_info(110000, 4096, 151936, 8192, num_seqs=2, dh_fp32=False)


E_NULL, E_VALUE, E_WORKSPACE, E_UNSUPPORTED = 1, 3, 4, 5  # grpo_status in include/grpo.h


def test_offload_workspace_and_validation():
    # grpo_logp_bwd_offload's workspace: the backward's plus two staging buffers of one chunk's
    # rows of H; the flag goes only with a backward mode
    for (T, D, V, C, dt) in [(110000, 4096, 151936, 8192, 0), (20480, 4096, 128256, 2048, 0), (700, 68, 333, 50, 1)]:
        base = B.grpo_workspace_bytes(T, D, V, C, dt)
        host = B.grpo_workspace_bytes(T, D, V, C, dt, host_h=True)
        stage = -(-C * D * (2 if dt == 0 else 4) // 256) * 256
        assert base < host <= base + 2 * stage + 256, (T, D, V, C, base, host)
        assert host <= C * V * 4 + 64 * T + 64 * 2 ** 20 + 8 * C * (V // 256 + 1) + 32 * C * D
        assert B.grpo_workspace_bytes(T, D, V, C, dt, with_dW=dt == 0, host_h=True) > 0
    lib = B.lib()
    s = shape()
    for mode in (3, 4, 7, 8, -1):
        assert lib.grpo_workspace_bytes(ctypes.byref(s), 1, mode) == 0, mode
        info = (ctypes.c_int64 * 4)()
        assert lib.grpo_plan_info(ctypes.byref(s), 1, mode, info) == E_VALUE, mode
    # host-checkable errors come before any HIP call (no GPU needed): a missing context,
    # misalignment, a short workspace
    off = ctypes.c_void_p(0)
    fake, ws = FAKE, ctypes.c_void_p(1 << 21)
    # grpo_logp_fwd_offload(shape, H, W, targets, logp, lse, H_host, ws, ws_bytes, stream, timer, offload)
    assert lib.grpo_logp_fwd_offload(ctypes.byref(s), fake, fake, fake, fake, fake, fake, ws, 1 << 30, None, None,
                                     off) == E_NULL
    # grpo_logp_bwd_offload(shape, H_host, W, targets, lse, grad, dH, dW, ws, ws_bytes, stream, timer, offload)
    assert lib.grpo_logp_bwd_offload(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, ws, 1 << 30, None,
                                     None, off) == E_NULL
    ctx = ctypes.c_void_p(1 << 22)  # never dereferenced: the checks below fail first
    assert lib.grpo_logp_bwd_offload(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 8), fake, fake, fake, fake, fake,
                                     None, ws, 1 << 30, None, None, ctx) == E_UNSUPPORTED
    assert lib.grpo_logp_bwd_offload(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, ws, 16, None, None,
                                     ctx) == E_WORKSPACE
    with pytest.raises(ValueError):
        B.grpo_logp_bwd_offload(torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(3, 8, dtype=torch.bfloat16),
                                     torch.zeros(4, dtype=torch.int32), torch.zeros(4), torch.zeros(4), 4, None)
