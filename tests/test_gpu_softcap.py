"""GPU parity of the logit scale and softcapping (every entry point) against the fp64
oracle: z = c tanh(s x / c) / tau with s = multiply / divide."""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import (Timer, grpo_ce_loss_fwd_bwd, grpo_logp_bwd, grpo_logp_fwd,
                                grpo_loss_fwd_bwd)

from gpu_cases import (DH_REL_L2, LOGP_ATOL, LOSS_RTOL, case, check_loss_outputs, check_rows, host_matrix, say,
                       to_device)

pytestmark = pytest.mark.gpu


def _logit_kw(mul, div, cap):
    return dict(logit_scale_multiply=mul, logit_scale_divide=div, logit_softcapping=cap)


def _scale(mul, div):
    return (mul if mul > 0 else 1.0) / (div if div > 0 else 1.0)


@pytest.mark.parametrize("dtype,D,V,lengths,chunk,tau,mul,div,cap", [
    ("bf16", 256, 10000, [300, 400, 324], 512, 0.7, 1.5, 1.2, 5.0),   # W^T copy, edge vocab tile
    ("bf16", 264, 1000, [700, 1], 128, 1.0, 0.0, 2.0, 2.0),            # in-register W^T, split
    ("bf16", 256, 1000, [300, 212], 512, 0.7, 3.0, 0.0, 0.0),          # scale only
    ("f32", 68, 333, [90, 40, 70], 50, 0.7, 1.5, 0.0, 4.0),
])
def test_loss_with_logit_scale_and_softcap(dtype, D, V, lengths, chunk, tau, mul, div, cap):
    say(f"loss softcap {dtype} D={D} V={V} T={sum(lengths)} chunk={chunk} tau={tau} mul={mul} div={div} cap={cap}")
    # W scaled up so that s x / c reaches the tanh's curved part
    k = case(61 + D, D=D, V=V, lengths=lengths, G=3 if len(lengths) == 3 else 2, dtype=dtype, chunk=chunk,
             tau=tau, w_std=0.2, old_std=0.3, ref_std=0.3, beta=0.05, scale=_scale(mul, div), softcap=cap,
             bad_targets=(3,))
    d = to_device(k)
    got = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], chunk,
                            temperature=tau, mask=d["mask"], **_logit_kw(mul, div, cap), **k["prm"])
    torch.cuda.synchronize()
    r = check_loss_outputs(k, got, dh_bar=1e-4 if dtype == "f32" else DH_REL_L2)
    say(f"  logp err {r['logp_err']:.2e} dH worst row {r['dH_row_worst']:.2e} whole {r['dH_rel']:.2e} "
        f"loss {r['loss']:.6e} vs {r['loss_ref']:.6e}")


@pytest.mark.parametrize("dtype,cap", [("bf16", 3.0), ("f32", 3.0), ("bf16", 0.0)])
def test_logp_fwd_bwd_ce_with_softcap(dtype, cap):
    say(f"logp fwd/bwd and ce with softcap {cap} ({dtype})")
    D, V, lengths, chunk, tau, mul, div = (256, 10000, [300, 400, 324], 512, 0.7, 1.5, 1.2)
    if dtype == "f32":
        D, V, lengths, chunk = 68, 333, [90, 40, 70], 50
    k = case(71, D=D, V=V, lengths=lengths, G=3, dtype=dtype, chunk=chunk, tau=tau, w_std=0.2,
             scale=_scale(mul, div), softcap=cap, bad_targets=(4,))
    d = to_device(k)
    kw = _logit_kw(mul, div, cap)
    y = k["targets"]
    T = k["T"]
    ref_lp, ref_lse = oracle.selective_log_softmax(k["H64"], k["W64"], y, tau, scale=_scale(mul, div), softcap=cap)
    lp, lse = grpo_logp_fwd(d["H"], d["W"], d["targets"], chunk, tau, return_lse=True, **kw)
    lp = lp.cpu().numpy().astype(np.float64)
    ok = np.isfinite(ref_lp)
    assert np.array_equal(np.isfinite(lp), ok)
    assert np.abs(lp[ok] - ref_lp[ok]).max() <= LOGP_ATOL
    grad = np.random.default_rng(72).standard_normal(T).astype(np.float32) * 0.01
    tm = Timer(1024)
    dH = grpo_logp_bwd(d["H"], d["W"], d["targets"], lse, torch.from_numpy(grad).cuda(), chunk, tau, timer=tm, **kw)
    torch.cuda.synchronize()
    assert tm.read("target_logit")[1] == 1  # the exact target entries need the target logits
    tm.close()
    ref = oracle.logp_backward(k["H64"], k["W64"], y, grad.astype(np.float64), tau, scale=_scale(mul, div),
                               softcap=cap)
    worst, e = check_rows(oracle.widen(host_matrix(dH, dtype), dtype), ref, 1e-4 if dtype == "f32" else DH_REL_L2)
    say(f"  logp_bwd dH worst row {worst:.2e}, whole {e:.2e}")
    mask = np.ones(T, np.uint8)
    mask[4] = 0
    out = oracle.cross_entropy_loss_and_grad(k["H64"], k["W64"], y, mask, tau, scale=_scale(mul, div), softcap=cap)
    got = grpo_ce_loss_fwd_bwd(d["H"], d["W"], d["targets"], chunk, temperature=tau,
                               mask=torch.from_numpy(mask).cuda(), **kw)
    torch.cuda.synchronize()
    L = float(got["loss"].cpu()[0])
    assert abs(L - out["loss"]) <= LOSS_RTOL * abs(out["loss"])
    worst, e = check_rows(oracle.widen(host_matrix(got["dH"], dtype), dtype), out["dH"],
                          1e-4 if dtype == "f32" else DH_REL_L2)
    say(f"  ce loss {L:.8f} vs {out['loss']:.8f}, dH worst row {worst:.2e}, whole {e:.2e}")
