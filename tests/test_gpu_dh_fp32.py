"""fp32 dH for bf16 inputs (grpo_shape.dh_fp32): every row against the oracle at the fp32 bar,
relative L2 <= 1e-4 per row, through the unsplit and the split-vocabulary dH GEMM, the split
backward, the cross-entropy and kept logits."""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import grpo_ce_loss_fwd_bwd, grpo_logp_bwd, grpo_logp_fwd, grpo_loss_fwd_bwd

from gpu_cases import backward_passes, case, check_loss_outputs, check_rows, say, to_device

pytestmark = pytest.mark.gpu

BAR = 1e-4


@pytest.mark.parametrize("D,V,lengths,chunk,keep", [
    (256, 10000, [300, 400, 324], 512, False),     # vocabulary split 8 ways (few token tiles)
    (4096, 1000, [2048, 2048], 4096, False),       # unsplit dH GEMM (256 tiles)
    (264, 999, [700, 1], 128, False),              # in-register W^T, ragged tail
    (512, 3000, [700, 324], 1024, True),           # kept logits
])
def test_loss_fp32_dH(D, V, lengths, chunk, keep):
    say(f"fp32 dH loss D={D} V={V} T={sum(lengths)} chunk={chunk} keep={keep}")
    k = case(401 + D, D=D, V=V, lengths=lengths, G=len(lengths), chunk=chunk, old_std=0.3, ref_std=0.05,
             beta=0.001, mask_frac=0.1, bad_targets=(5,))
    d = to_device(k)
    got = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], chunk,
                            temperature=k["tau"], mask=d["mask"], keep_chunk_logits=keep, dh_fp32=True, **k["prm"])
    torch.cuda.synchronize()
    assert got["dH"].dtype == torch.float32
    r = check_loss_outputs(k, got, dh_bar=BAR)
    say(f"  dH worst row {r['dH_row_worst']:.2e}, whole {r['dH_rel']:.2e}")
    # the bf16 output of the same call is the fp32 one rounded to nearest even
    b = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], chunk,
                          temperature=k["tau"], mask=d["mask"], keep_chunk_logits=keep, **k["prm"])
    check_rows(b["dH"].float().cpu().numpy(), got["dH"].cpu().numpy(), 4e-3)


def test_logp_bwd_and_ce_fp32_dH():
    k = case(431, D=256, V=10000, lengths=[300, 400, 324], G=3, chunk=512, bad_targets=(6,))
    d = to_device(k)
    T = k["T"]
    say("fp32 dH logp_bwd and cross-entropy")
    grad = np.random.default_rng(432).standard_normal(T).astype(np.float32) * 0.01
    grad[::9] = 0.0
    _, lse = grpo_logp_fwd(d["H"], d["W"], d["targets"], 512, return_lse=True)
    dH = grpo_logp_bwd(d["H"], d["W"], d["targets"], lse, torch.from_numpy(grad).cuda(), 512, dh_fp32=True)
    assert dH.dtype == torch.float32
    ref = oracle.logp_backward(k["H64"], k["W64"], k["targets"], grad.astype(np.float64))
    worst, e = check_rows(dH.cpu().numpy().astype(np.float64), ref, BAR)
    say(f"  logp_bwd worst row {worst:.2e}, whole {e:.2e}")
    mask = np.ones(T, np.uint8)
    mask[6] = 0
    out = oracle.cross_entropy_loss_and_grad(k["H64"], k["W64"], k["targets"], mask)
    got = grpo_ce_loss_fwd_bwd(d["H"], d["W"], d["targets"], 512, mask=torch.from_numpy(mask).cuda(), dh_fp32=True)
    worst, e = check_rows(got["dH"].cpu().numpy().astype(np.float64), out["dH"], BAR)
    say(f"  ce worst row {worst:.2e}, whole {e:.2e}")
