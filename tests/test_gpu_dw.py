"""GPU parity of the lm_head gradient dW (full fine-tuning) against the fp64 oracle, for the
GRPO loss (recompute and kept-logits paths, softcap), the split backward and the
cross-entropy."""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import Timer, grpo_ce_loss_fwd_bwd, grpo_logp_bwd, grpo_logp_fwd, grpo_loss_fwd_bwd

from gpu_cases import DH_REL_L2, backward_passes, case, check_loss_outputs, check_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,V,lengths,chunk,tau,cap,keep", [
    (264, 10000, [300, 400, 324], 512, 0.7, 0.0, False),   # hidden edge tile, vocabulary edge tile, 2 chunks
    (256, 1000, [300, 212], 128, 1.0, 3.0, False),        # softcap, 4 chunks, ragged tail
    (512, 3000, [700, 324], 1024, 1.0, 0.0, True),        # kept logits
    (256, 10000, [300, 400, 324], 512, 1.0, 0.0, False),  # W^T copy (without dW this shape's backward runs in slices)
    (256, 10000, [1200, 848], 2048, 1.0, 0.0, False),     # copies of W and W^T, one 2048-token chunk
])
def test_grpo_loss_dW(D, V, lengths, chunk, tau, cap, keep):
    say(f"dW grpo D={D} V={V} T={sum(lengths)} chunk={chunk} tau={tau} cap={cap} keep={keep}")
    k = case(111 + D, D=D, V=V, lengths=lengths, G=len(lengths), chunk=chunk, tau=tau, w_std=0.2 if cap else 0.02,
             old_std=0.3, ref_std=0.3, beta=0.05, softcap=cap, mask_frac=0.1, bad_targets=(3,))
    ref = oracle.grpo_loss_and_grad(k["H64"], k["W64"], k["targets"], k["c"].cu, k["mask"],
                                    k["old"].astype(np.float64), k["ref"].astype(np.float64),
                                    k["adv"].astype(np.float64), tau, softcap=cap, with_dW=True, **k["prm"])
    d = to_device(k)
    tm = Timer(4096)
    got = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], chunk,
                            temperature=tau, mask=d["mask"], logit_softcapping=cap, keep_chunk_logits=keep,
                            dW=True, timer=tm, **k["prm"])
    torch.cuda.synchronize()
    npass, info = backward_passes(k["T"], D, V, chunk, num_seqs=len(lengths), keep=keep, dW=True)
    say(f"  plan {info}, backward passes {npass}")
    assert npass == -(-k["T"] // chunk)  # with dW the backward takes whole chunks
    assert tm.read("ht_copy")[1] == npass
    # the dW GEMM runs band by band of at most 32 vocabulary tiles, each band after its Q^T
    ndw = tm.read("dw_gemm")[1]
    assert ndw == tm.read("qt_band")[1] and ndw % npass == 0 and ndw // npass >= -(-V // (32 * 256))
    assert tm.read("frag_copy")[1] == npass
    assert tm.read("w_copy")[1] == int(info["w_copy"])
    tm.close()
    check_loss_outputs(k, got)  # dH and the forward outputs are unchanged by asking for dW
    worst, e = check_rows(got["dW"].cpu().numpy(), ref["dW"], DH_REL_L2, "dW")
    say(f"  dW worst row {worst:.2e}, whole {e:.2e}")


def test_logp_bwd_and_ce_dW():
    k = case(121, D=264, V=10000, lengths=[300, 400, 324], G=3, chunk=512, bad_targets=(6,))
    d = to_device(k)
    T = k["T"]
    grad = np.random.default_rng(122).standard_normal(T).astype(np.float32) * 0.01
    grad[::7] = 0.0
    _, lse = grpo_logp_fwd(d["H"], d["W"], d["targets"], 512, return_lse=True)
    dH, dW = grpo_logp_bwd(d["H"], d["W"], d["targets"], lse, torch.from_numpy(grad).cuda(), 512, dW=True)
    rdH, rdW = oracle.logp_backward(k["H64"], k["W64"], k["targets"], grad.astype(np.float64), with_dW=True)
    worst, e = check_rows(dW.cpu().numpy(), rdW, DH_REL_L2, "dW")
    say(f"dW logp_bwd worst row {worst:.2e}, whole {e:.2e}")
    mask = np.ones(T, np.uint8)
    mask[6] = 0
    out = oracle.cross_entropy_loss_and_grad(k["H64"], k["W64"], k["targets"], mask, with_dW=True)
    got = grpo_ce_loss_fwd_bwd(d["H"], d["W"], d["targets"], 512, mask=torch.from_numpy(mask).cuda(), dW=True)
    worst, e = check_rows(got["dW"].cpu().numpy(), out["dW"], DH_REL_L2, "dW")
    say(f"dW ce worst row {worst:.2e}, whole {e:.2e}")


def test_dW_without_tokens_is_zero():
    D, V = 64, 300
    H = torch.zeros(0, D, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(V, D, device="cuda").bfloat16()
    y = torch.zeros(0, dtype=torch.int32, device="cuda")
    e = torch.zeros(0, dtype=torch.float32, device="cuda")
    dW = torch.full((V, D), 7.0, dtype=torch.float32, device="cuda")
    grpo_logp_bwd(H, W, y, e, e, 16, dW=dW)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW).item() == 0
