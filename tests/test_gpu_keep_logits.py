"""GPU parity of the variant that keeps the chunk's logits (keep_chunk_logits = 1: no
recompute GEMM) against the fp64 oracle, and its bitwise agreement with the recompute
path on every forward output."""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import Timer, grpo_ce_loss_fwd_bwd, grpo_loss_fwd_bwd

from gpu_cases import DH_REL_L2, backward_passes, case, check_loss_outputs, check_rows, host_matrix, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,V,lengths,chunk,tau,cap", [
    (256, 10000, [300, 400, 324], 512, 0.7, 0.0),     # W^T copy, edge vocabulary tile, split dH
    (264, 999, [700, 1], 128, 1.0, 0.0),              # in-register W^T, ragged tail
    (1024, 32000, [1500, 548], 4096, 1.0, 0.0),       # one chunk, several tiles each way
    (256, 1000, [300, 212], 512, 0.7, 3.0),           # softcap
    (256, 10000, [1200, 848], 2048, 1.0, 0.0),        # copies of W and W^T (room in one 2048-token chunk)
    (256, 10000, [1200, 848], 2048, 0.7, 3.0),        # the same with a softcap
])
def test_grpo_loss_keeping_chunk_logits(D, V, lengths, chunk, tau, cap):
    say(f"keep logits D={D} V={V} T={sum(lengths)} chunk={chunk} tau={tau} cap={cap}")
    k = case(81 + D, D=D, V=V, lengths=lengths, G=len(lengths) if len(lengths) < 3 else 3, chunk=chunk, tau=tau,
             w_std=0.2 if cap else 0.02, old_std=0.3, ref_std=0.3, beta=0.05, softcap=cap, mask_frac=0.1,
             bad_targets=(3,))
    d = to_device(k)
    kw = dict(temperature=tau, mask=d["mask"], logit_softcapping=cap, **k["prm"])
    tm = Timer(4096)
    kept = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], chunk,
                             keep_chunk_logits=True, timer=tm, **kw)
    torch.cuda.synchronize()
    nchunks = -(-k["T"] // chunk)
    assert tm.read("probs")[1] == 0 and tm.read("probs_kept")[1] == nchunks
    npass, info = backward_passes(k["T"], D, V, chunk, num_seqs=len(lengths), keep=True)
    say(f"  plan {info}")
    assert npass == nchunks and tm.read("w_copy")[1] == int(info["w_copy"])
    tm.close()
    r = check_loss_outputs(k, kept)
    say(f"  logp err {r['logp_err']:.2e} dH rel {r['dH_rel']:.2e} loss {r['loss']:.6e} vs {r['loss_ref']:.6e}")
    base = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], chunk, **kw)
    for key in ("loss", "logp", "token_loss"):
        assert torch.equal(torch.nan_to_num(kept[key], nan=7.0), torch.nan_to_num(base[key], nan=7.0)), key
    worst, rel = check_rows(kept["dH"].float().cpu().numpy(), base["dH"].float().cpu().numpy(), DH_REL_L2)
    say(f"  dH kept vs recomputed: worst row {worst:.2e}, whole {rel:.2e}")
    assert rel <= 5e-3


def test_ce_keeping_chunk_logits():
    k = case(91, D=256, V=10000, lengths=[300, 400, 324], G=3, chunk=512, bad_targets=(5,))
    d = to_device(k)
    mask = np.ones(k["T"], np.uint8)
    mask[5] = 0
    dm = torch.from_numpy(mask).cuda()
    out = oracle.cross_entropy_loss_and_grad(k["H64"], k["W64"], k["targets"], mask, 1.0)
    kept = grpo_ce_loss_fwd_bwd(d["H"], d["W"], d["targets"], 512, mask=dm, keep_chunk_logits=True)
    base = grpo_ce_loss_fwd_bwd(d["H"], d["W"], d["targets"], 512, mask=dm)
    torch.cuda.synchronize()
    assert torch.equal(kept["loss"], base["loss"])
    assert abs(float(kept["loss"].cpu()[0]) - out["loss"]) <= 1e-4 * abs(out["loss"])
    worst, e = check_rows(oracle.widen(host_matrix(kept["dH"], "bf16"), "bf16"), out["dH"], DH_REL_L2)
    say(f"keep logits ce: dH worst row {worst:.2e}, whole {e:.2e}")
