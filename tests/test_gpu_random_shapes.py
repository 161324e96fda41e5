"""GPU parity on seeded random small shapes, against the fp64 oracle: hidden and vocabulary
sizes that are not multiples of the 256-row tiles, chunk sizes from one token to past T
(so that the workspace layouts differ: with or without the fragment-major copies of W and
W^T, the backward whole or in token slices), variable sequence lengths and group sizes,
masks, an out-of-range target, temperature, logit scale and softcap, kept logits and dW."""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import grpo_loss_fwd_bwd, grpo_plan_info

from gpu_cases import DH_REL_L2, case, check_loss_outputs, check_rows, say, to_device

pytestmark = pytest.mark.gpu

N_CASES = 128


def params(i):
    rng = np.random.default_rng(9000 + i)
    dtype = "f32" if i % 6 == 5 else "bf16"
    D = 8 * int(rng.integers(1, 65)) if dtype == "bf16" else 4 * int(rng.integers(1, 50))
    V = int(rng.integers(17, 8000))
    G = int(rng.integers(1, 4))
    S = G * int(rng.integers(1, 3))
    lengths = [int(x) for x in rng.integers(1, 1500 // S + 1, size=S)]
    T = sum(lengths)
    chunk = int(rng.choice([int(rng.integers(1, T + 64)), 256, 512, 700, 1024, 2048]))
    tau = float(rng.choice([1.0, 0.7]))
    cap = float(rng.uniform(2.0, 30.0)) if i % 4 == 2 else 0.0
    scale = float(rng.uniform(0.5, 2.0)) if i % 5 == 3 else 1.0
    keep = dtype == "bf16" and i % 3 == 0
    dW = dtype == "bf16" and i % 4 == 1
    return dict(dtype=dtype, D=D, V=V, G=G, lengths=lengths, chunk=chunk, tau=tau, cap=cap, scale=scale,
                keep=keep, dW=dW)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    p = params(i)
    T = sum(p["lengths"])
    info = grpo_plan_info(T, p["D"], p["V"], p["chunk"], dtype=0 if p["dtype"] == "bf16" else 1,
                          num_seqs=len(p["lengths"]), keep_chunk_logits=p["keep"], with_dW=p["dW"])
    say(f"random case {i}: {p} T={T}; plan {info}")
    k = case(9100 + i, D=p["D"], V=p["V"], lengths=p["lengths"], G=p["G"], dtype=p["dtype"], chunk=p["chunk"],
             tau=p["tau"], w_std=0.2 if p["cap"] else 0.02, old_std=0.3, ref_std=0.3, beta=0.05, mask_frac=0.1,
             bad_targets=(T // 2,), scale=p["scale"], softcap=p["cap"])
    d = to_device(k)
    got = grpo_loss_fwd_bwd(d["H"], d["W"], d["targets"], k["c"].cu, d["old"], d["ref"], d["adv"], p["chunk"],
                            temperature=p["tau"], logit_scale_multiply=p["scale"], logit_softcapping=p["cap"],
                            mask=d["mask"], keep_chunk_logits=p["keep"], dW=True if p["dW"] else None, **k["prm"])
    torch.cuda.synchronize()
    r = check_loss_outputs(k, got, dh_bar=1e-4 if p["dtype"] == "f32" else DH_REL_L2)
    say(f"  logp err {r['logp_err']:.2e} dH worst row {r['dH_row_worst']:.2e}, whole {r['dH_rel']:.2e}")
    if p["dW"]:
        ref = oracle.grpo_loss_and_grad(k["H64"], k["W64"], k["targets"], k["c"].cu, k["mask"],
                                        k["old"].astype(np.float64), k["ref"].astype(np.float64),
                                        k["adv"].astype(np.float64), p["tau"], scale=p["scale"],
                                        softcap=p["cap"], with_dW=True, **k["prm"])
        worst, e = check_rows(got["dW"].cpu().numpy(), ref["dW"], DH_REL_L2, "dW")
        say(f"  dW worst row {worst:.2e}, whole {e:.2e}")
