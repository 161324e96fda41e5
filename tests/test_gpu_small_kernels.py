"""GPU parity of the advantages and token-index kernels, and of the kernel timer."""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import Timer, grpo_advantages, grpo_debug_token_index, grpo_logp_fwd
from synth import make_case

from gpu_cases import dev_matrix, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,G,mode", [(64, 8, "unbiased"), (4, 4, "population"), (2, 2, "unbiased"),
                                      (300, 3, "unbiased"), (7, 1, "unbiased")])
def test_advantages(S, G, mode):
    rng = np.random.default_rng(S * 10 + G)
    r = rng.random(S).astype(np.float32)
    if S >= 4 and G > 1:
        r[:G] = 0.25  # a degenerate group
    say(f"advantages S={S} G={G} {mode}")
    got = grpo_advantages(torch.from_numpy(r).cuda(), G, mode, 1e-4).cpu().numpy()
    ref = oracle.group_advantages(r, G, std=mode, eps=1e-4)
    assert np.abs(got - ref).max() <= 1e-6
    if S >= 4 and G > 1:
        assert np.all(got[:G] == 0)


def test_advantages_worked_example():
    got = grpo_advantages(torch.tensor([1.0, 0.0, 0.0, 0.0], device="cuda"), 4).cpu().numpy()
    np.testing.assert_allclose(got, [1.4997000599880024] + [-0.4999000199960008] * 3, rtol=0, atol=1e-6)


@pytest.mark.parametrize("lengths,chunk", [([5, 0, 7, 1, 0, 13], 4), ([55000, 55000], 8192),
                                           ([1] * 300, 7), ([1000], 1000), ([0, 3] * 400, 16)])
def test_token_index_bit_exact(lengths, chunk):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    say(f"token index S={len(lengths)} T={T} chunk={chunk}")
    seq, cid, pos = [x.cpu().numpy() for x in grpo_debug_token_index(cu, T, chunk)]
    s = oracle.sequence_of_token(cu)
    assert np.array_equal(seq, s)
    assert np.array_equal(cid, np.arange(T) // chunk)
    assert np.array_equal(pos, np.arange(T) - cu[s])


def test_timer_counts_launches():
    c = make_case(3, D=64, V=600, G=1, lengths=[700])
    H, W = dev_matrix(c.H, "bf16"), dev_matrix(c.W, "bf16")
    y = torch.from_numpy(c.targets).cuda()
    tm = Timer(64)
    grpo_logp_fwd(H, W, y, 256, timer=tm)
    torch.cuda.synchronize()
    ms, n, dropped = tm.read("logits_lse")
    assert n == 3 and ms > 0 and dropped == 0
    # bf16: the logits GEMM captures the target logits itself; fp32 takes a row dot product
    assert tm.read("merge")[1] == 3 and tm.read("target_logit")[1] == 0
    tm.reset()
    grpo_logp_fwd(dev_matrix(c.H, "bf16").float(), dev_matrix(c.W, "bf16").float(), y, 256, timer=tm)
    torch.cuda.synchronize()
    assert tm.read("logits_lse")[1] == 3 and tm.read("target_logit")[1] == 1
    tm.close()
