"""Full-size workloads (the four bf16 model shapes) in the chunking the benchmark
times, checked against the oracle on sampled tokens.

Every per-token output (logp, l_t, dH row) depends on its own row only, so the
oracle computes the sampled rows exactly: the first and last 8 tokens of every
chunk, 4 tokens on each side of every sequence boundary, and 128 uniform tokens.
Sampled tokens get old/ref log-probabilities = oracle logp + the workload's noise;
the others get -log V + noise, which only moves the loss.  The loss is checked against
the oracle's loss from the GPU's own log-probabilities at every token, and through its
fixed relation to the per-token terms (L = sum_t w_t l_t).
"""
import numpy as np
import pytest
import torch

import oracle
from rl_fine_tuning_amd import grpo_loss_fwd_bwd, grpo_workspace_bytes
from synth import make_config

from gpu_cases import (DH_REL_L2, LOGP_ATOL, LOSS_RTOL, check_rows, dev_matrix, f32, host_matrix, near_clip_boundary,
                       dh_rows_at, rel_l2, say)

pytestmark = pytest.mark.gpu


def sample_rows(c, rng):
    T, C = c.T, c.chunk
    rows = set()
    for t0 in range(0, T, C):
        t1 = min(T, t0 + C)
        rows.update(range(t0, min(t1, t0 + 8)))
        rows.update(range(max(t0, t1 - 8), t1))
    for b in c.cu[1:-1]:
        rows.update(range(max(0, b - 4), min(T, b + 4)))
    rows.update(rng.integers(0, T, 128).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("cfg,keep,dh32", [(1, False, False), (2, False, False), (3, False, False),
                                           (4, False, False), (3, True, False), (3, False, True)])
def test_full_size_sampled(cfg, keep, dh32):
    c = make_config(cfg)
    T, D, V, C = c.T, c.D, c.V, c.chunk
    say(f"full size config {cfg}: T={T} D={D} V={V} chunk={C} keep_chunk_logits={keep} dh_fp32={dh32}")
    rng = np.random.default_rng(cfg)
    rows = sample_rows(c, rng)
    W64 = oracle.widen(c.W, "bf16")
    H_rows = oracle.widen(c.H[rows], "bf16")
    lp_rows, lse_rows = oracle.selective_log_softmax(H_rows, W64, c.targets[rows])
    base = np.full(T, -np.log(V))
    base[rows] = lp_rows
    old = f32(base + c.noise_old)
    ref = f32(base + c.noise_ref)
    adv = f32(oracle.group_advantages(c.rewards, c.G))

    H = dev_matrix(c.H, "bf16")
    W = dev_matrix(c.W, "bf16")
    ws_bytes = grpo_workspace_bytes(T, D, V, C, 0, num_seqs=c.S, keep_chunk_logits=keep, dh_fp32=dh32)
    assert ws_bytes <= C * V * 4  # extra memory stays below one chunk's fp32 logits
    before = torch.cuda.memory_allocated()
    got = grpo_loss_fwd_bwd(H, W, torch.from_numpy(c.targets).cuda(), c.cu, torch.from_numpy(old).cuda(),
                            torch.from_numpy(ref).cuda(), torch.from_numpy(adv).cuda(), C, keep_chunk_logits=keep,
                            dh_fp32=dh32)
    torch.cuda.synchronize()
    say(f"  gpu done; extra allocated {(torch.cuda.memory_allocated() - before) / 2**30:.2f} GiB")

    logp = got["logp"].cpu().numpy().astype(np.float64)
    tl = got["token_loss"].cpu().numpy().astype(np.float64)
    err = np.abs(logp[rows] - lp_rows).max()
    assert err <= LOGP_ATOL, err

    s = oracle.sequence_of_token(c.cu)
    w = oracle.token_weights(c.cu, c.mask)
    terms = oracle.grpo_token_terms(lp_rows, old[rows].astype(np.float64), ref[rows].astype(np.float64),
                                    adv.astype(np.float64)[s[rows]], 0.2, 0.2, 0.001)
    assert np.all(np.abs(tl[rows] - terms["ell"]) <= LOGP_ATOL * (1 + np.abs(adv[s[rows]])))
    g_rows = w[rows] * terms["dell"]
    dH_ref = oracle.grad_rows(H_rows, W64, c.targets[rows], lse_rows, g_rows)
    dH_sel = got["dH"][torch.from_numpy(rows).cuda()]
    dH = dH_sel.cpu().numpy().astype(np.float64) if dh32 else oracle.widen(host_matrix(dH_sel, "bf16"), "bf16")
    bar = 1e-4 if dh32 else DH_REL_L2  # fp32 dH: the probabilities enter the GEMM as bf16 hi + lo pairs
    amb = near_clip_boundary(lp_rows, old[rows].astype(np.float64), 0.2, 0.2)
    e = rel_l2(dH[~amb], dH_ref[~amb])
    assert e <= DH_REL_L2, e
    # every sampled row at its own scale, against the oracle's dH at the GPU's log-probabilities
    # (a token whose g_t nearly cancels would otherwise measure the fp32-vs-fp64 logp difference)
    terms_at = oracle.grpo_token_terms(logp[rows], old[rows].astype(np.float64), ref[rows].astype(np.float64),
                                       adv.astype(np.float64)[s[rows]], 0.2, 0.2, 0.001)
    dH_at = dh_rows_at(H_rows, W64, c.targets[rows], lse_rows, logp[rows], w[rows] * terms_at["dell"])
    worst, _ = check_rows(dH[~amb], dH_at[~amb], bar)

    L = float(got["loss"].cpu().numpy()[0])
    L_terms = float(np.sum(w * tl))
    scale = float(np.sum(np.abs(w * tl)))
    assert abs(L - L_terms) <= 1e-6 * scale, (L, L_terms)
    # the loss over every token: the oracle's loss from the GPU's own log-probabilities (the
    # GEMM side of logp is checked on the sampled rows above; this pins the per-token
    # objective, the weights and the fp64 reduction at all T tokens)
    L_or, ell_or, _ = oracle.grpo_loss_from_logp(logp, old.astype(np.float64), ref.astype(np.float64),
                                                 adv.astype(np.float64), c.cu, c.mask)
    scale_or = max(abs(L_or), float(np.sum(np.abs(w * ell_or))))
    assert abs(L - L_or) <= LOSS_RTOL * scale_or, (L, L_or, scale_or)
    assert np.all(np.abs(tl - ell_or) <= LOGP_ATOL * (1 + np.abs(adv[oracle.sequence_of_token(c.cu)])))
    say(f"  logp err {err:.2e}, dH worst row {worst:.2e}, whole {e:.2e}, loss {L:.6e}, "
        f"workspace {ws_bytes / 2**30:.2f} GiB")


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_dW_sampled_rows(cfg):
    # dW at full size in the benchmark's chunking (every chunk's bands accumulated in order),
    # checked on selected vocabulary rows: the first and last row of every 32-tile band, rows of
    # the last (partial) tile and the tail of V.  Each row of dW is
    #   dW[v] = sum_t g_t (onehot(y_t)_v - p_t,v) H_t,   p_t,v = exp(z_t,v - lse_t),
    # computed in fp64 over all T tokens from the GPU's own lse and logp (as the per-row dH
    # reference does), so it measures the dW path itself.
    from rl_fine_tuning_amd import grpo_logp_fwd
    c = make_config(cfg)
    T, D, V, C = c.T, c.D, c.V, c.chunk
    say(f"full size dW config {cfg}: T={T} D={D} V={V} chunk={C}")
    H = dev_matrix(c.H, "bf16")
    W = dev_matrix(c.W, "bf16")
    y = torch.from_numpy(c.targets).cuda()
    logp0, lse = grpo_logp_fwd(H, W, y, C, return_lse=True)
    old = (logp0.double() + torch.from_numpy(c.noise_old).cuda()).float()
    ref = (logp0.double() + torch.from_numpy(c.noise_ref).cuda()).float()
    adv = torch.from_numpy(f32(oracle.group_advantages(c.rewards, c.G))).cuda()
    got = grpo_loss_fwd_bwd(H, W, y, c.cu, old, ref, adv, C, dW=True)
    torch.cuda.synchronize()
    logp = got["logp"].cpu().numpy().astype(np.float64)
    assert torch.equal(got["logp"], logp0)  # the loss call's logp is the forward's, bit for bit
    band = 32 * 256
    vs = set()
    for b0 in range(0, V, band):
        vs.update([b0, min(V, b0 + band) - 1])
    last_tile = (V - 1) // 256 * 256
    vs.update([last_tile, last_tile + 1, V - 2, V - 1, V // 2])
    vs = np.array(sorted(vs))
    s = oracle.sequence_of_token(c.cu)
    w = oracle.token_weights(c.cu, c.mask)
    terms = oracle.grpo_token_terms(logp, old.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64),
                                    adv.cpu().numpy().astype(np.float64)[s], 0.2, 0.2, 0.001)
    g = w * terms["dell"]
    lse64 = lse.cpu().numpy().astype(np.float64)
    Wv = oracle.widen(c.W[vs], "bf16")
    ref_rows = np.zeros((len(vs), D))
    for t0 in range(0, T, 8192):  # fp64 over row blocks of H
        Hb = oracle.widen(c.H[t0:t0 + 8192], "bf16")
        coef = -np.exp(Hb @ Wv.T - lse64[t0:t0 + 8192, None])  # -p_t,v
        yb = c.targets[t0:t0 + 8192]
        hit = yb[:, None] == vs[None, :]
        coef[hit] += 1.0
        ref_rows += (g[t0:t0 + 8192, None] * coef).T @ Hb
    dW_rows = got["dW"][torch.from_numpy(vs).cuda()].cpu().numpy().astype(np.float64)
    worst, whole = check_rows(dW_rows, ref_rows, DH_REL_L2, "dW")
    say(f"  dW rows {len(vs)}: worst row {worst:.2e}, whole {whole:.2e}")
