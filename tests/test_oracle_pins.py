"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than its own formulas:
hand-derived closed forms (tests/golden), library routines (scipy, torch
autograd on the CPU), brute-force enumeration and finite differences.  A
dropped term, a wrong sign or index or a transposed operand in the oracle
fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _tiny(seed=0, T=12, D=8, V=16, scale=1.0):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, D))
    W = rng.standard_normal((V, D)) * scale
    y = rng.integers(0, V, T)
    return H, W, y


# ------------------------------------------------------------ log-softmax

@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_logp_matches_scipy_log_softmax(tau):
    H, W, y = _tiny(1, T=40, D=16, V=64)
    logp, lse = oracle.selective_log_softmax(H, W, y, tau, block=7)
    z = (H @ W.T) / tau
    ref = scipy.special.log_softmax(z, axis=1)[np.arange(40), y]
    np.testing.assert_allclose(logp, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=0, atol=1e-12)


def test_logp_direct_softmax_form():
    # log(exp(z_y) / sum_v exp(z_v)) written out with Python floats, no shift needed here
    H, W, y = _tiny(2, T=6, D=5, V=9)
    logp, _ = oracle.selective_log_softmax(H, W, y)
    for t in range(6):
        zs = [sum(H[t, d] * W[v, d] for d in range(5)) for v in range(9)]
        direct = math.log(math.exp(zs[y[t]]) / sum(math.exp(z) for z in zs))
        assert abs(logp[t] - direct) < 1e-12


def test_probabilities_sum_to_one_all_targets():
    # every token expanded to all V targets: sum_v exp(logp_{t,v}) = 1
    H, W, _ = _tiny(3, T=5, D=8, V=33)
    T, V = 5, 33
    Hx = np.repeat(H, V, axis=0)
    yx = np.tile(np.arange(V), T)
    logp, _ = oracle.selective_log_softmax(Hx, W, yx)
    sums = np.exp(logp.reshape(T, V)).sum(axis=1)
    np.testing.assert_allclose(sums, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("scale", [0.2 * 16, 1e3])
def test_peaked_logits_stay_finite_and_exact(scale):
    H, W, y = _tiny(4, T=20, D=16, V=50, scale=scale)
    logp, lse = oracle.selective_log_softmax(H, W, y)
    assert np.all(np.isfinite(logp)) and np.all(np.isfinite(lse))
    ref = scipy.special.log_softmax(H @ W.T, axis=1)[np.arange(20), y]
    np.testing.assert_allclose(logp, ref, rtol=1e-13, atol=1e-9)


def test_out_of_range_target_is_nan_only_there():
    H, W, y = _tiny(5, T=6, D=4, V=8)
    y = y.copy()
    y[2] = 8
    y[4] = -1
    logp, lse = oracle.selective_log_softmax(H, W, y)
    assert np.isnan(logp[2]) and np.isnan(logp[4])
    assert np.all(np.isfinite(np.delete(logp, [2, 4]))) and np.all(np.isfinite(lse))


def test_widen_bf16_exact():
    # bf16 bit patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3EAB = 0.333984375, 0x0001 = 2^-133
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0001, 0x7F7F], dtype=np.uint16)
    v = oracle.widen(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.333984375
    assert v[3] == 2.0 ** -133
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127


# ------------------------------------------------------------ advantages

def test_advantages_worked_examples():
    for row in _rows("advantages_worked.txt"):
        lhs, rhs = row.split("->")
        mode, eps, r = lhs.split()
        r = np.array([float(x) for x in r.split(",")])
        want = np.array([float(x) for x in rhs.split(",")])
        got = oracle.group_advantages(r, len(r), std=mode, eps=float(eps))
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, err_msg=row)


def test_advantages_equal_scipy_zscore_when_eps_zero():
    rng = np.random.default_rng(6)
    r = rng.random(24)
    for G in (2, 3, 8):
        A = oracle.group_advantages(r, G, std="unbiased", eps=0.0)
        want = np.concatenate([scipy.stats.zscore(r[i:i + G], ddof=1) for i in range(0, 24, G)])
        np.testing.assert_allclose(A, want, rtol=0, atol=1e-12)
        A0 = oracle.group_advantages(r, G, std="population", eps=0.0)
        want0 = np.concatenate([scipy.stats.zscore(r[i:i + G], ddof=0) for i in range(0, 24, G)])
        np.testing.assert_allclose(A0, want0, rtol=0, atol=1e-12)


def test_advantages_group_invariants():
    rng = np.random.default_rng(7)
    r = rng.random(64)
    eps = 1e-4
    A = oracle.group_advantages(r, 8, eps=eps).reshape(8, 8)
    grp = r.reshape(8, 8)
    np.testing.assert_allclose(A.sum(axis=1), 0.0, atol=1e-12)
    sig = grp.std(axis=1, ddof=1)
    np.testing.assert_allclose(A.std(axis=1, ddof=1), sig / (sig + eps), atol=1e-12)


def test_advantages_degenerate_and_shape_errors():
    assert np.all(oracle.group_advantages(np.array([0.5, 0.7, 0.9]), 1) == 0)
    assert np.all(oracle.group_advantages(np.array([1.0, 1.0, 0.0, 1.0]), 2)[:2] == 0)
    with pytest.raises(ValueError):
        oracle.group_advantages(np.zeros(5), 2)


# ------------------------------------------------------------ ratio, clip, k3

def test_clip_cases():
    for row in _rows("clip_cases.txt"):
        vals = list(map(float, row.split()))
        rho, A, surr, dsurr = vals[:4]
        lo, hi = vals[4:6] if len(vals) == 6 else (0.2, 0.2)
        logp = np.array([0.3])
        old = logp - math.log(rho)
        t = oracle.grpo_token_terms(logp, old, None, np.array([A]), lo, hi, beta=0.0)
        assert abs(t["surr"][0] - surr) < 1e-12, row
        # l = -surr, dl/dlogp = -dsurr
        assert abs(t["ell"][0] + surr) < 1e-12, row
        assert abs(t["dell"][0] + dsurr) < 1e-12, row


def test_k3_values_and_reverse_kl_expectation():
    for row in _rows("k3_values.txt"):
        d, k3 = map(float, row.split())
        t = oracle.grpo_token_terms(np.array([-1.0]), np.array([-1.0]), np.array([-1.0 + d]),
                                    np.array([0.0]), beta=1.0)
        assert abs(t["k3"][0] - k3) < 1e-15, row
    # E_{v ~ p}[k3(ref_v - logp_v)] = KL(p || ref): pins d = ref - logp (not logp - ref)
    rng = np.random.default_rng(8)
    lp = scipy.special.log_softmax(rng.standard_normal(40))
    lr = scipy.special.log_softmax(rng.standard_normal(40))
    t = oracle.grpo_token_terms(lp, lp, lr, np.zeros(40), beta=1.0)
    kl = scipy.special.rel_entr(np.exp(lp), np.exp(lr)).sum()
    assert abs((np.exp(lp) * t["k3"]).sum() - kl) < 1e-12
    assert np.all(t["k3"] >= 0)


def test_token_term_derivative_by_finite_differences():
    rng = np.random.default_rng(9)
    n = 200
    logp = -rng.random(n) * 5
    old = logp + rng.normal(0, 0.3, n)
    ref = logp + rng.normal(0, 0.5, n)
    A = rng.standard_normal(n)
    h = 1e-6
    f = lambda lp: oracle.grpo_token_terms(lp, old, ref, A, 0.2, 0.28, beta=0.3)["ell"]
    fd = (f(logp + h) - f(logp - h)) / (2 * h)
    rho = np.exp(logp - old)
    away = (np.abs(rho - 0.8) > 1e-3) & (np.abs(rho - 1.28) > 1e-3)
    an = oracle.grpo_token_terms(logp, old, ref, A, 0.2, 0.28, beta=0.3)["dell"]
    np.testing.assert_allclose(an[away], fd[away], rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------ index, weights

def test_sequence_index_against_scan_and_searchsorted():
    rng = np.random.default_rng(10)
    L = rng.integers(0, 6, 30)
    L[3] = 0
    cu = np.concatenate([[0], np.cumsum(L)])
    T = int(cu[-1])
    s = oracle.sequence_of_token(cu)
    scan = []
    i = 0
    for t in range(T):
        while cu[i + 1] <= t:
            i += 1
        scan.append(i)
    assert s.tolist() == scan
    assert np.array_equal(s, np.searchsorted(cu, np.arange(T), side="right") - 1)


def test_token_weights_hand_example():
    cu = np.array([0, 2, 4])
    w = oracle.token_weights(cu, np.array([1, 1, 0, 0]), "seq_mean")
    assert w.tolist() == [0.25, 0.25, 0.0, 0.0]
    w = oracle.token_weights(cu, np.array([1, 0, 1, 1]), "seq_mean")
    assert w.tolist() == [0.5, 0.0, 0.25, 0.25]
    w = oracle.token_weights(cu, np.array([1, 0, 1, 1]), "token_mean")
    np.testing.assert_allclose(w, [1 / 3, 0, 1 / 3, 1 / 3], atol=1e-16)
    # equal lengths and no mask: both aggregations agree
    cu = np.array([0, 5, 10, 15])
    np.testing.assert_allclose(oracle.token_weights(cu, np.ones(15), "seq_mean"),
                               oracle.token_weights(cu, np.ones(15), "token_mean"), atol=1e-16)


# ------------------------------------------------------------ loss and gradient

def _case(seed=11, lengths=(3, 5, 4, 6), D=8, V=16, tau=0.7, old_std=0.3, ref_std=0.5):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    H = rng.standard_normal((T, D))
    W = rng.standard_normal((V, D)) * 0.7
    y = rng.integers(0, V, T)
    logp, _ = oracle.selective_log_softmax(H, W, y, tau)
    old = logp + rng.normal(0, old_std, T)
    ref = logp + rng.normal(0, ref_std, T)
    mask = np.ones(T, dtype=np.uint8)
    mask[[1, 7]] = 0
    adv = oracle.group_advantages(rng.random(len(lengths)), 2)
    return H, W, y, cu, mask, old, ref, adv, tau


def test_on_policy_identity():
    # old = ref = logp, mask = 1, seq-mean: rho = 1, k3 = 0, so l_t = -A_s(t) and
    # L = -(1/S) sum_i A_i = 0 for zero-mean groups; g_t = -w_t A_t exactly.
    rng = np.random.default_rng(12)
    lengths = [4, 7, 3, 9, 5, 5]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    logp = -rng.random(T) * 3
    adv = oracle.group_advantages(rng.random(6), 3)
    L, ell, g = oracle.grpo_loss_from_logp(logp, logp, logp, adv, cu, np.ones(T))
    s = np.repeat(np.arange(6), lengths)
    assert abs(L) < 1e-15
    np.testing.assert_array_equal(ell, -adv[s])
    w = 1.0 / (6 * np.array(lengths, dtype=float))[s]
    np.testing.assert_array_equal(g, -w * adv[s])


def test_well_conditioned_loss_value():
    # beta = 1 and a KL-dominated case: L = sum_t w_t (beta k3_t - surr_t), evaluated here
    # token by token with Python floats from the definitions.
    H, W, y, cu, mask, old, ref, adv, tau = _case(13)
    logp, _ = oracle.selective_log_softmax(H, W, y, tau)
    L, ell, g = oracle.grpo_loss_from_logp(logp, old, ref, adv, cu, mask, beta=1.0)
    S = len(cu) - 1
    total = 0.0
    for i in range(S):
        toks = [t for t in range(cu[i], cu[i + 1]) if mask[t]]
        for t in toks:
            rho = math.exp(logp[t] - old[t])
            surr = min(rho * adv[i], min(max(rho, 0.8), 1.2) * adv[i])
            d = ref[t] - logp[t]
            total += (math.exp(d) - d - 1 - surr) / (S * len(toks))
    assert abs(L - total) < 1e-13


def test_masked_tokens_have_zero_gradient():
    H, W, y, cu, mask, old, ref, adv, tau = _case(14)
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, old, ref, adv, tau, beta=0.1)
    for t in np.nonzero(mask == 0)[0]:
        assert out["g"][t] == 0.0
        assert np.all(out["dH"][t] == 0.0)


@pytest.mark.parametrize("agg", ["seq_mean", "token_mean"])
def test_dH_matches_central_finite_differences(agg):
    H, W, y, cu, mask, old, ref, adv, tau = _case(15)
    kw = dict(clip_eps_low=0.2, clip_eps_high=0.2, beta=0.1, agg=agg)
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, old, ref, adv, tau, **kw)
    rho = np.exp(out["logp"] - old)
    assert np.all(np.abs(rho - 0.8) > 1e-3) and np.all(np.abs(rho - 1.2) > 1e-3)
    assert np.any(rho > 1.2) or np.any(rho < 0.8)  # some clipped tokens are exercised

    def loss(Hx):
        lp, _ = oracle.selective_log_softmax(Hx, W, y, tau)
        return oracle.grpo_loss_from_logp(lp, old, ref, adv, cu, mask, **kw)[0]

    h = 1e-6
    fd = np.zeros_like(H)
    for t in range(H.shape[0]):
        for d in range(H.shape[1]):
            e = np.zeros_like(H)
            e[t, d] = h
            fd[t, d] = (loss(H + e) - loss(H - e)) / (2 * h)
    err = np.linalg.norm(out["dH"] - fd) / np.linalg.norm(fd)
    assert err < 1e-6, err


def test_g_matches_finite_differences_in_logp():
    H, W, y, cu, mask, old, ref, adv, tau = _case(16)
    logp, _ = oracle.selective_log_softmax(H, W, y, tau)
    kw = dict(beta=0.2)
    L, ell, g = oracle.grpo_loss_from_logp(logp, old, ref, adv, cu, mask, **kw)
    h = 1e-6
    for t in range(len(logp)):
        e = np.zeros_like(logp)
        e[t] = h
        fd = (oracle.grpo_loss_from_logp(logp + e, old, ref, adv, cu, mask, **kw)[0]
              - oracle.grpo_loss_from_logp(logp - e, old, ref, adv, cu, mask, **kw)[0]) / (2 * h)
        assert abs(fd - g[t]) < 1e-8 * max(1.0, abs(g[t])), t


def test_dH_equals_weighted_cross_entropy_gradient_on_policy():
    # With old = logp, beta = 0 and A = +1 for every token the surrogate gradient is
    # g_t = -w_t, so dH is the gradient of sum_t w_t * CE(z_t, y_t): torch autograd on CPU.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    lengths = [5, 3, 6, 2]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, D, V, tau = 16, 6, 20, 0.7
    H = rng.standard_normal((T, D))
    W = rng.standard_normal((V, D))
    y = rng.integers(0, V, T)
    logp, _ = oracle.selective_log_softmax(H, W, y, tau)
    mask = np.ones(T)
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, logp, None, np.ones(4), tau, beta=0.0)
    w = oracle.token_weights(cu, mask)
    Ht = torch.tensor(H, requires_grad=True)
    z = Ht @ torch.tensor(W).T / tau
    ce = torch.nn.functional.cross_entropy(z, torch.tensor(y), reduction="none")
    (ce * torch.tensor(w)).sum().backward()
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=0, atol=1e-13)


def test_grad_rows_agrees_with_full_gradient():
    H, W, y, cu, mask, old, ref, adv, tau = _case(18)
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, old, ref, adv, tau, beta=0.1)
    rows = np.array([0, 3, 7, 11])
    dr = oracle.grad_rows(H[rows], W, y[rows], out["lse"][rows], out["g"][rows], tau)
    np.testing.assert_allclose(dr, out["dH"][rows], rtol=0, atol=1e-13)


# ------------------------------------------------- split backward, cross-entropy

def test_logp_backward_matches_finite_differences():
    # d/dH of sum_t c_t * logp_t for arbitrary c (zeros included), tau = 0.7
    H, W, y = _tiny(21, T=9, D=6, V=13)
    tau = 0.7
    c = np.random.default_rng(22).standard_normal(9)
    c[[2, 5]] = 0.0
    dH = oracle.logp_backward(H, W, y, c, tau)

    def f(Hx):
        lp, _ = oracle.selective_log_softmax(Hx, W, y, tau)
        return float(np.dot(c, lp))

    h = 1e-6
    fd = np.zeros_like(H)
    for t in range(H.shape[0]):
        for d in range(H.shape[1]):
            e = np.zeros_like(H)
            e[t, d] = h
            fd[t, d] = (f(H + e) - f(H - e)) / (2 * h)
    assert np.linalg.norm(dH - fd) / np.linalg.norm(fd) < 1e-6
    assert np.all(dH[[2, 5]] == 0)


def test_logp_backward_invalid_target_row_is_zero():
    H, W, y = _tiny(23, T=6, D=5, V=9)
    y = y.copy()
    y[3] = 9  # out of range
    dH = oracle.logp_backward(H, W, y, np.ones(6))
    assert np.all(dH[3] == 0) and np.all(np.isfinite(dH))


def test_cross_entropy_matches_torch_autograd():
    # mean cross-entropy over unmasked tokens: torch.nn.functional.cross_entropy with
    # ignore_index on the masked tokens, in float64 on the CPU, and its autograd gradient
    torch = pytest.importorskip("torch")
    H, W, y = _tiny(24, T=14, D=7, V=19)
    tau = 0.7
    mask = np.ones(14)
    mask[[1, 8, 9]] = 0
    out = oracle.cross_entropy_loss_and_grad(H, W, y, mask, tau)
    Ht = torch.tensor(H, requires_grad=True)
    z = Ht @ torch.tensor(W).T / tau
    yt = torch.tensor(np.where(mask > 0, y, -100))
    ce = torch.nn.functional.cross_entropy(z, yt, ignore_index=-100, reduction="mean")
    ce.backward()
    assert abs(out["loss"] - ce.item()) <= 1e-14 * abs(ce.item())
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["g"], -mask / mask.sum(), rtol=0, atol=0)


def test_cross_entropy_all_masked_and_masked_invalid_target():
    H, W, y = _tiny(25, T=5, D=4, V=7)
    out = oracle.cross_entropy_loss_and_grad(H, W, y, np.zeros(5))
    assert out["loss"] == 0.0 and np.all(out["dH"] == 0)
    y = y.copy()
    y[2] = -1
    mask = np.ones(5)
    mask[2] = 0
    out = oracle.cross_entropy_loss_and_grad(H, W, y, mask)
    assert np.isfinite(out["loss"]) and np.isnan(out["logp"][2]) and np.all(out["dH"][2] == 0)
    mask[2] = 1
    assert np.isnan(oracle.cross_entropy_loss_and_grad(H, W, y, mask)["loss"])


# ------------------------------------------------------ logit scale and softcap

def test_logit_map_derivative_and_limits():
    x = np.linspace(-40, 40, 81)
    for (tau, s, c) in [(1.0, 1.0, 0.0), (0.7, 0.5, 0.0), (0.7, 1.3, 10.0), (1.0, 1.0, 30.0)]:
        z, dz = oracle.logit_map(x, tau, s, c)
        h = 1e-6
        fd = (oracle.logit_map(x + h, tau, s, c)[0] - oracle.logit_map(x - h, tau, s, c)[0]) / (2 * h)
        np.testing.assert_allclose(dz, fd, rtol=1e-7, atol=2e-8)  # FD rounding ~ eps |z| / h
        if c > 0:
            assert np.all(np.abs(z) <= c / tau + 1e-12)  # the cap bounds |z| by c / tau
    z_big, _ = oracle.logit_map(x, 0.7, 1.3, 1e9)  # a cap far above every |s x| changes nothing
    np.testing.assert_allclose(z_big, 1.3 * x / 0.7, rtol=1e-12)
    np.testing.assert_allclose(oracle.logit_map(x, 2.0, 2.0)[0], x, rtol=0, atol=0)


def test_softcapped_loss_gradient_by_finite_differences():
    H, W, y, cu, mask, old, ref, adv, tau = _case(31)
    kw = dict(clip_eps_low=0.2, clip_eps_high=0.2, beta=0.1, scale=0.8, softcap=3.0)
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, old, ref, adv, tau, **kw)
    rho = np.exp(out["logp"] - old)
    assert np.all(np.abs(rho - 0.8) > 1e-3) and np.all(np.abs(rho - 1.2) > 1e-3)
    lkw = {k: kw[k] for k in ("clip_eps_low", "clip_eps_high", "beta")}

    def loss(Hx):
        lp, _ = oracle.selective_log_softmax(Hx, W, y, tau, scale=0.8, softcap=3.0)
        return oracle.grpo_loss_from_logp(lp, old, ref, adv, cu, mask, **lkw)[0]

    h = 1e-6
    fd = np.zeros_like(H)
    for t in range(H.shape[0]):
        for d in range(H.shape[1]):
            e = np.zeros_like(H)
            e[t, d] = h
            fd[t, d] = (loss(H + e) - loss(H - e)) / (2 * h)
    assert np.linalg.norm(out["dH"] - fd) / np.linalg.norm(fd) < 1e-6


def test_softcapped_cross_entropy_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    H, W, y = _tiny(32, T=11, D=6, V=17, scale=2.0)
    tau, s, c = 0.7, 1.5, 4.0
    out = oracle.cross_entropy_loss_and_grad(H, W, y, None, tau, scale=s, softcap=c)
    Ht = torch.tensor(H, requires_grad=True)
    z = c * torch.tanh(s * (Ht @ torch.tensor(W).T) / c) / tau
    ce = torch.nn.functional.cross_entropy(z, torch.tensor(y), reduction="mean")
    ce.backward()
    assert abs(out["loss"] - ce.item()) <= 1e-14 * abs(ce.item())
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=0, atol=1e-14)
    lp, _ = oracle.selective_log_softmax(H, W, y, tau, scale=s, softcap=c)
    ref = torch.log_softmax(z.detach(), dim=1)[torch.arange(11), torch.tensor(y)].numpy()
    np.testing.assert_allclose(lp, ref, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ dW

def test_dW_matches_finite_differences_in_W():
    # GRPO loss with a softcap and a logit scale: d L / d W by central differences
    H, W, y, cu, mask, old, ref, adv, tau = _case(41, lengths=(3, 4, 2, 3), V=9, D=5)
    kw = dict(clip_eps_low=0.2, clip_eps_high=0.2, beta=0.1)
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, old, ref, adv, tau, scale=0.8, softcap=3.0, with_dW=True,
                                    **kw)
    rho = np.exp(out["logp"] - old)
    assert np.all(np.abs(rho - 0.8) > 1e-3) and np.all(np.abs(rho - 1.2) > 1e-3)

    def loss(Wx):
        lp, _ = oracle.selective_log_softmax(H, Wx, y, tau, scale=0.8, softcap=3.0)
        return oracle.grpo_loss_from_logp(lp, old, ref, adv, cu, mask, **kw)[0]

    h = 1e-6
    fd = np.zeros_like(W)
    for v in range(W.shape[0]):
        for d in range(W.shape[1]):
            e = np.zeros_like(W)
            e[v, d] = h
            fd[v, d] = (loss(W + e) - loss(W - e)) / (2 * h)
    assert np.linalg.norm(out["dW"] - fd) / np.linalg.norm(fd) < 1e-6


def test_dW_cross_entropy_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    H, W, y = _tiny(42, T=13, D=6, V=11)
    tau = 0.7
    mask = np.ones(13)
    mask[[2, 9]] = 0
    out = oracle.cross_entropy_loss_and_grad(H, W, y, mask, tau, with_dW=True)
    Wt = torch.tensor(W, requires_grad=True)
    z = torch.tensor(H) @ Wt.T / tau
    yt = torch.tensor(np.where(mask > 0, y, -100))
    torch.nn.functional.cross_entropy(z, yt, ignore_index=-100).backward()
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=0, atol=1e-15)
    dH, dW = oracle.logp_backward(H, W, y, out["g"], tau, with_dW=True)
    np.testing.assert_allclose(dW, out["dW"], rtol=0, atol=0)


@pytest.mark.parametrize("agg,cap", [("seq_mean", 0.0), ("token_mean", 0.0), ("seq_mean", 2.5)])
def test_full_grpo_gradient_matches_torch_autograd(agg, cap):
    # The whole objective written with torch's own operators in float64 on the CPU (softcapped
    # logits, log_softmax, gather, ratio, clamp, min, k3, the aggregation's weights), and its
    # autograd gradient with respect to H and W: an independent derivative of every term the
    # oracle differentiates by hand (the clipped branch, the KL term, temperature, softcap).
    torch = pytest.importorskip("torch")
    H, W, y, cu, mask, old, ref, adv, tau = _case(23, lengths=(4, 6, 3, 5), D=7, V=19)
    eps_lo, eps_hi, beta = 0.15, 0.25, 0.1
    out = oracle.grpo_loss_and_grad(H, W, y, cu, mask, old, ref, adv, tau, clip_eps_low=eps_lo,
                                    clip_eps_high=eps_hi, beta=beta, agg=agg, softcap=cap, with_dW=True)
    rho = np.exp(out["logp"] - old)
    assert np.any(rho > 1 + eps_hi) and np.any(rho < 1 - eps_lo)  # both clip sides present
    assert np.all(np.abs(rho - (1 + eps_hi)) > 1e-6) and np.all(np.abs(rho - (1 - eps_lo)) > 1e-6)
    T, S = len(y), len(cu) - 1
    seq = np.searchsorted(cu, np.arange(T), side="right") - 1
    m = torch.tensor(mask, dtype=torch.float64)
    if agg == "seq_mean":
        lens = torch.zeros(S, dtype=torch.float64).index_add_(0, torch.tensor(seq), m)
        w = m / (S * lens[torch.tensor(seq)])
    else:
        w = m / m.sum()
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    x = Ht @ Wt.T
    z = (cap * torch.tanh(x / cap) if cap else x) / tau
    lp = torch.log_softmax(z, dim=1).gather(1, torch.tensor(y)[:, None])[:, 0]
    A = torch.tensor(adv)[torch.tensor(seq)]
    ratio = torch.exp(lp - torch.tensor(old))
    surr = torch.minimum(ratio * A, torch.clamp(ratio, 1 - eps_lo, 1 + eps_hi) * A)
    d = torch.tensor(ref) - lp
    k3 = torch.exp(d) - d - 1
    L = (w * -(surr - beta * k3)).sum()
    L.backward()
    np.testing.assert_allclose(out["loss"], L.item(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=0, atol=1e-12 * np.abs(Ht.grad.numpy()).max())
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=0, atol=1e-12 * np.abs(Wt.grad.numpy()).max())
