"""Plain, slow, fp64 CPU oracle for chunked GRPO log-probabilities, loss and dH.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import or run this module.  The library never calls it,
and it shares no code with the HIP path.

What it computes, and where the pages state it (page titles as printed):

[P4] "Reinforcement Learning GRPO mit 7x laengerem Kontext" (Unsloth docs).
     Section "Chunking der abgeflachten Sequenzlaenge" (Eq. 3) and the
     following call of ``chunked_hidden_states_selective_log_softmax``: logits
     are ``hidden_states @ lm_head`` taken over the flattened
     (batch x context) tokens, upcast to float32, divided by the temperature,
     log-softmaxed and gathered at the target id.  Section "Auslagern von
     Aktivierungen fuer Log-Softmax": the backward recomputes the same
     quantity and back-propagates ``grad_output`` through it.
[P2] "Unsloth internals", section "The relationship to TRL": the trainer
     samples a group of completions per prompt, computes group-relative
     advantages and forms the clipped surrogate objective with a
     KL-to-reference term.
[P3] "You can now train reasoning models with 5GB VRAM thanks to Unsloth",
     section "Under the Hood": the KL is the reverse KL; the importance ratio
     ``exp(q - q.detach())`` times the per-sequence advantage broadcast over
     tokens equals 1 in value and carries gradient A on policy.
[P1] "Unsloth GRPO Implementation ...", section "Corrected Hyperparameters
     for GRPO Stability": beta = 0.001.
[P2] "Unsloth internals", the paragraph on the fused, chunked cross-entropy:
     the supervised loss over the vocabulary is computed without the full fp32
     logits tensor or its same-shape gradient; here it is the mean over the
     unmasked tokens of -logp through the same chunked log-softmax.

Readings where the pages are silent (each is also listed in the design notes):
unbiased std, eps added to the std (default 1e-4), A = 0 for a group whose
rewards are all equal or whose size is 1, sequences grouped as consecutive
runs of G, symmetric inclusive clip range [1-eps_lo, 1+eps_hi], the k3
estimator exp(d) - d - 1 with d = ref_logp - logp subtracted outside the min,
per-sequence-mean aggregation (token-mean as an option), and row t of H
predicting targets[t].  The chunk size never changes any value computed here:
every per-token quantity depends on its own row only.

All arithmetic is float64.  bf16 inputs are widened exactly from their bit
patterns, so comparisons measure kernel error and not input rounding.

Parity pins: every function here is pinned in tests/test_oracle_pins.py.  Parity
unpinned against the pages for the readings they leave open (the std estimator, where
eps enters, the per-sequence-mean aggregation, and the order of logit scale, softcap
and temperature): the pages fix none of them, so the pins check each chosen reading's
own closed forms, limits and derivatives, not a value the pages print.
"""
from __future__ import annotations

import math

import numpy as np

ROW_BLOCK = 1024


# ---------------------------------------------------------------- inputs

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of an input tensor.

    ``dtype == "bf16"``: ``x`` holds uint16 bit patterns; a bf16 value is the
    float32 whose upper 16 bits are the pattern and lower 16 bits are zero.
    ``dtype == "f32"``: ``x`` holds float32 values.
    """
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- log-softmax

def logit_map(x: np.ndarray, temperature: float = 1.0, scale: float = 1.0, softcap: float = 0.0):
    """Logits z from the raw lm_head products x = H[t] . W[v], and dz/dx.

    [P4] lists the call's arguments logit_scale_multiply, logit_scale_divide,
    logit_softcapping and temperature (item 3 after the call: softcapping
    and temperature scaling are supported) without fixing their order; the
    reading taken here: u = scale * x (scale = multiply / divide), with a
    softcap c > 0 u = c * tanh(u / c), and z = u / temperature.
    """
    u = scale * x
    if softcap > 0:
        t = np.tanh(u / softcap)
        return softcap * t / temperature, scale * (1.0 - t * t) / temperature
    return u / temperature, np.full(np.shape(x), scale / temperature)


def logits(H: np.ndarray, W: np.ndarray, temperature: float = 1.0, scale: float = 1.0,
           softcap: float = 0.0) -> np.ndarray:
    """z[t, v] for every vocabulary entry: logit_map of H[t] . W[v] ([P4], call args)."""
    return logit_map(H @ W.T, temperature, scale, softcap)[0]


def _dx_rows(H_rows, W, y, lse_rows, g_rows, temperature, scale, softcap):
    """g_t * d logp_t / dx_t (x = the raw lm_head products) for rows with a valid target:
    the recomputed logits give softmax p; d logp / dz = onehot(y) - p; dz/dx from logit_map."""
    z, dz = logit_map(H_rows @ W.T, temperature, scale, softcap)
    p = np.exp(z - lse_rows[:, None])
    dl = -p
    dl[np.arange(dl.shape[0]), y] += 1.0
    return g_rows[:, None] * (dl * dz)


def _dH_rows(H_rows, W, y, lse_rows, g_rows, temperature, scale, softcap):
    """g_t * d logp_t / dH_t = (g_t d logp_t / dx_t) W, since dx/dH = W."""
    return _dx_rows(H_rows, W, y, lse_rows, g_rows, temperature, scale, softcap) @ W


def selective_log_softmax(H: np.ndarray, W: np.ndarray, targets: np.ndarray,
                          temperature: float = 1.0, block: int = ROW_BLOCK, scale: float = 1.0,
                          softcap: float = 0.0):
    """Per-token log-probability of the target id, and the log-sum-exp.

    Brute force over the full vocabulary, a block of rows at a time ([P4]:
    logits, log-softmax, gather of the target id).  A target outside
    [0, V) yields NaN log-probability.  Returns (logp[T], lse[T]).
    """
    T = H.shape[0]
    V = W.shape[0]
    logp = np.empty(T)
    lse = np.empty(T)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        z = logits(H[r0:r1], W, temperature, scale, softcap)
        m = z.max(axis=1)
        l = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        y = targets[r0:r1].astype(np.int64)
        ok = (y >= 0) & (y < V)
        zy = np.full(r1 - r0, np.nan)
        zy[ok] = z[np.nonzero(ok)[0], y[ok]]
        lse[r0:r1] = l
        logp[r0:r1] = zy - l
    return logp, lse


# ---------------------------------------------------------------- advantages

def group_advantages(rewards: np.ndarray, group_size: int, std: str = "unbiased",
                     eps: float = 1e-4) -> np.ndarray:
    """Group-relative advantages ([P2], "The relationship to TRL").

    Sequence i belongs to group i // group_size.  Within a group,
    A_i = (r_i - mean) / (std + eps).  A group of one, or whose rewards are
    all equal, gets A = 0.
    """
    r = np.asarray(rewards, dtype=np.float64)
    S = r.shape[0]
    if group_size <= 0 or S % group_size != 0:
        raise ValueError("number of sequences must be a multiple of the group size")
    A = np.zeros(S)
    for g0 in range(0, S, group_size):
        grp = r[g0:g0 + group_size]
        if group_size == 1 or np.all(grp == grp[0]):
            continue
        mu = grp.sum() / group_size
        dev = grp - mu
        ddof = 1 if std == "unbiased" else 0
        sigma = math.sqrt(float((dev * dev).sum()) / (group_size - ddof))
        A[g0:g0 + group_size] = dev / (sigma + eps)
    return A


# ---------------------------------------------------------------- token index

def sequence_of_token(cu: np.ndarray) -> np.ndarray:
    """s(t): the sequence i with cu[i] <= t < cu[i+1] in the flattened stream ([P4], Eq. 3 section)."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.repeat(np.arange(cu.shape[0] - 1), np.diff(cu))


def token_weights(cu: np.ndarray, mask: np.ndarray, agg: str = "seq_mean") -> np.ndarray:
    """Loss weight w_t of every token.

    seq_mean: w_t = mask_t / (S * L_s(t)), L_i the number of unmasked tokens
    of sequence i (0 when L_i = 0; the sequence still counts in S).
    token_mean: w_t = mask_t / sum(mask).
    """
    cu = np.asarray(cu, dtype=np.int64)
    S = cu.shape[0] - 1
    m = np.asarray(mask).astype(np.float64)
    s = sequence_of_token(cu)
    if agg == "seq_mean":
        L = np.array([m[cu[i]:cu[i + 1]].sum() for i in range(S)])
        denom = S * L[s]
    elif agg == "token_mean":
        denom = np.full(m.shape[0], m.sum())
    else:
        raise ValueError(agg)
    w = np.zeros(m.shape[0])
    nz = m != 0
    w[nz] = m[nz] / denom[nz]
    return w


# ---------------------------------------------------------------- GRPO objective

def grpo_token_terms(logp, old_logp, ref_logp, adv_t, clip_eps_low=0.2, clip_eps_high=0.2,
                     beta=0.001):
    """Per-token objective l_t and its derivative with respect to logp_t.

    rho   = exp(logp - old)                       (importance ratio, [P3])
    surr  = min(rho A, clip(rho, 1-eps_lo, 1+eps_hi) A)   ([P2])
    d     = ref - logp
    k3    = exp(d) - d - 1                        (reverse-KL estimate, [P3])
    l     = -(surr - beta k3)
    dl/dlogp = -(rho A if rho A <= clip(rho) A else 0) + beta (1 - exp(d))

    ``ref_logp`` may be None only when beta == 0.  Returns a dict of arrays.
    """
    logp = np.asarray(logp, dtype=np.float64)
    A = np.asarray(adv_t, dtype=np.float64)
    rho = np.exp(logp - np.asarray(old_logp, dtype=np.float64))
    c = np.clip(rho, 1.0 - clip_eps_low, 1.0 + clip_eps_high)
    unclipped = rho * A
    clipped = c * A
    surr = np.minimum(unclipped, clipped)
    dsurr = np.where(unclipped <= clipped, unclipped, 0.0)
    if ref_logp is None:
        if beta != 0:
            raise ValueError("ref_logp is required when beta != 0")
        k3 = np.zeros_like(logp)
        dk3 = np.zeros_like(logp)
    else:
        d = np.asarray(ref_logp, dtype=np.float64) - logp
        em1 = np.expm1(d)
        k3 = em1 - d
        dk3 = -em1
    ell = -(surr - beta * k3)
    dell = -dsurr + beta * dk3
    return dict(ell=ell, dell=dell, rho=rho, surr=surr, k3=k3)


def grpo_loss_from_logp(logp, old_logp, ref_logp, adv, cu, mask, clip_eps_low=0.2,
                        clip_eps_high=0.2, beta=0.001, agg="seq_mean"):
    """Loss L = sum_t w_t l_t, per-token l_t and g_t = dL/dlogp_t, from given log-probs.

    Masked tokens get g_t = 0.  The sum is taken with math.fsum (exactly
    rounded), so it carries no summation-order error of its own.
    Returns (L, ell[T], g[T]).
    """
    s = sequence_of_token(cu)
    A_t = np.asarray(adv, dtype=np.float64)[s]
    w = token_weights(cu, mask, agg)
    terms = grpo_token_terms(logp, old_logp, ref_logp, A_t, clip_eps_low, clip_eps_high, beta)
    ell = terms["ell"]
    g = np.where(np.asarray(mask) != 0, w * terms["dell"], 0.0)
    contrib = np.where(w != 0, w * ell, 0.0)
    L = math.fsum(contrib.tolist())
    return L, ell, g


def grpo_loss_and_grad(H, W, targets, cu, mask, old_logp, ref_logp, adv, temperature=1.0,
                       clip_eps_low=0.2, clip_eps_high=0.2, beta=0.001, agg="seq_mean",
                       block: int = ROW_BLOCK, scale: float = 1.0, softcap: float = 0.0,
                       with_dW: bool = False):
    """Loss, log-probs and the gradient of the loss with respect to H.

    dH_t = (g_t / temperature) * (W[y_t] - sum_v softmax(z_t)_v W[v]), the
    chain rule through logp_t = z_{t,y_t} - LSE_t, whose derivative with
    respect to z_t is onehot(y_t) - softmax(z_t) ([P4], the recompute
    backward); with a logit scale or softcap the softmax term carries dz/dx (see
    logit_map).  Rows with g_t = 0 or an out-of-range target are exactly 0.  With
    with_dW, also dW = sum_t (g_t dlogp_t/dx_t)^T H_t, the lm_head gradient a full
    fine-tune needs (x = H W^T).
    """
    T, D = H.shape
    V = W.shape[0]
    logp, lse = selective_log_softmax(H, W, targets, temperature, block, scale, softcap)
    L, ell, g = grpo_loss_from_logp(logp, old_logp, ref_logp, adv, cu, mask, clip_eps_low,
                                    clip_eps_high, beta, agg)
    dH = np.zeros((T, D))
    dW = np.zeros((V, D)) if with_dW else None
    y_all = np.asarray(targets, dtype=np.int64)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        rows = np.arange(r0, r1)
        y = y_all[r0:r1]
        live = (g[r0:r1] != 0) & (y >= 0) & (y < V)
        if not live.any():
            continue
        gx = _dx_rows(H[r0:r1][live], W, y[live], lse[rows[live]], g[rows[live]], temperature, scale,
                      softcap)
        dH[rows[live]] = gx @ W
        if dW is not None:
            dW += gx.T @ H[r0:r1][live]
    return dict(loss=L, logp=logp, lse=lse, token_loss=ell, g=g, dH=dH, dW=dW)


def logp_backward(H, W, targets, grad_logp, temperature=1.0, block: int = ROW_BLOCK, scale: float = 1.0,
                  softcap: float = 0.0, with_dW: bool = False):
    """Gradient with respect to H of sum_t grad_logp[t] * logp_t.

    The backward of the chunked selective log-softmax ([P4], "Auslagern von
    Aktivierungen fuer Log-Softmax"): the forward keeps only the log-sum-exp,
    the backward recomputes the logits and applies the incoming gradient of
    the log-probabilities, dH_t = (grad_t / temperature) * (W[y_t] - sum_v
    softmax(z_t)_v W[v]).  Rows with grad_t = 0 or an out-of-range target are
    exactly 0.  With with_dW, returns (dH, dW) with dW the gradient with respect to W.
    """
    T, D = H.shape
    V = W.shape[0]
    g = np.asarray(grad_logp, dtype=np.float64)
    _, lse = selective_log_softmax(H, W, targets, temperature, block, scale, softcap)
    dH = np.zeros((T, D))
    dW = np.zeros((V, D)) if with_dW else None
    y_all = np.asarray(targets, dtype=np.int64)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        rows = np.arange(r0, r1)
        y = y_all[r0:r1]
        live = (g[r0:r1] != 0) & (y >= 0) & (y < V)
        if not live.any():
            continue
        gx = _dx_rows(H[r0:r1][live], W, y[live], lse[rows[live]], g[rows[live]], temperature, scale,
                      softcap)
        dH[rows[live]] = gx @ W
        if dW is not None:
            dW += gx.T @ H[r0:r1][live]
    return (dH, dW) if with_dW else dH


def cross_entropy_loss_and_grad(H, W, targets, mask=None, temperature=1.0, block: int = ROW_BLOCK,
                                scale: float = 1.0, softcap: float = 0.0, with_dW: bool = False):
    """Chunked cross-entropy (the supervised loss the same chunked log-softmax
    serves): L = -(1/N) sum_t mask_t logp_t with N = sum_t mask_t (L = 0 and
    dH = 0 when N = 0), per-token loss -logp_t, g_t = dL/dlogp_t = -mask_t / N,
    dH by the backward above.  A masked token contributes exactly 0 even when
    its target is out of range.
    """
    T = H.shape[0]
    m = np.ones(T) if mask is None else np.asarray(mask, dtype=np.float64)
    logp, lse = selective_log_softmax(H, W, targets, temperature, block, scale, softcap)
    n = m.sum()
    w = m / n if n > 0 else np.zeros(T)
    terms = [w[t] * (-logp[t]) for t in range(T) if w[t] != 0]
    L = math.fsum(terms) if terms else 0.0
    g = -w
    out = logp_backward(H, W, targets, g, temperature, block, scale, softcap, with_dW)
    dH, dW = out if with_dW else (out, None)
    return dict(loss=L, logp=logp, lse=lse, token_loss=-logp, g=g, dH=dH, dW=dW)


def grad_rows(H_rows, W, targets_rows, lse_rows, g_rows, temperature=1.0, scale=1.0, softcap=0.0):
    """dH for selected rows given their lse and g (row-local, for sampled checks)."""
    V = W.shape[0]
    out = np.zeros(H_rows.shape)
    y = np.asarray(targets_rows, dtype=np.int64)
    live = (g_rows != 0) & (y >= 0) & (y < V)
    if live.any():
        out[live] = _dH_rows(H_rows[live], W, y[live], lse_rows[live], g_rows[live], temperature, scale,
                             softcap)
    return out
