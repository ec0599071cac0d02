"""Float64 CPU oracle for the REINFORCE Zero learner hot path.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plainly written definition
that the GPU path is checked against.  Only the test suite, the package smoke
check and the CPU-baseline leg of the benchmark may import it; the product path
never calls it, and it shares no code with the HIP kernels or their binding.

Sources (the pages are cited by title and section; no page prints code):

* [P2] "Zero mismatch, simple async RL: REINFORCE Zero, DeepSeek-V4.1 and
  Kimi K3.1" (vLLM blog, Chinese translation at todayforai.com):
  §2 (importance ratio pi/mu per token), §3 (the gap identity and the D3
  diagnostic), §4 "Recipe" items 1-3 and the loss equation, §4 "What happens
  without alignment" (rollout-to-learner KL).
* [P5] "REINFORCE Zero" project page (hujian.website): §02 "The mechanism",
  block "A minimal REINFORCE objective" (the loss, T_i = number of valid
  action tokens, gradient through the numerator only); "The full IS
  correction" (the identities E_q[w s] = 0 and E_q[w A s] = E_p[A s]).

Everything is computed exactly as those passages state it, in float64, with
no blocking, fusion or reordering beyond chunking rows to bound memory (each
row is independent, so chunking changes no value).

Readings where the pages are silent (each is repeated in the design notes):

* The policy pi_theta(a | h) is a plain linear LM head without bias on the
  final hidden state, W laid out [V, H], temperature 1, followed by a
  log-softmax over the whole vocabulary.  The pages never spell out the head.
* The advantage is the reward minus the plain mean reward of the response's
  group (the mean includes the response itself; no division by a standard
  deviation).  A group id names the group; any ids may appear.
* T_i counts the rows of response i whose mask is 1.  A response with
  T_i = 0 contributes nothing to the loss or the gradient, but still counts
  in B.
* D3 is a flat mean of w - 1 - log w over the call's valid tokens, written as
  expm1(d) - d with d = log pi - log mu so that w = 1 gives exactly 0.
* The "sampled rollout-to-learner KL" is the k1 estimator
  mean(log mu - log pi) over valid tokens (KL(mu || pi) sampled under mu).
* Masked rows get log pi = 0 and zero gradient rows in the fused call.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, library routines it does not itself call, brute force,
finite differences and the exact-enumeration IS identities).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16",
    "to_f64",
    "lm_head_logits",
    "log_softmax_rows",
    "token_logprobs",
    "log_ratio",
    "valid_token_counts",
    "group_mean_advantages",
    "is_reinforce_loss",
    "token_coefficients",
    "diagnostics",
    "loss_stage",
    "backward",
    "reinforce_zero_fwd_bwd",
]

ROW_CHUNK = 256  # rows per logits block; bounds memory only


# ---------------------------------------------------------------- input decode
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper 16 bits of an IEEE binary32, so shifting the
    pattern into the high half of a 32-bit word gives the float32 value, which
    widens to float64 with no rounding.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen an input array ('f32' values or 'bf16' bit patterns) to float64."""
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------- per-token logprobs
def lm_head_logits(hidden: np.ndarray, lm_head: np.ndarray) -> np.ndarray:
    """z[t, v] = sum_h hidden[t, h] * W[v, h]  (reading: linear head, no bias).

    The policy pi_theta(a_it | h_it) of [P2] §4 loss equation and [P5]
    "A minimal REINFORCE objective" is the softmax of these logits.
    """
    return hidden @ lm_head.T


def log_softmax_rows(z: np.ndarray):
    """Row-wise log-sum-exp and log-softmax, the textbook max-shifted form.

    lse_t = M_t + log sum_v exp(z[t, v] - M_t) with M_t = max_v z[t, v];
    log p[t, v] = z[t, v] - lse_t.
    """
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    return lse, z - lse[:, None]


def token_logprobs(hidden: np.ndarray, lm_head: np.ndarray, tokens: np.ndarray,
                   row_chunk: int = ROW_CHUNK):
    """log pi_theta(a_t | h_t) for every row, plus its log-sum-exp.

    [P2] §4 Recipe item 2: the learner's own probability of the token the
    rollout sampled.  Rows are independent; they are processed in blocks of
    `row_chunk` only to bound the size of the logits block.
    """
    n = hidden.shape[0]
    logpi = np.empty(n, dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        z = lm_head_logits(hidden[r0:r1], lm_head)
        l, _ = log_softmax_rows(z)
        lse[r0:r1] = l
        logpi[r0:r1] = z[np.arange(r1 - r0), tokens[r0:r1]] - l
    return logpi, lse


# -------------------------------------------------------------- the IS loss
def log_ratio(logpi: np.ndarray, logmu: np.ndarray) -> np.ndarray:
    """d_t = log pi_t - log mu_t, so the unclipped weight is w_t = exp(d_t).

    [P2] §2 and §4 Recipe item 2: the learner's probability divided by the
    probability the rollout recorded, used as is (no truncation, no filter).
    """
    return np.asarray(logpi, np.float64) - np.asarray(logmu, np.float64)


def valid_token_counts(cu_rows: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """T_i = number of valid action tokens of response i ([P5] objective)."""
    B = len(cu_rows) - 1
    T = np.zeros(B, dtype=np.int64)
    for i in range(B):
        T[i] = int(np.sum(mask[cu_rows[i]:cu_rows[i + 1]] != 0))
    return T


def group_mean_advantages(rewards: np.ndarray, group_ids: np.ndarray) -> np.ndarray:
    """A_i = r_i - (mean reward of the group of response i).

    [P2] §4 Recipe item 3: each response's advantage is its reward minus the
    average reward of its group; there is no value model.
    """
    r = np.asarray(rewards, np.float64)
    g = np.asarray(group_ids, np.int64)
    A = np.empty_like(r)
    for i in range(len(r)):
        members = r[g == g[i]]
        A[i] = r[i] - members.sum() / len(members)
    return A


def is_reinforce_loss(w: np.ndarray, mask: np.ndarray, cu_rows: np.ndarray,
                      A: np.ndarray, T: np.ndarray) -> float:
    """L = -(1/B) sum_i (1/T_i) sum_{valid t of i} A_i * w_t.

    [P2] §4 loss equation; [P5] "A minimal REINFORCE objective": average over
    the action tokens within each response, then over the B responses.
    """
    B = len(cu_rows) - 1
    total = 0.0
    for i in range(B):
        if T[i] == 0:
            continue
        rows = slice(cu_rows[i], cu_rows[i + 1])
        s_i = float(np.sum(w[rows][mask[rows] != 0]))
        total += A[i] * s_i / T[i]
    return -total / B


def token_coefficients(w: np.ndarray, mask: np.ndarray, cu_rows: np.ndarray,
                       A: np.ndarray, T: np.ndarray) -> np.ndarray:
    """c_t = dL/d(log pi_t) negated: c_t = A_i * w_t / (B * T_i) on valid rows.

    [P5] "A minimal REINFORCE objective": the gradient flows through the
    current-policy numerator only, so d w_t = w_t * d log pi_t while mu, A_i
    and T_i are constants.  dL/d log pi_t = -A_i w_t / (B T_i) = -c_t.
    """
    B = len(cu_rows) - 1
    c = np.zeros(len(w), dtype=np.float64)
    for i in range(B):
        if T[i] == 0:
            continue
        for t in range(cu_rows[i], cu_rows[i + 1]):
            if mask[t]:
                c[t] = A[i] * w[t] / (B * T[i])
    return c


def diagnostics(logpi: np.ndarray, logmu: np.ndarray, mask=None):
    """(D3, KL) over the valid tokens.

    D3: [P2] §3 -- the mean over the update's tokens of w - 1 - log w, which is
    0 at w = 1; written expm1(d) - d (same value, no cancellation near 0).
    KL: the sampled rollout-to-learner KL of [P2] §4 and [P5] §01, read as
    the k1 estimate mean(log mu - log pi) under the rollout's samples.
    An empty valid set gives NaN for both.
    """
    d = log_ratio(logpi, logmu)
    if mask is not None:
        d = d[np.asarray(mask) != 0]
    if d.size == 0:
        return float("nan"), float("nan")
    d3 = float(np.mean(np.expm1(d) - d))
    kl = float(np.mean(-d))
    return d3, kl


def loss_stage(logpi, logmu, mask, cu_rows, rewards, group_ids):
    """Steps after the logprobs: w, T, A, loss, per-token c, D3 and KL."""
    mask = np.asarray(mask)
    d = log_ratio(logpi, logmu)
    w = np.where(mask != 0, np.exp(np.where(mask != 0, d, 0.0)), 0.0)
    T = valid_token_counts(cu_rows, mask)
    A = group_mean_advantages(rewards, group_ids)
    loss = is_reinforce_loss(w, mask, cu_rows, A, T)
    c = token_coefficients(w, mask, cu_rows, A, T)
    d3, kl = diagnostics(logpi, logmu, mask)
    return {"w": w, "T": T, "adv": A, "loss": loss, "coef": c,
            "d3": d3, "kl": kl}


# ----------------------------------------------------------------- gradient
def backward(hidden: np.ndarray, lm_head: np.ndarray, tokens: np.ndarray,
             lse: np.ndarray, coef: np.ndarray, row_chunk: int = ROW_CHUNK):
    """Gradients of the loss with respect to the hidden states and the head.

    With G[t, v] = dL/dz[t, v] = c_t * (p[t, v] - [v == a_t]) and
    p = exp(z - lse): dL/dhidden = G @ W and dL/dW = G^T @ hidden.
    Rows with c_t = 0 (masked rows) contribute nothing.
    """
    n, H = hidden.shape
    V = lm_head.shape[0]
    d_hidden = np.zeros((n, H), dtype=np.float64)
    d_head = np.zeros((V, H), dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        z = lm_head_logits(hidden[r0:r1], lm_head)
        p = np.exp(z - lse[r0:r1, None])
        p[np.arange(r1 - r0), tokens[r0:r1]] -= 1.0
        G = coef[r0:r1, None] * p
        d_hidden[r0:r1] = G @ lm_head
        d_head += G.T @ hidden[r0:r1]
    return d_hidden, d_head


def reinforce_zero_fwd_bwd(hidden, lm_head, tokens, logmu, mask, cu_rows,
                           rewards, group_ids, row_chunk: int = ROW_CHUNK):
    """The whole learner step: logprobs, loss, advantages, D3/KL, gradients.

    hidden [N, H] and lm_head [V, H] are float64 (already widened).  Masked
    rows report log pi = 0 and a zero gradient row.
    """
    mask = np.asarray(mask)
    logpi_all, lse = token_logprobs(hidden, lm_head, tokens, row_chunk)
    logpi = np.where(mask != 0, logpi_all, 0.0)
    st = loss_stage(logpi, logmu, mask, cu_rows, rewards, group_ids)
    d_hidden, d_head = backward(hidden, lm_head, tokens, lse, st["coef"],
                                row_chunk)
    out = dict(st)
    out.update({"logpi": logpi, "lse": lse, "d_hidden": d_hidden,
                "d_lm_head": d_head})
    return out
