"""Float64 CPU oracle of the score-centering (SC) update.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path;
it shares no code with the HIP kernels.

Source: the "REINFORCE Zero" project page (hujian.website), "The full IS
correction", blocks 02 and 03.  At a fixed history, with target p, sampler q,
advantage A and score s = grad log p: the uncorrected update E_q[A s] is
Cov_q(A, s) plus the drift E_q[A] E_q[s]; score centering removes the drift
and keeps g_SC = Cov_q(A, s).  Its gap to the target update is
Cov_q(A, s) - Cov_p(A, s).  The vLLM blog "Zero mismatch, simple async RL"
(Chinese translation), section 4 "Results", trains a "Score Centering without
IS" arm with aligned kernels.

Reading (the pages give SC as an expectation, not as a loss): a covariance
needs one centred factor, Cov_q(A, s) = E_q[(A - E_q A) s], and the
group-mean advantage A_i = r_i - mean of r over the group is that centred
factor, estimated from the sampler's own draws.  So the SC estimate is the
REINFORCE Zero update with the importance weight replaced by 1:

    L_SC = -(1/B) sum_i (1/T_i) sum_{valid t of i} A_i log pi_t,

whose gradient through log pi is the SC update (negated), with per-token
coefficient c_t = A_i / (B T_i).  T_i, A_i, the two-level mean and the
masked-row conventions are those of reinforce_zero.py.

Parity status: pinned by tests/test_oracle_pins.py (the covariance identities
by exact enumeration, finite differences of L_SC, a hand case, equal rewards).
"""

from __future__ import annotations

import numpy as np

from .reinforce_zero import (backward, diagnostics, group_mean_advantages,
                             token_logprobs, valid_token_counts)

__all__ = ["score_centering_surrogate", "score_centering_fwd_bwd"]


def score_centering_surrogate(logpi, mask, cu_rows, A, T) -> float:
    """L_SC = -(1/B) sum_i (1/T_i) sum_{valid t of i} A_i * log pi_t.

    Each response's tokens are averaged, then the responses (as in the
    REINFORCE Zero objective); a response with T_i = 0 adds nothing.
    """
    B = len(cu_rows) - 1
    total = 0.0
    for i in range(B):
        if T[i] == 0:
            continue
        rows = slice(cu_rows[i], cu_rows[i + 1])
        total += A[i] * float(np.sum(np.asarray(logpi)[rows][np.asarray(mask)[rows] != 0])) / T[i]
    return -total / B


def score_centering_fwd_bwd(hidden, lm_head, tokens, mask, cu_rows, rewards,
                            group_ids, logmu=None):
    """The SC step: logprobs, L_SC, A, c_t = A_i / (B T_i), and the
    gradients of L_SC with respect to the hidden states and the head.
    With log mu given, D3 and KL of the records as well (they do not enter
    the update).  Masked rows report log pi = 0 and zero gradient rows."""
    mask = np.asarray(mask)
    logpi_all, lse = token_logprobs(hidden, lm_head, tokens)
    logpi = np.where(mask != 0, logpi_all, 0.0)
    T = valid_token_counts(cu_rows, mask)
    A = group_mean_advantages(rewards, group_ids)
    B = len(cu_rows) - 1
    c = np.zeros(len(logpi), dtype=np.float64)
    for i in range(B):
        if T[i] == 0:
            continue
        for t in range(cu_rows[i], cu_rows[i + 1]):
            if mask[t]:
                c[t] = A[i] / (B * T[i])
    loss = score_centering_surrogate(logpi, mask, cu_rows, A, T)
    d_hidden, d_head = backward(hidden, lm_head, tokens, lse, c)
    out = {"logpi": logpi, "lse": lse, "T": T, "adv": A, "coef": c,
           "loss": loss, "d_hidden": d_hidden, "d_lm_head": d_head}
    if logmu is not None:
        out["d3"], out["kl"] = diagnostics(logpi, logmu, mask)
    return out
