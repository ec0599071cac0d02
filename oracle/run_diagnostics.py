"""Float64 CPU oracle of the run-level diagnostics built from one learner
step's outputs.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: imported by the tests
and never by the product path; it shares no code with the HIP kernels.

Sources:

* [P2] "Zero mismatch, simple async RL: REINFORCE Zero, DeepSeek-V4.1 and
  Kimi K3.1" (vLLM blog, Chinese translation): §3, Figure 1 (the
  peak-to-median ratio of the per-update D3 over a run); §4 "What happens
  without alignment" (the rollout-to-learner KL median over the first and
  the last 1,000 updates, the largest gradient norm before clipping, and the
  share of sequences a gate rejects -- none for REINFORCE Zero).
* [P5] "REINFORCE Zero" project page, §01 Figure 2 (batch-averaged D3, peak
  over median).

Readings:

* The gradient norms are the plain L2 norms of this path's two gradients,
  dL/dhidden [n_rows, H] and dL/dW [V, H], each over all its elements (the
  path owns only these two; a trainer adds the rest of the network's).
* Per-response D3 and KL are the step diagnostics restricted to one
  response's valid tokens (NaN for a response with none).
* Run level: over the recorded steps, D3 peak / median; the median KL of the
  first and of the last `window` steps and their ratio; the largest gradient
  norm.  The median is the usual one (mean of the two middle values for an
  even count).  Quotients are IEEE divisions (a zero median gives inf or
  NaN); a NaN step value makes its statistics NaN.

Parity status: pinned by tests/test_oracle_pins.py (hand cases, a library
norm on a tiny array, permutation and scaling identities).
"""

from __future__ import annotations

import numpy as np

__all__ = ["grad_norms", "response_diagnostics", "run_summary"]


def grad_norms(d_hidden: np.ndarray, d_lm_head: np.ndarray):
    """(||dL/dhidden||_2, ||dL/dW||_2) over all elements, float64."""
    def l2(x):
        x = np.asarray(x, dtype=np.float64).ravel()
        return float(np.sqrt(np.dot(x, x)))
    return l2(d_hidden), l2(d_lm_head)


def response_diagnostics(logpi, logmu, mask, cu_rows):
    """Per response i: D3_i = mean over its valid tokens of expm1(d) - d and
    KL_i = mean of -d (d = log pi - log mu); NaN where it has none."""
    logpi = np.asarray(logpi, np.float64)
    logmu = np.asarray(logmu, np.float64)
    valid = np.asarray(mask) != 0
    cu = np.asarray(cu_rows, np.int64)
    B = len(cu) - 1
    d3 = np.full(B, np.nan)
    kl = np.full(B, np.nan)
    for i in range(B):
        rows = np.arange(cu[i], cu[i + 1])
        rows = rows[valid[rows]]
        if rows.size == 0:
            continue
        d = logpi[rows] - logmu[rows]
        d3[i] = float(np.mean(np.expm1(d) - d))
        kl[i] = float(np.mean(-d))
    return d3, kl


def run_summary(d3_steps, kl_steps, grad_norm_steps, window: int = 1000):
    """Run-level view over recorded steps (see the module docstring)."""
    d3 = np.asarray(d3_steps, np.float64)
    kl = np.asarray(kl_steps, np.float64)
    g = np.asarray(grad_norm_steps, np.float64)
    w = min(window, len(kl))
    first = np.float64(np.median(kl[:w])) if w else np.float64(np.nan)
    last = np.float64(np.median(kl[-w:])) if w else np.float64(np.nan)
    peak = np.float64(np.max(d3)) if len(d3) else np.float64(np.nan)
    med = np.float64(np.median(d3)) if len(d3) else np.float64(np.nan)
    with np.errstate(divide="ignore", invalid="ignore"):
        # IEEE quotients: a run with D3 = 0 at every step has a zero median
        ratio_d3, ratio_kl = peak / med, last / first
    return {
        "d3_peak": float(peak),
        "d3_median": float(med),
        "d3_peak_over_median": float(ratio_d3),
        "kl_median_first": float(first),
        "kl_median_last": float(last),
        "kl_median_ratio": float(ratio_kl),
        "grad_norm_max": float(np.max(g)) if len(g) else np.nan,
    }
