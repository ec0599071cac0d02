"""Float64 CPU oracle of the LM head with a LoRA adapter: the logprobs and
the learner step when the head carries a trained low-rank update on frozen
weights.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: imported by the tests
and never by the product path; it shares no code with the HIP kernels.

Sources:

* [P2] "Zero mismatch, simple async RL: REINFORCE Zero, DeepSeek-V4.1 and
  Kimi K3.1" (vLLM blog), the "Support for Flagship Models" list and the
  Kimi K3.1 section: zero mismatch holds with LoRA adapters on every module,
  and a LoRA run of DAPO training keeps diff 0 at every step.
* LoRA itself (Hu et al., "LoRA: Low-Rank Adaptation of Large Language
  Models", 2021): a frozen weight W plus a trained update s B A, with A
  [r, H], B [V, r] and a scale s (alpha / r).

Readings (the pages name LoRA only):

* On this path the adapter sits on the head: z = h (W + s B A)^T, W frozen,
  A and B trained; the caller passes s.
* The adapter's activation u = s (h A^T) [N, r] is materialised in the head's
  precision, as a LoRA layer in that precision outputs it: rounded to the
  nearest bfloat16 (ties to even) for a bf16 head, to the nearest float32 for
  an fp32 head.  The logits are then z = h W^T + u B^T, i.e. the plain head
  over the operands [h | u] and [W | B] concatenated along H.
* Gradients go through u as if its rounding were the identity: with
  G = dL/dz, dL/du = G B, dL/dB = G^T u, dL/dA = s (dL/du)^T h and
  dL/dh = G W + s (dL/du) A.  W gets no gradient.

Parity status: pinned by tests/test_oracle_pins.py (the rounding against
torch's float32 -> bfloat16 conversion, the merged-weight identity with an
unrounded activation, a zero B reducing to the plain head, and central
finite differences of the loss in A, B and h).
"""

from __future__ import annotations

import numpy as np

from .reinforce_zero import reinforce_zero_fwd_bwd, token_logprobs

__all__ = ["round_to_bf16", "round_to_f32", "lora_activation",
           "token_logprobs_lora", "reinforce_zero_fwd_bwd_lora"]


def _round_bits(x, bits: int, min_exp: int) -> np.ndarray:
    # nearest number with `bits` significant bits, ties to even; quanta no
    # finer than 2^min_exp (the format's smallest subnormal step)
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - bits, min_exp)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits), ties to even."""
    return _round_bits(x, 8, -133)


def round_to_f32(x) -> np.ndarray:
    """float64 -> nearest float32 value (24 significant bits), ties to even."""
    return _round_bits(x, 24, -149)


def lora_activation(hidden, lora_A, scale: float, dtype: str, round_u: bool = True):
    """u = s (h A^T), rounded to the head's precision (dtype 'bf16' or 'f32')
    unless round_u is False."""
    u = float(scale) * (np.asarray(hidden, np.float64) @ np.asarray(lora_A, np.float64).T)
    if not round_u:
        return u
    return round_to_bf16(u) if dtype == "bf16" else round_to_f32(u)


def _augmented(hidden, lm_head, lora_A, lora_B, scale, dtype, round_u):
    u = lora_activation(hidden, lora_A, scale, dtype, round_u)
    h_aug = np.concatenate([np.asarray(hidden, np.float64), u], axis=1)
    W_aug = np.concatenate([np.asarray(lm_head, np.float64),
                            np.asarray(lora_B, np.float64)], axis=1)
    return u, h_aug, W_aug


def token_logprobs_lora(hidden, lm_head, lora_A, lora_B, scale, tokens,
                        dtype: str, round_u: bool = True):
    """(log pi, lse) of the adapted head: token_logprobs over [h | u] and
    [W | B]."""
    _, h_aug, W_aug = _augmented(hidden, lm_head, lora_A, lora_B, scale,
                                 dtype, round_u)
    return token_logprobs(h_aug, W_aug, tokens)


def reinforce_zero_fwd_bwd_lora(hidden, lm_head, lora_A, lora_B, scale,
                                tokens, logmu, mask, cu_rows, rewards,
                                group_ids, dtype: str, round_u: bool = True):
    """The learner step on the adapted head.  Returns the entries of
    reinforce_zero_fwd_bwd (logpi, loss, adv, d3, kl, ...) with d_hidden the
    gradient with respect to h through both paths, plus d_lora_A [r, H] and
    d_lora_B [V, r]; the frozen head gets none."""
    H = np.asarray(hidden).shape[1]
    u, h_aug, W_aug = _augmented(hidden, lm_head, lora_A, lora_B, scale,
                                 dtype, round_u)
    out = reinforce_zero_fwd_bwd(h_aug, W_aug, tokens, logmu, mask, cu_rows,
                                 rewards, group_ids)
    d_h_aug, d_W_aug = out.pop("d_hidden"), out.pop("d_lm_head")
    d_u = d_h_aug[:, H:]                       # G B
    A = np.asarray(lora_A, np.float64)
    out["d_hidden"] = d_h_aug[:, :H] + float(scale) * (d_u @ A)
    out["d_lora_A"] = float(scale) * (d_u.T @ np.asarray(hidden, np.float64))
    out["d_lora_B"] = d_W_aug[:, H:]           # G^T u
    out["u"] = u
    return out
