"""Float64 CPU oracle of the rollout-side head: draw each row's token from
the full softmax and record its logprob.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: imported by the tests
and never by the product path; it shares no code with the HIP kernels.

Sources:

* [P2] "Zero mismatch, simple async RL: REINFORCE Zero, DeepSeek-V4.1 and
  Kimi K3.1" (vLLM blog, Chinese translation), §4 "Recipe" item 2: the
  rollout records the logprob of every token it samples, and the learner
  divides its own probability by that record; §5: "diff 0", rollout and
  trainer compute bit-identical logprobs for every sampled token.
* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
  Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): four 32-bit
  counter words, a two-word key, ten rounds; each round multiplies words 0
  and 2 by fixed 32-bit constants, and the key grows by fixed Weyl
  increments between rounds.

Readings (the pages do not say how tokens are drawn):

* A token is drawn from softmax(z_t) at temperature 1, the policy of the
  learner oracle, by the Gumbel-max rule
      a_t = argmax_v  z[t, v] + g[t, v],   g = -log(-log u[t, v]),
  ties going to the smallest v.
* u[t, v] = (x + 1/2) / 2^32 with x = word (v mod 4) of
  Philox4x32-10(counter = (v div 4, id_lo, id_hi, 0), key = (seed_lo,
  seed_hi)), where id is the row's caller-given 64-bit identity.  The draw
  of a row then depends on (seed, id, its hidden state) only, never on the
  batch it is drawn in.
* The recorded behaviour logprob is log mu_t = log softmax(z_t)[a_t], the
  same definition as the learner's log pi (token_logprobs).

Parity status: philox4x32_10 is pinned by published known-answer vectors,
gumbel_uniforms by its range and moments, sample_tokens by the frequencies
of many draws against softmax (tests/test_oracle_pins.py).
"""

from __future__ import annotations

import numpy as np

from .reinforce_zero import lm_head_logits, log_softmax_rows

__all__ = ["philox4x32_10", "gumbel_uniforms", "sample_tokens"]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57        # round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85        # key (Weyl) increments
_MASK = 0xFFFFFFFF


def philox4x32_10(counter: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Philox4x32 with 10 rounds.  counter: (..., 4) uint32, key: (..., 2)
    uint32 (broadcast against each other); returns (..., 4) uint32.

    One round, with (hi, lo) the halves of a 64-bit product:
        (hi0, lo0) = M0 * c0,   (hi1, lo1) = M1 * c2,
        c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0),
    and before every round after the first, k <- (k0 + W0, k1 + W1) mod 2^32.
    """
    c = np.asarray(counter, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    shape = np.broadcast_shapes(c.shape[:-1], k.shape[:-1])
    c = np.broadcast_to(c, shape + (4,))
    k = np.broadcast_to(k, shape + (2,))
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_W0)) & np.uint64(_MASK)
            k1 = (k1 + np.uint64(_W1)) & np.uint64(_MASK)
        p0 = np.uint64(_M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def gumbel_uniforms(seed: int, row_ids: np.ndarray, V: int) -> np.ndarray:
    """u[t, v] in (0, 1), float64, for rows with the given ids (see the
    module docstring for the counter and key layout)."""
    ids = np.asarray(row_ids, dtype=np.uint64)
    n = ids.shape[0]
    nq = (V + 3) // 4
    ctr = np.zeros((n, nq, 4), dtype=np.uint64)
    ctr[:, :, 0] = np.arange(nq, dtype=np.uint64)[None, :]
    ctr[:, :, 1] = (ids & np.uint64(_MASK))[:, None]
    ctr[:, :, 2] = (ids >> np.uint64(32))[:, None]
    seed = int(seed)
    key = np.array([seed & _MASK, (seed >> 32) & _MASK], dtype=np.uint64)
    x = philox4x32_10(ctr, key).reshape(n, nq * 4)[:, :V].astype(np.float64)
    return (x + 0.5) / 2.0 ** 32


def sample_tokens(hidden: np.ndarray, lm_head: np.ndarray, row_ids: np.ndarray,
                  seed: int, row_chunk: int = 256):
    """Gumbel-max draw per row and its recorded logprob.

    Returns (tokens int64 [n], logmu float64 [n], score_gap float64 [n]);
    score_gap is the distance between the best and second-best z + g of the
    row, the margin by which a lower-precision evaluation could pick
    another token.
    """
    hidden = np.asarray(hidden, np.float64)
    lm_head = np.asarray(lm_head, np.float64)
    ids = np.asarray(row_ids)
    n, V = hidden.shape[0], lm_head.shape[0]
    tokens = np.zeros(n, dtype=np.int64)
    logmu = np.zeros(n, dtype=np.float64)
    gap = np.zeros(n, dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        z = lm_head_logits(hidden[r0:r1], lm_head)
        g = -np.log(-np.log(gumbel_uniforms(seed, ids[r0:r1], V)))
        score = z + g
        a = np.argmax(score, axis=1)          # first maximum: smallest v
        tokens[r0:r1] = a
        _, lp = log_softmax_rows(z)
        logmu[r0:r1] = lp[np.arange(r1 - r0), a]
        top2 = np.sort(score, axis=1)[:, -2:]
        gap[r0:r1] = top2[:, 1] - top2[:, 0]
    return tokens, logmu, gap
