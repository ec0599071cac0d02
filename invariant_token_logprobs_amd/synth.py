"""Seeded synthetic inputs shaped like the workloads the REINFORCE Zero pages train on.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic.  Both the GPU path and the float64 oracle consume the
same host arrays it returns, so they see bit-identical inputs.

Recipe (no page measures on data that is available here, so these stand in for
the reasoning / tool-use / agentic rollouts the pages describe):

* hidden states ~ N(0, 1) and LM-head weights ~ N(0, 0.02^2), drawn in
  float32 with NumPy's PCG64 and, for bf16 workloads, rounded to bfloat16 by
  round-to-nearest-even (returned as uint16 bit patterns);
* sampled tokens uniform on [0, V);
* response i belongs to group floor(i / group_size);
* rewards Bernoulli(1/2) in {0, 1}, or U[0, 1] for the tool-use workload;
* behaviour logprobs log mu = float32(log pi + sigma * N(0, 1)), where log pi
  is supplied by the caller and sigma stands for the policy lag (0.02 at lag 2,
  0.1 at lag 64);
* seeds: workload k draws its data from seed 1000 + k and its behaviour-logprob
  noise from seed 2000 + k.

Harder inputs for the method's edges (the pages' runs use real policies, whose
softmax is peaked and whose tokens follow a heavy-tailed law):
* tokens Zipf-distributed over the vocabulary (zipf_tokens: rank k drawn with
  probability proportional to k^-s, the ranks assigned to token ids by a
  seeded permutation);
* a wider head (random_lm_head's scale; 0.3 at H = 2560 gives logits of
  standard deviation about 15);
* hidden rows pulled toward (or away from) their token's head row
  (aligned_rows), which makes that token nearly certain (or nearly
  impossible);
* logits near two large levels by vocabulary half (two_level_logits), so
  that a row's vocabulary tiles have maxima tens of nats apart.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

QWEN_VOCAB = 151936


@dataclass
class Workload:
    name: str
    H: int
    V: int
    dtype: str               # 'f32' or 'bf16' (hidden and LM head)
    n_resp: int
    group_size: int
    len_lo: int
    len_hi: int
    sigma: float             # std of the behaviour-logprob noise
    rewards: str             # 'bernoulli' or 'uniform'
    masked_frac: float = 0.0  # share of masked (tool) rows
    long_tail: float = 0.0    # share of responses pinned at len_hi
    index: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 256, 1024, "f32", 8, 4, 8, 64, 0.05, "bernoulli",
                     index=0),
    "r1_distill_1p5b": Workload("r1_distill_1p5b", 1536, QWEN_VOCAB, "bf16", 64,
                                8, 512, 8192, 0.02, "bernoulli", index=1),
    "qwen3_4b_tool": Workload("qwen3_4b_tool", 2560, QWEN_VOCAB, "bf16", 32, 8,
                              1024, 16384, 0.1, "uniform", masked_frac=0.40,
                              index=2),
    "qwen3_30b_a3b": Workload("qwen3_30b_a3b", 2048, QWEN_VOCAB, "bf16", 128,
                              8, 256, 8192, 0.02, "bernoulli", long_tail=0.10,
                              index=3),
}


@dataclass
class Batch:
    name: str
    dtype: str
    H: int
    V: int
    hidden: np.ndarray        # [N, H] float32 or uint16 (bf16 bits)
    lm_head: np.ndarray       # [V, H] float32 or uint16 (bf16 bits)
    tokens: np.ndarray        # [N] int32
    mask: np.ndarray          # [N] uint8, 1 = valid action token
    cu_rows: np.ndarray       # [B + 1] int32
    rewards: np.ndarray       # [B] float32
    group_ids: np.ndarray     # [B] int32
    sigma: float
    noise_seed: int
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def B(self) -> int:
        return int(self.rewards.shape[0])

    @property
    def n_valid(self) -> int:
        return int(np.count_nonzero(self.mask))


# ------------------------------------------------------------------ helpers
def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, scale: float, dtype: str,
            chunk_rows: int = 1 << 14) -> np.ndarray:
    """N(0, scale^2) in float32, rounded to bf16 bits when dtype == 'bf16'."""
    rows, cols = shape
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        out[r0:r1] = round_bf16(blk) if dtype == "bf16" else blk
    return out


def _span_mask(rng: np.random.Generator, lengths, frac: float) -> np.ndarray:
    """Alternating valid / masked spans per response, first row valid.

    Valid spans are U{16..512} rows; masked spans are U{16..512} scaled by a
    factor found by bisection so that the whole batch is `frac` masked.
    """
    draws = []
    for L in lengths:
        k = max(2, 2 * (int(L) // 16 + 2))
        draws.append((rng.integers(16, 513, size=k), rng.integers(16, 513, size=k)))

    def build(ratio):
        parts = []
        for L, (vd, md) in zip(lengths, draws):
            m = np.zeros(int(L), dtype=np.uint8)
            pos, j = 0, 0
            while pos < L:
                v = int(vd[j % len(vd)])
                m[pos:pos + v] = 1
                pos += v
                mk = max(1, int(round(md[j % len(md)] * ratio)))
                pos += mk
                j += 1
            parts.append(m)
        return np.concatenate(parts)

    lo, hi = 0.0, 8.0
    mask = build(1.0)
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        mask = build(mid)
        f = 1.0 - mask.mean()
        if abs(f - frac) < 0.002:
            break
        if f < frac:
            lo = mid
        else:
            hi = mid
    return mask


def workload_layout(name: str):
    """Response lengths, mask, rewards and group ids of the named workload
    (the small arrays; draws in a fixed order from seed 1000 + k)."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(np.random.PCG64(1000 + wl.index))
    B = wl.n_resp
    lengths = rng.integers(wl.len_lo, wl.len_hi + 1, size=B)
    if wl.long_tail > 0:
        n_long = int(round(wl.long_tail * B))
        lengths[rng.choice(B, size=n_long, replace=False)] = wl.len_hi
    if wl.masked_frac > 0:
        mask = _span_mask(rng, lengths, wl.masked_frac)
    else:
        mask = np.ones(int(lengths.sum()), dtype=np.uint8)
    if wl.rewards == "bernoulli":
        rewards = rng.integers(0, 2, size=B).astype(np.float32)
    else:
        rewards = rng.random(B, dtype=np.float32)
    group_ids = (np.arange(B) // wl.group_size).astype(np.int32)
    return rng, lengths, mask, rewards, group_ids


def make_workload(name: str, *, max_responses: Optional[int] = None,
                  max_valid: Optional[int] = None,
                  max_rows_per_response: Optional[int] = None,
                  tokens: str = "uniform") -> Batch:
    """Draw the named workload.  Optional caps truncate it for oracle-sized
    checks at the full H and V: max_rows_per_response keeps the first rows
    of every response (their mask as drawn), max_responses the first
    responses, max_valid the rows up to that many valid ones (the last kept
    response may be cut).  tokens = "zipf" replaces the uniform tokens by
    Zipf(1.1) ones (zipf_tokens, seed 3000 + k); the other arrays are
    unchanged."""
    wl = WORKLOADS[name]
    rng, lengths, mask, rewards, group_ids = workload_layout(name)
    B = wl.n_resp
    if max_rows_per_response is not None:
        starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
        lengths = np.minimum(lengths, max_rows_per_response)
        mask = np.concatenate([mask[s0:s0 + L] for s0, L in zip(starts, lengths)])

    # truncate (by responses, then by valid rows) before drawing the big arrays
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    keep_b, keep_n = B, int(cu[-1])
    if max_responses is not None:
        keep_b = min(keep_b, max_responses)
        keep_n = int(cu[keep_b])
    if max_valid is not None:
        csum = np.cumsum(mask[:keep_n].astype(np.int64))
        if csum.size and csum[-1] > max_valid:
            keep_n = int(np.searchsorted(csum, max_valid, side="right"))
            keep_b = int(np.searchsorted(cu, keep_n, side="left"))
            cu = cu.copy()
            cu[keep_b] = keep_n
    cu_rows = cu[: keep_b + 1].astype(np.int32)
    N = keep_n
    mask = mask[:N].copy()
    rewards = rewards[:keep_b].copy()
    group_ids = group_ids[:keep_b].copy()

    toks = rng.integers(0, wl.V, size=N).astype(np.int32)
    hidden = _normal(rng, (N, wl.H), 1.0, wl.dtype)
    lm_head = _normal(rng, (wl.V, wl.H), 0.02, wl.dtype)
    if tokens == "zipf":
        toks = zipf_tokens(N, wl.V, 1.1, 3000 + wl.index)
    elif tokens != "uniform":
        raise ValueError(f"unknown token law {tokens!r}")
    return Batch(name, wl.dtype, wl.H, wl.V, hidden, lm_head, toks, mask,
                 cu_rows, rewards, group_ids, wl.sigma, 2000 + wl.index)


def make_logmu(logpi: np.ndarray, sigma: float, seed: int) -> np.ndarray:
    """Behaviour logprobs: the given log pi plus N(0, sigma^2) lag noise."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    eps = rng.standard_normal(np.asarray(logpi).shape)
    return (np.asarray(logpi, np.float64) + sigma * eps).astype(np.float32)


def random_rows(n: int, H: int, V: int, dtype: str, seed: int):
    """n fresh rows: hidden ~ N(0, 1) and uniform tokens (filler / reference rows)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    tokens = rng.integers(0, V, size=n).astype(np.int32)
    hidden = _normal(rng, (n, H), 1.0, dtype)
    return hidden, tokens


def random_lm_head(V: int, H: int, dtype: str, seed: int,
                   scale: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(np.random.PCG64(seed))
    return _normal(rng, (V, H), scale, dtype)


def zipf_tokens(n: int, V: int, s: float, seed: int) -> np.ndarray:
    """n tokens whose ranks follow a Zipf law truncated to V: rank k (1-based)
    with probability k^-s / sum_j j^-s, drawn by inverse transform from
    PCG64 uniforms; rank k is token perm[k - 1] for a seeded permutation."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    w = np.arange(1, V + 1, dtype=np.float64) ** -s
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    perm = rng.permutation(V)
    ranks = np.searchsorted(cdf, rng.random(n), side="right")
    return perm[np.minimum(ranks, V - 1)].astype(np.int32)


def aligned_rows(lm_head: np.ndarray, tokens: np.ndarray, dtype: str,
                 kappa: np.ndarray, seed: int) -> np.ndarray:
    """Hidden rows kappa_t * W[a_t] + N(0, 1) (rounded to bf16 bits for a
    bf16 head): kappa_t > 0 pulls row t toward its token's head row, < 0
    pushes it away, 0 leaves a plain N(0, 1) row."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    W = (lm_head.astype(np.uint32) << np.uint32(16)).view(np.float32) \
        if dtype == "bf16" else np.asarray(lm_head, np.float32)
    h = rng.standard_normal((len(tokens), W.shape[1]), dtype=np.float32)
    h += np.asarray(kappa, np.float32)[:, None] * W[np.asarray(tokens)]
    return round_bf16(h) if dtype == "bf16" else h


def two_level_logits(n: int, H: int, V: int, levels, beta, seed: int):
    """Hidden rows and a head whose logits sit near two levels by vocabulary
    half: head rows W[v] = a_v u + N(0, 0.02^2) with a_v = levels[0] / H for
    v < V / 2 and levels[1] / H above, hidden rows h_t = beta_t u +
    N(0, 0.1^2), u ~ N(0, 1)^H, so z[t, v] is about beta_t levels[half(v)]
    (|u|^2 is about H).  bf16 bit patterns (hidden, head)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    u = rng.standard_normal(H, dtype=np.float32)
    a = np.where(np.arange(V) < V // 2, levels[0], levels[1]).astype(np.float32) / H
    W = a[:, None] * u[None, :] + 0.02 * rng.standard_normal((V, H), dtype=np.float32)
    h = (np.asarray(beta, np.float32)[:, None] * u[None, :]
         + 0.1 * rng.standard_normal((n, H), dtype=np.float32))
    return round_bf16(h), round_bf16(W)


def random_mx_head(V: int, H: int, fmt: str, seed: int, scale_code: int = 121):
    """A release-precision head in MX storage, drawn directly as codes.

    Element codes: a random sign and a magnitude code drawn with weights
    falling off with the code (small magnitudes most common, as in a head
    quantized from a bell-shaped distribution); E4M3 magnitude codes span
    0x00 .. 0x7E (never the NaN code).  Scales: E8M0 code scale_code +
    {-1, 0, +1} per 32-value block (121 = 2^-6, so values stay near 0.02).
    Returns (codes, scales) as uint8 arrays: codes [V, H/2] packed two per
    byte (low nibble first) for "mxfp4", [V, H] for "mxfp8"; scales
    [V, H/32].
    """
    rng = np.random.default_rng(np.random.PCG64(seed))
    if fmt == "mxfp4":
        p = np.array([4, 4, 3, 3, 2, 2, 1, 1], dtype=np.float64)
        mag = rng.choice(8, size=(V, H), p=p / p.sum()).astype(np.uint8)
        elem = mag | (rng.integers(0, 2, size=(V, H), dtype=np.uint8) << 3)
        codes = (elem[:, 0::2] | (elem[:, 1::2] << 4)).astype(np.uint8)
    elif fmt == "mxfp8":
        # exponent field weighted toward the middle, mantissa uniform
        pe = np.array([1, 1, 2, 3, 4, 5, 6, 6, 5, 3, 1, .5, 0, 0, 0, 0])
        e = rng.choice(16, size=(V, H), p=pe / pe.sum()).astype(np.uint8)
        m = rng.integers(0, 8, size=(V, H), dtype=np.uint8)
        codes = ((e << 3) | m | (rng.integers(0, 2, size=(V, H), dtype=np.uint8) << 7)).astype(np.uint8)
    else:
        raise ValueError(fmt)
    scales = (scale_code + rng.integers(-1, 2, size=(V, H // 32))).astype(np.uint8)
    return codes, scales


def random_lora(r: int, H: int, V: int, dtype: str, seed: int, b_scale: float = 0.05):
    """A LoRA adapter for the head: A [r, H] ~ N(0, 0.02^2) and B [V, r] ~
    N(0, b_scale^2) (non-zero, unlike a fresh adapter, so the adapter's path
    carries weight in the tests), in the head's precision."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    return _normal(rng, (r, H), 0.02, dtype), _normal(rng, (V, r), b_scale, dtype)
