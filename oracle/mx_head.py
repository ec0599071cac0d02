"""Float64 CPU oracle of the release-precision LM head: weights stored in the
OCP microscaling (MX) formats, MXFP4 (E2M1 elements) or MXFP8 (E4M3
elements), each block of 32 consecutive values along H sharing one E8M0
scale.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: imported by the tests
and never by the product path; it shares no code with the HIP kernels.

Sources:

* [P2] "Zero mismatch, simple async RL: REINFORCE Zero, DeepSeek-V4.1 and
  Kimi K3.1" (vLLM blog), the "Support for Flagship Models" list and the
  DeepSeek-V4.1-Flash section: the aligned path keeps release precision,
  FP8 and MXFP4 weights included, with zero mismatch between rollout and
  trainer.
* The element and scale encodings are those of the OCP Microscaling Formats
  (MX) v1.0 specification: E2M1 (1 sign, 2 exponent bits with bias 1, 1
  mantissa bit; no inf or NaN; largest 6), E4M3 (1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits; no inf; S.1111.111 is NaN; largest 448) and E8M0
  (an unsigned exponent with bias 127, the value 2^(code - 127); code 255 is
  NaN).  An element's value is its decoded value times its block's scale.

Readings (the pages name the formats only):

* Only the head's weights W [V, H] are in an MX format; the hidden states
  keep their own precision and the logits are z = h dequant(W)^T, followed by
  the same log-softmax and gather as the bf16 head (token_logprobs).
* Storage: E4M3 codes one per byte, [V, H]; E2M1 codes two per byte,
  [V, H / 2], element 2j in the low nibble and 2j + 1 in the high nibble of
  byte j; scales [V, H / 32] E8M0 bytes, block b of row v covering
  W[v, 32 b : 32 b + 32].
* Every dequantized value must be exactly a bfloat16 number, so that the
  dequantized head is the bf16 head the rest of the path runs on, bit for
  bit.  With scale 2^s that holds for every E2M1 value when s <= 125 and for
  every E4M3 value when -124 <= s <= 119 (bf16 has 8 significant bits,
  exponents down to its smallest subnormal 2^-133 and up to 2^127).  A block
  whose scale is outside that range, or is the NaN code, is invalid: all its
  values are NaN.  An E4M3 NaN code is a NaN value.

Parity status: the decoders are pinned by the specification's listed values
and by torch's float8_e4m3fn and float8_e8m0fnu decoders over all 256 codes;
dequantize_head by hand blocks, the block-to-scale map and the exactness
claim above (tests/test_oracle_pins.py).
"""

from __future__ import annotations

import numpy as np

from .reinforce_zero import token_logprobs

__all__ = ["MX_BLOCK", "decode_e2m1", "decode_e4m3", "decode_e8m0",
           "unpack_fp4", "scale_range", "dequantize_head",
           "token_logprobs_mx"]

MX_BLOCK = 32


def decode_e2m1(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64: normal (1 + m/2) 2^(e - 1) for e > 0,
    subnormal (m/2) 2^0 for e = 0."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e > 0, (1.0 + m / 2.0) * np.exp2(e - 1.0), (m / 2.0))
    return s * mag


def decode_e4m3(codes) -> np.ndarray:
    """E4M3 codes (0..255) -> float64: normal (1 + m/8) 2^(e - 7) for e > 0,
    subnormal (m/8) 2^-6 for e = 0; S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0, (1.0 + m / 8.0) * np.exp2(e - 7.0),
                   (m / 8.0) * 2.0 ** -6)
    out = s * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 codes -> 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def unpack_fp4(packed) -> np.ndarray:
    """[V, H/2] bytes -> [V, H] E2M1 codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def scale_range(fmt: str):
    """(lowest, highest) scale exponent s for which every value of the
    element format times 2^s is a bfloat16 number (see the readings)."""
    return {"mxfp4": (-127, 125), "mxfp8": (-124, 119)}[fmt]


def dequantize_head(codes, scales, fmt: str) -> np.ndarray:
    """float64 W [V, H] from MX storage.  codes: [V, H/2] packed E2M1 bytes
    (fmt "mxfp4") or [V, H] E4M3 bytes (fmt "mxfp8"); scales: [V, H/32]
    E8M0 bytes."""
    if fmt == "mxfp4":
        vals = decode_e2m1(unpack_fp4(codes))
    elif fmt == "mxfp8":
        vals = decode_e4m3(codes)
    else:
        raise ValueError(f"unknown MX format {fmt!r}")
    V, H = vals.shape
    sc = np.asarray(scales, dtype=np.int64)
    assert sc.shape == (V, H // MX_BLOCK), (sc.shape, V, H)
    lo, hi = scale_range(fmt)
    s = sc - 127
    block_ok = (sc != 255) & (s >= lo) & (s <= hi)
    factor = np.where(block_ok, decode_e8m0(sc), np.nan)
    return vals * np.repeat(factor, MX_BLOCK, axis=1)


def token_logprobs_mx(hidden, codes, scales, fmt: str, tokens):
    """(log pi of tokens, lse) with the head dequantized first; the same
    definition as token_logprobs over dequantize_head(codes, scales, fmt)."""
    return token_logprobs(np.asarray(hidden, np.float64),
                          dequantize_head(codes, scales, fmt), tokens)
