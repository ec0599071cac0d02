"""The release-precision head on the GPU: rz_dequantize_head against the
float64 oracle (oracle/mx_head.py), bit for bit, and the logprob path run
on its output against the oracle's token_logprobs_mx.

Dequantization is exact by construction (every valid value is a bfloat16
number), so the bf16 head must equal the oracle's float64 decode exactly,
signed zeros included, with NaN exactly where the oracle has NaN.  The
logprobs then carry the bf16 head's tolerance (rtol 2e-3, atol 1e-4), and
rollout records on the dequantized head equal learner logprobs bit for bit.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import TOL, assert_close, host, mat_to_dev, say, torch_mod, vec_to_dev
from invariant_token_logprobs_amd import synth

pytestmark = pytest.mark.gpu


def _dequant(codes, scales, fmt, err=None):
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    W = rz.dequantize_head(vec_to_dev(codes), vec_to_dev(scales), fmt, err_flag=err)
    torch.cuda.synchronize()
    return W


def _bf16_to_f64(W):
    torch = torch_mod()
    return W.to(torch.float64).cpu().numpy()


def _assert_exact(got, want, what):
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w), (what, np.argwhere(nan_g != nan_w)[:5])
    ok = ~nan_w
    assert np.array_equal(got[ok], want[ok]), what
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok])), what


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_dequantize_every_code_at_every_scale(fmt):
    """Row r has scale code r (0 .. 255, the invalid ones included) and holds
    every element code of the format; a NaN-free head leaves the flag clear."""
    torch = torch_mod()
    if fmt == "mxfp4":
        H = 64
        elem = np.tile(np.arange(16, dtype=np.uint8), (256, H // 16))
        codes = (elem[:, 0::2] | (elem[:, 1::2] << 4)).astype(np.uint8)
    else:
        H = 256
        codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], H // 32, axis=1)
    say("dequant exhaustive", fmt)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    W = _dequant(codes, scales, fmt, err)
    _assert_exact(_bf16_to_f64(W), O.dequantize_head(codes, scales, fmt), fmt)
    assert int(host(err)[0]) == 8
    lo, hi = O.scale_range(fmt)
    valid = np.arange(127 + lo, 127 + hi + 1)
    err.zero_()
    W = _dequant(codes[valid], scales[valid], fmt, err)
    _assert_exact(_bf16_to_f64(W), O.dequantize_head(codes[valid], scales[valid], fmt),
                  fmt + " valid rows")
    assert int(host(err)[0]) == 0


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_head_logprobs_and_diff0(fmt):
    """A random MX head (V = 1000: three full vocab tiles and a ragged one),
    300 rows: the dequantized head is the oracle's exactly, the logprobs
    match token_logprobs_mx, and the rollout draw on it records exactly the
    learner's logprobs."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    V, H, n = 1000, 256, 300
    codes, scales = synth.random_mx_head(V, H, fmt, 41)
    hid, tok = synth.random_rows(n, H, V, "bf16", 42)
    say("mx head parity", fmt)
    W = _dequant(codes, scales, fmt)
    W64 = O.dequantize_head(codes, scales, fmt)
    _assert_exact(_bf16_to_f64(W), W64, fmt)
    hidden = mat_to_dev(hid, "bf16")
    lp, lse = rz.token_logprobs(hidden, W, vec_to_dev(tok), want_lse=True)
    want_lp, want_lse = O.token_logprobs_mx(O.to_f64(hid, "bf16"), codes, scales,
                                            fmt, tok)
    t = TOL["bf16"]
    assert_close(host(lp), want_lp, t["rtol"], t["atol"], f"{fmt} logprobs")
    assert_close(host(lse), want_lse, t["rtol"], t["atol"], f"{fmt} lse")
    ids = vec_to_dev(np.arange(n, dtype=np.int64) * 7919)
    tokens, logmu = rz.sample_tokens(hidden, W, ids, 0xABCDEF)
    lp2 = rz.token_logprobs(hidden, W, tokens)
    torch.cuda.synchronize()
    assert np.array_equal(host(logmu).view(np.uint32), host(lp2).view(np.uint32))


def test_mx_qwen3_4b_head_mxfp4():
    """The Qwen3-4B head shape [151936, 2560] in MXFP4: 512 sampled rows of
    the dequantized head equal the oracle's decode exactly; 48 rows'
    logprobs over the full vocabulary match the oracle."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    V, H = 151936, 2560
    codes, scales = synth.random_mx_head(V, H, "mxfp4", 77)
    say("mx qwen3-4b head: dequant")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    W = _dequant(codes, scales, "mxfp4", err)
    assert int(host(err)[0]) == 0
    rows = np.sort(np.random.default_rng(78).choice(V, size=512, replace=False))
    rows[-1] = V - 1
    got = W[torch.from_numpy(rows).to("cuda:0")].to(torch.float64).cpu().numpy()
    _assert_exact(got, O.dequantize_head(codes[rows], scales[rows], "mxfp4"), "rows")
    say("mx qwen3-4b head: logprobs")
    hid, tok = synth.random_rows(48, H, V, "bf16", 79)
    lp = rz.token_logprobs(mat_to_dev(hid, "bf16"), W, vec_to_dev(tok))
    torch.cuda.synchronize()
    want, _ = O.token_logprobs_mx(O.to_f64(hid, "bf16"), codes, scales, "mxfp4", tok)
    t = TOL["bf16"]
    assert_close(host(lp), want, t["rtol"], t["atol"], "qwen3-4b mxfp4 logprobs")
    del W
    torch.cuda.empty_cache()


def _same_bits(a, b):
    a, b = host(a), host(b)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("n,H", [(1, 256), (64, 256), (200, 256), (300, 256), (40, 192)])
def test_mx_entry_points_equal_the_expanded_head(fmt, n, H):
    """rz_token_logprobs_mx / rz_sample_tokens_mx against the bf16 calls on
    rz_dequantize_head's output, bit for bit: the codes read by the 64-row
    tile (n <= 128 / 256, H % 128 == 0) and the expansion path (the rest)."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    V = 1000
    codes, scales = synth.random_mx_head(V, H, fmt, 51 + n + H)
    hid, tok = synth.random_rows(n, H, V, "bf16", 52 + n)
    say("mx entry points", fmt, n, H)
    cd, sd = vec_to_dev(codes), vec_to_dev(scales)
    hidden = mat_to_dev(hid, "bf16")
    W = rz.dequantize_head(cd, sd, fmt)
    tokens = vec_to_dev(tok)
    lp, lse = rz.token_logprobs_mx(hidden, cd, sd, fmt, tokens, want_lse=True)
    lp2, lse2 = rz.token_logprobs(hidden, W, tokens, want_lse=True)
    ids = vec_to_dev(np.arange(n, dtype=np.int64) * 31 + 7)
    t1, m1, l1 = rz.sample_tokens_mx(hidden, cd, sd, fmt, ids, 0xFEED, want_lse=True)
    t2, m2, l2 = rz.sample_tokens(hidden, W, ids, 0xFEED, want_lse=True)
    torch.cuda.synchronize()
    assert _same_bits(lp, lp2) and _same_bits(lse, lse2)
    assert torch.equal(t1, t2) and _same_bits(m1, m2) and _same_bits(l1, l2)
    # and the record is the learner's logprob of the drawn token (diff 0)
    assert _same_bits(m1, rz.token_logprobs_mx(hidden, cd, sd, fmt, t1))


@pytest.mark.parametrize("which", range(3))
def test_mx_head_equals_the_split_bf16_tile(which):
    """An MXFP4 head at the vocabularies that take each branch of the bf16
    tile's column split (few statistics tiles; whole rounds of 256-column
    workgroups plus at most one 128-column one per CU; further 256-column
    ones, V not a multiple of 128), whose bf16 calls run split while the MX
    tile runs whole 256-column tiles: at 64 and 37 rows the logprobs, lse and
    draws equal the bf16 calls on the expanded head bit for bit."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    V = [1000, 128 * (2 * ncu + ncu // 2), 128 * (3 * ncu + 37) - 50][which]
    H = 128
    codes, scales = synth.random_mx_head(V, H, "mxfp4", 91 + which)
    cd, sd = vec_to_dev(codes), vec_to_dev(scales)
    W = rz.dequantize_head(cd, sd, "mxfp4")
    for n in (64, 37):
        say("mx column split", which, "V", V, "rows", n)
        hid, tok = synth.random_rows(n, H, V, "bf16", 93 + n + which)
        hidden, tokens = mat_to_dev(hid, "bf16"), vec_to_dev(tok)
        lp, lse = rz.token_logprobs_mx(hidden, cd, sd, "mxfp4", tokens, want_lse=True)
        lp2, lse2 = rz.token_logprobs(hidden, W, tokens, want_lse=True)
        ids = vec_to_dev(np.arange(n, dtype=np.int64) * 17 + which)
        t1, m1, l1 = rz.sample_tokens_mx(hidden, cd, sd, "mxfp4", ids, 0xBEEF, want_lse=True)
        t2, m2, l2 = rz.sample_tokens(hidden, W, ids, 0xBEEF, want_lse=True)
        torch.cuda.synchronize()
        assert _same_bits(lp, lp2) and _same_bits(lse, lse2), (V, n)
        assert torch.equal(t1, t2) and _same_bits(m1, m2) and _same_bits(l1, l2), (V, n)
    del W
    torch.cuda.empty_cache()


def test_mx_entry_points_invalid_scale():
    """A NaN scale code in the head: the same NaNs as the expanded head's,
    and the device flag."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    V, H, n = 600, 256, 48
    codes, scales = synth.random_mx_head(V, H, "mxfp4", 61)
    scales[5, 2] = 255
    hid, tok = synth.random_rows(n, H, V, "bf16", 62)
    cd, sd = vec_to_dev(codes), vec_to_dev(scales)
    hidden, tokens = mat_to_dev(hid, "bf16"), vec_to_dev(tok)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    lp = rz.token_logprobs_mx(hidden, cd, sd, "mxfp4", tokens, err_flag=err)
    W = rz.dequantize_head(cd, sd, "mxfp4")
    lp2 = rz.token_logprobs(hidden, W, tokens)
    torch.cuda.synchronize()
    assert int(host(err)[0]) & 8
    assert np.array_equal(np.isnan(host(lp)), np.isnan(host(lp2)))
    assert np.isnan(host(lp)).all()          # a NaN logit reaches every lse


def test_mx_qwen3_4b_head_fused_decode():
    """The Qwen3-4B head in MXFP4 at 64 live rows: the fused draw equals the
    draw on the expanded head bit for bit."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    V, H, n = 151936, 2560, 64
    codes, scales = synth.random_mx_head(V, H, "mxfp4", 77)
    hid, _ = synth.random_rows(n, H, V, "bf16", 81)
    cd, sd = vec_to_dev(codes), vec_to_dev(scales)
    hidden = mat_to_dev(hid, "bf16")
    ids = vec_to_dev(np.arange(n, dtype=np.int64))
    say("mx qwen3-4b fused decode")
    t1, m1 = rz.sample_tokens_mx(hidden, cd, sd, "mxfp4", ids, 99)
    W = rz.dequantize_head(cd, sd, "mxfp4")
    t2, m2 = rz.sample_tokens(hidden, W, ids, 99)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2) and _same_bits(m1, m2)
    del W
    torch.cuda.empty_cache()


def test_release_precision_rollout_learner_diff0():
    """Zero mismatch at release precision: the rollout draws on the MXFP4
    Qwen3-4B head with the codes read directly (rz_sample_tokens_mx, 48
    rows), the learner expands the head once and runs its step on the same
    rows (rz_reinforce_zero_fwd_bwd): the learner's log pi equals the
    recorded log mu bit for bit on every row, so w = 1, D3 = KL = 0."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    V, H, n = 151936, 2560, 48
    codes, scales = synth.random_mx_head(V, H, "mxfp4", 83)
    hid, _ = synth.random_rows(n, H, V, "bf16", 84)
    cd, sd = vec_to_dev(codes), vec_to_dev(scales)
    hidden = mat_to_dev(hid, "bf16")
    ids = vec_to_dev(np.arange(n, dtype=np.int64) + 1000)
    say("release precision: rollout draw")
    tokens, logmu = rz.sample_tokens_mx(hidden, cd, sd, "mxfp4", ids, 2026)
    say("release precision: learner step")
    W = rz.dequantize_head(cd, sd, "mxfp4")
    dev = "cuda:0"
    out = rz.reinforce_zero_fwd_bwd(
        hidden, W, tokens, logmu, torch.ones(n, dtype=torch.uint8, device=dev),
        torch.tensor([0, 20, 48], dtype=torch.int32, device=dev),
        torch.tensor([1.0, 0.0], dtype=torch.float32, device=dev),
        torch.zeros(2, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert _same_bits(out["logprobs"], logmu)
    d = host(out["diag"])
    assert d[0] == 0.0 and d[1] == 0.0
    del W
    torch.cuda.empty_cache()
