"""The rollout-side draw (rz_sample_tokens) on the GPU against the float64
oracle, and the property the pages turn on ("diff 0"): the recorded logprob
is bit-identical to the learner's rz_token_logprobs of the same token at the
same weights, whatever batch either call runs in.

Tokens are compared with the oracle's exact argmax of z + g.  The GPU takes
that argmax in fp32 (logits from the MFMA GEMM, noise from fp32 logs), so it
may pick another token only where the oracle's best and second-best scores
are closer than the fp32 error of a score; such rows must have an oracle gap
below GAP_TOL and the GPU's pick must score within GAP_TOL of the best.
GAP_TOL = 1e-3 covers logits of magnitude < 30 at fp32 (relative 1e-5 after
the K-sum) plus the noise's ~1e-6, with a wide margin.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import (TOL, assert_close, host, mat_to_dev, say, small_batch,
                      torch_mod, vec_to_dev)
from invariant_token_logprobs_amd import synth

pytestmark = pytest.mark.gpu

GAP_TOL = 1e-3
SEED = 0x1234_5678_9ABC  # uses both 32-bit words of the key


def _ids(n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 62, size=n, dtype=np.int64)


def _run(hidden, W, ids, seed, **kw):
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    out = rz.sample_tokens(hidden, W, vec_to_dev(ids), seed, want_lse=True, **kw)
    torch.cuda.synchronize()
    return [host(t) for t in out]


def _check_tokens(tok_gpu, hidden64, W64, ids, seed, what):
    tok_o, logmu_o, gap = O.sample_tokens(hidden64, W64, ids, seed)
    diff = np.flatnonzero(tok_gpu != tok_o)
    if diff.size:
        u = O.gumbel_uniforms(seed, ids[diff], W64.shape[0])
        z = hidden64[diff] @ W64.T
        score = z - np.log(-np.log(u))
        best = score.max(axis=1)
        mine = score[np.arange(diff.size), tok_gpu[diff]]
        assert np.all(gap[diff] < GAP_TOL), (what, diff, gap[diff])
        assert np.all(best - mine < GAP_TOL), (what, diff, best - mine)
    assert diff.size <= max(1, tok_gpu.size // 100), (what, diff.size)
    return tok_o, logmu_o


def _diff0(hidden, W, tokens, logmu, lse, what):
    """logmu and lse equal rz_token_logprobs of the drawn tokens, bit for bit."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    lp, lse2 = rz.token_logprobs(hidden, W, vec_to_dev(tokens.astype(np.int32)),
                                 want_lse=True)
    torch.cuda.synchronize()
    lp, lse2 = host(lp), host(lse2)
    assert np.array_equal(lp.view(np.uint32), logmu.view(np.uint32)), what
    assert np.array_equal(lse2.view(np.uint32), lse.view(np.uint32)), what


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampler_parity_and_diff0(dtype):
    b = small_batch(N_resp=3, group_size=3, H=256, V=1000, lo=80, hi=140,
                    dtype=dtype, seed=21)
    say("sampler parity", dtype, "rows", b.N)
    hidden = mat_to_dev(b.hidden, dtype)
    W = mat_to_dev(b.lm_head, dtype)
    ids = _ids(b.N, 5)
    tok, logmu, lse = _run(hidden, W, ids, SEED)
    h64, W64 = O.to_f64(b.hidden, dtype), O.to_f64(b.lm_head, dtype)
    assert tok.min() >= 0 and tok.max() < b.V
    _check_tokens(tok.astype(np.int64), h64, W64, ids, SEED, f"sampler-{dtype}")
    # the record against the oracle's log pi of the drawn token
    logpi_o, lse_o = O.token_logprobs(h64, W64, tok)
    t = TOL[dtype]
    assert_close(logmu, logpi_o, t["rtol"], t["atol"], f"sampler-{dtype} logmu")
    assert_close(lse, lse_o, t["rtol"], t["atol"], f"sampler-{dtype} lse")
    _diff0(hidden, W, tok, logmu, lse, f"sampler-{dtype} diff0")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_batches_match_the_large_batch(dtype):
    """Up to 64 rows the forward runs the single-stage 64-row tile, up to 192
    rows (draw) or 128 rows (logits) the two-stage 64-row tile, and beyond that
    the 256-row tile; up to 256 rows the tile partials are stored row-major,
    beyond that tile-major.  The first 1, 37, 64, 65, 192, 193 and 256 rows
    of a batch, drawn and scored alone, give the same tokens, records and
    log-sum-exps, bit for bit, as they do inside the whole batch."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    b = small_batch(N_resp=3, group_size=3, H=256, V=1000, lo=100, hi=140,
                    dtype=dtype, seed=23)
    assert b.N > 256
    say("small batches vs large", dtype, "rows", b.N)
    hidden = mat_to_dev(b.hidden, dtype)
    W = mat_to_dev(b.lm_head, dtype)
    ids = _ids(b.N, 9)
    tok, logmu, lse = _run(hidden, W, ids, SEED)
    lp_all, lse_all = rz.token_logprobs(hidden, W, vec_to_dev(b.tokens), want_lse=True)
    torch.cuda.synchronize()
    lp_all, lse_all = host(lp_all), host(lse_all)
    bits = lambda x: np.asarray(x, np.float32).view(np.uint32)
    for n in (1, 37, 64, 65, 192, 193, 256):
        what = f"{dtype} first {n} rows"
        t_n, m_n, l_n = _run(hidden[:n].contiguous(), W, ids[:n], SEED)
        assert np.array_equal(t_n, tok[:n]), what
        assert np.array_equal(bits(m_n), bits(logmu[:n])), what
        assert np.array_equal(bits(l_n), bits(lse[:n])), what
        lp, ls = rz.token_logprobs(hidden[:n].contiguous(), W, vec_to_dev(b.tokens[:n]),
                                   want_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(lp)), bits(lp_all[:n])), what
        assert np.array_equal(bits(host(ls)), bits(lse_all[:n])), what


def test_sampler_frequencies_follow_softmax():
    """60000 draws from one hidden state over V = 24 (fp32): chi-square of
    the counts against the oracle's float64 softmax, 23 degrees of freedom
    (60 is past the 0.01% point)."""
    torch = torch_mod()
    rng = np.random.default_rng(8)
    H, V, n = 64, 24, 60000
    h = rng.normal(size=(1, H)).astype(np.float32)
    W = (rng.normal(size=(V, H)) * 0.2).astype(np.float32)
    hidden = mat_to_dev(np.repeat(h, n, axis=0), "f32")
    tok, logmu, lse = _run(hidden, mat_to_dev(W, "f32"), np.arange(n, dtype=np.int64), 77)
    z = h.astype(np.float64) @ W.astype(np.float64).T
    p = np.exp(z[0] - z.max())
    p /= p.sum()
    counts = np.bincount(tok, minlength=V)
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    say("sampler chi2", round(chi2, 2))
    assert chi2 < 60.0, (chi2, counts, n * p)
    del hidden
    torch.cuda.empty_cache()


def _split_vocabs(ncu):
    """Vocabulary sizes that take each branch of the single-stage 64-row
    form's column split on a device with ncu CUs: all 128-column workgroups
    (few statistics tiles), whole rounds of 256-column workgroups plus at most
    one 128-column workgroup per CU, and whole rounds plus further 256-column
    workgroups (an odd tile count, V not a multiple of 128)."""
    return [1000, 128 * (2 * ncu + ncu // 2), 128 * (3 * ncu + 37) - 50, 151936]


@pytest.mark.parametrize("which", range(4))
def test_column_splits_match_the_large_batch(which):
    """At up to 64 rows the forward takes 256- and 128-column workgroups by
    the head's width and the CU count; at 300 rows it takes the 256-row tile.
    For a vocabulary in each branch of that split, the first 64 and 37 rows
    give the same tokens, records, log-sum-exps and logprobs, bit for bit, as
    inside the 300-row batch, and four rows match the oracle."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    V = _split_vocabs(ncu)[which]
    H, N = 128, 300
    say("column split", which, "V", V, "CUs", ncu)
    hb, tok = synth.random_rows(N, H, V, "bf16", 1201 + which)
    W_np = synth.random_lm_head(V, H, "bf16", 1301 + which, scale=0.3)
    hidden, W = mat_to_dev(hb, "bf16"), mat_to_dev(W_np, "bf16")
    ids = _ids(N, 1401 + which)
    t_all, m_all, l_all = _run(hidden, W, ids, SEED)
    lp_all, ls_all = rz.token_logprobs(hidden, W, vec_to_dev(tok), want_lse=True)
    torch.cuda.synchronize()
    lp_all, ls_all = host(lp_all), host(ls_all)
    bits = lambda x: np.asarray(x, np.float32).view(np.uint32)
    for n in (64, 37):
        what = f"V={V} first {n} rows"
        t_n, m_n, l_n = _run(hidden[:n].contiguous(), W, ids[:n], SEED)
        assert np.array_equal(t_n, t_all[:n]), what
        assert np.array_equal(bits(m_n), bits(m_all[:n])), what
        assert np.array_equal(bits(l_n), bits(l_all[:n])), what
        lp, ls = rz.token_logprobs(hidden[:n].contiguous(), W, vec_to_dev(tok[:n]),
                                   want_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(lp)), bits(lp_all[:n])), what
        assert np.array_equal(bits(host(ls)), bits(ls_all[:n])), what
    h64, W64 = O.to_f64(hb[:4], "bf16"), O.to_f64(W_np, "bf16")
    _check_tokens(t_all[:4].astype(np.int64), h64, W64, ids[:4], SEED, f"V={V}")
    logpi_o, _ = O.token_logprobs(h64, W64, tok[:4])
    t = TOL["bf16"]
    assert_close(lp_all[:4], logpi_o, t["rtol"], t["atol"], f"V={V} logprobs")
    del hidden, W
    torch.cuda.empty_cache()


def test_sampler_batch_invariance_qwen3_4b_head():
    """The same 64 reference rows (fixed ids) drawn inside batches of
    1 .. 1100 rows at random slots, at the Qwen3-4B head shape: tokens,
    records and lse are bit-identical in every batch, and the records are
    the learner's rz_token_logprobs of the drawn tokens."""
    torch = torch_mod()
    H, V = 2560, 151936
    rng = np.random.default_rng(17)
    ref_h, _ = synth.random_rows(64, H, V, "bf16", 901)
    W_np = synth.random_lm_head(V, H, "bf16", 902)
    W = mat_to_dev(W_np, "bf16")
    ref_ids = _ids(64, 903)
    ref_tok = ref_lmu = ref_lse = None
    for n in (64, 1, 7, 300, 1024, 1100):
        if n < 64:
            sel = rng.choice(64, size=n, replace=False)
            hb, ib, slots = ref_h[sel], ref_ids[sel], np.arange(n)
        else:
            filler, _ = synth.random_rows(n - 64, H, V, "bf16", 904 + n)
            slots = np.sort(rng.choice(n, size=64, replace=False))
            hb = np.empty((n, H), dtype=ref_h.dtype)
            ib = _ids(n, 905 + n)
            rest = np.setdiff1d(np.arange(n), slots)
            hb[rest] = filler
            hb[slots] = ref_h
            ib[slots] = ref_ids
            sel = np.arange(64)
        say("sampler invariance batch", n)
        hidden = mat_to_dev(hb, "bf16")
        tok, lmu, lse = _run(hidden, W, ib, SEED)
        if ref_tok is None:
            ref_tok, ref_lmu, ref_lse = tok[slots], lmu[slots], lse[slots]
            _diff0(hidden, W, tok, lmu, lse, "qwen3_4b diff0")
        else:
            assert np.array_equal(tok[slots], ref_tok[sel]), n
            assert np.array_equal(lmu[slots].view(np.uint32), ref_lmu[sel].view(np.uint32)), n
            assert np.array_equal(lse[slots].view(np.uint32), ref_lse[sel].view(np.uint32)), n
        del hidden
    # four reference rows against the oracle at the full vocabulary
    h64 = O.to_f64(ref_h[:4], "bf16")
    W64 = O.to_f64(W_np, "bf16")
    _check_tokens(ref_tok[:4].astype(np.int64), h64, W64, ref_ids[:4], SEED, "qwen3_4b")
    logpi_o, _ = O.token_logprobs(h64, W64, ref_tok[:4])
    t = TOL["bf16"]
    assert_close(ref_lmu[:4], logpi_o, t["rtol"], t["atol"], "qwen3_4b logmu")
    del W
    torch.cuda.empty_cache()


def test_sampler_seed_and_id_select_the_draw():
    b = small_batch(N_resp=2, group_size=2, H=128, V=700, lo=60, hi=60,
                    dtype="bf16", seed=33)
    hidden = mat_to_dev(b.hidden, "bf16")
    W = mat_to_dev(b.lm_head, "bf16")
    ids = _ids(b.N, 9)
    t1, _, _ = _run(hidden, W, ids, 1)
    t2, _, _ = _run(hidden, W, ids, 1)
    t3, _, _ = _run(hidden, W, ids, 2)
    t4, _, _ = _run(hidden, W, ids + 1, 1)
    assert np.array_equal(t1, t2)
    assert (t1 != t3).mean() > 0.5 and (t1 != t4).mean() > 0.5
