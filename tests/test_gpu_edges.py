"""GPU parity at the method's edges, against the float64 oracle.

The pages train real policies (vLLM blog "Zero mismatch, simple async RL",
section 4 "Learning at lag 64"; "REINFORCE Zero" project page, section 04):
their softmax is peaked, their tokens heavy-tailed, and the importance weight
is used unclipped ("no truncation, no filtering", vLLM blog section 4
"Recipe" item 2).  These cases take each of those to its extreme:

* a head with logits of standard deviation about 15, rows whose token is
  nearly certain (p ~ 1: log pi must come out <= 0, and exactly 0 where the
  other tokens' mass is below fp32 resolution) and rows with log pi far
  below -60;
* log-ratios of +-30 (w ~ 1e13 and 1e-13), and a row past overflow (w = inf
  in both float64 and fp32), where the loss must be the same infinity and
  the gradients non-finite exactly where the oracle's are;
* Zipf(1.1) tokens over more rows than one backward chunk, and a token on
  30% of the rows, for the dW one-hot fix-up.
"""
import math

import numpy as np
import pytest

import oracle as O
from invariant_token_logprobs_amd import synth
import invariant_token_logprobs_amd as rz

from gpu_util import (TOL, assert_close, assert_grad_close, batch_to_dev,
                      compare_full, host, logmu_from_oracle, mat_to_dev,
                      oracle_full, report_grad_error, run_fwd_bwd, say,
                      scalar_tols, small_batch, softmax_grad_bounds, torch_mod,
                      vec_to_dev)

pytestmark = pytest.mark.gpu


def _peaked_batch(dtype, H, V, w_scale, seed, N_resp=6, lo=40, hi=120, kappa=0.5):
    """small_batch's layout with a wide head and one third of the rows pulled
    toward their token (nearly certain), one third pushed away (log pi far
    below -60), one third plain (log pi around -60 at this logit scale)."""
    b = small_batch(N_resp=N_resp, group_size=3, H=H, V=V, lo=lo, hi=hi,
                    dtype=dtype, masked=0.2, seed=seed)
    b.lm_head = synth.random_lm_head(V, H, dtype, seed + 5, scale=w_scale)
    k = np.zeros(b.N, np.float32)
    k[0::3] = kappa
    k[1::3] = -kappa
    b.hidden = synth.aligned_rows(b.lm_head, b.tokens, dtype, k, seed + 6)
    b.extra["kappa"] = k
    return b


def _check_peaked(b, what):
    logmu = logmu_from_oracle(b)
    out = run_fwd_bwd(batch_to_dev(b, logmu))
    ref = oracle_full(b, logmu)
    lp = host(out["logprobs"])
    valid = b.mask != 0
    up = valid & (b.extra["kappa"] > 0)
    down = valid & (b.extra["kappa"] < 0)
    say(what, f"oracle log pi: pulled rows max {ref['logpi'][up].min():.3e}..{ref['logpi'][up].max():.3e}, "
        f"pushed rows {ref['logpi'][down].max():.1f}..{ref['logpi'][down].min():.1f}")
    assert np.all(lp <= 0.0), f"{what}: a logprob above 0"
    assert ref["logpi"][up].min() > -1e-6 and ref["logpi"][down].max() < -60
    # where the other tokens' mass is below half an ulp of 1, the learner's
    # gathered logit is the tile maximum itself: log pi is exactly 0
    certain = up & (ref["logpi"] > -1e-9)
    assert certain.sum() > 10
    assert np.all(lp[certain] == 0.0), f"{what}: p ~ 1 rows not exactly 0"
    # such a row's gradient is c_t (p - onehot) ~ 0: its token's column is
    # applied exactly in fp32 (c_t (p[a_t] - 1) = -c_t expm1(log pi)), not as a
    # bf16-rounded c_t p[a_t] minus c_t, which would leave 2^-9 c_t |W| of noise
    dh = host(out["d_hidden"])
    scale = float(np.abs(ref["d_hidden"]).max())
    worst = float(np.abs(dh[certain]).max()) / scale
    say(what, f"p ~ 1 rows: max |d_hidden| / max|oracle| = {worst:.2e}")
    assert worst < 1e-5, f"{what}: p ~ 1 rows carry gradient noise {worst:.2e}"
    compare_full(out, ref, b, what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_peaked_softmax_full_parity(dtype):
    if dtype == "bf16":
        b = _peaked_batch("bf16", 2560, 4000, 0.3, 41)
    else:  # logit std 15 at H = 256
        b = _peaked_batch("f32", 256, 1000, 0.95, 42)
    say(f"peaked-{dtype}", f"N={b.N} valid={b.n_valid} H={b.H} V={b.V}")
    _check_peaked(b, f"peaked-{dtype}")


def test_peaked_softmax_qwen3_4b_head():
    """The same construction at the full Qwen3-4B head (H = 2560,
    V = 151936, 1187 statistics tiles of 128 columns)."""
    b = _peaked_batch("bf16", 2560, synth.QWEN_VOCAB, 0.3, 43, N_resp=3, lo=60, hi=100,
                      kappa=0.7)
    say("peaked-qwen3-4b", f"N={b.N} valid={b.n_valid}")
    _check_peaked(b, "peaked-qwen3-4b")


@pytest.mark.parametrize("n", [1, 37, 64, 65, 300])
def test_certain_tokens_in_every_tile_form(n):
    """rz_token_logprobs on p ~ 1 rows at 1 .. 300 rows (the single-stage
    64-row tile, the 64-row tile and the 256-row tile): log pi is exactly 0,
    and a pushed-away row's value is the same bits as in the 300-row batch."""
    torch = torch_mod()
    V, H = 3000, 2560
    W = synth.random_lm_head(V, H, "bf16", 51, scale=0.3)
    rng = np.random.default_rng(np.random.PCG64(52))
    tokens = rng.integers(0, V, size=300).astype(np.int32)
    kappa = np.where(np.arange(300) % 2 == 0, 0.6, -0.6).astype(np.float32)
    hidden = synth.aligned_rows(W, tokens, "bf16", kappa, 53)
    Wd = mat_to_dev(W, "bf16")
    full = host(rz.token_logprobs(mat_to_dev(hidden, "bf16"), Wd, vec_to_dev(tokens)))
    lp = host(rz.token_logprobs(mat_to_dev(hidden[:n], "bf16"), Wd, vec_to_dev(tokens[:n])))
    torch.cuda.synchronize()
    say(f"certain-n{n}")
    assert np.array_equal(lp, full[:n])
    assert np.all(lp[0::2] == 0.0) and np.all(lp[1::2] < -60)


def _weights_batch(dtype, seed):
    b = small_batch(N_resp=6, group_size=3, H=256, V=1000, lo=40, hi=160,
                    dtype=dtype, masked=0.25, seed=seed)
    return b


def test_rows_across_the_e_window():
    """bf16 learner: rows whose logits sit near +-60 nats on one half of the
    vocabulary and +-52 on the other, so that their tiles' maxima fall on
    both sides of the window the stored e keeps (2^-32 .. 2^80 for a tile's
    largest term) and the tiles are rebased to the row's reference by exact
    powers of two; rows near 0 and +-30 nats share one reference as they
    are.  The lower half still carries about e^-8 of the mass, so the
    rebased tiles weigh in the gradients.  Every output against the oracle."""
    H, V = 256, 2048
    b = small_batch(N_resp=6, group_size=3, H=H, V=V, lo=40, hi=120,
                    dtype="bf16", masked=0.2, seed=81)
    beta = np.array([1.0, -1.0, 0.0, 0.5], np.float32)[np.arange(b.N) % 4]
    b.hidden, b.lm_head = synth.two_level_logits(b.N, H, V, (66.0, 58.0), beta, 82)
    logmu = logmu_from_oracle(b)
    out = run_fwd_bwd(batch_to_dev(b, logmu))
    ref = oracle_full(b, logmu)
    lse = ref["lse"]
    say("e-window", f"oracle lse by row kind: {[float(np.median(lse[np.arange(b.N) % 4 == k])) for k in range(4)]}")
    compare_full(out, ref, b, "e-window")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_huge_finite_weights_full_parity(dtype):
    """log mu = log pi - 30 on some valid rows (w ~ 1.1e13) and + 30 on
    others (w ~ 9e-14): unclipped, every output compared."""
    b = _weights_batch(dtype, 61)
    logmu = logmu_from_oracle(b)
    vidx = np.flatnonzero(b.mask)
    logmu[vidx[3::17]] -= 30.0
    logmu[vidx[5::17]] += 30.0
    out = run_fwd_bwd(batch_to_dev(b, logmu))
    ref = oracle_full(b, logmu)
    say(f"huge-w-{dtype}", f"max w {ref['w'].max():.3e}, loss {ref['loss']:.4e}, D3 {ref['d3']:.4e}")
    assert ref["w"].max() > 1e12
    compare_full(out, ref, b, f"huge-w-{dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_overflowing_weight(dtype):
    """One valid row with log pi - log mu = 800: w = inf in float64 and in
    fp32 alike.  The loss is the same signed infinity, D3 is inf, KL and the
    advantages stay finite and match, log pi is untouched, that row's
    d_hidden is wholly non-finite and every other row matches, and d_lm_head
    is non-finite exactly where the oracle's is.  (Where the oracle has
    -inf, the learner's split of dlogits into its softmax part and its
    one-hot part can give inf - inf = NaN: the token's own row of dW.)"""
    b = _weights_batch(dtype, 62)
    logmu = logmu_from_oracle(b)
    # a valid row of a response whose advantage is not 0
    A = O.group_mean_advantages(b.rewards, b.group_ids)
    i = int(np.flatnonzero(np.abs(A) > 1e-3)[0])
    rows = np.arange(b.cu_rows[i], b.cu_rows[i + 1])
    t_bad = int(rows[b.mask[rows] != 0][1])
    logmu[t_bad] = np.float32(logmu[t_bad] - 800.0)
    out = run_fwd_bwd(batch_to_dev(b, logmu))
    ref = oracle_full(b, logmu)
    t = TOL[b.dtype]
    loss = float(host(out["loss"])[0])
    say(f"overflow-{dtype}", f"row {t_bad}, oracle loss {ref['loss']}, gpu {loss}")
    assert math.isinf(ref["loss"]) and loss == ref["loss"]
    diag = host(out["diag"])
    assert math.isinf(ref["d3"]) and diag[0] == ref["d3"]
    valid = b.mask != 0
    assert_close(host(out["logprobs"])[valid], ref["logpi"][valid], t["rtol"], t["atol"],
                 "overflow logprobs")
    assert_close(host(out["adv"]), ref["adv"], 1e-6, 1e-7, "overflow adv")
    _, _, kl_tol = scalar_tols(ref, b.mask, b.cu_rows, b.dtype)
    assert_close([diag[1]], [ref["kl"]], t["rtol"], 1e-7 + kl_tol, "overflow KL")
    dh = host(out["d_hidden"])
    assert not np.isfinite(ref["d_hidden"][t_bad]).any()
    assert not np.isfinite(dh[t_bad]).any()
    keep = np.ones(b.N, bool)
    keep[t_bad] = False
    assert np.isfinite(dh[keep]).all()
    # the other rows: their coefficients are finite; compare them with the
    # bound of the finite rows
    c_fin = np.where(np.isfinite(ref["coef"]), ref["coef"], 0.0)
    dlp = np.where(valid, host(out["logprobs"]).astype(np.float64) - ref["logpi"], 0.0)
    bh, _, ch, _ = softmax_grad_bounds(O.to_f64(b.hidden, b.dtype),
                                       O.to_f64(b.lm_head, b.dtype), ref["lse"], c_fin,
                                       tokens=b.tokens, dlogpi=dlp)
    bh = bh[keep] if b.dtype == "bf16" else None
    assert_grad_close(dh[keep], ref["d_hidden"][keep], b.dtype, "overflow d_hidden", bh,
                      ch[keep])
    dw = host(out["d_lm_head"])
    assert np.array_equal(np.isfinite(dw), np.isfinite(ref["d_lm_head"]))
    tok = int(b.tokens[t_bad])
    other = np.ones(b.V, bool)
    other[tok] = False
    assert np.array_equal(dw[other], ref["d_lm_head"][other]), "dW infinities differ"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zipf_tokens_multi_chunk(dtype):
    """Zipf(1.1) tokens over more valid rows than one backward chunk (32768):
    the most frequent token takes thousands of rows, its one-hot fix-up runs
    across many pieces of the sorted list.  Every output against the oracle;
    dW reproducible bit for bit."""
    b = small_batch(N_resp=8, group_size=4, H=64, V=4096, lo=4500, hi=6500,
                    dtype=dtype, masked=0.2, seed=71)
    b.tokens = synth.zipf_tokens(b.N, b.V, 1.1, 72)
    counts = np.bincount(b.tokens[b.mask != 0], minlength=b.V)
    say(f"zipf-{dtype}", f"valid={b.n_valid}, top token rows {counts.max()}")
    assert b.n_valid > 32768 and counts.max() > 5000
    logmu = logmu_from_oracle(b)
    d = batch_to_dev(b, logmu)
    out = run_fwd_bwd(d)
    dw1 = host(out["d_lm_head"]).copy()
    compare_full(out, oracle_full(b, logmu), b, f"zipf-{dtype}")
    again = run_fwd_bwd(d)
    assert np.array_equal(host(again["d_lm_head"]), dw1), "dW not reproducible"


def test_one_token_on_30_percent_of_rows():
    b = small_batch(N_resp=6, group_size=3, H=128, V=2000, lo=300, hi=900,
                    dtype="bf16", masked=0.1, seed=73)
    rng = np.random.default_rng(np.random.PCG64(74))
    b.tokens[rng.random(b.N) < 0.3] = 1234
    say("hot-token", f"N={b.N} rows on token 1234: {(b.tokens == 1234).sum()}")
    logmu = logmu_from_oracle(b)
    out = run_fwd_bwd(batch_to_dev(b, logmu))
    compare_full(out, oracle_full(b, logmu), b, "hot-token")


# ------------------------------------------------------------ score centering
def _sc_case(b, what, with_logmu=True):
    torch = torch_mod()
    logmu = logmu_from_oracle(b)
    d = batch_to_dev(b, logmu)
    out = rz.score_centering_fwd_bwd(d["hidden"], d["lm_head"], d["tokens"], d["mask"],
                                     d["cu_rows"], d["rewards"], d["group_ids"],
                                     logmu=d["logmu"] if with_logmu else None)
    is_out = run_fwd_bwd(d)
    torch.cuda.synchronize()
    ref = O.score_centering_fwd_bwd(O.to_f64(b.hidden, b.dtype), O.to_f64(b.lm_head, b.dtype),
                                    b.tokens, b.mask, b.cu_rows, b.rewards, b.group_ids,
                                    logmu.astype(np.float64) if with_logmu else None)
    say(what, f"N={b.N} B={b.B} loss oracle {ref['loss']:.6e}")
    t = TOL[b.dtype]
    valid = b.mask != 0
    lp = host(out["logprobs"])
    # the same forward kernels as the IS step: the same bits
    assert np.array_equal(lp, host(is_out["logprobs"])), f"{what}: logprobs differ from IS"
    assert_close(lp[valid], ref["logpi"][valid], t["rtol"], t["atol"], f"{what} logprobs")
    assert_close(host(out["adv"]), ref["adv"], 1e-6, 1e-7, f"{what} adv")
    # loss: sum_i |A_i| / (B T_i) sum_t tol_t propagated from the logprobs
    tol_lp = t["atol"] + t["rtol"] * np.abs(ref["logpi"])
    lt = sum(abs(ref["adv"][i]) / (b.B * ref["T"][i]) *
             float(np.sum(tol_lp[b.cu_rows[i]:b.cu_rows[i + 1]][valid[b.cu_rows[i]:b.cu_rows[i + 1]]]))
             for i in range(b.B) if ref["T"][i])
    assert_close([float(host(out["loss"])[0])], [ref["loss"]], t["rtol"], 1e-7 + lt, f"{what} loss")
    if with_logmu:
        diag = host(out["diag"])
        assert np.array_equal(diag, host(is_out["diag"]))
        assert_close(diag, [ref["d3"], ref["kl"]], t["rtol"], 1e-4, f"{what} diag")
    else:
        assert out["diag"] is None
    bh = bw = None
    if b.dtype == "bf16":
        bh, bw = softmax_grad_bounds(O.to_f64(b.hidden, b.dtype), O.to_f64(b.lm_head, b.dtype),
                                     ref["lse"], ref["coef"])
    assert_grad_close(host(out["d_hidden"]), ref["d_hidden"], b.dtype, f"{what} d_hidden", bh)
    assert_grad_close(host(out["d_lm_head"]), ref["d_lm_head"], b.dtype, f"{what} d_lm_head", bw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_score_centering_full_parity(dtype):
    _sc_case(small_batch(dtype=dtype, seed=81), f"sc-{dtype}")


def test_score_centering_without_records_and_singleton_group():
    b = small_batch(N_resp=5, group_size=2, dtype="bf16", seed=82, rewards="bernoulli",
                    V=777, H=128)
    b.group_ids[:] = np.array([0, 1, 0, 1, 2], dtype=np.int32)
    _sc_case(b, "sc-no-logmu", with_logmu=False)


def test_score_centering_qwen3_4b_truncated():
    b = synth.make_workload("qwen3_4b_tool", max_responses=8, max_rows_per_response=100)
    assert np.abs(O.group_mean_advantages(b.rewards, b.group_ids)).max() > 0
    _sc_case(b, "sc-qwen3-4b")
