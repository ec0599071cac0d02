"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small cases compare every output element by element; they span several
256 x 256 tiles with ragged row and vocab tails, masked rows, shuffled group
ids, a response without valid tokens and the multi-chunk backward.  At the
full workload sizes (in the launch configuration the benchmark times) the
oracle computes sampled rows one by one, and the rest is checked through
properties that hold at any size.
"""
import math

import numpy as np
import pytest

import oracle as O
from invariant_token_logprobs_amd import synth
import invariant_token_logprobs_amd as rz

from gpu_util import (TOL, assert_close, assert_grad_close, batch_to_dev,
                      behaviour_logprobs_torch, compare_full, device, host,
                      logmu_from_oracle, mat_to_dev, oracle_full, run_fwd_bwd,
                      say, small_batch, softmax_grad_bounds, torch_mod,
                      vec_to_dev)

pytestmark = pytest.mark.gpu


def _case(b, what):
    say(what, f"N={b.N} B={b.B} H={b.H} V={b.V} dtype={b.dtype} valid={b.n_valid}")
    logmu = logmu_from_oracle(b)
    out = run_fwd_bwd(batch_to_dev(b, logmu))
    ref = oracle_full(b, logmu)
    compare_full(out, ref, b, what)


def test_tiny_workload_full_parity():
    _case(synth.make_workload("tiny"), "tiny")


def test_tiny_workload_masked_full_parity():
    b = synth.make_workload("tiny")
    rng = np.random.default_rng(np.random.PCG64(99))
    b.mask[rng.random(b.N) < 0.35] = 0
    b.mask[b.cu_rows[:-1]] = 1
    b.mask[b.cu_rows[3]:b.cu_rows[4]] = 0          # response 3: T_i = 0
    _case(b, "tiny-masked")


def test_tiny_token_logprobs():
    b = synth.make_workload("tiny")
    say("tiny token_logprobs")
    lp, lse = rz.token_logprobs(mat_to_dev(b.hidden, "f32"),
                                mat_to_dev(b.lm_head, "f32"),
                                vec_to_dev(b.tokens), want_lse=True)
    ref_lp, ref_lse = O.token_logprobs(O.to_f64(b.hidden, "f32"),
                                       O.to_f64(b.lm_head, "f32"), b.tokens)
    t = TOL["f32"]
    assert_close(host(lp), ref_lp, t["rtol"], t["atol"], "tiny logprobs")
    assert_close(host(lse), ref_lse, t["rtol"], t["atol"], "tiny lse")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_tiles_full_parity(dtype):
    # 6 responses, ~700 rows (3 row tiles, ragged), V = 1000 (ragged vocab tile)
    _case(small_batch(dtype=dtype, seed=11), f"ragged-{dtype}")


def test_bernoulli_rewards_singleton_group():
    b = small_batch(N_resp=5, group_size=2, dtype="bf16", seed=12,
                    rewards="bernoulli", V=777, H=128)
    b.group_ids[:] = np.array([0, 1, 0, 1, 2], dtype=np.int32)  # group 2 is a singleton
    _case(b, "bernoulli-singleton")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_chunk_backward(dtype):
    # more valid rows than one backward chunk (32768): dW accumulates chunks
    b = small_batch(N_resp=8, group_size=4, H=64, V=300, lo=4500, hi=6500,
                    dtype=dtype, masked=0.2, seed=13)
    assert b.n_valid > 32768
    _case(b, f"multichunk-{dtype}")


@pytest.mark.parametrize("n_vtiles", [256, 257, 308, 356])
def test_dw_last_round_split(n_vtiles):
    """The dW GEMM runs one 256 x 256 tile per CU per round and splits the
    tiles of its last round along K, summing the pieces in a fixed order.
    With H = 64 (one column tile) the tile count is the vocab tile count: on
    a 256-CU part, 256 fills whole rounds (no split), 257 leaves one tile
    (four pieces), 308 leaves 52 (four pieces, the count at the Qwen3-4B
    head) and 356 leaves 100 (two pieces).  Each matches the oracle, and a
    second call gives the same dW bit for bit."""
    V = 256 * n_vtiles - 37  # a ragged last vocab tile
    b = small_batch(N_resp=4, group_size=2, H=64, V=V, lo=60, hi=120,
                    dtype="bf16", seed=21)
    what = f"dw-split-{n_vtiles}"
    say(what, f"N={b.N} V={V} tiles={n_vtiles}")
    logmu = logmu_from_oracle(b)
    d = batch_to_dev(b, logmu)
    out = run_fwd_bwd(d)
    dw1 = host(out["d_lm_head"]).copy()
    compare_full(out, oracle_full(b, logmu), b, what)
    again = run_fwd_bwd(d)
    assert np.array_equal(host(again["d_lm_head"]), dw1), f"{what}: dW not reproducible"


@pytest.mark.parametrize("name", ["qwen3_4b_tool", "r1_distill_1p5b", "qwen3_30b_a3b"])
def test_truncated_full_parity(name):
    """Each workload's shape at its full H and V = 151936, every output
    compared, on its first group (8 responses, so the advantages and the
    gradients are not zero) cut to the first rows of each response (about
    1000 valid rows).  The 1.5B head has 6 column tiles of 256, the 30B head
    8, the Qwen3-4B head 10, each with its own dW last-round split."""
    b = synth.make_workload(name, max_responses=8,
                            max_rows_per_response=200 if name == "qwen3_4b_tool" else 128)
    assert b.B == 8 and len(set(b.group_ids.tolist())) == 1
    assert np.abs(O.group_mean_advantages(b.rewards, b.group_ids)).max() > 0
    _case(b, f"{name}-truncated")


# ----------------------------------------------------------- full sizes
def _full_size(name, n_sample_rows=4096, n_sample_grad=16):
    torch = torch_mod()
    b = synth.make_workload(name)
    say(f"{name}: N={b.N} B={b.B} valid={b.n_valid}")
    d = batch_to_dev(b, np.zeros(b.N, np.float32))
    mu_ref = behaviour_logprobs_torch(d["hidden"], d["lm_head"], d["tokens"])
    logmu = synth.make_logmu(host(mu_ref), b.sigma, b.noise_seed)
    del mu_ref
    d["logmu"] = vec_to_dev(logmu)
    out = run_fwd_bwd(d)
    t = TOL[b.dtype]
    valid = b.mask != 0
    vidx = np.flatnonzero(valid)
    rng = np.random.default_rng(np.random.PCG64(4242))

    # sampled logprobs against the oracle, row by row
    rows = np.sort(rng.choice(vidx, size=min(n_sample_rows, len(vidx)), replace=False))
    W64 = O.to_f64(b.lm_head, b.dtype)
    h64 = O.to_f64(b.hidden[rows], b.dtype)
    ref_lp, ref_lse = O.token_logprobs(h64, W64, b.tokens[rows])
    lp = host(out["logprobs"])
    say(f"{name}: {len(rows)} sampled rows checked against the oracle")
    assert_close(lp[rows], ref_lp, t["rtol"], t["atol"], f"{name} sampled logprobs")
    assert np.all(lp[~valid] == 0.0)
    assert np.all(lp[valid] <= 0.0)

    # the loss stage of the oracle (w, T, A, loss, D3, KL) fed this call's
    # own log pi: the GPU's reductions against the plain definition
    st = O.loss_stage(lp.astype(np.float64), logmu.astype(np.float64), b.mask,
                      b.cu_rows, b.rewards, b.group_ids)
    assert_close(host(out["adv"]), st["adv"], 1e-6, 1e-7, f"{name} adv")
    loss = float(host(out["loss"])[0])
    # fp32 weights and an fp32 result: a few fp32 roundings of each term
    scale = float(np.sum(np.abs(st["adv"]) / b.B)) * float(np.max(st["w"][valid]))
    assert abs(loss - st["loss"]) <= 1e-6 * abs(st["loss"]) + 1e-6 * scale, (loss, st["loss"])
    diag = host(out["diag"])
    assert_close(diag, [st["d3"], st["kl"]], 1e-5, 1e-9, f"{name} D3/KL")
    A, T = st["adv"], st["T"]

    # sampled d_hidden rows: c_t from the oracle's own log pi for that row
    grows = rows[:n_sample_grad]
    resp = np.searchsorted(b.cu_rows, grows, side="right") - 1
    lp_g = ref_lp[:n_sample_grad]
    w = np.exp(lp_g - logmu[grows].astype(np.float64))
    c = A[resp] * w / (b.B * T[resp])
    dh_ref, _ = O.backward(h64[:n_sample_grad], W64, b.tokens[grows],
                           ref_lse[:n_sample_grad], c)
    # c_t of the kernel comes from its own log pi: that difference is
    # carried into the bound (see gpu_util)
    bh, _, ch, _ = softmax_grad_bounds(h64[:n_sample_grad], W64, ref_lse[:n_sample_grad], c,
                                       tokens=b.tokens[grows],
                                       dlogpi=lp[grows].astype(np.float64) - lp_g)
    dh = host(out["d_hidden"][torch.from_numpy(grows).to(device())])
    assert_grad_close(dh, dh_ref, b.dtype, f"{name} sampled d_hidden", bh, ch)
    mrows = np.flatnonzero(~valid)[:64]
    if mrows.size:
        assert not host(out["d_hidden"][torch.from_numpy(mrows).to(device())]).any()

    # properties of the whole-batch outputs
    diag2 = host(rz.diagnostics(out["logprobs"], d["logmu"], d["mask"]))
    assert np.array_equal(diag, diag2), "fwd_bwd diag != rz_diagnostics"
    nv = len(vidx)
    e_d3 = math.expm1(b.sigma ** 2 / 2)
    assert abs(diag[0] - e_d3) < 6 * b.sigma ** 2 / math.sqrt(2 * nv) + 3 * t["rtol"] * e_d3, (diag, e_d3)
    assert abs(diag[1]) < 6 * b.sigma / math.sqrt(nv), diag
    # dW: every column sums to zero (sum_v p = 1), and <dW, W> = <dH, h>
    dW = out["d_lm_head"]
    dH = out["d_hidden"]
    colsum = dW.double().sum(dim=0)
    colabs = dW.double().abs().sum(dim=0)
    assert float((colsum.abs() / colabs.clamp_min(1e-30)).max()) < 1e-3
    lhs = float((dW.double() * d["lm_head"].double()).sum())
    rhs = float((dH.double() * d["hidden"].double()).sum())
    assert abs(lhs - rhs) <= 2e-3 * max(abs(lhs), abs(rhs)) + 1e-9, (lhs, rhs)
    del out, d
    torch.cuda.empty_cache()


def test_qwen3_4b_full_size_sampled():
    _full_size("qwen3_4b_tool")


def test_r1_distill_1p5b_full_size_sampled():
    _full_size("r1_distill_1p5b", n_sample_grad=8)


def test_qwen3_30b_full_size_sampled():
    _full_size("qwen3_30b_a3b", n_sample_grad=8)


def test_qwen3_4b_zipf_tokens_full_size():
    """The headline workload with Zipf(1.1) tokens (the most frequent token
    on ~8% of the rows): the one-hot fix-up of dW at full size, checked by
    dW's column sums and <dW, W> = <dH, h>, and dW reproducible bit for
    bit."""
    torch = torch_mod()
    b = synth.make_workload("qwen3_4b_tool", tokens="zipf")
    counts = np.bincount(b.tokens[b.mask != 0], minlength=b.V)
    say(f"qwen3_4b zipf: valid={b.n_valid} top token rows {counts.max()}")
    d = batch_to_dev(b, np.zeros(b.N, np.float32))
    mu_ref = behaviour_logprobs_torch(d["hidden"], d["lm_head"], d["tokens"])
    d["logmu"] = vec_to_dev(synth.make_logmu(host(mu_ref), b.sigma, b.noise_seed))
    del mu_ref
    out = run_fwd_bwd(d)
    dW1 = out["d_lm_head"].clone()
    colsum = dW1.double().sum(dim=0)
    colabs = dW1.double().abs().sum(dim=0)
    assert float((colsum.abs() / colabs.clamp_min(1e-30)).max()) < 1e-3
    lhs = float((dW1.double() * d["lm_head"].double()).sum())
    rhs = float((out["d_hidden"].double() * d["hidden"].double()).sum())
    assert abs(lhs - rhs) <= 2e-3 * max(abs(lhs), abs(rhs)) + 1e-9, (lhs, rhs)
    again = run_fwd_bwd(d)
    assert torch.equal(again["d_lm_head"], dW1), "dW not reproducible"
    del out, again, d, dW1
    torch.cuda.empty_cache()
