"""Pins of the float64 oracle to facts fixed outside itself.

Each test checks the oracle against something it does not compute the same
way: closed forms, a library routine the oracle does not call (SciPy,
torch.log_softmax), brute force with Python loops, central finite differences,
the exact-enumeration importance-sampling identities of the REINFORCE Zero
project page ("The full IS correction"), and hand-derived worked cases under
tests/golden/.  A plausible slip anywhere in the oracle (a dropped term, a
flipped sign, a transposed operand, a wrong average) fails at least one test.
"""
import json
import math
import pathlib
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax
from scipy.special import logsumexp as sp_logsumexp

import oracle as O

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _frac(s):
    return float(Fraction(s))


def _rng(seed):
    return np.random.default_rng(np.random.PCG64(seed))


def _small_problem(seed, B=4, H=8, V=16, lo=2, hi=6, masked=True, sigma=0.3,
                   group_size=2):
    rng = _rng(seed)
    lengths = rng.integers(lo, hi + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = int(cu[-1])
    mask = np.ones(N, dtype=np.uint8)
    if masked:
        mask[rng.random(N) < 0.3] = 0
        mask[cu[:-1]] = 1   # every response keeps a valid row
    hidden = rng.standard_normal((N, H))
    W = 0.5 * rng.standard_normal((V, H))
    tokens = rng.integers(0, V, size=N)
    rewards = rng.random(B)
    group_ids = np.arange(B) // group_size
    logpi, _ = O.token_logprobs(hidden, W, tokens)
    logmu = logpi + sigma * rng.standard_normal(N)
    return dict(hidden=hidden, W=W, tokens=tokens, mask=mask, cu=cu,
                rewards=rewards, group_ids=group_ids, logmu=logmu)


def _loss_of(p, hidden, W):
    logpi_all, _ = O.token_logprobs(hidden, W, p["tokens"])
    logpi = np.where(p["mask"] != 0, logpi_all, 0.0)
    return O.loss_stage(logpi, p["logmu"], p["mask"], p["cu"], p["rewards"],
                        p["group_ids"])["loss"]


# ------------------------------------------------------------ input decode
def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001],
                    dtype=np.uint16)
    got = O.decode_bf16(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0,
            (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    assert got.tolist() == want


# --------------------------------------------------------- logits/logsoftmax
@pytest.mark.parametrize("V", [1024, 151936])
def test_zero_head_gives_uniform_policy(V):
    """W = 0: every logit is 0, so log pi = -ln V exactly."""
    hidden = _rng(1).standard_normal((3, 4))
    W = np.zeros((V, 4))
    tokens = np.array([0, V // 2, V - 1])
    logpi, lse = O.token_logprobs(hidden, W, tokens)
    assert np.allclose(logpi, -math.log(V), rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-12)


def test_onehot_hidden_selects_head_column():
    """hidden = e_k gives z = W[:, k]; compare with SciPy's log_softmax."""
    rng = _rng(2)
    V, H = 37, 5
    W = rng.standard_normal((V, H))
    for k in range(H):
        hidden = np.zeros((V, H))
        hidden[:, k] = 1.0
        tokens = np.arange(V)
        logpi, lse = O.token_logprobs(hidden, W, tokens)
        ref = sp_log_softmax(W[:, k])
        assert np.allclose(logpi, ref, rtol=0, atol=1e-13)
        assert np.allclose(lse, sp_logsumexp(W[:, k]), rtol=0, atol=1e-13)


def test_two_class_closed_form():
    """V = 2: log pi(0) = -log(1 + exp(z1 - z0))."""
    rng = _rng(3)
    hidden = rng.standard_normal((50, 6))
    W = 3.0 * rng.standard_normal((2, 6))
    z = np.array([[sum(hidden[t, h] * W[v, h] for h in range(6)) for v in range(2)]
                  for t in range(50)])
    for a in (0, 1):
        logpi, _ = O.token_logprobs(hidden, W, np.full(50, a))
        want = -np.log1p(np.exp(z[:, 1 - a] - z[:, a]))
        assert np.allclose(logpi, want, rtol=0, atol=1e-13)


def test_probabilities_sum_to_one():
    rng = _rng(4)
    V, H = 64, 7
    hidden = rng.standard_normal((5, H))
    W = rng.standard_normal((V, H))
    tot = np.zeros(5)
    for a in range(V):
        lp, _ = O.token_logprobs(hidden, W, np.full(5, a))
        tot += np.exp(lp)
    assert np.allclose(tot, 1.0, rtol=0, atol=1e-13)


def test_gather_brute_force_python_loops():
    rng = _rng(5)
    N, H, V = 6, 4, 9
    hidden = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    tokens = rng.integers(0, V, size=N)
    logpi, lse = O.token_logprobs(hidden, W, tokens, row_chunk=4)
    for t in range(N):
        z = [math.fsum(hidden[t, h] * W[v, h] for h in range(H)) for v in range(V)]
        m = max(z)
        l = m + math.log(math.fsum(math.exp(x - m) for x in z))
        assert abs(lse[t] - l) < 1e-13
        assert abs(logpi[t] - (z[tokens[t]] - l)) < 1e-13


def test_log_softmax_against_torch_f64():
    torch = pytest.importorskip("torch")
    rng = _rng(6)
    hidden = rng.standard_normal((40, 16))
    W = 0.3 * rng.standard_normal((300, 16))
    tokens = rng.integers(0, 300, size=40)
    logpi, _ = O.token_logprobs(hidden, W, tokens, row_chunk=7)
    z = torch.from_numpy(hidden) @ torch.from_numpy(W).T
    ref = torch.log_softmax(z, dim=1)[torch.arange(40), torch.from_numpy(tokens)]
    assert np.allclose(logpi, ref.numpy(), rtol=0, atol=1e-12)


def test_large_logits_do_not_overflow():
    hidden = np.array([[1000.0, -1000.0]])
    W = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 0.0]])
    logpi, lse = O.token_logprobs(hidden, W, np.array([2]))
    z = np.array([1000.0, -1000.0, 500.0])
    assert np.isfinite(logpi).all()
    assert abs(lse[0] - sp_logsumexp(z)) < 1e-9
    assert abs(logpi[0] - (500.0 - sp_logsumexp(z))) < 1e-9


# -------------------------------------------------------------- advantages
def test_group_advantages_sum_to_zero_per_group():
    rng = _rng(7)
    rewards = rng.integers(0, 2, size=64).astype(np.float64)
    groups = rng.permutation(np.arange(64) // 8)
    A = O.group_mean_advantages(rewards, groups)
    for g in range(8):
        assert abs(A[groups == g].sum()) < 1e-15
    rewards = rng.random(64)
    A = O.group_mean_advantages(rewards, groups)
    for g in range(8):
        assert abs(A[groups == g].sum()) < 1e-14


def test_advantage_values_hand_case():
    A = O.group_mean_advantages(np.array([1.0, 0.0, 0.5, 0.25, 3.0]),
                                np.array([3, 3, 9, 9, 1]))
    assert A.tolist() == [0.5, -0.5, 0.125, -0.125, 0.0]


def test_equal_rewards_give_zero_loss_and_gradient():
    p = _small_problem(8)
    p["rewards"] = np.full_like(p["rewards"], 0.7)
    out = O.reinforce_zero_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["logmu"],
                                   p["mask"], p["cu"], p["rewards"], p["group_ids"])
    assert out["loss"] == 0.0
    assert not out["d_hidden"].any() and not out["d_lm_head"].any()


# --------------------------------------------------------- the loss itself
def test_two_level_mean_golden():
    g = json.loads((GOLDEN / "two_level_mean.json").read_text())
    cu = np.array(g["cu_rows"])
    mask = np.array(g["mask"], dtype=np.uint8)
    w = np.array(g["weights"])
    logmu = np.zeros(len(w))
    logpi = np.log(w)      # so that log pi - log mu = ln w
    st = O.loss_stage(logpi, logmu, mask, cu, np.array(g["rewards"]),
                      np.array(g["group_ids"]))
    e = g["expected"]
    assert st["adv"].tolist() == [_frac(a) for a in e["adv"]]
    assert st["T"].tolist() == e["T"]
    assert abs(st["loss"] - _frac(e["loss"])) < 1e-15
    assert abs(st["loss"] - _frac(e["flat_token_mean_loss_for_contrast"])) > 0.1
    assert np.allclose(st["coef"], [_frac(c) for c in e["coef"]], rtol=0, atol=1e-15)
    assert abs(st["d3"] - (7 / 8 - math.log(2) / 2)) < 1e-15
    assert abs(st["kl"] - (-math.log(2) / 2)) < 1e-15


def test_T_counts_valid_rows_not_length():
    cu = np.array([0, 4, 6])
    mask = np.array([1, 0, 0, 1, 1, 1], dtype=np.uint8)
    assert O.valid_token_counts(cu, mask).tolist() == [2, 2]


def test_response_without_valid_tokens_contributes_nothing():
    cu = np.array([0, 2, 4, 5])
    mask = np.array([1, 1, 0, 0, 1], dtype=np.uint8)
    logpi = np.array([-1.0, -2.0, -3.0, -4.0, -0.5])
    logmu = logpi - np.array([0.1, -0.2, 5.0, 5.0, 0.3])
    rewards = np.array([1.0, 0.0, 0.0])
    groups = np.array([0, 0, 1])
    st = O.loss_stage(logpi, logmu, mask, cu, rewards, groups)
    # B = 3 still divides; response 1 (T = 0) adds nothing; response 2 has A = 0
    want = -(1 / 3) * (0.5 * (math.exp(0.1) + math.exp(-0.2)) / 2)
    assert abs(st["loss"] - want) < 1e-15
    assert st["coef"][2] == 0.0 and st["coef"][3] == 0.0


# ------------------------------------------------------------- diagnostics
def test_unit_weights_give_exact_zero_diagnostics():
    rng = _rng(9)
    logpi = -rng.random(1000) * 12
    d3, kl = O.diagnostics(logpi, logpi.copy())
    assert d3 == 0.0 and kl == 0.0


def test_empty_valid_set_gives_nan():
    d3, kl = O.diagnostics(np.zeros(3), np.zeros(3), np.zeros(3, dtype=np.uint8))
    assert math.isnan(d3) and math.isnan(kl)


def test_lag_noise_closed_form():
    g = json.loads((GOLDEN / "lag_noise_d3.json").read_text())
    n = 1_000_000
    for case in g["cases"]:
        sigma = case["sigma"]
        rng = _rng(11)
        logpi = -12.0 + rng.standard_normal(n)
        logmu = logpi + sigma * rng.standard_normal(n)
        d3, kl = O.diagnostics(logpi, logmu)
        se_d3 = sigma ** 2 / math.sqrt(2 * n)
        assert abs(d3 - case["expected_d3"]) < 5 * se_d3
        assert abs(kl) < 5 * sigma / math.sqrt(n)


# ---------------------------------------------------------------- gradient
def _fd_check(p, seed):
    out = O.reinforce_zero_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["logmu"],
                                   p["mask"], p["cu"], p["rewards"], p["group_ids"])
    rng = _rng(seed)
    eps = 1e-6
    for name, arr, grad in (("hidden", p["hidden"], out["d_hidden"]),
                            ("W", p["W"], out["d_lm_head"])):
        scale = np.abs(grad).max()
        flat = rng.choice(arr.size, size=min(64, arr.size), replace=False)
        for f in flat:
            idx = np.unravel_index(f, arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            if name == "hidden":
                fd = (_loss_of(p, plus, p["W"]) - _loss_of(p, minus, p["W"])) / (2 * eps)
            else:
                fd = (_loss_of(p, p["hidden"], plus) - _loss_of(p, p["hidden"], minus)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * scale + 1e-6 * abs(grad[idx]), (name, idx)
    # random directions through both inputs at once
    for _ in range(4):
        dh = rng.standard_normal(p["hidden"].shape)
        dw = rng.standard_normal(p["W"].shape)
        fd = (_loss_of(p, p["hidden"] + eps * dh, p["W"] + eps * dw)
              - _loss_of(p, p["hidden"] - eps * dh, p["W"] - eps * dw)) / (2 * eps)
        an = float((out["d_hidden"] * dh).sum() + (out["d_lm_head"] * dw).sum())
        assert abs(fd - an) <= 1e-6 * max(1e-12, abs(an)) + 1e-9


@pytest.mark.parametrize("seed", [21, 22])
def test_finite_difference_gradients(seed):
    _fd_check(_small_problem(seed), seed + 100)


def test_finite_difference_gradients_unmasked_single_group():
    _fd_check(_small_problem(23, masked=False, group_size=4), 123)


def test_unit_weights_gradient_is_plain_reinforce():
    """log mu := log pi makes w = 1; the IS loss's gradient must then equal the
    gradient of the plain REINFORCE surrogate
    J = -(1/B) sum_i (A_i / T_i) sum_t log pi_t, taken by finite differences."""
    p = _small_problem(24)
    logpi_all, _ = O.token_logprobs(p["hidden"], p["W"], p["tokens"])
    p["logmu"] = np.where(p["mask"] != 0, logpi_all, 0.0)
    out = O.reinforce_zero_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["logmu"],
                                   p["mask"], p["cu"], p["rewards"], p["group_ids"])
    assert out["d3"] == 0.0 and out["kl"] == 0.0
    assert abs(out["loss"] + np.sum(out["adv"]) / len(p["rewards"])) < 1e-15
    B = len(p["rewards"])
    A = out["adv"]
    T = out["T"]

    def surrogate(hidden, W):
        lp, _ = O.token_logprobs(hidden, W, p["tokens"])
        tot = 0.0
        for i in range(B):
            rows = range(p["cu"][i], p["cu"][i + 1])
            tot += A[i] / T[i] * sum(lp[t] for t in rows if p["mask"][t])
        return -tot / B

    rng = _rng(124)
    eps = 1e-6
    for _ in range(6):
        dh = rng.standard_normal(p["hidden"].shape)
        dw = rng.standard_normal(p["W"].shape)
        fd = (surrogate(p["hidden"] + eps * dh, p["W"] + eps * dw)
              - surrogate(p["hidden"] - eps * dh, p["W"] - eps * dw)) / (2 * eps)
        an = float((out["d_hidden"] * dh).sum() + (out["d_lm_head"] * dw).sum())
        assert abs(fd - an) <= 1e-6 * abs(an) + 1e-10


def test_masked_rows_do_not_affect_loss_or_gradients():
    p = _small_problem(25)
    base = O.reinforce_zero_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["logmu"],
                                    p["mask"], p["cu"], p["rewards"], p["group_ids"])
    q = dict(p)
    m0 = p["mask"] == 0
    assert m0.any()
    rng = _rng(26)
    q["hidden"] = p["hidden"].copy()
    q["hidden"][m0] = rng.standard_normal((int(m0.sum()), p["hidden"].shape[1]))
    q["logmu"] = p["logmu"].copy()
    q["logmu"][m0] = -50.0
    q["tokens"] = p["tokens"].copy()
    q["tokens"][m0] = 0
    other = O.reinforce_zero_fwd_bwd(q["hidden"], q["W"], q["tokens"], q["logmu"],
                                     q["mask"], q["cu"], q["rewards"], q["group_ids"])
    assert base["loss"] == other["loss"]
    assert np.array_equal(base["d_lm_head"], other["d_lm_head"])
    assert not base["d_hidden"][m0].any() and not base["logpi"][m0].any()


# ------------------------------------------- exact-enumeration IS identities
def test_importance_sampling_identities_by_enumeration():
    """'The full IS correction' on the REINFORCE Zero project page: at a fixed
    history with sampler q = mu and target p = pi, E_q[w s] = 0 and
    E_q[w A s] = Cov_p(A, s) = E_p[A s], where s = grad_z log pi.  A batch of
    single-token responses whose token multiset is exactly mu turns the batch
    means into these expectations, with no sampling error."""
    mu = np.array([0.5, 0.25, 0.125, 0.125])
    tokens = np.array([0, 0, 0, 0, 1, 1, 2, 3])       # multiset reproduces mu
    reward_of = np.array([1.0, 0.0, 0.5, 1.0])
    z = np.array([0.3, -0.1, 0.7, 0.0])
    W = z[:, None]                                     # H = 1, hidden = [1]
    hidden = np.ones((8, 1))
    B = 8
    logmu = np.log(mu[tokens])
    mask = np.ones(8, dtype=np.uint8)
    cu = np.arange(9)
    rewards = reward_of[tokens]
    groups = np.zeros(8, dtype=np.int64)
    out = O.reinforce_zero_fwd_bwd(hidden, W, tokens, logmu, mask, cu, rewards, groups)

    pi = np.exp(z) / np.exp(z).sum()
    score = np.eye(4) - pi                     # row a: grad_z log pi(a)
    # E_q[w s] = sum_a mu(a) (pi(a)/mu(a)) s(a) = sum_a pi(a) s(a) = 0
    w = np.exp(O.log_ratio(out["logpi"], logmu))
    assert np.allclose((w[:, None] * score[tokens]).mean(axis=0), 0.0, atol=1e-15)
    # the loss gradient wrt the shared logits is -(1/B) sum_i A_i w_i s(a_i)
    # and dW[:, 0] collects it (hidden = 1); it must equal -E_p[A s].
    rbar = (mu * reward_of).sum()
    target = (pi[:, None] * (reward_of - rbar)[:, None] * score).sum(axis=0)
    assert np.allclose(-out["d_lm_head"][:, 0], target, rtol=0, atol=1e-14)
    # D3 = E_mu[w - 1 - log w] = KL(mu || pi) exactly, and so is the k1 KL
    kl_exact = float((mu * np.log(mu / pi)).sum())
    assert abs(out["d3"] - kl_exact) < 1e-15
    assert abs(out["kl"] - kl_exact) < 1e-15
    assert kl_exact > 0.0
    assert B == len(rewards)


# --------------------------------------------------------- score centering
def _enumeration_batch():
    mu = np.array([0.5, 0.25, 0.125, 0.125])
    tokens = np.array([0, 0, 0, 0, 1, 1, 2, 3])       # multiset reproduces mu
    reward_of = np.array([1.0, 0.0, 0.5, 1.0])
    z = np.array([0.3, -0.1, 0.7, 0.0])
    return dict(mu=mu, tokens=tokens, reward_of=reward_of, z=z, W=z[:, None],
                hidden=np.ones((8, 1)), mask=np.ones(8, dtype=np.uint8),
                cu=np.arange(9), rewards=reward_of[tokens],
                groups=np.zeros(8, dtype=np.int64), logmu=np.log(mu[tokens]))


def test_score_centering_is_the_sampler_covariance_by_enumeration():
    """'The full IS correction', block 03: g_SC = Cov_q(A, s), and its gap to
    the target update is Cov_q(A, s) - Cov_p(A, s).  One group of
    single-token responses whose tokens reproduce q = mu exactly: the SC
    update (minus the loss gradient wrt the shared logits, collected in
    dW[:, 0] with hidden = 1) must equal the covariance written in its
    two-sided form E_q[(A - E_q A)(s - E_q s)], and the gap to the IS update
    must equal the difference of the two covariances."""
    e = _enumeration_batch()
    sc = O.score_centering_fwd_bwd(e["hidden"], e["W"], e["tokens"], e["mask"],
                                   e["cu"], e["rewards"], e["groups"], e["logmu"])
    is_ = O.reinforce_zero_fwd_bwd(e["hidden"], e["W"], e["tokens"], e["logmu"],
                                   e["mask"], e["cu"], e["rewards"], e["groups"])
    pi = np.exp(e["z"]) / np.exp(e["z"]).sum()
    q, R = e["mu"], e["reward_of"]
    score = np.eye(4) - pi                      # row a: grad_z log pi(a)
    s_q = (q[:, None] * score).sum(axis=0)      # E_q[s] = q - pi (not 0)
    cov_q = sum(q[a] * (R[a] - q @ R) * (score[a] - s_q) for a in range(4))
    cov_p = sum(pi[a] * (R[a] - pi @ R) * score[a] for a in range(4))
    g_sc = -sc["d_lm_head"][:, 0]
    g_is = -is_["d_lm_head"][:, 0]
    assert np.allclose(g_sc, cov_q, rtol=0, atol=1e-15)
    assert np.allclose(g_sc - g_is, cov_q - cov_p, rtol=0, atol=1e-15)
    assert np.abs(cov_q - cov_p).max() > 1e-2   # q != p: SC keeps a bias
    # the drift SC removes: the update with uncentred rewards is
    # Cov_q(R, s) + E_q[R] E_q[s] (block 02)
    uncentred = sum(q[a] * R[a] * score[a] for a in range(4))
    assert np.allclose(uncentred, cov_q + (q @ R) * s_q, rtol=0, atol=1e-15)
    # the diagnostics of the records are those of the IS call
    assert sc["d3"] == is_["d3"] and sc["kl"] == is_["kl"]


def test_score_centering_surrogate_hand_case():
    """One group, r = (1, 0): A = (1/2, -1/2); T = (1, 3) with a masked row
    in between.  L_SC = -1/2 (1/2 lp_1 - 1/2 (lp_3 + lp_4 + lp_5) / 3) with
    lp = (-1/2, *, -1, -2, -1/4) = -7/48."""
    logpi = np.array([-0.5, -9.0, -1.0, -2.0, -0.25])
    mask = np.array([1, 0, 1, 1, 1], dtype=np.uint8)
    cu = np.array([0, 1, 5])
    A = O.group_mean_advantages(np.array([1.0, 0.0]), np.array([0, 0]))
    T = O.valid_token_counts(cu, mask)
    assert list(T) == [1, 3] and list(A) == [0.5, -0.5]
    assert abs(O.score_centering_surrogate(logpi, mask, cu, A, T) - _frac("-7/48")) < 1e-16


def test_score_centering_finite_difference_gradients():
    p = _small_problem(31)
    out = O.score_centering_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["mask"],
                                    p["cu"], p["rewards"], p["group_ids"])
    A, T = out["adv"], out["T"]

    def loss(hidden, W):
        lp, _ = O.token_logprobs(hidden, W, p["tokens"])
        lp = np.where(p["mask"] != 0, lp, 0.0)
        return O.score_centering_surrogate(lp, p["mask"], p["cu"], A, T)

    assert loss(p["hidden"], p["W"]) == out["loss"]
    rng = _rng(131)
    eps = 1e-6
    for _ in range(6):
        dh = rng.standard_normal(p["hidden"].shape)
        dw = rng.standard_normal(p["W"].shape)
        fd = (loss(p["hidden"] + eps * dh, p["W"] + eps * dw)
              - loss(p["hidden"] - eps * dh, p["W"] - eps * dw)) / (2 * eps)
        an = float((out["d_hidden"] * dh).sum() + (out["d_lm_head"] * dw).sum())
        assert abs(fd - an) <= 1e-6 * abs(an) + 1e-10


def test_score_centering_equals_is_at_unit_weights_and_vanishes_at_equal_rewards():
    p = _small_problem(32)
    logpi_all, _ = O.token_logprobs(p["hidden"], p["W"], p["tokens"])
    at_pi = np.where(p["mask"] != 0, logpi_all, 0.0)
    is_ = O.reinforce_zero_fwd_bwd(p["hidden"], p["W"], p["tokens"], at_pi,
                                   p["mask"], p["cu"], p["rewards"], p["group_ids"])
    sc = O.score_centering_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["mask"],
                                   p["cu"], p["rewards"], p["group_ids"])
    for k in ("d_hidden", "d_lm_head"):
        assert np.allclose(sc[k], is_[k], rtol=1e-13, atol=1e-16)
    flat = O.score_centering_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["mask"],
                                     p["cu"], np.full(len(p["rewards"]), 0.7),
                                     p["group_ids"])
    assert flat["loss"] == 0.0
    assert not flat["d_hidden"].any() and not flat["d_lm_head"].any()


# ------------------------------------------------------- rollout-side sampler
# Published known-answer vectors of Philox4x32-10 (Salmon, Moraes, Dror and
# Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011; the
# known-answer file of its reference implementation): counter, key, output.
PHILOX_KAT = [
    ([0x00000000] * 4, [0x00000000] * 2,
     [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
    ([0xffffffff] * 4, [0xffffffff] * 2,
     [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
    ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
     [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    got = O.philox4x32_10(np.array(ctr, dtype=np.uint64), np.array(key, dtype=np.uint64))
    assert [int(x) for x in got] == want


def test_philox_batches_like_single_calls():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2 ** 32, size=(7, 4), dtype=np.uint64)
    key = np.array([0x12345678, 0x9abcdef0], dtype=np.uint64)
    batch = O.philox4x32_10(ctr, key)
    for i in range(7):
        assert np.array_equal(batch[i], O.philox4x32_10(ctr[i], key))


def test_gumbel_uniforms_range_moments_and_layout():
    ids = np.arange(200, dtype=np.int64)
    u = O.gumbel_uniforms(7, ids, 1000)
    assert u.shape == (200, 1000)
    assert u.min() > 0.0 and u.max() < 1.0
    # mean 1/2 and variance 1/12 of U(0, 1): 2e5 draws, standard errors
    # 6.5e-4 and 1.9e-4; the bounds are ~8 standard errors
    assert abs(u.mean() - 0.5) < 5e-3
    assert abs(u.var() - 1.0 / 12.0) < 1.5e-3
    # word v % 4 of counter v // 4: four consecutive columns share a call
    x = O.philox4x32_10(np.array([2, 13, 0, 0], dtype=np.uint64),
                        np.array([7, 0], dtype=np.uint64))
    assert np.array_equal(np.round(u[13, 8:12] * 2.0 ** 32 - 0.5), x.astype(np.float64))
    # the high word of the id and the seed's high word both enter
    hi = O.gumbel_uniforms(7, np.array([13 + (1 << 32)]), 1000)
    assert not np.array_equal(hi[0], u[13])
    assert not np.array_equal(O.gumbel_uniforms(7 + (1 << 32), ids[:1], 1000)[0], u[0])


def test_sampler_frequencies_match_softmax():
    """Gumbel-max draws over many row ids follow softmax(z): chi-square of
    60000 draws over 6 classes (5 degrees of freedom; 30 is far past the
    0.01% point, so a correct sampler passes for any seed with certainty
    in practice, and a biased one fails)."""
    z = np.array([0.3, -1.2, 2.0, 0.0, 0.5, -0.7])
    n = 60000
    hidden = np.tile(z, (n, 1))
    tokens, logmu, gap = O.sample_tokens(hidden, np.eye(6), np.arange(n), seed=11,
                                         row_chunk=4096)
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = np.bincount(tokens, minlength=6)
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 30.0, (chi2, counts, n * p)
    assert np.allclose(logmu, np.log(p)[tokens], rtol=0, atol=1e-12)
    assert np.all(gap >= 0.0)


def test_sampler_draw_depends_on_row_id_not_batch():
    rng = np.random.default_rng(3)
    H, V = 8, 50
    W = rng.normal(size=(V, H))
    hidden = rng.normal(size=(12, H))
    ids = rng.integers(0, 2 ** 40, size=12)
    tok, lmu, _ = O.sample_tokens(hidden, W, ids, seed=99)
    perm = rng.permutation(12)
    tok_p, lmu_p, _ = O.sample_tokens(hidden[perm], W, ids[perm], seed=99)
    assert np.array_equal(tok_p, tok[perm])
    assert np.array_equal(lmu_p, lmu[perm])
    # each row alone gives the same draw (its log mu only to rounding: the
    # float64 matrix product itself varies with the batch shape in its last
    # bits), and the record is the learner's log pi
    for i in range(12):
        t1, l1, _ = O.sample_tokens(hidden[i:i + 1], W, ids[i:i + 1], seed=99)
        assert t1[0] == tok[i] and abs(l1[0] - lmu[i]) < 1e-12
    logpi, _ = O.token_logprobs(hidden, W, tok)
    assert np.allclose(logpi, lmu, rtol=0, atol=1e-12)
    # brute force: the argmax of z + g, smallest index on ties
    u = O.gumbel_uniforms(99, ids, V)
    score = hidden @ W.T - np.log(-np.log(u))
    for i in range(12):
        best = max(range(V), key=lambda v: (score[i, v], -v))
        assert best == tok[i]


# ------------------------------------------------------ run-level diagnostics
def test_grad_norms_hand_case_and_identities():
    dh = np.array([[3.0, 0.0], [0.0, 4.0]])
    dw = np.array([[1.0, 2.0, 2.0]])
    assert O.grad_norms(dh, dw) == (5.0, 3.0)
    rng = np.random.default_rng(4)
    a = rng.normal(size=(37, 11))
    b = rng.normal(size=(5, 11))
    na, nb = O.grad_norms(a, b)
    # a library norm of a different formulation (scipy's BLAS nrm2 path)
    import scipy.linalg
    assert abs(na - scipy.linalg.norm(a)) < 1e-12 * na
    # permutation and scaling identities
    assert abs(O.grad_norms(a[::-1], b)[0] - na) < 1e-12 * na
    assert abs(O.grad_norms(a, 3.0 * b)[1] - 3.0 * nb) < 1e-12 * nb


def test_response_diagnostics_hand_case():
    # two responses: rows 0-2 (row 1 masked) and rows 3-4; a third with no
    # valid row
    logpi = np.array([-1.0, -5.0, -2.0, -0.5, -0.5, -3.0])
    logmu = np.array([-1.5, -1.0, -2.0, -0.5, -1.0, -3.0])
    mask = np.array([1, 0, 1, 1, 1, 0], dtype=np.uint8)
    cu = np.array([0, 3, 5, 6])
    d3, kl = O.response_diagnostics(logpi, logmu, mask, cu)
    f = lambda d: math.expm1(d) - d
    assert abs(d3[0] - (f(0.5) + f(0.0)) / 2) < 1e-15
    assert abs(kl[0] - (-0.5 + 0.0) / 2) < 1e-15
    assert abs(d3[1] - (f(0.0) + f(0.5)) / 2) < 1e-15
    assert abs(kl[1] - (0.0 - 0.5) / 2) < 1e-15
    assert np.isnan(d3[2]) and np.isnan(kl[2])
    # the token-weighted mean of per-response values is the flat step value
    flat_d3, flat_kl = O.diagnostics(logpi, logmu, mask)
    counts = np.array([2, 2])
    assert abs((counts * d3[:2]).sum() / counts.sum() - flat_d3) < 1e-15
    assert abs((counts * kl[:2]).sum() / counts.sum() - flat_kl) < 1e-15


def test_run_summary_hand_case():
    d3 = [0.1, 0.2, 0.15, 3.0, 0.1]          # median 0.15, one spike
    kl = [1.0, 2.0, 3.0, 10.0, 20.0, 30.0]   # window 3: medians 2 and 20
    g = [0.5, 38.27, 1.0]
    s = O.run_summary(d3, kl, g, window=3)
    assert s["d3_peak"] == 3.0 and s["d3_median"] == 0.15
    assert abs(s["d3_peak_over_median"] - 20.0) < 1e-12
    assert s["kl_median_first"] == 2.0 and s["kl_median_last"] == 20.0
    assert s["kl_median_ratio"] == 10.0
    assert s["grad_norm_max"] == 38.27
    # even count: the mean of the two middle values
    assert O.run_summary([1.0, 2.0, 4.0, 8.0], [1.0], [0.0])["d3_median"] == 3.0
    # a run at diff 0 has D3 = 0 at every step: the quotient is IEEE 0/0
    z = O.run_summary([0.0, 0.0, 0.0], [0.0, 0.0], [1.0], window=1)
    assert z["d3_peak"] == 0.0 and np.isnan(z["d3_peak_over_median"])
    assert np.isnan(z["kl_median_ratio"])
    assert O.run_summary([0.0, 0.0, 2.0], [1.0], [1.0])["d3_peak_over_median"] == np.inf
    # a NaN step value (a step without valid tokens) poisons its statistics
    n = O.run_summary([0.1, np.nan, 0.2], [1.0, 2.0], [3.0, np.nan], window=1)
    assert np.isnan(n["d3_peak"]) and np.isnan(n["d3_median"])
    assert n["kl_median_first"] == 1.0 and n["kl_median_last"] == 2.0
    assert np.isnan(n["grad_norm_max"])
    # a window longer than the run takes all of it for both medians
    w = O.run_summary([1.0], [3.0, 1.0, 2.0], [0.0], window=1000)
    assert w["kl_median_first"] == w["kl_median_last"] == 2.0


# ------------------------------------------------------------ MX-format head
def test_e2m1_values_of_the_specification():
    # OCP MX v1.0: E2M1 magnitudes 0, 0.5 (the subnormal), 1 (smallest
    # normal), 1.5, 2, 3, 4, 6 (largest); bit 3 is the sign
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = O.decode_e2m1(np.arange(16))
    assert got[:8].tolist() == mags
    assert (-got[8:]).tolist() == mags
    assert math.copysign(1.0, got[8]) == -1.0          # code 8 is -0


def test_e4m3_against_the_specification_and_torch():
    import torch
    codes = np.arange(256)
    got = O.decode_e4m3(codes)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.flatnonzero(np.isnan(got)).tolist() == [0x7F, 0xFF]
    # listed values: largest normal 448, smallest normal 2^-6, largest
    # subnormal 0.875 * 2^-6, smallest subnormal 2^-9
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6
    assert got[0x07] == 0.875 * 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0xFE] == -448.0


def test_e8m0_against_torch():
    import torch
    codes = np.arange(256)
    got = O.decode_e8m0(codes)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_unpack_fp4_nibble_order():
    codes = O.unpack_fp4(np.array([[0x21, 0xF8]], dtype=np.uint8))
    assert codes.tolist() == [[1, 2, 8, 15]]
    assert O.decode_e2m1(codes).tolist() == [[0.5, 1.0, -0.0, -6.0]]


def test_dequantize_head_blocks_and_invalid_scales():
    # two rows, H = 64: two blocks per row with their own scales
    V, H = 2, 64
    codes = np.full((V, H), 0x38, dtype=np.uint8)        # E4M3 1.0
    codes[1, 40] = 0x7F                                   # a NaN code
    scales = np.array([[127 + 3, 127 - 2], [127 + 120, 127 - 124]], dtype=np.uint8)
    W = O.dequantize_head(codes, scales, "mxfp8")
    assert np.all(W[0, :32] == 8.0) and np.all(W[0, 32:] == 0.25)
    assert np.all(np.isnan(W[1, :32]))                    # s = 120 > 119
    assert np.all(W[1, 32:40] == 2.0 ** -124) and np.isnan(W[1, 40])
    # E2M1: the NaN scale code and s = 126 > 125 are invalid, s = -127 valid
    packed = np.full((V, H // 2), 0x77, dtype=np.uint8)   # 6.0, 6.0
    sc4 = np.array([[255, 127 + 125], [127 + 126, 0]], dtype=np.uint8)
    W4 = O.dequantize_head(packed, sc4, "mxfp4")
    assert np.all(np.isnan(W4[0, :32])) and np.all(W4[0, 32:] == 6.0 * 2.0 ** 125)
    assert np.all(np.isnan(W4[1, :32])) and np.all(W4[1, 32:] == 6.0 * 2.0 ** -127)


def test_valid_dequantized_values_are_bfloat16_numbers():
    """The reading's exactness claim, checked by brute force: every element
    code at every valid scale (the range ends included) round-trips through
    bfloat16 unchanged, and one step past each end does not for some code."""
    import torch

    def exact(v):
        t = torch.from_numpy(v)
        return bool(torch.equal(t.to(torch.bfloat16).double(), t))

    for fmt, vals in (("mxfp4", O.decode_e2m1(np.arange(16))),
                      ("mxfp8", O.decode_e4m3(np.arange(256)))):
        vals = vals[~np.isnan(vals)]
        lo, hi = O.scale_range(fmt)
        for s in range(lo, hi + 1):
            assert exact(vals * 2.0 ** s), (fmt, s)
        assert not exact(vals * 2.0 ** (hi + 1)), fmt
        if lo > -127:
            assert not exact(vals * 2.0 ** (lo - 1)), fmt


def test_token_logprobs_mx_is_the_bf16_head_definition():
    rng = np.random.default_rng(3)
    V, H, n = 40, 64, 5
    codes = rng.integers(0, 256, size=(V, H // 2), dtype=np.uint8)
    scales = rng.integers(120, 125, size=(V, H // 32), dtype=np.uint8)
    hidden = rng.normal(size=(n, H))
    tok = rng.integers(0, V, size=n)
    lp, lse = O.token_logprobs_mx(hidden, codes, scales, "mxfp4", tok)
    # brute force from the decoded table, element by element
    W = np.zeros((V, H))
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for v in range(V):
        for k in range(H):
            b = int(codes[v, k // 2])
            c = (b & 0xF) if k % 2 == 0 else (b >> 4)
            W[v, k] = (-1 if c & 8 else 1) * table[c & 7] * 2.0 ** (int(scales[v, k // 32]) - 127)
    z = hidden @ W.T
    want = z[np.arange(n), tok] - np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) - z.max(1)
    assert np.allclose(lp, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------- LoRA on the head
def test_round_to_bf16_and_f32_against_torch():
    """Rounding to bfloat16 and float32 agrees with torch's conversions on
    values where a single rounding is taken (float32 inputs for bf16; float64
    inputs for f32), ties and subnormals included."""
    import torch
    rng = _rng(51)
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormal
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -133,
                  3 * 2 ** -134, 0.0, -0.0], dtype=np.float32)])  # ties
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.round_to_bf16(x32.astype(np.float64)), want)
    x64 = np.concatenate([rng.standard_normal(20000), rng.standard_normal(200) * 1e-42])
    want32 = torch.from_numpy(x64).to(torch.float32).double().numpy()
    assert np.array_equal(O.round_to_f32(x64), want32)


def _lora_problem(seed, r=3):
    p = _small_problem(seed)
    rng = _rng(seed + 7)
    H, V = p["hidden"].shape[1], p["W"].shape[0]
    p["A"] = 0.3 * rng.standard_normal((r, H))
    p["B"] = 0.3 * rng.standard_normal((V, r))
    p["s"] = 0.75
    return p


def test_lora_unrounded_is_the_merged_head():
    """With an unrounded activation the adapted head is the plain head with
    W + s B A (the LoRA identity), in logprobs and in the loss."""
    p = _lora_problem(61)
    lp, lse = O.token_logprobs_lora(p["hidden"], p["W"], p["A"], p["B"], p["s"],
                                    p["tokens"], "f32", round_u=False)
    W_eff = p["W"] + p["s"] * (p["B"] @ p["A"])
    lp2, lse2 = O.token_logprobs(p["hidden"], W_eff, p["tokens"])
    assert np.allclose(lp, lp2, rtol=0, atol=1e-12)
    assert np.allclose(lse, lse2, rtol=0, atol=1e-12)
    out = O.reinforce_zero_fwd_bwd_lora(p["hidden"], p["W"], p["A"], p["B"], p["s"],
                                        p["tokens"], p["logmu"], p["mask"], p["cu"],
                                        p["rewards"], p["group_ids"], "f32", round_u=False)
    assert abs(out["loss"] - _loss_of(p, p["hidden"], W_eff)) < 1e-12
    # the hidden-state gradient equals the merged head's
    ref = O.reinforce_zero_fwd_bwd(p["hidden"], W_eff, p["tokens"], p["logmu"], p["mask"],
                                   p["cu"], p["rewards"], p["group_ids"])
    assert np.allclose(out["d_hidden"], ref["d_hidden"], rtol=0, atol=1e-12)
    # and dL/dA, dL/dB are the chain rule through W_eff = W + s B A
    assert np.allclose(out["d_lora_A"], p["s"] * p["B"].T @ ref["d_lm_head"], rtol=0, atol=1e-12)
    assert np.allclose(out["d_lora_B"], p["s"] * ref["d_lm_head"] @ p["A"].T, rtol=0, atol=1e-12)


def test_lora_zero_B_is_the_plain_head():
    p = _lora_problem(62)
    B0 = np.zeros_like(p["B"])
    for dtype in ("bf16", "f32"):
        lp, _ = O.token_logprobs_lora(p["hidden"], p["W"], p["A"], B0, p["s"], p["tokens"], dtype)
        lp2, _ = O.token_logprobs(p["hidden"], p["W"], p["tokens"])
        assert np.array_equal(lp, lp2)
        out = O.reinforce_zero_fwd_bwd_lora(p["hidden"], p["W"], p["A"], B0, p["s"],
                                            p["tokens"], p["logmu"], p["mask"], p["cu"],
                                            p["rewards"], p["group_ids"], dtype)
        assert not out["d_lora_A"].any()
        ref = O.reinforce_zero_fwd_bwd(p["hidden"], p["W"], p["tokens"], p["logmu"], p["mask"],
                                       p["cu"], p["rewards"], p["group_ids"])
        assert np.allclose(out["d_hidden"], ref["d_hidden"], rtol=0, atol=1e-15)


def test_lora_activation_rounding():
    p = _lora_problem(63)
    u = O.lora_activation(p["hidden"], p["A"], p["s"], "bf16")
    exact = p["s"] * p["hidden"] @ p["A"].T
    assert np.all(np.abs(u - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-300)
    assert np.array_equal(O.round_to_bf16(u), u)         # already bf16 values


def test_lora_finite_difference_gradients():
    """Central differences of the loss (unrounded activation) in A, B and h."""
    p = _lora_problem(64)

    def loss(hidden, A, B):
        out = O.reinforce_zero_fwd_bwd_lora(hidden, p["W"], A, B, p["s"], p["tokens"],
                                            p["logmu"], p["mask"], p["cu"], p["rewards"],
                                            p["group_ids"], "f32", round_u=False)
        return out["loss"]

    out = O.reinforce_zero_fwd_bwd_lora(p["hidden"], p["W"], p["A"], p["B"], p["s"],
                                        p["tokens"], p["logmu"], p["mask"], p["cu"],
                                        p["rewards"], p["group_ids"], "f32", round_u=False)
    rng = _rng(65)
    eps = 1e-6
    for _ in range(6):
        dh = rng.standard_normal(p["hidden"].shape)
        dA = rng.standard_normal(p["A"].shape)
        dB = rng.standard_normal(p["B"].shape)
        fd = (loss(p["hidden"] + eps * dh, p["A"] + eps * dA, p["B"] + eps * dB)
              - loss(p["hidden"] - eps * dh, p["A"] - eps * dA, p["B"] - eps * dB)) / (2 * eps)
        an = float((out["d_hidden"] * dh).sum() + (out["d_lora_A"] * dA).sum()
                   + (out["d_lora_B"] * dB).sum())
        assert abs(fd - an) <= 1e-6 * abs(an) + 1e-9, (fd, an)
