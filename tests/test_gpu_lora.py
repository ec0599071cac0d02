"""A LoRA adapter on the head, on the GPU, against the float64 oracle
(oracle/lora_head.py): the augmented operands, the adapted logprobs, the
learner step's loss and gradients (dL/dh, dL/dA, dL/dB), and diff 0 between
the rollout's records and the learner's logprobs.

The GPU rounds u = s h A^T to the head's precision from an fp32 GEMM sum;
the oracle rounds the exact value.  Where the fp32 sum straddles a rounding
boundary the two differ by one unit in the last place of u; the test allows
that for a small share of the entries and checks every other entry exactly.
Logprob and gradient tolerances are those of the plain head (tests/gpu_util),
with the bf16 gradient bounds taken on the augmented operands."""
import numpy as np
import pytest

import oracle as O
from gpu_util import (TOL, assert_close, assert_grad_close, batch_to_dev, host,
                      mat_to_dev, say, small_batch, softmax_grad_bounds,
                      torch_mod, vec_to_dev)
from invariant_token_logprobs_amd import synth

pytestmark = pytest.mark.gpu

SCALE = 0.5
R = 16


def _lora(b, r=R, seed=71):
    A, B = synth.random_lora(r, b.H, b.V, b.dtype, seed)
    return A, B, O.to_f64(A, b.dtype), O.to_f64(B, b.dtype)


def _as_f64(t):
    torch = torch_mod()
    return t.to(torch.float64).cpu().numpy()


def _check_u(u_gpu, u_o, dtype, what, mag):
    """bf16: one unit in the last place where the fp32 sum crossed a rounding
    boundary, exact elsewhere (>97%).  fp32: the GEMM's forward error,
    1e-5 s (|h| |A|^T) per entry (mag), the fp32 tolerance of the path."""
    diff = np.abs(u_gpu - u_o)
    if dtype == "bf16":
        assert np.all(diff <= 2.0 ** -7 * np.abs(u_o) + 1e-30), what
        assert (diff == 0).mean() > 0.97, (what, (diff == 0).mean())
    else:
        assert np.all(diff <= 1e-5 * mag), what


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lora_augment_and_logprobs(dtype):
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    b = small_batch(N_resp=3, group_size=3, H=256, V=1000, lo=80, hi=140,
                    dtype=dtype, seed=81)
    A, B, A64, B64 = _lora(b)
    say("lora augment", dtype, b.N)
    hidden = mat_to_dev(b.hidden, dtype)
    h_aug = rz.lora_augment(hidden, mat_to_dev(A, dtype), SCALE)
    W_aug = rz.lora_merge_head(mat_to_dev(b.lm_head, dtype), mat_to_dev(B, dtype))
    torch.cuda.synchronize()
    H = b.H
    h64 = O.to_f64(b.hidden, dtype)
    ha = _as_f64(h_aug)
    assert np.array_equal(ha[:, :H], h64)
    assert not ha[:, H + R:].any()
    u_o = O.lora_activation(h64, A64, SCALE, dtype)
    _check_u(ha[:, H:H + R], u_o, dtype, f"u {dtype}",
             SCALE * np.abs(h64) @ np.abs(A64).T)
    wa = _as_f64(W_aug)
    assert np.array_equal(wa[:, :H], O.to_f64(b.lm_head, dtype))
    assert np.array_equal(wa[:, H:H + R], B64) and not wa[:, H + R:].any()
    lp = rz.token_logprobs(h_aug, W_aug, vec_to_dev(b.tokens.astype(np.int32)))
    want, _ = O.token_logprobs_lora(h64, O.to_f64(b.lm_head, dtype), A64, B64, SCALE,
                                    b.tokens, dtype)
    t = TOL[dtype]
    assert_close(host(lp), want, t["rtol"], t["atol"], f"lora logprobs {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lora_learner_step_parity(dtype):
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    b = small_batch(N_resp=6, group_size=3, H=256, V=1000, lo=40, hi=200,
                    dtype=dtype, seed=82)
    A, B, A64, B64 = _lora(b, seed=72)
    h64, W64 = O.to_f64(b.hidden, dtype), O.to_f64(b.lm_head, dtype)
    lp_ref, _ = O.token_logprobs_lora(h64, W64, A64, B64, SCALE, b.tokens, dtype)
    logmu = synth.make_logmu(lp_ref, b.sigma, b.noise_seed)
    say("lora learner", dtype, b.N)
    d = batch_to_dev(b, logmu)
    out = rz.reinforce_zero_fwd_bwd_lora(d["hidden"], d["lm_head"], mat_to_dev(A, dtype),
                                         mat_to_dev(B, dtype), SCALE, d["tokens"],
                                         d["logmu"], d["mask"], d["cu_rows"],
                                         d["rewards"], d["group_ids"])
    torch.cuda.synchronize()
    ref = O.reinforce_zero_fwd_bwd_lora(h64, W64, A64, B64, SCALE, b.tokens, logmu,
                                        b.mask, b.cu_rows, b.rewards, b.group_ids, dtype)
    t = TOL[dtype]
    assert_close(host(out["logprobs"]), ref["logpi"], t["rtol"], t["atol"], "logprobs")
    assert abs(host(out["loss"])[0] - ref["loss"]) <= 1e-3 * abs(ref["loss"]) + 1e-5
    bound = None
    if dtype == "bf16":
        h_aug = np.concatenate([h64, ref["u"]], axis=1)
        W_aug = np.concatenate([W64, B64], axis=1)
        bh, bw = softmax_grad_bounds(h_aug, W_aug, ref["lse"], ref["coef"])
        H = b.H
        bound = {"d_hidden": bh[:, :H] + SCALE * bh[:, H:] @ np.abs(A64),
                 "d_lora_A": SCALE * bh[:, H:].T @ np.abs(h64),
                 "d_lora_B": bw[:, H:]}
    for k in ("d_hidden", "d_lora_A", "d_lora_B"):
        assert_grad_close(host(out[k]), ref[k], dtype, f"{k} {dtype}",
                          None if bound is None else bound[k])


def test_lora_diff0_qwen3_4b_head():
    """Rollout and learner on the adapted Qwen3-4B head (bf16, rank 64): the
    rollout's recorded log mu equals the learner's log pi bit for bit, and a
    row's u does not depend on the batch it is augmented in."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    H, V, n, r = 2560, 151936, 96, 64
    hid, _ = synth.random_rows(n, H, V, "bf16", 91)
    W_np = synth.random_lm_head(V, H, "bf16", 92)
    A, B = synth.random_lora(r, H, V, "bf16", 93)
    hidden, W = mat_to_dev(hid, "bf16"), mat_to_dev(W_np, "bf16")
    Ad, Bd = mat_to_dev(A, "bf16"), mat_to_dev(B, "bf16")
    say("lora diff0: rollout")
    h_aug = rz.lora_augment(hidden, Ad, SCALE)
    W_aug = rz.lora_merge_head(W, Bd)
    ids = torch.arange(n, dtype=torch.int64, device="cuda:0")
    tokens, logmu = rz.sample_tokens(h_aug, W_aug, ids, 0xC0FFEE)
    # the same rows augmented one at a time and inside a larger batch
    part = rz.lora_augment(hidden[17:18].contiguous(), Ad, SCALE)
    assert torch.equal(part.view(torch.int16), h_aug[17:18].view(torch.int16))
    say("lora diff0: learner")
    mask = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    cu = torch.tensor([0, 40, 96], dtype=torch.int32, device="cuda:0")
    rewards = torch.tensor([1.0, 0.0], dtype=torch.float32, device="cuda:0")
    gids = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    out = rz.reinforce_zero_fwd_bwd_lora(hidden, W, Ad, Bd, SCALE, tokens, logmu, mask,
                                         cu, rewards, gids)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["logprobs"]).view(np.uint32), host(logmu).view(np.uint32))
    d = host(out["diag"])
    assert d[0] == 0.0 and d[1] == 0.0           # w = 1 exactly: D3 = KL = 0
    del W, W_aug
    torch.cuda.empty_cache()
