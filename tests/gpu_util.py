"""Shared helpers of the GPU tests: host arrays -> device tensors, the
tolerances, and the stand-in behaviour policy used to draw log mu.

Tolerances (per element, |gpu - oracle| <= atol + rtol * |oracle|):
* logprobs: bf16 rtol 2e-3 / atol 1e-4, fp32 rtol 1e-5 / atol 1e-5;
* gradients: normwise ||gpu - oracle|| / ||oracle|| <= rtol, and per element
  fp32: |gpu - oracle| <= 1e-5 * max|oracle| + cbound + rtol * |oracle|;
  bf16: the softmax part of dL/dz is quantized to bf16 before the GEMMs
  (unit roundoff u = 2^-8; the stored exp(z - m_tile) adds at most 2^-11),
  so the forward-error bound of each element is 2u * (|G_s| |W|)[t, h] for
  dL/dhidden and 2u * (|G_s|^T |h|)[v, h] for dL/dW, G_s = c_t softmax(z_t)
  (the row's own token column, c_t (p[a_t] - 1), is applied exactly in fp32,
  so this bound is conservative there); per element
  |gpu - oracle| <= 2u * bound + cbound + 1e-6 * max|oracle| + rtol * |oracle|.
  cbound carries the logprob error into the gradients: c_t = A_i w_t / (B T_i)
  is computed from the kernel's own log pi_t, so a logprob off by d_t (the
  measured gpu - oracle difference, itself checked against the logprob
  tolerance) scales row t's whole dL/dz, one-hot part included, by
  exp(d_t): cbound = (|G_c| |W|)[t, h] and (|G_c|^T |h|)[v, h] with
  G_c = |expm1(d_t)| |c_t| (softmax(z_t) + onehot(a_t)).  Where one-hot
  terms of several rows cancel in an element of dL/dW, this is the whole
  error.  Normwise, ||gpu - oracle|| <= rtol ||oracle|| + ||cbound||.
* scalars: the loss, D3 and KL are sums of many terms whose inputs
  (the logprobs) already carry the logprob tolerance, so their tolerance is
  propagated from it: |dL| <= sum_i |A_i| / (B T_i) sum_t w_t tol_t,
  |dKL| <= mean tol_t, |dD3| <= mean |w_t - 1| tol_t, plus rtol * |value|.
"""
import os

import numpy as np
import pytest

import oracle as O
from invariant_token_logprobs_amd import synth

TOL = {"bf16": dict(rtol=2e-3, atol=1e-4, gscale=1e-4),
       "f32": dict(rtol=1e-5, atol=1e-5, gscale=1e-5)}


def torch_mod():
    import torch
    return torch


def device():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch.device("cuda:0")


def say(*a):
    print("[gpu-test]", *a, flush=True)


def mat_to_dev(x: np.ndarray, dtype: str):
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device())


def vec_to_dev(x: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x)).to(device())


def batch_to_dev(b: synth.Batch, logmu: np.ndarray) -> dict:
    return dict(hidden=mat_to_dev(b.hidden, b.dtype),
                lm_head=mat_to_dev(b.lm_head, b.dtype),
                tokens=vec_to_dev(b.tokens.astype(np.int32)),
                logmu=vec_to_dev(logmu.astype(np.float32)),
                mask=vec_to_dev(b.mask.astype(np.uint8)),
                cu_rows=vec_to_dev(b.cu_rows.astype(np.int32)),
                rewards=vec_to_dev(b.rewards.astype(np.float32)),
                group_ids=vec_to_dev(b.group_ids.astype(np.int32)))


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def behaviour_logprobs_torch(hidden, lm_head, tokens, rows_per_chunk=2048):
    """Stand-in rollout policy for drawing log mu at sizes the oracle cannot
    finish: a plain torch fp32 log-softmax on the GPU (an independent third
    implementation, never our kernels).  Only used to place log mu near
    log pi; nothing is compared against it."""
    torch = torch_mod()
    Wf = lm_head.float().t().contiguous()
    out = torch.empty(hidden.shape[0], dtype=torch.float32, device=hidden.device)
    for r0 in range(0, hidden.shape[0], rows_per_chunk):
        r1 = min(hidden.shape[0], r0 + rows_per_chunk)
        z = hidden[r0:r1].float() @ Wf
        lp = torch.log_softmax(z, dim=1)
        out[r0:r1] = lp.gather(1, tokens[r0:r1].long()[:, None])[:, 0]
    del Wf
    return out


def assert_close(got, want, rtol, atol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; first "
            f"{i.tolist()} got {got.ravel()[i].tolist()} want {want.ravel()[i].tolist()}")


U_BF16 = 2.0 ** -8


def softmax_grad_bounds(hidden64, W64, lse, coef, row_chunk=256, tokens=None,
                        dlogpi=None):
    """(|G_s| |W|, |G_s|^T |h|) with G_s = |c_t| exp(z - lse_t): the
    magnitudes the bf16 dlogits quantization error scales with.  Given the
    tokens and the measured logprob errors dlogpi, also the propagated
    coefficient-error bounds (|G_c| |W|, |G_c|^T |h|) with
    G_c = |expm1(dlogpi_t)| |c_t| (softmax(z_t) + onehot(a_t))."""
    n, H = hidden64.shape
    bh = np.zeros((n, H))
    bw = np.zeros((W64.shape[0], H))
    with_c = dlogpi is not None
    if with_c:
        ch = np.zeros((n, H))
        cw = np.zeros((W64.shape[0], H))
        fac = np.abs(np.expm1(np.asarray(dlogpi, np.float64)))
        fac = np.where(np.isfinite(fac), fac, 0.0)
    aW, ah = np.abs(W64), np.abs(hidden64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        P = np.exp(hidden64[r0:r1] @ W64.T - lse[r0:r1, None])
        G = np.abs(coef[r0:r1, None]) * P
        bh[r0:r1] = G @ aW
        bw += G.T @ ah[r0:r1]
        if with_c:
            P[np.arange(r1 - r0), np.asarray(tokens)[r0:r1]] += 1.0
            Gc = (fac[r0:r1] * np.abs(coef[r0:r1]))[:, None] * P
            ch[r0:r1] = Gc @ aW
            cw += Gc.T @ ah[r0:r1]
    if with_c:
        return bh, bw, ch, cw
    return bh, bw


def report_grad_error(got, want, what):
    """Print the worst per-element error of a gradient in units of
    max|oracle| (the plain per-element bound of 1e-4 times the output's
    largest magnitude)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    if not fin.any():
        return
    scale = float(np.abs(want[fin]).max())
    if scale > 0:
        worst = float(np.abs(got[fin] - want[fin]).max()) / scale
        say(f"{what}: worst |gpu - oracle| / max|oracle| = {worst:.3e} (plain bound 1e-4)")


def assert_grad_close(got, want, dtype, what, bound=None, cbound=None):
    t = TOL[dtype]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    report_grad_error(got, want, what)
    scale = float(np.abs(want).max()) if want.size else 0.0
    if dtype == "bf16" and bound is not None:
        atol = 2 * U_BF16 * np.asarray(bound) + 1e-6 * scale
    else:
        atol = t["gscale"] * scale
    if cbound is not None:
        atol = atol + np.asarray(cbound)
    assert_close(got, want, t["rtol"], atol, what)
    nw = np.linalg.norm(want)
    if nw > 0:
        # the propagated coefficient error bounds each element, so its norm
        # bounds that part of the error's norm
        nc = float(np.linalg.norm(cbound)) if cbound is not None else 0.0
        err = np.linalg.norm(got - want)
        assert err <= t["rtol"] * nw + nc, (
            f"{what}: normwise relative error {err / nw:.3e} "
            f"(allowed {t['rtol']:.1e} + {nc / nw:.2e} from the logprobs)")


def scalar_tols(ref: dict, mask, cu_rows, dtype):
    """Propagated absolute tolerances of (loss, D3, KL) from the logprob
    tolerance, evaluated on the oracle's values."""
    t = TOL[dtype]
    valid = np.asarray(mask) != 0
    lp = ref["logpi"]
    tol = t["atol"] + t["rtol"] * np.abs(lp)
    w = ref["w"]
    B = len(cu_rows) - 1
    T = ref["T"]
    A = ref["adv"]
    loss_tol = 0.0
    for i in range(B):
        if T[i] == 0:
            continue
        rows = slice(cu_rows[i], cu_rows[i + 1])
        loss_tol += abs(A[i]) / (B * T[i]) * float(np.sum((w[rows] * tol[rows])[valid[rows]]))
    nv = max(1, int(valid.sum()))
    kl_tol = float(np.sum(tol[valid])) / nv
    d3_tol = float(np.sum((np.abs(w - 1) * tol)[valid])) / nv
    return loss_tol, d3_tol, kl_tol


def oracle_full(b: synth.Batch, logmu):
    return O.reinforce_zero_fwd_bwd(
        O.to_f64(b.hidden, b.dtype), O.to_f64(b.lm_head, b.dtype), b.tokens,
        np.asarray(logmu, np.float64), b.mask, b.cu_rows, b.rewards,
        b.group_ids)


def logmu_from_oracle(b: synth.Batch):
    logpi, _ = O.token_logprobs(O.to_f64(b.hidden, b.dtype),
                                O.to_f64(b.lm_head, b.dtype), b.tokens)
    return synth.make_logmu(logpi, b.sigma, b.noise_seed)


def small_batch(*, N_resp=6, group_size=3, H=256, V=1000, lo=40, hi=200,
                dtype="bf16", masked=0.3, seed=7, sigma=0.05,
                rewards="uniform", shuffle_groups=True) -> synth.Batch:
    """A seeded batch at oracle-friendly sizes with ragged tails."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    lengths = rng.integers(lo, hi + 1, size=N_resp)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = int(cu[-1])
    mask = np.ones(N, dtype=np.uint8)
    if masked > 0:
        mask[rng.random(N) < masked] = 0
        mask[cu[:-1]] = 1
    if rewards == "uniform":
        r = rng.random(N_resp, dtype=np.float32)
    else:
        r = rng.integers(0, 2, size=N_resp).astype(np.float32)
    gids = (np.arange(N_resp) // group_size).astype(np.int32)
    if shuffle_groups:
        gids = rng.permutation(gids).astype(np.int32)
    hidden, tokens = synth.random_rows(N, H, V, dtype, seed + 1)
    head = synth.random_lm_head(V, H, dtype, seed + 2)
    return synth.Batch("small", dtype, H, V, hidden, head, tokens, mask, cu, r,
                       gids, sigma, seed + 3)


def run_fwd_bwd(d: dict, err=None, workspace=None):
    import invariant_token_logprobs_amd as rz
    out = rz.reinforce_zero_fwd_bwd(d["hidden"], d["lm_head"], d["tokens"],
                                    d["logmu"], d["mask"], d["cu_rows"],
                                    d["rewards"], d["group_ids"], err_flag=err,
                                    workspace=workspace)
    torch_mod().cuda.synchronize()
    return out


def compare_full(out: dict, ref: dict, b: synth.Batch, what: str):
    """Element-by-element comparison of every fwd_bwd output."""
    t = TOL[b.dtype]
    valid = b.mask != 0
    lp = host(out["logprobs"])
    assert np.all(lp[~valid] == 0.0), f"{what}: masked logprobs not 0"
    assert_close(lp[valid], ref["logpi"][valid], t["rtol"], t["atol"],
                 f"{what} logprobs")
    assert_close(host(out["adv"]), ref["adv"], 1e-6, 1e-7, f"{what} adv")
    lt, dt3, dkl = scalar_tols(ref, b.mask, b.cu_rows, b.dtype)
    diag = host(out["diag"])
    assert_close([float(host(out["loss"])[0])], [ref["loss"]], t["rtol"], 1e-7 + lt,
                 f"{what} loss")
    assert_close([diag[0]], [ref["d3"]], t["rtol"], 1e-7 + dt3, f"{what} D3")
    assert_close([diag[1]], [ref["kl"]], t["rtol"], 1e-7 + dkl, f"{what} KL")
    dh = host(out["d_hidden"])
    assert np.all(dh[~valid] == 0.0), f"{what}: masked d_hidden rows not 0"
    dlp = np.where(valid, lp.astype(np.float64) - ref["logpi"], 0.0)
    bh, bw, ch, cw = softmax_grad_bounds(O.to_f64(b.hidden, b.dtype),
                                         O.to_f64(b.lm_head, b.dtype), ref["lse"],
                                         ref["coef"], tokens=b.tokens, dlogpi=dlp)
    if b.dtype != "bf16":
        bh = bw = None
    assert_grad_close(dh, ref["d_hidden"], b.dtype, f"{what} d_hidden", bh, ch)
    assert_grad_close(host(out["d_lm_head"]), ref["d_lm_head"], b.dtype,
                      f"{what} d_lm_head", bw, cw)
