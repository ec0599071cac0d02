"""Device-detected input faults and degenerate batches.

Bad token ids, group ids and cu_rows set their err_flag bits and turn the
affected outputs into NaN, while every kernel still runs to completion
(the faults are fed from the host as ordinary data; no kernel traps).
"""
import math

import numpy as np
import pytest

import oracle as O
import invariant_token_logprobs_amd as rz

from gpu_util import (TOL, assert_close, batch_to_dev, host, logmu_from_oracle,
                      mat_to_dev, run_fwd_bwd, say, small_batch, torch_mod,
                      vec_to_dev)

pytestmark = pytest.mark.gpu


def _err():
    torch = torch_mod()
    return torch.zeros(1, dtype=torch.int32, device="cuda:0")


def test_bad_tokens_flag_and_nan_only_those_rows():
    b = small_batch(dtype="bf16", seed=31, N_resp=3, V=500, H=128)
    h = mat_to_dev(b.hidden, "bf16")
    W = mat_to_dev(b.lm_head, "bf16")
    clean = host(rz.token_logprobs(h, W, vec_to_dev(b.tokens)))
    tok = b.tokens.copy()
    bad = np.array([0, 17, len(tok) - 1])
    tok[bad] = np.array([500, -1, 1 << 30], dtype=np.int32)
    err = _err()
    lp = host(rz.token_logprobs(h, W, vec_to_dev(tok), err_flag=err))
    assert int(host(err)[0]) & rz.RZ_DEVERR_TOKEN
    assert np.isnan(lp[bad]).all()
    ok = np.setdiff1d(np.arange(len(tok)), bad)
    assert np.array_equal(lp[ok].view(np.uint32), clean[ok].view(np.uint32))


def test_bad_group_id_flags_and_nans_loss():
    b = small_batch(dtype="f32", seed=32, N_resp=4, group_size=2, V=300, H=64)
    d = batch_to_dev(b, logmu_from_oracle(b))
    d["group_ids"] = vec_to_dev(np.array([0, 1, 9, 1], np.int32))
    err = _err()
    out = run_fwd_bwd(d, err=err)
    assert int(host(err)[0]) & rz.RZ_DEVERR_GROUP
    assert math.isnan(float(host(out["loss"])[0]))
    assert np.isnan(host(out["adv"])).all()


@pytest.mark.parametrize("cu", [[0, 50, 40, None], [0, 50, 90, -7], [3, 50, 90, None]])
def test_bad_cu_rows_flags_and_nans_loss(cu):
    b = small_batch(dtype="f32", seed=33, N_resp=3, group_size=3, V=300, H=64)
    cu = [b.N if c is None else (b.N + c if c < 0 else c) for c in cu]
    d = batch_to_dev(b, logmu_from_oracle(b))
    d["cu_rows"] = vec_to_dev(np.array(cu, np.int32))
    err = _err()
    out = run_fwd_bwd(d, err=err)
    assert int(host(err)[0]) & rz.RZ_DEVERR_CU_ROWS
    assert math.isnan(float(host(out["loss"])[0]))


def test_all_rows_masked():
    torch = torch_mod()
    b = small_batch(dtype="bf16", seed=34, N_resp=3, V=300, H=64)
    b.mask[:] = 0
    d = batch_to_dev(b, np.zeros(b.N, np.float32))
    out = run_fwd_bwd(d)
    assert float(host(out["loss"])[0]) == 0.0
    assert not host(out["logprobs"]).any()
    assert not host(out["d_hidden"]).any()
    assert not host(out["d_lm_head"]).any()
    assert np.isnan(host(out["diag"])).all()
    assert_close(host(out["adv"]), O.group_mean_advantages(b.rewards, b.group_ids),
                 1e-6, 1e-7, "adv")


def test_empty_batch():
    torch = torch_mod()
    dev = "cuda:0"
    H, V, B = 64, 300, 2
    head = torch.randn(V, H, device=dev) * 0.02
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt, device=dev)
    out = rz.reinforce_zero_fwd_bwd(
        z(0, H), head, z(0, dt=torch.int32), z(0), z(0, dt=torch.uint8),
        vec_to_dev(np.zeros(B + 1, np.int32)),
        vec_to_dev(np.array([1, 0], np.float32)),
        vec_to_dev(np.array([0, 0], np.int32)))
    torch.cuda.synchronize()
    assert float(host(out["loss"])[0]) == 0.0
    assert not host(out["d_lm_head"]).any()
    assert np.isnan(host(out["diag"])).all()
    assert host(out["adv"]).tolist() == [0.5, -0.5]
    assert rz.token_logprobs(z(0, H), head, z(0, dt=torch.int32)).numel() == 0


def test_diagnostics_mask_and_empty():
    torch = torch_mod()
    rng = np.random.default_rng(np.random.PCG64(35))
    n = 10000
    lp = (-rng.random(n) * 10).astype(np.float32)
    mu = (lp + 0.1 * rng.standard_normal(n)).astype(np.float32)
    m = (rng.random(n) < 0.6).astype(np.uint8)
    got = host(rz.diagnostics(vec_to_dev(lp), vec_to_dev(mu), vec_to_dev(m)))
    d3, kl = O.diagnostics(lp.astype(np.float64), mu.astype(np.float64), m)
    assert_close(got, [d3, kl], 1e-5, 1e-9, "diag")
    got = host(rz.diagnostics(vec_to_dev(lp), vec_to_dev(mu)))
    d3, kl = O.diagnostics(lp.astype(np.float64), mu.astype(np.float64))
    assert_close(got, [d3, kl], 1e-5, 1e-9, "diag unmasked")
    e = host(rz.diagnostics(vec_to_dev(lp[:0]), vec_to_dev(mu[:0])))
    assert np.isnan(e).all()
