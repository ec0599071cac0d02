"""Run-level diagnostics on the GPU (rz_grad_norms, rz_response_diagnostics,
RunTracker over rz_run_summary) against the float64 oracle on the same
seeded inputs.

Tolerances: both kernels accumulate in float64 and round once to float32,
so they agree with the oracle to the float32 rounding of the result,
|gpu - oracle| <= 2^-23 |oracle| (one ulp, twice the rounding bound), plus,
for the signed KL sum, the float64 cancellation error 1e-13 * mean |d|.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import host, say, torch_mod, vec_to_dev

pytestmark = pytest.mark.gpu

ULP = 2.0 ** -23


def _dev_f32(x):
    return vec_to_dev(np.ascontiguousarray(x, dtype=np.float32))


def _norms(dh, dw):
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    out = rz.grad_norms(dh, dw)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


@pytest.mark.parametrize("N,H,V", [(1000, 320, 3001), (0, 64, 7), (3, 37, 5),
                                   (129, 2560, 1)])
def test_grad_norms_parity(N, H, V):
    """Several 65536-value chunks with a ragged tail, an empty d_hidden, H
    not a multiple of 4 (the scalar tail path), a one-row d_lm_head."""
    rng = np.random.default_rng(N + 7 * H + V)
    dh = (rng.standard_normal((N, H)) * 1e-3).astype(np.float32)
    dw = (rng.standard_normal((V, H)) * 3e-5).astype(np.float32)
    say("grad_norms", N, H, V)
    got = _norms(_dev_f32(dh).reshape(N, H), _dev_f32(dw).reshape(V, H))
    want = np.array(O.grad_norms(dh.astype(np.float64), dw.astype(np.float64)))
    assert np.all(np.abs(got - want) <= ULP * want), (got, want)
    again = _norms(_dev_f32(dh).reshape(N, H), _dev_f32(dw).reshape(V, H))
    assert np.array_equal(got, again)


def test_grad_norms_qwen3_4b_shape():
    """dL/dW at the Qwen3-4B head shape [151936, 2560] and dL/dhidden of a
    24576-row step, with a heavy-tailed magnitude mix (rows scaled by a
    lognormal factor, as the softmax rows of dW are)."""
    torch = torch_mod()
    V, H, N = 151936, 2560, 24576
    rng = np.random.default_rng(31)
    dw = rng.standard_normal((V, H), dtype=np.float32)
    dw *= rng.lognormal(-9.0, 2.0, size=(V, 1)).astype(np.float32)
    dh = rng.standard_normal((N, H), dtype=np.float32) * np.float32(1e-4)
    sq = 0.0
    for r0 in range(0, V, 8192):
        c = dw[r0:r0 + 8192].astype(np.float64)
        sq += float(np.einsum("ij,ij->", c, c))
    want_w = np.sqrt(sq)
    want_h = O.grad_norms(dh.astype(np.float64), np.zeros((1, H)))[0]
    say("grad_norms qwen3-4b shape")
    dwd = torch.from_numpy(dw).to("cuda:0")
    del dw
    dhd = torch.from_numpy(dh).to("cuda:0")
    got = _norms(dhd, dwd)
    assert abs(got[0] - want_h) <= ULP * want_h, (got[0], want_h)
    assert abs(got[1] - want_w) <= ULP * want_w, (got[1], want_w)
    del dwd, dhd
    torch.cuda.empty_cache()


def _resp_inputs(seed, B, lo, hi, masked=0.3, empty_every=0):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=B)
    if empty_every:
        lengths[::empty_every] = 0
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n = int(cu[-1])
    logpi = -rng.exponential(2.0, size=n)
    logmu = logpi + rng.normal(0.0, 0.05, size=n)
    mask = (rng.random(n) >= masked).astype(np.uint8)
    # one response with every row masked
    if B > 2 and lengths[1] > 0:
        mask[cu[1]:cu[2]] = 0
    return (logpi.astype(np.float32), logmu.astype(np.float32), mask, cu)


def _resp_gpu(logpi, logmu, mask, cu, err=None):
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    d3, kl = rz.response_diagnostics(
        _dev_f32(logpi), _dev_f32(logmu),
        None if mask is None else vec_to_dev(mask), vec_to_dev(cu), err_flag=err)
    torch.cuda.synchronize()
    return host(d3), host(kl)


def _check_resp(got, want, logpi, logmu, mask, cu, what):
    d3, kl = got
    wd3, wkl = want
    assert np.array_equal(np.isnan(d3), np.isnan(wd3)), what
    assert np.array_equal(np.isnan(kl), np.isnan(wkl)), what
    ok = ~np.isnan(wd3)
    d = np.abs(logpi.astype(np.float64) - logmu.astype(np.float64))
    scale = np.array([d[cu[i]:cu[i + 1]].mean() if cu[i + 1] > cu[i] else 0.0
                      for i in range(len(cu) - 1)])
    assert np.all(np.abs(d3[ok] - wd3[ok]) <= ULP * np.abs(wd3[ok])), what
    assert np.all(np.abs(kl[ok] - wkl[ok])
                  <= ULP * np.abs(wkl[ok]) + 1e-13 * scale[ok]), what


@pytest.mark.parametrize("B,lo,hi,masked,empty_every,use_mask", [
    (37, 1, 300, 0.3, 5, True),     # ragged, empty and all-masked responses
    (4, 2000, 5000, 0.1, 0, True),  # long responses: many rows per lane
    (9, 1, 70, 0.0, 0, False),      # mask = NULL
])
def test_response_diagnostics_parity(B, lo, hi, masked, empty_every, use_mask):
    logpi, logmu, mask, cu = _resp_inputs(B * 11 + lo, B, lo, hi, masked,
                                          empty_every)
    say("response_diagnostics", B, lo, hi, int(cu[-1]))
    got = _resp_gpu(logpi, logmu, mask if use_mask else None, cu)
    eff_mask = mask if use_mask else np.ones_like(mask)
    want = O.response_diagnostics(logpi.astype(np.float64),
                                  logmu.astype(np.float64), eff_mask, cu)
    _check_resp(got, want, logpi, logmu, eff_mask, cu, (B, lo, hi))


def test_response_diagnostics_position_invariance():
    """A response's values depend on its own rows only: bit-identical alone
    and at another offset inside a larger batch."""
    logpi, logmu, mask, cu = _resp_inputs(5, 12, 50, 900)
    d3, kl = _resp_gpu(logpi, logmu, mask, cu)
    for i in (0, 5, 11):
        r0, r1 = int(cu[i]), int(cu[i + 1])
        one = _resp_gpu(logpi[r0:r1], logmu[r0:r1], mask[r0:r1],
                        np.array([0, r1 - r0], np.int32))
        # shifted: 77 filler rows in front, as a response of its own
        pad = 77
        sp = np.concatenate([np.full(pad, -1.0, np.float32), logpi[r0:r1]])
        sm = np.concatenate([np.full(pad, -1.2, np.float32), logmu[r0:r1]])
        sk = np.concatenate([np.ones(pad, np.uint8), mask[r0:r1]])
        two = _resp_gpu(sp, sm, sk, np.array([0, pad, pad + r1 - r0], np.int32))
        for a, b in ((one[0][0], d3[i]), (one[1][0], kl[i]),
                     (two[0][1], d3[i]), (two[1][1], kl[i])):
            assert np.array_equal(np.float32(a).view(np.uint32),
                                  np.float32(b).view(np.uint32)), i


def test_response_diagnostics_bad_cu_rows():
    torch = torch_mod()
    logpi, logmu, mask, cu = _resp_inputs(3, 6, 5, 20)
    bad = cu.copy()
    bad[3] = bad[2] - 1              # response 2's range runs backwards
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    d3, kl = _resp_gpu(logpi, logmu, mask, bad, err=err)
    assert int(host(err)[0]) & 4
    assert np.isnan(d3[2]) and np.isnan(kl[2])
    want = O.response_diagnostics(logpi.astype(np.float64),
                                  logmu.astype(np.float64), mask, cu)
    for i in (0, 1, 4, 5):
        if not np.isnan(want[0][i]):
            assert abs(d3[i] - want[0][i]) <= ULP * abs(want[0][i])


def test_run_tracker_matches_the_oracle():
    """Per-step values recorded on the device (past the initial capacity)
    summarise exactly as the oracle's run_summary of the same values."""
    import invariant_token_logprobs_amd as rz
    torch = torch_mod()
    rng = np.random.default_rng(44)
    steps = 2600
    d3 = rng.gamma(0.5, 1e-3, size=steps).astype(np.float32)
    d3[1700] = 0.5                                   # one spike
    kl = np.abs(rng.normal(1e-4, 1e-4, size=steps)).astype(np.float32)
    g = rng.lognormal(0.0, 0.5, size=steps).astype(np.float32)
    dev_vals = _dev_f32(np.stack([d3, kl, g], axis=1).ravel()).reshape(steps, 3)
    tr = rz.RunTracker("cuda:0", window=1000, capacity=1000)
    for i in range(steps):
        tr.record(dev_vals[i, 0:2], dev_vals[i, 2:3])
    hd3, hkl, hg = tr.values()
    assert np.array_equal(hd3, d3) and np.array_equal(hkl, kl)
    assert np.array_equal(hg, g)
    got = tr.summary()
    want = O.run_summary(d3.astype(np.float64), kl.astype(np.float64),
                         g.astype(np.float64), window=1000)
    for k, v in want.items():
        assert got[k] == v, (k, got[k], v)
    assert got["steps"] == steps and got["rejected_sequences"] == 0
    del dev_vals
    torch.cuda.empty_cache()
