"""Trainer-inference invariance on the GPU, checked bit for bit.

The REINFORCE Zero pages rest on the learner and the rollout computing the
same logprob for the same weights and history ("diff 0", vLLM blog section 5;
"Remove kernel mismatch", project page section 02).  Here the same reference
rows are evaluated alone and inside batches of 1 .. 65536 rows, at random
slots and random row offsets, through both entry points, and every logprob
must be bitwise equal to its value computed alone.
"""
import numpy as np
import pytest

from invariant_token_logprobs_amd import synth
import invariant_token_logprobs_amd as rz

from gpu_util import (batch_to_dev, device, host, logmu_from_oracle,
                      mat_to_dev, run_fwd_bwd, say, small_batch, torch_mod,
                      vec_to_dev)

pytestmark = pytest.mark.gpu

H, V = 2560, synth.QWEN_VOCAB
N_REF = 4096


@pytest.fixture(scope="module")
def stress():
    torch = torch_mod()
    dev = device()
    head = mat_to_dev(synth.random_lm_head(V, H, "bf16", 3001), "bf16")
    ref_h, ref_tok = synth.random_rows(N_REF, H, V, "bf16", 3002)
    fill_h, fill_tok = synth.random_rows(65536 + 1024, H, V, "bf16", 3003)
    ref_h = mat_to_dev(ref_h, "bf16")
    ref_tok = vec_to_dev(ref_tok)
    fill_h = mat_to_dev(fill_h, "bf16")
    fill_tok = vec_to_dev(fill_tok)
    ws = rz.Workspace()
    # canonical values: every reference row alone (N = 1)
    canon = torch.empty(N_REF, dtype=torch.float32, device=dev)
    for i in range(N_REF):
        rz.token_logprobs(ref_h[i:i + 1], head, ref_tok[i:i + 1], workspace=ws,
                          out=canon[i:i + 1])
    torch.cuda.synchronize()
    say("stress: canonical N=1 values computed")
    return dict(head=head, ref_h=ref_h, ref_tok=ref_tok, fill_h=fill_h,
                fill_tok=fill_tok, canon=host(canon), ws=ws)


def _sizes():
    rng = np.random.default_rng(np.random.PCG64(5005))
    s = {1 << k for k in range(17)} | {3, 127, 129, 255, 257, 1000, 4095, 4097, 65535}
    s |= set(int(x) for x in rng.integers(2, 65536, size=8))
    return sorted(s)


def test_batch_invariance_stress(stress):
    torch = torch_mod()
    dev = device()
    rng = np.random.default_rng(np.random.PCG64(6006))
    head, ws = stress["head"], stress["ws"]
    buf_h = torch.empty((65536 + 1024, H), dtype=torch.bfloat16, device=dev)
    buf_t = torch.empty(65536 + 1024, dtype=torch.int32, device=dev)
    residues = np.zeros(256, dtype=bool)
    for N in _sizes():
        per = min(N_REF, (N + 1) // 2) if N < N_REF else N_REF
        order = rng.permutation(N_REF)
        got = np.full(N_REF, np.nan, dtype=np.float32)
        for b0 in range(0, N_REF, per):
            refs = order[b0:b0 + per]
            off = int(rng.integers(0, 1024))
            slots = np.sort(rng.choice(N, size=len(refs), replace=False))
            # filler everywhere, reference rows at their slots
            fsel = torch.from_numpy(rng.integers(0, 65536 + 1024, size=N)).to(dev)
            buf_h[off:off + N] = stress["fill_h"][fsel]
            buf_t[off:off + N] = stress["fill_tok"][fsel]
            sl = torch.from_numpy(off + slots).to(dev)
            rf = torch.from_numpy(refs).to(dev)
            buf_h[sl] = stress["ref_h"][rf]
            buf_t[sl] = stress["ref_tok"][rf]
            lp = rz.token_logprobs(buf_h[off:off + N], head, buf_t[off:off + N],
                                   workspace=ws)
            got[refs] = host(lp)[slots]
            residues[slots % 256] = True
        bad = np.flatnonzero(got.view(np.uint32) != stress["canon"].view(np.uint32))
        assert bad.size == 0, f"N={N}: {bad.size} reference rows differ, e.g. {bad[:4]}"
        # diagnostics over the gathered reference rows in canonical order
        lmu = vec_to_dev(stress["canon"] + np.float32(0.1))
        d_ref = host(rz.diagnostics(vec_to_dev(stress["canon"]), lmu))
        d_got = host(rz.diagnostics(vec_to_dev(got), lmu))
        assert np.array_equal(d_ref.view(np.uint32), d_got.view(np.uint32))
    say("stress: all sizes bitwise equal")
    assert residues.all(), "not every row residue mod 256 was exercised"


def test_learner_entry_point_matches_rollout(stress):
    """fwd_bwd's logprobs for the reference rows equal rz_token_logprobs
    bit for bit (diff 0 between the rollout and the learner call paths)."""
    torch = torch_mod()
    dev = device()
    rng = np.random.default_rng(np.random.PCG64(7007))
    n_ref = 1024
    N = 6000
    slots = np.sort(rng.choice(N, size=n_ref, replace=False))
    hidden = stress["fill_h"][:N].clone()
    tokens = stress["fill_tok"][:N].clone()
    sl = torch.from_numpy(slots).to(dev)
    hidden[sl] = stress["ref_h"][:n_ref]
    tokens[sl] = stress["ref_tok"][:n_ref]
    mask = np.ones(N, dtype=np.uint8)
    mask[rng.random(N) < 0.4] = 0
    mask[slots] = 1
    cu = np.array([0, 1000, 2500, 2600, 4000, 6000], dtype=np.int32)
    mask[cu[:-1]] = 1
    d = dict(hidden=hidden, lm_head=stress["head"], tokens=tokens,
             logmu=vec_to_dev(np.full(N, -12.0, np.float32)),
             mask=vec_to_dev(mask), cu_rows=vec_to_dev(cu),
             rewards=vec_to_dev(np.array([1, 0, 1, 0, 1], np.float32)),
             group_ids=vec_to_dev(np.array([0, 0, 1, 1, 1], np.int32)))
    out = run_fwd_bwd(d)
    lp = host(out["logprobs"])[slots]
    assert np.array_equal(lp.view(np.uint32), stress["canon"][:n_ref].view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeat_runs_are_bitwise_identical(dtype):
    b = small_batch(dtype=dtype, seed=21, N_resp=8, group_size=4)
    d = batch_to_dev(b, logmu_from_oracle(b))
    a = {k: host(v).copy() for k, v in run_fwd_bwd(d).items()}
    for _ in range(2):
        o = run_fwd_bwd(d)
        for k, v in a.items():
            assert np.array_equal(host(o[k]).view(np.uint32), v.view(np.uint32)), k


def test_unit_weights_give_exact_zero_diagnostics():
    """log mu set to the learner's own log pi: w = 1 exactly, so D3 and KL
    are exactly 0 and the loss is -(1/B) sum A_i = 0 up to rounding."""
    b = small_batch(dtype="bf16", seed=22)
    d = batch_to_dev(b, np.zeros(b.N, np.float32))
    lp = rz.token_logprobs(d["hidden"], d["lm_head"], d["tokens"])
    d["logmu"] = lp.clone()
    out = run_fwd_bwd(d)
    diag = host(out["diag"])
    assert diag[0] == 0.0 and diag[1] == 0.0
    assert abs(float(host(out["loss"])[0])) < 1e-7


def test_response_permutation_keeps_d_hidden_rows():
    """Moving whole responses around (same groups, same T_i and B) leaves
    each row's logprob and d_hidden row bit-identical."""
    torch = torch_mod()
    b = small_batch(dtype="bf16", seed=23, N_resp=6, group_size=3,
                    rewards="bernoulli")
    logmu = logmu_from_oracle(b)
    d = batch_to_dev(b, logmu)
    o1 = {k: host(v).copy() for k, v in run_fwd_bwd(d).items()}
    perm = np.array([3, 0, 5, 1, 4, 2])
    rows = np.concatenate([np.arange(b.cu_rows[i], b.cu_rows[i + 1]) for i in perm])
    lens = np.diff(b.cu_rows)[perm]
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    r = torch.from_numpy(rows).to(device())
    d2 = dict(hidden=d["hidden"][r].contiguous(), lm_head=d["lm_head"],
              tokens=d["tokens"][r].contiguous(), logmu=d["logmu"][r].contiguous(),
              mask=d["mask"][r].contiguous(), cu_rows=vec_to_dev(cu2),
              rewards=vec_to_dev(b.rewards[perm]),
              group_ids=vec_to_dev(b.group_ids[perm]))
    o2 = run_fwd_bwd(d2)
    assert np.array_equal(host(o2["logprobs"]).view(np.uint32),
                          o1["logprobs"][rows].view(np.uint32))
    assert np.array_equal(host(o2["d_hidden"]).view(np.uint32),
                          o1["d_hidden"][rows].view(np.uint32))
    assert np.array_equal(host(o2["adv"]), o1["adv"][perm])
