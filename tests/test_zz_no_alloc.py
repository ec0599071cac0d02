"""The allocation-free draw, rz_sample_tokens_noalloc, against the draw with
a caller's workspace, rz_sample_tokens, through the C ABI.

Both run the same kernels, so tokens, recorded log mu and lse must agree bit
for bit.  Two calls in a row (the second with fewer rows, so the static
scratch still holds the first call's contents) at the Qwen3-4B head, an fp32
head, and sizes past the static scratch rejected before any GPU work."""
import ctypes

import numpy as np
import pytest

import invariant_token_logprobs_amd as rz
from invariant_token_logprobs_amd import synth


def _noalloc_status(n, H, V, dt):
    lib = rz.load_library()
    P = ctypes.c_void_p(0x1000)
    return lib.rz_sample_tokens_noalloc(P, P, P, n, H, V, dt, ctypes.c_uint64(1), P, P,
                                        None, None)


def test_sizes_past_the_static_scratch_are_rejected():
    # no GPU work: the size check comes before any HIP call (fake pointers)
    V, H = synth.QWEN_VOCAB, 2560
    per_row = rz.workspace_bytes(rz.RZ_OP_SAMPLE, 1000, 1, H, V, rz.RZ_DTYPE_BF16) / 1000
    too_many = int(rz.RZ_NOALLOC_SCRATCH_BYTES / per_row) + 50
    assert _noalloc_status(too_many, H, V, rz.RZ_DTYPE_BF16) == -5     # RZ_ERR_SCRATCH
    assert _noalloc_status(4, 100, V, rz.RZ_DTYPE_BF16) == -2          # H % 64 != 0
    assert _noalloc_status(-1, H, V, rz.RZ_DTYPE_BF16) == -1


def _compare(hidden, lm_head, ids, seed, what):
    import torch
    t_ref, mu_ref, lse_ref = rz.sample_tokens(hidden, lm_head, ids, seed, want_lse=True)
    t, mu, lse = rz.sample_tokens_noalloc(hidden, lm_head, ids, seed, want_lse=True)
    torch.cuda.synchronize()
    print(f"[gpu-test] {what}: n={hidden.shape[0]}", flush=True)
    assert torch.equal(t, t_ref), f"{what}: tokens differ"
    assert torch.equal(mu, mu_ref), f"{what}: log mu differs"
    assert torch.equal(lse, lse_ref), f"{what}: lse differs"


@pytest.mark.gpu
def test_noalloc_draw_matches_the_workspace_draw():
    import torch
    dev = torch.device("cuda:0")
    V, H = synth.QWEN_VOCAB, 2560
    W = torch.from_numpy(synth.random_lm_head(V, H, "bf16", 301).view(np.int16)).view(
        torch.bfloat16).to(dev)
    # the largest row count the static scratch holds at this head
    per_row = rz.workspace_bytes(rz.RZ_OP_SAMPLE, 1000, 1, H, V, rz.RZ_DTYPE_BF16) / 1000
    n_max = int(rz.RZ_NOALLOC_SCRATCH_BYTES / per_row) - 8
    assert rz.workspace_bytes(rz.RZ_OP_SAMPLE, n_max, 1, H, V,
                              rz.RZ_DTYPE_BF16) <= rz.RZ_NOALLOC_SCRATCH_BYTES
    hid, _ = synth.random_rows(n_max, H, V, "bf16", 302)
    hidden = torch.from_numpy(hid.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.arange(10_000, 10_000 + n_max, dtype=torch.int64, device=dev)
    # the largest row count that fits, then fewer rows over the same scratch
    for n in (n_max, 300, 37):
        _compare(hidden[:n], W, ids[:n], 77, f"noalloc-bf16-{n}")
    # fp32 head, two calls in a row
    Wf = torch.from_numpy(synth.random_lm_head(1000, 256, "f32", 303)).to(dev)
    hf, _ = synth.random_rows(500, 256, 1000, "f32", 304)
    hf = torch.from_numpy(hf).to(dev)
    idf = torch.arange(500, dtype=torch.int64, device=dev)
    _compare(hf, Wf, idf, 5, "noalloc-f32-500")
    _compare(hf[:65], Wf, idf[:65], 5, "noalloc-f32-65")
