"""The C ABI without a GPU: the library loads, exports every function that
include/rz.h declares, and rejects bad host-visible arguments with the
documented status before making any HIP call."""
import ctypes
import os
import re

import pytest

import invariant_token_logprobs_amd as rz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rz.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
F32, BF16 = rz.RZ_DTYPE_F32, rz.RZ_DTYPE_BF16


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rz.library_path()):
        pytest.fail("librz.so is not built (python -m invariant_token_logprobs_amd.build)")
    return rz.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rz_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rz_token_logprobs", "rz_reinforce_zero_fwd_bwd", "rz_diagnostics",
              "rz_workspace_bytes", "rz_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(rz.EXPORTS) == declared_functions()


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, 17):
        assert lib.rz_status_string(code)


# fake device pointers: never dereferenced, the calls must fail before HIP
P = ctypes.c_void_p(0x1000)
NULL = None


def tlp(lib, hidden=P, head=P, tokens=P, n=4, H=64, V=10, dt=BF16, out=P,
        ws=P, ws_bytes=0):
    return lib.rz_token_logprobs(hidden, head, tokens, n, H, V, dt, out, NULL,
                                 NULL, ws, ws_bytes, NULL)


def test_token_logprobs_argument_errors(lib):
    assert tlp(lib, n=-1) == INVALID
    assert tlp(lib, H=0) == INVALID
    assert tlp(lib, V=0) == INVALID
    assert tlp(lib, H=96) == UNSUPPORTED          # not a multiple of 64
    assert tlp(lib, dt=7) == UNSUPPORTED
    assert tlp(lib, V=1 << 25) == UNSUPPORTED
    assert tlp(lib, hidden=NULL) == INVALID
    assert tlp(lib, tokens=NULL) == INVALID
    assert tlp(lib, out=NULL) == INVALID
    assert tlp(lib, ws=NULL, ws_bytes=1 << 30) == WORKSPACE
    need = lib.rz_workspace_bytes_op(0, 4, 1, 64, 10, BF16)
    assert need > 0
    assert tlp(lib, ws_bytes=need - 1) == WORKSPACE
    assert tlp(lib, ws=ctypes.c_void_p(0x1001), ws_bytes=need) == WORKSPACE
    assert tlp(lib, n=0) == OK                    # empty call: no work at all


def fb(lib, n=8, B=2, H=64, V=10, dt=F32, ws=P, ws_bytes=0, **null):
    args = dict(hidden=P, head=P, tokens=P, logmu=P, mask=P, cu=P, rewards=P,
                gid=P, logprobs=P, loss=P, dh=P, dw=P)
    for k in null:
        args[k] = NULL
    a = args
    return lib.rz_reinforce_zero_fwd_bwd(
        a["hidden"], a["head"], a["tokens"], a["logmu"], a["mask"], a["cu"],
        a["rewards"], a["gid"], n, B, H, V, dt, a["logprobs"], a["loss"],
        a["dh"], a["dw"], NULL, NULL, NULL, ws, ws_bytes, NULL)


def test_fwd_bwd_argument_errors(lib):
    assert fb(lib, n=-5) == INVALID
    assert fb(lib, B=0) == INVALID
    assert fb(lib, H=-64) == INVALID
    assert fb(lib, H=100) == UNSUPPORTED
    assert fb(lib, dt=3) == UNSUPPORTED
    for name in ("hidden", "head", "tokens", "logmu", "mask", "cu", "rewards",
                 "gid", "logprobs", "loss", "dh", "dw"):
        assert fb(lib, **{name: True}) == INVALID, name
    need = lib.rz_workspace_bytes_op(1, 8, 2, 64, 10, F32)
    assert need > 0
    assert fb(lib, ws=NULL, ws_bytes=need) == WORKSPACE
    assert fb(lib, ws_bytes=need - 1) == WORKSPACE


def test_diagnostics_argument_errors(lib):
    f = lib.rz_diagnostics
    assert f(P, P, NULL, -1, P, P, 1 << 20, NULL) == INVALID
    assert f(P, P, NULL, 10, NULL, P, 1 << 20, NULL) == INVALID
    assert f(NULL, P, NULL, 10, P, P, 1 << 20, NULL) == INVALID
    assert f(P, P, NULL, 10, P, NULL, 0, NULL) == WORKSPACE


def test_workspace_sizes(lib):
    ws = lib.rz_workspace_bytes_op
    assert ws(0, -1, 1, 64, 10, F32) == 0
    assert ws(0, 10, 1, 65, 10, F32) == 0
    assert ws(1, 10, 0, 64, 10, F32) == 0
    assert ws(0, 0, 1, 64, 10, F32) == 0
    a = ws(1, 1000, 4, 256, 1024, F32)
    b = ws(1, 2000, 4, 256, 1024, F32)
    assert 0 < a < b
    assert ws(1, 1000, 4, 256, 1024, BF16) < a
    for op in (0, 1, 2):
        assert ws(op, 12345, 7, 2560, 151936, BF16) % 256 == 0
    # the headline tool-use workload fits comfortably in one MI355X's HBM
    assert ws(1, 295658, 32, 2560, 151936, BF16) < 40 * 2 ** 30


def test_common_workspace_query_serves_the_three_calls(lib):
    """rz_workspace_bytes(n_rows, n_resp, H, V, dt) is one size for
    rz_token_logprobs, rz_reinforce_zero_fwd_bwd and rz_diagnostics: the
    largest of their own needs."""
    ws_op = lib.rz_workspace_bytes_op
    for (n, B, H, V, dt) in ((1000, 4, 256, 1024, F32), (295658, 32, 2560, 151936, BF16),
                             (0, 1, 64, 10, BF16), (7, 3, 128, 777, F32)):
        need = [ws_op(op, n, B, H, V, dt) for op in (0, 1, 2)]
        assert lib.rz_workspace_bytes(n, B, H, V, dt) == max(need)
        assert ws_op(rz.RZ_OP_SCORE_CENTERING, n, B, H, V, dt) == need[1]
    # an invalid n_resp leaves the learner step out, not the other two
    assert lib.rz_workspace_bytes(100, 0, 64, 10, F32) == max(
        ws_op(0, 100, 1, 64, 10, F32), ws_op(2, 100, 1, 64, 10, F32))
    assert lib.rz_workspace_bytes(-1, 1, 64, 10, F32) == 0
    assert ws_op(1, 10, (1 << 24) + 1, 64, 10, F32) == 0


def sc(lib, n=8, B=2, H=64, V=10, dt=F32, ws=P, ws_bytes=0, diag=NULL, **null):
    args = dict(hidden=P, head=P, tokens=P, logmu=P, mask=P, cu=P, rewards=P,
                gid=P, logprobs=P, loss=P, dh=P, dw=P)
    for k in null:
        args[k] = NULL
    a = args
    return lib.rz_score_centering_fwd_bwd(
        a["hidden"], a["head"], a["tokens"], a["logmu"], a["mask"], a["cu"],
        a["rewards"], a["gid"], n, B, H, V, dt, a["logprobs"], a["loss"],
        a["dh"], a["dw"], diag, NULL, NULL, ws, ws_bytes, NULL)


def test_score_centering_argument_errors(lib):
    assert sc(lib, n=-5) == INVALID
    assert sc(lib, B=0) == INVALID
    assert sc(lib, H=100) == UNSUPPORTED
    for name in ("hidden", "head", "tokens", "mask", "cu", "rewards", "gid",
                 "logprobs", "loss", "dh", "dw"):
        assert sc(lib, **{name: True}) == INVALID, name
    need = lib.rz_workspace_bytes_op(rz.RZ_OP_SCORE_CENTERING, 8, 2, 64, 10, F32)
    # log mu is optional: without it the call gets as far as the workspace
    # check, but then it cannot report D3 / KL
    assert sc(lib, logmu=True, ws=NULL, ws_bytes=need) == WORKSPACE
    assert sc(lib, logmu=True, diag=P, ws_bytes=need) == INVALID
    assert sc(lib, ws_bytes=need - 1) == WORKSPACE


def test_timer_without_gpu_work(lib):
    rz.timing_enable(True)
    t = rz.timing_read()
    assert "fwd_logits_gemm" in t and all(v == (0.0, 0) for v in t.values())
    rz.timing_enable(False)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    h = torch.zeros(4, 64)
    with pytest.raises(rz.RzError):
        rz.token_logprobs(h, torch.zeros(10, 64), torch.zeros(4, dtype=torch.int32))


def test_product_path_never_loads_the_oracle():
    """The package, its binding and the input generators work without the
    oracle: importing them (and calling every binding entry that needs no
    GPU) must not pull oracle/ in, and no package source imports it."""
    import pathlib
    import subprocess
    import sys
    code = (
        "import sys\n"
        "import invariant_token_logprobs_amd as rz\n"
        "from invariant_token_logprobs_amd import synth, binding\n"
        "rz.load_library(); rz.workspace_bytes(rz.RZ_OP_FWD_BWD, 64, 2, 64, 100, rz.RZ_DTYPE_BF16)\n"
        "synth.make_workload('tiny')\n"
        "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), "
        "sorted(m for m in sys.modules if 'oracle' in m)\n")
    root = pathlib.Path(__file__).resolve().parents[1]
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    for src in (root / "invariant_token_logprobs_amd").rglob("*.py"):
        text = src.read_text()
        assert "import oracle" not in text and "from oracle" not in text, src


def smp(lib, n=4, H=64, V=10, dt=BF16, seed=1, ws=P, ws_bytes=0, **null):
    args = dict(hidden=P, head=P, ids=P, tokens=P, logmu=P)
    for k in null:
        args[k] = NULL
    a = args
    return lib.rz_sample_tokens(a["hidden"], a["head"], a["ids"], n, H, V, dt,
                                ctypes.c_uint64(seed), a["tokens"], a["logmu"],
                                NULL, ws, ws_bytes, NULL)


def test_sample_tokens_argument_errors(lib):
    assert smp(lib, n=-1) == INVALID
    assert smp(lib, H=0) == INVALID
    assert smp(lib, V=0) == INVALID
    assert smp(lib, H=96) == UNSUPPORTED
    assert smp(lib, dt=5) == UNSUPPORTED
    for name in ("hidden", "head", "ids", "tokens", "logmu"):
        assert smp(lib, **{name: True}) == INVALID, name
    need = lib.rz_workspace_bytes_op(rz.RZ_OP_SAMPLE, 4, 1, 64, 10, BF16)
    assert need > 0 and need % 256 == 0
    assert smp(lib, ws=NULL, ws_bytes=need) == WORKSPACE
    assert smp(lib, ws_bytes=need - 1) == WORKSPACE
    assert smp(lib, n=0) == OK
    # per (row, 128-column statistics tile): the (m, s) partial, the draw
    # candidate (score, index) and its logit
    nt = (151936 + 127) // 128
    big = lib.rz_workspace_bytes_op(rz.RZ_OP_SAMPLE, 4096, 1, 2560, 151936, BF16)
    assert big >= (8 + 8 + 4) * nt * 4096


# ----------------------------------------------------- run-level diagnostics
def test_grad_norms_argument_errors(lib):
    ws_need = rz.workspace_bytes(rz.RZ_OP_GRAD_NORMS, 100, 0, 64, 1000, 0)
    assert ws_need > 0
    assert rz.workspace_bytes(rz.RZ_OP_GRAD_NORMS, 100, 0, 0, 1000, 0) == 0
    out = P
    def gn(dh=P, n=100, H=64, dw=P, V=1000, o=out, ws=P, wsb=ws_need):
        return lib.rz_grad_norms(dh, n, H, dw, V, o, ws, wsb, NULL)
    assert gn(n=-1) == INVALID
    assert gn(H=0) == INVALID
    assert gn(V=0) == INVALID
    assert gn(o=NULL) == INVALID
    assert gn(dw=NULL) == INVALID
    assert gn(dh=NULL) == INVALID
    assert gn(dh=ctypes.c_void_p(0x1004)) == INVALID       # not 16-byte aligned
    assert gn(ws=NULL) == WORKSPACE
    assert gn(wsb=ws_need - 1) == WORKSPACE
    assert gn(ws=ctypes.c_void_p(0x1010)) == WORKSPACE     # not 256-byte aligned


def test_response_diagnostics_argument_errors(lib):
    def rd(lp=P, lm=P, cu=P, n=10, B=2, d3=P, kl=P):
        return lib.rz_response_diagnostics(lp, lm, NULL, cu, n, B, d3, kl, NULL, NULL)
    assert rd(n=-1) == INVALID
    assert rd(B=-1) == INVALID
    assert rd(B=0) == OK                                     # no-op, no launch
    assert rd(cu=NULL) == INVALID
    assert rd(d3=NULL) == INVALID
    assert rd(kl=NULL) == INVALID
    assert rd(lp=NULL) == INVALID


def test_run_summary_matches_the_oracle():
    """rz_run_summary is host code: exact agreement with the oracle on the
    same float32 values (odd and even counts, windows longer than the run,
    zero medians, NaN steps, missing arrays)."""
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(12)
    cases = []
    for n in (1, 2, 3, 10, 999, 1000, 2501):
        d3 = rng.gamma(0.5, 1e-3, size=n).astype(np.float32)
        kl = rng.normal(1e-4, 1e-3, size=n).astype(np.float32)
        g = rng.lognormal(0.0, 1.0, size=n).astype(np.float32)
        for window in (1, 7, 1000):
            cases.append((d3, kl, g, window))
    z = np.zeros(6, np.float32)
    cases.append((z, z, z, 3))
    cases.append((np.array([0.1, np.nan, 0.3], np.float32),
                  np.array([1.0, 2.0, 4.0], np.float32),
                  np.array([np.nan, 1.0, 2.0], np.float32), 2))
    for d3, kl, g, window in cases:
        got = rz.run_summary(d3, kl, g, window)
        want = O.run_summary(d3.astype(np.float64), kl.astype(np.float64),
                             g.astype(np.float64), window)
        for k in rz.RUN_SUMMARY_KEYS:
            a, b = got[k], want[k]
            assert (np.isnan(a) and np.isnan(b)) or a == b, (len(d3), window, k, a, b)
    empty = rz.run_summary(None, None, None)
    assert all(np.isnan(v) for v in empty.values())
    with pytest.raises(rz.RzError):
        rz.run_summary([1.0], [1.0], [1.0], window=0)
    with pytest.raises(rz.RzError):
        rz.run_summary([1.0, 2.0], [1.0], [1.0])


def test_dequantize_head_argument_errors(lib):
    def dq(codes=P, scales=P, V=10, H=64, fmt=0, out=P):
        return lib.rz_dequantize_head(codes, scales, V, H, fmt, out, NULL, NULL)
    assert dq(fmt=2) == UNSUPPORTED
    assert dq(V=0) == INVALID
    assert dq(H=48) == INVALID                         # not a multiple of 32
    assert dq(H=0) == INVALID
    assert dq(codes=NULL) == INVALID
    assert dq(scales=NULL) == INVALID
    assert dq(out=NULL) == INVALID
    assert dq(codes=ctypes.c_void_p(0x1008)) == INVALID   # not 16-byte aligned
    assert dq(out=ctypes.c_void_p(0x1002)) == INVALID


def test_random_mx_head_is_valid_storage():
    """The generator's heads decode (oracle) to finite weights near 0.02."""
    import numpy as np
    import oracle as O
    from invariant_token_logprobs_amd import synth
    for fmt in ("mxfp4", "mxfp8"):
        codes, scales = synth.random_mx_head(64, 128, fmt, 5)
        W = O.dequantize_head(codes, scales, fmt)
        assert W.shape == (64, 128) and np.isfinite(W).all()
        assert 0.003 < W.std() < 0.1, (fmt, W.std())


def test_lora_argument_errors(lib):
    f = ctypes.c_float(0.5)
    def aug(h=P, A=P, n=10, H=64, r=8, dt=BF16, out=P):
        return lib.rz_lora_augment(h, A, f, n, H, r, dt, out, NULL)
    assert aug(r=0) == INVALID and aug(r=65) == INVALID
    assert aug(H=48) == UNSUPPORTED and aug(dt=7) == UNSUPPORTED
    assert aug(n=-1) == INVALID
    assert aug(n=0) == OK                               # nothing to do
    assert aug(h=NULL) == INVALID and aug(out=NULL) == INVALID
    def merge(W=P, B=P, V=10, H=64, r=8, dt=BF16, out=P):
        return lib.rz_lora_merge_head(W, B, V, H, r, dt, out, NULL)
    assert merge(r=0) == INVALID and merge(V=0) == UNSUPPORTED
    assert merge(B=NULL) == INVALID
    nb = rz.workspace_bytes(rz.RZ_OP_FWD_BWD_LORA, 10, 2, 64, 10, BF16)
    assert nb > rz.workspace_bytes(rz.RZ_OP_FWD_BWD, 10, 2, 64, 10, BF16)
    def fb(r=8, ws=P, wsb=nb, dA=P):
        return lib.rz_reinforce_zero_fwd_bwd_lora(
            P, P, P, P, f, r, P, P, P, P, P, P, 10, 2, 64, 10, BF16, P, P, P, dA, P,
            NULL, NULL, NULL, ws, wsb, NULL)
    assert fb(r=0) == INVALID and fb(r=65) == INVALID
    assert fb(dA=NULL) == INVALID
    assert fb(ws=NULL) == WORKSPACE and fb(wsb=nb - 1) == WORKSPACE


def test_misaligned_arrays_are_rejected(lib):
    """Arrays read in 16-byte pieces must be 16-byte aligned; a misaligned
    one is an argument error, caught before any HIP call."""
    bad = ctypes.c_void_p(0x1002)
    assert tlp(lib, hidden=bad) == INVALID
    assert tlp(lib, head=bad) == INVALID
    ids = P
    assert lib.rz_sample_tokens(bad, P, ids, 4, 64, 10, BF16, ctypes.c_uint64(1), P, P,
                                NULL, P, 0, NULL) == INVALID
    f = ctypes.c_float(0.5)
    assert lib.rz_lora_augment(bad, P, f, 10, 64, 8, BF16, P, NULL) == INVALID
    assert lib.rz_token_logprobs_mx(bad, P, P, 0, P, 4, 128, 10, P, NULL, NULL, P, 0,
                                    NULL) == INVALID
