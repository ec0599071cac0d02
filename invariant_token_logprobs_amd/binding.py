"""ctypes binding of librz (C ABI in include/rz.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of librz.so.  torch supplies device memory and the stream; the
functions take torch tensors already on the GPU and return torch tensors.
There is no fallback: if the library is missing or the GPU is absent, the
call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

RZ_DTYPE_F32 = 0
RZ_DTYPE_BF16 = 1
RZ_OP_TOKEN_LOGPROBS = 0
RZ_OP_FWD_BWD = 1
RZ_OP_DIAGNOSTICS = 2
RZ_OP_SAMPLE = 3
RZ_OP_GRAD_NORMS = 4
RZ_OP_FWD_BWD_LORA = 5
RZ_OP_TOKEN_LOGPROBS_MX = 6
RZ_OP_SAMPLE_MX = 7
RZ_OP_SCORE_CENTERING = 8
RZ_LORA_COLS = 64

RZ_DEVERR_TOKEN = 1
RZ_DEVERR_GROUP = 2
RZ_DEVERR_CU_ROWS = 4
RZ_DEVERR_MX_SCALE = 8

RZ_MX_FORMATS = {"mxfp4": 0, "mxfp8": 1}

_STATUS = {0: "RZ_OK", -1: "RZ_ERR_INVALID_ARG", -2: "RZ_ERR_UNSUPPORTED",
           -3: "RZ_ERR_WORKSPACE", -4: "RZ_ERR_HIP", -5: "RZ_ERR_SCRATCH"}
RZ_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = [
    "rz_workspace_bytes", "rz_workspace_bytes_op", "rz_status_string",
    "rz_token_logprobs", "rz_reinforce_zero_fwd_bwd", "rz_diagnostics",
    "rz_score_centering_fwd_bwd", "rz_sample_tokens", "rz_sample_tokens_noalloc",
    "rz_grad_norms", "rz_response_diagnostics", "rz_run_summary",
    "rz_dequantize_head", "rz_lora_augment", "rz_lora_merge_head",
    "rz_reinforce_zero_fwd_bwd_lora", "rz_token_logprobs_mx",
    "rz_sample_tokens_mx",
    "rz_timing_enable", "rz_timing_num_kernels", "rz_timing_kernel_name",
    "rz_timing_read", "rz_calibrate_mfma",
]


class RzError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


_lib = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "librz.so")


def load_library():
    """Load librz.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RzError(f"{path} is not built; run "
                      "`python -m invariant_token_logprobs_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.rz_workspace_bytes.argtypes = [i64, i32, i32, i32, ctypes.c_int]
    lib.rz_workspace_bytes.restype = sz
    lib.rz_workspace_bytes_op.argtypes = [ctypes.c_int, i64, i32, i32, i32, ctypes.c_int]
    lib.rz_workspace_bytes_op.restype = sz
    lib.rz_status_string.argtypes = [ctypes.c_int]
    lib.rz_status_string.restype = ctypes.c_char_p
    lib.rz_token_logprobs.argtypes = [vp, vp, vp, i64, i32, i32, ctypes.c_int,
                                      vp, vp, vp, vp, sz, vp]
    lib.rz_token_logprobs.restype = ctypes.c_int
    lib.rz_reinforce_zero_fwd_bwd.argtypes = [
        vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, ctypes.c_int,
        vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.rz_reinforce_zero_fwd_bwd.restype = ctypes.c_int
    lib.rz_score_centering_fwd_bwd.argtypes = lib.rz_reinforce_zero_fwd_bwd.argtypes
    lib.rz_score_centering_fwd_bwd.restype = ctypes.c_int
    lib.rz_diagnostics.argtypes = [vp, vp, vp, i64, vp, vp, sz, vp]
    lib.rz_diagnostics.restype = ctypes.c_int
    lib.rz_sample_tokens.argtypes = [vp, vp, vp, i64, i32, i32, ctypes.c_int,
                                     ctypes.c_uint64, vp, vp, vp, vp, sz, vp]
    lib.rz_sample_tokens.restype = ctypes.c_int
    lib.rz_sample_tokens_noalloc.argtypes = [vp, vp, vp, i64, i32, i32, ctypes.c_int,
                                             ctypes.c_uint64, vp, vp, vp, vp]
    lib.rz_sample_tokens_noalloc.restype = ctypes.c_int
    lib.rz_grad_norms.argtypes = [vp, i64, i32, vp, i32, vp, vp, sz, vp]
    lib.rz_grad_norms.restype = ctypes.c_int
    lib.rz_response_diagnostics.argtypes = [vp, vp, vp, vp, i64, i32, vp, vp,
                                            vp, vp]
    lib.rz_response_diagnostics.restype = ctypes.c_int
    lib.rz_run_summary.argtypes = [vp, vp, vp, i64, i32,
                                   ctypes.POINTER(ctypes.c_double)]
    lib.rz_run_summary.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.rz_lora_augment.argtypes = [vp, vp, f32, i64, i32, i32, ctypes.c_int, vp, vp]
    lib.rz_lora_augment.restype = ctypes.c_int
    lib.rz_lora_merge_head.argtypes = [vp, vp, i32, i32, i32, ctypes.c_int, vp, vp]
    lib.rz_lora_merge_head.restype = ctypes.c_int
    lib.rz_reinforce_zero_fwd_bwd_lora.argtypes = [
        vp, vp, vp, vp, f32, i32, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32,
        ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.rz_reinforce_zero_fwd_bwd_lora.restype = ctypes.c_int
    lib.rz_token_logprobs_mx.argtypes = [vp, vp, vp, ctypes.c_int, vp, i64, i32, i32,
                                         vp, vp, vp, vp, sz, vp]
    lib.rz_token_logprobs_mx.restype = ctypes.c_int
    lib.rz_sample_tokens_mx.argtypes = [vp, vp, vp, ctypes.c_int, vp, i64, i32, i32,
                                        ctypes.c_uint64, vp, vp, vp, vp, vp, sz, vp]
    lib.rz_sample_tokens_mx.restype = ctypes.c_int
    lib.rz_dequantize_head.argtypes = [vp, vp, i32, i32, ctypes.c_int, vp, vp, vp]
    lib.rz_dequantize_head.restype = ctypes.c_int
    lib.rz_timing_enable.argtypes = [ctypes.c_int]
    lib.rz_timing_enable.restype = ctypes.c_int
    lib.rz_timing_num_kernels.argtypes = []
    lib.rz_timing_num_kernels.restype = ctypes.c_int
    lib.rz_timing_kernel_name.argtypes = [ctypes.c_int]
    lib.rz_timing_kernel_name.restype = ctypes.c_char_p
    lib.rz_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    lib.rz_timing_read.restype = ctypes.c_int
    lib.rz_calibrate_mfma.argtypes = [i32, i32, i32, i64, vp, vp]
    lib.rz_calibrate_mfma.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        lib = load_library()
        msg = lib.rz_status_string(status).decode()
        raise RzError(f"{what}: {_STATUS.get(status, status)} ({msg})", status)


# ------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RZ_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return RZ_DTYPE_BF16
    raise RzError(f"hidden / lm_head must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, ndim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise RzError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise RzError(f"{name} must live on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise RzError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise RzError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise RzError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise RzError(f"{name} is on {t.device}, expected {device}")


def _stream_obj(stream):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream()


def _stream(stream):
    return ctypes.c_void_p(_stream_obj(stream).cuda_stream)


class Workspace:
    """A grow-only device byte buffer reused across calls.

    Calls that share one Workspace must not overlap (they would race on its
    contents): use one per stream.  A larger buffer is allocated on the
    stream of the call that needs it, so the caching allocator hands the old
    one out again only in that stream's order."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, device, stream=None):
        torch = _torch()
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            s = _stream_obj(stream)
            if self.buf is not None:
                self.buf.record_stream(s)
            self.buf = None
            with torch.cuda.stream(s):
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_default_ws = {}


def _workspace(ws: Optional[Workspace], nbytes: int, device, stream=None):
    """The caller's workspace, else the default one of (device, stream)."""
    if ws is None:
        key = (str(device), int(_stream_obj(stream).cuda_stream))
        ws = _default_ws.setdefault(key, Workspace())
    return ws.get(nbytes, device, stream)


def workspace_bytes(op: int, n_rows: int, n_resp: int, H: int, V: int,
                    dtype_code: int) -> int:
    """Workspace bytes of one entry point (rz_workspace_bytes_op)."""
    return int(load_library().rz_workspace_bytes_op(op, n_rows, n_resp, H, V,
                                                    dtype_code))


def workspace_bytes_common(n_rows: int, n_resp: int, H: int, V: int,
                           dtype_code: int) -> int:
    """Workspace bytes that serve rz_token_logprobs, the learner step and
    rz_diagnostics at these sizes (rz_workspace_bytes)."""
    return int(load_library().rz_workspace_bytes(n_rows, n_resp, H, V,
                                                 dtype_code))


# ------------------------------------------------------------ entry points
def token_logprobs(hidden, lm_head, tokens, *, want_lse: bool = False,
                   err_flag=None, workspace: Optional[Workspace] = None,
                   stream=None, out=None):
    """log pi(tokens[t] | hidden[t]) for every row (rz_token_logprobs)."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", None, 2)
    dev = hidden.device
    _need(lm_head, "lm_head", hidden.dtype, 2, dev)
    _need(tokens, "tokens", torch.int32, 1, dev)
    N, H = hidden.shape
    V = lm_head.shape[0]
    if lm_head.shape[1] != H or tokens.shape[0] != N:
        raise RzError("shape mismatch between hidden, lm_head and tokens")
    logprobs = out if out is not None else torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev) if want_lse else None
    nbytes = workspace_bytes(RZ_OP_TOKEN_LOGPROBS, N, 1, H, V, dt)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_token_logprobs(_ptr(hidden), _ptr(lm_head), _ptr(tokens), N, H,
                                 V, dt, _ptr(logprobs), _ptr(lse), _ptr(err_flag),
                                 _ptr(ws), nbytes, _stream(stream)),
           "rz_token_logprobs")
    return (logprobs, lse) if want_lse else logprobs


def sample_tokens(hidden, lm_head, row_ids, seed: int, *, want_lse: bool = False,
                  workspace: Optional[Workspace] = None, stream=None):
    """Draw each row's token and record its logprob (rz_sample_tokens).

    row_ids: int64 tensor [n_rows], each row's identity (its bits are the
    uint64 id of the draw); seed: 0 <= seed < 2**64.  Returns (tokens int32,
    logmu float32[, lse float32])."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", None, 2)
    dev = hidden.device
    _need(lm_head, "lm_head", hidden.dtype, 2, dev)
    _need(row_ids, "row_ids", torch.int64, 1, dev)
    N, H = hidden.shape
    V = lm_head.shape[0]
    if lm_head.shape[1] != H or row_ids.shape[0] != N:
        raise RzError("shape mismatch between hidden, lm_head and row_ids")
    if not 0 <= int(seed) < 2 ** 64:
        raise RzError("seed must be in [0, 2**64)")
    tokens = torch.empty(N, dtype=torch.int32, device=dev)
    logmu = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev) if want_lse else None
    nbytes = workspace_bytes(RZ_OP_SAMPLE, N, 1, H, V, dt)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_sample_tokens(_ptr(hidden), _ptr(lm_head), _ptr(row_ids), N, H,
                                V, dt, ctypes.c_uint64(int(seed)), _ptr(tokens),
                                _ptr(logmu), _ptr(lse), _ptr(ws), nbytes,
                                _stream(stream)),
           "rz_sample_tokens")
    return (tokens, logmu, lse) if want_lse else (tokens, logmu)


def sample_tokens_noalloc(hidden, lm_head, row_ids, seed: int, *, out=None,
                          want_lse: bool = False, stream=None):
    """rz_sample_tokens_noalloc: the draw with the library's static scratch
    and no workspace.  out: optional (tokens int32, logmu float32[, lse])
    tensors to write into, so a caller that must not allocate passes its
    own.  Returns (tokens, logmu[, lse])."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", None, 2)
    dev = hidden.device
    _need(lm_head, "lm_head", hidden.dtype, 2, dev)
    _need(row_ids, "row_ids", torch.int64, 1, dev)
    N, H = hidden.shape
    V = lm_head.shape[0]
    if lm_head.shape[1] != H or row_ids.shape[0] != N:
        raise RzError("shape mismatch between hidden, lm_head and row_ids")
    if not 0 <= int(seed) < 2 ** 64:
        raise RzError("seed must be in [0, 2**64)")
    if out is None:
        out = (torch.empty(N, dtype=torch.int32, device=dev),
               torch.empty(N, dtype=torch.float32, device=dev),
               torch.empty(N, dtype=torch.float32, device=dev) if want_lse else None)
    tokens, logmu = out[0], out[1]
    lse = out[2] if len(out) > 2 else None
    _check(lib.rz_sample_tokens_noalloc(_ptr(hidden), _ptr(lm_head), _ptr(row_ids), N,
                                        H, V, dt, ctypes.c_uint64(int(seed)),
                                        _ptr(tokens), _ptr(logmu), _ptr(lse),
                                        _stream(stream)),
           "rz_sample_tokens_noalloc")
    return (tokens, logmu, lse) if lse is not None else (tokens, logmu)


def _learner_step(fn, op, what, hidden, lm_head, tokens, logmu, mask, cu_rows,
                  rewards, group_ids, err_flag, workspace, stream, outputs):
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", None, 2)
    dev = hidden.device
    _need(lm_head, "lm_head", hidden.dtype, 2, dev)
    _need(tokens, "tokens", torch.int32, 1, dev)
    if logmu is not None:
        _need(logmu, "logmu", torch.float32, 1, dev)
    _need(mask, "mask", torch.uint8, 1, dev)
    _need(cu_rows, "cu_rows", torch.int32, 1, dev)
    _need(rewards, "rewards", torch.float32, 1, dev)
    _need(group_ids, "group_ids", torch.int32, 1, dev)
    N, H = hidden.shape
    V = lm_head.shape[0]
    B = rewards.shape[0]
    if (lm_head.shape[1] != H or tokens.shape[0] != N
            or (logmu is not None and logmu.shape[0] != N)
            or mask.shape[0] != N or cu_rows.shape[0] != B + 1
            or group_ids.shape[0] != B):
        raise RzError(f"shape mismatch between the {what} arguments")
    o = outputs if outputs is not None else {}
    f32 = torch.float32
    if "logprobs" not in o:
        o["logprobs"] = torch.empty(N, dtype=f32, device=dev)
        o["loss"] = torch.empty(1, dtype=f32, device=dev)
        o["d_hidden"] = torch.empty((N, H), dtype=f32, device=dev)
        o["d_lm_head"] = torch.empty((V, H), dtype=f32, device=dev)
        o["diag"] = torch.empty(2, dtype=f32, device=dev) if logmu is not None else None
        o["adv"] = torch.empty(B, dtype=f32, device=dev)
    nbytes = workspace_bytes(op, N, B, H, V, dt)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(fn(
        _ptr(hidden), _ptr(lm_head), _ptr(tokens), _ptr(logmu), _ptr(mask),
        _ptr(cu_rows), _ptr(rewards), _ptr(group_ids), N, B, H, V, dt,
        _ptr(o["logprobs"]), _ptr(o["loss"]), _ptr(o["d_hidden"]),
        _ptr(o["d_lm_head"]), _ptr(o["diag"]), _ptr(o["adv"]), _ptr(err_flag),
        _ptr(ws), nbytes, _stream(stream)), what)
    return o


def reinforce_zero_fwd_bwd(hidden, lm_head, tokens, logmu, mask, cu_rows,
                           rewards, group_ids, *, err_flag=None,
                           workspace: Optional[Workspace] = None, stream=None,
                           outputs: Optional[dict] = None):
    """One learner step (rz_reinforce_zero_fwd_bwd).  Returns a dict with
    logprobs, loss, d_hidden, d_lm_head, diag (D3, KL) and adv."""
    if logmu is None:
        raise RzError("logmu is required")
    return _learner_step(load_library().rz_reinforce_zero_fwd_bwd, RZ_OP_FWD_BWD,
                         "rz_reinforce_zero_fwd_bwd", hidden, lm_head, tokens,
                         logmu, mask, cu_rows, rewards, group_ids, err_flag,
                         workspace, stream, outputs)


def score_centering_fwd_bwd(hidden, lm_head, tokens, mask, cu_rows, rewards,
                            group_ids, *, logmu=None, err_flag=None,
                            workspace: Optional[Workspace] = None, stream=None,
                            outputs: Optional[dict] = None):
    """The score-centering step (rz_score_centering_fwd_bwd): the learner step
    with w = 1.  Returns logprobs, loss (the SC surrogate), d_hidden,
    d_lm_head, adv, and diag (D3, KL of the records) when logmu is given."""
    return _learner_step(load_library().rz_score_centering_fwd_bwd,
                         RZ_OP_SCORE_CENTERING, "rz_score_centering_fwd_bwd",
                         hidden, lm_head, tokens, logmu, mask, cu_rows, rewards,
                         group_ids, err_flag, workspace, stream, outputs)


def diagnostics(logpi, logmu, mask=None, *, workspace: Optional[Workspace] = None,
                stream=None, out=None):
    """(D3, KL) over the valid entries (rz_diagnostics)."""
    torch = _torch()
    lib = load_library()
    _need(logpi, "logpi", torch.float32, 1)
    dev = logpi.device
    _need(logmu, "logmu", torch.float32, 1, dev)
    if mask is not None:
        _need(mask, "mask", torch.uint8, 1, dev)
    n = logpi.shape[0]
    if logmu.shape[0] != n or (mask is not None and mask.shape[0] != n):
        raise RzError("shape mismatch between logpi, logmu and mask")
    diag = out if out is not None else torch.empty(2, dtype=torch.float32, device=dev)
    nbytes = workspace_bytes(RZ_OP_DIAGNOSTICS, n, 1, 64, 1, 0)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_diagnostics(_ptr(logpi), _ptr(logmu), _ptr(mask), n, _ptr(diag),
                              _ptr(ws), nbytes, _stream(stream)), "rz_diagnostics")
    return diag


# ------------------------------------------------------- LoRA on the head
def _lora_shapes(hidden_or_head, lora, name, rank_dim):
    torch = _torch()
    _need(lora, name, hidden_or_head.dtype, 2, hidden_or_head.device)
    r = lora.shape[rank_dim]
    if not 1 <= r <= RZ_LORA_COLS:
        raise RzError(f"LoRA rank must be in [1, {RZ_LORA_COLS}], got {r}")
    return r


def lora_augment(hidden, lora_A, scale: float, *, stream=None, out=None):
    """[h | u | 0] with u = scale * h A^T in the head's precision
    (rz_lora_augment): [n, H + RZ_LORA_COLS]."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", None, 2)
    n, H = hidden.shape
    r = _lora_shapes(hidden, lora_A, "lora_A", 0)
    if lora_A.shape[1] != H:
        raise RzError("lora_A must be [r, H]")
    h_aug = out if out is not None else torch.empty(
        (n, H + RZ_LORA_COLS), dtype=hidden.dtype, device=hidden.device)
    _check(lib.rz_lora_augment(_ptr(hidden), _ptr(lora_A), float(scale), n, H, r,
                               dt, _ptr(h_aug), _stream(stream)), "rz_lora_augment")
    return h_aug


def lora_merge_head(lm_head, lora_B, *, stream=None, out=None):
    """[W | B | 0] (rz_lora_merge_head): [V, H + RZ_LORA_COLS]."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(lm_head)
    _need(lm_head, "lm_head", None, 2)
    V, H = lm_head.shape
    r = _lora_shapes(lm_head, lora_B, "lora_B", 1)
    if lora_B.shape[0] != V:
        raise RzError("lora_B must be [V, r]")
    W_aug = out if out is not None else torch.empty(
        (V, H + RZ_LORA_COLS), dtype=lm_head.dtype, device=lm_head.device)
    _check(lib.rz_lora_merge_head(_ptr(lm_head), _ptr(lora_B), V, H, r, dt,
                                  _ptr(W_aug), _stream(stream)), "rz_lora_merge_head")
    return W_aug


def reinforce_zero_fwd_bwd_lora(hidden, lm_head, lora_A, lora_B, scale: float,
                                tokens, logmu, mask, cu_rows, rewards, group_ids,
                                *, err_flag=None,
                                workspace: Optional[Workspace] = None,
                                stream=None):
    """The learner step with a LoRA adapter on a frozen head
    (rz_reinforce_zero_fwd_bwd_lora).  Returns a dict with logprobs, loss,
    d_hidden, d_lora_A, d_lora_B, diag and adv."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", None, 2)
    dev = hidden.device
    _need(lm_head, "lm_head", hidden.dtype, 2, dev)
    for t, nm, d in ((tokens, "tokens", torch.int32), (logmu, "logmu", torch.float32),
                     (mask, "mask", torch.uint8), (cu_rows, "cu_rows", torch.int32),
                     (rewards, "rewards", torch.float32),
                     (group_ids, "group_ids", torch.int32)):
        _need(t, nm, d, 1, dev)
    N, H = hidden.shape
    V = lm_head.shape[0]
    B = rewards.shape[0]
    r = _lora_shapes(hidden, lora_A, "lora_A", 0)
    _need(lora_B, "lora_B", hidden.dtype, 2, dev)
    if (lm_head.shape[1] != H or lora_A.shape[1] != H
            or tuple(lora_B.shape) != (V, r) or tokens.shape[0] != N
            or logmu.shape[0] != N or mask.shape[0] != N
            or cu_rows.shape[0] != B + 1 or group_ids.shape[0] != B):
        raise RzError("shape mismatch between the fwd_bwd_lora arguments")
    f32 = torch.float32
    o = {"logprobs": torch.empty(N, dtype=f32, device=dev),
         "loss": torch.empty(1, dtype=f32, device=dev),
         "d_hidden": torch.empty((N, H), dtype=f32, device=dev),
         "d_lora_A": torch.empty((r, H), dtype=f32, device=dev),
         "d_lora_B": torch.empty((V, r), dtype=f32, device=dev),
         "diag": torch.empty(2, dtype=f32, device=dev),
         "adv": torch.empty(B, dtype=f32, device=dev)}
    nbytes = workspace_bytes(RZ_OP_FWD_BWD_LORA, N, B, H, V, dt)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_reinforce_zero_fwd_bwd_lora(
        _ptr(hidden), _ptr(lm_head), _ptr(lora_A), _ptr(lora_B), float(scale), r,
        _ptr(tokens), _ptr(logmu), _ptr(mask), _ptr(cu_rows), _ptr(rewards),
        _ptr(group_ids), N, B, H, V, dt, _ptr(o["logprobs"]), _ptr(o["loss"]),
        _ptr(o["d_hidden"]), _ptr(o["d_lora_A"]), _ptr(o["d_lora_B"]),
        _ptr(o["diag"]), _ptr(o["adv"]), _ptr(err_flag), _ptr(ws), nbytes,
        _stream(stream)), "rz_reinforce_zero_fwd_bwd_lora")
    return o


# ------------------------------------------------------------ MX-format head
def dequantize_head(codes, scales, fmt: str, *, err_flag=None, stream=None,
                    out=None):
    """The bf16 head [V, H] of an MX-format head (rz_dequantize_head).

    codes: uint8 [V, H/2] (fmt "mxfp4", two E2M1 codes per byte, low nibble
    first) or [V, H] ("mxfp8", E4M3); scales: uint8 [V, H/32] E8M0."""
    torch = _torch()
    lib = load_library()
    if fmt not in RZ_MX_FORMATS:
        raise RzError(f"fmt must be one of {sorted(RZ_MX_FORMATS)}, got {fmt!r}")
    _need(codes, "codes", torch.uint8, 2)
    dev = codes.device
    _need(scales, "scales", torch.uint8, 2, dev)
    V = codes.shape[0]
    H = codes.shape[1] * (2 if fmt == "mxfp4" else 1)
    if tuple(scales.shape) != (V, H // 32) or H % 32:
        raise RzError(f"scales must be [V, H/32] = [{V}, {H // 32}] with H % 32 == 0")
    W = out if out is not None else torch.empty((V, H), dtype=torch.bfloat16, device=dev)
    _check(lib.rz_dequantize_head(_ptr(codes), _ptr(scales), V, H,
                                  RZ_MX_FORMATS[fmt], _ptr(W), _ptr(err_flag),
                                  _stream(stream)), "rz_dequantize_head")
    return W


def _mx_head(codes, scales, fmt, dev):
    torch = _torch()
    if fmt not in RZ_MX_FORMATS:
        raise RzError(f"fmt must be one of {sorted(RZ_MX_FORMATS)}, got {fmt!r}")
    _need(codes, "codes", torch.uint8, 2, dev)
    _need(scales, "scales", torch.uint8, 2, dev)
    V = codes.shape[0]
    H = codes.shape[1] * (2 if fmt == "mxfp4" else 1)
    if tuple(scales.shape) != (V, H // 32):
        raise RzError("scales must be [V, H/32]")
    return V, H


def token_logprobs_mx(hidden, codes, scales, fmt: str, tokens, *,
                      want_lse: bool = False, err_flag=None,
                      workspace: Optional[Workspace] = None, stream=None):
    """log pi on an MX-format head (rz_token_logprobs_mx); bf16 hidden."""
    torch = _torch()
    lib = load_library()
    _need(hidden, "hidden", torch.bfloat16, 2)
    dev = hidden.device
    V, H = _mx_head(codes, scales, fmt, dev)
    _need(tokens, "tokens", torch.int32, 1, dev)
    N = hidden.shape[0]
    if hidden.shape[1] != H or tokens.shape[0] != N:
        raise RzError("shape mismatch between hidden, the MX head and tokens")
    logprobs = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev) if want_lse else None
    nbytes = workspace_bytes(RZ_OP_TOKEN_LOGPROBS_MX, N, 1, H, V, RZ_DTYPE_BF16)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_token_logprobs_mx(_ptr(hidden), _ptr(codes), _ptr(scales),
                                    RZ_MX_FORMATS[fmt], _ptr(tokens), N, H, V,
                                    _ptr(logprobs), _ptr(lse), _ptr(err_flag),
                                    _ptr(ws), nbytes, _stream(stream)),
           "rz_token_logprobs_mx")
    return (logprobs, lse) if want_lse else logprobs


def sample_tokens_mx(hidden, codes, scales, fmt: str, row_ids, seed: int, *,
                     want_lse: bool = False, err_flag=None,
                     workspace: Optional[Workspace] = None, stream=None):
    """The rollout draw on an MX-format head (rz_sample_tokens_mx)."""
    torch = _torch()
    lib = load_library()
    _need(hidden, "hidden", torch.bfloat16, 2)
    dev = hidden.device
    V, H = _mx_head(codes, scales, fmt, dev)
    _need(row_ids, "row_ids", torch.int64, 1, dev)
    N = hidden.shape[0]
    if hidden.shape[1] != H or row_ids.shape[0] != N:
        raise RzError("shape mismatch between hidden, the MX head and row_ids")
    if not 0 <= int(seed) < 2 ** 64:
        raise RzError("seed must be in [0, 2**64)")
    tokens = torch.empty(N, dtype=torch.int32, device=dev)
    logmu = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev) if want_lse else None
    nbytes = workspace_bytes(RZ_OP_SAMPLE_MX, N, 1, H, V, RZ_DTYPE_BF16)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_sample_tokens_mx(_ptr(hidden), _ptr(codes), _ptr(scales),
                                   RZ_MX_FORMATS[fmt], _ptr(row_ids), N, H, V,
                                   ctypes.c_uint64(int(seed)), _ptr(tokens),
                                   _ptr(logmu), _ptr(lse), _ptr(err_flag),
                                   _ptr(ws), nbytes, _stream(stream)),
           "rz_sample_tokens_mx")
    return (tokens, logmu, lse) if want_lse else (tokens, logmu)


# ------------------------------------------------------- run-level diagnostics
def grad_norms(d_hidden, d_lm_head, *, workspace: Optional[Workspace] = None,
               stream=None, out=None):
    """(||d_hidden||_2, ||d_lm_head||_2) as a float32 device tensor [2]
    (rz_grad_norms)."""
    torch = _torch()
    lib = load_library()
    _need(d_lm_head, "d_lm_head", torch.float32, 2)
    dev = d_lm_head.device
    _need(d_hidden, "d_hidden", torch.float32, 2, dev)
    N, H = d_hidden.shape
    V = d_lm_head.shape[0]
    if d_lm_head.shape[1] != H:
        raise RzError("d_hidden and d_lm_head disagree on H")
    norms = out if out is not None else torch.empty(2, dtype=torch.float32, device=dev)
    nbytes = workspace_bytes(RZ_OP_GRAD_NORMS, N, 0, H, V, 0)
    ws = _workspace(workspace, nbytes, dev, stream)
    _check(lib.rz_grad_norms(_ptr(d_hidden), N, H, _ptr(d_lm_head), V,
                             _ptr(norms), _ptr(ws), nbytes, _stream(stream)),
           "rz_grad_norms")
    return norms


def response_diagnostics(logpi, logmu, mask, cu_rows, *, err_flag=None,
                         stream=None):
    """Per-response (D3, KL), two float32 device tensors [n_resp]
    (rz_response_diagnostics); mask may be None (all rows valid)."""
    torch = _torch()
    lib = load_library()
    _need(logpi, "logpi", torch.float32, 1)
    dev = logpi.device
    _need(logmu, "logmu", torch.float32, 1, dev)
    _need(cu_rows, "cu_rows", torch.int32, 1, dev)
    if mask is not None:
        _need(mask, "mask", torch.uint8, 1, dev)
    n = logpi.shape[0]
    B = cu_rows.shape[0] - 1
    if B < 0 or logmu.shape[0] != n or (mask is not None and mask.shape[0] != n):
        raise RzError("shape mismatch between logpi, logmu, mask and cu_rows")
    d3 = torch.empty(B, dtype=torch.float32, device=dev)
    kl = torch.empty(B, dtype=torch.float32, device=dev)
    _check(lib.rz_response_diagnostics(_ptr(logpi), _ptr(logmu), _ptr(mask),
                                       _ptr(cu_rows), n, B, _ptr(d3), _ptr(kl),
                                       _ptr(err_flag), _stream(stream)),
           "rz_response_diagnostics")
    return d3, kl


RUN_SUMMARY_KEYS = ("d3_peak", "d3_median", "d3_peak_over_median",
                    "kl_median_first", "kl_median_last", "kl_median_ratio",
                    "grad_norm_max")


def run_summary(d3_steps, kl_steps, grad_norm_steps, window: int = 1000) -> dict:
    """Run-level view over per-step host values (rz_run_summary): sequences
    of floats (or None) in step order, all of the same length."""
    import numpy as np
    lib = load_library()
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.float32)
            for a in (d3_steps, kl_steps, grad_norm_steps)]
    lens = {a.shape[0] for a in arrs if a is not None}
    if len(lens) > 1 or any(a is not None and a.ndim != 1 for a in arrs):
        raise RzError("per-step arrays must be 1-D and of one length")
    n = lens.pop() if lens else 0
    out = (ctypes.c_double * 7)()
    ptrs = [None if a is None else ctypes.c_void_p(a.ctypes.data) for a in arrs]
    _check(lib.rz_run_summary(*ptrs, n, int(window), out), "rz_run_summary")
    return dict(zip(RUN_SUMMARY_KEYS, list(out)))


class RunTracker:
    """Per-step D3, KL and gradient norm of a training run, kept on the GPU
    until a summary is asked for (one copy to the host then, none per step).

    record(diag, grad_norm): diag is the [2] (D3, KL) output of
    reinforce_zero_fwd_bwd or diagnostics; grad_norm a one-element tensor,
    e.g. grad_norms(...)[1:] for this path's parameter gradient or the
    trainer's global norm before clipping."""

    def __init__(self, device, window: int = 1000, capacity: int = 4096):
        torch = _torch()
        self.window = int(window)
        self.n = 0
        self.buf = torch.empty((max(1, capacity), 3), dtype=torch.float32,
                               device=device)

    def record(self, diag, grad_norm):
        torch = _torch()
        if self.n == self.buf.shape[0]:
            grown = torch.empty((2 * self.n, 3), dtype=torch.float32,
                                device=self.buf.device)
            grown[: self.n].copy_(self.buf)
            self.buf = grown
        self.buf[self.n, 0:2].copy_(diag.reshape(2))
        self.buf[self.n, 2:3].copy_(grad_norm.reshape(1))
        self.n += 1

    def values(self):
        """(d3, kl, grad_norm) per step as host float32 arrays."""
        h = self.buf[: self.n].cpu().numpy()
        return h[:, 0].copy(), h[:, 1].copy(), h[:, 2].copy()

    def summary(self) -> dict:
        """rz_run_summary over the recorded steps, plus the count of
        sequences a gate rejected: always 0, since this loss has no gate
        (every valid token of every response enters it, unclipped)."""
        out = run_summary(*self.values(), window=self.window)
        out["steps"] = self.n
        out["rejected_sequences"] = 0
        return out


# ------------------------------------------------------------ kernel timer
def timing_enable(on: bool = True):
    _check(load_library().rz_timing_enable(1 if on else 0), "rz_timing_enable")


def timing_read(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    lib = load_library()
    n = lib.rz_timing_num_kernels()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib.rz_timing_read(ms, cnt, 1 if reset else 0), "rz_timing_read")
    return {lib.rz_timing_kernel_name(k).decode(): (ms[k], cnt[k])
            for k in range(n)}


def calibrate_mfma(data: bool, from_lds: bool, n_workgroups: int, iters: int,
                   sink, stream=None):
    """rz_calibrate_mfma (measurement support): launch the matrix-core
    ceiling kernel; returns the FLOP it issues."""
    torch = _torch()
    _need(sink, "sink", torch.float32, 1)
    if sink.numel() < n_workgroups * 256:
        raise RzError("sink must hold n_workgroups * 256 floats")
    lib = load_library()
    _check(lib.rz_calibrate_mfma(1 if data else 0, 1 if from_lds else 0,
                                 n_workgroups, iters, _ptr(sink), _stream(stream)),
           "rz_calibrate_mfma")
    return float(n_workgroups) * 4 * iters * 128 * 32768
