"""Strict, batch- and partition-invariant token log-probabilities on MI355X.

Thin Python binding of ``librlk_logp.so`` (C ABI declared in
``include/rlk_logp.h``). This module only marshals arguments: it checks
tensor dtypes, devices and shapes, passes raw device pointers and the current
HIP stream, and turns negative status codes into exceptions. Every step of the
computation runs in the HIP kernels of the library; there is no fallback.

Build the library first with ``python -m invariant_token_log_fp32_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple, Union

__all__ = [
    "LIB_PATH", "HEADER_PATH", "VocabLayout", "load_library", "status_string", "workspace_bytes",
    "summary_bytes", "logp_full", "logp_nucleus", "logp_shard_summaries", "logp_merge", "logp_backward",
    "support_state_fields", "l2norm", "l2norm_zero", "l2norm_accumulate", "l2norm_finalize", "NORM_BIN_WORDS",
    "linear", "linear_logp", "linear_logp_workspace_bytes", "linear_logp_summaries", "linear_logp_merge",
    "logp_nucleus_noalloc", "NOALLOC_MAX_ROWS", "RlkError", "N_SHARDS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# RLK_LIBRARY names another build of the same library (the host-sanitizer build
# that the CPU tests use); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("RLK_LIBRARY") or os.path.join(_PKG, "librlk_logp.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "rlk_logp.h")
HEADER_PATHS = [HEADER_PATH] + [os.path.join(os.path.dirname(_PKG), "include", n) for n in ("rlk_norm.h", "rlk_linear.h")]
N_SHARDS = 8
NORM_BIN_WORDS = 264  # uint64 words of rlk_norm_bins
NOALLOC_MAX_ROWS = 32768  # RLK_NOALLOC_MAX_ROWS

RLK_OK = 0
STATUS_NAMES = {
    0: "RLK_OK", -1: "RLK_ERR_NULL", -2: "RLK_ERR_ALIGN", -3: "RLK_ERR_SHAPE",
    -4: "RLK_ERR_GROUPS", -5: "RLK_ERR_WORKSPACE", -6: "RLK_ERR_HIP", -7: "RLK_ERR_SCRATCH",
}


class RlkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class VocabLayout(ctypes.Structure):
    """Mirror of ``rlk_vocab_layout``."""

    _fields_ = [
        ("vocab_padded", ctypes.c_int64),
        ("vocab_real", ctypes.c_int64),
        ("row_stride", ctypes.c_int64),
        ("n_shards", ctypes.c_int32),
        ("groups", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m invariant_token_log_fp32_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lay = ctypes.POINTER(VocabLayout)
    lib.rlk_logp_full.argtypes = [vp, i64, lay, vp, vp, vp, vp, vp, sz, vp]
    lib.rlk_logp_full.restype = i32
    lib.rlk_logp_nucleus.argtypes = [vp, i64, lay, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.rlk_logp_nucleus.restype = i32
    lib.rlk_logp_nucleus_noalloc.argtypes = [vp, i64, lay, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.rlk_logp_nucleus_noalloc.restype = i32
    lib.rlk_logp_workspace_bytes.argtypes = [i64, lay, i32]
    lib.rlk_logp_workspace_bytes.restype = sz
    lib.rlk_status_string.argtypes = [i32]
    lib.rlk_status_string.restype = ctypes.c_char_p
    lib.rlk_logp_shard_summaries.argtypes = [vp, i64, lay, i32, i64, vp, vp, vp, sz, vp]
    lib.rlk_logp_shard_summaries.restype = i32
    lib.rlk_logp_merge.argtypes = [vp, sz, i64, lay, vp, vp, vp, vp, vp]
    lib.rlk_logp_merge.restype = i32
    lib.rlk_logp_summary_bytes.argtypes = [i64, lay]
    lib.rlk_logp_summary_bytes.restype = sz
    lib.rlk_logp_backward.argtypes = [vp, i64, lay, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
    lib.rlk_logp_backward.restype = i32
    lib.rlk_l2norm_zero.argtypes = [vp, vp]
    lib.rlk_l2norm_zero.restype = i32
    lib.rlk_l2norm_accumulate.argtypes = [vp, i64, vp, vp]
    lib.rlk_l2norm_accumulate.restype = i32
    lib.rlk_l2norm_finalize.argtypes = [vp, vp, vp, vp]
    lib.rlk_l2norm_finalize.restype = i32
    lib.rlk_l2norm.argtypes = [vp, i64, vp, vp, vp, vp]
    lib.rlk_l2norm.restype = i32
    lib.rlk_linear.argtypes = [vp, i64, i64, i64, vp, i64, lay, vp, vp]
    lib.rlk_linear.restype = i32
    lib.rlk_linear_logp.argtypes = [vp, i64, i64, i64, vp, i64, lay, vp, vp, vp, vp, vp, sz, vp]
    lib.rlk_linear_logp.restype = i32
    lib.rlk_linear_logp_workspace_bytes.argtypes = [i64, lay]
    lib.rlk_linear_logp_workspace_bytes.restype = sz
    lib.rlk_linear_logp_summaries.argtypes = [vp, i64, i64, i64, vp, i64, lay, i32, vp, vp, vp, sz, vp]
    lib.rlk_linear_logp_summaries.restype = i32
    lib.rlk_linear_logp_merge.argtypes = [vp, sz, i64, lay, vp, vp, vp, vp, vp]
    lib.rlk_linear_logp_merge.restype = i32
    lib.rlk_linear_logp_summary_bytes.argtypes = [i64, lay]
    lib.rlk_linear_logp_summary_bytes.restype = sz
    _lib = lib
    return lib


def declared_functions(headers=None):
    """Names of the functions that the headers under include/ declare."""
    names = set()
    for h in (headers or HEADER_PATHS):
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(rlk_\w+)\s*\(", text, re.M))
    return sorted(names)


def status_string(status: int) -> str:
    return load_library().rlk_status_string(int(status)).decode()


def make_layout(vocab_padded: int, vocab_real: int, row_stride: int, groups: int = 1) -> VocabLayout:
    return VocabLayout(int(vocab_padded), int(vocab_real), int(row_stride), N_SHARDS, int(groups))


def workspace_bytes(n_rows: int, vocab_padded: int, vocab_real: int, row_stride: Optional[int] = None,
                    groups: int = 1, nucleus: bool = False) -> int:
    lay = make_layout(vocab_padded, vocab_real, row_stride or vocab_padded, groups)
    return int(load_library().rlk_logp_workspace_bytes(int(n_rows), ctypes.byref(lay), 1 if nucleus else 0))


def summary_bytes(n_rows: int, vocab_padded: int, vocab_real: int, groups: int = 1) -> int:
    """Bytes of one rank's shard summaries (rlk_logp_summary_bytes)."""
    lay = make_layout(vocab_padded, vocab_real, vocab_padded, groups)
    return int(load_library().rlk_logp_summary_bytes(int(n_rows), ctypes.byref(lay)))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _check_logits(logits):
    torch = _torch()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [n_rows, row_stride]")
    if logits.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("logits must hold BF16 bit patterns (bfloat16, int16 or uint16)")
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    return logits.stride(0) if logits.shape[0] > 1 else max(logits.stride(0), logits.shape[1])


def _per_row(value, n, dtype, device, name):
    torch = _torch()
    if isinstance(value, (int, float)):
        return torch.full((n,), value, dtype=dtype, device=device)
    if value.dtype != dtype or value.device != device or value.shape != (n,) or not value.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape ({n},) on {device}")
    return value


def _out(value, shape, dtype, device, name):
    """A caller-supplied output tensor, checked (the C ABI cannot see buffer
    sizes, so a short or mistyped buffer must never reach it), or a new one."""
    torch = _torch()
    if value is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if value.dtype != dtype or value.device != device or tuple(value.shape) != tuple(shape) or \
            not value.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")
    return value


def _workspace(value, need, device, name="workspace"):
    """(tensor or None, size in bytes) of a caller-supplied workspace, checked,
    or a new one of `need` bytes."""
    torch = _torch()
    if value is None:
        if need == 0:
            return None, 0
        value = torch.empty(need, dtype=torch.uint8, device=device)
    if value.device != device or not value.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    nbytes = value.numel() * value.element_size()
    if nbytes < need:
        raise ValueError(f"{name} holds {nbytes} bytes, {need} needed")
    return value, nbytes


def _stream_handle(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def logp_full(logits, temperature: Union[float, "torch.Tensor"], target, *, vocab_real: int,
              vocab_padded: Optional[int] = None, groups: int = 1, return_lse: bool = False,
              out=None, lse_out=None, workspace=None, stream=None):
    """Full-vocabulary reference logprob of ``target`` per row (rlk_logp_full).

    ``logits`` is a [n_rows, >= vocab_padded] device tensor of BF16 bits whose
    row stride is a multiple of 8 elements; ``temperature`` is a float or a
    float32 [n_rows] tensor; ``target`` is int64 [n_rows]. Returns the float32
    logprobs (and the log-sum-exps when ``return_lse``).
    """
    torch = _torch()
    stride = _check_logits(logits)
    n = logits.shape[0]
    dev = logits.device
    vp = int(vocab_padded if vocab_padded is not None else logits.shape[1])
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    target = _per_row(target, n, torch.int64, dev, "target")
    out = _out(out, (n,), torch.float32, dev, "out")
    if return_lse or lse_out is not None:
        lse_out = _out(lse_out, (n,), torch.float32, dev, "lse_out")
    lay = make_layout(vp, vocab_real, stride, groups)
    lib = load_library()
    need = int(lib.rlk_logp_workspace_bytes(n, ctypes.byref(lay), 0))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    st = lib.rlk_logp_full(
        logits.data_ptr(), n, ctypes.byref(lay), temperature.data_ptr(), target.data_ptr(),
        out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None,
        workspace.data_ptr() if workspace is not None else None, ws_bytes, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_logp_full")
    return (out, lse_out) if return_lse else out


def logp_nucleus(logits, temperature, top_p, top_k, target, *, vocab_real: int,
                 vocab_padded: Optional[int] = None, groups: int = 1, return_state: bool = False,
                 policy_out=None, ref_out=None, lse_out=None, state_out=None, workspace=None, stream=None):
    """Policy logprob over the top-k-then-top-p support and the full-vocabulary
    reference logprob (rlk_logp_nucleus). ``top_p`` float or float32 [n_rows],
    ``top_k`` int or int32 [n_rows]. Returns (policy, reference), or with
    ``return_state`` (policy, reference, lse, state) where ``state`` is the
    int32 [n_rows, 4] view of the rlk_support_state records (see
    ``support_state_fields``)."""
    torch = _torch()
    stride = _check_logits(logits)
    n = logits.shape[0]
    dev = logits.device
    vp = int(vocab_padded if vocab_padded is not None else logits.shape[1])
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    top_p = _per_row(top_p, n, torch.float32, dev, "top_p")
    top_k = _per_row(top_k, n, torch.int32, dev, "top_k")
    target = _per_row(target, n, torch.int64, dev, "target")
    policy_out = _out(policy_out, (n,), torch.float32, dev, "policy_out")
    ref_out = _out(ref_out, (n,), torch.float32, dev, "ref_out")
    if return_state or lse_out is not None:
        lse_out = _out(lse_out, (n,), torch.float32, dev, "lse_out")
    if return_state or state_out is not None:
        state_out = _out(state_out, (n, 4), torch.int32, dev, "state_out")
    lay = make_layout(vp, vocab_real, stride, groups)
    lib = load_library()
    need = int(lib.rlk_logp_workspace_bytes(n, ctypes.byref(lay), 1))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    st = lib.rlk_logp_nucleus(
        logits.data_ptr(), n, ctypes.byref(lay), temperature.data_ptr(), top_p.data_ptr(),
        top_k.data_ptr(), target.data_ptr(), policy_out.data_ptr(), ref_out.data_ptr(),
        lse_out.data_ptr() if lse_out is not None else None,
        state_out.data_ptr() if state_out is not None else None,
        workspace.data_ptr() if workspace is not None else None, ws_bytes, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_logp_nucleus")
    if return_state:
        return policy_out, ref_out, lse_out, state_out
    return policy_out, ref_out


def logp_nucleus_noalloc(logits, temperature, top_p, top_k, target, *, vocab_real: int,
                         vocab_padded: Optional[int] = None, groups: int = 1, policy_out=None, ref_out=None,
                         lse_out=None, state_out=None, stream=None):
    """rlk_logp_nucleus_noalloc: rlk_logp_nucleus without a workspace (the
    library's static per-GPU scratch holds the shard summaries when groups > 1,
    for at most NOALLOC_MAX_ROWS rows). Calls that overlap on one GPU race.
    Returns (policy, reference); lse_out / state_out are filled when given."""
    torch = _torch()
    stride = _check_logits(logits)
    n = logits.shape[0]
    dev = logits.device
    vp = int(vocab_padded if vocab_padded is not None else logits.shape[1])
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    top_p = _per_row(top_p, n, torch.float32, dev, "top_p")
    top_k = _per_row(top_k, n, torch.int32, dev, "top_k")
    target = _per_row(target, n, torch.int64, dev, "target")
    policy_out = _out(policy_out, (n,), torch.float32, dev, "policy_out")
    ref_out = _out(ref_out, (n,), torch.float32, dev, "ref_out")
    if lse_out is not None:
        lse_out = _out(lse_out, (n,), torch.float32, dev, "lse_out")
    if state_out is not None:
        state_out = _out(state_out, (n, 4), torch.int32, dev, "state_out")
    lay = make_layout(vp, vocab_real, stride, groups)
    st = load_library().rlk_logp_nucleus_noalloc(
        logits.data_ptr(), n, ctypes.byref(lay), temperature.data_ptr(), top_p.data_ptr(), top_k.data_ptr(),
        target.data_ptr(), policy_out.data_ptr(), ref_out.data_ptr(),
        lse_out.data_ptr() if lse_out is not None else None,
        state_out.data_ptr() if state_out is not None else None, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_logp_nucleus_noalloc")
    return policy_out, ref_out


def support_state_fields(state):
    """(lse_support float32, threshold float32, status int32) columns of an
    int32 [n_rows, 4] tensor of rlk_support_state records."""
    torch = _torch()
    return state[:, 0].view(torch.float32), state[:, 1].view(torch.float32), state[:, 2]


def logp_backward(logits, temperature, target, *, vocab_real: int, vocab_padded: Optional[int] = None,
                  ref_logp=None, lse=None, grad_ref=None, policy_logp=None, support_state=None, grad_policy=None,
                  out=None, stream=None):
    """BF16 gradient of sum_i (grad_ref[i] * ref_i + grad_policy[i] * policy_i)
    with respect to the logits (rlk_logp_backward). ``ref_logp``/``lse`` come
    from logp_full (or logp_nucleus with ``return_state``), ``policy_logp`` and
    ``support_state`` from logp_nucleus; a term whose upstream gradient is None
    is absent. Upstream gradients are floats or float32 [n_rows] tensors.
    Returns a bfloat16 [n_rows, vocab_padded] tensor (or fills ``out``, a 2-D
    BF16-bits tensor whose first vocab_padded columns are written)."""
    torch = _torch()
    stride = _check_logits(logits)
    n = logits.shape[0]
    dev = logits.device
    vp = int(vocab_padded if vocab_padded is not None else logits.shape[1])
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    target = _per_row(target, n, torch.int64, dev, "target")
    if grad_ref is not None:
        grad_ref = _per_row(grad_ref, n, torch.float32, dev, "grad_ref")
        ref_logp = _per_row(ref_logp, n, torch.float32, dev, "ref_logp")
        lse = _per_row(lse, n, torch.float32, dev, "lse")
    if grad_policy is not None:
        grad_policy = _per_row(grad_policy, n, torch.float32, dev, "grad_policy")
        policy_logp = _per_row(policy_logp, n, torch.float32, dev, "policy_logp")
        if support_state is None or support_state.dtype != torch.int32 or support_state.shape != (n, 4) or \
                not support_state.is_contiguous() or support_state.device != dev:
            raise ValueError(f"support_state must be a contiguous int32 tensor of shape ({n}, 4) on {dev}")
    if out is None:
        out = torch.empty((n, vp), dtype=torch.bfloat16, device=dev)
    out_stride = _check_logits(out)
    if out.device != dev or out.shape[0] != n or out.shape[1] < vp or (out_stride % 8) != 0:
        raise ValueError(f"out must hold {n} rows of at least {vp} BF16 columns, row stride a multiple of 8, on {dev}")
    lay = make_layout(vp, vocab_real, stride, 1)

    def ptr(t):
        return t.data_ptr() if t is not None else None

    st = load_library().rlk_logp_backward(
        logits.data_ptr(), n, ctypes.byref(lay), temperature.data_ptr(), target.data_ptr(),
        ptr(ref_logp), ptr(lse), ptr(grad_ref), ptr(policy_logp), ptr(support_state), ptr(grad_policy),
        out.data_ptr(), int(out_stride), _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_logp_backward")
    return out


def logp_shard_summaries(logits_slice, temperature, target, *, rank: int, groups: int, vocab_real: int,
                         vocab_padded: int, out=None, stream=None):
    """One rank's shard summaries (rlk_logp_shard_summaries). ``logits_slice``
    is [n_rows, >= vocab_padded/groups] BF16 bits holding that rank's columns.
    Returns a uint8 tensor of rlk_logp_summary_bytes() bytes."""
    torch = _torch()
    stride = _check_logits(logits_slice)
    n = logits_slice.shape[0]
    dev = logits_slice.device
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    target = _per_row(target, n, torch.int64, dev, "target")
    lay = make_layout(vocab_padded, vocab_real, vocab_padded, groups)
    lib = load_library()
    need = int(lib.rlk_logp_summary_bytes(n, ctypes.byref(lay)))
    out, out_bytes = _workspace(out if out is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=dev),
                                need, dev, "out")
    st = lib.rlk_logp_shard_summaries(
        logits_slice.data_ptr(), n, ctypes.byref(lay), int(rank), int(stride), temperature.data_ptr(),
        target.data_ptr(), out.data_ptr(), out_bytes, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_logp_shard_summaries")
    return out


def logp_merge(summaries, temperature, target, *, n_rows: int, groups: int, vocab_real: int, vocab_padded: int,
               return_lse: bool = False, out=None, lse_out=None, stream=None):
    """Merge the rank-ordered concatenation of every rank's summaries
    (rlk_logp_merge); the result equals logp_full on the whole rows."""
    torch = _torch()
    dev = summaries.device
    temperature = _per_row(temperature, n_rows, torch.float32, dev, "temperature")
    target = _per_row(target, n_rows, torch.int64, dev, "target")
    out = _out(out, (n_rows,), torch.float32, dev, "out")
    if return_lse or lse_out is not None:
        lse_out = _out(lse_out, (n_rows,), torch.float32, dev, "lse_out")
    lay = make_layout(vocab_padded, vocab_real, vocab_padded, groups)
    if not summaries.is_contiguous():
        raise ValueError("summaries must be contiguous")
    nbytes = summaries.numel() * summaries.element_size()
    st = load_library().rlk_logp_merge(
        summaries.data_ptr(), nbytes, int(n_rows), ctypes.byref(lay), temperature.data_ptr(), target.data_ptr(),
        out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_logp_merge")
    return (out, lse_out) if return_lse else out


# ---------------------------------------------------------------------------
# gradient L2 norm (include/rlk_norm.h)
# ---------------------------------------------------------------------------

def _bins_tensor(bins, device):
    torch = _torch()
    if bins is None:
        return torch.empty(NORM_BIN_WORDS, dtype=torch.int64, device=device)
    if bins.dtype not in (torch.int64, torch.uint64) or bins.numel() != NORM_BIN_WORDS or not bins.is_contiguous() \
            or bins.device != device:
        raise ValueError(f"bins must be a contiguous 64-bit tensor of {NORM_BIN_WORDS} words on {device}")
    return bins


def _f32_flat(x):
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("values must be a contiguous float32 device tensor")
    return x


def l2norm_zero(bins, stream=None):
    """Clear an accumulator (rlk_l2norm_zero)."""
    bins = _bins_tensor(bins, bins.device)
    st = load_library().rlk_l2norm_zero(bins.data_ptr(), _stream_handle(stream, bins.device))
    if st != RLK_OK:
        raise RlkError(st, "rlk_l2norm_zero")
    return bins


def l2norm_accumulate(x, bins, stream=None):
    """Add the float32 squares of ``x`` to ``bins`` (rlk_l2norm_accumulate)."""
    x = _f32_flat(x)
    bins = _bins_tensor(bins, x.device)
    st = load_library().rlk_l2norm_accumulate(x.data_ptr() if x.numel() else None, x.numel(), bins.data_ptr(),
                                              _stream_handle(stream, bins.device))
    if st != RLK_OK:
        raise RlkError(st, "rlk_l2norm_accumulate")
    return bins


def l2norm_finalize(bins, sumsq_out=None, norm_out=None, stream=None):
    """(sum of squares float64 [1], norm float32 [1]) from ``bins`` (rlk_l2norm_finalize)."""
    torch = _torch()
    dev = bins.device
    bins = _bins_tensor(bins, dev)
    sumsq_out = _out(sumsq_out, (1,), torch.float64, dev, "sumsq_out")
    norm_out = _out(norm_out, (1,), torch.float32, dev, "norm_out")
    st = load_library().rlk_l2norm_finalize(bins.data_ptr(), sumsq_out.data_ptr(), norm_out.data_ptr(),
                                            _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_l2norm_finalize")
    return sumsq_out, norm_out


def l2norm(xs, *, workspace=None, sumsq_out=None, norm_out=None, stream=None):
    """Order-independent L2 norm of one float32 device tensor (rlk_l2norm, one
    launch) or of a list of them (zero + one accumulate per tensor +
    finalize). Returns (sum of squares float64 [1], norm float32 [1]).
    ``workspace`` (264 int64 words) must be all-zero when given for a single
    tensor; rlk_l2norm leaves it all-zero."""
    torch = _torch()
    if isinstance(xs, (list, tuple)):
        if not xs:
            raise ValueError("l2norm needs at least one tensor")
        bins = _bins_tensor(workspace, xs[0].device)
        l2norm_zero(bins, stream)
        for x in xs:
            l2norm_accumulate(x, bins, stream)
        return l2norm_finalize(bins, sumsq_out, norm_out, stream)
    x = _f32_flat(xs)
    dev = x.device
    ws = workspace if workspace is not None else torch.zeros(NORM_BIN_WORDS, dtype=torch.int64, device=dev)
    ws = _bins_tensor(ws, dev)
    sumsq_out = _out(sumsq_out, (1,), torch.float64, dev, "sumsq_out")
    norm_out = _out(norm_out, (1,), torch.float32, dev, "norm_out")
    st = load_library().rlk_l2norm(x.data_ptr() if x.numel() else None, x.numel(), ws.data_ptr(),
                                   sumsq_out.data_ptr(), norm_out.data_ptr(), _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_l2norm")
    return sumsq_out, norm_out


# ---------------------------------------------------------------------------
# LM-head linear and fused linear + logprob (include/rlk_linear.h)
# ---------------------------------------------------------------------------

def _bf16_matrix(x, name):
    torch = _torch()
    if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not x.is_cuda or x.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D device tensor of BF16 bits with contiguous rows")
    return x.stride(0) if x.shape[0] > 1 else max(x.stride(0), x.shape[1])


def linear_logp_workspace_bytes(n_rows: int, vocab_padded: int, vocab_real: int) -> int:
    lay = make_layout(vocab_padded, vocab_real, vocab_padded)
    return int(load_library().rlk_linear_logp_workspace_bytes(int(n_rows), ctypes.byref(lay)))


def linear(hidden, weight, *, vocab_padded: int, out=None, stream=None):
    """BF16 logits bf16(hidden . weight^T) [n_rows, vocab_padded], pads -inf (rlk_linear).
    ``weight`` holds the vocab_real rows of the projection."""
    torch = _torch()
    ldh = _bf16_matrix(hidden, "hidden")
    ldw = _bf16_matrix(weight, "weight")
    n, d = hidden.shape
    vr = weight.shape[0]
    if weight.shape[1] != d:
        raise ValueError("hidden and weight must have the same d_model")
    if out is None:
        out = torch.empty((n, vocab_padded), dtype=torch.bfloat16, device=hidden.device)
    ldo = _check_logits(out)
    if out.device != hidden.device or out.shape[0] != n or out.shape[1] < vocab_padded or (ldo % 8) != 0:
        raise ValueError(f"out must hold {n} rows of at least {vocab_padded} BF16 columns, row stride a multiple "
                         f"of 8, on {hidden.device}")
    if weight.device != hidden.device:
        raise ValueError("hidden and weight must be on the same device")
    lay = make_layout(vocab_padded, vr, ldo)
    st = load_library().rlk_linear(hidden.data_ptr(), n, d, ldh, weight.data_ptr(), ldw, ctypes.byref(lay),
                                   out.data_ptr(), _stream_handle(stream, hidden.device))
    if st != RLK_OK:
        raise RlkError(st, "rlk_linear")
    return out


def linear_logp(hidden, weight, temperature, target, *, vocab_padded: int, return_lse: bool = False, out=None,
                lse_out=None, workspace=None, stream=None):
    """Reference logprob of ``target`` from bf16(hidden . weight^T) without writing
    the logits (rlk_linear_logp)."""
    torch = _torch()
    ldh = _bf16_matrix(hidden, "hidden")
    ldw = _bf16_matrix(weight, "weight")
    n, d = hidden.shape
    vr = weight.shape[0]
    dev = hidden.device
    if weight.shape[1] != d:
        raise ValueError("hidden and weight must have the same d_model")
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    target = _per_row(target, n, torch.int64, dev, "target")
    out = _out(out, (n,), torch.float32, dev, "out")
    if return_lse or lse_out is not None:
        lse_out = _out(lse_out, (n,), torch.float32, dev, "lse_out")
    lay = make_layout(vocab_padded, vr, vocab_padded)
    lib = load_library()
    need = int(lib.rlk_linear_logp_workspace_bytes(n, ctypes.byref(lay)))
    workspace, ws_bytes = _workspace(
        workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=dev), need, dev)
    st = lib.rlk_linear_logp(hidden.data_ptr(), n, d, ldh, weight.data_ptr(), ldw, ctypes.byref(lay),
                             temperature.data_ptr(), target.data_ptr(), out.data_ptr(),
                             lse_out.data_ptr() if lse_out is not None else None, workspace.data_ptr(),
                             ws_bytes, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_linear_logp")
    return (out, lse_out) if return_lse else out


def linear_logp_summaries(hidden, weight_shard, temperature, target, *, rank: int, groups: int, vocab_real: int,
                          vocab_padded: int, out=None, stream=None):
    """One rank's 128-column summaries of bf16(hidden . weight^T) over its columns
    [rank*C, (rank+1)*C), C = vocab_padded / groups (rlk_linear_logp_summaries).
    ``weight_shard`` holds that rank's projection rows below vocab_real."""
    torch = _torch()
    ldh = _bf16_matrix(hidden, "hidden")
    ldw = _bf16_matrix(weight_shard, "weight_shard")
    n, d = hidden.shape
    dev = hidden.device
    temperature = _per_row(temperature, n, torch.float32, dev, "temperature")
    target = _per_row(target, n, torch.int64, dev, "target")
    lay = make_layout(vocab_padded, vocab_real, vocab_padded, groups)
    lib = load_library()
    need = int(lib.rlk_linear_logp_summary_bytes(n, ctypes.byref(lay)))
    out, out_bytes = _workspace(out if out is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=dev),
                                need, dev, "out")
    st = lib.rlk_linear_logp_summaries(hidden.data_ptr(), n, d, ldh, weight_shard.data_ptr(), ldw, ctypes.byref(lay),
                                       int(rank), temperature.data_ptr(), target.data_ptr(), out.data_ptr(),
                                       out_bytes, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_linear_logp_summaries")
    return out


def linear_logp_merge(summaries, temperature, target, *, n_rows: int, groups: int, vocab_real: int,
                      vocab_padded: int, return_lse: bool = False, out=None, lse_out=None, stream=None):
    """Merge every rank's linear-logp summaries, concatenated in rank order
    (rlk_linear_logp_merge); equals rlk_linear_logp on the whole projection."""
    torch = _torch()
    dev = summaries.device
    temperature = _per_row(temperature, n_rows, torch.float32, dev, "temperature")
    target = _per_row(target, n_rows, torch.int64, dev, "target")
    out = _out(out, (n_rows,), torch.float32, dev, "out")
    if return_lse or lse_out is not None:
        lse_out = _out(lse_out, (n_rows,), torch.float32, dev, "lse_out")
    lay = make_layout(vocab_padded, vocab_real, vocab_padded, groups)
    if not summaries.is_contiguous():
        raise ValueError("summaries must be contiguous")
    nbytes = summaries.numel() * summaries.element_size()
    st = load_library().rlk_linear_logp_merge(
        summaries.data_ptr(), nbytes, int(n_rows), ctypes.byref(lay), temperature.data_ptr(), target.data_ptr(),
        out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None, _stream_handle(stream, dev))
    if st != RLK_OK:
        raise RlkError(st, "rlk_linear_logp_merge")
    return (out, lse_out) if return_lse else out
