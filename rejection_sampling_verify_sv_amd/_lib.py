"""ctypes binding of libsv.so (the C ABI in include/sv.h).

Argument marshalling only: every step of the verify computation runs in the
HIP kernels of the library.  Torch supplies device memory and the stream.
There is no fallback: if the library is missing or the tensors are not on a
GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsv.so")

SV_F32, SV_BF16 = 0, 1
SV_MAX_TOP_K = 64
ERRORS = {0: "SV_OK", -1: "SV_EINVAL", -2: "SV_EWORKSPACE", -3: "SV_EHIP", -4: "SV_ESCRATCH"}
EXPORTED = ("sv_verify", "sv_verify_profiled", "sv_sample", "sv_accept_stats",
            "sv_workspace_bytes", "sv_strerror", "sv_launch_count", "sv_launch_name",
            "sv_stream_read", "sv_verify_tree", "sv_verify_noalloc", "sv_noalloc_scratch_bytes")


class SvConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("max_draft", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("target_row_stride", ctypes.c_int64),
        ("draft_row_stride", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("diag", ctypes.c_void_p),
        ("step_mode", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libsv.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.sv_workspace_bytes.restype = ctypes.c_size_t
        lib.sv_workspace_bytes.argtypes = [ctypes.c_int32] * 4
        lib.sv_verify.restype = ctypes.c_int
        lib.sv_verify.argtypes = [ctypes.c_void_p] * 8 + [ctypes.POINTER(SvConfig)]
        lib.sv_verify_profiled.restype = ctypes.c_int
        lib.sv_verify_profiled.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.POINTER(SvConfig)]
                                           + [ctypes.c_void_p, ctypes.c_int32])
        lib.sv_sample.restype = ctypes.c_int
        lib.sv_sample.argtypes = [ctypes.c_void_p] * 5 + [ctypes.POINTER(SvConfig)]
        lib.sv_accept_stats.restype = ctypes.c_int
        lib.sv_accept_stats.argtypes = [ctypes.c_void_p] * 4 + [ctypes.POINTER(SvConfig)]
        lib.sv_strerror.restype = ctypes.c_char_p
        lib.sv_strerror.argtypes = [ctypes.c_int]
        lib.sv_launch_count.restype = ctypes.c_int32
        lib.sv_launch_count.argtypes = [ctypes.c_int32] * 3
        lib.sv_verify_tree.restype = ctypes.c_int
        lib.sv_verify_tree.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int32, ctypes.c_int32]
                                       + [ctypes.POINTER(SvConfig)])
        lib.sv_verify_noalloc.restype = ctypes.c_int
        lib.sv_verify_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.POINTER(SvConfig)]
        lib.sv_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.sv_stream_read.restype = ctypes.c_int
        lib.sv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_void_p]
        lib.sv_launch_name.restype = ctypes.c_char_p
        lib.sv_launch_name.argtypes = [ctypes.c_int32] * 4
        _lib = lib
    return _lib


_WS_BYTES = {}


def workspace_bytes(batch: int, max_draft: int, vocab: int, dtype: int) -> int:
    key = (batch, max_draft, vocab, dtype)
    n = _WS_BYTES.get(key)
    if n is None:
        n = _WS_BYTES[key] = int(load().sv_workspace_bytes(batch, max_draft, vocab, dtype))
    return n


def _as(t: torch.Tensor, dev, dtype) -> torch.Tensor:
    """t on dev as a contiguous tensor of dtype, without a copy (or a call
    into torch) when it already is one."""
    if t.dtype != dtype or t.device != dev:
        t = t.to(dev, dtype)
    return t if t.is_contiguous() else t.contiguous()


def _raw_stream(dev) -> int:
    """Handle of the current stream of device dev."""
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is not None:
        return get(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


SV_STEP_AUTO, SV_STEP_POSITIONS, SV_STEP_DENSE = 0, 1, 2
STEP_MODES = {"auto": SV_STEP_AUTO, "positions": SV_STEP_POSITIONS, "dense": SV_STEP_DENSE}


def launch_names(batch: int, max_draft: int, step_mode: str = "auto") -> list:
    lib = load()
    m = STEP_MODES[step_mode]
    return [lib.sv_launch_name(batch, max_draft, m, i).decode()
            for i in range(lib.sv_launch_count(batch, max_draft, m))]


def stream_read(data: torch.Tensor, out: torch.Tensor, stream: torch.cuda.Stream | None = None):
    """Enqueue sv_stream_read over the bytes of ``data`` (a contiguous CUDA
    tensor, 16-byte aligned, size a multiple of 16); ``out`` is a zeroed
    one-element int32 CUDA tensor.  A measurement aid: the sustainable
    streaming-read rate with the row pass's tiling."""
    lib = load()
    if not (data.is_cuda and out.is_cuda and data.is_contiguous()):
        raise RuntimeError("stream_read needs contiguous GPU tensors")
    st = stream if stream is not None else torch.cuda.current_stream(data.device)
    rc = lib.sv_stream_read(data.data_ptr(), data.numel() * data.element_size(), out.data_ptr(),
                            st.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"sv_stream_read failed: {ERRORS.get(rc, rc)}: "
                           f"{lib.sv_strerror(rc).decode()}")


def params_tensor(params, device) -> torch.Tensor:
    """Sampler parameters as a [B, 4] int32 device tensor holding the 16-byte
    {float temperature, int32 top_k, float top_p, int32 reserved} records.
    Accepts a numpy structured array or an existing [B, 4] int32 tensor."""
    if isinstance(params, torch.Tensor):
        if params.dtype != torch.int32 or params.dim() != 2 or params.shape[1] != 4:
            raise TypeError("params tensor must be [B, 4] int32")
        return _as(params, device, torch.int32)
    arr = np.ascontiguousarray(params)
    if arr.dtype.itemsize != 16:
        raise TypeError("params must be 16-byte records")
    raw = arr.view(np.int32).reshape(-1, 4)
    return torch.from_numpy(raw.copy()).to(device)


def _rows_layout(t: torch.Tensor, nrows: int):
    """(tensor, row_stride) such that row r = (b, k) starts at r * stride."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
        t = t.contiguous()
    return t, t.stride(1)


def verify(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
           draft_len: torch.Tensor | None, params, uniforms: torch.Tensor, *,
           diag: bool = False, workspace: torch.Tensor | None = None,
           out_tokens: torch.Tensor | None = None, out_accept_len: torch.Tensor | None = None,
           stream: torch.cuda.Stream | None = None, events=None, step_mode: str = "auto"):
    """Enqueue one verify step; returns (out_tokens, out_accept_len, diag|None).

    target [B, K+1, V], draft [B, K, V]: float32 or bfloat16 CUDA tensors.
    draft_tokens [B, K] int32; draft_len [B] int32 or None; params as in
    params_tensor(); uniforms [B, K+1] float32.  With K = 0, draft and
    draft_tokens may be None.  step_mode: "auto", "positions" or "dense"
    (see sv_config.step_mode).  Nothing is synchronised.
    """
    lib = load()
    if not target.is_cuda:
        raise RuntimeError("verify needs GPU tensors (no CPU path exists)")
    dev = target.device
    if target.dtype == torch.float32:
        code = SV_F32
    elif target.dtype == torch.bfloat16:
        code = SV_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    B, K1, V = target.shape
    K = K1 - 1
    target, ts = _rows_layout(target, B * K1)
    if K == 0 and draft is None:
        ds = 0
    else:
        if draft.dtype != target.dtype or draft.device != dev:
            raise TypeError("draft must match target's dtype and device")
        if tuple(draft.shape) != (B, K, V):
            raise ValueError(f"draft shape {tuple(draft.shape)} != {(B, K, V)}")
        draft, ds = _rows_layout(draft, B * K) if K > 0 else (None, 0)
    tok = None
    if K > 0 or draft_tokens is not None:
        tok = _as(draft_tokens, dev, torch.int32)
        if tuple(tok.shape) != (B, K):
            raise ValueError("draft_tokens must be [B, K]")
        if K == 0:
            tok = None
    dl = None
    if draft_len is not None:
        dl = _as(draft_len, dev, torch.int32)
        if tuple(dl.shape) != (B,):
            raise ValueError("draft_len must be [B]")
    prm = params_tensor(params, dev)
    if prm.shape[0] != B:
        raise ValueError("params must have B rows")
    uni = _as(uniforms, dev, torch.float32)
    if tuple(uni.shape) != (B, K1):
        raise ValueError("uniforms must be [B, K+1]")
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if out_accept_len is None:
        out_accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    dg = torch.empty((B, K1, 4), dtype=torch.float64, device=dev) if diag else None
    need = workspace_bytes(B, K, V, code)
    if need == 0:
        raise ValueError("invalid shape for sv_verify")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wptr = workspace.data_ptr()
    pad = (-wptr) % 256
    cfg = SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = B, K, V, code
    cfg.target_row_stride, cfg.draft_row_stride = ts, ds
    cfg.stream = stream.cuda_stream if stream is not None else _raw_stream(dev)
    cfg.workspace = wptr + pad
    cfg.workspace_bytes = workspace.numel() * workspace.element_size() - pad
    cfg.diag = dg.data_ptr() if dg is not None else None
    cfg.step_mode = STEP_MODES[step_mode]
    args = (target.data_ptr(), draft.data_ptr() if draft is not None else None,
            tok.data_ptr() if tok is not None else None,
            dl.data_ptr() if dl is not None else None, prm.data_ptr(), uni.data_ptr(),
            out_tokens.data_ptr(), out_accept_len.data_ptr(), ctypes.byref(cfg))
    if events is None:
        rc = lib.sv_verify(*args)
    else:  # events: a ctypes array of hipEvent_t handles (see sv_verify_profiled)
        rc = lib.sv_verify_profiled(*args, ctypes.cast(events, ctypes.c_void_p), len(events))
    if rc != 0:
        raise RuntimeError(f"sv_verify failed: {ERRORS.get(rc, rc)}: "
                           f"{lib.sv_strerror(rc).decode()}")
    if stream is not None:
        # temporaries were allocated on the current stream; keep them alive
        # until the work enqueued on `stream` has finished
        for t in (target, draft, tok, dl, prm, uni, workspace, out_tokens, out_accept_len, dg):
            if t is not None:
                t.record_stream(stream)
    return out_tokens, out_accept_len, dg


def verify_tree(target: torch.Tensor, draft: torch.Tensor | None, node_tokens: torch.Tensor | None,
                node_parents: torch.Tensor | None, n_cand: torch.Tensor | None, params,
                uniforms: torch.Tensor, *, max_depth: int, max_children: int, diag: bool = False,
                workspace: torch.Tensor | None = None, out_tokens: torch.Tensor | None = None,
                out_accept_len: torch.Tensor | None = None, out_path: torch.Tensor | None = None,
                stream: torch.cuda.Stream | None = None):
    """Enqueue one tree verify (sv_verify_tree); returns (out_tokens,
    out_accept_len, out_path, diag|None).

    target [B, K+1, V] (row v = node v), draft [B, K, V] (row v = node v):
    float32 or bfloat16 CUDA tensors.  node_tokens, node_parents [B, K] int32
    (entry c-1 = candidate node c); n_cand [B] int32 or None; params as in
    params_tensor(); uniforms [B, K+1] float32 (column c-1 tests node c,
    column K the final draw).  Nothing is synchronised."""
    lib = load()
    if not target.is_cuda:
        raise RuntimeError("verify_tree needs GPU tensors (no CPU path exists)")
    dev = target.device
    if target.dtype == torch.float32:
        code = SV_F32
    elif target.dtype == torch.bfloat16:
        code = SV_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    B, K1, V = target.shape
    K = K1 - 1
    target, ts = _rows_layout(target, B * K1)
    ds = 0
    if K > 0:
        if draft is None or draft.dtype != target.dtype or tuple(draft.shape) != (B, K, V):
            raise ValueError("draft must be [B, K, V] of target's dtype")
        draft, ds = _rows_layout(draft, B * K)
    tok = par = None
    if K > 0:
        tok = node_tokens.to(dev, torch.int32).contiguous()
        par = node_parents.to(dev, torch.int32).contiguous()
        if tuple(tok.shape) != (B, K) or tuple(par.shape) != (B, K):
            raise ValueError("node_tokens and node_parents must be [B, K]")
    nc = None
    if n_cand is not None:
        nc = n_cand.to(dev, torch.int32).contiguous()
        if tuple(nc.shape) != (B,):
            raise ValueError("n_cand must be [B]")
    prm = params_tensor(params, dev)
    if prm.shape[0] != B:
        raise ValueError("params must have B rows")
    uni = uniforms.to(dev, torch.float32).contiguous()
    if tuple(uni.shape) != (B, K1):
        raise ValueError("uniforms must be [B, K+1]")
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if out_accept_len is None:
        out_accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_path is None:
        out_path = torch.empty((B, K1), dtype=torch.int32, device=dev)
    dg = torch.empty((B, K1, 4), dtype=torch.float64, device=dev) if diag else None
    need = workspace_bytes(B, K, V, code)
    if need == 0:
        raise ValueError("invalid shape for sv_verify_tree")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wptr = workspace.data_ptr()
    pad = (-wptr) % 256
    cfg = SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = B, K, V, code
    cfg.target_row_stride, cfg.draft_row_stride = ts, ds
    cfg.stream = stream.cuda_stream if stream is not None else _raw_stream(dev)
    cfg.workspace = wptr + pad
    cfg.workspace_bytes = workspace.numel() * workspace.element_size() - pad
    cfg.diag = dg.data_ptr() if dg is not None else None
    rc = lib.sv_verify_tree(target.data_ptr(), draft.data_ptr() if draft is not None else None,
                            tok.data_ptr() if tok is not None else None,
                            par.data_ptr() if par is not None else None,
                            nc.data_ptr() if nc is not None else None, prm.data_ptr(),
                            uni.data_ptr(), out_tokens.data_ptr(), out_accept_len.data_ptr(),
                            out_path.data_ptr(), int(max_depth), int(max_children),
                            ctypes.byref(cfg))
    if rc != 0:
        raise RuntimeError(f"sv_verify_tree failed: {ERRORS.get(rc, rc)}: "
                           f"{lib.sv_strerror(rc).decode()}")
    if stream is not None:
        for t in (target, draft, tok, par, nc, prm, uni, workspace, out_tokens, out_accept_len,
                  out_path, dg):
            if t is not None:
                t.record_stream(stream)
    return out_tokens, out_accept_len, out_path, dg


def sample(logits: torch.Tensor, params, uniforms: torch.Tensor, *, diag: bool = False,
           workspace: torch.Tensor | None = None, out_tokens: torch.Tensor | None = None,
           out_status: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Enqueue one draw per row from the truncated distribution of each row of
    logits [B, V] (float32 or bfloat16 CUDA tensor; rows may be strided).
    params as in params_tensor(); uniforms [B] float32.  Returns
    (out_tokens [B] int32, out_status [B] int32, diag [B, 1, 4] | None).
    Nothing is synchronised."""
    lib = load()
    if not logits.is_cuda:
        raise RuntimeError("sample needs GPU tensors (no CPU path exists)")
    dev = logits.device
    if logits.dtype == torch.float32:
        code = SV_F32
    elif logits.dtype == torch.bfloat16:
        code = SV_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    if logits.stride(1) != 1:
        logits = logits.contiguous()
    prm = params_tensor(params, dev)
    if prm.shape[0] != B:
        raise ValueError("params must have B rows")
    uni = uniforms.to(dev, torch.float32).contiguous().reshape(-1)
    if uni.shape[0] != B:
        raise ValueError("uniforms must be [B]")
    if out_tokens is None:
        out_tokens = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_status is None:
        out_status = torch.empty((B,), dtype=torch.int32, device=dev)
    dg = torch.empty((B, 1, 4), dtype=torch.float64, device=dev) if diag else None
    need = workspace_bytes(B, 0, V, code)
    if need == 0:
        raise ValueError("invalid shape for sv_sample")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wptr = workspace.data_ptr()
    pad = (-wptr) % 256
    cfg = SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = B, 0, V, code
    cfg.target_row_stride = logits.stride(0)
    cfg.stream = stream.cuda_stream if stream is not None else _raw_stream(dev)
    cfg.workspace = wptr + pad
    cfg.workspace_bytes = workspace.numel() * workspace.element_size() - pad
    cfg.diag = dg.data_ptr() if dg is not None else None
    rc = lib.sv_sample(logits.data_ptr(), prm.data_ptr(), uni.data_ptr(), out_tokens.data_ptr(),
                       out_status.data_ptr(), ctypes.byref(cfg))
    if rc != 0:
        raise RuntimeError(f"sv_sample failed: {ERRORS.get(rc, rc)}: "
                           f"{lib.sv_strerror(rc).decode()}")
    if stream is not None:
        for t in (logits, prm, uni, workspace, out_tokens, out_status, dg):
            if t is not None:
                t.record_stream(stream)
    return out_tokens, out_status, dg


def accept_stats(target: torch.Tensor, draft: torch.Tensor, params, *,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Enqueue the acceptance statistics of one draft position (sv_accept_stats):
    target and draft logits [B, V] (float32 or bfloat16 CUDA tensors of one
    dtype; rows may be strided), params as in params_tensor().  Returns out
    [B, 4] float64: sum min(p, q), sum p q, sum min(p~, q), sum min(p~, q~).
    Nothing is synchronised."""
    lib = load()
    if not (target.is_cuda and draft.is_cuda):
        raise RuntimeError("accept_stats needs GPU tensors (no CPU path exists)")
    dev = target.device
    if target.dtype != draft.dtype:
        raise TypeError("target and draft must share a dtype")
    if target.dtype == torch.float32:
        code = SV_F32
    elif target.dtype == torch.bfloat16:
        code = SV_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    if target.dim() != 2 or draft.dim() != 2 or target.shape != draft.shape:
        raise ValueError("target and draft must both be [B, V]")
    B, V = target.shape
    if target.stride(1) != 1:
        target = target.contiguous()
    if draft.stride(1) != 1:
        draft = draft.contiguous()
    prm = params_tensor(params, dev)
    if prm.shape[0] != B:
        raise ValueError("params must have B rows")
    if out is None:
        out = torch.empty((B, 4), dtype=torch.float64, device=dev)
    need = workspace_bytes(B, 1, V, code)
    if need == 0:
        raise ValueError("invalid shape for sv_accept_stats")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wptr = workspace.data_ptr()
    pad = (-wptr) % 256
    cfg = SvConfig()
    cfg.batch, cfg.max_draft, cfg.vocab, cfg.dtype = B, 1, V, code
    cfg.target_row_stride, cfg.draft_row_stride = target.stride(0), draft.stride(0)
    cfg.stream = stream.cuda_stream if stream is not None else _raw_stream(dev)
    cfg.workspace = wptr + pad
    cfg.workspace_bytes = workspace.numel() * workspace.element_size() - pad
    cfg.diag = None
    rc = lib.sv_accept_stats(target.data_ptr(), draft.data_ptr(), prm.data_ptr(), out.data_ptr(),
                             ctypes.byref(cfg))
    if rc != 0:
        raise RuntimeError(f"sv_accept_stats failed: {ERRORS.get(rc, rc)}: "
                           f"{lib.sv_strerror(rc).decode()}")
    if stream is not None:
        for t in (target, draft, prm, workspace, out):
            t.record_stream(stream)
    return out
