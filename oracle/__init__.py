"""CPU oracle for the speculative-sampling verify step (fp64, plain C).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never calls it and shares no code with it.

The arithmetic lives in ``sv_oracle.c`` (see its header for the page
citations and the readings R1-R12 of the points the pages leave open); this
module only loads the compiled library and marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, exact enumeration on tiny vocabularies, hand-worked fixtures under
``tests/golden/`` and a Monte-Carlo chi-square test.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB = os.path.join(_HERE, "libsv_oracle.so")

PARAMS_DTYPE = np.dtype(
    [("temperature", "<f4"), ("top_k", "<i4"), ("top_p", "<f4"), ("reserved", "<i4")]
)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = [
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.sv_oracle_verify.restype = ctypes.c_int
        lib.sv_oracle_verify.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.sv_oracle_explain.restype = ctypes.c_int
        lib.sv_oracle_explain.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.sv_oracle_verify_tree.restype = ctypes.c_int
        lib.sv_oracle_verify_tree.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 9 + [ctypes.c_int]
        lib.sv_oracle_explain_tree.restype = ctypes.c_int
        lib.sv_oracle_explain_tree.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 13 + [ctypes.c_int]
        lib.sv_oracle_dist.restype = ctypes.c_int
        lib.sv_oracle_dist.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p,
        ]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def verify(target, draft, tokens, draft_len, params, uniforms, *, dtype="f32",
           nthreads: int = 0):
    """Run the oracle on host arrays.

    target: [B, K+1, V] float32 (dtype="f32") or uint16 bf16 bit patterns
    (dtype="bf16"); draft: [B, K, V] same dtype; tokens [B, K] int32;
    draft_len [B] int32 or None; params [B] PARAMS_DTYPE; uniforms [B, K+1]
    float32.  Returns (out_tokens [B, K+1], accept_len [B], diag [B, K+1, 4],
    cut_margin [B], threads_used).
    """
    lib = _load()
    code = {"f32": 0, "bf16": 1}[dtype]
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    want = np.float32 if code == 0 else np.uint16
    if target.dtype != want:
        raise TypeError(f"target must be {want.__name__} for dtype={dtype}")
    if K > 0:
        draft = np.ascontiguousarray(draft)
        if draft.shape != (B, K, V) or draft.dtype != want:
            raise TypeError("draft must be [B, K, V] of the same dtype as target")
    else:
        draft = None
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, max(K, 0))
    if tokens.size == 0:
        tokens = np.zeros((B, 1), np.int32)
    if draft_len is not None:
        draft_len = np.ascontiguousarray(draft_len, dtype=np.int32).reshape(B)
    params = np.ascontiguousarray(params)
    if params.dtype != PARAMS_DTYPE or params.shape != (B,):
        raise TypeError("params must be [B] of PARAMS_DTYPE")
    uniforms = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K + 1)
    out_tok = np.empty((B, K + 1), np.int32)
    acc = np.empty(B, np.int32)
    diag = np.empty((B, K + 1, 4), np.float64)
    cut = np.empty(B, np.float64)
    used = lib.sv_oracle_verify(
        _ptr(target), _ptr(draft), code, B, K, V, V, V, _ptr(tokens), _ptr(draft_len),
        _ptr(params), _ptr(uniforms), _ptr(out_tok), _ptr(acc), _ptr(diag), _ptr(cut),
        int(nthreads),
    )
    if used < 0:
        raise ValueError("sv_oracle_verify rejected its arguments")
    return out_tok, acc, diag, cut, used


def explain(target, draft, tokens, draft_len, params, acc, y, *, dtype="f32",
            nthreads: int = 0):
    """The rule's decisions along given outcomes (accept length ``acc[b]``,
    final token ``y[b]``) of rows laid out as for ``verify`` (K = 0: the one
    draw per row of ``sample``).

    Returns a dict of arrays: ``a``, ``px``, ``qx`` [B, K] (accept
    probability and p(x), q(x) of each draft the outcome reaches: positions
    0..min(acc, L-1), NaN past them); ``lo``, ``hi`` [B] (edges of y's bin in
    the inverse CDF of the final distribution: the residual at acc when
    acc < L, p at L otherwise); ``py`` [B] (probability of y under it);
    ``status`` [B] (0, 1 for a greedy row, -1 invalid row or outcome).  An
    outcome is what the rule gives for uniforms u' iff u'_j < a_j for j < acc,
    u'_acc >= a_acc when acc < L, lo <= u'_K < hi and py > 0."""
    lib = _load()
    code = {"f32": 0, "bf16": 1}[dtype]
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    draft = np.ascontiguousarray(draft) if K > 0 else None
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, K)
    if K == 0:
        tokens = np.zeros((B, 1), np.int32)
    if draft_len is not None:
        draft_len = np.ascontiguousarray(draft_len, dtype=np.int32).reshape(B)
    params = np.ascontiguousarray(params)
    acc = np.ascontiguousarray(acc, dtype=np.int32).reshape(B)
    y = np.ascontiguousarray(y, dtype=np.int32).reshape(B)
    out = {n: np.empty((B, max(K, 1)), np.float64) for n in ("a", "px", "qx")}
    out.update({n: np.empty(B, np.float64) for n in ("lo", "hi", "py")})
    out["status"] = np.empty(B, np.int32)
    used = lib.sv_oracle_explain(
        _ptr(target), _ptr(draft), code, B, K, V, V, V, _ptr(tokens), _ptr(draft_len),
        _ptr(params), _ptr(acc), _ptr(y), _ptr(out["a"]), _ptr(out["px"]), _ptr(out["qx"]),
        _ptr(out["lo"]), _ptr(out["hi"]), _ptr(out["py"]), _ptr(out["status"]), int(nthreads))
    if used < 0:
        raise ValueError("sv_oracle_explain rejected its arguments")
    for n in ("a", "px", "qx"):
        out[n] = out[n][:, :K]
    return out


def _tree_args(target, draft, tok, par, n_cand, params, dtype):
    code = {"f32": 0, "bf16": 1}[dtype]
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    want = np.float32 if code == 0 else np.uint16
    if target.dtype != want:
        raise TypeError(f"target must be {want.__name__} for dtype={dtype}")
    draft = np.ascontiguousarray(draft) if K > 0 else None
    if draft is not None and (draft.shape != (B, K, V) or draft.dtype != want):
        raise TypeError("draft must be [B, K, V] of the same dtype as target")
    tok = np.ascontiguousarray(tok, dtype=np.int32).reshape(B, K)
    par = np.ascontiguousarray(par, dtype=np.int32).reshape(B, K)
    if K == 0:
        tok = np.zeros((B, 1), np.int32)
        par = np.zeros((B, 1), np.int32)
    if n_cand is not None:
        n_cand = np.ascontiguousarray(n_cand, dtype=np.int32).reshape(B)
    params = np.ascontiguousarray(params)
    if params.dtype != PARAMS_DTYPE or params.shape != (B,):
        raise TypeError("params must be [B] of PARAMS_DTYPE")
    return code, target, draft, tok, par, n_cand, params, B, K, V


def verify_tree(target, draft, tokens, parents, n_cand, params, uniforms, *, dtype="f32",
                nthreads: int = 0):
    """Tree / multi-candidate verify on host arrays (see sv_oracle_verify_tree
    in sv_oracle.c for the rule, readings R17-R20).

    target [B, K+1, V] (row v = node v), draft [B, K, V] (row v = node v < K),
    tokens / parents [B, K] int32 (entry c-1 = candidate node c; parent in
    [0, c)), n_cand [B] in [0, K] or None, params [B] PARAMS_DTYPE,
    uniforms [B, K+1] float32 (column c-1 tests node c, column K the final
    draw).  Returns (out_tokens [B, K+1], out_len [B] (accepted path length,
    -1 invalid row), out_path [B, K+1] (accepted nodes, -1 padded),
    diag [B, K+1, 4], threads_used)."""
    lib = _load()
    code, target, draft, tok, par, n_cand, params, B, K, V = _tree_args(
        target, draft, tokens, parents, n_cand, params, dtype)
    uniforms = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K + 1)
    out_tok = np.empty((B, K + 1), np.int32)
    out_len = np.empty(B, np.int32)
    out_path = np.empty((B, K + 1), np.int32)
    diag = np.empty((B, K + 1, 4), np.float64)
    used = lib.sv_oracle_verify_tree(
        _ptr(target), _ptr(draft), code, B, K, V, V, V, _ptr(tok), _ptr(par), _ptr(n_cand),
        _ptr(params), _ptr(uniforms), _ptr(out_tok), _ptr(out_len), _ptr(out_path), _ptr(diag),
        int(nthreads))
    if used < 0:
        raise ValueError("sv_oracle_verify_tree rejected its arguments")
    return out_tok, out_len, out_path, diag, used


def explain_tree(target, draft, tokens, parents, n_cand, params, path, length, y, *,
                 dtype="f32", nthreads: int = 0):
    """The tree rule's decisions along given outcomes: accepted nodes
    ``path[b, :length[b]]`` and final token ``y[b]``.  Returns a dict:
    ``a`` [B, K] (accept probability of node c's test at [c-1], NaN if the
    outcome does not test c), ``need`` [B, K] (+1 accepted, -1 rejected, 0
    untested), ``lo``, ``hi``, ``py`` [B] (y's bin and probability in the final
    draw) and ``status`` [B] (0, 1 greedy row, -1 invalid row or outcome)."""
    lib = _load()
    code, target, draft, tok, par, n_cand, params, B, K, V = _tree_args(
        target, draft, tokens, parents, n_cand, params, dtype)
    path = np.ascontiguousarray(path, dtype=np.int32).reshape(B, K + 1)
    length = np.ascontiguousarray(length, dtype=np.int32).reshape(B)
    y = np.ascontiguousarray(y, dtype=np.int32).reshape(B)
    Kc = max(K, 1)
    out = {"a": np.empty((B, Kc), np.float64), "need": np.empty((B, Kc), np.int32)}
    out.update({n: np.empty(B, np.float64) for n in ("lo", "hi", "py")})
    out["status"] = np.empty(B, np.int32)
    used = lib.sv_oracle_explain_tree(
        _ptr(target), _ptr(draft), code, B, K, V, V, V, _ptr(tok), _ptr(par), _ptr(n_cand),
        _ptr(params), _ptr(path), _ptr(length), _ptr(y), _ptr(out["a"]), _ptr(out["need"]),
        _ptr(out["lo"]), _ptr(out["hi"]), _ptr(out["py"]), _ptr(out["status"]), int(nthreads))
    if used < 0:
        raise ValueError("sv_oracle_explain_tree rejected its arguments")
    out["a"], out["need"] = out["a"][:, :K], out["need"][:, :K]
    return out


def dist(logits, temperature: float, top_k: int, top_p: float):
    """Truncated tempered distribution of one fp64 logits row (T > 0).

    Returns (prob [V] float64, cut_margin)."""
    lib = _load()
    x = np.ascontiguousarray(logits, dtype=np.float64).reshape(-1)
    prob = np.empty_like(x)
    cm = ctypes.c_double(0.0)
    rc = lib.sv_oracle_dist(_ptr(x), x.size, float(temperature), int(top_k), float(top_p),
                            _ptr(prob), ctypes.addressof(cm))
    if rc != 0:
        raise ValueError("distribution undefined (T <= 0 or no finite logit)")
    return prob, cm.value


def sample(logits, params, uniforms, *, dtype="f32", nthreads: int = 0):
    """One draw per row from the truncated distribution of each row of
    logits [B, V] (float32, or uint16 bf16 bit patterns for dtype="bf16"):
    the final draw of ``verify`` with no drafts (K = 0), that is
    invcdf(dist(row, T, top_k, top_p), u) in ascending token-id order, or the
    argmax (lowest id on ties) when T = 0.  uniforms [B] float32.
    Returns (tokens [B], status [B] (0, or -1 for an invalid row),
    diag [B, 1, 4])."""
    logits = np.ascontiguousarray(logits)
    B, V = logits.shape
    out, acc, diag, _, _ = verify(logits.reshape(B, 1, V), None, np.zeros((B, 0), np.int32),
                                  None, params, np.asarray(uniforms, np.float32).reshape(B, 1),
                                  dtype=dtype, nthreads=nthreads)
    return out[:, 0].copy(), acc, diag


def _row_f64(row, dtype):
    if dtype == "f32":
        return np.asarray(row, dtype=np.float32).astype(np.float64)
    bits = np.asarray(row, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def accept_stats(target, draft, params, *, dtype="f32"):
    """Acceptance statistics of one draft position, per row (the quantities
    sv_accept_stats computes).

    deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…": the check
    that compares two independent draws agrees with probability sum p q
    (section "Örnekleme altında doğrulama yanlıştı"); the rejection test keeps
    a draft token x ~ q with min(1, p(x)/q(x)), so its acceptance is
    sum min(p, q), the overlap of the two distributions (section "Kesme her
    iki tarafta eşleşmek zorunda"), which is why truncating only one side
    lowers it.

    target, draft: [B, V] float32 (or uint16 bf16 patterns with
    dtype="bf16"); params: [B] PARAMS_DTYPE.  p, q are the distributions of
    dist() with the row's parameters, p~, q~ those with temperature only.
    Returns (stats [B, 4] float64 = sum min(p, q), sum p q, sum min(p~, q),
    sum min(p~, q~); cut_margin [B], the smaller of the two sides' cut
    margins from dist()).  Greedy rows (T = 0): 1 in every slot when the
    argmaxes (lowest id among equal logits) agree, else 0.  Rows with T < 0
    or not finite, top_p <= 0, or no finite logit on a side: NaN."""
    target = np.asarray(target)
    draft = np.asarray(draft)
    B = target.shape[0]
    params = np.ascontiguousarray(params)
    out = np.full((B, 4), np.nan)
    margin = np.full(B, np.inf)
    for b in range(B):
        T = float(params["temperature"][b])
        k = int(params["top_k"][b])
        tp = float(params["top_p"][b])
        if not (T >= 0.0 and np.isfinite(T) and tp > 0.0):
            continue
        t = _row_f64(target[b], dtype)
        d = _row_f64(draft[b], dtype)
        if T == 0.0:
            if not (np.isfinite(t).any() and np.isfinite(d).any()):
                continue
            out[b] = 1.0 if int(np.argmax(t)) == int(np.argmax(d)) else 0.0
            continue
        try:
            p, mp = dist(t, T, k, tp)
            q, mq = dist(d, T, k, tp)
            pu, _ = dist(t, T, 0, 1.0)
            qu, _ = dist(d, T, 0, 1.0)
        except ValueError:
            continue
        out[b, 0] = np.minimum(p, q).sum()
        out[b, 1] = (p * q).sum()
        out[b, 2] = np.minimum(pu, q).sum()
        out[b, 3] = np.minimum(pu, qu).sum()
        margin[b] = min(mp, mq)
    return out, margin
