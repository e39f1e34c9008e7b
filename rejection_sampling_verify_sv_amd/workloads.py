"""Seeded synthetic inputs for the verify step.

This module only synthesises inputs (logits, draft tokens, sampler
parameters, uniforms).  It holds none of the verify arithmetic, imports
neither the GPU library nor the oracle, and is the one piece of code the two
sides share.

Recipes (the pages print no dataset; these stand in for model logits):

* ``tiny_v1000``: V=1000, K=1, fp32.  One fixed logits pair, target rows
  ~ N(0, 3^2), draft = target + N(0, 1).  T=1, top_k=20, top_p=0.95.  Every
  batch row repeats the same logits with its own draft token and uniforms, so
  a batch of 10,000 rows is 10,000 independent verify steps.
* ``decode_b1``: V=151936, B=1, K=1, bf16, Zipf recipe, rho=0.8.
  T=1, top_k=20, top_p=0.95.
* ``mixed_greedy_b64``: V=151936, B=64, K=4, bf16, Zipf recipe, rho=0.8.
  A seeded half of the rows is greedy (T=0); the rest use T=0.6, top_k=20,
  top_p=0.95.
* ``fullvocab_ragged_b256``: V=248320, B=256, K=4, draft_len ~ U{1..4},
  bf16.  Target ~ N(0, 2^2); draft = 0.7 t + sqrt(0.51) N(0, 2^2).
  T=1, top_k=0, top_p=1 (untruncated).
* ``mixed_samplers_b1024``: V=151936, B=1024, K=3, fp32, Zipf recipe with a
  per-row rho ~ U[0.5, 0.95].  Per row T in {0, 0.6, 1.0}, top_k in
  {0, 20, 50}, top_p in {0.8, 0.95, 1.0}, each drawn independently.

Tree recipe (``make_tree``, for the tree / multi-candidate verify): the
mixed-sampler recipe over the nodes of a candidate tree, B=256, V=151936,
bf16, a Medusa-shaped tree of 12 candidates (3 children at the root, 2 under
each of them, then 1 under each of those) per row: node v's target row is
the target after v's path and its draft row the draft there (rho per row as
above), and candidate c's token is drawn from q at its parent's draft row.

Zipf recipe: t_i = log Zipf_{s=1.1}(rank_i) + N(0, 0.5^2) with a fresh random
permutation of the ranks for every (row, position); the draft of a Zipf
workload mixes the target with an independent copy of the same recipe,
d = rho t + (1 - rho) t'.

Draft tokens: greedy rows take the argmax of the draft logits (lowest id among
equal maxima).  Sampling rows draw x ~ q, the draft distribution the verify
step itself forms: temperature T, the top_k largest draft logits (ranked by
logit descending, id ascending; all of them when top_k is 0 or >= V), the
nucleus walk over that set renormalised (a token is kept while the mass ranked
ahead of it is below top_p; top_p >= 1 keeps all), then a Gumbel-max draw over
the kept set at temperature T.  This is the draft model's own sampling step
(the deniz.in page, section "Kesme her iki tarafta eşleşmek zorunda": the
draft samples with the same truncation the target applies); it is written
here independently of both the verify library and the oracle.

Seeds: numpy PCG64 with SeedSequence(20261202 + recipe_id).spawn(4) giving
separate streams for logits, draft tokens, uniforms and sampler parameters.
bf16 logits are rounded from fp32 with round-to-nearest-even and stored as
uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PARAMS_DTYPE = np.dtype(
    [("temperature", "<f4"), ("top_k", "<i4"), ("top_p", "<f4"), ("reserved", "<i4")]
)

RECIPES = {
    "tiny_v1000": dict(id=1, V=1000, B=10000, K=1, dtype="f32"),
    "decode_b1": dict(id=2, V=151936, B=1, K=1, dtype="bf16"),
    "mixed_greedy_b64": dict(id=3, V=151936, B=64, K=4, dtype="bf16"),
    "fullvocab_ragged_b256": dict(id=4, V=248320, B=256, K=4, dtype="bf16"),
    "mixed_samplers_b1024": dict(id=5, V=151936, B=1024, K=3, dtype="f32"),
}


@dataclasses.dataclass
class Workload:
    name: str
    V: int
    B: int
    K: int
    dtype: str  # "f32" (float32 arrays) or "bf16" (uint16 bit patterns)
    target: np.ndarray  # [B, K+1, V]
    draft: np.ndarray  # [B, K, V]
    tokens: np.ndarray  # [B, K] int32
    draft_len: np.ndarray  # [B] int32
    params: np.ndarray  # [B] PARAMS_DTYPE
    uniforms: np.ndarray  # [B, K+1] float32

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def target_f32(self, b: int, k: int) -> np.ndarray:
        return as_f32(self.target[b, k], self.dtype)

    def draft_f32(self, b: int, k: int) -> np.ndarray:
        return as_f32(self.draft[b, k], self.dtype)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint16)
    step = 1 << 22

    def work(s):
        u = flat[s:s + step].view(np.uint32)
        r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        o = (r >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(flat[s:s + step])
        o[nan] = 0x7FC0
        out[s:s + step] = o

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(work, range(0, flat.size, step)))
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.astype(np.float32) if dtype == "f32" else bf16_bits_to_f32(a)


def _zipf_base(V: int, s: float = 1.1) -> np.ndarray:
    ranks = np.arange(1, V + 1, dtype=np.float64)
    logw = -s * np.log(ranks)
    logw -= math.log(np.exp(logw).sum())
    return logw


def _normal_rows(seed: np.random.SeedSequence, n: int, V: int, sd: float) -> np.ndarray:
    """n rows of N(0, sd^2) fp32 values, 64-row blocks with child seeds."""
    out = np.empty((n, V), np.float32)
    blocks = list(range(0, n, 64))
    seeds = seed.spawn(len(blocks))

    def work(i):
        rng = np.random.Generator(np.random.PCG64(seeds[i]))
        s = blocks[i]
        e = min(n, s + 64)
        rng.standard_normal((e - s, V), dtype=np.float32, out=out[s:e])
        out[s:e] *= np.float32(sd)

    with ThreadPoolExecutor(max_workers=min(8, len(blocks))) as ex:
        list(ex.map(work, range(len(blocks))))
    return out


def _zipf_rows(seed: np.random.SeedSequence, base: np.ndarray, n: int,
               noise_sd: float = 0.5) -> np.ndarray:
    """n rows of log-Zipf over a fresh permutation plus Gaussian noise (fp32).

    Rows are generated in blocks of 64, each from its own child seed, so the
    result does not depend on how the blocks are spread over threads."""
    V = base.size
    out = np.empty((n, V), np.float32)
    b32 = base.astype(np.float32)
    blocks = list(range(0, n, 64))
    seeds = seed.spawn(len(blocks))

    def work(i):
        rng = np.random.Generator(np.random.PCG64(seeds[i]))
        s = blocks[i]
        e = min(n, s + 64)
        for r in range(s, e):
            out[r] = b32[rng.permutation(V)]
        out[s:e] += rng.standard_normal((e - s, V), dtype=np.float32) * np.float32(noise_sd)

    with ThreadPoolExecutor(max_workers=min(8, len(blocks))) as ex:
        list(ex.map(work, range(len(blocks))))
    return out


def _kept_set(row: np.ndarray, T: float, top_k: int, top_p: float) -> np.ndarray:
    """Ids of the truncated draft distribution of one row (see the module
    docstring), in ranking order."""
    V = row.size
    if top_p >= 1.0 and not 0 < top_k < V:
        return np.arange(V)  # untruncated: every id (the draw does not need an order)
    if 0 < top_k < V:
        # the top_k best by (logit desc, id asc): partition, then an exact
        # stable order of the candidates and of the ties at the k-th value
        cut = np.partition(row, V - top_k)[V - top_k]
        cand = np.flatnonzero(row >= cut)
    else:
        cand = np.arange(V)
    order = cand[np.argsort(-row[cand], kind="stable")]
    if 0 < top_k < V:
        order = order[:top_k]
    if top_p >= 1.0:
        return order
    lv = row[order].astype(np.float64)
    w = np.exp((lv - lv[0]) / T)
    P = w / w.sum()
    before = np.concatenate(([0.0], np.cumsum(P)[:-1]))
    n = int(np.count_nonzero(before < top_p))
    return order[:max(n, 1)]


def _draft_tokens(seed: np.random.SeedSequence, draft_f32: np.ndarray, params: np.ndarray,
                  draft_len: np.ndarray) -> np.ndarray:
    """Draft tokens x ~ q (see the module docstring); -1 past draft_len.
    One child seed per batch row."""
    B, K, V = draft_f32.shape
    tok = np.full((B, K), -1, np.int32)
    seeds = seed.spawn(B)

    def work(b):
        rng = np.random.Generator(np.random.PCG64(seeds[b]))
        T = float(params["temperature"][b])
        kk = int(params["top_k"][b])
        tp = float(params["top_p"][b])
        for k in range(int(draft_len[b])):
            row = draft_f32[b, k]
            if T == 0.0:
                tok[b, k] = int(np.argmax(row))
                continue
            kept = _kept_set(row, T, kk, tp)
            vals = row[kept].astype(np.float64)
            g = -np.log(-np.log(rng.random(vals.size)))
            tok[b, k] = int(kept[int(np.argmax(vals / T + g))])

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(work, range(B)))
    return tok


def _finish(name, V, B, K, dtype, t32, d32, draft_len, params, seeds, rngs, poison):
    tok = _draft_tokens(seeds[1], d32, params, draft_len)
    uniforms = rngs[2].random((B, K + 1), dtype=np.float32)
    if poison:
        for b in range(B):
            L = int(draft_len[b])
            t32[b, L + 1:] = np.nan
            d32[b, L:] = np.nan
    if dtype == "bf16":
        target = f32_to_bf16_bits(t32)
        draft = f32_to_bf16_bits(d32)
    else:
        target, draft = t32, d32
    return Workload(name, V, B, K, dtype, target, draft, tok, draft_len.astype(np.int32),
                    params, uniforms)


def _params(B, T, top_k, top_p):
    p = np.zeros(B, PARAMS_DTYPE)
    p["temperature"] = T
    p["top_k"] = top_k
    p["top_p"] = top_p
    return p


def make(name: str, *, batch: int | None = None, poison: bool = False,
         vocab: int | None = None) -> Workload:
    """Build a recipe; ``batch``/``vocab`` shrink it for quick tests."""
    r = RECIPES[name]
    V = vocab or r["V"]
    B = batch or r["B"]
    K = r["K"]
    dtype = r["dtype"]
    seeds = np.random.SeedSequence(20261202 + r["id"]).spawn(4)
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in seeds]
    g_logit, g_par = rngs[0], rngs[3]
    draft_len = np.full(B, K, np.int32)

    if name == "tiny_v1000":
        t = (g_logit.standard_normal((K + 1, V)) * 3.0).astype(np.float32)
        d = (t[:K].astype(np.float64) + g_logit.standard_normal((K, V))).astype(np.float32)
        t32 = np.broadcast_to(t, (B, K + 1, V)).copy()
        d32 = np.broadcast_to(d, (B, K, V)).copy()
        params = _params(B, 1.0, 20, 0.95)
    elif name in ("decode_b1", "mixed_greedy_b64", "mixed_samplers_b1024"):
        base = _zipf_base(V)
        s_t, s_d = seeds[0].spawn(2)
        t32 = _zipf_rows(s_t, base, B * (K + 1)).reshape(B, K + 1, V)
        tp = _zipf_rows(s_d, base, B * K).reshape(B, K, V)
        if name == "mixed_samplers_b1024":
            rho = g_par.uniform(0.5, 0.95, size=B).astype(np.float32)
        else:
            rho = np.full(B, 0.8, np.float32)
        tp *= (1 - rho)[:, None, None]
        tp += rho[:, None, None] * t32[:, :K]
        d32 = tp
        if name == "decode_b1":
            params = _params(B, 1.0, 20, 0.95)
        elif name == "mixed_greedy_b64":
            params = _params(B, 0.6, 20, 0.95)
            greedy = g_par.permutation(B)[: B // 2]
            params["temperature"][greedy] = 0.0
        else:
            params = _params(B, 0.0, 0, 1.0)
            params["temperature"] = g_par.choice(np.array([0.0, 0.6, 1.0], np.float32), B)
            params["top_k"] = g_par.choice(np.array([0, 20, 50], np.int32), B)
            params["top_p"] = g_par.choice(np.array([0.8, 0.95, 1.0], np.float32), B)
    elif name == "fullvocab_ragged_b256":
        s_t, s_d = seeds[0].spawn(2)
        t32 = _normal_rows(s_t, B * (K + 1), V, 2.0).reshape(B, K + 1, V)
        d32 = _normal_rows(s_d, B * K, V, 2.0).reshape(B, K, V)
        d32 *= np.float32(math.sqrt(0.51))
        d32 += np.float32(0.7) * t32[:, :K]
        draft_len = g_par.integers(1, K + 1, size=B).astype(np.int32)
        params = _params(B, 1.0, 0, 1.0)
    else:
        raise KeyError(name)
    return _finish(name, V, B, K, dtype, t32, d32, draft_len, params, seeds, rngs, poison)


def tree_parents(K: int, shape: str = "medusa") -> np.ndarray:
    """Parents of candidates 1..K: "medusa" (3 at the root, 2 under each of
    them, then 1 under each of those; K <= 12), "wide" (all at the root) or
    "path" (a chain)."""
    if shape == "path":
        return np.arange(K, dtype=np.int32)
    if shape == "wide":
        return np.zeros(K, np.int32)
    if shape != "medusa" or K > 12:
        raise ValueError(shape)
    par = [0 if c <= 3 else ((c - 4) // 2 + 1 if c <= 9 else c - 6) for c in range(1, K + 1)]
    return np.array(par, np.int32)


def make_tree(*, batch: int = 256, vocab: int = 151936, K: int = 12, shape: str = "medusa",
              dtype: str = "bf16"):
    """The tree recipe (see the module docstring): (Workload, parents [B, K])
    for sv_verify_tree, every row offering all K candidates."""
    B, V = batch, vocab
    seeds = np.random.SeedSequence(20261202 + 6).spawn(4)
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in seeds]
    g_par = rngs[3]
    base = _zipf_base(V)
    s_t, s_d = seeds[0].spawn(2)
    t32 = _zipf_rows(s_t, base, B * (K + 1)).reshape(B, K + 1, V)
    d32 = _zipf_rows(s_d, base, B * K).reshape(B, K, V)
    rho = g_par.uniform(0.5, 0.95, size=B).astype(np.float32)
    d32 *= (1 - rho)[:, None, None]
    d32 += rho[:, None, None] * t32[:, :K]
    params = _params(B, 0.0, 0, 1.0)
    params["temperature"] = g_par.choice(np.array([0.0, 0.6, 1.0], np.float32), B)
    params["top_k"] = g_par.choice(np.array([0, 20, 50], np.int32), B)
    params["top_p"] = g_par.choice(np.array([0.8, 0.95, 1.0], np.float32), B)
    par = np.tile(tree_parents(K, shape), (B, 1))
    # candidate c is drawn at its parent: the chain generator over the
    # parents' draft rows gives each candidate a draw from q there
    tok = _draft_tokens(seeds[1], d32[:, par[0]], params, np.full(B, K, np.int32))
    uniforms = rngs[2].random((B, K + 1), dtype=np.float32)
    if dtype == "bf16":
        target, draft = f32_to_bf16_bits(t32), f32_to_bf16_bits(d32)
    else:
        target, draft = t32, d32
    wl = Workload(f"tree_{shape}_b{B}", V, B, K, dtype, target, draft, tok,
                  np.full(B, K, np.int32), params, uniforms)
    return wl, par


def custom(target_f32: np.ndarray, draft_f32: np.ndarray, tokens, draft_len, params,
           uniforms, *, dtype: str = "f32", name: str = "custom") -> Workload:
    """Wrap hand-built arrays (fp32 values; rounded to bf16 when asked)."""
    t = np.ascontiguousarray(target_f32, dtype=np.float32)
    d = np.ascontiguousarray(draft_f32, dtype=np.float32)
    B, K1, V = t.shape
    if dtype == "bf16":
        t, d = f32_to_bf16_bits(t), f32_to_bf16_bits(d)
    return Workload(name, V, B, K1 - 1, dtype, t, d,
                    np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, K1 - 1),
                    np.ascontiguousarray(draft_len, dtype=np.int32).reshape(B),
                    np.ascontiguousarray(params), np.ascontiguousarray(uniforms, np.float32))


def to_torch(wl: Workload, device):
    """Device tensors (target, draft, tokens, draft_len, params [B,4] int32,
    uniforms) for a workload; bf16 bit patterns are reinterpreted, not
    converted."""
    import torch

    if wl.dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(wl.target)).to(device)
        d = torch.from_numpy(np.ascontiguousarray(wl.draft)).to(device)
    else:
        t = torch.from_numpy(np.ascontiguousarray(wl.target).view(np.int16)).to(device)
        d = torch.from_numpy(np.ascontiguousarray(wl.draft).view(np.int16)).to(device)
        t, d = t.view(torch.bfloat16), d.view(torch.bfloat16)
    prm = torch.from_numpy(np.ascontiguousarray(wl.params).view(np.int32).reshape(-1, 4).copy())
    return (t, d, torch.from_numpy(wl.tokens).to(device),
            torch.from_numpy(wl.draft_len).to(device), prm.to(device),
            torch.from_numpy(wl.uniforms).to(device))
