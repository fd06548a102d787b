"""Seeded synthetic decode workloads for the ReTopK attention path.

This module only draws inputs. It holds none of the method's arithmetic: no
normalisation, scoring, selection or softmax. Both the CPU oracle (through the
tests) and the HIP path receive exactly the arrays produced here.

The shapes follow the attention layer the ReTopK paper evaluates ("Recall
Before You Rank", Experiments: Qwen2.5-7B, 28 query heads, K=512, C=W=32, R=4,
tau=0.85, T_r=128, BF16). Real model queries and keys are replaced by:

* keys and values: iid N(0, 1) per element; in configurations with heavy keys,
  64 distinct prompt rows per KV head are multiplied by 3 so that attention is
  peaked, as it is on real text;
* queries: one AR(1) stream per query head, x_0 ~ N(0, I),
  x_{n+1} = rho * x_n + sqrt(1 - rho^2) * eps_n, so consecutive decode queries
  are similar (the premise of the paper's Motivation section) while the
  stationary variance stays 1.

Everything is rounded to bf16 (round to nearest even) from float32 at the end;
the AR recursion runs unrounded in float64. Arrays are returned as raw uint16
bf16 bit patterns.

Draw order per sequence (numpy PCG64, ``default_rng(seed)``):
  1. K  float64 normals, shape [Hkv, L0 + T, d] (for multi-GB arrays drawn in
     chunks of rows, the same normals in the same order; see _sequence_chunked)
  2. heavy rows: for each KV head, ``choice(L0, n_heavy, replace=False)``
  3. V  float64 normals, shape [Hkv, L0 + T, d]
  4. query innovations, shape [Hq, n0 + T, d]
The default seed of sequence b in configuration number c is 1000 * c + b.

Decode step t (1-based) appends key/value row L0 + t - 1, so at step t the
visible length is L_t = L0 + t, and uses query row n0 + t - 1. Query rows
0 .. n0 - 1 belong to prompt positions L0 - n0 .. L0 - 1 and initialise the
query-support cache.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prompt_len: int          # L0
    decode_steps: int        # T
    top_k: int               # K
    cache_cap: int           # C
    window: int              # W
    top_r: int               # R
    tau: float
    refresh_every: int       # T_r (0 disables scheduled refresh)
    n_heavy: int             # heavy prompt rows per KV head (0 = none)
    query_rho: float         # AR(1) coefficient of the query streams

    @property
    def n_prompt_queries(self) -> int:
        return min(self.cache_cap, self.prompt_len)

    @property
    def max_len(self) -> int:
        return self.prompt_len + self.decode_steps

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_BASE = dict(head_dim=128, cache_cap=32, window=32, top_r=4, tau=0.85,
             refresh_every=128, query_rho=0.9)

WORKLOADS = {
    # Tiny single head, d=128, L0=4096, K=64, no heavy keys, 64 decode steps.
    "tiny": Workload(name="tiny", config_id=1, batch=1, n_q_heads=1, n_kv_heads=1,
                     prompt_len=4096, decode_steps=64, top_k=64, n_heavy=0, **_BASE),
    # Qwen2.5-7B-shaped GQA layer (28 q heads / 4 kv heads), L0=16384, K=512.
    "gqa16k": Workload(name="gqa16k", config_id=2, batch=1, n_q_heads=28, n_kv_heads=4,
                       prompt_len=16384, decode_steps=256, top_k=512, n_heavy=64, **_BASE),
    # Same layer at 32K and 64K, batch 4.
    "gqa32k_b4": Workload(name="gqa32k_b4", config_id=3, batch=4, n_q_heads=28, n_kv_heads=4,
                          prompt_len=32768, decode_steps=256, top_k=512, n_heavy=64, **_BASE),
    "gqa64k_b4": Workload(name="gqa64k_b4", config_id=4, batch=4, n_q_heads=28, n_kv_heads=4,
                          prompt_len=65536, decode_steps=256, top_k=512, n_heavy=64, **_BASE),
    # Headline: 128K context, batch 1, K=512, 512 decode steps.
    "headline128k": Workload(name="headline128k", config_id=5, batch=1, n_q_heads=28,
                             n_kv_heads=4, prompt_len=131072, decode_steps=512, top_k=512,
                             n_heavy=64, **_BASE),
    # Exact-path stress: batch 8, K=2048, tau=0.99, T_r=32, low query similarity.
    "stress128k_b8": Workload(name="stress128k_b8", config_id=6, batch=8, n_q_heads=28,
                              n_kv_heads=4, prompt_len=131072, decode_steps=256, top_k=2048,
                              n_heavy=64, **{**_BASE, "tau": 0.99, "refresh_every": 32,
                                             "query_rho": 0.5}),
    # One-layer scaling: the headline layer at 1M context (K + V = 2.1 GB per layer).
    "scale1m": Workload(name="scale1m", config_id=7, batch=1, n_q_heads=28, n_kv_heads=4,
                        prompt_len=1 << 20, decode_steps=256, top_k=512, n_heavy=64, **_BASE),
    # ... and at 4M (K + V = 8.6 GB per layer; drawn in chunks, see _sequence_chunked).
    "scale4m": Workload(name="scale4m", config_id=8, batch=1, n_q_heads=28, n_kv_heads=4,
                        prompt_len=1 << 22, decode_steps=128, top_k=512, n_heavy=64, **_BASE),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


# Key/value arrays of more elements than this are drawn in chunks of rows (the
# same normals in the same order) to bound host memory; their heavy rows are
# then scaled from the float32-rounded draws (a second rounding the smaller
# workloads do not have).
_CHUNKED_ABOVE = 1 << 31
_CHUNK_ROWS = 1 << 18


def _sequence_chunked(w: Workload, rng):
    hkv, d = w.n_kv_heads, w.head_dim
    n_rows = w.prompt_len + w.decode_steps
    k32 = np.empty((hkv, n_rows, d), np.float32)
    for g in range(hkv):
        for r0 in range(0, n_rows, _CHUNK_ROWS):
            r1 = min(n_rows, r0 + _CHUNK_ROWS)
            k32[g, r0:r1] = rng.standard_normal((r1 - r0, d))
    if w.n_heavy:
        for g in range(hkv):
            rows = rng.choice(w.prompt_len, w.n_heavy, replace=False)
            k32[g, rows, :] *= np.float32(3.0)
    k = f32_to_bf16_bits(k32)
    del k32
    v = np.empty((hkv, n_rows, d), np.uint16)
    for g in range(hkv):
        for r0 in range(0, n_rows, _CHUNK_ROWS):
            r1 = min(n_rows, r0 + _CHUNK_ROWS)
            v[g, r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, d)).astype(np.float32))
    return k, v


def _sequence(w: Workload, seed: int):
    rng = np.random.default_rng(seed)
    hkv, hq, d = w.n_kv_heads, w.n_q_heads, w.head_dim
    n_rows = w.prompt_len + w.decode_steps
    to16 = lambda a: f32_to_bf16_bits(a.astype(np.float32))
    if hkv * n_rows * d > _CHUNKED_ABOVE:
        k16, v16 = _sequence_chunked(w, rng)
    else:
        k = rng.standard_normal((hkv, n_rows, d))
        if w.n_heavy:
            for g in range(hkv):
                rows = rng.choice(w.prompt_len, w.n_heavy, replace=False)
                k[g, rows, :] *= 3.0
        v = rng.standard_normal((hkv, n_rows, d))
        k16, v16 = to16(k), to16(v)
        del k, v
    n_q = w.n_prompt_queries + w.decode_steps
    eps = rng.standard_normal((hq, n_q, d))
    q = np.empty_like(eps)
    q[:, 0] = eps[:, 0]
    s = math.sqrt(1.0 - w.query_rho * w.query_rho)
    for n in range(1, n_q):
        q[:, n] = w.query_rho * q[:, n - 1] + s * eps[:, n]
    return k16, v16, to16(q)


def generate(w: Workload, seed_base: int | None = None):
    """Draw one batch for workload ``w``.

    Returns a dict of uint16 (bf16 bits) arrays:
      k, v     [B, Hkv, L0 + T, d]   key/value cache, decode rows pre-drawn
      q_tail   [B, Hq, n0, d]        prompt-tail queries (cache initialisation)
      q_dec    [T, B, Hq, d]         decode queries, step t uses q_dec[t - 1]
    """
    base = 1000 * w.config_id if seed_base is None else seed_base
    ks, vs, qs = zip(*(_sequence(w, base + b) for b in range(w.batch)))
    k = np.stack(ks)
    v = np.stack(vs)
    q = np.stack(qs)                                  # [B, Hq, n0 + T, d]
    n0 = w.n_prompt_queries
    q_tail = np.ascontiguousarray(q[:, :, :n0])
    q_dec = np.ascontiguousarray(q[:, :, n0:].transpose(2, 0, 1, 3))
    return {"k": k, "v": v, "q_tail": q_tail, "q_dec": q_dec}
