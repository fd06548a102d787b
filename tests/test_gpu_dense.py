"""Dense softmax attention (retopk_dense_attn, through the C ABI) against the
CPU oracle's dense_attention, every head, on seeded synthetic inputs.

Acceptance: max|o_gpu - o_ref| / max|o_ref| <= 5e-3 per head (fp32
accumulation of bf16 keys and values against the oracle's float64), the
output tolerance of the sparse paths. Lengths span one row, partial and whole
16-row tiles and 128-row stages, and ragged slices; the launch splits the rows
of each KV group into slices the same way at every size, so the headline-size
case runs the launch configuration the benchmark times.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle.retopk_oracle as O
from sparse_long_context_head_amd.workload import WORKLOADS, f32_to_bf16_bits, generate

pytestmark = pytest.mark.gpu

OUT_REL = 5e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(wl, data, lengths, heads=None):
    import torch
    from sparse_long_context_head_amd import binding as B
    layer = B.ReTopKLayer.from_workload(wl)
    k = B.bf16_tensor(data["k"])
    v = B.bf16_tensor(data["v"])
    q_bits = data["q_dec"][0]
    q = B.bf16_tensor(q_bits)
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    worst = 0.0
    for L in lengths:
        log(f"[dense] {wl.name} B={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} L={L}")
        out.fill_(float("nan"))
        layer.dense_attn(q, k, v, L, out)
        o = out.cpu().numpy()
        bh = [(b, h) for b in range(wl.batch) for h in range(wl.n_q_heads)] if heads is None else heads
        for b, h in bh:
            g = h * wl.n_kv_heads // wl.n_q_heads
            ref = O.dense_attention(q_bits[b:b + 1, h:h + 1], data["k"][b:b + 1, g:g + 1],
                                    data["v"][b:b + 1, g:g + 1], L)[0, 0]
            err = float(np.max(np.abs(o[b, h].astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))
            assert err <= OUT_REL, f"dense L={L} b={b} h={h}: relative error {err:.3e} > {OUT_REL}"
            worst = max(worst, err)
    layer.close()
    log(f"[dense] worst relative error {worst:.2e}")
    return worst


def test_dense_tiny_lengths():
    """One head: lengths at and around tile (16), stage (128) and slice edges."""
    wl = WORKLOADS["tiny"]
    _run(wl, generate(wl), [1, 2, 15, 16, 17, 127, 128, 129, 255, 256, 257, 1000, 4096, 4160])


def test_dense_gqa16k():
    """28 query heads over 4 KV heads (7 per group), ragged lengths up to 16K."""
    wl = WORKLOADS["gqa16k"].replace(decode_steps=8)
    _run(wl, generate(wl), [300, 5000, 16385, 16391])


def test_dense_more_groups_than_compute_units():
    """40 batch rows x 4 KV heads: 160 KV groups, two slices each at most."""
    wl = WORKLOADS["tiny"].replace(batch=40, n_q_heads=8, n_kv_heads=4, prompt_len=1200, decode_steps=4)
    _run(wl, generate(wl), [1200, 65, 5])


def test_dense_eight_heads_per_group():
    """Eight query heads per KV head, the most the dense kernel takes."""
    wl = WORKLOADS["tiny"].replace(n_q_heads=16, n_kv_heads=2, prompt_len=3000, decode_steps=4)
    _run(wl, generate(wl), [3000, 129])


def test_dense_zero_query_is_mean_of_values():
    """A zero query weights every row equally: the output is the mean value row."""
    import torch
    from sparse_long_context_head_amd import binding as B
    rng = np.random.default_rng(31)
    L = 5000
    k = f32_to_bf16_bits(rng.standard_normal((1, 2, L, 128)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((1, 2, L, 128)).astype(np.float32))
    q = np.zeros((1, 4, 128), np.uint16)
    layer = B.ReTopKLayer(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, max_len=L, top_k=64,
                          cache_cap=2, window=1, top_r=1, refresh_every=0, tau=0.5)
    out = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    layer.dense_attn(B.bf16_tensor(q), B.bf16_tensor(k), B.bf16_tensor(v), L, out)
    o = out.cpu().numpy()
    for h in range(4):
        ref = O.bf16_to_f64(v[0, h // 2]).mean(0)
        np.testing.assert_allclose(o[0, h], ref, rtol=1e-4, atol=1e-5)
    layer.close()


def test_dense_rejects_more_than_eight_heads_per_group():
    import torch
    from sparse_long_context_head_amd import binding as B
    layer = B.ReTopKLayer(batch=1, n_q_heads=16, n_kv_heads=1, head_dim=128, max_len=64, top_k=8,
                          cache_cap=2, window=1, top_r=1, refresh_every=0, tau=0.5)
    q = torch.zeros((1, 16, 128), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    kv = torch.zeros((1, 1, 64, 128), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = torch.empty((1, 16, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(B.RetopkError) as e:
        layer.dense_attn(q, kv, kv, 64, out)
    assert e.value.status == 2
    with pytest.raises(B.RetopkError) as e:
        layer.dense_attn(q, kv, kv, 65, out)
    assert e.value.status == 2
    layer.close()


@pytest.mark.slow
def test_dense_headline_128k():
    """L0 = 131072, 28/4 heads: every head at the first decode length."""
    wl = WORKLOADS["headline128k"].replace(decode_steps=8)
    _run(wl, generate(wl), [131072 + 1])


@pytest.mark.slow
def test_dense_scale_1m():
    """L0 = 1,048,576: the heads of KV group 1 at the first decode length."""
    wl = WORKLOADS["scale1m"].replace(decode_steps=8)
    _run(wl, generate(wl), [(1 << 20) + 1], heads=[(0, h) for h in range(7, 14)])
