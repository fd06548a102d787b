"""The entry point that allocates nothing (retopk_dense_attn_noalloc) against
the handle-based dense attention it varies, through the C ABI, on two calls in
a row (the second smaller), and against the CPU oracle."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle.retopk_oracle as O
from sparse_long_context_head_amd.workload import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def _run_pair(B, wl, length):
    import torch
    data = generate(wl)
    q = B.bf16_tensor(data["q_dec"][0])
    k = B.bf16_tensor(data["k"])
    v = B.bf16_tensor(data["v"])
    shape = (wl.batch, wl.n_q_heads, wl.head_dim)
    out_h = torch.empty(shape, dtype=torch.float32, device="cuda")
    out_n = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    layer = B.ReTopKLayer.from_workload(wl)
    layer.dense_attn(q, k, v, length, out_h)
    B.retopk_dense_attn_noalloc(q, k, v, length, out_n)
    torch.cuda.synchronize()
    layer.close()
    a, b = out_h.cpu().numpy(), out_n.cpu().numpy()
    # the same kernels and row split: bit-identical to the handle's call
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref = O.dense_attention(data["q_dec"][0], data["k"], data["v"], length)
    for bb in range(wl.batch):
        for h in range(wl.n_q_heads):
            err = np.max(np.abs(b[bb, h] - ref[bb, h])) / np.max(np.abs(ref[bb, h]))
            assert err <= 5e-3, (bb, h, err)


def test_noalloc_dense_matches_handle_call_twice():
    from sparse_long_context_head_amd import binding as B
    big = WORKLOADS["gqa16k"].replace(batch=2, prompt_len=9000, decode_steps=8)
    _run_pair(B, big, 9000 + 3)
    small = WORKLOADS["gqa16k"].replace(batch=1, n_q_heads=8, n_kv_heads=2, prompt_len=700, decode_steps=4)
    _run_pair(B, small, 700 + 1)


def test_noalloc_dense_refuses_more_scratch_than_it_has():
    import torch
    from sparse_long_context_head_amd import binding as B
    lib = B.load_library()
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    # 128 batch rows x 64 query heads over 8 KV heads: 8192 slices of 528 bytes > 4 MiB
    st = lib.retopk_dense_attn_noalloc(128, 64, 8, 100, p, p, p, 10, p, None)
    assert st == 2  # RETOPK_OUT_OF_RANGE, before any device work
    assert b"scratch" in lib.retopk_last_error()
    torch.cuda.synchronize()
