"""Several layers sharing one workspace, one decode token replayed from a HIP
graph (retopk_group_*), through the C ABI, against the CPU oracle in lockstep:
before each replay every layer's oracle adopts that layer's cache, and after it
each layer's path, rho_max and M_t (statistics ring), its new cache entry (the
q_bar bits and the selected support) and its output are compared. A second
group run eagerly, layer by layer, must give bit-identical outputs and caches.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.retopk_oracle as O
from parity_util import OUT_REL, check_output, check_support
from sparse_long_context_head_amd.workload import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def _layers_data(wl, n_layers):
    # a different seeded sequence per layer
    return [generate(wl, seed_base=7000 + 100 * l) for l in range(n_layers)]


def _compare_layer(l, layer, orc, data, t, L, out_gpu, state_before, swaps):
    rec = orc.step(data["q_dec"][t - 1], data["k"], data["v"], L, t)
    path, rho, m = layer.stats(t, 1)
    qb, supp, slen, count = layer.read_state()
    G = orc.hq // orc.hkv
    for b in range(orc.batch):
        for h in range(orc.hq):
            where = f"layer {l} t={t} b={b} h={h}"
            assert (path[0, b, h] & 1) == rec.path[b, h], f"{where}: path"
            if np.isfinite(rec.rho_max[b, h]):
                assert abs(rho[0, b, h] - rec.rho_max[b, h]) <= 1e-12, f"{where}: rho_max"
            if rec.path[b, h] == O.REUSE:
                assert m[0, b, h] == rec.n_cand[b, h], f"{where}: M_t"
            n = int(count[b, h])
            assert n == min(int(state_before[3][b, h]) + 1, orc.c), f"{where}: FIFO count"
            assert np.array_equal(qb[b, h, n - 1].view(np.uint32),
                                  O.normalize_query(data["q_dec"][t - 1][b, h]).view(np.uint32)), f"{where}: q_bar"
            sel = supp[b, h, n - 1, :slen[b, h, n - 1]]
            gs = check_support(sel, rec.support[b][h], data["q_dec"][t - 1][b, h], data["k"][b, h // G], where,
                               swaps)
            check_output(out_gpu[b, h], gs, data["v"][b, h // G, sel], orc.d, where)
    return rec


def test_graph_token_three_layers_lockstep():
    import torch
    from sparse_long_context_head_amd import binding as B
    n_layers, steps = 3, 8
    wl = WORKLOADS["gqa16k"].replace(prompt_len=6000, decode_steps=steps, refresh_every=4)
    datas = _layers_data(wl, n_layers)
    dev = [{k: B.bf16_tensor(v) for k, v in d.items()} for d in datas]
    stream = torch.cuda.Stream()
    shape = (wl.batch, wl.n_q_heads, wl.head_dim)
    qbuf = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    outs = [torch.empty(shape, dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    grp = B.ReTopKGroup.from_workload(wl, n_layers)
    eager = B.ReTopKGroup.from_workload(wl, n_layers)
    with torch.cuda.stream(stream):
        for l in range(n_layers):
            grp.layers[l].init_from_prefill(dev[l]["q_tail"], dev[l]["k"], wl.prompt_len, stream)
            eager.layers[l].init_from_prefill(dev[l]["q_tail"], dev[l]["k"], wl.prompt_len, stream)
    stream.synchronize()
    grp.capture(qbuf, [d["k"] for d in dev], [d["v"] for d in dev], outs, stream)
    grp.set_position(wl.prompt_len + 1, 1)
    orcs = [O.ReTopKOracle.from_workload(wl) for _ in range(n_layers)]
    e_out = torch.empty(shape, dtype=torch.float32, device="cuda")
    swaps, paths = [], []
    for t in range(1, steps + 1):
        L = wl.prompt_len + t
        before = [grp.layers[l].read_state() for l in range(n_layers)]
        for l in range(n_layers):
            orcs[l].set_state(*before[l])
        with torch.cuda.stream(stream):
            for l in range(n_layers):
                qbuf[l].copy_(dev[l]["q_dec"][t - 1])
        grp.replay(stream)
        stream.synchronize()
        for l in range(n_layers):
            rec = _compare_layer(l, grp.layers[l], orcs[l], datas[l], t, L, outs[l].cpu().numpy(), before[l],
                                 swaps)
            paths.append(rec.path.copy())
        # the same token decoded eagerly, layer by layer, on the second group
        for l in range(n_layers):
            eager.layers[l].decode_step(dev[l]["q_dec"][t - 1], dev[l]["k"], dev[l]["v"], L, t, e_out, stream)
            stream.synchronize()
            assert np.array_equal(e_out.cpu().numpy().view(np.uint32), outs[l].cpu().numpy().view(np.uint32)), (
                f"layer {l} t={t}: graph and eager outputs differ")
    for l in range(n_layers):
        for a, b_ in zip(grp.layers[l].read_state(), eager.layers[l].read_state()):
            assert np.array_equal(a, b_), f"layer {l}: graph and eager caches differ"
        assert B.retopk_read_device_error(grp.layers[l].handle) == 0
    paths = np.array(paths)
    assert paths[3 * n_layers:4 * n_layers].all()  # step 4 refreshes every head of every layer
    print(f"[graph] {n_layers} layers x {steps} tokens: exact head-steps {int(paths.sum())}/{paths.size}, "
          f"swaps {len(swaps)}", flush=True)
    assert grp.device_bytes() < n_layers * B.retopk_device_bytes(grp.layers[0].handle) + eager.device_bytes()
    grp.close()
    eager.close()


def test_group_layers_share_one_workspace():
    """A group's layer holds its caches only; the workspaces are counted once."""
    from sparse_long_context_head_amd import binding as B
    wl = WORKLOADS["gqa16k"].replace(prompt_len=6000, decode_steps=8)
    one = B.ReTopKLayer.from_workload(wl)
    grp = B.ReTopKGroup.from_workload(wl, 4)
    solo = B.retopk_device_bytes(one.handle)
    per_layer = B.retopk_device_bytes(grp.layers[0].handle)
    assert per_layer < solo
    assert grp.device_bytes() < 4 * solo
    assert grp.device_bytes() == 4 * per_layer + (solo - per_layer)
    one.close()
    grp.close()


def test_graph_replay_errors():
    import torch
    from sparse_long_context_head_amd import binding as B
    wl = WORKLOADS["tiny"].replace(prompt_len=100, decode_steps=2)
    grp = B.ReTopKGroup.from_workload(wl, 2)
    stream = torch.cuda.Stream()
    with pytest.raises(B.RetopkError) as e:
        grp.replay(stream)          # nothing captured
    assert e.value.status == 1
    with pytest.raises(B.RetopkError) as e:
        grp.set_position(wl.max_len + 1, 1)
    assert e.value.status == 2
    grp.close()
