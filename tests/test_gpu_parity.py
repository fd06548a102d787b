"""HIP path (through the C ABI) against the CPU oracle, element by element.

Workloads are the seeded synthetic configurations of
sparse_long_context_head_amd.workload; smaller variants keep the oracle's
run time to seconds while still spanning several work-group tiles and a ragged
tail. Full-size configurations are checked on sampled (batch row, KV group)
sub-problems, which the oracle computes independently of the other heads.
"""
from __future__ import annotations

import functools
import math
import sys

import numpy as np
import pytest

import oracle.retopk_oracle as O
from parity_util import (check_output, check_support, compare_cache_entry, compare_step,
                         sub_problem)
from sparse_long_context_head_amd.workload import WORKLOADS, f32_to_bf16_bits, generate

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _B():
    from sparse_long_context_head_amd import binding
    return binding


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def _data(name, **kw):
    wl = WORKLOADS[name].replace(**kw) if kw else WORKLOADS[name]
    return wl, generate(wl)


def data_for(name, **kw):
    return _data(name, **kw)


def upload(data):
    B = _B()
    return {k: B.bf16_tensor(v) for k, v in data.items()}


def _oracle_for(wl, sub, override):
    p = dict(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
             head_dim=wl.head_dim, top_k=wl.top_k, cache_cap=wl.cache_cap, window=wl.window,
             top_r=wl.top_r, refresh_every=wl.refresh_every, tau=wl.tau)
    p.update(override)
    if sub is not None:
        p.update(batch=1, n_q_heads=p["n_q_heads"] // p["n_kv_heads"], n_kv_heads=1)
    return O.ReTopKOracle(**p), p


def compare_init(layer, orc, odata, prompt_len, sl, swaps):
    gq, gs, gl, gc = [a[sl] for a in layer.read_state()]
    oq, os_, ol, oc = orc.get_state()
    assert np.array_equal(gc, oc), "init: entry counts differ"
    n0 = odata["q_tail"].shape[2]
    for b in range(orc.batch):
        for h in range(orc.hq):
            g = orc.kv_head(h)
            for i in range(int(oc[b, h])):
                p = prompt_len - n0 + i
                where = f"init b={b} h={h} entry={i}"
                assert np.array_equal(gq[b, h, i].view(np.uint32), oq[b, h, i].view(np.uint32)), (
                    f"{where}: q_bar not bit-identical")
                sel = gs[b, h, i, :gl[b, h, i]]
                assert len(sel) and sel.max() <= p, f"{where}: support not causal"
                check_support(sel, os_[b, h, i, :ol[b, h, i]], odata["q_tail"][b, h, i],
                              odata["k"][b, g], where, swaps)


def close_checked(layer):
    """Every call completed its work (no score work group gave up waiting), then free."""
    assert _B().retopk_read_device_error(layer.handle) == 0
    layer.close()


def run_lockstep(name, n_steps, sub=None, override=None, check_init=True, wl_kw=None, given=None):
    """Run n_steps decode steps; before each, the oracle adopts the GPU's cache.
    `given` = (workload, data) replaces the seeded workload's inputs."""
    torch = _torch()
    B = _B()
    override = dict(override or {})
    wl, data = given if given is not None else data_for(name, **(wl_kw or {}))
    n0 = min(override.get("cache_cap", wl.cache_cap), wl.prompt_len)
    if n0 != data["q_tail"].shape[2]:
        data = {**data, "q_tail": np.ascontiguousarray(data["q_tail"][:, :, -n0:])}
    dev = upload(data)
    layer = B.ReTopKLayer.from_workload(wl, **override)
    orc, p = _oracle_for(wl, sub, override)
    G = wl.n_q_heads // wl.n_kv_heads
    if sub is None:
        odata, sl = data, (slice(None), slice(None))
    else:
        odata = sub_problem(data, sub[0], sub[1], G)
        sl = (slice(sub[0], sub[0] + 1), slice(sub[1] * G, (sub[1] + 1) * G))
    L0 = wl.prompt_len
    swaps, errs = [], []
    log(f"[lockstep] {name} sub={sub} override={override} steps={n_steps}")
    layer.init_from_prefill(dev["q_tail"], dev["k"], L0)
    if check_init is True:
        orc.init_from_prefill(odata["q_tail"], odata["k"], L0)
        compare_init(layer, orc, odata, L0, sl, swaps)
    elif check_init:
        # the initialisation compared on one (batch row, KV group) only
        ib, ig = check_init
        iorc, _ = _oracle_for(wl, (ib, ig), override)
        idata = sub_problem(data, ib, ig, G)
        iorc.init_from_prefill(idata["q_tail"], idata["k"], L0)
        compare_init(layer, iorc, idata, L0, (slice(ib, ib + 1), slice(ig * G, (ig + 1) * G)), swaps)
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    paths, ms = [], []
    heads = [(b, h) for b in range(orc.batch) for h in range(orc.hq)]
    for t in range(1, n_steps + 1):
        L = L0 + t
        before = [a[sl] for a in layer.read_state()]
        orc.set_state(*before)
        layer.decode_step(dev["q_dec"][t - 1], dev["k"], dev["v"], L, t, out)
        rec = orc.step(odata["q_dec"][t - 1], odata["k"], odata["v"], L, t)
        info = {k: v[sl] for k, v in layer.step_info().items()}
        o = out.cpu().numpy()[sl]
        compare_step(rec, info, o, odata["q_dec"][t - 1], odata["k"], odata["v"], orc, p["tau"],
                     heads, swaps, errs)
        after = [a[sl] for a in layer.read_state()]
        for b, h in heads:
            where = f"t={t} b={b} h={h}"
            n_prev = int(before[3][b, h])
            n_new = int(after[3][b, h])
            assert n_new == min(n_prev + 1, p["cache_cap"]), f"{where}: FIFO count"
            drop = 1 if n_prev == p["cache_cap"] else 0
            for i in range(n_new - 1):
                assert np.array_equal(after[0][b, h, i], before[0][b, h, i + drop]), f"{where}: FIFO order"
                assert after[2][b, h, i] == before[2][b, h, i + drop], f"{where}: FIFO order"
            compare_cache_entry(after, O.normalize_query(odata["q_dec"][t - 1][b, h]), b, h,
                                info["sel"][b, h, :info["sel_len"][b, h]], where)
        paths.append(rec.path.copy())
        ms.extend(int(m) for m, pth in zip(rec.n_cand.ravel(), rec.path.ravel()) if pth == O.REUSE)
    paths = np.array(paths)
    log(f"[lockstep] {name}: exact head-steps {int(paths.sum())}/{paths.size}, "
        f"M_t mean {np.mean(ms) if ms else 0:.1f} max {max(ms) if ms else 0}, "
        f"swaps {len(swaps)}, max out err {max(errs):.2e}")
    close_checked(layer)
    return dict(paths=paths, swaps=swaps, max_err=max(errs), ms=ms)


# ---------------------------------------------------------------------------
# Exact Top-K attention baseline
# ---------------------------------------------------------------------------

def run_exact(name, lengths, top_k=None, sub=None, wl_kw=None, q_override=None):
    torch = _torch()
    B = _B()
    wl, data = data_for(name, **(wl_kw or {}))
    K = top_k or wl.top_k
    layer = B.ReTopKLayer.from_workload(wl, top_k=K, window=min(wl.window, 16384 - wl.top_r * K))
    dev = upload({"k": data["k"], "v": data["v"]})
    G = wl.n_q_heads // wl.n_kv_heads
    q = data["q_dec"][0] if q_override is None else q_override
    qd = _B().bf16_tensor(q)
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    sel = torch.empty((wl.batch, wl.n_q_heads, K), dtype=torch.int32, device="cuda")
    swaps = []
    for L in lengths:
        log(f"[exact] {name} L={L} K={K}")
        layer.exact_topk_attn(qd, dev["k"], dev["v"], L, out, sel)
        o = out.cpu().numpy()
        s = sel.cpu().numpy()
        info = layer.step_info()
        bs = range(wl.batch) if sub is None else [sub[0]]
        hs = range(wl.n_q_heads) if sub is None else range(sub[1] * G, (sub[1] + 1) * G)
        for b in bs:
            for h in hs:
                g = h // G
                where = f"exact L={L} b={b} h={h}"
                keff = min(K, L)
                assert np.all(s[b, h, keff:] == -1), f"{where}: sel_out padding"
                osel, _ = O.exact_topk_support(q[b, h], data["k"][b, g], L, K)
                gs = check_support(s[b, h, :keff], osel, q[b, h], data["k"][b, g], where, swaps)
                assert info["path"][b, h] == 1
                check_output(o[b, h], gs, data["v"][b, g, s[b, h, :keff]], wl.head_dim, where)
    close_checked(layer)
    return swaps


def test_exact_tiny_lengths():
    """Single head, K=64: lengths below K, at tile edges and ragged."""
    run_exact("tiny", [1, 2, 63, 64, 65, 1023, 1024, 1025, 4096, 4160])


def test_exact_gqa16k():
    """28 query heads over 4 KV heads, K=512, several lengths incl. ragged tails."""
    run_exact("gqa16k", [300, 512, 513, 5000, 16385, 16640])


def test_exact_more_groups_than_score_work_groups():
    """40 batch rows x 4 KV heads x 2 query heads, K=64: 160 KV groups over at
    most 128 score work groups, so one work group scores and writes survivors
    for segments of several KV groups and finishes several heads; with 320
    head work groups the launch also holds more work groups than the GPU has
    CUs, and the score work groups start as head work groups end."""
    run_exact("tiny", [1200, 700, 65, 64, 5],
              wl_kw=dict(batch=40, n_q_heads=8, n_kv_heads=4, prompt_len=1200, decode_steps=4))


def test_exact_sixteen_heads_per_group():
    """16 query heads on one KV head, every column of the MFMA score tile used."""
    run_exact("tiny", [5000, 4097, 129, 128, 127], top_k=128,
              wl_kw=dict(n_q_heads=16, n_kv_heads=1, prompt_len=5000, decode_steps=4))


def test_exact_large_top_k():
    """K = 4096 (R = 2 keeps R K + W within the candidate limit): the finish's
    support, the boundary bin and the softmax-V span many rounds."""
    run_exact("tiny", [20000, 4097, 4096, 4095, 9000], top_k=4096,
              wl_kw=dict(prompt_len=20000, decode_steps=4, top_r=2))


def test_exact_integer_ties():
    """Integer-valued keys and queries make fp32 scores exact, so equal scores
    are real ties: the lower index must win, with no near-tie allowance."""
    torch = _torch()
    B = _B()
    rng = np.random.default_rng(21)
    L, Hq, Hkv, D, K = 3000, 8, 2, 128, 100
    k = f32_to_bf16_bits(rng.integers(-2, 3, size=(1, Hkv, L, D)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((1, Hkv, L, D)).astype(np.float32))
    q = f32_to_bf16_bits(rng.integers(-1, 2, size=(1, Hq, D)).astype(np.float32))
    layer = B.ReTopKLayer(batch=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, max_len=L, top_k=K,
                          cache_cap=4, window=4, top_r=2, refresh_every=0, tau=0.5)
    out = torch.empty((1, Hq, D), dtype=torch.float32, device="cuda")
    sel = torch.empty((1, Hq, K), dtype=torch.int32, device="cuda")
    for length in (L, 1500, 99, 100, 101):
        layer.exact_topk_attn(B.bf16_tensor(q), B.bf16_tensor(k), B.bf16_tensor(v), length, out, sel)
        s = sel.cpu().numpy()
        for h in range(Hq):
            osel, _ = O.exact_topk_support(q[0, h], k[0, h // 4], length, K)
            assert np.array_equal(s[0, h, :min(K, length)], osel), f"L={length} h={h}"
    close_checked(layer)


def test_exact_degenerate_all_equal():
    """Zero query: every score is 0, the support is the K lowest indices.
    The boundary bin holds every key (at 20,000 more than the LDS holds, at
    9,000 fewer)."""
    torch = _torch()
    B = _B()
    rng = np.random.default_rng(22)
    L, K = 20000, 300
    k = f32_to_bf16_bits(rng.standard_normal((1, 1, L, 128)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((1, 1, L, 128)).astype(np.float32))
    q = np.zeros((1, 1, 128), np.uint16)
    layer = B.ReTopKLayer(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=128, max_len=L, top_k=K,
                          cache_cap=2, window=1, top_r=1, refresh_every=0, tau=0.5)
    out = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((1, 1, K), dtype=torch.int32, device="cuda")
    for length in (L, 9000):
        layer.exact_topk_attn(B.bf16_tensor(q), B.bf16_tensor(k), B.bf16_tensor(v), length, out, sel)
        assert np.array_equal(sel.cpu().numpy()[0, 0], np.arange(K)), length
        ref = O.bf16_to_f64(v[0, 0, :K]).mean(0)
        np.testing.assert_allclose(out.cpu().numpy()[0, 0], ref, rtol=1e-4, atol=1e-5)
    close_checked(layer)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_exact_long_history_integer_ties_and_all_equal():
    """Histories whose scores do not fit the score work groups' LDS: 28 query
    heads over 4 KV heads at 600,000 and 530,001 keys (more than 8,192 rows
    per score work group: per-segment K-best lists) and at 230,000 keys
    (about 4,000 rows: scores stored to and re-read from the workspace).
    Integer-valued keys and queries make every score exact with many ties,
    which must be broken by the lower index with no near-tie allowance; a zero
    query makes every score equal (the K lowest indices; the lists then cut on
    their rows, and the boundary bin holds far more keys than the LDS)."""
    torch = _torch()
    B = _B()
    rng = np.random.default_rng(31)
    L, Hq, Hkv, D, K = 600_000, 28, 4, 128, 512
    G = Hq // Hkv
    k = f32_to_bf16_bits(rng.integers(-2, 3, size=(1, Hkv, L, D), dtype=np.int8).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((1, Hkv, L, D), dtype=np.float32))
    q = f32_to_bf16_bits(rng.integers(-1, 2, size=(1, Hq, D), dtype=np.int8).astype(np.float32))
    layer = B.ReTopKLayer(batch=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, max_len=L, top_k=K,
                          cache_cap=4, window=4, top_r=2, refresh_every=0, tau=0.5)
    out = torch.empty((1, Hq, D), dtype=torch.float32, device="cuda")
    sel = torch.empty((1, Hq, K), dtype=torch.int32, device="cuda")
    kd, vd = B.bf16_tensor(k), B.bf16_tensor(v)
    heads = list(range(G, 2 * G)) + [0, Hq - 1]
    for length in (L, 530_001, 230_000):
        log(f"[long ties] length {length}")
        layer.exact_topk_attn(B.bf16_tensor(q), kd, vd, length, out, sel)
        s, o = sel.cpu().numpy(), out.cpu().numpy()
        for h in heads:
            osel, osc = O.exact_topk_support(q[0, h], k[0, h // G], length, K)
            assert np.array_equal(s[0, h], osel), f"L={length} h={h}"
            check_output(o[0, h], osc, v[0, h // G, osel], D, f"L={length} h={h}")
    for length in (L, 230_000):
        log(f"[long ties] zero query, length {length}")
        layer.exact_topk_attn(B.bf16_tensor(np.zeros((1, Hq, D), np.uint16)), kd, vd, length, out, sel)
        s, o = sel.cpu().numpy(), out.cpu().numpy()
        for h in range(Hq):
            assert np.array_equal(s[0, h], np.arange(K)), f"zero query L={length} h={h}"
            ref = O.bf16_to_f64(v[0, h // G, :K]).mean(0)
            np.testing.assert_allclose(o[0, h], ref, rtol=1e-4, atol=1e-5)
    close_checked(layer)


# ---------------------------------------------------------------------------
# Decode steps
# ---------------------------------------------------------------------------

def test_decode_tiny_lockstep():
    r = run_lockstep("tiny", 64)
    assert r["paths"].sum() >= 0


def test_decode_tiny_refresh_every_8():
    r = run_lockstep("tiny", 40, override=dict(refresh_every=8))
    for t in (8, 16, 24, 32, 40):
        assert r["paths"][t - 1].all()


def test_decode_tiny_forced_exact():
    r = run_lockstep("tiny", 20, override=dict(tau=2.0))
    assert r["paths"].all()


def test_decode_tiny_forced_reuse():
    r = run_lockstep("tiny", 40, override=dict(tau=-2.0, refresh_every=0))
    assert not r["paths"].any()


def test_decode_tiny_window_covers_history():
    """W >= L_t: the candidate set is every key, so reuse equals exact Top-K."""
    run_lockstep("tiny", 6, override=dict(tau=-2.0, refresh_every=0, window=8192))


def test_decode_small_cache_no_window():
    """C = R = 1 and W = 0 (the ablation without the recent-token guard)."""
    run_lockstep("tiny", 30, override=dict(cache_cap=1, top_r=1, window=0))


def test_decode_sixteen_heads_lockstep():
    """16 query heads on one KV head, a refresh every 4 steps."""
    run_lockstep("tiny", 8, override=dict(refresh_every=4),
                 wl_kw=dict(n_q_heads=16, n_kv_heads=1, prompt_len=3000, decode_steps=8))


def test_decode_largest_cache():
    """C = 64 (the largest cache) and R = 8: recall ranks 64 entries, the union
    merges 8 supports."""
    run_lockstep("tiny", 12, wl_kw=dict(cache_cap=64, top_r=8, decode_steps=12))


def test_decode_gqa16k_lockstep():
    run_lockstep("gqa16k", 24, override=dict(refresh_every=12))


def test_decode_gqa32k_batch4_lockstep():
    run_lockstep("gqa32k_b4", 6, wl_kw=dict(decode_steps=8), override=dict(refresh_every=3))


def integer_tie_data(seed, prompt_len=3000, steps=6, hq=8, hkv=2, cache_cap=8, nonzero=3,
                     zero_query_step=None, zero_heads=()):
    """Keys with entries in {-1, 0, 1} and queries with `nonzero` entries of
    +-1: every score is a small integer, exact in fp32, so a reuse head's
    candidates share few distinct scores and the one holding the K-th largest
    is shared by more than 64 of them (the rerank's radix-select fallback),
    with real ties decided by the lower index. Optionally the query of one
    decode step is zero for some heads: all its candidate scores are equal."""
    rng = np.random.default_rng(seed)
    k = f32_to_bf16_bits(rng.integers(-1, 2, size=(1, hkv, prompt_len + steps, 128)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((1, hkv, prompt_len + steps, 128)).astype(np.float32))
    q = np.zeros((1, hq, cache_cap + steps, 128), np.float32)
    for h in range(hq):
        for n in range(cache_cap + steps):
            dims = rng.choice(128, nonzero, replace=False)
            q[0, h, n, dims] = rng.choice([-1.0, 1.0], nonzero)
    if zero_query_step is not None:
        q[0, list(zero_heads), cache_cap + zero_query_step - 1] = 0.0
    q = f32_to_bf16_bits(q)
    wl = WORKLOADS["tiny"].replace(name="integer_ties", n_q_heads=hq, n_kv_heads=hkv, prompt_len=prompt_len,
                                   decode_steps=steps, top_k=100, cache_cap=cache_cap, window=16, top_r=4,
                                   tau=-2.0, refresh_every=0)
    data = dict(k=k, v=v, q_tail=np.ascontiguousarray(q[:, :, :cache_cap]),
                q_dec=np.ascontiguousarray(q[:, :, cache_cap:].transpose(2, 0, 1, 3)))
    return wl, data


def _boundary_crowding(wl, data, steps):
    """Per reuse head-step of the oracle's trajectory: (M_t, candidates sharing
    the K-th score, of which the support keeps `need`)."""
    orc = O.ReTopKOracle.from_workload(wl)
    orc.init_from_prefill(data["q_tail"], data["k"], wl.prompt_len)
    rows = []
    for t in range(1, steps + 1):
        rec = orc.step(data["q_dec"][t - 1], data["k"], data["v"], wl.prompt_len + t, t)
        for h in range(wl.n_q_heads):
            cand = rec.candidates[0][h]
            s = O.qk_scores(data["q_dec"][t - 1][0, h], data["k"][0, h * wl.n_kv_heads // wl.n_q_heads, cand])
            kth = np.sort(s)[::-1][wl.top_k - 1]
            rows.append((len(cand), int((s == kth).sum()), wl.top_k - int((s > kth).sum())))
    return rows


def test_decode_reuse_rerank_integer_ties():
    """Forced reuse on integer-valued scores: the K-th largest candidate score
    is shared by more than 64 candidates at every head-step (checked on the
    oracle's trajectory first), so the rerank takes its radix-select fallback;
    real ties must go to the lower index, with no near-tie allowance."""
    wl, data = integer_tie_data(31)
    rows = _boundary_crowding(wl, data, wl.decode_steps)
    assert all(m > wl.top_k and cnt > 64 and need < cnt for m, cnt, need in rows), rows
    r = run_lockstep("integer_ties", wl.decode_steps, given=(wl, data))
    assert not r["paths"].any()
    assert not r["swaps"], f"integer scores leave no near-tie: {r['swaps'][:3]}"


def test_decode_reuse_zero_query_all_scores_equal():
    """Forced reuse where step 3's query is zero for heads 0-3: every candidate
    score is 0 (minimum = maximum), so the rerank goes straight to the radix
    select and keeps the K lowest candidate indices; the zero q_bar enters the
    cache and step 4 recalls against it (rho = 0)."""
    wl, data = integer_tie_data(32, zero_query_step=3, zero_heads=(0, 1, 2, 3))
    r = run_lockstep("integer_ties", wl.decode_steps, given=(wl, data))
    assert not r["paths"].any() and not r["swaps"]


def test_decode_empty_candidate_set():
    """W = 0 and a restored cache whose supports name only keys past the
    visible length: the reuse heads have no candidate, an empty support and
    the zero output; the entry pushed has support size 0 (restored again
    below, which write_state accepts)."""
    torch = _torch()
    B = _B()
    wl, data = data_for("tiny")
    wl = wl.replace(window=0)
    dev = upload(data)
    L = wl.prompt_len + 1
    layer = B.ReTopKLayer.from_workload(wl, window=0, tau=-2.0, refresh_every=0)
    orc = O.ReTopKOracle.from_workload(wl, window=0, tau=-2.0, refresh_every=0)
    C, K = wl.cache_cap, wl.top_k
    qbar = np.zeros((1, 1, C, 128), np.float32)
    qbar[0, 0, :, 0] = 1.0
    supp = np.zeros((1, 1, C, K), np.int32)
    supp[0, 0, :, :3] = [L, L + 5, wl.max_len - 1]
    slen = np.full((1, 1, C), 3, np.int32)
    count = np.array([[C]], np.int32)
    layer.write_state(qbar, supp, slen, count)
    out = torch.full((1, 1, 128), 7.0, dtype=torch.float32, device="cuda")
    orc.set_state(*layer.read_state())
    layer.decode_step(dev["q_dec"][0], dev["k"], dev["v"], L, 1, out)
    rec = orc.step(data["q_dec"][0], data["k"], data["v"], L, 1)
    info = layer.step_info()
    assert rec.n_cand[0, 0] == 0 and len(rec.support[0][0]) == 0
    assert info["path"][0, 0] == 0 and info["n_cand"][0, 0] == 0 and info["sel_len"][0, 0] == 0
    assert np.array_equal(out.cpu().numpy(), np.zeros((1, 1, 128), np.float32))
    st = layer.read_state()
    assert st[3][0, 0] == C and st[2][0, 0, C - 1] == 0
    layer.write_state(*st)
    close_checked(layer)


def test_decode_tiny_recent_r():
    """Recent-R retrieval (the component ablation): the R newest entries and
    rho_max over them, in lockstep with the oracle, a refresh every 8 steps."""
    r = run_lockstep("tiny", 24, override=dict(retrieval="recent", refresh_every=8))
    assert r["paths"][7].all()


def periodic_query_data(seed, period=8, noise=0.3, steps=24):
    """Queries cycling through `period` random directions (plus noise): the
    entries most similar to q_t are `period` steps old, while the R < period
    newest point elsewhere, so the two retrievals decide differently."""
    wl = WORKLOADS["tiny"].replace(name="periodic", decode_steps=steps, prompt_len=3000)
    data = dict(generate(wl))
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((period, 128))
    n0 = data["q_tail"].shape[2]
    qs = np.stack([base[n % period] + noise * rng.standard_normal(128) for n in range(n0 + steps)])
    q = f32_to_bf16_bits(qs.astype(np.float32))
    data["q_tail"] = np.ascontiguousarray(q[:n0][None, None])
    data["q_dec"] = np.ascontiguousarray(q[n0:][:, None, None])
    return wl, data


def test_decode_periodic_queries_both_retrievals():
    """Similarity-guided retrieval finds the same-direction entries (rho_max
    about 0.9: reuse); recent-R sees only the newest, unrelated ones (rho_max
    near 0: the exact path). Both in lockstep with the oracle."""
    wl, data = periodic_query_data(41)
    sim = run_lockstep("periodic", wl.decode_steps, given=(wl, data))
    rec = run_lockstep("periodic", wl.decode_steps, given=(wl, data), override=dict(retrieval="recent"))
    assert sim["paths"].mean() < 0.2 and rec["paths"].mean() > 0.8, (sim["paths"].mean(), rec["paths"].mean())


def test_decode_free_running_tiny():
    """Without re-synchronisation the GPU trajectory matches the oracle's until
    the first near-tie swap (if any)."""
    torch = _torch()
    B = _B()
    wl, data = data_for("tiny")
    dev = upload(data)
    layer = B.ReTopKLayer.from_workload(wl, refresh_every=16)
    orc = O.ReTopKOracle.from_workload(wl, refresh_every=16)
    layer.init_from_prefill(dev["q_tail"], dev["k"], wl.prompt_len)
    orc.init_from_prefill(data["q_tail"], data["k"], wl.prompt_len)
    out = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    matched = 0
    for t in range(1, wl.decode_steps + 1):
        L = wl.prompt_len + t
        layer.decode_step(dev["q_dec"][t - 1], dev["k"], dev["v"], L, t, out)
        rec = orc.step(data["q_dec"][t - 1], data["k"], data["v"], L, t)
        info = layer.step_info()
        swaps, errs = [], []
        compare_step(rec, info, out.cpu().numpy(), data["q_dec"][t - 1], data["k"], data["v"], orc,
                     wl.tau, [(0, 0)], swaps, errs)
        if swaps:
            break
        matched = t
    log(f"[free-running] tiny: identical for {matched} of {wl.decode_steps} steps")
    close_checked(layer)


def test_determinism_and_resume():
    """Same inputs give bit-identical outputs and caches; a snapshot restored
    into a fresh handle continues identically."""
    torch = _torch()
    B = _B()
    wl, data = data_for("gqa16k")
    dev = upload(data)
    n1, n2 = 6, 6

    def run(layer, t0, n):
        outs = []
        out = torch.empty((1, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
        for t in range(t0, t0 + n):
            layer.decode_step(dev["q_dec"][t - 1], dev["k"], dev["v"], wl.prompt_len + t, t, out)
            outs.append(out.cpu().numpy().copy())
        return np.stack(outs)

    a = B.ReTopKLayer.from_workload(wl, refresh_every=4)
    a.init_from_prefill(dev["q_tail"], dev["k"], wl.prompt_len)
    oa1 = run(a, 1, n1)
    snap = a.read_state()
    oa2 = run(a, 1 + n1, n2)
    sa = a.read_state()
    b = B.ReTopKLayer.from_workload(wl, refresh_every=4)
    b.init_from_prefill(dev["q_tail"], dev["k"], wl.prompt_len)
    ob1 = run(b, 1, n1)
    assert np.array_equal(oa1.view(np.uint32), ob1.view(np.uint32))
    c = B.ReTopKLayer.from_workload(wl, refresh_every=4)
    c.write_state(*snap)
    assert all(np.array_equal(x, y) for x, y in zip(c.read_state(), snap))
    oc2 = run(c, 1 + n1, n2)
    assert np.array_equal(oa2.view(np.uint32), oc2.view(np.uint32))
    assert all(np.array_equal(x, y) for x, y in zip(c.read_state(), sa))
    for layer in (a, b, c):
        close_checked(layer)


def test_stats_ring_matches_step_info():
    torch = _torch()
    B = _B()
    wl, data = data_for("gqa16k")
    dev = upload(data)
    layer = B.ReTopKLayer.from_workload(wl, refresh_every=5)
    layer.init_from_prefill(dev["q_tail"], dev["k"], wl.prompt_len)
    out = torch.empty((1, wl.n_q_heads, 128), dtype=torch.float32, device="cuda")
    infos = []
    for t in range(1, 11):
        layer.decode_step(dev["q_dec"][t - 1], dev["k"], dev["v"], wl.prompt_len + t, t, out)
        infos.append(layer.step_info())
    path, rho, m = layer.stats(1, 10)
    for i, info in enumerate(infos):
        t = i + 1
        assert np.array_equal(path[i] & 1, info["path"])
        assert np.all(((path[i] >> 1) & 1) == (1 if t % 5 == 0 else 0))
        assert np.array_equal(rho[i], info["rho_max"])
        assert np.array_equal(m[i], np.where(info["path"] == 1, 0, info["n_cand"]))
    close_checked(layer)


# ---------------------------------------------------------------------------
# Full-size configurations: every head for a few steps, then longer sampled runs
# ---------------------------------------------------------------------------

@pytest.mark.slow
@pytest.mark.timeout(900)
def test_headline_128k_every_head():
    """L0 = 131072, 28/4 heads, K = 512, in the launch configuration the bench
    times: every query head in lockstep for 6 steps with a refresh at step 3
    (the initialisation compared on KV group 1), then the Exact Top-K baseline
    on every head."""
    r = run_lockstep("headline128k", 6, override=dict(refresh_every=3), wl_kw=dict(decode_steps=16),
                     check_init=(0, 1))
    assert r["paths"][2].all()
    swaps = run_exact("headline128k", [131072 + 5], wl_kw=dict(decode_steps=16))
    log(f"[exact] headline every head: swaps {len(swaps)}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_headline_128k_longer_lockstep():
    """L0 = 131072: KV group 2 in lockstep for 40 steps with a refresh every 16
    (the cache from the GPU's initialisation), so that the cache turns over
    more than once at full size."""
    r = run_lockstep("headline128k", 40, sub=(0, 2), override=dict(refresh_every=16), check_init=False,
                     wl_kw=dict(decode_steps=48))
    assert r["paths"].sum() >= 2 * 7  # two refreshes at least


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_headline_128k_forced_reuse_k1024():
    """K = 1024 at 128K (the pages' cross-model budget): every head forced onto
    the reuse path (tau = -2, T_r = 0) for 4 lockstep steps, R K + W = 4128
    candidates at most."""
    r = run_lockstep("headline128k", 4, override=dict(top_k=1024, tau=-2.0, refresh_every=0),
                     check_init=False, wl_kw=dict(decode_steps=8))
    assert not r["paths"].any()
    assert max(r["ms"]) > 1024


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_gqa64k_b4_every_head():
    """Batch 4 at L0 = 65536 (scores in the workspace, exact calls on every
    CU): all 112 query heads in lockstep for 4 steps with a refresh at step 2,
    then the Exact Top-K baseline on every head."""
    run_lockstep("gqa64k_b4", 4, override=dict(refresh_every=2), check_init=False, wl_kw=dict(decode_steps=8))
    run_exact("gqa64k_b4", [65536 + 2], wl_kw=dict(decode_steps=8))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stress_128k_b8_every_head():
    """Batch 8 at L0 = 131072 with K = 2048 and tau = 0.99 (mostly exact): all
    224 query heads in lockstep for 3 steps, then the Exact Top-K baseline on
    every head."""
    r = run_lockstep("stress128k_b8", 3, check_init=False, wl_kw=dict(decode_steps=8))
    assert r["paths"].mean() > 0.9
    run_exact("stress128k_b8", [131072 + 3], wl_kw=dict(decode_steps=8))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stress_shape_forced_reuse_k2048():
    """The stress layer's largest reuse layout: one batch row at L0 = 131072,
    K = 2048, every head forced onto the reuse path (tau = -2, T_r = 0) for 4
    lockstep steps; R K + W = 8224 candidates at most (low query similarity
    keeps the retrieved supports apart, so the union is large)."""
    r = run_lockstep("stress128k_b8", 4, override=dict(tau=-2.0, refresh_every=0), check_init=False,
                     wl_kw=dict(batch=1, decode_steps=8))
    assert not r["paths"].any()
    assert max(r["ms"]) > 4096


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_scale_1m_every_head():
    """L0 = 1,048,576 (one-layer scaling): every head in lockstep for 4 steps
    with a refresh every 2 steps (the cache from the GPU's initialisation); the
    reuse steps' unions merge the sorted supports (R K = 2048, beyond one LDS
    bitmap window of 262,144 positions). Then the Exact Top-K baseline on
    every head."""
    run_lockstep("scale1m", 4, override=dict(refresh_every=2), check_init=False, wl_kw=dict(decode_steps=8))
    run_exact("scale1m", [(1 << 20) + 3], wl_kw=dict(decode_steps=8))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_merged_union_with_empty_list_slots():
    """Past one LDS bitmap window (L0 = 300,000) the reuse union merges the
    retrieved supports, in a form compiled for 4 lists or for 8, with the slots
    past the number retrieved left empty. R = 3 at K = 512 leaves one of 4 slots
    empty; R = 6 at K = 256 (R K = 1536) takes the 8-list form with two empty.
    KV group 1, every head forced onto the reuse path, 3 lockstep steps each."""
    for top_r, top_k in ((3, 512), (6, 256)):
        r = run_lockstep("scale1m", 3, sub=(0, 1), override=dict(top_k=top_k, top_r=top_r, tau=-2.0, refresh_every=0),
                         check_init=False, wl_kw=dict(prompt_len=300000, decode_steps=8))
        assert not r["paths"].any()
        assert max(r["ms"]) > top_k


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_scale_1m_forced_reuse_k1024_bitmap_windows():
    """L0 = 1,048,576 with K = 1024, KV group 1 forced onto the reuse path
    (tau = -2, T_r = 0) for 3 lockstep steps: R K = 4096 is more than the
    merged union takes, so the union sweeps four LDS bitmap windows of 262,144
    positions, each ranked on its own and appended after the previous ones."""
    r = run_lockstep("scale1m", 3, sub=(0, 1), override=dict(top_k=1024, tau=-2.0, refresh_every=0),
                     check_init=False, wl_kw=dict(decode_steps=8))
    assert not r["paths"].any()
    assert max(r["ms"]) > 1024


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_scale_4m_sampled():
    """L0 = 4,194,304 (K and V of the layer 8.6 GB; scores, survivors and
    boundary keys in their workspaces): KV group 1 in lockstep for 4 steps
    with a refresh every 2 steps (the cache from the GPU's initialisation), the
    reuse unions merging the sorted supports; then the Exact Top-K baseline on
    KV group 3."""
    run_lockstep("scale4m", 4, sub=(0, 1), override=dict(refresh_every=2), check_init=False,
                 wl_kw=dict(decode_steps=8))
    run_exact("scale4m", [(1 << 22) + 3], sub=(0, 3), wl_kw=dict(decode_steps=8))
