"""Helpers for comparing the HIP path (through the C ABI) with the CPU oracle.

Acceptance rules (decode step, per batch row b and query head h):
  * path, refresh and the retrieved FIFO positions: identical; a path may only
    differ if the oracle's rho_max lies within 1e-12 of tau;
  * rho_max: within 1e-12 (both fp64 dot products of identical fp32 inputs);
  * candidate set A_t and M_t on reuse heads: identical;
  * selected support: identical as a set, except for swaps between keys whose
    oracle (fp64) scores lie within 1e-5 * |s_(K)| of the oracle's K-th score;
  * output: max|o_gpu - o_ref| / max|o_ref| <= 5e-3, where o_ref is the
    oracle's Eq. (12) over the support the GPU selected (the oracle's own
    output when the sets agree);
  * cache: the new entry's q_bar is bit-identical to the oracle's, its support
    is the GPU's selection.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.retopk_oracle as O

SWAP_REL = 1e-5
OUT_REL = 5e-3
RHO_ABS = 1e-12


def sub_problem(data, b, g, group):
    """Slice one (batch row, KV group) out of a batch: heads are independent."""
    hs = slice(g * group, (g + 1) * group)
    return dict(k=data["k"][b:b + 1, g:g + 1], v=data["v"][b:b + 1, g:g + 1],
                q_tail=data["q_tail"][b:b + 1, hs], q_dec=data["q_dec"][:, b:b + 1, hs])


def check_support(gpu_sel, orc_sel, q_bits, k_head_bits, where, swaps):
    """Compare selected index sets with the near-tie allowance; returns the
    fp64 scores of the GPU's support."""
    gpu_sel = np.asarray(gpu_sel, dtype=np.int64)
    orc_sel = np.asarray(orc_sel, dtype=np.int64)
    assert len(gpu_sel) == len(orc_sel), f"{where}: support size {len(gpu_sel)} != {len(orc_sel)}"
    assert np.all(np.diff(gpu_sel) > 0), f"{where}: GPU support not strictly ascending"
    gs = O.qk_scores(q_bits, k_head_bits[gpu_sel])
    if np.array_equal(gpu_sel, orc_sel):
        return gs
    os_ = O.qk_scores(q_bits, k_head_bits[orc_sel])
    s_k = float(np.min(os_))
    tol = SWAP_REL * max(abs(s_k), 1e-30)
    diff = np.setxor1d(gpu_sel, orc_sel)
    ds = O.qk_scores(q_bits, k_head_bits[diff])
    worst = float(np.max(np.abs(ds - s_k)))
    assert worst <= tol, (f"{where}: support differs beyond a near-tie: {len(diff)} indices, "
                          f"worst |s - s_K| = {worst:.3e} > {tol:.3e}")
    swaps.append((where, len(diff) // 2, worst / max(abs(s_k), 1e-30)))
    return gs


def check_output(out_gpu, gs, v_rows_bits, d, where):
    ref = O.sparse_softmax_v(gs, O.bf16_to_f64(v_rows_bits), d)
    err = float(np.max(np.abs(out_gpu.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))
    assert err <= OUT_REL, f"{where}: output relative error {err:.3e} > {OUT_REL}"
    return err


def compare_step(rec, info, out_gpu, q_bits, k_bits, v_bits, orc, tau, heads, swaps, errs):
    """Check one decode step. `heads` lists (b, h) in the oracle's indexing."""
    hkv, hq, d = orc.hkv, orc.hq, orc.d
    for b, h in heads:
        g = h * hkv // hq
        where = f"t={rec.t_dec} b={b} h={h}"
        margin = abs(rec.rho_max[b, h] - tau) if math.isfinite(rec.rho_max[b, h]) else math.inf
        if info["path"][b, h] != rec.path[b, h]:
            assert margin < 1e-12, f"{where}: path differs (gpu {info['path'][b, h]}, oracle {rec.path[b, h]})"
            continue
        if math.isinf(rec.rho_max[b, h]):
            assert math.isinf(info["rho_max"][b, h]), f"{where}: rho_max"
        else:
            assert abs(info["rho_max"][b, h] - rec.rho_max[b, h]) <= RHO_ABS, (
                f"{where}: rho_max {info['rho_max'][b, h]!r} vs {rec.rho_max[b, h]!r}")
        n_ret = len(rec.retrieved[b][h])
        assert list(info["retrieved"][b, h, :n_ret]) == list(rec.retrieved[b][h]), f"{where}: retrieved"
        assert np.all(info["retrieved"][b, h, n_ret:] == -1), f"{where}: retrieved padding"
        if rec.path[b, h] == O.REUSE:
            m = int(rec.n_cand[b, h])
            assert info["n_cand"][b, h] == m, f"{where}: M_t {info['n_cand'][b, h]} != {m}"
            assert np.array_equal(info["cand"][b, h, :m], rec.candidates[b][h]), f"{where}: A_t differs"
        n = int(info["sel_len"][b, h])
        gsel = info["sel"][b, h, :n]
        gs = check_support(gsel, rec.support[b][h], q_bits[b, h], k_bits[b, g], where, swaps)
        np.testing.assert_allclose(info["sel_scores"][b, h, :n], gs, rtol=0,
                                   atol=SWAP_REL * max(1.0, float(np.max(np.abs(gs)))),
                                   err_msg=f"{where}: selected scores")
        errs.append(check_output(out_gpu[b, h], gs, v_bits[b, g, gsel], d, where))


def compare_cache_entry(state, orc_qbar, b, h, gpu_sel, where):
    qbar, supp, slen, count = state
    n = int(count[b, h])
    assert n >= 1
    assert np.array_equal(qbar[b, h, n - 1].view(np.uint32), orc_qbar.view(np.uint32)), (
        f"{where}: cached q_bar not bit-identical")
    assert np.array_equal(supp[b, h, n - 1, :slen[b, h, n - 1]], gpu_sel), f"{where}: cached support"
