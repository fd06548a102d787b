"""CPU oracle for ReTopK decode-step attention.

TEST INFRASTRUCTURE ONLY. This module is imported solely by ``tests/``, by
``__graft_entry__.smoke()`` (to check one small GPU call) and by the
``cpu_baseline`` leg of ``bench.py``. The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this module
imports nothing from the product. The two share no code; only the seeded input
generator (which holds none of the method's arithmetic) feeds both.

It is a plain, slow, obviously-correct implementation in float64 of what the
paper "Recall Before You Rank: Similarity-Guided Top-K Reuse for Efficient
Long-Context Attention" (ReTopK, arXiv 2607.27692) computes at one decode step,
written from its Methodology section, in the paper's order and notation:

  Exact Top-K support S_t ........ Motivation, Eq. (1); scores Eq. (4)
  query-support FIFO cache B_t ... Recall-Before-Rerank Selection, Eq. (5)
  cosine recall rho_{t,c} ........ Eq. (6)
  TopR retrieval and rho_max ..... Eq. (7)
  recent-R retrieval (ablation) .. Experiments, component ablation, Table 3
  recent window L_t .............. Eq. (8)
  candidate set A_t, M_t ......... Eq. (9)
  candidate scores e_hat ......... Eq. (10)
  reranked support S_hat_t ....... Eq. (11)
  sparse softmax-V output ........ Eq. (12)
  dense attention (comparison) ... Eq. (4) over all keys, then Eq. (12);
                                   Table 1 "Full Attention", Figure 9
  fallback / refresh path P_t .... Reliable Reuse via Fallback and Refresh, Eq. (13)
  cache update after both paths .. same subsection, closing sentence
  cache initialisation ........... Query-support cache paragraph (final C prompt
                                   tokens during prefill)

Readings taken where the paper is silent:
  * indices are 0-based; the window of Eq. (8) is [max(0, L_t - W), L_t);
  * L_t counts the key of the token being decoded (the caller appends it first);
  * the first decode step has t_dec = 1, so refresh fires at t_dec = T_r, 2T_r, ...;
  * the fallback test is strict: rho_max < tau takes the exact path, rho_max = tau reuses;
  * an empty cache gives rho_max = -inf, hence the exact path;
  * TopR ties go to the older cache entry (lower FIFO position, 0 = oldest);
  * TopK ties go to the lower token index; selection ranks the unscaled score
    q.k, which orders keys exactly as q.k / sqrt(d) does;
  * fewer than K keys (or candidates) available: all of them are taken;
  * q_bar is stored as float32: fp64 sum of squares, fp64 sqrt, fp64 divide,
    one rounding to float32 (round to nearest even); a zero query gives 0;
  * rho is an fp64 dot product of the float32 q_bar values;
  * query head h reads KV head floor(h * Hkv / Hq) (contiguous GQA groups),
    and every query head keeps its own cache;
  * refresh applies to all heads at once; the similarity fallback is per head;
  * recent-R retrieval (ablation): the R newest entries, newest first, and
    rho_max over them only (under which the exact-path rate rises, as the
    ablation reports);
  * supports are stored in ascending token order;
  * a stored support entry that is not a visible key at step t (>= L_t; only a
    restored snapshot can hold one) is not a candidate; a reuse head with no
    candidate at all (W = 0) has an empty support and the zero output;
  * softmax is evaluated with the maximum subtracted (identical in exact
    arithmetic to Eq. (12));
  * prompt entry p of the cache holds the causal Exact Top-K support of prompt
    query p over keys 0..p; entries are pushed oldest first.

Inputs are raw bf16 bit patterns (numpy uint16); this module decodes them
itself.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

EXACT = 1
REUSE = 0


# ----------------------------------------------------------------------------
# Elementary steps
# ----------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64, exactly.

    A bf16 value is the upper half of an IEEE float32, so shifting the 16 bits
    into the top of a 32-bit word gives that float32, which float64 holds
    exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def normalize_query(q_bits) -> np.ndarray:
    """q_bar = q / ||q||_2 (Eq. (5) and Eq. (6)), stored as float32.

    Sum of squares, square root and division in float64, then one rounding to
    float32. The zero query maps to the zero vector.
    """
    x = bf16_to_f64(q_bits)
    n = math.sqrt(float(np.sum(x * x)))
    if n == 0.0:
        return np.zeros(x.shape, dtype=np.float32)
    return (x / n).astype(np.float32)


def cosine_recall(qbar_t: np.ndarray, cached_qbars) -> list[float]:
    """rho_{t,c} = q_bar_t . q_bar_c for every cache entry c (Eq. (6)), in float64."""
    a = qbar_t.astype(np.float64)
    return [float(np.dot(a, c.astype(np.float64))) for c in cached_qbars]


def top_r(rho: list[float], r: int):
    """R_t = TopR(rho, R) and rho_max = max_c rho (Eq. (7)).

    Returns FIFO positions (0 = oldest), best first; ties go to the older
    entry. With fewer than R entries all are returned; with none, rho_max is
    -inf.
    """
    order = sorted(range(len(rho)), key=lambda c: (-rho[c], c))
    rho_max = max(rho) if rho else -math.inf
    return order[: min(r, len(rho))], rho_max


def recent_r(rho: list[float], r: int):
    """The recent-R retrieval of the component ablation (Experiments,
    "Hyperparameter sensitivity and component ablation", Table 3), in place of
    Eq. (7): R_t = the min(R, |B_t|) newest entries, newest first, whatever
    their similarity. rho_max is taken over those entries only, the reading
    under which this ablation changes the exact-path rate, as the paper
    reports (11.6% -> 16.7%); with none, -inf.
    """
    n = len(rho)
    chosen = [n - 1 - i for i in range(min(r, n))]
    rho_max = max(rho[c] for c in chosen) if chosen else -math.inf
    return chosen, rho_max


def recent_window(length: int, window: int) -> np.ndarray:
    """L_t of Eq. (8), 0-based: the last W key positions [max(0, L-W), L)."""
    return np.arange(max(0, length - window), length, dtype=np.int64)


def candidate_set(supports, retrieved, length: int, window: int) -> np.ndarray:
    """A_t = Unique(union of the retrieved supports and the window) (Eq. (9)).

    Only keys visible at this step can be candidates: a stored support entry
    >= length (possible only in a cache restored from a snapshot, since a
    cache written by decoding holds earlier steps' supports of shorter
    lengths) is left out, as the scores of Eq. (10) range over the keys
    currently available. Returned sorted ascending; M_t is its length.
    """
    pool: set[int] = set()
    for c in retrieved:
        pool.update(int(i) for i in supports[c] if int(i) < length)
    pool.update(int(i) for i in recent_window(length, window))
    return np.array(sorted(pool), dtype=np.int64)


def qk_scores(q_bits, k_rows_bits) -> np.ndarray:
    """Unscaled scores q . k_i for the given key rows (numerators of Eqs. (4), (10))."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_rows_bits)
    return k @ q


def top_k(indices: np.ndarray, scores: np.ndarray, k: int) -> np.ndarray:
    """TopK of Eq. (1) / Eq. (11): the k largest scores, ties to the lower index.

    Returns the chosen token indices in ascending order. Fewer than k inputs:
    all of them.
    """
    indices = np.asarray(indices, dtype=np.int64)
    order = np.lexsort((indices, -np.asarray(scores, dtype=np.float64)))
    return np.sort(indices[order[: min(k, len(indices))]])


def sparse_softmax_v(scores: np.ndarray, v_rows: np.ndarray, head_dim: int) -> np.ndarray:
    """o = sum_i softmax(e)_i v_i over the selected entries, e = s / sqrt(d) (Eq. (12)).

    An empty support (a reuse head left with no candidate, possible only with
    W = 0) gives the zero vector: the sum of Eq. (12) has no terms.
    """
    if len(scores) == 0:
        return np.zeros(head_dim)
    e = np.asarray(scores, dtype=np.float64) / math.sqrt(head_dim)
    w = np.exp(e - np.max(e))
    return (w @ np.asarray(v_rows, dtype=np.float64)) / np.sum(w)


def exact_topk_support(q_bits, k_bits_head, length: int, k: int):
    """S_t over keys 0..length-1 (Eq. (1)); returns (indices ascending, their scores)."""
    s = qk_scores(q_bits, k_bits_head[:length])
    sel = top_k(np.arange(length), s, k)
    return sel, s[sel]


def exact_topk_attention(q_bits, k_bits, v_bits, length: int, k: int):
    """Exact Top-K attention baseline (Problem Setup, Eqs. (1), (4), then Eq. (12)).

    q_bits [B, Hq, d]; k_bits, v_bits [B, Hkv, >=length, d].
    Returns (out [B, Hq, d] float64, list of selected index arrays per (b, h)).
    """
    bsz, hq, d = q_bits.shape
    hkv = k_bits.shape[1]
    out = np.zeros((bsz, hq, d))
    sel_all = []
    for b in range(bsz):
        row = []
        for h in range(hq):
            g = h * hkv // hq
            sel, s = exact_topk_support(q_bits[b, h], k_bits[b, g], length, k)
            out[b, h] = sparse_softmax_v(s, bf16_to_f64(v_bits[b, g, sel]), d)
            row.append(sel)
        sel_all.append(row)
    return out, sel_all


def dense_attention(q_bits, k_bits, v_bits, length: int):
    """Full (dense) softmax attention over every cached key, the "Full
    Attention" column set beside Exact Top-K (Experimental Results, Table 1;
    Kernel efficiency analysis, Figure 9): the scores of Eq. (4) for all
    i < length and Eq. (12)'s softmax-value aggregation with the support taken
    as all of them.

    q_bits [B, Hq, d]; k_bits, v_bits [B, Hkv, >=length, d] (rows >= length are
    not read). Returns out [B, Hq, d] float64.
    """
    bsz, hq, d = q_bits.shape
    hkv = k_bits.shape[1]
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        for h in range(hq):
            kv_head = h * hkv // hq
            every = k_bits[b, kv_head, :length]
            out[b, h] = sparse_softmax_v(qk_scores(q_bits[b, h], every),
                                         bf16_to_f64(v_bits[b, kv_head, :length]), d)
    return out


# ----------------------------------------------------------------------------
# The per-head query-support cache and the decode step
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class StepRecord:
    """Everything one decode step decides and produces, per (b, h)."""
    t_dec: int
    length: int
    refresh: bool
    path: np.ndarray          # [B, Hq] EXACT / REUSE
    rho_max: np.ndarray       # [B, Hq] float64
    retrieved: list           # [B][Hq] FIFO positions (reuse and exact alike)
    candidates: list          # [B][Hq] A_t ascending (None on exact heads)
    n_cand: np.ndarray        # [B, Hq] M_t (0 on exact heads)
    support: list             # [B][Hq] S_hat_t ascending
    support_scores: list      # [B][Hq] unscaled scores of S_hat_t
    out: np.ndarray           # [B, Hq, d] float64


class ReTopKOracle:
    """Reference ReTopK state machine for one attention layer.

    Keeps, for every (batch, query head), a FIFO list of (q_bar, support)
    pairs, oldest first, of capacity C (Eq. (5)).
    """

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, top_k, cache_cap,
                 window, top_r, refresh_every, tau, retrieval="similarity"):
        if n_q_heads % n_kv_heads:
            raise ValueError("query heads must be a multiple of KV heads")
        self.batch, self.hq, self.hkv, self.d = batch, n_q_heads, n_kv_heads, head_dim
        self.k, self.c, self.w, self.r = top_k, cache_cap, window, top_r
        self.refresh_every, self.tau = refresh_every, float(tau)
        if retrieval not in ("similarity", "recent"):
            raise ValueError("retrieval is 'similarity' (Eq. (7)) or 'recent' (ablation)")
        self.retrieval = retrieval
        self.cache = [[[] for _ in range(n_q_heads)] for _ in range(batch)]

    @classmethod
    def from_workload(cls, wl, **override):
        p = dict(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                 head_dim=wl.head_dim, top_k=wl.top_k, cache_cap=wl.cache_cap,
                 window=wl.window, top_r=wl.top_r, refresh_every=wl.refresh_every,
                 tau=wl.tau)
        p.update(override)
        return cls(**p)

    def kv_head(self, h: int) -> int:
        return h * self.hkv // self.hq

    def push(self, b: int, h: int, qbar: np.ndarray, support: np.ndarray):
        """FIFO insert; the oldest entry is dropped once more than C are held."""
        entries = self.cache[b][h]
        entries.append((qbar.astype(np.float32), np.asarray(support, dtype=np.int64)))
        if len(entries) > self.c:
            entries.pop(0)

    def init_from_prefill(self, q_tail, k_bits, prompt_len: int):
        """Fill each cache from the final min(C, L0) prompt queries.

        q_tail [B, Hq, n0, d] holds prompt positions L0-n0 .. L0-1 in order.
        Entry for position p: (q_bar_p, causal Exact Top-K support over keys 0..p).
        """
        n0 = min(self.c, prompt_len)
        if q_tail.shape[2] != n0:
            raise ValueError(f"q_tail must hold {n0} prompt queries")
        for b in range(self.batch):
            for h in range(self.hq):
                g = self.kv_head(h)
                self.cache[b][h] = []
                for i in range(n0):
                    p = prompt_len - n0 + i
                    sel, _ = exact_topk_support(q_tail[b, h, i], k_bits[b, g], p + 1, self.k)
                    self.push(b, h, normalize_query(q_tail[b, h, i]), sel)

    def step(self, q_bits, k_bits, v_bits, length: int, t_dec: int) -> StepRecord:
        """One decode step over all (b, h) at visible length L_t = ``length``."""
        bsz, hq, d = self.batch, self.hq, self.d
        refresh = self.refresh_every > 0 and t_dec % self.refresh_every == 0
        rec = StepRecord(t_dec=t_dec, length=length, refresh=refresh,
                         path=np.zeros((bsz, hq), dtype=np.int64),
                         rho_max=np.zeros((bsz, hq)), retrieved=[], candidates=[],
                         n_cand=np.zeros((bsz, hq), dtype=np.int64), support=[],
                         support_scores=[], out=np.zeros((bsz, hq, d)))
        for b in range(bsz):
            r_row, a_row, s_row, sc_row = [], [], [], []
            for h in range(hq):
                g = self.kv_head(h)
                entries = self.cache[b][h]
                qbar = normalize_query(q_bits[b, h])
                rho = cosine_recall(qbar, [e[0] for e in entries])
                if self.retrieval == "similarity":
                    retrieved, rho_max = top_r(rho, self.r)
                else:
                    retrieved, rho_max = recent_r(rho, self.r)
                exact = refresh or rho_max < self.tau
                if exact:
                    sel, sel_s = exact_topk_support(q_bits[b, h], k_bits[b, g], length, self.k)
                    cand = None
                else:
                    cand = candidate_set([e[1] for e in entries], retrieved, length, self.w)
                    cand_s = qk_scores(q_bits[b, h], k_bits[b, g, cand])
                    sel = top_k(cand, cand_s, self.k)
                    sel_s = cand_s[np.searchsorted(cand, sel)]
                    rec.n_cand[b, h] = len(cand)
                rec.out[b, h] = sparse_softmax_v(sel_s, bf16_to_f64(v_bits[b, g, sel]), d)
                rec.path[b, h] = EXACT if exact else REUSE
                rec.rho_max[b, h] = rho_max
                self.push(b, h, qbar, sel)
                r_row.append(retrieved)
                a_row.append(cand)
                s_row.append(sel)
                sc_row.append(sel_s)
            rec.retrieved.append(r_row)
            rec.candidates.append(a_row)
            rec.support.append(s_row)
            rec.support_scores.append(sc_row)
        return rec

    # -- state exchange in the library's snapshot layout (oldest entry first) --

    def get_state(self):
        """Return (qbar [B,Hq,C,d] f32, supp [B,Hq,C,K] i32, supp_len [B,Hq,C] i32,
        count [B,Hq] i32), entries oldest first, unused slots zero."""
        bsz, hq, c, k, d = self.batch, self.hq, self.c, self.k, self.d
        qbar = np.zeros((bsz, hq, c, d), np.float32)
        supp = np.zeros((bsz, hq, c, k), np.int32)
        slen = np.zeros((bsz, hq, c), np.int32)
        count = np.zeros((bsz, hq), np.int32)
        for b in range(bsz):
            for h in range(hq):
                entries = self.cache[b][h]
                count[b, h] = len(entries)
                for i, (qb, s) in enumerate(entries):
                    qbar[b, h, i] = qb
                    supp[b, h, i, : len(s)] = s
                    slen[b, h, i] = len(s)
        return qbar, supp, slen, count

    def set_state(self, qbar, supp, supp_len, count):
        for b in range(self.batch):
            for h in range(self.hq):
                n = int(count[b, h])
                self.cache[b][h] = [
                    (np.array(qbar[b, h, i], dtype=np.float32),
                     np.array(supp[b, h, i, : supp_len[b, h, i]], dtype=np.int64))
                    for i in range(n)]
