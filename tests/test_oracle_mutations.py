"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and check that the pins catch every one of them."""
import os
import sys
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "retopk_oracle.py")

# (name, text in the oracle, planted replacement)
MUTATIONS = [
    ("window_off_by_one", "np.arange(max(0, length - window), length,",
     "np.arange(max(0, length - window - 1), length - 1,"),
    ("window_dropped", "pool.update(int(i) for i in recent_window(length, window))", "pass"),
    ("topk_ties_to_higher_index", "np.lexsort((indices, -np.asarray(scores",
     "np.lexsort((-indices, -np.asarray(scores"),
    ("topk_picks_smallest", "np.lexsort((indices, -np.asarray(scores, dtype=np.float64)))",
     "np.lexsort((indices, np.asarray(scores, dtype=np.float64)))"),
    ("topr_least_similar", "key=lambda c: (-rho[c], c)", "key=lambda c: (rho[c], c)"),
    ("topr_ties_to_newer", "key=lambda c: (-rho[c], c)", "key=lambda c: (-rho[c], -c)"),
    ("fifo_drops_newest", "entries.pop(0)", "entries.pop(-1)"),
    ("softmax_unscaled", "e = np.asarray(scores, dtype=np.float64) / math.sqrt(head_dim)",
     "e = np.asarray(scores, dtype=np.float64)"),
    ("softmax_wrong_sign", "w = np.exp(e - np.max(e))", "w = np.exp(np.max(e) - e)"),
    ("exact_drops_newest_key", "s = qk_scores(q_bits, k_bits_head[:length])",
     "s = qk_scores(q_bits, k_bits_head[:length - 1])"),
    ("fallback_not_strict", "exact = refresh or rho_max < self.tau",
     "exact = refresh or rho_max <= self.tau"),
    ("fallback_inverted", "exact = refresh or rho_max < self.tau",
     "exact = refresh or rho_max > self.tau"),
    ("refresh_off_by_one", "t_dec % self.refresh_every == 0",
     "(t_dec + 1) % self.refresh_every == 0"),
    ("norm_without_sqrt", "n = math.sqrt(float(np.sum(x * x)))", "n = float(np.sum(x * x))"),
    ("gqa_interleaved", "return h * self.hkv // self.hq", "return h % self.hkv"),
    ("no_update_on_exact", "self.push(b, h, qbar, sel)",
     "(None if exact else self.push(b, h, qbar, sel))"),
    ("init_not_causal", "exact_topk_support(q_tail[b, h, i], k_bits[b, g], p + 1, self.k)",
     "exact_topk_support(q_tail[b, h, i], k_bits[b, g], prompt_len, self.k)"),
    ("init_newest_first", "for i in range(n0):\n                    p = prompt_len - n0 + i",
     "for i in reversed(range(n0)):\n                    p = prompt_len - n0 + i"),
    ("rerank_uses_wrong_query", "cand_s = qk_scores(q_bits[b, h], k_bits[b, g, cand])",
     "cand_s = qk_scores(q_bits[b, (h + 1) % hq], k_bits[b, g, cand])"),
    ("bf16_decode_shift_15", "astype(np.uint32) << np.uint32(16)", "astype(np.uint32) << np.uint32(15)"),
    ("dense_drops_newest_key", "every = k_bits[b, kv_head, :length]",
     "every = k_bits[b, kv_head, :length - 1]"),
    ("dense_gqa_interleaved", "kv_head = h * hkv // hq", "kv_head = h % hkv"),
    ("dense_reads_past_length", "bf16_to_f64(v_bits[b, kv_head, :length]), d)",
     "bf16_to_f64(v_bits[b, kv_head, 1:length + 1]), d)"),
    ("snapshot_newest_first", "for i, (qb, s) in enumerate(entries):",
     "for i, (qb, s) in enumerate(reversed(entries)):"),
    ("snapshot_ignores_support_len", "supp[b, h, i, : supp_len[b, h, i]]", "supp[b, h, i, :]"),
    ("snapshot_drops_last_entry", "for i in range(n)]", "for i in range(max(n - 1, 0))]"),
    ("candidates_keep_invisible_keys", "for i in supports[c] if int(i) < length)", "for i in supports[c])"),
    ("empty_support_not_zero", "if len(scores) == 0:\n        return np.zeros(head_dim)",
     "if len(scores) == 0:\n        return np.full(head_dim, np.nan)"),
    ("recent_r_oldest_first", "chosen = [n - 1 - i for i in range(min(r, n))]",
     "chosen = [i for i in range(min(r, n))]"),
    ("recent_r_rho_over_all", "rho_max = max(rho[c] for c in chosen) if chosen else -math.inf",
     "rho_max = max(rho) if chosen else -math.inf"),
    ("recent_r_ignored", "if self.retrieval == \"similarity\":", "if True:"),
    ("recall_uses_raw_query", "rho = cosine_recall(qbar, [e[0] for e in entries])",
     "rho = cosine_recall(bf16_to_f64(q_bits[b, h]), [e[0] for e in entries])"),
]


def _mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation target not found: {old!r}"
    name = "retopk_oracle_mutant"
    mod = types.ModuleType(name)
    mod.__file__ = SRC
    sys.modules[name] = mod          # dataclasses look their module up here
    try:
        exec(compile(text.replace(old, new), SRC, "exec"), mod.__dict__)
    finally:
        sys.modules.pop(name, None)
    return mod


def _caught(mod):
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert _caught(_mutant(old, new)) is not None, f"no pin catches mutation {name}"
