"""The seeded input generator: determinism, shapes and the stated recipe."""
import numpy as np

from sparse_long_context_head_amd.workload import WORKLOADS, f32_to_bf16_bits, generate


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    assert list(f32_to_bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]


def test_generate_shapes_and_determinism():
    wl = WORKLOADS["gqa16k"].replace(prompt_len=2048, decode_steps=8)
    a = generate(wl)
    b = generate(wl)
    assert a["k"].shape == (1, 4, 2056, 128) and a["k"].dtype == np.uint16
    assert a["q_tail"].shape == (1, 28, 32, 128)
    assert a["q_dec"].shape == (8, 1, 28, 128)
    for key in a:
        assert np.array_equal(a[key], b[key])
    c = generate(wl, seed_base=7)
    assert not np.array_equal(a["k"], c["k"])


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_heavy_rows_and_query_correlation():
    wl = WORKLOADS["gqa16k"].replace(prompt_len=4096, decode_steps=64)
    d = generate(wl)
    norms = np.linalg.norm(_f(d["k"][0]), axis=-1)            # [Hkv, L]
    for g in range(4):
        heavy = norms[g, :4096] > 2 * np.median(norms[g])
        assert heavy.sum() == 64                                # 64 rows scaled by 3
        assert not (norms[g, 4096:] > 2 * np.median(norms[g])).any()
    q = _f(d["q_dec"][:, 0])                                     # [T, Hq, D]
    corr = np.mean(np.sum(q[1:] * q[:-1], -1) / (np.linalg.norm(q[1:], axis=-1) *
                                                 np.linalg.norm(q[:-1], axis=-1)))
    assert 0.85 < corr < 0.95                                   # AR(1) with rho = 0.9
