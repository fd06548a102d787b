"""The C-ABI library loads and exports every symbol include/retopk.h declares;
argument checks fail cleanly with status codes (no GPU needed, no compute)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retopk.h")


def _lib():
    from sparse_long_context_head_amd import binding
    return binding, binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(retopk_[a-z_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for required in ("retopk_init_from_prefill", "retopk_decode_step", "retopk_exact_topk_attn",
                     "retopk_create", "retopk_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    _, lib = _lib()
    raw = ctypes.CDLL(os.path.join(ROOT, "sparse_long_context_head_amd", "libretopk.so"))
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in retopk.h but not exported"


def test_binding_covers_every_symbol():
    binding, _ = _lib()
    for name in declared_functions():
        assert name in binding._SIGNATURES, f"{name} has no binding signature"


def test_status_strings_and_kernel_names():
    binding, lib = _lib()
    assert lib.retopk_status_string(0) == b"ok"
    assert lib.retopk_status_string(2) == b"argument out of range"
    names = binding.retopk_kernel_names()
    assert {"k_step", "k_dense", "k_dense_merge"} <= set(names)
    assert len(names) == lib.retopk_kernel_count()


GOOD = dict(batch=1, n_q_heads=28, n_kv_heads=4, head_dim=128, max_len=1000, top_k=512,
            cache_cap=32, window=32, top_r=4, refresh_every=128, tau=0.85)


@pytest.mark.parametrize("change,status", [
    (dict(n_kv_heads=5), 1), (dict(head_dim=64), 1), (dict(batch=0), 1),
    (dict(n_q_heads=34, n_kv_heads=2), 1), (dict(max_len=0), 2), (dict(top_k=0), 2),
    (dict(top_k=9000), 2), (dict(cache_cap=0), 2), (dict(cache_cap=65), 2),
    (dict(top_r=33), 2), (dict(window=-1), 2), (dict(refresh_every=-1), 2),
    (dict(top_k=4096, window=100), 2), (dict(tau=float("nan")), 1),
])
def test_create_rejects_bad_params(change, status):
    binding, _ = _lib()
    with pytest.raises(binding.RetopkError) as e:
        binding.retopk_create(**{**GOOD, **change})
    assert e.value.status == status


def test_create_rejects_unknown_retrieval():
    import ctypes
    binding, lib = _lib()
    p = binding.RetopkParams(**{k: v for k, v in GOOD.items()}, retrieval=2)
    out = ctypes.c_void_p()
    assert lib.retopk_create(ctypes.byref(p), ctypes.byref(out)) == 1 and out.value is None
    assert b"retrieval" in lib.retopk_last_error()


def test_create_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    binding, _ = _lib()
    with pytest.raises(binding.RetopkError) as e:
        binding.retopk_create(**GOOD)
    assert e.value.status == 5


def test_null_handle_calls_fail_cleanly():
    _, lib = _lib()
    assert lib.retopk_decode_step(None, None, None, None, 10, 1, None, None) == 4
    assert lib.retopk_exact_topk_attn(None, None, None, None, 10, None, None, None) == 4
    assert lib.retopk_dense_attn(None, None, None, None, 10, None, None) == 4
    assert lib.retopk_init_from_prefill(None, None, None, 10, None) == 4
    assert lib.retopk_read_state(None, None, None, None, None) == 4
    assert lib.retopk_set_timing(None, 1) == 4
    assert b"NULL handle" in lib.retopk_last_error()
    # the streaming-read probe checks its arguments before touching a device
    assert lib.retopk_stream_read(None, 16, None, None) == 1
    assert b"NULL pointer" in lib.retopk_last_error()
    assert lib.retopk_score_probe(1, None, 16, None, None, None) == 1
    assert b"NULL pointer" in lib.retopk_last_error()
    lib.retopk_destroy(None)
    out = ctypes.c_void_p()
    assert lib.retopk_create(None, ctypes.byref(out)) == 1 and out.value is None


def test_header_compiles_as_c_and_cxx():
    import shutil
    import subprocess
    for cc, lang in (("gcc", "c"), ("g++", "c++")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Wextra", "-Werror", "-x", lang, HEADER],
                           capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, r.stderr
