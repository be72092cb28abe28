"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and validates configurations without touching a GPU."""
import ctypes as C
import os
import re

import pytest

import q3synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from decoder_only_qwen3_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libq3.so not built")
    return _lib, _lib.load()


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(q3\w*)\s*\(", text, re.M))
    return names


def test_every_declared_symbol_is_exported():
    mod, lib = _lib()
    decl = declared_functions()
    assert "q3_prefill" in decl and "q3_decode_step" in decl and "q3_load_weights" in decl
    for name in sorted(decl):
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(mod.EXPORTS) <= decl


def _cfg(mod, **kw):
    d = q3synth.ModelDims()
    base = dict(n_layers=d.n_layers, hidden=d.hidden, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                head_dim=d.head_dim, ffn=d.ffn, vocab=d.vocab, rms_eps=d.rms_eps,
                rope_theta=d.rope_theta, dtype=mod.Q3_BF16, max_slots=4, max_positions=1024,
                max_prefill_tokens=1024, kv_tokens=4096)
    base.update(kw)
    return mod.q3_config(**base)


def test_weight_bytes_match_the_parameter_count():
    mod, lib = _lib()
    cfg = _cfg(mod)
    wb = lib.q3_weights_bytes(C.byref(cfg))
    # 596,049,920 parameters in bf16 (tied head), norms stored float32, plus
    # the RoPE table and 256-byte alignment of each tensor.
    proj = 28 * 15_728_640 * 2 + 155_582_464 * 2
    norms = (28 * 2304 + 1024) * 4
    rope = 2 * 1024 * 64 * 4
    assert proj + norms + rope <= wb <= proj + norms + rope + 256 * (28 * 8 + 4)
    kvb = lib.q3_kv_bytes(C.byref(cfg))
    assert kvb == 4096 * 114_688  # 28 layers x 2 x 8 heads x 128 x 2 bytes per token


@pytest.mark.parametrize("bad", [dict(head_dim=64), dict(n_kv_heads=3), dict(hidden=1000),
                                 dict(vocab=151937), dict(dtype=7), dict(max_slots=0),
                                 dict(dtype=0, max_positions=9000), dict(n_q_heads=16, n_kv_heads=1)])
def test_create_rejects_unsupported_configs(bad):
    mod, lib = _lib()
    cfg = _cfg(mod, **bad)
    h = C.c_void_p()
    st = lib.q3_create(C.byref(cfg), C.byref(h))
    assert st == mod.Q3_E_UNSUPPORTED
    assert lib.q3_last_error()
    assert lib.q3_weights_bytes(C.byref(cfg)) == 0


def test_create_and_destroy_without_gpu_and_state_errors():
    mod, lib = _lib()
    cfg = _cfg(mod)
    h = C.c_void_p()
    assert lib.q3_create(C.byref(cfg), C.byref(h)) == mod.Q3_OK
    # every call that needs bound memory reports Q3_E_STATE before touching HIP
    slots = mod.i32_array([0])
    cu = mod.i32_array([0, 4])
    st = lib.q3_prefill(h, 1, slots, cu, C.c_void_p(16), None, C.c_void_p(16), 0, None)
    assert st == mod.Q3_E_STATE
    assert b"bind" in lib.q3_last_error()
    assert lib.q3_decode_step(h, 1, slots, C.c_void_p(16), None, C.c_void_p(16), None) == mod.Q3_E_STATE
    assert lib.q3_seq_alloc(h, 0, 16, None) == mod.Q3_E_STATE
    assert lib.q3_set_option(h, 99, 1) == mod.Q3_E_ARG
    n = C.c_int64(-1)
    assert lib.q3_seq_length(h, 0, C.byref(n)) == mod.Q3_OK and n.value == 0
    assert lib.q3_seq_length(h, 9, C.byref(n)) == mod.Q3_E_ARG
    lib.q3_destroy(h)


def test_check_tokens_on_the_host():
    """q3_check_tokens: every ID in [0, vocab), else Q3_E_ARG naming the first
    bad one (host only, no device)."""
    mod, lib = _lib()
    cfg = _cfg(mod)
    h = C.c_void_p()
    assert lib.q3_create(C.byref(cfg), C.byref(h)) == mod.Q3_OK
    V = cfg.vocab
    assert lib.q3_check_tokens(h, mod.i32_array([0, 1, V - 1]), 3) == mod.Q3_OK
    assert lib.q3_check_tokens(h, None, 0) == mod.Q3_OK
    assert lib.q3_check_tokens(h, mod.i32_array([5, V, 7]), 3) == mod.Q3_E_ARG
    assert b"token 1" in lib.q3_last_error() and str(V).encode() in lib.q3_last_error()
    assert lib.q3_check_tokens(h, mod.i32_array([-1]), 1) == mod.Q3_E_ARG
    assert lib.q3_check_tokens(h, None, 2) == mod.Q3_E_ARG
    lib.q3_destroy(h)


def test_bf16_key_layout_helper():
    """The tests' model of the bf16 key cache layout (include/q3_ops.h, arena
    description) is a bijection of each head's cap x 128 elements, and each
    32-key block holds, as 16-byte chunk (sbk*4 + ks)*64 + fq*16 + fr, dims
    ks*32 + fq*8 .. +7 of key 8*(fr//4) + 4*sbk + fr%4."""
    import numpy as np
    from gpu_helpers import k_blocks, k_logical, k_perm
    for cap in (64, 192):
        p = k_perm(cap)
        assert np.array_equal(np.sort(p.reshape(-1)), np.arange(cap * 128))
        for key in (0, 5, 31, 32, 63, cap - 1):
            for dim in (0, 7, 8, 33, 64, 127):
                t, k = key, key % 32
                sbk, fr = (k // 4) % 2, (k // 8) * 4 + k % 4
                want = (t // 32) * 4096 + (((sbk * 4 + dim // 32) * 4 + (dim // 8) % 4) * 16 + fr) * 8 + dim % 8
                assert p[key, dim] == want
    K = np.arange(2 * 64 * 128, dtype=np.float32).reshape(2, 64, 128)
    assert np.array_equal(k_logical(k_blocks(K), 2, 64), K)
