"""Pins for the CPU oracle: each check ties it to something other than itself.

The facts come from "Dentro de un LLM: Inferencia en Python puro para
Qwen3-0.6B en MLX" (Pasos 3-9) and from mathematics: closed forms, invariants,
special cases that reduce to a textbook routine, library conversions, and brute
force against an independent scalar implementation (tests/scalar_model.py).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import q3synth
from oracle import (OracleModel, attention_rows, dequantize_affine, greedy_pick, quantize_affine,
                    quantized_weights, rms_norm, rope_cos_sin, rope_rotate, sample_top_p, silu, swiglu,
                    to_bf16)
from scalar_model import scalar_forward_all

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- bf16 rounding
def test_to_bf16_matches_torch_conversion():
    x = np.concatenate([RNG.standard_normal(20000) * 10.0 ** RNG.integers(-8, 8, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e38, 1e-40]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(to_bf16(x), ref)


def test_to_bf16_ties_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7: even wins (1).
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    np.testing.assert_array_equal(to_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])),
                                  [1.0, 1 + 2.0 ** -6])


def test_generator_rounding_matches_torch():
    x = RNG.standard_normal(5000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(q3synth.round_to_bf16(x), ref)


# ---------------------------------------------------------------- Paso 3: RMSNorm
def test_rmsnorm_unit_rms_closed_form():
    x = RNG.standard_normal((7, 1024)) * RNG.uniform(0.001, 30, (7, 1))
    y = rms_norm(x, np.ones(1024), 1e-6)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-6), rtol=1e-12)


def test_rmsnorm_constant_vector_and_weight():
    c = 0.37
    y = rms_norm(np.full((1, 8), c), np.ones(8), 1e-6)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    w = RNG.standard_normal(8)
    x = RNG.standard_normal((3, 8))
    np.testing.assert_allclose(rms_norm(x, w, 1e-6), rms_norm(x, np.ones(8), 1e-6) * w, rtol=1e-14)


def test_rmsnorm_no_mean_subtraction():
    # a shifted vector is NOT re-centred: rmsnorm(1 + small) stays near all-ones
    x = 1.0 + 1e-3 * RNG.standard_normal((1, 64))
    assert np.all(rms_norm(x, np.ones(64), 1e-6) > 0.99)


# ---------------------------------------------------------------- Paso 4: RoPE
def _rot(u, p, D=128, theta=1e6):
    c, s = rope_cos_sin([p], D, theta)
    return rope_rotate(u[None, None, :], c, s)[0, 0]


def test_rope_pair0_turns_one_radian_per_position_into_second_half():
    e0 = np.zeros(128); e0[0] = 1.0
    r = _rot(e0, 1)
    expect = np.zeros(128); expect[0] = math.cos(1.0); expect[64] = math.sin(1.0)
    np.testing.assert_allclose(r, expect, atol=1e-15)
    e64 = np.zeros(128); e64[64] = 1.0
    r = _rot(e64, 1)
    expect = np.zeros(128); expect[0] = -math.sin(1.0); expect[64] = math.cos(1.0)
    np.testing.assert_allclose(r, expect, atol=1e-15)


def test_rope_frequency_uses_theta_1e6():
    # pair 32 of 64 has frequency theta^(-1/2) = 1e-3: position 1000 turns it by 1 rad
    e = np.zeros(128); e[32] = 1.0
    r = _rot(e, 1000)
    assert abs(r[32] - math.cos(1.0)) < 1e-12 and abs(r[96] - math.sin(1.0)) < 1e-12
    # pair 48 has frequency 1e6^(-3/4) = 10^-4.5
    e = np.zeros(128); e[48] = 1.0
    r = _rot(e, 31623)
    ang = 31623 * 10 ** -4.5
    assert abs(r[48] - math.cos(ang)) < 1e-12 and abs(r[112] - math.sin(ang)) < 1e-12


def test_rope_identity_norm_and_composition():
    u = RNG.standard_normal(128)
    np.testing.assert_allclose(_rot(u, 0), u, atol=0)
    for p in (1, 17, 32767):
        r = _rot(u, p)
        # each (i, i+64) pair keeps its length
        np.testing.assert_allclose(r[:64] ** 2 + r[64:] ** 2, u[:64] ** 2 + u[64:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(_rot(_rot(u, 5), 1234), _rot(u, 1239), atol=1e-12)


def test_rope_dot_depends_only_on_relative_position():
    q, k = RNG.standard_normal(128), RNG.standard_normal(128)
    base = _rot(q, 10) @ _rot(k, 3)
    for s in (1, 100, 20000):
        assert abs(_rot(q, 10 + s) @ _rot(k, 3 + s) - base) < 1e-10


# ---------------------------------------------------------------- Paso 5: attention
def _rand_qkv(T, n_q, n_kv, D):
    return (RNG.standard_normal((T, n_q, D)), RNG.standard_normal((T, n_kv, D)),
            RNG.standard_normal((T, n_kv, D)))


def test_attention_first_position_returns_its_value():
    q, k, v = _rand_qkv(5, 4, 2, 8)
    pos = np.arange(5)
    o = attention_rows(q, k, v, pos, pos)
    np.testing.assert_array_equal(o[0, 0], v[0, 0])
    np.testing.assert_array_equal(o[0, 3], v[0, 1])


def test_attention_zero_query_is_prefix_mean():
    _, k, v = _rand_qkv(9, 4, 2, 8)
    q = np.zeros((9, 4, 8))
    pos = np.arange(9)
    o = attention_rows(q, k, v, pos, pos)
    for t in range(9):
        for h in range(4):
            np.testing.assert_allclose(o[t, h], v[:t + 1, h // 2].mean(axis=0), rtol=1e-13)


def test_attention_two_keys_closed_form_scale():
    D = 128
    q, k, v = _rand_qkv(2, 1, 1, D)
    o = attention_rows(q, k, v, np.array([0, 1]), np.array([0, 1]))
    ds = (q[1, 0] @ k[1, 0] - q[1, 0] @ k[0, 0]) / math.sqrt(D)
    sig = 1.0 / (1.0 + math.exp(-ds))
    np.testing.assert_allclose(o[1, 0], v[0, 0] + (v[1, 0] - v[0, 0]) * sig, rtol=1e-12)


def test_gqa_head_map_is_floor_division():
    T, D = 4, 8
    q = RNG.standard_normal((T, 16, D))
    k = RNG.standard_normal((T, 8, D))
    v = np.zeros((T, 8, D))
    for g in range(8):
        v[:, g, :] = g + 1.0          # every value of kv head g equals g + 1
    o = attention_rows(q, k, v, np.arange(T), np.arange(T))
    for h in range(16):
        np.testing.assert_allclose(o[:, h, :], h // 2 + 1.0, rtol=1e-14)


@pytest.mark.parametrize("n_q,n_kv", [(16, 8), (16, 1), (4, 2)])
def test_gqa_equals_mha_with_repeated_heads(n_q, n_kv):
    q, k, v = _rand_qkv(6, n_q, n_kv, 16)
    pos = np.arange(6)
    grouped = attention_rows(q, k, v, pos, pos)
    rep = n_q // n_kv
    mha = attention_rows(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), pos, pos)
    np.testing.assert_allclose(grouped, mha, rtol=1e-13, atol=1e-15)


def test_causal_future_does_not_leak():
    q, k, v = _rand_qkv(8, 4, 2, 8)
    pos = np.arange(8)
    o1 = attention_rows(q, k, v, pos, pos)
    k2, v2 = k.copy(), v.copy()
    k2[5:] = RNG.standard_normal(k2[5:].shape)
    v2[5:] = RNG.standard_normal(v2[5:].shape)
    o2 = attention_rows(q, k2, v2, pos, pos)
    np.testing.assert_array_equal(o1[:5], o2[:5])
    assert not np.allclose(o1[5:], o2[5:])


def _scalar_attention(q, k, v):
    T, n_q, D = q.shape
    g = n_q // k.shape[1]
    out = np.zeros_like(q)
    for t in range(T):
        for h in range(n_q):
            sc = [sum(q[t, h, i] * k[j, h // g, i] for i in range(D)) / math.sqrt(D) + (-1e9 if j > t else 0.0)
                  for j in range(T)]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            for i in range(D):
                out[t, h, i] = sum(e[j] / z * v[j, h // g, i] for j in range(T))
    return out


def test_attention_matches_scalar_masked_softmax():
    q, k, v = _rand_qkv(7, 4, 2, 8)
    pos = np.arange(7)
    np.testing.assert_allclose(attention_rows(q, k, v, pos, pos, block=3),
                               _scalar_attention(q, k, v), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- Paso 6: SwiGLU
def test_silu_special_values():
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(np.array([1.0])), [1.0 / (1.0 + math.exp(-1.0))], rtol=1e-15)
    np.testing.assert_allclose(silu(np.array([40.0])), [40.0], rtol=1e-15)
    assert abs(silu(np.array([-40.0]))[0]) < 1e-15
    assert silu(np.array([-800.0]))[0] == 0.0   # exp overflow -> exact 0, not NaN


def test_swiglu_identity_weights():
    h = RNG.standard_normal((3, 6))
    I6 = np.eye(6)
    np.testing.assert_allclose(swiglu(h, I6, I6, I6), h * h / (1 + np.exp(-h)), rtol=1e-14)
    # gate and up are not interchangeable
    wg, wu = 2 * I6, I6
    np.testing.assert_allclose(swiglu(h, wg, wu, I6), silu(2 * h) * h, rtol=1e-14)


# ---------------------------------------------------------------- Paso 8: greedy
def test_greedy_lowest_index_on_tie_and_rejects_nan():
    assert greedy_pick(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    with pytest.raises(FloatingPointError):
        greedy_pick(np.array([1.0, np.nan]))


# ---------------------------------------------------------------- Paso 8: top-p sampling
def test_top_p_worked_examples():
    path = os.path.join(os.path.dirname(__file__), "golden", "top_p_worked_examples.json")
    for case in json.load(open(path))["cases"]:
        scale = case["temperature"] if case["temperature"] > 0 else 1.0
        logits = scale * np.log(np.array(case["probs"]))
        for u, tok in case["draws"]:
            got = sample_top_p(logits, case["temperature"], case["top_p"], u)
            assert got == tok, (case["work"], u, got, tok)


def _nucleus_by_subsets(probs, top_p):
    """The page's comment read as a set: the smallest set of tokens whose total
    probability reaches top_p (among sets of that size, the heaviest), found by
    enumerating every subset of a tiny vocabulary."""
    V = len(probs)
    best = None
    for mask in range(1, 1 << V):
        ids = [i for i in range(V) if mask >> i & 1]
        mass = sum(probs[i] for i in ids)
        if mass >= top_p or mask == (1 << V) - 1:
            key = (len(ids), -mass)
            if best is None or key < best[0]:
                best = (key, ids)
    return best[1]


@pytest.mark.parametrize("seed", range(6))
def test_top_p_nucleus_is_smallest_heaviest_set_and_draw_frequencies(seed):
    rng = np.random.default_rng(seed)
    V = 7
    logits = rng.standard_normal(V) * 2.0
    T = [0.5, 1.0, 1.7][seed % 3]
    e = np.exp(logits / T - np.max(logits / T))
    probs = e / e.sum()
    for top_p in (0.3, 0.6, 0.9, 0.99):
        nucleus = _nucleus_by_subsets(list(probs), top_p)
        # inverse transform on a fine regular grid of u: each kept token is
        # drawn in proportion to its renormalised probability, the rest never
        N = 4000
        counts = np.zeros(V)
        for k in range(N):
            counts[sample_top_p(logits, T, top_p, (k + 0.5) / N)] += 1
        want = np.zeros(V)
        want[nucleus] = probs[nucleus] / probs[nucleus].sum()
        np.testing.assert_allclose(counts / N, want, atol=1.5 / N)


def test_top_p_shift_and_temperature_invariance():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal(300) * 3
    for u in rng.random(40):
        a = sample_top_p(logits, 0.8, 0.9, u)
        assert a == sample_top_p(logits + 123.0, 0.8, 0.9, u)
        assert a == sample_top_p(logits / 0.8, 1.0, 0.9, u)


def test_top_p_rejects_nonfinite_and_bad_u():
    with pytest.raises(FloatingPointError):
        sample_top_p(np.array([0.0, np.nan]), 1.0, 0.9, 0.5)
    with pytest.raises(ValueError):
        sample_top_p(np.array([0.0, 1.0]), 1.0, 0.9, 1.0)


# ---------------------------------------------------------------- weight-only quantization
@pytest.mark.parametrize("bits", [8, 4])
def test_quantizer_reproduces_values_on_its_grid(bits):
    # rows built as b0 + q * s0 with float16 s0, b0 and both end codes present:
    # the quantizer must return exactly those codes, scale and offset
    rng = np.random.default_rng(bits)
    levels = 2 ** bits - 1
    s0 = np.float16(2.0 ** -10)
    b0 = np.float16(-0.125)
    q0 = rng.integers(0, levels + 1, size=(3, 128))
    q0[:, 0::64] = 0
    q0[:, 1::64] = levels
    w = (q0 * np.float64(s0) + np.float64(b0)).astype(np.float32)
    q, s, b = quantize_affine(w, bits)
    np.testing.assert_array_equal(q, q0)
    assert np.all(s == s0) and np.all(b == b0)
    np.testing.assert_array_equal(dequantize_affine(q, s, b), w.astype(np.float64))


@pytest.mark.parametrize("bits", [8, 4])
def test_quantizer_error_within_half_a_step(bits):
    rng = np.random.default_rng(10 + bits)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    q, s, b = quantize_affine(w, bits)
    assert q.max() <= 2 ** bits - 1
    err = np.abs(dequantize_affine(q, s, b) - w).reshape(16, 8, 64).max(axis=2)
    g = w.reshape(16, 8, 64)
    # half a step, plus what the float16 rounding of offset and scale moves
    bound = 0.5 * s.astype(np.float64) + 2.0 ** -11 * (np.abs(g.min(axis=2)) + np.abs(g.max(axis=2))) * 1.01
    assert np.all(err <= bound), float(np.max(err - bound))


def test_quantizer_constant_group_and_row_independence():
    w = np.full((2, 64), 0.3, np.float32)
    w[1] = np.linspace(-1, 1, 64)
    q, s, b = quantize_affine(w, 8)
    assert np.all(q[0] == 0) and s[0, 0] == 0 and b[0, 0] == np.float16(0.3)
    q1, _, _ = quantize_affine(w[1:], 8)
    np.testing.assert_array_equal(q[1:], q1)


def test_quantized_storage_matches_the_page():
    # bits/8 + 4/64 bytes per parameter at group 64 with float16 scale and
    # offset: 1.0625 (8-bit) and 0.5625 (4-bit), as the page states
    N, K = 32, 1024
    for bits, per in ((8, 1.0625), (4, 0.5625)):
        q, s, b = quantize_affine(np.zeros((N, K), np.float32), bits)
        nbytes = q.size * bits / 8 + s.nbytes + b.nbytes
        assert nbytes / (N * K) == per


def test_quantized_weights_touch_only_block_projections():
    d = q3synth.tiny_dims(dtype="bf16", hidden=64, n_q_heads=2, n_kv_heads=1, head_dim=32, ffn=128)
    w = {k: q3synth.round_to_bf16(v) for k, v in q3synth.make_weights(d, seed=7).items()}
    qw = quantized_weights(w, 8)
    for name, a in w.items():
        if name.endswith("_proj.weight"):
            assert not np.array_equal(qw[name], a)
            np.testing.assert_allclose(qw[name], a, atol=float(np.ptp(a)) / 255)  # within one step
        else:
            assert qw[name] is a


# ---------------------------------------------------------------- whole model
def _tiny_model(**kw):
    d = q3synth.tiny_dims(**kw)
    w = q3synth.make_weights(d, seed=7)
    return d, w


@pytest.mark.parametrize("kw", [{}, {"n_kv_heads": 1}, {"n_kv_heads": 4}, {"n_layers": 1}])
def test_model_matches_scalar_brute_force(kw):
    d, w = _tiny_model(**kw)
    ids = [3, 96, 0, 41, 41, 7]
    m = OracleModel(d, w)
    got = m.forward(ids, m.new_cache(len(ids)), logit_rows=range(len(ids)))
    ref = np.array(scalar_forward_all(d, w, ids))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_untied_head_matches_brute_force_and_reduces_to_tied():
    d, w = _tiny_model()
    ids = [3, 96, 0, 41]
    tied = OracleModel(d, w).forward(ids, OracleModel(d, w).new_cache(4), logit_rows=range(4))
    same = dict(w, **{"lm_head.weight": w["model.embed_tokens.weight"].copy()})
    m = OracleModel(d, same)
    np.testing.assert_array_equal(m.forward(ids, m.new_cache(4), logit_rows=range(4)), tied)
    rng = np.random.default_rng(8)
    untied = dict(w, **{"lm_head.weight": (rng.standard_normal(w["model.embed_tokens.weight"].shape) * 0.05)
                        .astype(np.float32)})
    m = OracleModel(d, untied)
    got = m.forward(ids, m.new_cache(4), logit_rows=range(4))
    np.testing.assert_allclose(got, np.array(scalar_forward_all(d, untied, ids)), rtol=1e-11, atol=1e-13)
    assert not np.allclose(got, tied)


def test_zero_layer_model_is_norm_then_embedding_product():
    d, w = _tiny_model(n_layers=0)
    E = w["model.embed_tokens.weight"].astype(np.float64)
    wf = w["model.norm.weight"].astype(np.float64)
    m = OracleModel(d, w)
    got = m.forward([5], m.new_cache(1))[0]
    x = E[5]
    h = x / math.sqrt(float(np.dot(x, x)) / x.size + d.rms_eps) * wf
    ref = np.array([float(np.dot(E[j], h)) for j in range(d.vocab)])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("contract", [False, True])
def test_kv_cache_decode_equals_full_recompute(contract):
    d, w = _tiny_model(dtype="bf16" if contract else "f32")
    if contract:
        w = {k: q3synth.round_to_bf16(v) for k, v in w.items()}
    m = OracleModel(d, w, contract=contract)
    ids = [10, 20, 30, 40, 50, 60, 70]
    cache = m.new_cache(len(ids))
    m.forward(ids[:3], cache)
    for n in range(3, len(ids)):
        step = m.forward([ids[n]], cache)[0]
        full = m.forward(ids[:n + 1], m.new_cache(n + 1))[0]
        np.testing.assert_allclose(step, full, rtol=1e-12, atol=1e-14)
    forced = m.forced_logits(ids[:3], ids[3:])
    cache = m.new_cache(len(ids))
    first = m.forward(ids[:3], cache)[0]
    np.testing.assert_allclose(forced[0], first, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("contract", [False, True])
def test_chunked_prefill_equals_single_prefill(contract):
    """A prompt fed in chunks (each chunk at the positions after the cached
    ones, attending to them) gives the rows of one call over the whole prompt,
    and those rows match the scalar brute force on the concatenation."""
    d, w = _tiny_model(dtype="bf16" if contract else "f32")
    if contract:
        w = {k: q3synth.round_to_bf16(v) for k, v in w.items()}
    m = OracleModel(d, w, contract=contract)
    ids = [10, 20, 30, 40, 50, 60, 70, 80, 90, 5, 6]
    whole = m.forward(ids, m.new_cache(len(ids)), logit_rows=range(len(ids)))
    cache = m.new_cache(len(ids))
    parts = []
    for a, b in [(0, 4), (4, 5), (5, 9), (9, 11)]:
        parts.append(m.forward(ids[a:b], cache, logit_rows=range(b - a)))
        assert cache.length == b
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=1e-12, atol=1e-14)
    if not contract:
        ref = np.array(scalar_forward_all(d, w, ids))
        np.testing.assert_allclose(np.concatenate(parts), ref, rtol=1e-11, atol=1e-13)


def test_prefix_logits_unchanged_by_later_tokens():
    d, w = _tiny_model()
    m = OracleModel(d, w)
    a = m.forward([1, 2, 3, 4], m.new_cache(4), logit_rows=range(4))
    b = m.forward([1, 2, 3, 90], m.new_cache(4), logit_rows=range(4))
    np.testing.assert_allclose(a[:3], b[:3], rtol=1e-13, atol=1e-15)
    assert not np.allclose(a[3], b[3])


def test_greedy_loop_feeds_back_argmax():
    d, w = _tiny_model()
    m = OracleModel(d, w)
    toks, logits = m.generate_greedy([4, 5, 6], 5)
    assert len(toks) == 6 and logits.shape == (6, d.vocab)
    np.testing.assert_array_equal(toks, np.argmax(logits, axis=1))
    forced = m.forced_logits([4, 5, 6], toks[:-1])
    np.testing.assert_allclose(forced, logits, rtol=1e-12, atol=1e-14)


def test_contract_rounds_cache_to_bf16():
    d, w = _tiny_model(dtype="bf16")
    w = {k: q3synth.round_to_bf16(v) for k, v in w.items()}
    m = OracleModel(d, w)
    assert m.contract
    cache = m.new_cache(4)
    m.forward([1, 2, 3, 4], cache)
    for layer in range(d.n_layers):
        np.testing.assert_array_equal(cache.k[layer], to_bf16(cache.k[layer]))
        np.testing.assert_array_equal(cache.v[layer], to_bf16(cache.v[layer]))


def test_capacity_overflow_raises():
    d, w = _tiny_model()
    m = OracleModel(d, w)
    with pytest.raises(ValueError):
        m.forward([1, 2, 3], m.new_cache(2))


def test_page_prompt_ids_are_valid_tokens():
    path = os.path.join(os.path.dirname(__file__), "golden", "capital_of_france_ids.json")
    ids = json.load(open(path))["ids"]
    assert ids == [785, 6722, 315, 9625, 374]
    assert all(0 <= t < q3synth.ModelDims().vocab for t in ids)


def test_last_layer_row_pruning_matches_full_rows():
    # Returning logits for a subset of rows skips work in the last block only;
    # the kept rows must equal the same rows of the all-rows computation.
    for n_layers in (1, 2):
        d, w = _tiny_model(n_layers=n_layers)
        m = OracleModel(d, w)
        ids = [5, 17, 3, 3, 88, 41, 0]
        full = m.forward(ids, m.new_cache(7), logit_rows=range(7))
        part = m.forward(ids, m.new_cache(7), logit_rows=[1, 6])
        np.testing.assert_allclose(part, full[[1, 6]], rtol=1e-13, atol=1e-15)
        # and the cache filled by a pruned call supports exact decode afterwards
        c1, c2 = m.new_cache(8), m.new_cache(8)
        m.forward(ids, c1, logit_rows=range(7))
        m.forward(ids, c2)
        np.testing.assert_allclose(m.forward([9], c1), m.forward([9], c2), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- bf16 contract mode
def test_scalar_bf16_rounder_matches_torch_conversion():
    """The scalar model's bf16 rounding (integer bits) against torch's
    float32 -> bfloat16 conversion, ties and carries included."""
    from scalar_model import Bf16Rounder
    r = Bf16Rounder()
    vals = list(RNG.standard_normal(2000) * 10.0 ** RNG.integers(-6, 6, 2000))
    # exact float32 midpoints between neighbouring bf16 values, odd and even lower neighbours
    for hi in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x4049, 0x7F7E):
        vals.append(float(np.array([(hi << 16) | 0x8000], np.uint32).view(np.float32)[0]))
    vals.append(float(np.array([0x3F80FFFF], np.uint32).view(np.float32)[0]))   # carry into the exponent field
    got = np.array([r(v) for v in vals])
    ref = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("kw,seed,mlp_scale", [({}, 7, 1.0), ({"n_kv_heads": 1}, 8, 1.0),
                                                ({"n_layers": 1, "n_kv_heads": 4}, 9, 1.0), ({}, 7, 8.0)])
def test_contract_mode_matches_scalar_bf16_brute_force(kw, seed, mlp_scale):
    """The oracle's contract mode (bf16 weights and cache, activations rounded
    at the bf16 model's points) against the scalar model's own bf16 mode: same
    rounding points, different code.  Every rounded value of the scalar run
    sits far from a rounding decision point (checked), so the small
    differences of summation order between the two cannot flip a rounding, and
    the logits agree to float64 precision.  Dropping any one rounding point
    fails at least one case: with mlp_scale = 8 (gate, up and down weights
    times 8, still bf16 values) the MLP output dominates the residual, so the
    rounding of the SwiGLU product is not absorbed by the roundings after it."""
    from scalar_model import Bf16Rounder
    d = q3synth.tiny_dims(dtype="bf16", **kw)
    w = q3synth.make_weights(d, seed=seed)
    if mlp_scale != 1.0:
        w = {k: (v * np.float32(mlp_scale) if ".mlp." in k else v) for k, v in w.items()}
    ids = [3, 96, 0, 41, 41, 7]
    m = OracleModel(d, w)
    assert m.contract
    got = m.forward(ids, m.new_cache(len(ids)), logit_rows=range(len(ids)))
    r = Bf16Rounder()
    ref = np.array(scalar_forward_all(d, w, ids, rounder=r))
    assert r.closest > 1e-10, f"a rounded value sits {r.closest:.1e} (relative) from a rounding decision point"
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # and the rounding is not a no-op at this shape: the unrounded model differs
    plain = np.array(scalar_forward_all(d, w, ids))
    assert np.max(np.abs(plain - ref)) > 1e-5
