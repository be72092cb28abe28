"""End-to-end parity of the HIP path (through the C ABI) against the CPU oracle.

Bars (from the numerics contract): float32 model -> max|dlogit| <= 1e-3 * RMS;
bf16 model -> <= 3e-2 * RMS; greedy tokens identical unless the oracle's top
two logits are within that bound (a near-tie, reported and counted).
"""
import json
import os

import numpy as np
import pytest
import torch

import q3synth
from gpu_helpers import margin_ok, rel_err, weights_for
from oracle import OracleModel

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-3
TOL_BF16 = 3e-2


def _model(dims, **cap):
    from decoder_only_qwen3_amd import Q3Model
    return Q3Model(dims, **cap)


def _greedy_gpu(m, slot, prompt, steps):
    """Prefill then `steps` decode steps feeding the device-side next token."""
    dev = m.device
    V = m.dims.vocab
    logits, nxt = m.prefill([slot], [prompt])
    with torch.cuda.stream(m.stream):   # every read of a result is queued behind the call
        toks = [torch.empty(1, dtype=torch.int32, device=dev) for _ in range(2)]
        lg = [torch.empty((1, V), dtype=torch.float32, device=dev) for _ in range(2)]
        toks[0].copy_(nxt)
        out_logits = [logits[0].clone()]
        out_tokens = [nxt.clone()]
    for i in range(steps):
        a, b = toks[i % 2], toks[(i + 1) % 2]
        m.decode_raw([slot], a, lg[i % 2], b)
        with torch.cuda.stream(m.stream):
            out_logits.append(lg[i % 2][0].clone())
            out_tokens.append(b.clone())
    m.synchronize()
    return (np.stack([t.cpu().numpy() for t in out_logits]),
            np.array([int(t.item()) for t in out_tokens]))


def _forced_gpu(m, slot, prompt, forced):
    """Prefill then one decode step per forced token; logits after each."""
    dev = m.device
    V = m.dims.vocab
    logits, nxt = m.prefill([slot], [prompt])
    with torch.cuda.stream(m.stream):
        rows, nexts = [logits[0].clone()], [nxt.clone()]
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        lg = torch.empty((1, V), dtype=torch.float32, device=dev)
        nx = torch.empty(1, dtype=torch.int32, device=dev)
    for t in forced:
        with torch.cuda.stream(m.stream):
            tok.fill_(int(t))
        m.decode_raw([slot], tok, lg, nx)
        with torch.cuda.stream(m.stream):
            rows.append(lg[0].clone())
            nexts.append(nx.clone())
    m.synchronize()
    return np.stack([r.cpu().numpy() for r in rows]), np.array([int(n.item()) for n in nexts])


def test_f32_two_layer_greedy_matches_oracle():
    wl = q3synth.WORKLOADS["tiny2l_f32_p5_d16"]
    d = wl.dims
    w = weights_for(d, wl.seed)
    prompt = q3synth.make_tokens(wl.prompt_len, d.vocab, wl.seed + 1).tolist()
    steps = wl.decode_steps
    ref_tokens, ref_logits = OracleModel(d, w).generate_greedy(prompt, steps)
    m = _model(d, max_slots=2, max_positions=64, max_prefill_tokens=64, kv_tokens=128)
    m.load_weights(w)
    m.seq_alloc(0, len(prompt) + steps)
    g_logits, g_tokens = _greedy_gpu(m, 0, prompt, steps)
    assert m.error_flags() == 0
    for i in range(steps + 1):
        e = rel_err(g_logits[i], ref_logits[i])
        assert e <= TOL_F32, f"step {i}: logits error {e:.3e} > {TOL_F32}"
        rms = float(np.sqrt(np.mean(ref_logits[i] ** 2)))
        assert margin_ok(ref_logits[i], int(g_tokens[i]), TOL_F32 * rms), f"step {i}: token differs"
        if g_tokens[i] != ref_tokens[i]:
            break  # near-tie: the two runs continue from different tokens


def test_f32_page_prompt_ids():
    path = os.path.join(os.path.dirname(__file__), "golden", "capital_of_france_ids.json")
    ids = json.load(open(path))["ids"]
    d = q3synth.WORKLOADS["tiny2l_f32_p5_d16"].dims
    w = weights_for(d, 1000)
    ref = OracleModel(d, w).forward(ids, OracleModel(d, w).new_cache(5))[0]
    m = _model(d, max_slots=1, max_positions=64, max_prefill_tokens=64, kv_tokens=64)
    m.load_weights(w)
    m.seq_alloc(0, 8)
    logits, nxt = m.prefill([0], [ids])
    m.synchronize()
    assert rel_err(logits[0].cpu().numpy(), ref) <= TOL_F32
    assert int(nxt[0].item()) == int(np.argmax(ref))


@pytest.fixture(scope="module")
def bf16_two_layer():
    d = q3synth.QWEN3_06B.replace(n_layers=2)
    w = weights_for(d, 77)
    return d, w


def test_bf16_forced_decode_matches_oracle(bf16_two_layer):
    d, w = bf16_two_layer
    prompt = q3synth.make_tokens(100, d.vocab, 5).tolist()
    forced = q3synth.make_tokens(12, d.vocab, 6).tolist()
    ref = OracleModel(d, w).forced_logits(prompt, forced)
    m = _model(d, max_slots=2, max_positions=256, max_prefill_tokens=256, kv_tokens=512)
    m.load_weights(w)
    m.seq_alloc(1, 128)
    g, nx = _forced_gpu(m, 1, prompt, forced)
    assert m.error_flags() == 0
    errs = [rel_err(g[i], ref[i]) for i in range(len(ref))]
    print("bf16 forced rel errors:", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL_BF16
    for i in range(len(ref)):
        rms = float(np.sqrt(np.mean(ref[i] ** 2)))
        assert margin_ok(ref[i], int(nx[i]), TOL_BF16 * rms), f"step {i}"


def test_bf16_varlen_all_logits_matches_oracle(bf16_two_layer):
    d, w = bf16_two_layer
    lens = [1, 65, 130]
    prompts = [q3synth.make_tokens(L, d.vocab, 40 + i).tolist() for i, L in enumerate(lens)]
    m = _model(d, max_slots=4, max_positions=256, max_prefill_tokens=512, kv_tokens=1024)
    m.load_weights(w)
    for s, L in zip([2, 0, 3], lens):
        m.seq_alloc(s, L + 4)
    logits, nxt = m.prefill([2, 0, 3], prompts, all_logits=True)
    m.synchronize()
    g = logits.cpu().numpy()
    o = OracleModel(d, w)
    row = 0
    for i, p in enumerate(prompts):
        ref = o.forward(p, o.new_cache(len(p)), logit_rows=range(len(p)))
        for r in range(len(p)):
            e = rel_err(g[row + r], ref[r])
            assert e <= TOL_BF16, f"seq {i} row {r}: {e:.3e}"
        assert margin_ok(ref[-1], int(nxt[i].item()), TOL_BF16 * float(np.sqrt(np.mean(ref[-1] ** 2))))
        row += len(p)
    assert m.error_flags() == 0


# ---------------------------------------------------------------- chunked prefill
def _check_rows(got, ref, tol, what):
    for r in range(len(ref)):
        e = rel_err(got[r], ref[r])
        assert e <= tol, f"{what} row {r}: {e:.3e} > {tol}"


def test_bf16_chunked_prefill_matches_single_prefill_oracle(bf16_two_layer):
    """A 200-token prompt fed as four prefill calls into one slot (chunks that
    start on and off 64-token tiles), then forced decode steps: every row
    matches the oracle's one-call prefill of the whole prompt."""
    d, w = bf16_two_layer
    prompt = q3synth.make_tokens(200, d.vocab, 11).tolist()
    forced = q3synth.make_tokens(6, d.vocab, 12).tolist()
    o = OracleModel(d, w)
    ref = o.forward(prompt + forced, o.new_cache(206), logit_rows=range(206))
    m = _model(d, max_slots=2, max_positions=256, max_prefill_tokens=128, kv_tokens=512)
    m.load_weights(w)
    m.seq_alloc(1, 256)
    row = 0
    for a, b in [(0, 64), (64, 65), (65, 150), (150, 200)]:
        logits, nxt = m.prefill([1], [prompt[a:b]], all_logits=True)
        m.synchronize()
        assert m.seq_length(1) == b
        _check_rows(logits.cpu().numpy(), ref[a:b], TOL_BF16, f"chunk {a}:{b}")
        rms = float(np.sqrt(np.mean(ref[b - 1] ** 2)))
        assert margin_ok(ref[b - 1], int(nxt[0].item()), TOL_BF16 * rms), f"chunk {a}:{b} next token"
    dev = m.device
    with torch.cuda.stream(m.stream):
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        lg = torch.empty((1, d.vocab), dtype=torch.float32, device=dev)
        nx = torch.empty(1, dtype=torch.int32, device=dev)
    for i, t in enumerate(forced):
        with torch.cuda.stream(m.stream):
            tok.fill_(int(t))
        m.decode_raw([1], tok, lg, nx)
        m.synchronize()
        _check_rows(lg.cpu().numpy(), ref[200 + i:201 + i], TOL_BF16, f"decode {i}")
    assert m.error_flags() == 0


def test_bf16_chunked_prefill_mixed_batch(bf16_two_layer):
    """One call continuing two slots (after 70 and after 1 cached tokens) and
    starting a fresh one, then a decode step for all three."""
    d, w = bf16_two_layer
    full = [q3synth.make_tokens(L, d.vocab, 60 + i).tolist() for i, L in enumerate([150, 40, 90])]
    first = {0: 70, 2: 1}
    o = OracleModel(d, w)
    m = _model(d, max_slots=4, max_positions=256, max_prefill_tokens=256, kv_tokens=1024)
    m.load_weights(w)
    slots = [3, 0, 1]
    for s, p in zip(slots, full):
        m.seq_alloc(s, len(p) + 4)
    lg0, _ = m.prefill([slots[0], slots[2]], [full[0][:70], full[2][:1]])
    m.synchronize()
    rest = [full[0][70:], full[1], full[2][1:]]
    logits, nxt = m.prefill(slots, rest, all_logits=True)
    m.synchronize()
    g = logits.cpu().numpy()
    row = 0
    refs = []
    for i, p in enumerate(full):
        ref = o.forward(p, o.new_cache(len(p) + 1), logit_rows=range(len(p)))
        refs.append(ref)
        start = first.get(i, 0)
        n = len(p) - start
        _check_rows(g[row:row + n], ref[start:], TOL_BF16, f"seq {i}")
        rms = float(np.sqrt(np.mean(ref[-1] ** 2)))
        assert margin_ok(ref[-1], int(nxt[i].item()), TOL_BF16 * rms), f"seq {i} next token"
        row += n
    for s, p in zip(slots, full):
        assert m.seq_length(s) == len(p)
    # one decode step on top of the continued slots (the oracle's next rows)
    toks = [q3synth.make_tokens(1, d.vocab, 80 + i).tolist()[0] for i in range(3)]
    with torch.cuda.stream(m.stream):
        dt = torch.tensor(toks, dtype=torch.int32, device=m.device)
    lg, _ = m.decode(slots, dt)
    m.synchronize()
    gd = lg.cpu().numpy()
    for i, p in enumerate(full):
        ref = o.forward(p + [toks[i]], o.new_cache(len(p) + 1), logit_rows=[len(p)])
        _check_rows(gd[i:i + 1], ref, TOL_BF16, f"decode seq {i}")
    assert m.error_flags() == 0


def test_f32_chunked_prefill_matches_oracle():
    wl = q3synth.WORKLOADS["tiny2l_f32_p5_d16"]
    d = wl.dims
    w = weights_for(d, 31)
    prompt = q3synth.make_tokens(90, d.vocab, 32).tolist()
    o = OracleModel(d, w)
    ref = o.forward(prompt, o.new_cache(90), logit_rows=range(90))
    m = _model(d, max_slots=1, max_positions=128, max_prefill_tokens=64, kv_tokens=128)
    m.load_weights(w)
    m.seq_alloc(0, 96)
    for a, b in [(0, 3), (3, 64), (64, 90)]:
        logits, nxt = m.prefill([0], [prompt[a:b]], all_logits=True)
        m.synchronize()
        _check_rows(logits.cpu().numpy(), ref[a:b], TOL_F32, f"chunk {a}:{b}")
        rms = float(np.sqrt(np.mean(ref[b - 1] ** 2)))
        assert margin_ok(ref[b - 1], int(nxt[0].item()), TOL_F32 * rms)
    assert m.error_flags() == 0


def test_prefill_rejects_overflowing_continuation(bf16_two_layer):
    from decoder_only_qwen3_amd import Q3Error
    d, w = bf16_two_layer
    m = _model(d, max_slots=1, max_positions=256, max_prefill_tokens=128, kv_tokens=128)
    m.load_weights(w)
    m.seq_alloc(0, 64)
    m.prefill([0], [q3synth.make_tokens(60, d.vocab, 1).tolist()])
    with pytest.raises(Q3Error) as ei:
        m.prefill([0], [q3synth.make_tokens(5, d.vocab, 2).tolist()])
    assert "CAPACITY" in str(ei.value)
    m.synchronize()
    assert m.seq_length(0) == 60
    m.prefill([0], [q3synth.make_tokens(4, d.vocab, 3).tolist()])  # exactly to the slot's end
    m.synchronize()
    assert m.seq_length(0) == 64 and m.error_flags() == 0


# ---------------------------------------------------------------- Paso 8 sampling
def test_bf16_decode_then_top_p_sample(bf16_two_layer):
    """A batched decode step's logits sampled by q3_sample agree with the
    oracle's sampler on the same logits; temperature 0 gives the step's own
    greedy token."""
    from gpu_helpers import sample_agrees
    d, w = bf16_two_layer
    m = _model(d, max_slots=8, max_positions=128, max_prefill_tokens=512, kv_tokens=1024)
    m.load_weights(w)
    prompts = [q3synth.make_tokens(20 + 7 * i, d.vocab, 90 + i).tolist() for i in range(8)]
    slots = list(range(8))
    for s_, p in zip(slots, prompts):
        m.seq_alloc(s_, 128)
    _, nxt = m.prefill(slots, prompts)
    lg, nx = m.decode(slots, nxt)
    rng = np.random.default_rng(5)
    with torch.cuda.stream(m.stream):
        u = torch.from_numpy(rng.random(8).astype(np.float32)).to(m.device)
    tok = m.sample(lg, 0.8, 0.9, u)
    greedy = m.sample(lg, 0.0, 0.9)
    m.synchronize()
    logits = lg.cpu().numpy()
    uh = u.cpu().numpy()
    for r in range(8):
        ok, _ = sample_agrees(logits[r].astype(np.float64), 0.8, 0.9, float(uh[r]), int(tok[r].item()))
        assert ok, r
    np.testing.assert_array_equal(greedy.cpu().numpy(), nx.cpu().numpy())
    assert m.error_flags() == 0


def test_bf16_fused_qkv_epilogue_equals_separate_kernels(bf16_two_layer):
    """Large prefills fold QK-Norm, RoPE and the key append into the q/k/v
    projection's epilogue.  The same calls with the fold switched off (float32
    projection rows, then the separate kernel) must give the same bits: the
    last rows' logits, the next tokens and the whole KV cache, after a packed
    call of three prompts (4,877 tokens: the 256 x 256 tile path) and a
    continuation of one of them by 4,000 tokens."""
    from decoder_only_qwen3_amd import _lib
    d, w = bf16_two_layer
    lib = _lib.load()
    lens = [1500, 2600, 777]
    prompts = [q3synth.make_tokens(L, d.vocab, 300 + i).tolist() for i, L in enumerate(lens)]
    more = q3synth.make_tokens(4000, d.vocab, 310).tolist()
    runs = []
    for mode in (-1, 0):
        _lib.check(lib.q3op_tune(5, mode))
        try:
            m = _model(d, max_slots=4, max_positions=5568, max_prefill_tokens=4992, kv_tokens=9152)
            m.load_weights(w)
            with torch.cuda.stream(m.stream):
                m.bufs[1].zero_()  # unused cache rows compare equal too
            for s, cap in zip([0, 1, 2], [5568, 2624, 832]):
                m.seq_alloc(s, cap)
            lg1, nx1 = m.prefill([0, 1, 2], prompts)
            lg2, nx2 = m.prefill([0], [more])
            m.synchronize()
            assert m.error_flags() == 0
            runs.append([t.cpu() for t in (lg1, nx1, lg2, nx2, m.bufs[1])])
            m.close()
        finally:
            _lib.check(lib.q3op_tune(5, -1))
    for name, a, b in zip(["logits 1", "next 1", "logits 2", "next 2", "kv cache"], runs[0], runs[1]):
        assert torch.equal(a, b), name
