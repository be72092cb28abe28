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
