"""Weight-only affine group quantization on the GPU, through the C ABI: the
quantizer's codes, scales and offsets bit for bit against the oracle's, the
dequantizer, the single-row GEMV on codes, and whole models with 8- and
4-bit projections against the oracle run on the dequantized weights."""
import numpy as np
import pytest
import torch

import q3synth
from checkpoint_files import write_checkpoint
from gpu_helpers import call, dev_bf16, dev_f32, host_bf16, margin_ok, ops, rand_bf16, rel_err, weights_for
from oracle import OracleModel, dequantize_affine, quantize_affine, quantized_weights, rms_norm, silu, to_bf16

pytestmark = pytest.mark.gpu


def _pack(q, bits):
    if bits == 8:
        return q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def _sb_words(s, b):
    return s.view(np.uint16).astype(np.uint32) | (b.view(np.uint16).astype(np.uint32) << 16)


def _quantize_gpu(W, bits):
    _, lib = ops()
    rows, K = W.shape
    codes = torch.zeros(rows * K * bits // 8, dtype=torch.uint8, device="cuda:0")
    sb = torch.zeros(rows * (K // 64), dtype=torch.int32, device="cuda:0")
    dw = dev_bf16(W)
    call(lib.q3op_quantize(dw.data_ptr(), rows, K, bits, codes.data_ptr(), sb.data_ptr(), None))
    torch.cuda.synchronize()
    return codes, sb


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K", [1024, 3072])
def test_quantize_matches_oracle_bit_for_bit(bits, K):
    rng = np.random.default_rng(bits * 100 + K)
    W = rand_bf16(rng, (70, K), 0.02)
    W[3, 64:128] = q3synth.round_to_bf16(np.float32(0.3))      # constant group
    W[5, :64] = rand_bf16(rng, (64,), 1e-6)                     # tiny range
    W[7, 128:192] = rand_bf16(rng, (64,), 3.0)                  # wide range
    codes, sb = _quantize_gpu(W, bits)
    q, s, b = quantize_affine(W, bits)
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(70, -1), _pack(q, bits))
    np.testing.assert_array_equal(sb.cpu().numpy().view(np.uint32).reshape(70, -1), _sb_words(s, b))


@pytest.mark.parametrize("bits", [8, 4])
def test_dequantize_matches_oracle(bits):
    _, lib = ops()
    rng = np.random.default_rng(bits)
    W = rand_bf16(rng, (33, 1024), 0.05)
    codes, sb = _quantize_gpu(W, bits)
    out = torch.zeros((33, 1024), dtype=torch.int16, device="cuda:0")
    call(lib.q3op_dequantize(codes.data_ptr(), sb.data_ptr(), 33, 1024, bits, out.data_ptr(), None))
    torch.cuda.synchronize()
    ref = to_bf16(dequantize_affine(*quantize_affine(W, bits)))
    np.testing.assert_array_equal(host_bf16(out), ref.astype(np.float32))


def _qlinear(bits, epi, x, codes, sb, N, K, gnorm=None, out_init=None):
    _, lib = ops()
    if gnorm is not None:
        dx = dev_f32(x)
    else:
        dx = dev_bf16(x)
    if epi == 2:
        out = torch.zeros(N // 2, dtype=torch.int16, device="cuda:0")
    else:
        out = dev_f32(out_init if out_init is not None else np.zeros(N, np.float32))
    dg = dev_f32(gnorm) if gnorm is not None else None
    call(lib.q3op_qlinear(bits, epi, dx.data_ptr(), codes.data_ptr(), sb.data_ptr(), N, K,
                          dg.data_ptr() if dg is not None else None, 1e-6, out.data_ptr(), None))
    torch.cuda.synchronize()
    return host_bf16(out) if epi == 2 else out.cpu().numpy()


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K", [1024, 2048, 3072])
def test_qlinear_store_residual_swiglu(bits, K):
    rng = np.random.default_rng(bits + K)
    N = 1088  # rows that leave a partial last wavefront for every row grouping
    W = rand_bf16(rng, (N, K), 0.02)
    codes, sb = _quantize_gpu(W, bits)
    Wq = to_bf16(dequantize_affine(*quantize_affine(W, bits)))  # the weights the kernels multiply by
    x = rand_bf16(rng, (K,))
    ref = Wq @ x.astype(np.float64)
    got = _qlinear(bits, 0, x, codes, sb, N, K)
    assert rel_err(got, ref) < 2e-5
    base = rng.standard_normal(N).astype(np.float32)
    got = _qlinear(bits, 1, x, codes, sb, N, K, out_init=base)
    assert rel_err(got - base, ref) < 2e-5
    # SwiGLU: rows interleaved [gate 16 | up 16]
    g_rows = np.concatenate([np.arange(c * 32, c * 32 + 16) for c in range(N // 32)])
    u_rows = g_rows + 16
    got = _qlinear(bits, 2, x, codes, sb, N, K)
    want = to_bf16(silu(ref[g_rows]) * ref[u_rows])
    np.testing.assert_allclose(got, want, rtol=2 ** -7, atol=1e-6)


@pytest.mark.parametrize("bits", [8, 4])
def test_qlinear_rmsnorm_prologue(bits):
    rng = np.random.default_rng(50 + bits)
    N, K = 4096, 1024
    W = rand_bf16(rng, (N, K), 0.02)
    codes, sb = _quantize_gpu(W, bits)
    Wq = to_bf16(dequantize_affine(*quantize_affine(W, bits)))
    x = rng.standard_normal(K).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    a = to_bf16(rms_norm(x.astype(np.float64)[None], g.astype(np.float64), 1e-6))[0]
    ref = Wq @ a
    got = _qlinear(bits, 0, x, codes, sb, N, K, gnorm=g)
    # an activation rounded to the other bf16 neighbour moves a few outputs
    assert rel_err(got, ref) < 5e-3
    assert np.median(np.abs(got - ref)) < 1e-5 * np.sqrt(np.mean(ref ** 2)) + 1e-6


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [2, 17, 64])
def test_qlinear_rows_weight_streaming(bits, M):
    """M activation rows by the weight-streaming kernel on codes: store,
    split-K residual, SwiGLU, and the RMSNorm prologue for M <= 16."""
    _, lib = ops()
    rng = np.random.default_rng(bits * 7 + M)
    for N, K in ((1024, 2048), (2048, 1024)):
        W = rand_bf16(rng, (N, K), 0.02)
        codes, sb = _quantize_gpu(W, bits)
        Wq = to_bf16(dequantize_affine(*quantize_affine(W, bits)))
        X = rand_bf16(rng, (M, K))
        ref = X.astype(np.float64) @ Wq.T
        ws = torch.zeros(max(256, lib.q3op_qlinear_rows_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda:0")
        dx = dev_bf16(X)
        for epi in (0, 1, 2):
            base = rng.standard_normal((M, N)).astype(np.float32)
            if epi == 2:
                out = torch.zeros((M, N // 2), dtype=torch.int16, device="cuda:0")
                ldo = N // 2
            else:
                out = dev_f32(base if epi == 1 else np.zeros((M, N), np.float32))
                ldo = N
            call(lib.q3op_qlinear_rows(bits, epi, dx.data_ptr(), M, codes.data_ptr(), sb.data_ptr(), N, K, None, 1e-6,
                                       out.data_ptr(), ldo, ws.data_ptr(), ws.numel(), None))
            torch.cuda.synchronize()
            if epi == 2:
                g_rows = np.concatenate([np.arange(c * 32, c * 32 + 16) for c in range(N // 32)])
                want = to_bf16(silu(ref[:, g_rows]) * ref[:, g_rows + 16])
                np.testing.assert_allclose(host_bf16(out), want, rtol=2 ** -7, atol=1e-6)
            else:
                got = out.cpu().numpy() - (base if epi == 1 else 0)
                assert rel_err(got, ref) < 2e-5, (N, K, epi)
        if M <= 16:
            x = rng.standard_normal((M, K)).astype(np.float32)
            g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
            a = to_bf16(rms_norm(x.astype(np.float64), g.astype(np.float64), 1e-6))
            out = dev_f32(np.zeros((M, N), np.float32))
            dxf, dg = dev_f32(x), dev_f32(g)
            call(lib.q3op_qlinear_rows(bits, 0, dxf.data_ptr(), M, codes.data_ptr(), sb.data_ptr(), N, K, dg.data_ptr(),
                                       1e-6, out.data_ptr(), N, None, 0, None))
            torch.cuda.synchronize()
            assert rel_err(out.cpu().numpy(), a @ Wq.T) < 5e-3


def test_qlinear_rejects_bad_arguments():
    mod, lib = ops()
    z = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda:0")
    for bits, epi, N, K in [(3, 0, 32, 1024), (8, 0, 32, 512), (8, 2, 40, 1024), (8, 3, 32, 1024)]:
        assert lib.q3op_qlinear(bits, epi, z.data_ptr(), z.data_ptr(), z.data_ptr(), N, K, None, 1e-6,
                                z.data_ptr(), None) != 0


# ---------------------------------------------------------------- whole model
@pytest.fixture(scope="module")
def two_layer():
    d = q3synth.QWEN3_06B.replace(n_layers=2)
    return d, weights_for(d, 77)


def _model(d, bits, **kw):
    from decoder_only_qwen3_amd import Q3Model
    return Q3Model(d, max_slots=4, max_positions=256, max_prefill_tokens=512, kv_tokens=1024, weight_bits=bits, **kw)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_model_matches_oracle(two_layer, bits):
    """Prefill (dequantized layer + GEMM), batch-1 decode (GEMV on codes) and
    a batch-3 decode step (dequantized layer + batched kernels) against the
    oracle on the dequantized weights."""
    d, w = two_layer
    m = _model(d, bits)
    from decoder_only_qwen3_amd import Q3Model  # noqa: F401
    full = _model(d, 0)
    # the block projections shrink from 2 to bits/8 + 4/64 bytes per weight
    per_layer = (4096 + 2048 + 6144 + 3072) * 1024
    saved = full.nbytes[0] - m.nbytes[0]
    assert abs(saved - d.n_layers * per_layer * (2 - (bits / 8 + 4 / 64))) < d.n_layers * 64 * 1024, saved
    full.close()
    m.load_weights(w)
    o = OracleModel(d, quantized_weights(w, bits), contract=True)
    prompt = q3synth.make_tokens(100, d.vocab, 5).tolist()
    forced = q3synth.make_tokens(4, d.vocab, 6).tolist()
    ref = o.forced_logits(prompt, forced)
    m.seq_alloc(0, 128)
    lg, nx = m.prefill([0], [prompt])
    with torch.cuda.stream(m.stream):  # read the result behind the call that writes it
        rows = [lg[0].clone()]
    for t in forced:
        with torch.cuda.stream(m.stream):
            tok = torch.tensor([t], dtype=torch.int32, device=m.device)
        lg1, _ = m.decode([0], tok)
        with torch.cuda.stream(m.stream):
            rows.append(lg1[0].clone())
    m.synchronize()
    for i, r in enumerate(rows):
        g = r.cpu().numpy()
        assert rel_err(g, ref[i]) <= 3e-2, (i, rel_err(g, ref[i]))
        assert margin_ok(ref[i], int(np.argmax(g)), 3e-2 * float(np.sqrt(np.mean(ref[i] ** 2))))
    # three sequences in one decode step
    prompts = [q3synth.make_tokens(L, d.vocab, 30 + L).tolist() for L in (9, 40, 77)]
    for s_ in (1, 2, 3):
        m.seq_alloc(s_, 128)
    m.prefill([1, 2, 3], prompts)
    toks = [11, 22, 33]
    with torch.cuda.stream(m.stream):
        dt = torch.tensor(toks, dtype=torch.int32, device=m.device)
    lg3, _ = m.decode([1, 2, 3], dt)
    m.synchronize()
    g3 = lg3.cpu().numpy()
    for i, p in enumerate(prompts):
        r = o.forced_logits(p, [toks[i]])[1]
        assert rel_err(g3[i], r) <= 3e-2, (i, rel_err(g3[i], r))
    assert m.error_flags() == 0


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_small_model_general_shapes(bits):
    """A 512-wide model: the single-row GEMV on codes needs K % 1024 == 0, so
    one-sequence decode takes the weight-streaming kernel on codes."""
    from decoder_only_qwen3_amd import Q3Model
    d = q3synth.QWEN3_06B.replace(n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=2, ffn=1024, vocab=4096)
    w = weights_for(d, 91)
    m = Q3Model(d, max_slots=2, max_positions=128, max_prefill_tokens=128, kv_tokens=256, weight_bits=bits)
    m.load_weights(w)
    o = OracleModel(d, quantized_weights(w, bits), contract=True)
    prompt = q3synth.make_tokens(37, d.vocab, 92).tolist()
    ref = o.forced_logits(prompt, [5, 6])
    m.seq_alloc(0, 64)
    lg, _ = m.prefill([0], [prompt])
    with torch.cuda.stream(m.stream):
        rows = [lg[0].clone()]
    for t in (5, 6):
        with torch.cuda.stream(m.stream):
            tok = torch.tensor([t], dtype=torch.int32, device=m.device)
        lg1, _ = m.decode([0], tok)
        with torch.cuda.stream(m.stream):
            rows.append(lg1[0].clone())
    m.synchronize()
    for i, r in enumerate(rows):
        assert rel_err(r.cpu().numpy(), ref[i]) <= 3e-2, (i, rel_err(r.cpu().numpy(), ref[i]))
    assert m.error_flags() == 0


def test_quantized_checkpoint_load_equals_upload(two_layer, tmp_path):
    d, w = two_layer
    path = str(tmp_path / "model.safetensors")
    write_checkpoint(w, [path])
    prompt = q3synth.make_tokens(20, d.vocab, 8).tolist()
    outs = []
    for how in ("upload", "file"):
        m = _model(d, 8)
        if how == "upload":
            m.load_weights(w)
        else:
            m.load_safetensors([path])
        m.seq_alloc(0, 64)
        lg, _ = m.prefill([0], [prompt])
        with torch.cuda.stream(m.stream):
            a = lg.clone()
        m.synchronize()
        outs.append(a.cpu().numpy())
        m.close()
    np.testing.assert_array_equal(outs[0], outs[1])


def test_quantized_model_rejects_host_tensors(two_layer):
    import ctypes as C
    from decoder_only_qwen3_amd import _lib
    d, w = two_layer
    m = _model(d, 8)
    host = np.zeros(10, np.uint16)
    t = (_lib.q3_tensor * 1)()
    t[0].name = b"model.layers.0.self_attn.q_proj.weight"
    t[0].data = host.ctypes.data
    t[0].dtype = _lib.Q3_BF16
    t[0].ndim = 2
    t[0].shape[0], t[0].shape[1] = 2048, 1024
    st = m.lib.q3_load_weights(m.handle, t, 1, m.sh)
    assert st == _lib.Q3_E_ARG and b"device memory" in m.lib.q3_last_error()
    m.close()
