"""Kernel-level parity: each libq3 kernel (through include/q3_ops.h) against
the matching oracle function on seeded random inputs, at sizes that span
several tiles and a ragged tail."""
import ctypes as C

import numpy as np
import pytest
import torch

import q3synth
from gpu_helpers import (call, dev_bf16, dev_f32, host_bf16, k_blocks, k_logical, ops, rand_bf16, vt_blocks,
                         vt_logical)
from oracle import attention_rows, rms_norm, rope_cos_sin, rope_rotate, silu, to_bf16

pytestmark = pytest.mark.gpu

EPI_STORE, EPI_RESADD, EPI_SWIGLU, EPI_ARGMAX = 0, 1, 2, 3
GEMM, SKINNY, GEMV_F32, ROWDOT, ROWGEMV, HEADSTREAM = 0, 1, 2, 3, 4, 5
BF16, F32 = 1, 0


def _sync():
    torch.cuda.synchronize()


def _ws(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda:0")


# ---------------------------------------------------------------- Paso 2 / Paso 3
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_embed_gather_and_bad_id(dtype):
    mod, lib = ops()
    rng = np.random.default_rng(1)
    V, H = 1000, 256
    table = rand_bf16(rng, (V, H)) if dtype == BF16 else rng.standard_normal((V, H)).astype(np.float32)
    ids = np.array([0, 999, 5, 5, 1000, -1, 17], dtype=np.int32)
    dt = dev_bf16(table) if dtype == BF16 else dev_f32(table)
    di = torch.from_numpy(ids).to("cuda:0")
    out = torch.empty((len(ids), H), dtype=torch.float32, device="cuda:0")
    err = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    call(lib.q3op_embed(dtype, di.data_ptr(), len(ids), dt.data_ptr(), V, H, out.data_ptr(), err.data_ptr(), None))
    _sync()
    got = out.cpu().numpy()
    for r, t in enumerate(ids):
        expect = table[t] if 0 <= t < V else np.zeros(H, np.float32)
        np.testing.assert_array_equal(got[r], expect)
    assert int(err[0].item()) & 1


@pytest.mark.parametrize("rows", [1, 5, 67])
@pytest.mark.parametrize("out_dtype", [F32, BF16])
def test_rmsnorm(rows, out_dtype):
    mod, lib = ops()
    rng = np.random.default_rng(rows)
    H = 1024
    x = (rng.standard_normal((rows, H)) * rng.uniform(0.01, 20, (rows, 1))).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    out = torch.empty((rows, H), dtype=torch.float32 if out_dtype == F32 else torch.int16, device="cuda:0")
    dx, dw = dev_f32(x), dev_f32(w)   # keep the device copies alive until the kernel ran
    call(lib.q3op_rmsnorm(out_dtype, dx.data_ptr(), rows, dw.data_ptr(), H, 1e-6, out.data_ptr(), None))
    _sync()
    ref = rms_norm(x.astype(np.float64), w.astype(np.float64), 1e-6)
    if out_dtype == F32:
        np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=2e-6, atol=1e-6)
    else:
        got = host_bf16(out)
        # same rounding point as the oracle's contract; fp32 vs fp64 may flip a tie by 1 ulp
        np.testing.assert_allclose(got, to_bf16(ref), rtol=2 ** -7, atol=1e-30)
        assert np.mean(got == to_bf16(ref)) > 0.99


# ---------------------------------------------------------------- projections
def _pack_gate_up(g, u):
    I = g.shape[0]
    out = np.empty((2 * I, g.shape[1]), dtype=g.dtype)
    for r in range(I // 16):
        out[32 * r:32 * r + 16] = g[16 * r:16 * r + 16]
        out[32 * r + 16:32 * r + 32] = u[16 * r:16 * r + 16]
    return out


def _linear(kernel, epi, X, W, out_init=None, ldo=None, want_next=False):
    mod, lib = ops()
    M, K = X.shape
    N = W.shape[0]
    bf = kernel in (GEMM, SKINNY, ROWDOT, ROWGEMV, HEADSTREAM)
    dx = dev_bf16(X) if bf else dev_f32(X)
    dw = dev_bf16(W) if bf else dev_f32(W)
    if epi == EPI_SWIGLU:
        ldo = ldo or N // 2
        out = torch.zeros((M, ldo), dtype=torch.int16 if bf else torch.float32, device="cuda:0")
    else:
        ldo = ldo or N
        out = dev_f32(out_init) if out_init is not None else torch.zeros((M, ldo), dtype=torch.float32, device="cuda:0")
    nxt = torch.full((max(M, 1),), -7, dtype=torch.int32, device="cuda:0")
    ws = _ws(lib.q3op_linear_workspace_bytes(kernel, epi, M, N, K))
    call(lib.q3op_linear(kernel, epi, dx.data_ptr(), M, dw.data_ptr(), N, K, out.data_ptr(), ldo,
                         nxt.data_ptr() if want_next else None, ws.data_ptr(), ws.numel(), None))
    _sync()
    got = host_bf16(out) if (epi == EPI_SWIGLU and bf) else out.cpu().numpy()
    return got, nxt.cpu().numpy()


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


@pytest.mark.parametrize("kernel,M", [(GEMM, 1), (GEMM, 5), (GEMM, 130), (GEMM, 257),
                                      (SKINNY, 1), (SKINNY, 3), (SKINNY, 16), (SKINNY, 17), (SKINNY, 64),
                                      (ROWGEMV, 1)])
@pytest.mark.parametrize("N,K", [(4096, 1024), (1024, 2048), (1024, 3072)])
def test_linear_store_and_residual(kernel, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    X = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), 0.02)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    got, _ = _linear(kernel, EPI_STORE, X, W)
    assert _rel(got, ref) < 2e-5
    base = rng.standard_normal((M, N)).astype(np.float32)
    got, _ = _linear(kernel, EPI_RESADD, X, W, out_init=base)
    assert _rel(got - base, ref) < 2e-5


@pytest.mark.parametrize("M", [64, 500, 512, 1000, 4000, 4096])
@pytest.mark.parametrize("N,K", [(1024, 2048), (1024, 3072), (2048, 1024)])
def test_gemm_split_k_residual(M, N, K):
    """Residual GEMMs on grids too small to fill the chip are split over K; the
    slices merge in a fixed order, so repeated calls agree bit for bit."""
    rng = np.random.default_rng(M + N + K)
    X = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), 0.02)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    base = rng.standard_normal((M, N)).astype(np.float32)
    got1, _ = _linear(GEMM, EPI_RESADD, X, W, out_init=base)
    got2, _ = _linear(GEMM, EPI_RESADD, X, W, out_init=base)
    assert _rel(got1 - base, ref) < 2e-5
    assert np.array_equal(got1, got2)


@pytest.mark.parametrize("M", [5, 17, 33, 64])
@pytest.mark.parametrize("N,K", [(1024, 2048), (1024, 3072)])
def test_skinny_split_k_residual(M, N, K):
    """The decode residual projections (1024 outputs) split K over block
    slices; the last slice adds the partials in slice order, then the
    residual, so repeated calls agree bit for bit and every row matches the
    float64 product, including the rows of a partly filled 16-row tile."""
    rng = np.random.default_rng(7 * M + N + K)
    X = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), 0.02)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    base = rng.standard_normal((M, N)).astype(np.float32)
    got1, _ = _linear(SKINNY, EPI_RESADD, X, W, out_init=base)
    got2, _ = _linear(SKINNY, EPI_RESADD, X, W, out_init=base)
    assert _rel(got1 - base, ref) < 2e-5
    assert np.array_equal(got1, got2)


@pytest.mark.parametrize("cfg", list(range(12)))
def test_gemm_tile_configurations(cfg):
    """Every prefill GEMM tile shape, with ragged row and column tails."""
    _, lib = ops()
    call(lib.q3op_tune(1, cfg))
    try:
        M, N, K = 300, 1088, 1024
        rng = np.random.default_rng(100 + cfg)
        X = rand_bf16(rng, (M, K))
        W = rand_bf16(rng, (N, K), 0.02)
        ref = X.astype(np.float64) @ W.astype(np.float64).T
        got, _ = _linear(GEMM, EPI_STORE, X, W)
        assert _rel(got, ref) < 2e-5
        base = rng.standard_normal((M, N)).astype(np.float32)
        got, _ = _linear(GEMM, EPI_RESADD, X, W, out_init=base)
        assert _rel(got - base, ref) < 2e-5
        g, u = ref.reshape(M, N // 32, 2, 16)[:, :, 0, :], ref.reshape(M, N // 32, 2, 16)[:, :, 1, :]
        act = (silu(g) * u).reshape(M, N // 2)
        got, _ = _linear(GEMM, EPI_SWIGLU, X, W)
        np.testing.assert_allclose(got, to_bf16(act), rtol=2.0 ** -7, atol=1e-6 * np.sqrt(np.mean(act ** 2)))
    finally:
        call(lib.q3op_tune(1, -1))


def test_tune_rejects_bad_values():
    _, lib = ops()
    assert lib.q3op_tune(1, 12) != 0
    assert lib.q3op_tune(2, 3) != 0
    assert lib.q3op_tune(2, 4) != 0
    assert lib.q3op_tune(3, 3 + 256) != 0
    assert lib.q3op_tune(3, 4 + 5 * 256) != 0
    assert lib.q3op_tune(4, 0) != 0
    assert lib.q3op_tune(4, 65) != 0
    assert lib.q3op_tune(99, 0) != 0


@pytest.mark.parametrize("rows", [1, 2, 4, 8])
@pytest.mark.parametrize("waves", [1, 2, 4])
def test_rowgemv_shapes(rows, waves):
    """Every single-row GEMV shape, with row counts that leave partial wavefronts and blocks."""
    _, lib = ops()
    call(lib.q3op_tune(3, rows + 256 * waves))
    try:
        rng = np.random.default_rng(rows * 10 + waves)
        K = 2048
        X = rand_bf16(rng, (1, K))
        for N in (1040, 1041):
            W = rand_bf16(rng, (N, K), 0.02)
            ref = X.astype(np.float64) @ W.astype(np.float64).T
            got, _ = _linear(ROWGEMV, EPI_STORE, X, W)
            assert _rel(got, ref) < 2e-5, N
            base = rng.standard_normal((1, N)).astype(np.float32)
            got, _ = _linear(ROWGEMV, EPI_RESADD, X, W, out_init=base)
            assert _rel(got - base, ref) < 2e-5, N
            got, nxt = _linear(ROWGEMV, EPI_ARGMAX, X, W, want_next=True)
            assert _rel(got, ref) < 2e-5, N
            assert nxt[0] == int(np.argmax(got[0]))
        if rows % 2 == 0:
            N = 1088
            G, U = rand_bf16(rng, (N // 2, K), 0.05), rand_bf16(rng, (N // 2, K), 0.05)
            got, _ = _linear(ROWGEMV, EPI_SWIGLU, X, _pack_gate_up(G, U))
            g = X.astype(np.float64) @ G.astype(np.float64).T
            u = X.astype(np.float64) @ U.astype(np.float64).T
            np.testing.assert_allclose(got, to_bf16(silu(g) * u), rtol=2 ** -7, atol=1e-6)
        else:
            mod, _ = ops()
            x = torch.zeros(K, dtype=torch.int16, device="cuda:0")
            w = torch.zeros((64, K), dtype=torch.int16, device="cuda:0")
            o = torch.zeros(32, dtype=torch.int16, device="cuda:0")
            st = lib.q3op_linear(ROWGEMV, EPI_SWIGLU, x.data_ptr(), 1, w.data_ptr(), 64, K, o.data_ptr(), 32, None,
                                 None, 0, None)
            assert st != 0, "odd rows per wavefront cannot pair gate and up rows"
    finally:
        call(lib.q3op_tune(3, -1))


@pytest.mark.parametrize("kernel,M", [(GEMM, 3), (GEMM, 200), (SKINNY, 1), (SKINNY, 40), (GEMV_F32, 6),
                                      (ROWGEMV, 1)])
def test_linear_swiglu(kernel, M):
    rng = np.random.default_rng(M)
    I, H = 3072, 1024
    bf = kernel != GEMV_F32
    mk = (lambda s, sc=1.0: rand_bf16(rng, s, sc)) if bf else (lambda s, sc=1.0: (rng.standard_normal(s) * sc).astype(np.float32))
    X = mk((M, H))
    G, U = mk((I, H), 0.05), mk((I, H), 0.05)
    got, _ = _linear(kernel, EPI_SWIGLU, X, _pack_gate_up(G, U))
    g = X.astype(np.float64) @ G.astype(np.float64).T
    u = X.astype(np.float64) @ U.astype(np.float64).T
    ref = silu(g) * u
    if bf:
        # one bf16 rounding of the product: at most one ulp (2^-7 relative) apart
        np.testing.assert_allclose(got, to_bf16(ref), rtol=2 ** -7, atol=1e-6)
        assert np.mean(got == to_bf16(ref)) > 0.99
    else:
        assert _rel(got, ref) < 1e-5


@pytest.mark.parametrize("M", [1, 2, 9])
def test_gemv_f32_store_and_residual(M):
    rng = np.random.default_rng(100 + M)
    X = rng.standard_normal((M, 1024)).astype(np.float32)
    W = (0.02 * rng.standard_normal((2048, 1024))).astype(np.float32)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    got, _ = _linear(GEMV_F32, EPI_STORE, X, W)
    assert _rel(got, ref) < 1e-5
    base = rng.standard_normal((M, 2048)).astype(np.float32)
    got, _ = _linear(GEMV_F32, EPI_RESADD, X, W, out_init=base)
    assert _rel(got - base, ref) < 1e-5


@pytest.mark.parametrize("kernel,M", [(SKINNY, 1), (SKINNY, 7), (SKINNY, 64), (GEMM, 3), (GEMV_F32, 2),
                                      (ROWGEMV, 1), (HEADSTREAM, 2), (HEADSTREAM, 17), (HEADSTREAM, 64)])
def test_logits_and_argmax(kernel, M):
    rng = np.random.default_rng(300 + M)
    V, H = 8192, 1024
    bf = kernel != GEMV_F32
    X = rand_bf16(rng, (M, H)) if bf else rng.standard_normal((M, H)).astype(np.float32)
    E = rand_bf16(rng, (V, H), 0.02) if bf else (0.02 * rng.standard_normal((V, H))).astype(np.float32)
    # plant exact ties: row 4100 duplicates row 4000, row 100 gets the winner's values too
    ref = X.astype(np.float64) @ E.astype(np.float64).T
    win = int(np.argmax(ref[0]))
    E[4100] = E[win]
    E[win + 1 if win + 1 < V else 0] = E[win]
    ref = X.astype(np.float64) @ E.astype(np.float64).T
    got, nxt = _linear(kernel, EPI_ARGMAX, X, E, want_next=True)
    assert _rel(got, ref) < 2e-5
    for m in range(M):
        # argmax of the kernel's own logits with lowest-index ties
        assert nxt[m] == int(np.argmax(got[m]))
        top = int(np.argmax(ref[m]))
        assert ref[m][top] - ref[m][nxt[m]] <= 1e-5 * np.sqrt(np.mean(ref[m] ** 2))


@pytest.mark.parametrize("M", [32, 64])
def test_headstream_full_vocabulary(M):
    """The streaming lm_head at the model's vocabulary (151,936 rows, several
    16-row groups per wavefront): logits against the float64 product, and the
    greedy pick with copies of each row's winner planted at higher and lower
    indices in other blocks (the lowest index must win)."""
    rng = np.random.default_rng(900 + M)
    V, H = 151936, 1024
    X = rand_bf16(rng, (M, H))
    E = rand_bf16(rng, (V, H), 0.02)
    ref = X.astype(np.float64) @ E.astype(np.float64).T
    win = int(np.argmax(ref[0]))
    E[(win + 77777) % V] = E[win]
    E[(win + 4096) % V] = E[win]
    ref = X.astype(np.float64) @ E.astype(np.float64).T
    got, nxt = _linear(HEADSTREAM, EPI_ARGMAX, X, E, want_next=True)
    assert _rel(got, ref) < 2e-5
    for m in range(M):
        assert nxt[m] == int(np.argmax(got[m])), m
    assert nxt[0] == min(win, (win + 77777) % V, (win + 4096) % V)


def test_headstream_rejects_unsupported_shapes():
    _, lib = ops()
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    ws = _ws(1 << 16)
    p = dummy.data_ptr()
    assert lib.q3op_linear(HEADSTREAM, EPI_STORE, p, 65, p, 4096, 1024, p, 4096, None, ws.data_ptr(), ws.numel(), None) != 0
    assert lib.q3op_linear(HEADSTREAM, EPI_STORE, p, 8, p, 4100, 1024, p, 4100, None, ws.data_ptr(), ws.numel(), None) != 0
    assert lib.q3op_linear(HEADSTREAM, EPI_STORE, p, 8, p, 4096, 1000, p, 4096, None, ws.data_ptr(), ws.numel(), None) != 0
    assert lib.q3op_linear(HEADSTREAM, EPI_STORE, p, 8, p, 4096, 768, p, 4096, None, ws.data_ptr(), ws.numel(), None) != 0
    assert lib.q3op_linear(HEADSTREAM, EPI_RESADD, p, 8, p, 4096, 1024, p, 4096, None, ws.data_ptr(), ws.numel(), None) != 0


# ---------------------------------------------------------------- Pasos 4-5: QK-Norm, RoPE, cache append
def _arena(lens_cap, n_kv, esz):
    bases, off = [], 0
    for cap in lens_cap:
        bases.append(off)
        off += 2 * n_kv * cap * 128
    return bases, off


@pytest.mark.parametrize("dtype", [BF16, F32])
@pytest.mark.parametrize("mode", ["prefill", "decode", "continue"])
def test_rope_append(dtype, mode):
    mod, lib = ops()
    decode = 1 if mode == "decode" else 0
    rng = np.random.default_rng(5 + decode + 7 * (mode == "continue"))
    n_q, n_kv = 16, 8
    if decode:
        lens = [1, 1, 1]
        cu = [0, 1, 2, 3]
        prior = [0, 70, 4000]
    else:
        lens = [3, 64, 130]
        cu = list(np.concatenate([[0], np.cumsum(lens)]))
        # continuation: new positions start inside a 32-key value block, on a
        # 64-position tile boundary, and mid-tile with a partial tail
        prior = [0, 0, 0] if mode == "prefill" else [5, 64, 3001]
    caps = [4096, 128, 4096]
    T = cu[-1]
    units = n_q + 2 * n_kv
    qkv = rng.standard_normal((T, units * 128)).astype(np.float32)
    qn = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    kn = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    if dtype == BF16:
        qn, kn = q3synth.round_to_bf16(qn), q3synth.round_to_bf16(kn)
    bases, total = _arena(caps, n_kv, 2 if dtype == BF16 else 4)
    kv = torch.zeros(total, dtype=torch.int16 if dtype == BF16 else torch.float32, device="cuda:0")
    qout = torch.zeros((T, n_q, 128), dtype=torch.int16 if dtype == BF16 else torch.float32, device="cuda:0")
    max_pos = 4100
    ws = _ws(lib.q3op_rope_workspace_bytes(len(lens), max_pos))
    dqkv, dqn, dkn = dev_f32(qkv), dev_f32(qn), dev_f32(kn)
    call(lib.q3op_rope_append(dtype, dqkv.data_ptr(), len(lens), mod.i32_array(cu), decode,
                              mod.i64_array(bases), mod.i32_array(caps), mod.i32_array(prior), kv.data_ptr(),
                              n_q, n_kv, dqn.data_ptr(), dkn.data_ptr(), 1e-6, 1e6, max_pos,
                              qout.data_ptr(), ws.data_ptr(), ws.numel(), None))
    _sync()
    rnd = to_bf16 if dtype == BF16 else (lambda a: a)
    read = host_bf16 if dtype == BF16 else (lambda t: t.cpu().numpy())
    q_got = read(qout).reshape(T, n_q, 128)
    kv_got = read(kv)
    tol = dict(rtol=2 ** -7, atol=1e-6) if dtype == BF16 else dict(rtol=1e-5, atol=1e-6)
    for b in range(len(lens)):
        rows = slice(cu[b], cu[b + 1])
        pos = prior[b] + np.arange(lens[b])
        x = qkv[rows].astype(np.float64).reshape(-1, units, 128)
        c, s = rope_cos_sin(pos, 128, 1e6)
        q_ref = rnd(rope_rotate(rms_norm(x[:, :n_q], qn, 1e-6), c, s))
        k_ref = rnd(rope_rotate(rms_norm(x[:, n_q:n_q + n_kv], kn, 1e-6), c, s))
        v_ref = rnd(x[:, n_q + n_kv:])
        np.testing.assert_allclose(q_got[rows], q_ref, **tol)
        cap = caps[b]
        region = kv_got[bases[b]:bases[b] + 2 * n_kv * cap * 128]
        if dtype == BF16:
            K = k_logical(region[:n_kv * cap * 128], n_kv, cap)
        else:
            K = region[:n_kv * cap * 128].reshape(n_kv, cap, 128)
        Vt = vt_logical(region[n_kv * cap * 128:], n_kv, cap)
        for i, p in enumerate(pos):
            np.testing.assert_allclose(K[:, p, :], k_ref[i], **tol)
            np.testing.assert_array_equal(Vt[:, :, p], v_ref[i].astype(np.float32))
        if not decode:  # nothing written outside the new positions (partial value tiles)
            end = prior[b] + lens[b]
            assert not np.any(K[:, end:, :]) and not np.any(Vt[:, :, end:])
            assert not np.any(K[:, :prior[b], :]) and not np.any(Vt[:, :, :prior[b]])


# ---------------------------------------------------------------- Paso 5: attention
def _attention_case(kernel, lens, prior, caps, n_q=16, n_kv=8, seed=0, splits=0, cached=None):
    """decode: query b at position prior[b] over keys 0..prior[b].  Prefill:
    token i of sequence b at position cached[b] + i (cached[b] = 0 by default)
    over keys 0..cached[b] + i."""
    mod, lib = ops()
    rng = np.random.default_rng(seed)
    decode = kernel == 1 or (kernel == 2 and prior is not None)
    bf = kernel != 2
    mk = (lambda s: rand_bf16(rng, s)) if bf else (lambda s: rng.standard_normal(s).astype(np.float32))
    n = len(lens)
    if decode:
        ctx = [p + 1 for p in prior]
        cu = list(range(n + 1))
        q = mk((n, n_q, 128))
    else:
        prior = list(cached) if cached is not None else [0] * n
        ctx = [p + L for p, L in zip(prior, lens)]
        cu = list(np.concatenate([[0], np.cumsum(lens)]))
        q = mk((cu[-1], n_q, 128))
    bases, total = _arena(caps, n_kv, 2 if bf else 4)
    arena = np.full(total, np.nan if not bf else 0, dtype=np.float32)
    if bf:
        arena = np.zeros(total, np.float32)
        # fill the unused cache area with NaN bit patterns later via torch (garbage must not leak)
    Ks, Vs = [], []
    for b in range(n):
        K = mk((ctx[b], n_kv, 128))
        V = mk((ctx[b], n_kv, 128))
        Ks.append(K)
        Vs.append(V)
        cap = caps[b]
        region = np.zeros(2 * n_kv * cap * 128, np.float32)
        Kc = np.zeros((n_kv, cap, 128), np.float32)
        Vt = np.zeros((n_kv, 128, cap), np.float32)
        Kc[:, :ctx[b], :] = K.transpose(1, 0, 2)
        Vt[:, :, :ctx[b]] = V.transpose(1, 2, 0)
        region[:n_kv * cap * 128] = k_blocks(Kc) if bf else Kc.reshape(-1)
        region[n_kv * cap * 128:] = vt_blocks(Vt)
        arena[bases[b]:bases[b] + region.size] = region
    if bf:
        bits = q3synth.bf16_bits(arena)
        # poison every cache slot beyond each sequence's context with NaN
        for b in range(n):
            cap = caps[b]
            reg = bits[bases[b]:bases[b] + 2 * n_kv * cap * 128]
            Kc = k_logical(reg[:n_kv * cap * 128], n_kv, cap)
            Vt = vt_logical(reg[n_kv * cap * 128:], n_kv, cap).copy()
            Kc[:, ctx[b]:, :] = 0x7FC0
            Vt[:, :, ctx[b]:] = 0x7FC0
            reg[:n_kv * cap * 128] = k_blocks(Kc)
            reg[n_kv * cap * 128:] = vt_blocks(Vt)
        dkv = torch.from_numpy(bits.view(np.int16)).to("cuda:0")
        dq = dev_bf16(q)
        out = torch.zeros((q.shape[0], n_q, 128), dtype=torch.int16, device="cuda:0")
    else:
        dkv = dev_f32(arena)
        dq = dev_f32(q)
        out = torch.zeros((q.shape[0], n_q, 128), dtype=torch.float32, device="cuda:0")
    keys = int(cu[-1]) if decode else int(sum(ctx))
    ws = _ws(lib.q3op_attention_workspace_bytes(kernel, n, keys, n_q, n_kv, splits))
    call(lib.q3op_attention(kernel, dq.data_ptr(), n, mod.i32_array(cu), 1 if decode else 0,
                            mod.i64_array(bases), mod.i32_array(caps), mod.i32_array(prior), dkv.data_ptr(),
                            n_q, n_kv, splits, out.data_ptr(), ws.data_ptr(), ws.numel(), None))
    _sync()
    got = host_bf16(out) if bf else out.cpu().numpy()
    worst = 0.0
    refs = []
    for b in range(n):
        if decode:
            qb = q[b:b + 1].astype(np.float64)
            ref = attention_rows(qb, Ks[b].astype(np.float64), Vs[b].astype(np.float64),
                                 np.array([prior[b]]), np.arange(ctx[b]))
            g = got[b:b + 1]
        else:
            qb = q[cu[b]:cu[b + 1]].astype(np.float64)
            pos = prior[b] + np.arange(lens[b])
            ref = attention_rows(qb, Ks[b].astype(np.float64), Vs[b].astype(np.float64), pos,
                                 np.arange(ctx[b]))
            g = got[cu[b]:cu[b + 1]]
        assert np.all(np.isfinite(g)), f"seq {b}: non-finite output"
        # Error in units of the allowed bound.  bf16 output: half an ulp of the
        # stored value (2^-8 relative) plus 2e-3 of the row RMS for the fp16
        # softmax weights; float32: 1e-5 of the row RMS.
        rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
        bound = (2.0 ** -8 * np.abs(ref) + 2e-3 * rms) if bf else 1e-5 * rms
        worst = max(worst, float(np.max(np.abs(g - ref) / bound)))
    return worst


@pytest.mark.parametrize("lens", [[1], [5], [64], [65], [130, 1, 63, 200], [513], [600, 3, 130, 1100]])
def test_flash_prefill_attention(lens):
    caps = [((L + 63) // 64) * 64 for L in lens]
    worst = _attention_case(0, lens, None, caps, seed=len(lens) + lens[0])
    assert worst < 1.0, worst


@pytest.mark.parametrize("rows", [1, 2])
def test_flash_prefill_rows_per_wavefront(rows):
    _, lib = ops()
    call(lib.q3op_tune(2, rows))
    try:
        for n_q, n_kv in [(16, 8), (16, 2), (8, 1)]:
            lens = [600, 3, 130, 257]
            caps = [((L + 63) // 64) * 64 for L in lens]
            worst = _attention_case(0, lens, None, caps, n_q=n_q, n_kv=n_kv, seed=rows * 10 + n_kv)
            assert worst < 1.0, (rows, n_q, n_kv, worst)
    finally:
        call(lib.q3op_tune(2, -1))


@pytest.mark.parametrize("lens,cached", [
    ([1], [1]), ([5], [64]), ([64], [37]), ([130, 1, 63, 200], [0, 500, 1, 64]),
    ([600, 3, 130, 1100], [2000, 0, 127, 31]), ([1], [8191])])
def test_flash_prefill_attention_continues_cache(lens, cached):
    """Prefill into a cache that already holds `cached` keys per sequence:
    queries at positions cached + i see every cached key and the new ones."""
    caps = [((c + L + 63) // 64) * 64 for L, c in zip(lens, cached)]
    worst = _attention_case(0, lens, None, caps, seed=3 * len(lens) + cached[0], cached=cached)
    assert worst < 1.0, worst


@pytest.mark.parametrize("rows", [1, 2])
def test_flash_prefill_continues_cache_rows_per_wavefront(rows):
    _, lib = ops()
    call(lib.q3op_tune(2, rows))
    try:
        lens, cached = [300, 3, 130], [70, 1000, 0]
        caps = [((c + L + 63) // 64) * 64 for L, c in zip(lens, cached)]
        worst = _attention_case(0, lens, None, caps, seed=rows + 50, cached=cached)
        assert worst < 1.0, (rows, worst)
    finally:
        call(lib.q3op_tune(2, -1))


def test_f32_prefill_attention_continues_cache():
    lens, cached = [5, 70], [3, 130]
    caps = [((c + L + 63) // 64) * 64 for L, c in zip(lens, cached)]
    worst = _attention_case(2, lens, None, caps, seed=9, cached=cached)
    assert worst < 1.0, worst


def test_flash_prefill_gqa_groups():
    for n_q, n_kv in [(8, 8), (16, 2), (8, 1)]:
        worst = _attention_case(0, [70, 9], None, [128, 64], n_q=n_q, n_kv=n_kv, seed=n_kv)
        assert worst < 1.0, (n_q, n_kv, worst)


@pytest.mark.parametrize("prior", [[0], [1], [31], [32], [255, 0, 8319], [32799]])
def test_decode_attention(prior):
    caps = [((p + 1 + 63) // 64) * 64 for p in prior]
    worst = _attention_case(1, [1] * len(prior), prior, caps, seed=prior[0] + 3)
    assert worst < 1.0, worst


def test_decode_attention_split_counts():
    for splits in (1, 3, 64):
        worst = _attention_case(1, [1, 1], [700, 40], [768, 64], seed=splits, splits=splits)
        assert worst < 1.0, (splits, worst)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_attention_f32(mode):
    if mode == "prefill":
        worst = _attention_case(2, [1, 37, 70], None, [64, 64, 128], seed=9)
    else:
        worst = _attention_case(2, [1, 1], [0, 300], [64, 320], seed=10)
    assert worst < 1.0, worst


@pytest.mark.parametrize("epi,M,N", [(EPI_STORE, 1, 4096), (EPI_SWIGLU, 3, 6144), (EPI_ARGMAX, 1, 8192),
                                     (EPI_STORE, 8, 4096), (EPI_SWIGLU, 1, 6144), (EPI_STORE, 17, 4096),
                                     (EPI_SWIGLU, 32, 6144), (EPI_SWIGLU, 64, 6144), (EPI_STORE, 64, 4096),
                                     (EPI_ARGMAX, 40, 8192)])
@pytest.mark.parametrize("kernel", [SKINNY, ROWGEMV])
def test_norm_linear_fused_prologue(kernel, epi, M, N):
    """RMSNorm folded into a decode projection's prologue equals rmsnorm -> bf16 -> projection."""
    if kernel == ROWGEMV and (M != 1 or epi not in (EPI_STORE, EPI_SWIGLU)):
        pytest.skip("the single-row GEMV fuses the norm for one row and epilogues 0 and 2")
    mod, lib = ops()
    rng = np.random.default_rng(50 + M + epi)
    K = 1024
    x = (rng.standard_normal((M, K)) * rng.uniform(0.05, 10, (M, 1))).astype(np.float32)
    g = q3synth.round_to_bf16((1 + 0.1 * rng.standard_normal(K)).astype(np.float32))
    W = rand_bf16(rng, (N, K), 0.02)
    h = to_bf16(rms_norm(x.astype(np.float64), g.astype(np.float64), 1e-6))
    dx, dg, dw = dev_f32(x), dev_f32(g), dev_bf16(W)
    if epi == EPI_SWIGLU:
        out = torch.zeros((M, N // 2), dtype=torch.int16, device="cuda:0")
        ldo = N // 2
    else:
        out = torch.zeros((M, N), dtype=torch.float32, device="cuda:0")
        ldo = N
    nxt = torch.zeros(M, dtype=torch.int32, device="cuda:0")
    ws = _ws(lib.q3op_linear_workspace_bytes(kernel, epi, M, N, K))
    call(lib.q3op_norm_linear(kernel, epi, dx.data_ptr(), M, dg.data_ptr(), 1e-6, dw.data_ptr(), N, K, out.data_ptr(),
                              ldo, nxt.data_ptr(), ws.data_ptr(), ws.numel(), None))
    _sync()
    if epi == EPI_SWIGLU:
        gg = h @ W[0::2].astype(np.float64).T  # not the packed layout: rebuild below
        Wp = W.astype(np.float64)
        gate = np.concatenate([Wp[32 * r:32 * r + 16] for r in range(N // 32)])
        up = np.concatenate([Wp[32 * r + 16:32 * r + 32] for r in range(N // 32)])
        ref = to_bf16(silu(h @ gate.T) * (h @ up.T))
        got = host_bf16(out)
        np.testing.assert_allclose(got, ref, rtol=2 ** -7, atol=1e-6)
        assert np.mean(got == ref) > 0.98
    else:
        ref = h @ W.astype(np.float64).T
        got = out.cpu().numpy()
        # the prologue rounds to bf16 like the oracle; rare one-ulp flips of h allowed
        assert _rel(got, ref) < 5e-3
        assert np.median(np.abs(got - ref)) < 1e-5 * np.sqrt(np.mean(ref ** 2)) + 1e-6
        if epi == EPI_ARGMAX:
            for m in range(M):
                assert nxt.cpu().numpy()[m] == int(np.argmax(got[m]))


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("N,K", [(1024, 2048), (1024, 3072), (4096, 1024)])
def test_rowdot_gemv(M, N, K):
    rng = np.random.default_rng(M * 13 + N + K)
    X = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), 0.02)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    got, _ = _linear(3, EPI_STORE, X, W)
    assert _rel(got, ref) < 2e-5
    base = rng.standard_normal((M, N)).astype(np.float32)
    got, _ = _linear(3, EPI_RESADD, X, W, out_init=base)
    assert _rel(got - base, ref) < 2e-5


@pytest.mark.parametrize("prior,smax", [([0], 0), ([5, 700], 0), ([1500], 0), ([1500, 40], 3), ([32799], 0),
                                        ([2047, 0, 4100], 0), ([31, 32, 33, 63, 64, 65, 95, 127], 1),
                                        ([126, 127, 128, 255, 256, 257], 2),
                                        # 32 ragged sequences: several splits each, launched longest first
                                        ([int(x) for x in np.random.default_rng(5).integers(0, 700, 32)], 0)])
def test_decode_attention_fused_rope_append(prior, smax):
    """QK-Norm + RoPE of the new token, its cache append, and attention over the
    cache, in one kernel, against the oracle's functions."""
    mod, lib = ops()
    rng = np.random.default_rng(sum(prior) + smax)
    n_q, n_kv, n = 16, 8, len(prior)
    units = n_q + 2 * n_kv
    caps = [((p + 1 + 63) // 64) * 64 for p in prior]
    bases, total = _arena(caps, n_kv, 2)
    arena = np.zeros(total, np.float32)
    old_k, old_v = [], []
    for b in range(n):
        K = rand_bf16(rng, (prior[b], n_kv, 128))
        V = rand_bf16(rng, (prior[b], n_kv, 128))
        old_k.append(K)
        old_v.append(V)
        cap = caps[b]
        # every slot past the new position holds NaN: the kernel reads whole
        # 32-key blocks, and what lies past a sequence's end must not leak
        kc = np.full((n_kv, cap, 128), np.nan, np.float32)
        kc[:, :prior[b] + 1, :] = 0.0
        kc[:, :prior[b], :] = K.transpose(1, 0, 2)
        vt = np.full((n_kv, 128, cap), np.nan, np.float32)
        vt[:, :, :prior[b] + 1] = 0.0
        vt[:, :, :prior[b]] = V.transpose(1, 2, 0)
        region = np.concatenate([k_blocks(kc), vt_blocks(vt)])
        arena[bases[b]:bases[b] + region.size] = region
    qkv = rng.standard_normal((n, units * 128)).astype(np.float32)
    qn = q3synth.round_to_bf16((1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    kn = q3synth.round_to_bf16((1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    dkv = dev_bf16(arena)
    dqkv, dqn, dkn = dev_f32(qkv), dev_f32(qn), dev_f32(kn)
    out = torch.zeros((n, n_q, 128), dtype=torch.int16, device="cuda:0")
    max_pos = max(prior) + 1
    ws = _ws(lib.q3op_decode_attn_fused_workspace_bytes(n, n_q, smax, max_pos))
    call(lib.q3op_decode_attn_fused(dqkv.data_ptr(), n, mod.i64_array(bases), mod.i32_array(caps),
                                    mod.i32_array(prior), dkv.data_ptr(), n_q, n_kv, dqn.data_ptr(), dkn.data_ptr(),
                                    1e-6, 1e6, max_pos, smax, out.data_ptr(), ws.data_ptr(), ws.numel(), None))
    _sync()
    got = host_bf16(out)
    kv_got = host_bf16(dkv)
    for b in range(n):
        x = qkv[b].astype(np.float64).reshape(units, 128)[None]
        c, s_ = rope_cos_sin([prior[b]], 128, 1e6)
        q_hat = to_bf16(rope_rotate(rms_norm(x[:, :n_q], qn, 1e-6), c, s_))
        k_new = to_bf16(rope_rotate(rms_norm(x[:, n_q:n_q + n_kv], kn, 1e-6), c, s_))
        v_new = to_bf16(x[:, n_q + n_kv:])
        cap = caps[b]
        region = kv_got[bases[b]:bases[b] + 2 * n_kv * cap * 128]
        Kc = k_logical(region[:n_kv * cap * 128], n_kv, cap)
        Vt = vt_logical(region[n_kv * cap * 128:], n_kv, cap)
        np.testing.assert_allclose(Kc[:, prior[b], :], k_new[0], rtol=2 ** -7, atol=1e-6)
        np.testing.assert_array_equal(Vt[:, :, prior[b]], v_new[0].astype(np.float32))
        keys = np.concatenate([old_k[b].astype(np.float64), k_new], axis=0)
        vals = np.concatenate([old_v[b].astype(np.float64), v_new], axis=0)
        ref = attention_rows(q_hat, keys, vals, np.array([prior[b]]), np.arange(prior[b] + 1))[0]
        rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
        bound = 2.0 ** -8 * np.abs(ref) + 2e-3 * rms
        # the kernel's own new key may differ from the oracle's by one bf16 ulp
        assert float(np.max(np.abs(got[b] - ref) / (bound + 4e-3 * rms))) < 1.0, b


@pytest.mark.parametrize("rows", [1, 2])
def test_flash_prefill_two_tiles_per_block(rows):
    """Blocks of two query tiles (eight wavefronts sharing the key/value
    tiles): odd and even tile counts, ragged tails, continued caches and the
    GQA groupings, against the oracle."""
    _, lib = ops()
    call(lib.q3op_tune(2, rows))
    call(lib.q3op_tune(6, 2))
    try:
        for n_q, n_kv in [(16, 8), (16, 2), (8, 1)]:
            lens = [600, 3, 130, 257, 64, 65]
            caps = [((L + 63) // 64) * 64 for L in lens]
            worst = _attention_case(0, lens, None, caps, n_q=n_q, n_kv=n_kv, seed=rows * 10 + n_kv + 7)
            assert worst < 1.0, (rows, n_q, n_kv, worst)
        lens, cached = [300, 3, 130], [70, 1000, 0]
        caps = [((c + L + 63) // 64) * 64 for L, c in zip(lens, cached)]
        worst = _attention_case(0, lens, None, caps, seed=rows + 70, cached=cached)
        assert worst < 1.0, (rows, worst)
    finally:
        call(lib.q3op_tune(6, -1))
        call(lib.q3op_tune(2, -1))
