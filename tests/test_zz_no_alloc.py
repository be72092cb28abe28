"""q3op_linear_noalloc (workspace in the library's static device scratch)
against q3op_linear (workspace passed in), through the C ABI: the same
kernels on the same inputs, so the outputs must be identical, on two calls in
a row with the second smaller, for every kernel family that uses a
workspace; and a call that needs more workspace than the scratch holds is
refused before anything is queued."""
import ctypes as C

import numpy as np
import pytest
import torch

from gpu_helpers import call, ops

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to("cuda:0").to(
        torch.bfloat16).view(torch.int16)


def _run(lib, mod, kernel, epi, x, M, w, N, K, out, nxt, stream, noalloc):
    ldo = N // 2 if epi == 2 else N
    nx = nxt.data_ptr() if nxt is not None else None
    if noalloc:
        call(lib.q3op_linear_noalloc(kernel, epi, x.data_ptr(), M, w.data_ptr(), N, K, out.data_ptr(), ldo, nx,
                                     stream.cuda_stream))
    else:
        n = lib.q3op_linear_workspace_bytes(kernel, epi, M, N, K)
        ws = torch.full((max(256, n),), 0x5A, dtype=torch.uint8, device="cuda:0")
        call(lib.q3op_linear(kernel, epi, x.data_ptr(), M, w.data_ptr(), N, K, out.data_ptr(), ldo, nx,
                             ws.data_ptr(), ws.numel(), stream.cuda_stream))
        torch.cuda.synchronize()


# (kernel, epi, [(M, N, K) of the first call, (M, N, K) of the second, smaller call])
CASES = [
    (1, 1, [(16, 1024, 3072), (5, 1024, 2048)]),     # weight-streaming, residual split over K
    (1, 3, [(8, 32768, 1024), (2, 16384, 1024)]),    # weight-streaming, logits + argmax partials
    (1, 2, [(4, 2048, 1024), (1, 1024, 1024)]),      # weight-streaming, SwiGLU
    (4, 3, [(1, 151936, 1024), (1, 4096, 1024)]),    # single-row GEMV, logits + argmax
    (0, 1, [(512, 1024, 2048), (130, 1024, 1024)]),  # tiled GEMM, residual split over K
]


@pytest.mark.parametrize("kernel,epi,shapes", CASES)
def test_noalloc_matches_linear_twice(kernel, epi, shapes):
    mod, lib = ops()
    rng = np.random.default_rng(100 + 10 * kernel + epi)
    stream = torch.cuda.Stream()
    for (M, N, K) in shapes:
        print(f"noalloc kernel {kernel} epi {epi} M {M} N {N} K {K}", flush=True)
        x = _bf16(rng, (M, K))
        w = _bf16(rng, (N, K), 0.02)
        if epi == 2:
            base = torch.zeros((M, N // 2), dtype=torch.int16, device="cuda:0")
        else:
            base = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to("cuda:0")
        outs, nexts = [], []
        for noalloc in (False, True):
            out = base.clone()
            nxt = torch.full((M,), -1, dtype=torch.int32, device="cuda:0") if epi == 3 else None
            with torch.cuda.stream(stream):
                _run(lib, mod, kernel, epi, x, M, w, N, K, out, nxt, stream, noalloc)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
            nexts.append(None if nxt is None else nxt.cpu().numpy())
        np.testing.assert_array_equal(outs[1], outs[0])
        if epi == 3:
            np.testing.assert_array_equal(nexts[1], nexts[0])
            np.testing.assert_array_equal(nexts[1], np.argmax(outs[1], axis=1))


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    mod, lib = ops()
    M, N, K = 64, 151936 * 16, 1024       # argmax partials alone exceed the scratch
    need = lib.q3op_linear_workspace_bytes(1, 3, M, N, K)
    assert need > (16 << 20)
    st = lib.q3op_linear_noalloc(1, 3, C.c_void_p(16), M, C.c_void_p(16), N, K, C.c_void_p(16), N, None, None)
    assert st == mod.Q3_E_CAPACITY
    assert b"static scratch" in lib.q3_last_error()
