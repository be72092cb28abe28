"""Temperature + top-p sampling (Paso 8) on the GPU, through the C ABI,
against the oracle's sampler on the same logits and uniforms.

The sampled token must equal the oracle's unless one of the oracle's decisions
lies within 1e-5 of its threshold, or the two tokens' weights are equal in
float32 (the kernel then orders them by ID, the float64 oracle by value).
Such near-ties are counted: rare for peaked rows, a few per cent of the draws
for nearly flat rows over 151,936 tokens, where each token spans ~7e-6 of the
unit interval and ~1,500 pairs of weights coincide in float32."""
import numpy as np
import pytest
import torch

from gpu_helpers import call, ops, sample_agrees

pytestmark = pytest.mark.gpu


def _run(logits, T, p, u, ld=None):
    mod, lib = ops()
    n, V = logits.shape
    ld = ld or V
    buf = np.zeros((n, ld), np.float32)
    buf[:, :V] = logits
    buf[:, V:] = 1e30  # padding past the row must not be read
    d = torch.from_numpy(buf).to("cuda:0")
    du = torch.from_numpy(np.asarray(u, np.float32)).to("cuda:0")
    nxt = torch.full((n,), -1, dtype=torch.int32, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(lib.q3op_sample_workspace_bytes(n), dtype=torch.uint8, device="cuda:0")
    call(lib.q3op_sample_top_p(d.data_ptr(), n, V, ld, T, p, du.data_ptr(), nxt.data_ptr(), err.data_ptr(),
                               ws.data_ptr(), ws.numel(), None))
    torch.cuda.synchronize()
    return nxt.cpu().numpy(), int(err.item())


def _check_rows(logits, T, p, u, got):
    near = 0
    for r in range(logits.shape[0]):
        ok, tie = sample_agrees(logits[r].astype(np.float64), T, p, float(u[r]), int(got[r]))
        assert ok, (r, T, p, float(u[r]), int(got[r]))
        near += tie
    return near


@pytest.mark.parametrize("V,n,scale", [(1000, 64, 1.0), (151936, 8, 3.0), (151936, 64, 0.05), (77, 5, 10.0),
                                       (1, 3, 1.0)])
@pytest.mark.parametrize("T,p", [(0.7, 0.95), (1.0, 0.9), (1.5, 0.5), (1.0, 1.0), (0.3, 0.0)])
def test_sample_matches_oracle(V, n, scale, T, p):
    rng = np.random.default_rng(V + n + int(T * 10) + int(p * 100))
    logits = (rng.standard_normal((n, V)) * scale).astype(np.float32)
    u = rng.random(n).astype(np.float32)
    got, err = _run(logits, T, p, u, ld=V + 3)
    assert err == 0
    near = _check_rows(logits, T, p, u, got)
    assert near <= max(2, n // 10), near


def test_sample_more_rows_than_one_batch():
    """70 rows: the sampler runs its launches 64 rows at a time."""
    rng = np.random.default_rng(11)
    logits = (rng.standard_normal((70, 5000)) * 2).astype(np.float32)
    u = rng.random(70).astype(np.float32)
    got, err = _run(logits, 0.9, 0.9, u)
    assert err == 0
    near = _check_rows(logits, 0.9, 0.9, u, got)
    assert near <= 2, near


def test_sample_temperature_zero_is_greedy():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((70, 151936)).astype(np.float32)  # more rows than one launch takes
    logits[3, 100] = logits[3, 7] = logits[3].max() + 1  # tie: the lower ID wins
    got, err = _run(logits, 0.0, 0.9, np.zeros(70, np.float32))
    assert err == 0
    np.testing.assert_array_equal(got, np.argmax(logits, axis=1))
    assert got[3] == 7


def test_sample_equal_logits_closed_form():
    """Equal logits: every probability is 1/V, so the nucleus is the first
    k = ceil(top_p * V) IDs and the draw is ID floor(u * k) (one off where
    u * k or top_p * V sits on an integer)."""
    rng = np.random.default_rng(2)
    V, n = 151936, 16
    logits = np.zeros((n, V), np.float32)
    u = rng.random(n).astype(np.float32)
    for p in (0.25, 0.9, 1.0):
        got, err = _run(logits, 1.0, p, u)
        assert err == 0
        k = min(V, int(np.ceil(np.float32(p) * V)))
        want = np.floor(u.astype(np.float64) * k).astype(np.int64)
        assert np.all(np.abs(got - want) <= 1) and np.all(got < k + 1), (p, got, want)


def test_sample_repeated_logit_values():
    """Rows of a few repeated logit values (thousands of exactly equal
    weights per value): the crossing inside a run of equal weights is an index
    count.  Float32 weights shift a running sum over thousands of equal terms
    by a fraction of one token against the float64 oracle, so a draw may land
    one token over; the oracle's choice must still be matched in most draws."""
    rng = np.random.default_rng(7)
    V, n = 151936, 32
    logits = (np.round(rng.standard_normal((n, V)) * 2) / 2).astype(np.float32)
    u = rng.random(n).astype(np.float32)
    exact = total = 0
    for p in (0.25, 0.9, 1.0):
        got, err = _run(logits, 1.0, p, u)
        assert err == 0
        near = _check_rows(logits, 1.0, p, u, got)
        exact += n - near
        total += n
    assert exact >= 0.75 * total, (exact, total)


def test_sample_u_grid_frequencies():
    """One row, 64 copies with uniforms on a regular grid: every kept token
    appears in proportion to its renormalised probability, exactly as the
    oracle's draws on the same grid."""
    rng = np.random.default_rng(3)
    V = 20
    row = (rng.standard_normal(V) * 1.5).astype(np.float32)
    u = ((np.arange(64) + 0.5) / 64).astype(np.float32)
    got, err = _run(np.tile(row, (64, 1)), 0.8, 0.8, u)
    assert err == 0
    near = _check_rows(np.tile(row, (64, 1)), 0.8, 0.8, u, got)
    assert near <= 1


def test_sample_nonfinite_row_raises_error_bit():
    logits = np.zeros((3, 500), np.float32)
    logits[1, 17] = np.nan
    got, err = _run(logits, 1.0, 0.9, np.array([0.5, 0.5, 0.5], np.float32))
    assert err & 2 and got[1] == 0


def test_sample_deterministic():
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((64, 151936)) * 0.5).astype(np.float32)
    u = rng.random(64).astype(np.float32)
    a, _ = _run(logits, 1.0, 0.95, u)
    b, _ = _run(logits, 1.0, 0.95, u)
    np.testing.assert_array_equal(a, b)


def test_sample_rejects_bad_arguments():
    mod, lib = ops()
    x = torch.zeros((2, 10), dtype=torch.float32, device="cuda:0")
    nx = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    e = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    u = torch.zeros(2, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(lib.q3op_sample_workspace_bytes(2), dtype=torch.uint8, device="cuda:0")
    for T, p, ld in [(-1.0, 0.9, 10), (float("nan"), 0.9, 10), (1.0, float("inf"), 10), (1.0, 0.9, 9), (1e-31, 0.9, 10)]:
        st = lib.q3op_sample_top_p(x.data_ptr(), 2, 10, ld, T, p, u.data_ptr(), nx.data_ptr(), e.data_ptr(),
                                   ws.data_ptr(), ws.numel(), None)
        assert st == mod.Q3_E_ARG, (T, p, ld)
    st = lib.q3op_sample_top_p(x.data_ptr(), 2, 10, 10, 1.0, 0.9, None, nx.data_ptr(), e.data_ptr(),
                               ws.data_ptr(), ws.numel(), None)
    assert st == mod.Q3_E_ARG
    st = lib.q3op_sample_top_p(x.data_ptr(), 2, 10, 10, 1.0, 0.9, u.data_ptr(), nx.data_ptr(), e.data_ptr(),
                               ws.data_ptr(), 100, None)
    assert st == mod.Q3_E_ARG
