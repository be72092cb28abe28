"""Single-kernel timing harness (HIP events) for libq3's kernels at the
Qwen3-0.6B shapes, through the entry points of include/q3_ops.h.

    python -m decoder_only_qwen3_amd.kbench [--kernels lm_head,qkv,...] [--reps 50]

Prints one JSON object per kernel: average launch time, algorithmic bytes or
FLOPs per launch and the achieved rate against the MI355X peak (HBM 8 TB/s,
dense bf16 MFMA 2.5 PFLOP/s).  It also runs one 256 MiB device copy, the
reference for scaling profiler byte counters.  Inputs are random (the
numbers produced are not checked here; the parity tests do that).
"""
from __future__ import annotations

import argparse
import json

import numpy as np
import torch

from . import _lib

HBM = 8000.0
MFMA = 2500.0
H, Q, KVW, I, V = 1024, 2048, 1024, 3072, 151936


def _rand_bf16(shape, scale=1.0):
    return (torch.randn(shape, device="cuda:0") * scale).to(torch.bfloat16).view(torch.int16)


def _time(fn, reps, stream):
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3  # microseconds


def linear_case(lib, name, epi, M, N, K, reps, stream, kernel=1, norm=False, pool=1):
    """`pool` > 1 cycles through that many copies of the weight matrix, so
    that they are not all resident in the GPU's caches."""
    if norm:
        x = torch.randn((M, K), device="cuda:0")
        g = 1 + 0.1 * torch.randn(K, device="cuda:0")
    else:
        x = _rand_bf16((M, K))
    ws_ = [_rand_bf16((N, K), 0.02) for _ in range(pool)]
    if epi == 2:
        out = torch.empty((M, N // 2), dtype=torch.int16, device="cuda:0")
        ldo = N // 2
    else:
        out = torch.zeros((M, N), dtype=torch.float32, device="cuda:0")
        ldo = N
    nxt = torch.zeros(max(M, 1), dtype=torch.int32, device="cuda:0")
    ws = torch.zeros(max(256, lib.q3op_linear_workspace_bytes(kernel, epi, M, N, K)), dtype=torch.uint8,
                     device="cuda:0")
    sh = stream.cuda_stream
    it = [0]

    def fn():
        w = ws_[it[0] % pool]
        it[0] += 1
        nx = nxt.data_ptr() if (epi == 3 and kernel != 1) else None
        if norm:
            _lib.check(lib.q3op_norm_linear(kernel, epi, x.data_ptr(), M, g.data_ptr(), 1e-6, w.data_ptr(), N, K,
                                            out.data_ptr(), ldo, nx, ws.data_ptr(), ws.numel(), sh))
        else:
            _lib.check(lib.q3op_linear(kernel, epi, x.data_ptr(), M, w.data_ptr(), N, K, out.data_ptr(), ldo, nx,
                                       ws.data_ptr(), ws.numel(), sh))
    us = _time(fn, reps, stream)
    if kernel != 0:
        out_b = M * N * 4 if epi != 2 else M * (N // 2) * 2
        byts = N * K * 2 + M * K * (8 if norm else 2) + out_b + (M * N * 4 if epi == 1 else 0)
        return {"kernel": name, "M": M, "N": N, "K": K, "us": round(us, 2), "bytes": byts,
                "GBs": round(byts / us / 1e3, 1), "hbm_frac": round(byts / us / 1e3 / HBM, 4)}
    fl = 2 * M * N * K
    return {"kernel": name, "M": M, "N": N, "K": K, "us": round(us, 2), "flops": fl,
            "TFLOPs": round(fl / us / 1e6, 1), "mfma_frac": round(fl / us / 1e6 / MFMA, 4)}


def attention_case(lib, name, kernel, L, B, reps, stream):
    n_q, n_kv = 16, 8
    cap = (L + 1 + 63) // 64 * 64
    region = 2 * n_kv * cap * 128
    kv = _rand_bf16((B * region,))
    bases = [b * region for b in range(B)]
    if kernel == 0:
        cu = [b * L for b in range(B + 1)]
        q = _rand_bf16((B * L, n_q, 128))
        out = torch.empty_like(q)
        lens, decode = [0] * B, 0
    else:
        cu = list(range(B + 1))
        q = _rand_bf16((B, n_q, 128))
        out = torch.empty_like(q)
        lens, decode = [L] * B, 1
    ws_bytes = lib.q3op_attention_workspace_bytes(kernel, B, int(cu[-1]), n_q, n_kv, 0)
    ws = torch.zeros(max(256, ws_bytes), dtype=torch.uint8, device="cuda:0")
    sh = stream.cuda_stream
    a_cu, a_b, a_c, a_l = _lib.i32_array(cu), _lib.i64_array(bases), _lib.i32_array([cap] * B), _lib.i32_array(lens)

    def fn():
        _lib.check(lib.q3op_attention(kernel, q.data_ptr(), B, a_cu, decode, a_b, a_c, a_l, kv.data_ptr(),
                                      n_q, n_kv, 0, out.data_ptr(), ws.data_ptr(), ws.numel(), sh))
    us = _time(fn, reps, stream)
    if kernel == 0:
        fl = B * 4 * n_q * 128 * L * (L + 1) // 2
        return {"kernel": name, "L": L, "B": B, "us": round(us, 2), "flops": fl,
                "TFLOPs": round(fl / us / 1e6, 1), "mfma_frac": round(fl / us / 1e6 / MFMA, 4)}
    byts = B * (L + 1) * n_kv * 128 * 2 * 2
    return {"kernel": name, "ctx": L + 1, "B": B, "us": round(us, 2), "bytes": byts,
            "GBs": round(byts / us / 1e3, 1), "hbm_frac": round(byts / us / 1e3 / HBM, 4)}


def flash_ragged_case(lib, name, lens, reps, stream):
    """Prefill attention over packed prompts of lengths `lens` (fresh slots)."""
    n_q, n_kv = 16, 8
    B = len(lens)
    caps = [(L + 63) // 64 * 64 for L in lens]
    regions = [2 * n_kv * c * 128 for c in caps]
    bases = [0]
    for r in regions[:-1]:
        bases.append(bases[-1] + r)
    kv = _rand_bf16((sum(regions),))
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    q = _rand_bf16((cu[-1], n_q, 128))
    out = torch.empty_like(q)
    ws_bytes = lib.q3op_attention_workspace_bytes(0, B, int(cu[-1]), n_q, n_kv, 0)
    ws = torch.zeros(max(256, ws_bytes), dtype=torch.uint8, device="cuda:0")
    a_cu, a_b, a_c, a_l = _lib.i32_array(cu), _lib.i64_array(bases), _lib.i32_array(caps), _lib.i32_array([0] * B)

    def fn():
        _lib.check(lib.q3op_attention(0, q.data_ptr(), B, a_cu, 0, a_b, a_c, a_l, kv.data_ptr(), n_q, n_kv, 0,
                                      out.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream))
    us = _time(fn, reps, stream)  # includes the op's value staging; use a kernel trace for the kernel
    fl = sum(4 * n_q * 128 * L * (L + 1) // 2 for L in lens)
    return {"kernel": name, "B": B, "tokens": cu[-1], "us_call": round(us, 2), "flops": fl}


def fused_attn_case(lib, name, lens, reps, stream, smax, pool=1):
    """Fused decode attention (QK-Norm, RoPE, append, split attention) over
    sequences with contexts `lens` (+1 new key each); bytes = cache read.
    `pool` > 1 cycles through that many copies of the cache (cold reads)."""
    n_q, n_kv = 16, 8
    B = len(lens)
    caps = [(L + 1 + 63) // 64 * 64 for L in lens]
    regions = [2 * n_kv * c * 128 for c in caps]
    bases = [0]
    for r in regions[:-1]:
        bases.append(bases[-1] + r)
    kvs = [_rand_bf16((sum(regions),)) for _ in range(pool)]
    it = [0]
    qkv = torch.randn((B, (n_q + 2 * n_kv) * 128), dtype=torch.float32, device="cuda:0")
    qn = torch.ones(128, dtype=torch.float32, device="cuda:0")
    out = torch.empty((B, n_q, 128), dtype=torch.int16, device="cuda:0")
    max_pos = max(caps)
    ws_bytes = lib.q3op_decode_attn_fused_workspace_bytes(B, n_q, smax, max_pos)
    ws = torch.zeros(max(256, ws_bytes), dtype=torch.uint8, device="cuda:0")
    a_b, a_c, a_l = _lib.i64_array(bases), _lib.i32_array(caps), _lib.i32_array(lens)

    def fn():
        kv = kvs[it[0] % pool]
        it[0] += 1
        _lib.check(lib.q3op_decode_attn_fused(qkv.data_ptr(), B, a_b, a_c, a_l, kv.data_ptr(), n_q, n_kv,
                                              qn.data_ptr(), qn.data_ptr(), 1e-6, 1e6, max_pos, smax,
                                              out.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream))
    us = _time(fn, reps, stream)  # includes the op's host-side table upload; use a kernel trace for the kernel
    byts = sum(L + 1 for L in lens) * n_kv * 128 * 2 * 2
    return {"kernel": name, "B": B, "keys": sum(L + 1 for L in lens), "smax": smax, "us_call": round(us, 2),
            "bytes": byts}


def sample_case(lib, name, n, reps, stream, scale=1.0):
    """Temperature + top-p sampling of n vocabulary-wide logit rows (T 0.8,
    top_p 0.95); bytes = one read of the logits."""
    logits = torch.randn((n, V), dtype=torch.float32, device="cuda:0") * scale
    u = torch.rand(n, dtype=torch.float32, device="cuda:0")
    nxt = torch.empty(n, dtype=torch.int32, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(lib.q3op_sample_workspace_bytes(n), dtype=torch.uint8, device="cuda:0")

    def fn():
        _lib.check(lib.q3op_sample_top_p(logits.data_ptr(), n, V, V, 0.8, 0.95, u.data_ptr(), nxt.data_ptr(),
                                         err.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream))
    us = _time(fn, reps, stream)
    byts = n * V * 4
    return {"kernel": name, "rows": n, "us": round(us, 2), "bytes": byts, "GBs": round(byts / us / 1e3, 1),
            "hbm_frac": round(byts / us / 1e3 / HBM, 4)}


def qlinear_case(lib, name, bits, epi, N, K, reps, stream, norm=False, pool=32):
    """Single-row GEMV on quantized weights (codes + fp16 scale/offset per 64),
    weights cycled through `pool` copies; bytes = codes + scales + activations
    + outputs."""
    codes = [torch.randint(0, 256, (N * K * bits // 8,), dtype=torch.uint8, device="cuda:0") for _ in range(pool)]
    # scale 2^-8 and offset -2^-7 in every group (float16 bits, scale low)
    word = int(np.array([0x1c00 | (0xa000 << 16)], dtype=np.uint32).view(np.int32)[0])
    sb = [torch.full((N * (K // 64),), word, dtype=torch.int32, device="cuda:0") for _ in range(pool)]
    x = (torch.randn(K, device="cuda:0") if norm else torch.randn(K, device="cuda:0").to(torch.bfloat16))
    g = torch.ones(K, device="cuda:0")
    out = torch.zeros(N // 2 if epi == 2 else N, dtype=torch.int16 if epi == 2 else torch.float32, device="cuda:0")
    it = [0]

    def fn():
        i = it[0] % pool
        it[0] += 1
        _lib.check(lib.q3op_qlinear(bits, epi, x.data_ptr(), codes[i].data_ptr(), sb[i].data_ptr(), N, K,
                                    g.data_ptr() if norm else None, 1e-6, out.data_ptr(), stream.cuda_stream))
    us = _time(fn, reps, stream)
    byts = N * K * bits // 8 + N * (K // 64) * 4 + K * (4 if norm else 2) + (N // 2 * 2 if epi == 2 else N * 4)
    return {"kernel": name, "bits": bits, "N": N, "K": K, "us": round(us, 2), "bytes": byts,
            "GBs": round(byts / us / 1e3, 1), "hbm_frac": round(byts / us / 1e3 / HBM, 4)}


class ARGS:  # command-line settings the cases read
    attn_smax = 0


def _ragged(n, lo, hi, seed):
    g = torch.Generator().manual_seed(seed)
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=g)]


CASES = {
    # batch-1 decode projections as the decode step runs them, weights cycled
    # through 32 copies (beyond the GPU's last-level cache)
    "row_qkv": lambda lib, r, s: linear_case(lib, "row_qkv", 0, 1, Q + 2 * KVW, H, r, s, kernel=4, norm=True, pool=32),
    "row_o": lambda lib, r, s: linear_case(lib, "row_o", 1, 1, H, Q, r, s, kernel=4, pool=32),
    "row_gate_up": lambda lib, r, s: linear_case(lib, "row_gate_up", 2, 1, 2 * I, H, r, s, kernel=4, norm=True,
                                                 pool=32),
    "row_down": lambda lib, r, s: linear_case(lib, "row_down", 1, 1, H, I, r, s, kernel=4, pool=32),
    "row_lm_head": lambda lib, r, s: linear_case(lib, "row_lm_head", 3, 1, V, H, r, s, kernel=4, pool=2),
    "sk_qkv": lambda lib, r, s: linear_case(lib, "sk_qkv", 0, 1, Q + 2 * KVW, H, r, s, kernel=1, norm=True, pool=32),
    "sk_gate_up": lambda lib, r, s: linear_case(lib, "sk_gate_up", 2, 1, 2 * I, H, r, s, kernel=1, norm=True, pool=32),
    # the batched decode projections at 64 rows (weight-streaming kernel, cold weights)
    "sk64_qkv": lambda lib, r, s: linear_case(lib, "sk64_qkv", 0, 64, Q + 2 * KVW, H, r, s, kernel=1, pool=32),
    "sk64_o": lambda lib, r, s: linear_case(lib, "sk64_o", 1, 64, H, Q, r, s, kernel=1, pool=32),
    "sk64_gate_up": lambda lib, r, s: linear_case(lib, "sk64_gate_up", 2, 64, 2 * I, H, r, s, kernel=1, pool=32),
    "sk64_down": lambda lib, r, s: linear_case(lib, "sk64_down", 1, 64, H, I, r, s, kernel=1, pool=32),
    "rd_o": lambda lib, r, s: linear_case(lib, "rd_o", 1, 1, H, Q, r, s, kernel=3, pool=32),
    "rd_down": lambda lib, r, s: linear_case(lib, "rd_down", 1, 1, H, I, r, s, kernel=3, pool=32),
    "sk_lm_head": lambda lib, r, s: linear_case(lib, "sk_lm_head", 3, 1, V, H, r, s, kernel=1, pool=2),
    "lm_head": lambda lib, r, s: linear_case(lib, "lm_head", 3, 1, V, H, r, s),
    "qkv": lambda lib, r, s: linear_case(lib, "qkv", 0, 1, Q + 2 * KVW, H, r, s),
    "o": lambda lib, r, s: linear_case(lib, "o", 1, 1, H, Q, r, s),
    "gate_up": lambda lib, r, s: linear_case(lib, "gate_up", 2, 1, 2 * I, H, r, s),
    "down": lambda lib, r, s: linear_case(lib, "down", 1, 1, H, I, r, s),
    "lm_head_b64": lambda lib, r, s: linear_case(lib, "lm_head_b64", 3, 64, V, H, r, s),
    # batched lm_head on the streaming kernel (the decode step's choice for 2-64 rows)
    "head_b64": lambda lib, r, s: linear_case(lib, "head_b64", 3, 64, V, H, r, s, kernel=5, pool=2),
    "head_b32": lambda lib, r, s: linear_case(lib, "head_b32", 3, 32, V, H, r, s, kernel=5, pool=2),
    "head_b8": lambda lib, r, s: linear_case(lib, "head_b8", 3, 8, V, H, r, s, kernel=5, pool=2),
    "sk_head_b32": lambda lib, r, s: linear_case(lib, "sk_head_b32", 3, 32, V, H, r, s, kernel=1, pool=2),
    "sk_head_b8": lambda lib, r, s: linear_case(lib, "sk_head_b8", 3, 8, V, H, r, s, kernel=1, pool=2),
    "gemm_qkv_32k": lambda lib, r, s: linear_case(lib, "gemm_qkv_32k", 0, 32768, Q + 2 * KVW, H, r, s, kernel=0),
    "gemm_gate_up_32k": lambda lib, r, s: linear_case(lib, "gemm_gate_up_32k", 2, 32768, 2 * I, H, r, s, kernel=0),
    "gemm_down_32k": lambda lib, r, s: linear_case(lib, "gemm_down_32k", 1, 32768, H, I, r, s, kernel=0),
    "gemm_qkv_512": lambda lib, r, s: linear_case(lib, "gemm_qkv_512", 0, 512, Q + 2 * KVW, H, r, s, kernel=0),
    "gemm_o_512": lambda lib, r, s: linear_case(lib, "gemm_o_512", 1, 512, H, Q, r, s, kernel=0),
    "gemm_gate_up_512": lambda lib, r, s: linear_case(lib, "gemm_gate_up_512", 2, 512, 2 * I, H, r, s, kernel=0),
    "gemm_down_512": lambda lib, r, s: linear_case(lib, "gemm_down_512", 1, 512, H, I, r, s, kernel=0),
    "gemm_qkv_4k": lambda lib, r, s: linear_case(lib, "gemm_qkv_4k", 0, 4096, Q + 2 * KVW, H, r, s, kernel=0),
    "gemm_o_4k": lambda lib, r, s: linear_case(lib, "gemm_o_4k", 1, 4096, H, Q, r, s, kernel=0),
    "gemm_gate_up_4k": lambda lib, r, s: linear_case(lib, "gemm_gate_up_4k", 2, 4096, 2 * I, H, r, s, kernel=0),
    "gemm_down_4k": lambda lib, r, s: linear_case(lib, "gemm_down_4k", 1, 4096, H, I, r, s, kernel=0),
    "sample_b1": lambda lib, r, s: sample_case(lib, "sample_b1", 1, r, s),
    "sample_b64": lambda lib, r, s: sample_case(lib, "sample_b64", 64, r, s),
    "sample_b64_flat": lambda lib, r, s: sample_case(lib, "sample_b64_flat", 64, r, s, scale=0.01),
    "q8_qkv": lambda lib, r, s: qlinear_case(lib, "q8_qkv", 8, 0, Q + 2 * KVW, H, r, s, norm=True),
    "q8_o": lambda lib, r, s: qlinear_case(lib, "q8_o", 8, 1, H, Q, r, s),
    "q8_gate_up": lambda lib, r, s: qlinear_case(lib, "q8_gate_up", 8, 2, 2 * I, H, r, s, norm=True),
    "q8_down": lambda lib, r, s: qlinear_case(lib, "q8_down", 8, 1, H, I, r, s),
    "q4_qkv": lambda lib, r, s: qlinear_case(lib, "q4_qkv", 4, 0, Q + 2 * KVW, H, r, s, norm=True),
    "q4_o": lambda lib, r, s: qlinear_case(lib, "q4_o", 4, 1, H, Q, r, s),
    "q4_gate_up": lambda lib, r, s: qlinear_case(lib, "q4_gate_up", 4, 2, 2 * I, H, r, s, norm=True),
    "q4_down": lambda lib, r, s: qlinear_case(lib, "q4_down", 4, 1, H, I, r, s),
    "flash_512": lambda lib, r, s: attention_case(lib, "flash_512", 0, 512, 1, r, s),
    # the headline workload's packed prefill: its 64 prompts of U[128, 8192] tokens
    "flash_ragged64": lambda lib, r, s: flash_ragged_case(lib, "flash_ragged64", _ragged_prompts(), max(2, r // 10), s),
    "flash_32k": lambda lib, r, s: attention_case(lib, "flash_32k", 0, 32768, 1, max(2, r // 10), s),
    "decode_attn_32k": lambda lib, r, s: attention_case(lib, "decode_attn_32k", 1, 32799, 1, r, s),
    "decode_attn_b64_8k": lambda lib, r, s: attention_case(lib, "decode_attn_b64_8k", 1, 8191, 64, r, s),
    # fused decode attention at batched shapes; --attn-smax sets the split count
    "fused_b64_ragged": lambda lib, r, s: fused_attn_case(lib, "fused_b64_ragged", _ragged(64, 128, 8192, 7), r, s,
                                                          ARGS.attn_smax),
    "fused_b64_uniform": lambda lib, r, s: fused_attn_case(lib, "fused_b64_uniform", [4160] * 64, r, s,
                                                           ARGS.attn_smax),
    "fused_b1_640": lambda lib, r, s: fused_attn_case(lib, "fused_b1_640", [640], r, s, ARGS.attn_smax),
    # one 32K-token sequence (the long-context workload's decode), three cache copies cycled (cold reads)
    "fused_b1_32k": lambda lib, r, s: fused_attn_case(lib, "fused_b1_32k", [32799], r, s, ARGS.attn_smax, pool=3),
    "fused_b32_2k": lambda lib, r, s: fused_attn_case(lib, "fused_b32_2k", [2112] * 32, r, s, ARGS.attn_smax, pool=3),
    # the headline workload's final decode state: the 64 ragged prompts of
    # the benchmark plus 128 decoded keys each, two arenas cycled (cold reads)
    "fused_ragged64_final": lambda lib, r, s: fused_attn_case(lib, "fused_ragged64_final", _ragged_final(), r, s,
                                                              ARGS.attn_smax, pool=2),
}


def _ragged_prompts():
    import q3synth
    return [int(L) for L in q3synth.WORKLOADS["q06b_bf16_b64_ragged_d128"].prompt_lengths()]


def _ragged_final():
    import q3synth
    wl = q3synth.WORKLOADS["q06b_bf16_b64_ragged_d128"]
    return [int(L) + wl.decode_steps for L in wl.prompt_lengths()]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernels", default="lm_head,qkv,o,gate_up,down")
    ap.add_argument("--reps", type=int, default=50)
    ap.add_argument("--gemm-tiles", type=int, default=-1, help="prefill GEMM tile configuration (-1 automatic)")
    ap.add_argument("--flash-rows", type=int, default=-1, help="prefill attention rows per wavefront / 16")
    ap.add_argument("--row-plan", type=int, default=-1, help="single-row GEMV: rows + 256 * wavefronts per block")
    ap.add_argument("--attn-smax", type=int, default=0, help="fused decode attention splits (0 = library choice)")
    ap.add_argument("--flash-tiles", type=int, default=-1, help="prefill attention query tiles per block (1, 2)")
    args = ap.parse_args()
    ARGS.attn_smax = args.attn_smax
    lib = _lib.load()
    _lib.check(lib.q3op_tune(1, args.gemm_tiles))
    _lib.check(lib.q3op_tune(2, args.flash_rows))
    _lib.check(lib.q3op_tune(3, args.row_plan))
    _lib.check(lib.q3op_tune(6, args.flash_tiles))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for k in args.kernels.split(","):
            print(json.dumps(CASES[k](lib, args.reps, stream)), flush=True)
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "copy_calibration", "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4}))


if __name__ == "__main__":
    main()
