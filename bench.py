"""Benchmark: prefill + greedy decode of the Qwen3-0.6B-shaped decoder on one MI355X.

One step = one pass of the whole path over one request of the workload:
reset the slot, prefill the 512-token prompt (embedding, 28 blocks, final norm,
tied lm_head, argmax), then 256 greedy decode steps, each feeding the previous
step's device-side token back in and writing logits.  Weights are seeded random
bf16 (the page's checkpoint is not used); inputs are resident in HBM before the
timed region starts.

Prints one JSON line.  `value` is decode tokens/s; prefill tokens/s, the
whole-step decode HBM fraction, the dominant kernel's roofline and the CPU
oracle's rate ride along.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
# rows per block of the single-row lm_head kernel (4 per wavefront x 4 wavefronts
# for K = 1024): one (max, index) partial per block
ROWGEMV_ARGMAX_ROWS_PER_BLOCK = 16

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_rowgemv_q06b_traffic.md")
TRAFFIC_SOURCES = ["decoder_only_qwen3_amd/csrc/k_rowgemv.hip", "decoder_only_qwen3_amd/csrc/common.h"]


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for p in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kname, M):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3
    counter summary, or None when there is none for this kernel or its sources
    have changed since the counters were taken."""
    import re
    if M != 1 or not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    dig = re.search(r"sources-sha256: ([0-9a-f]{64})", text)
    byts = re.search(r"traffic-bytes-per-launch: ([0-9.e+]+)", text)
    if not dig or not byts or dig.group(1) != sources_digest():
        return None
    return float(byts.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="q06b_bf16_p512_d256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graphs", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: decode steps sample (temperature + top-p, q3_sample) instead of the greedy pick")
    ap.add_argument("--top-p", type=float, default=0.95)
    ap.add_argument("--weight-bits", type=int, default=0, choices=[0, 8, 4],
                    help="8 or 4: block projections stored as affine group codes (weight-only quantization)")
    ap.add_argument("--checkpoint-load", action="store_true",
                    help="also time q3_load_safetensors on the workload's weights written as a safetensors file")
    return ap.parse_args()


def decode_bytes_per_step(d, ctxs, weight_bits=0):
    """Algorithmic HBM bytes of one decode step of len(ctxs) sequences, sequence b
    attending over ctxs[b] keys (its new token included): every weight once, each
    sequence's cache read, the new keys/values written, one logits row each.
    Quantized projections count bits/8 + 4/64 bytes per weight (codes plus the
    fp16 scale and offset of each group of 64)."""
    L, H, Q, KV, I, V = d.n_layers, d.hidden, d.n_q_heads * 128, d.n_kv_heads * 128, d.ffn, d.vocab
    e = 2 if d.dtype == "bf16" else 4
    B = len(ctxs)
    pe = (weight_bits / 8 + 4 / 64) if weight_bits else e
    weights = L * (H * (Q + 2 * KV) + Q * H + 2 * I * H + I * H) * pe + V * H * e
    norms = (L * (2 * H + 256) + H) * 4
    kv_read = sum(ctxs) * L * 2 * KV * e
    kv_write = B * L * 2 * KV * e
    logits = B * V * 4
    return weights + norms + kv_read + kv_write + logits


def prefill_flops(d, lens, calls=1):
    """Prefill FLOPs of the prompts `lens`, split into `calls` calls (each call
    ends with the head on every sequence's last row; attention is the same)."""
    L, H, Q, KV, I, V = d.n_layers, d.hidden, d.n_q_heads * 128, d.n_kv_heads * 128, d.ffn, d.vocab
    per_tok = 2 * L * (H * (Q + 2 * KV) + Q * H + 3 * I * H)
    attn = sum(4 * d.n_q_heads * 128 * L * n * (n + 1) // 2 for n in lens)
    head = 2 * V * H * len(lens) * calls
    return per_tok * sum(lens) + attn + head


def cpu_baseline(d, w, prompt, seconds_budget=12.0, max_steps=600):
    """Time the CPU oracle (float64 numpy) on a bounded sample: a short prefill,
    then greedy decode steps for about `seconds_budget` seconds."""
    from oracle import OracleModel
    cores = len(os.sched_getaffinity(0))
    m = OracleModel(d, w)
    n_prompt = 16
    cache = m.new_cache(n_prompt + max_steps)
    t0 = time.perf_counter()
    lg = m.forward(prompt[:n_prompt], cache)[0]   # also converts the weights to float64 once
    t1 = time.perf_counter()
    tok = int(np.argmax(lg))
    steps, t_dec = 0, 0.0
    while steps < max_steps and (steps < 2 or t_dec < seconds_budget):
        s0 = time.perf_counter()
        tok = int(np.argmax(m.forward([tok], cache)[0]))
        t_dec += time.perf_counter() - s0
        steps += 1
    return {"value": steps / t_dec, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle, {d.n_layers} layers: {n_prompt}-token prefill "
                      f"({t1 - t0:.1f} s incl. one-time float64 weight conversion) then {steps} "
                      f"greedy decode steps timed ({t_dec:.1f} s)"}


def checkpoint_load(m, w, d):
    """Seconds and GB/s of q3_load_safetensors for the weights written as one
    safetensors file (read back from the page cache: host memory -> HBM)."""
    import tempfile

    import torch
    from safetensors.torch import save_file
    dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32
    with tempfile.TemporaryDirectory(dir="/tmp") as td:
        path = os.path.join(td, "model.safetensors")
        save_file({k: torch.from_numpy(v).to(dt) for k, v in w.items()}, path)
        size = os.path.getsize(path)
        m.load_safetensors([path])  # warm: file in the page cache
        t0 = time.perf_counter()
        m.load_safetensors([path])
        sec = time.perf_counter() - t0
    return {"bytes": size, "seconds": round(sec, 3), "GBs": round(size / sec / 1e9, 2),
            "source": "page cache"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import q3synth
    from decoder_only_qwen3_amd import Q3Model, _lib

    wl = q3synth.WORKLOADS[args.workload]
    d = wl.dims
    lens = [int(x) for x in wl.prompt_lengths()]
    steps_dec = wl.decode_steps
    B = wl.n_seqs
    t_gen = time.perf_counter()
    w = q3synth.make_weights(d, wl.seed)
    prompts = [q3synth.make_tokens(L, d.vocab, wl.seed + 1 + i).tolist() for i, L in enumerate(lens)]
    t_gen = time.perf_counter() - t_gen

    cap = max(lens) + steps_dec
    # Chunked workloads prefill every prompt in calls of wl.chunk tokens.
    if wl.chunk > 0 and len(set(lens)) != 1:
        raise SystemExit("chunked workloads need equal prompt lengths")
    bounds = ([(a, min(a + wl.chunk, lens[0])) for a in range(0, lens[0], wl.chunk)] if wl.chunk > 0
              else [(0, None)])
    max_call = sum(lens) if wl.chunk <= 0 else B * wl.chunk
    m = Q3Model(d, max_slots=B, max_positions=cap, max_prefill_tokens=max_call, kv_tokens=B * ((cap + 63) // 64 * 64),
                weight_bits=args.weight_bits)
    m.load_weights(w)
    if args.no_graphs:
        m.set_graphs(False)
    slots = list(range(B))
    for s in slots:
        m.seq_alloc(s, cap)
    dev = m.device
    calls = []  # (cu_seqlens, device tokens) of each prefill call
    with torch.cuda.stream(m.stream):
        for a, b in bounds:
            parts = [np.asarray(p[a:b], np.int32) for p in prompts]
            cu = np.concatenate([[0], np.cumsum([len(x) for x in parts])]).astype(np.int32)
            calls.append((cu, torch.from_numpy(np.concatenate(parts)).to(dev)))
        d_tok = [torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(2)]
        d_greedy = torch.zeros(B, dtype=torch.int32, device=dev)
        # one uniform number per sequence and step, drawn before any timing
        g = torch.Generator(device=dev).manual_seed(wl.seed)
        d_unif = torch.rand((max(steps_dec, 1), B), generator=g, device=dev, dtype=torch.float32)
        d_logits = torch.empty((B, d.vocab), dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def one_step():
        m.seq_reset(slots)
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(m.stream)
        for cu, d_prompt in calls:
            m.prefill_raw(slots, cu, d_prompt, d_logits, d_tok[0])
        e1.record(m.stream)
        for i in range(steps_dec):
            if args.temperature > 0:
                m.decode_raw(slots, d_tok[i % 2], d_logits, d_greedy)
                _lib.check(m.lib.q3_sample(m.handle, B, d_logits.data_ptr(), d.vocab, args.temperature, args.top_p,
                                           d_unif[i].data_ptr(), d_tok[(i + 1) % 2].data_ptr(), m.sh))
            else:
                m.decode_raw(slots, d_tok[i % 2], d_logits, d_tok[(i + 1) % 2])
        e2.record(m.stream)
        return e0, e1, e2

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    if m.error_flags() != 0:
        raise RuntimeError("device error flags raised during warmup")
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        marks.append(one_step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [a.elapsed_time(b) for a, b, _ in marks]
    dec_ms = [b.elapsed_time(c) for _, b, c in marks]
    prefill_tok_s = sum(lens) * args.steps / (sum(pre_ms) / 1e3)
    decode_tok_s = B * steps_dec * args.steps / (sum(dec_ms) / 1e3)

    # Whole-step decode HBM fraction: algorithmic bytes averaged over the steps.
    byts = np.mean([decode_bytes_per_step(d, [L + 1 + i for L in lens], args.weight_bits) for i in range(steps_dec)])
    dec_step_s = (sum(dec_ms) / 1e3) / (args.steps * steps_dec)
    decode_hbm = {"bytes_per_step": float(byts), "achieved_GBs": byts / dec_step_s / 1e9,
                  "frac": byts / dec_step_s / 1e9 / HBM_PEAK_GBS}
    pf = prefill_flops(d, lens, len(calls))
    prefill_mfma = {"flops": pf, "achieved_TFLOPs": pf / (np.mean(pre_ms) / 1e3) / 1e12,
                    "frac": pf / (np.mean(pre_ms) / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}

    # Roofline kernel: the tied lm_head weight stream, the largest single transfer
    # of a decode step (151936 x 1024 bf16 = 311 MB per launch), in the kernel the
    # step itself uses (single-row GEMV for one sequence, the weight-streaming
    # MFMA kernel for several).  Timed with HIP events on the model's stream over
    # repeated launches on the model's own embedding table.
    lib = _lib.load()
    M = B
    N, K = d.vocab, d.hidden
    kern = 4 if M == 1 else 1
    with torch.cuda.stream(m.stream):
        x = torch.zeros((M, K), dtype=torch.int16, device=dev)
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
        wsb = lib.q3op_linear_workspace_bytes(kern, 3, M, N, K)
        ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev)
    embed_ptr = m.bufs[0].data_ptr()  # the embedding table sits at offset 0 of the weight region
    # d_next = NULL: only the lm_head kernel itself (logits + per-block partials) is launched
    for _ in range(3):
        _lib.check(lib.q3op_linear(kern, 3, x.data_ptr(), M, embed_ptr, N, K, out.data_ptr(), N, None,
                                   ws.data_ptr(), ws.numel(), m.sh))
    k0, k1 = ev(), ev()
    k0.record(m.stream)
    for _ in range(args.kernel_reps):
        _lib.check(lib.q3op_linear(kern, 3, x.data_ptr(), M, embed_ptr, N, K, out.data_ptr(), N, None,
                                   ws.data_ptr(), ws.numel(), m.sh))
    k1.record(m.stream)
    torch.cuda.synchronize()
    per_launch_ms = k0.elapsed_time(k1) / args.kernel_reps
    # A plain 256 MiB device copy: the reference that scales the profiler's
    # FETCH_SIZE / WRITE_SIZE counters to bytes (see the profiles directory).
    with torch.cuda.stream(m.stream):
        c_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        c_dst = torch.empty_like(c_src)
        c_dst.copy_(c_src)
    torch.cuda.synchronize()
    del c_src, c_dst
    parts = ROWGEMV_ARGMAX_ROWS_PER_BLOCK if M == 1 else 16
    alg_bytes = N * K * 2 + M * K * 2 + M * N * 4 + ((N + parts - 1) // parts) * M * 8
    achieved = alg_bytes / (per_launch_ms / 1e3) / 1e9
    kname = ("rowgemv_kernel<EPI_ARGMAX> (lm_head + argmax partials, M=1)" if M == 1 else
             "skinny_kernel<EPI_ARGMAX> (lm_head + argmax partials, M=%d)" % M)
    traffic = measured_traffic(kname, M)

    line = {
        "metric": "decode tok/s + prefill tok/s (1 GPU) and % of HBM / bf16-MFMA roofline",
        "value": round(decode_tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d.dtype == "bf16" else "f32",
        "data": "synthetic: seeded N(0,0.02) weights (norms 1+N(0,0.1)), uniform random token IDs",
        "config": {"workload": wl.name, "n_layers": d.n_layers, "n_seqs": B, "prompt_tokens": lens if B <= 4 else sum(lens),
                   "decode_steps": steps_dec, "graphs": not args.no_graphs,
                   **({"prefill_chunk": wl.chunk} if wl.chunk > 0 else {}),
                   **({"sampling": {"temperature": args.temperature, "top_p": args.top_p}}
                      if args.temperature > 0 else {}),
                   **({"weight_bits": args.weight_bits} if args.weight_bits else {})},
        "prefill_tok_s": round(prefill_tok_s, 1),
        "decode_tok_s": round(decode_tok_s, 2),
        "prefill_ms": round(float(np.mean(pre_ms)), 3),
        "decode_ms_per_token_step": round(float(np.mean(dec_ms)) / steps_dec, 4),
        "decode_hbm": decode_hbm,
        "prefill_mfma": prefill_mfma,
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "per_launch_us": round(per_launch_ms * 1e3, 2), "alg_bytes": alg_bytes},
        "host_setup_s": round(t_gen, 1),
    }
    if args.checkpoint_load:
        line["checkpoint_load"] = checkpoint_load(m, w, d)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d, w, prompts[0])
    m.close()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
