"""Benchmark: prefill + greedy decode of the Qwen3-0.6B-shaped decoder on one MI355X.

One step = one pass of the whole path over one batch of the workload: reset
the slots, prefill every prompt (embedding, 28 blocks, final norm, tied
lm_head, argmax), then the workload's greedy decode steps, each feeding the
previous step's device-side tokens back in and writing logits.  Weights are
seeded random bf16 (the page's checkpoint is not used); inputs are resident in
HBM before the timed region starts.

The headline workload (default) is the largest: 64 sequences with prompt
lengths uniform in [128, 8192], packed prefill, then 128 batched decode steps.
The other 28-layer workloads (one 512-token prompt + 256 steps; 32 x 2048 +
128 steps; one 32,768-token prompt + 32 steps) ride along as per-workload
blocks of the same JSON line.

Prints one JSON line.  `value` is the headline's decode tokens/s; prefill
tokens/s, the whole-phase HBM / MFMA fractions, the roofline of the headline's
dominant kernel (the fused decode attention, timed live with HIP events on the
model's stream) and the CPU oracle's rates ride along.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16

HEADLINE = "q06b_bf16_b64_ragged_d128"
PER_WORKLOAD = ["q06b_bf16_p512_d256", "q06b_bf16_b32_p2048_d128", "q06b_bf16_p32768_d32"]

# Counter-measured HBM traffic of the roofline kernel, kept with the kernel
# sources' digest: the figure is reported only while the sources match.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_fused_q06b_b64_ragged_traffic.md")
TRAFFIC_SOURCES = ["decoder_only_qwen3_amd/csrc/k_attn.hip", "decoder_only_qwen3_amd/csrc/common.h"]


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for p in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3
    counter summary, or None when there is none for this workload or the
    kernel's sources have changed since the counters were taken."""
    if workload != HEADLINE or not os.path.exists(TRAFFIC_FILE):
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
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--configs", default=",".join(PER_WORKLOAD),
                    help="comma-separated workloads run after the headline as per-workload blocks, or 'none'")
    ap.add_argument("--config-steps", type=int, default=2, help="timed steps of each per-workload block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graphs", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=28)
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


def decode_attention_bytes(d, lens):
    """Algorithmic bytes of one fused decode-attention launch (one layer) over
    sequences holding `lens` cached keys: read every cached key and value,
    write the new ones, read each sequence's fp32 q/k/v row, write its bf16
    attention output."""
    kvw = d.n_kv_heads * 128 * 2 * 2   # key + value bytes of one position, all kv heads
    row = (d.n_q_heads + 2 * d.n_kv_heads) * 128 * 4 + d.n_q_heads * 128 * 2
    return sum(lens) * kvw + len(lens) * (kvw + row)


def cpu_model_name():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, w, prompt, n_prefill=64, seconds_budget=12.0, max_steps=600):
    """Time the CPU oracle (float64 numpy) on a bounded sample of the workload:
    one prompt's first n_prefill tokens, then greedy decode steps for about
    `seconds_budget` seconds.  The one-time float64 conversion of the weights
    happens before the timing."""
    from threadpoolctl import threadpool_info

    from oracle import OracleModel
    m = OracleModel(d, w)
    t0 = time.perf_counter()
    m.forward(prompt[:1], m.new_cache(1))   # converts every weight to float64 once
    t_conv = time.perf_counter() - t0
    cache = m.new_cache(n_prefill + max_steps)
    t0 = time.perf_counter()
    lg = m.forward(prompt[:n_prefill], cache)[0]
    t_pre = time.perf_counter() - t0
    tok = int(np.argmax(lg))
    steps, t_dec = 0, 0.0
    while steps < max_steps and (steps < 2 or t_dec < seconds_budget):
        s0 = time.perf_counter()
        tok = int(np.argmax(m.forward([tok], cache)[0]))
        t_dec += time.perf_counter() - s0
        steps += 1
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    return {"value": round(steps / t_dec, 2), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "prefill_tok_s": round(n_prefill / t_pre, 2), "cpu_model": cpu_model_name(),
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"float64 numpy oracle, {d.n_layers} layers, sequence 0 of the workload: a {n_prefill}-token "
                      f"prefill ({t_pre:.1f} s) then {steps} greedy decode steps ({t_dec:.1f} s); the one-time "
                      f"float64 weight conversion ({t_conv:.1f} s) is not timed"}


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


def run_workload(name, args, steps, warmup, roofline=False, keep_weights=False):
    """Set up one workload's model, run warmup + timed steps, return its
    figures (and the model's weights when asked)."""
    import torch

    import q3synth
    from decoder_only_qwen3_amd import Q3Model, _lib

    wl = q3synth.WORKLOADS[name]
    d = wl.dims
    lens = [int(x) for x in wl.prompt_lengths()]
    steps_dec = wl.decode_steps
    B = wl.n_seqs
    t_gen = time.perf_counter()
    w = q3synth.make_weights(d, wl.seed, threads=min(16, os.cpu_count() or 1))
    prompts = wl.prompts()
    t_gen = time.perf_counter() - t_gen

    # room for the decode steps plus the key one more attention launch writes
    cap = max(lens) + steps_dec + 1
    if wl.chunk > 0 and len(set(lens)) != 1:
        raise SystemExit("chunked workloads need equal prompt lengths")
    bounds = ([(a, min(a + wl.chunk, lens[0])) for a in range(0, lens[0], wl.chunk)] if wl.chunk > 0
              else [(0, None)])
    max_call = sum(lens) if wl.chunk <= 0 else B * wl.chunk
    m = Q3Model(d, max_slots=B, max_positions=cap, max_prefill_tokens=max_call,
                kv_tokens=B * ((cap + 63) // 64 * 64), weight_bits=args.weight_bits)
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

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    if m.error_flags() != 0:
        raise RuntimeError("device error flags raised during warmup")
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        marks.append(one_step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if m.error_flags() != 0:
        raise RuntimeError("device error flags raised during the timed steps")
    pre_ms = [a.elapsed_time(b) for a, b, _ in marks]
    dec_ms = [b.elapsed_time(c) for _, b, c in marks]
    out = {"workload": wl.name, "n_layers": d.n_layers, "n_seqs": B,
           "prompt_tokens": lens if B <= 4 else sum(lens), "decode_steps": steps_dec,
           "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 3),
           "prefill_tok_s": round(sum(lens) * steps / (sum(pre_ms) / 1e3), 1),
           "prefill_ms": round(float(np.mean(pre_ms)), 3)}
    pf = prefill_flops(d, lens, len(calls))
    out["prefill_mfma"] = {"flops": pf, "achieved_TFLOPs": round(pf / (np.mean(pre_ms) / 1e3) / 1e12, 1),
                           "frac": round(pf / (np.mean(pre_ms) / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if steps_dec:
        dec_step_s = (sum(dec_ms) / 1e3) / (steps * steps_dec)
        byts = np.mean([decode_bytes_per_step(d, [L + 1 + i for L in lens], args.weight_bits)
                        for i in range(steps_dec)])
        out["decode_tok_s"] = round(B / dec_step_s, 2)
        out["decode_ms_per_token_step"] = round(dec_step_s * 1e3, 4)
        out["decode_hbm"] = {"bytes_per_step": float(byts), "achieved_GBs": round(byts / dec_step_s / 1e9, 1),
                             "frac": round(byts / dec_step_s / 1e9 / HBM_PEAK_GBS, 4)}
    out["_host_setup_s"] = round(t_gen, 1)

    if roofline and d.dtype == "bf16" and steps_dec:
        # The dominant kernel of the batched decode step: the fused decode
        # attention (one launch per layer and step).  Timed with HIP events on
        # the model's stream over repeated launches on the workload's final
        # state (every slot holding its prompt plus the decode steps), cycling
        # through the layers so each launch reads a different layer's cache.
        state = [L + steps_dec for L in lens]
        reps = max(1, args.kernel_reps)
        for i in range(3):
            m.decode_attention_kernel(i % d.n_layers, slots)
        k0, k1 = ev(), ev()
        k0.record(m.stream)
        for i in range(reps):
            m.decode_attention_kernel(i % d.n_layers, slots)
        k1.record(m.stream)
        torch.cuda.synchronize()
        per_launch_ms = k0.elapsed_time(k1) / reps
        alg = decode_attention_bytes(d, state)
        achieved = alg / (per_launch_ms / 1e3) / 1e9
        # A plain 256 MiB device copy: the reference that scales the profiler's
        # FETCH_SIZE / WRITE_SIZE counters to bytes (see the profiles directory).
        with torch.cuda.stream(m.stream):
            c_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
            c_dst = torch.empty_like(c_src)
            c_dst.copy_(c_src)
        torch.cuda.synchronize()
        del c_src, c_dst
        out["roofline"] = {"bound": "hbm", "kernel": "decode_attn_fused_kernel<4> (QK-Norm + RoPE + KV append + "
                                                      "split-K GQA attention, one layer)",
                           "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
                           "per_launch_us": round(per_launch_ms * 1e3, 2), "alg_bytes": alg,
                           "launches_timed": reps, "keys_per_launch": sum(state)}
    if args.checkpoint_load:
        out["checkpoint_load"] = checkpoint_load(m, w, d)
    m.close()
    del m
    torch.cuda.empty_cache()
    return (out, w, prompts) if keep_weights else (out, None, None)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import q3synth

    head, w, prompts = run_workload(args.workload, args, args.steps, args.warmup, roofline=True,
                                    keep_weights=not args.no_cpu_baseline)
    wl = q3synth.WORKLOADS[args.workload]
    d = wl.dims
    blocks = []
    if args.configs != "none":
        for name in [c for c in args.configs.split(",") if c and c != args.workload]:
            blk, _, _ = run_workload(name, args, args.config_steps, 1)
            blk.pop("_host_setup_s", None)
            blocks.append(blk)
    config = {"workload": wl.name, "n_layers": d.n_layers, "n_seqs": wl.n_seqs,
              "prompt_tokens": head["prompt_tokens"], "decode_steps": wl.decode_steps,
              "graphs": not args.no_graphs,
              **({"prefill_chunk": wl.chunk} if wl.chunk > 0 else {}),
              **({"sampling": {"temperature": args.temperature, "top_p": args.top_p}}
                 if args.temperature > 0 else {}),
              **({"weight_bits": args.weight_bits} if args.weight_bits else {})}
    line = {
        "metric": "decode tok/s + prefill tok/s (1 GPU) and % of HBM / bf16-MFMA roofline",
        "value": head.get("decode_tok_s", head["prefill_tok_s"]),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d.dtype == "bf16" else "f32",
        "data": "synthetic: seeded N(0,0.02) weights (norms 1+N(0,0.1)), uniform random token IDs",
        "config": config,
        "prefill_tok_s": head["prefill_tok_s"],
        "decode_tok_s": head.get("decode_tok_s"),
        "prefill_ms": head["prefill_ms"],
        "decode_ms_per_token_step": head.get("decode_ms_per_token_step"),
        "decode_hbm": head.get("decode_hbm"),
        "prefill_mfma": head["prefill_mfma"],
        "roofline": head.get("roofline"),
        "workloads": blocks,
        "host_setup_s": head["_host_setup_s"],
    }
    if args.checkpoint_load:
        line["checkpoint_load"] = head["checkpoint_load"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d, w, prompts[0])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
