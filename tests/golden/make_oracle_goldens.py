"""Writes the oracle's whole greedy runs at the four 28-layer workloads.

For each workload and each checked sequence, the float64 oracle (contract
mode) prefills the prompt and then runs its own greedy loop for every decode
step of the workload, one token per step ("Dentro de un LLM", Paso 9: prefill
once, then feed back the argmax).  Stored per step: the greedy token and the
final-norm output the head multiplies (bf16 values in contract mode, kept as
their 16-bit patterns, so nothing is lost).  A test rebuilds every logit of
every step with the oracle's own head.

Only `oracle/` and `q3synth` are called; this runs on the CPU (the 32,768-token
prompt took 1.9 hours with 7 BLAS threads).

    python tests/golden/make_oracle_goldens.py [workload ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import q3synth  # noqa: E402
from oracle import OracleModel  # noqa: E402


def checked_sequences(wl: q3synth.Workload):
    """The sequences whose runs are stored: the first and the last slot, the
    longest and the shortest prompt (distinct; ties go to the lower index),
    topped up with evenly spaced slots to four when some coincide."""
    if wl.n_seqs == 1:
        return [0]
    lens = [int(x) for x in wl.prompt_lengths()]
    picks = [0, wl.n_seqs - 1, int(np.argmax(lens)), int(np.argmin(lens))]
    out = []
    for p in picks:
        if p not in out:
            out.append(p)
    i = 1
    while len(out) < 4:
        c = (i * wl.n_seqs) // 4
        if c not in out:
            out.append(c)
        i += 1
    return out


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"oracle_{name}.npz")


def write(name: str):
    wl = q3synth.WORKLOADS[name]
    d = wl.dims
    t0 = time.time()
    w = q3synth.make_weights(d, wl.seed, threads=8)
    digest = q3synth.weights_digest(w)
    prompts = wl.prompts()
    seqs = checked_sequences(wl)
    o = OracleModel(d, w)
    n = wl.decode_steps
    toks = np.zeros((len(seqs), n + 1), np.int32)
    bits = np.zeros((len(seqs), n + 1, d.hidden), np.uint16)
    margin = np.zeros((len(seqs), n + 1), np.float64)
    for j, b in enumerate(seqs):
        s0 = time.time()
        tk, lg, hf = o.generate_greedy(prompts[b], n, return_hidden=True)
        f = hf.astype(np.float32)
        u = f.view(np.uint32)
        if np.any(u & 0xFFFF) or not np.array_equal(f.astype(np.float64), hf):
            raise AssertionError("final-norm output is not bf16-valued")
        toks[j] = tk
        bits[j] = (u >> 16).astype(np.uint16)
        top2 = np.sort(lg, axis=1)[:, -2:]
        margin[j] = (top2[:, 1] - top2[:, 0]) / np.sqrt(np.mean(lg * lg, axis=1))
        print(f"{name}: sequence {b} (prompt {len(prompts[b])}) done in {time.time() - s0:.0f} s", flush=True)
    np.savez_compressed(golden_path(name), workload=name, weights_sha256=digest, seqs=np.asarray(seqs, np.int32),
                        prompt_lens=np.asarray([len(prompts[b]) for b in seqs], np.int32), tokens=toks,
                        hidden_bf16=bits, top2_margin=margin)
    print(f"{name}: wrote {golden_path(name)} in {time.time() - t0:.0f} s", flush=True)


ORDER = ["q06b_bf16_p512_d256", "q06b_bf16_b32_p2048_d128", "q06b_bf16_b64_ragged_d128", "q06b_bf16_p32768_d32"]

if __name__ == "__main__":
    for nm in (sys.argv[1:] or ORDER):
        write(nm)
