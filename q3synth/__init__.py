"""Seeded synthetic inputs for the Qwen3-0.6B-shaped decoder forward pass.

This module is shared by the CPU oracle and by the HIP path's tests and
benchmark.  It generates data only: model dimensions, random-init weights,
token IDs and prompt lengths.  It holds none of the forward pass's arithmetic.

Source of the shapes: "Dentro de un LLM: Inferencia en Python puro para
Qwen3-0.6B en MLX" (reactapp.top), which fixes 28 layers, hidden size 1024,
16 query heads and 8 key/value heads of width 128 (Paso 5, the MHA/MQA/GQA
table and the `attention` listing), a 3072-wide SwiGLU (Paso 6), a 151,936-token
vocabulary (Paso 2 and the pipeline figure), EPS 1e-6 (Paso 3) and THETA 1e6
(Paso 4).  The tensor names follow the names that page's listings read from the
weight dictionary (Pasos 2, 5, 6, 7 and 8).

Recipe (the same on every machine):
  * RNG: numpy PCG64.  One child SeedSequence per tensor, spawned in the order
    `tensor_specs` lists them.
  * Linear and embedding weights: float32 N(0, 0.02).
  * Norm weights (input/post-attention/final RMSNorm, q_norm, k_norm):
    float32 1 + N(0, 0.1).
  * bf16 models: every weight is rounded from its float32 draw to the nearest
    bf16 value, ties to even.  The arrays stay float32 (holding bf16 values);
    `bf16_bits` gives the 16-bit patterns for upload.
  * Token IDs: uniform integers in [0, vocab).
  * Ragged prompt lengths: uniform integers in [lo, hi], both ends included.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "ModelDims", "Workload", "WORKLOADS", "tensor_specs", "make_weights",
    "make_tokens", "make_lengths", "bf16_bits", "round_to_bf16",
    "weights_digest", "tiny_dims",
]


@dataclasses.dataclass(frozen=True)
class ModelDims:
    """Shape of a Qwen3-style decoder.  `dtype` is "f32" or "bf16"."""
    n_layers: int = 28
    hidden: int = 1024
    n_q_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    ffn: int = 3072
    vocab: int = 151936
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    dtype: str = "bf16"

    def replace(self, **kw) -> "ModelDims":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity workload: model shape plus request mix."""
    name: str
    dims: ModelDims
    n_seqs: int
    prompt_len: int          # fixed length; 0 when lengths are drawn
    len_range: Tuple[int, int] = (0, 0)  # inclusive range for drawn lengths
    decode_steps: int = 0
    seed: int = 0
    chunk: int = 0           # > 0: each prompt is prefilled in calls of this many tokens

    def prompt_lengths(self) -> np.ndarray:
        if self.prompt_len > 0:
            return np.full(self.n_seqs, self.prompt_len, dtype=np.int64)
        return make_lengths(self.n_seqs, self.len_range[0], self.len_range[1],
                            seed=self.seed + 2)

    def prompts(self) -> List[List[int]]:
        """The token IDs of every prompt: sequence i draws its own with seed
        seed + 1 + i."""
        return [make_tokens(int(L), self.dims.vocab, self.seed + 1 + i).tolist()
                for i, L in enumerate(self.prompt_lengths())]


QWEN3_06B = ModelDims()

WORKLOADS: Dict[str, Workload] = {
    # 2-layer cut of the 0.6B shape, float32 weights and KV cache.
    "tiny2l_f32_p5_d16": Workload("tiny2l_f32_p5_d16", QWEN3_06B.replace(n_layers=2, dtype="f32"),
                                  n_seqs=1, prompt_len=5, decode_steps=16, seed=1000),
    # Full 28-layer shape, bf16; one 512-token prompt then 256 greedy steps.
    "q06b_bf16_p512_d256": Workload("q06b_bf16_p512_d256", QWEN3_06B, n_seqs=1, prompt_len=512,
                                    decode_steps=256, seed=1001),
    # 32 independent sequences, 2048-token prefixes, 128 batched decode steps.
    "q06b_bf16_b32_p2048_d128": Workload("q06b_bf16_b32_p2048_d128", QWEN3_06B, n_seqs=32,
                                         prompt_len=2048, decode_steps=128, seed=1002),
    # One 32,768-token prompt then 32 decode steps.
    "q06b_bf16_p32768_d32": Workload("q06b_bf16_p32768_d32", QWEN3_06B, n_seqs=1,
                                     prompt_len=32768, decode_steps=32, seed=1003),
    # The 32,768-token prompt above prefilled in eight calls of 4096 tokens
    # (each continuing the cache of the ones before), then 32 decode steps.
    "q06b_bf16_p32768_c4096_d32": Workload("q06b_bf16_p32768_c4096_d32", QWEN3_06B, n_seqs=1,
                                           prompt_len=32768, decode_steps=32, seed=1003, chunk=4096),
    # 64 sequences with lengths uniform in [128, 8192], packed prefill, 128 steps.
    "q06b_bf16_b64_ragged_d128": Workload("q06b_bf16_b64_ragged_d128", QWEN3_06B, n_seqs=64,
                                          prompt_len=0, len_range=(128, 8192),
                                          decode_steps=128, seed=1004),
}


def tiny_dims(**kw) -> ModelDims:
    """A very small decoder for brute-force checks (not a GPU shape)."""
    base = ModelDims(n_layers=2, hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=8,
                     ffn=24, vocab=97, dtype="f32")
    return base.replace(**kw)


def tensor_specs(d: ModelDims) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) in generation order; kind is "linear" or "norm".

    Linear weights are stored (out_features, in_features) and used as x @ W^T.
    """
    H, D, I, V = d.hidden, d.head_dim, d.ffn, d.vocab
    specs = [("model.embed_tokens.weight", (V, H), "linear")]
    for i in range(d.n_layers):
        p = f"model.layers.{i}"
        specs += [
            (f"{p}.self_attn.q_proj.weight", (d.n_q_heads * D, H), "linear"),
            (f"{p}.self_attn.k_proj.weight", (d.n_kv_heads * D, H), "linear"),
            (f"{p}.self_attn.v_proj.weight", (d.n_kv_heads * D, H), "linear"),
            (f"{p}.self_attn.o_proj.weight", (H, d.n_q_heads * D), "linear"),
            (f"{p}.self_attn.q_norm.weight", (D,), "norm"),
            (f"{p}.self_attn.k_norm.weight", (D,), "norm"),
            (f"{p}.input_layernorm.weight", (H,), "norm"),
            (f"{p}.post_attention_layernorm.weight", (H,), "norm"),
            (f"{p}.mlp.gate_proj.weight", (I, H), "linear"),
            (f"{p}.mlp.up_proj.weight", (I, H), "linear"),
            (f"{p}.mlp.down_proj.weight", (H, I), "linear"),
        ]
    specs.append(("model.norm.weight", (H,), "norm"))
    return specs


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    a = np.array(a, dtype=np.float32, copy=True, order="C")
    if not np.all(np.isfinite(a)):
        raise ValueError("round_to_bf16 expects finite values")
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)       # finite floats stay below 2^32 here
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def _draw(spec, ss, bf16: bool) -> np.ndarray:
    name, shape, kind = spec
    rng = np.random.Generator(np.random.PCG64(ss))
    a = rng.standard_normal(shape, dtype=np.float32)
    if kind == "linear":
        a *= np.float32(0.02)
    else:
        a *= np.float32(0.1)
        a += np.float32(1.0)
    return round_to_bf16(a) if bf16 else a


def make_weights(d: ModelDims, seed: int = 0, threads: int = 1) -> Dict[str, np.ndarray]:
    """Seeded random-init weights, float32 arrays (bf16 values for bf16 models).

    Each tensor has its own child seed, so drawing them on several threads gives
    the same arrays as drawing them one after another.
    """
    specs = tensor_specs(d)
    children = np.random.SeedSequence(seed).spawn(len(specs))
    bf = d.dtype == "bf16"
    if threads > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            arrays = list(ex.map(lambda a: _draw(a[0], a[1], bf), zip(specs, children)))
    else:
        arrays = [_draw(sp, ss, bf) for sp, ss in zip(specs, children)]
    return {sp[0]: a for sp, a in zip(specs, arrays)}


def make_tokens(n: int, vocab: int, seed: int) -> np.ndarray:
    """Uniform token IDs in [0, vocab) as int32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def make_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform integer lengths in [lo, hi], both ends included."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return rng.integers(lo, hi, endpoint=True, size=n, dtype=np.int64)


def weights_digest(w: Dict[str, np.ndarray]) -> str:
    """SHA-256 over every tensor's bytes in name order (run provenance)."""
    h = hashlib.sha256()
    for k in sorted(w):
        h.update(k.encode())
        h.update(np.ascontiguousarray(w[k]).tobytes())
    return h.hexdigest()
