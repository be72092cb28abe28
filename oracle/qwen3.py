"""Plain float64 forward pass of a Qwen3-style decoder (test infrastructure only).

Written from the page "Dentro de un LLM: Inferencia en Python puro para
Qwen3-0.6B en MLX" (reactapp.top).  Citations name the page's steps ("Paso N").

Two numeric modes:
  * exact (float32 models): no rounding anywhere; every value is float64.
  * contract (bf16 models): the weights and KV cache hold bf16 values, and the
    activations that feed a matrix product are rounded to bf16 at fixed points
    (listed in `OracleModel`).  Accumulation is still float64.

Readings of points the page leaves open (the page prints no `forward`, and its
mask is written for an empty cache):
  * forward = embedding gather -> blocks -> final norm -> head, with positions
    pos0 .. pos0+T-1 where pos0 is the number of tokens already cached.
  * causal rule: query at position p sees exactly the keys at positions <= p.
    Masked keys are excluded from the softmax, which equals adding -1e9 because
    every query sees at least its own key.
  * RoPE rotates the pair (i, i + D/2) ("rotate half"), angle p * theta^(-i/(D/2)),
    computed in float64.
  * grouped-query attention: query head h reads key/value head h // (n_q/n_kv),
    the element-repeat the page's listing uses.
  * logits come from the last position of each call unless rows are requested.
  * argmax ties go to the lowest index.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

__all__ = [
    "to_bf16", "rms_norm", "rope_cos_sin", "rope_rotate", "attention_rows",
    "silu", "swiglu", "greedy_pick", "sample_top_p", "quantize_affine", "dequantize_affine",
    "quantized_weights", "KVCache", "OracleModel",
]


# ----------------------------------------------------------------------------
# rounding used by the bf16 contract (not a step of the page's method)
# ----------------------------------------------------------------------------
def to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via float32, both ties-to-even); float64 out.

    float64 -> float32 uses numpy's conversion (round to nearest even).  The
    float32 -> bf16 step keeps the upper 16 bits after adding half an ulp of
    bf16, plus one when the kept part is odd, which is ties-to-even.
    """
    f = np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _identity(a: np.ndarray) -> np.ndarray:
    return a


# ----------------------------------------------------------------------------
# Paso 3: RMSNorm
# ----------------------------------------------------------------------------
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Divide each vector by the root of (its mean square + eps), then scale by w.

    No mean is subtracted and there is no bias; w multiplies directly.
    The reduction runs over the last axis.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


# ----------------------------------------------------------------------------
# Paso 4: RoPE
# ----------------------------------------------------------------------------
def rope_cos_sin(positions: Sequence[int], head_dim: int, theta: float):
    """cos and sin of the rotation angles, shape (len(positions), head_dim/2).

    Pair i (dims i and i + head_dim/2) turns by position * theta^(-i/(head_dim/2)).
    """
    half = head_dim // 2
    pos = np.asarray(positions, dtype=np.float64)
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) / half)
    ang = pos[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope_rotate(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE.  u: (T, heads, D); cos/sin: (T, D/2).

    First half a and second half b become (a cos - b sin, a sin + b cos).
    """
    half = u.shape[-1] // 2
    a = u[..., :half]
    b = u[..., half:]
    c = cos[:, None, :]
    s = sin[:, None, :]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# ----------------------------------------------------------------------------
# Paso 5: attention with grouped query heads
# ----------------------------------------------------------------------------
def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   q_pos: np.ndarray, k_pos: np.ndarray,
                   block: Optional[int] = None) -> np.ndarray:
    """Causal grouped-query attention for one sequence.

    q: (T, n_q, D) queries at positions q_pos (T,)
    k, v: (S, n_kv, D) cached keys/values at positions k_pos (S,)
    returns (T, n_q, D).

    For query head h the key/value head is h // (n_q // n_kv).  Scores are
    q.k / sqrt(D); a query at position p sees only keys at positions <= p;
    the softmax runs over those keys and weights the values.  Query rows are
    processed in blocks so that no T x S matrix is held at once; each row's
    sum is unchanged by the blocking.
    """
    T, n_q, D = q.shape
    S, n_kv, _ = k.shape
    group = n_q // n_kv
    scale = D ** -0.5
    if block is None:   # bound the score block to about 40M float64 values
        block = max(1, min(256, int(4e7 // max(1, n_q * S))))
    kt = np.transpose(k, (1, 2, 0))            # (n_kv, D, S)
    vv = np.transpose(v, (1, 0, 2))            # (n_kv, S, D)
    out = np.empty((T, n_q, D), dtype=np.float64)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        qb = q[t0:t1].reshape(t1 - t0, n_kv, group, D).transpose(1, 2, 0, 3)  # (n_kv, g, b, D)
        last = int(np.max(q_pos[t0:t1]))
        sel = np.nonzero(k_pos <= last)[0]
        s = np.matmul(qb, kt[:, None, :, :][..., sel]) * scale           # (n_kv, g, b, s)
        allowed = k_pos[sel][None, :] <= q_pos[t0:t1][:, None]           # (b, s)
        s = np.where(allowed[None, None], s, -np.inf)
        s = s - np.max(s, axis=-1, keepdims=True)
        p = np.exp(s)
        p /= np.sum(p, axis=-1, keepdims=True)
        o = np.matmul(p, vv[:, None, sel, :])                              # (n_kv, g, b, D)
        out[t0:t1] = o.transpose(2, 0, 1, 3).reshape(t1 - t0, n_q, D)
    return out


# ----------------------------------------------------------------------------
# Paso 6: SwiGLU feed-forward
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), written as z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(h: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
           rnd=_identity) -> np.ndarray:
    """down( silu(h gate^T) * (h up^T) ); `rnd` rounds the product before down."""
    g = h @ wg.T
    u = h @ wu.T
    return rnd(silu(g) * u) @ wd.T


# ----------------------------------------------------------------------------
# Paso 8: greedy choice
# ----------------------------------------------------------------------------
def greedy_pick(logits: np.ndarray) -> int:
    """Index of the largest logit; the lowest index wins a tie.  NaN is an error."""
    logits = np.asarray(logits)
    if not np.all(np.isfinite(logits)):
        raise FloatingPointError("non-finite logits")
    return int(np.argmax(logits))


# ----------------------------------------------------------------------------
# Paso 8: temperature + top-p (nucleus) sampling
# ----------------------------------------------------------------------------
def sample_top_p(logits: np.ndarray, temperature: float, top_p: float, u: float) -> int:
    """One token from temperature + top-p sampling, the page's steps in order.

    temperature == 0 is the greedy choice.  Otherwise: scale the logits by
    1/temperature, softmax, order the probabilities from largest to smallest
    (equal probabilities by increasing token ID), running sum, keep the first
    #(running sum < top_p) + 1 of them (all of them at most), renormalise the
    kept ones, and draw one.  The draw is taken by inverse transform with the
    caller's uniform u in [0, 1): the kept token whose renormalised running
    sum first exceeds u, in the same order.  (The page draws through a
    categorical sampler; with the random number an input, inverse transform
    is the plain deterministic form of that draw.)  Everything in float64.
    """
    z = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(z)):
        raise FloatingPointError("non-finite logits")
    if temperature == 0:
        return greedy_pick(z)
    if temperature < 0 or not 0.0 <= u < 1.0:
        raise ValueError("temperature must be >= 0 and u in [0, 1)")
    z = z / temperature
    e = np.exp(z - z.max())
    probs = e / e.sum()
    order = np.argsort(-probs, kind="stable")
    sorted_p = probs[order]
    cumsum = np.cumsum(sorted_p)
    cutoff = min(int(np.sum(cumsum < top_p)) + 1, z.size)
    kept = sorted_p[:cutoff] / np.sum(sorted_p[:cutoff])
    running = np.cumsum(kept)
    j = int(np.sum(running <= u))          # first running sum that exceeds u
    return int(order[min(j, cutoff - 1)])


# ----------------------------------------------------------------------------
# Weight-only affine group quantization ("Investigación de rendimiento de Laya MLX",
# "Cuantización" section: groups of 64 along the input dimension, 8 or 4 bits,
# fp16 scale and offset per group)
# ----------------------------------------------------------------------------
QUANT_GROUP = 64
LINEAR_SUFFIXES = ("q_proj.weight", "k_proj.weight", "v_proj.weight", "o_proj.weight",
                   "gate_proj.weight", "up_proj.weight", "down_proj.weight")


def quantize_affine(w: np.ndarray, bits: int, group: int = QUANT_GROUP):
    """Codes q (uint8, one per element), scales s and offsets b (float16, one
    per group of `group` consecutive elements of a row) with w ~ q*s + b.

    Per group: b is the minimum and s = (max - min) / (2^bits - 1), each
    rounded to float16; q = clamp(floor((w - b) / s + 1/2), 0, 2^bits - 1),
    computed in float32 from the float16 values (q = 0 when s is 0).  The page
    fixes the scheme (affine, per group, fp16 scale and offset); these are the
    plain formulas for it, and the float32 steps are the precision in which
    the codes are decided on both sides.
    """
    w = np.asarray(w, dtype=np.float32)
    rows, K = w.shape
    if K % group != 0:
        raise ValueError("the row length must be a multiple of the group size")
    g = w.reshape(rows, K // group, group)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    levels = np.float32(2 ** bits - 1)
    s16 = ((mx - mn) / levels).astype(np.float16)
    b16 = mn.astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    b32 = b16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.floor((g - b32) / s32 + np.float32(0.5))
    t = np.where(s32 == 0, 0, t)
    q = np.clip(t, 0, 2 ** bits - 1).astype(np.uint8).reshape(rows, K)
    return q, s16, b16


def dequantize_affine(q: np.ndarray, s: np.ndarray, b: np.ndarray, group: int = QUANT_GROUP) -> np.ndarray:
    """w' = q * s + b in float64 (exact for float16 s and b)."""
    rows, K = q.shape
    g = q.reshape(rows, K // group, group).astype(np.float64)
    return (g * s.astype(np.float64)[..., None] + b.astype(np.float64)[..., None]).reshape(rows, K)


def quantized_weights(weights: Dict[str, np.ndarray], bits: int) -> Dict[str, np.ndarray]:
    """The weights a weight-only quantized bf16 model computes with: every
    linear projection of the blocks replaced by its dequantized values, each
    rounded to bf16 like every other weight of the bf16 model (the matrix
    products of the bf16 contract take bf16 operands); embedding, head and
    norm weights unchanged."""
    out = {}
    for name, w in weights.items():
        if name.startswith("model.layers.") and name.endswith(LINEAR_SUFFIXES):
            out[name] = to_bf16(dequantize_affine(*quantize_affine(w, bits)))
        else:
            out[name] = w
    return out


# ----------------------------------------------------------------------------
# KV cache (Paso 5, cache note) and the model (Pasos 2, 7, 8, 9)
# ----------------------------------------------------------------------------
class KVCache:
    """Per-layer keys (after QK-Norm and RoPE) and raw values of one sequence."""

    def __init__(self, n_layers: int, n_kv: int, head_dim: int, capacity: int):
        self.k = [np.zeros((capacity, n_kv, head_dim)) for _ in range(n_layers)]
        self.v = [np.zeros((capacity, n_kv, head_dim)) for _ in range(n_layers)]
        self.length = 0
        self.capacity = capacity

    def positions(self, n: int) -> np.ndarray:
        return np.arange(n, dtype=np.int64)


class OracleModel:
    """float64 Qwen3-style decoder over a dict of named weights.

    Weights use the page's tensor names; linear weights are (out, in) and apply
    as x @ W^T.  The lm_head is tied to the embedding matrix.

    A weight named "lm_head.weight" (vocab, hidden), when present, is the head;
    otherwise the head is the embedding matrix.

    `contract=True` (bf16 models) rounds to bf16: each RMSNorm output that feeds
    a projection (including the final one before the head), the queries and
    keys after QK-Norm and RoPE, the values, the attention output and the
    SwiGLU product.  The residual stream, scores, softmax and logits are not
    rounded.
    """

    def __init__(self, dims, weights: Dict[str, np.ndarray], contract: Optional[bool] = None,
                 cache_weights: bool = True):
        self.d = dims
        self.w = weights
        self.contract = (dims.dtype == "bf16") if contract is None else contract
        self.rnd = to_bf16 if self.contract else _identity
        self._cache_weights = cache_weights
        self._w64: Dict[str, np.ndarray] = {}

    # -- weights -------------------------------------------------------------
    def W(self, name: str) -> np.ndarray:
        a = self._w64.get(name)
        if a is None:
            a = np.asarray(self.w[name], dtype=np.float64)
            if self._cache_weights:
                self._w64[name] = a
        return a

    def new_cache(self, capacity: int) -> KVCache:
        d = self.d
        return KVCache(d.n_layers, d.n_kv_heads, d.head_dim, capacity)

    # -- Paso 5 + Paso 7 ------------------------------------------------------
    def attention(self, h: np.ndarray, layer: int, cache: KVCache,
                  positions: np.ndarray, keep: Optional[np.ndarray] = None) -> np.ndarray:
        d = self.d
        p = f"model.layers.{layer}.self_attn"
        T = h.shape[0]
        q = (h @ self.W(f"{p}.q_proj.weight").T).reshape(T, d.n_q_heads, d.head_dim)
        k = (h @ self.W(f"{p}.k_proj.weight").T).reshape(T, d.n_kv_heads, d.head_dim)
        v = (h @ self.W(f"{p}.v_proj.weight").T).reshape(T, d.n_kv_heads, d.head_dim)
        q = rms_norm(q, self.W(f"{p}.q_norm.weight"), d.rms_eps)
        k = rms_norm(k, self.W(f"{p}.k_norm.weight"), d.rms_eps)
        cos, sin = rope_cos_sin(positions, d.head_dim, d.rope_theta)
        q = self.rnd(rope_rotate(q, cos, sin))
        k = self.rnd(rope_rotate(k, cos, sin))
        v = self.rnd(v)
        s0, s1 = int(positions[0]), int(positions[-1]) + 1
        if s1 > cache.capacity:
            raise ValueError("KV cache full")
        cache.k[layer][s0:s1] = k
        cache.v[layer][s0:s1] = v
        k_all = cache.k[layer][:s1]
        v_all = cache.v[layer][:s1]
        if keep is not None:
            q, positions, T = q[keep], positions[keep], len(keep)
        o = attention_rows(q, k_all, v_all, positions, np.arange(s1, dtype=np.int64))
        o = self.rnd(o.reshape(T, d.n_q_heads * d.head_dim))
        return o @ self.W(f"{p}.o_proj.weight").T

    def block(self, x: np.ndarray, layer: int, cache: KVCache,
              positions: np.ndarray, keep: Optional[np.ndarray] = None) -> np.ndarray:
        """Paso 7.  `keep`: indices of the rows whose output is wanted; every
        row's key and value still enter the cache, and the kept rows' values
        are exactly those of the full computation (rows do not mix outside
        attention, and attention reads only the cache)."""
        d = self.d
        p = f"model.layers.{layer}"
        h = self.rnd(rms_norm(x, self.W(f"{p}.input_layernorm.weight"), d.rms_eps))
        a = self.attention(h, layer, cache, positions, keep)
        if keep is not None:
            x = x[keep]
        x = x + a
        h = self.rnd(rms_norm(x, self.W(f"{p}.post_attention_layernorm.weight"), d.rms_eps))
        x = x + swiglu(h, self.W(f"{p}.mlp.gate_proj.weight"), self.W(f"{p}.mlp.up_proj.weight"),
                       self.W(f"{p}.mlp.down_proj.weight"), self.rnd)
        return x

    # -- Paso 2 + Paso 8: one call over new tokens ----------------------------
    def final_hidden(self, ids: Sequence[int], cache: KVCache,
                     logit_rows: Optional[Iterable[int]] = None) -> np.ndarray:
        """Run `ids` at positions cache.length.. and append them to the cache.

        Returns the final-norm output (n_rows, hidden) of the rows `logit_rows`
        (indices into ids; default: the last row only): the vectors the head
        multiplies (bf16 values in contract mode).
        """
        d = self.d
        ids = np.asarray(ids, dtype=np.int64)
        if ids.ndim != 1 or ids.size == 0:
            raise ValueError("ids must be a non-empty 1-D sequence")
        if np.any(ids < 0) or np.any(ids >= d.vocab):
            raise ValueError("token id out of range")
        pos0 = cache.length
        positions = pos0 + np.arange(ids.size, dtype=np.int64)
        E = self.W("model.embed_tokens.weight")
        rows = np.asarray([ids.size - 1] if logit_rows is None else list(logit_rows), dtype=np.int64)
        x = E[ids]
        for layer in range(d.n_layers):
            # The last block only needs the rows whose logits are returned.
            keep = rows if layer == d.n_layers - 1 else None
            x = self.block(x, layer, cache, positions, keep)
        cache.length = pos0 + ids.size
        if d.n_layers == 0:
            x = x[rows]
        return self.rnd(rms_norm(x, self.W("model.norm.weight"), d.rms_eps))

    def head(self, hf: np.ndarray) -> np.ndarray:
        """Paso 8: logits = hf @ head^T.  The head is tied to the embedding
        unless the weights carry a separate lm_head matrix (the page's listing
        reads one by that name)."""
        name = "lm_head.weight" if "lm_head.weight" in self.w else "model.embed_tokens.weight"
        return np.asarray(hf, dtype=np.float64) @ self.W(name).T

    def forward(self, ids: Sequence[int], cache: KVCache,
                logit_rows: Optional[Iterable[int]] = None) -> np.ndarray:
        """Run `ids` at positions cache.length.. and append them to the cache.

        Returns logits (n_rows, vocab) for `logit_rows` (indices into ids;
        default: the last row only).
        """
        return self.head(self.final_hidden(ids, cache, logit_rows))

    # -- Paso 9: generation loops ---------------------------------------------
    def generate_greedy(self, prompt: Sequence[int], n_steps: int, return_hidden: bool = False):
        """Prefill, then n_steps one-token steps feeding back the argmax.

        Returns (tokens, logits): n_steps + 1 greedy tokens (the first comes
        from the prefill's last row) and the logits each was picked from; with
        return_hidden, also the final-norm vectors those logits came from.
        """
        cache = self.new_cache(len(prompt) + n_steps)
        hf = self.final_hidden(prompt, cache)[0]
        lg = self.head(hf)
        toks, logits, hidden = [greedy_pick(lg)], [lg], [hf]
        for _ in range(n_steps):
            hf = self.final_hidden([toks[-1]], cache)[0]
            lg = self.head(hf)
            toks.append(greedy_pick(lg))
            logits.append(lg)
            hidden.append(hf)
        out = (np.asarray(toks, dtype=np.int64), np.stack(logits))
        return out + (np.stack(hidden),) if return_hidden else out

    def forced_logits(self, prompt: Sequence[int], forced: Sequence[int]) -> np.ndarray:
        """Logits after the prompt and after each forced token, in one pass.

        Equivalent to prefill(prompt) followed by one decode step per forced
        token (the cache makes the two the same computation); computed as a
        single call over prompt + forced with the rows of interest selected.
        Returns (len(forced) + 1, vocab).
        """
        ids = list(prompt) + list(forced)
        cache = self.new_cache(len(ids))
        rows = range(len(prompt) - 1, len(ids))
        return self.forward(ids, cache, logit_rows=rows)
