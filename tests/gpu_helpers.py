"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import functools

import numpy as np

import q3synth


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / RMS(ref): the logits error measure of the parity bar."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(np.asarray(gpu, dtype=np.float64) - ref)) / rms)


def margin_ok(ref_logits: np.ndarray, gpu_token: int, tol_abs: float) -> bool:
    """True when the GPU's token is the oracle's argmax, or within tol_abs of it (a near-tie)."""
    top = int(np.argmax(ref_logits))
    if gpu_token == top:
        return True
    return float(ref_logits[top] - ref_logits[gpu_token]) <= tol_abs


@functools.lru_cache(maxsize=4)
def weights_for(dims: q3synth.ModelDims, seed: int):
    return q3synth.make_weights(dims, seed)


# ---------------------------------------------------------------- KV cache value layout
def vt_blocks(vt: np.ndarray) -> np.ndarray:
    """Values as the kernels store them, from the logical transposed view
    vt [n_kv][128][cap]: blocks of 32 keys, each [128 dims][32 keys]."""
    n_kv, dim, cap = vt.shape
    return np.ascontiguousarray(vt.reshape(n_kv, dim, cap // 32, 32).transpose(0, 2, 1, 3)).reshape(-1)


def vt_logical(flat: np.ndarray, n_kv: int, cap: int) -> np.ndarray:
    """Inverse of vt_blocks: [n_kv][128][cap] view of a stored value region."""
    return flat.reshape(n_kv, cap // 32, 128, 32).transpose(0, 2, 1, 3).reshape(n_kv, 128, cap)


# ---------------------------------------------------------------- KV cache key layout (bf16)
def k_perm(cap: int) -> np.ndarray:
    """Element index of (key, dim) within one head's key region of a bf16
    cache: blocks of 32 keys, each stored in the order the attention kernels
    take it as MFMA operands -- 16-byte chunk (sbk*4 + ks)*64 + fq*16 + fr of a
    block holds dims ks*32 + fq*8 .. +7 of its key 8*(fr//4) + 4*sbk + fr%4."""
    key = np.arange(cap)[:, None]
    dim = np.arange(128)[None, :]
    k = key & 31
    sbk, fr = (k >> 2) & 1, ((k >> 3) << 2) | (k & 3)
    ks, fq = dim >> 5, (dim >> 3) & 3
    return (key >> 5) * 4096 + (((sbk * 4 + ks) * 4 + fq) * 16 + fr) * 8 + (dim & 7)


def k_blocks(k: np.ndarray) -> np.ndarray:
    """Keys as a bf16 cache stores them, from the logical k [n_kv][cap][128]."""
    n_kv, cap, _ = k.shape
    out = np.empty((n_kv, cap * 128), k.dtype)
    out[:, k_perm(cap).reshape(-1)] = k.reshape(n_kv, -1)
    return out.reshape(-1)


def k_logical(flat: np.ndarray, n_kv: int, cap: int) -> np.ndarray:
    """Inverse of k_blocks: [n_kv][cap][128] copy of a stored key region."""
    return flat.reshape(n_kv, cap * 128)[:, k_perm(cap).reshape(-1)].reshape(n_kv, cap, 128)


# ---------------------------------------------------------------- device marshalling
def dev_bf16(a: np.ndarray):
    """bf16-valued float32 array -> torch int16 tensor of its bit patterns on cuda:0."""
    import torch
    bits = q3synth.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).to("cuda:0")


def host_bf16(t) -> np.ndarray:
    """torch int16 tensor of bf16 bit patterns -> float32 numpy array."""
    bits = t.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32)


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def rand_bf16(rng, shape, scale=1.0) -> np.ndarray:
    return q3synth.round_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def ops():
    from decoder_only_qwen3_amd import _lib
    return _lib, _lib.load()


def call(status):
    from decoder_only_qwen3_amd import _lib
    _lib.check(status)


# ---------------------------------------------------------------- Paso 8 sampling
def sample_agrees(logits, temperature, top_p, u, gpu_token, eps=1e-5):
    """(ok, near_tie): the GPU's sampled token equals the oracle's, or differs
    only where a decision of the oracle sits within eps of its threshold (a
    running sum within eps of top_p, the uniform within eps of a renormalised
    running sum) or where two weights are equal to float32 precision."""
    from oracle import sample_top_p
    logits = np.asarray(logits, dtype=np.float64)
    ref = sample_top_p(logits, temperature, top_p, u)
    if gpu_token == ref:
        return True, False
    for dp in (-eps, 0.0, eps):
        for du in (-eps, 0.0, eps):
            uu = min(max(u + du, 0.0), 1.0 - 1e-12)
            if sample_top_p(logits, temperature, top_p + dp, uu) == gpu_token:
                return True, True
    z = logits / temperature
    if abs(z[gpu_token] - z[ref]) < 1e-6 * max(1.0, abs(z[ref])):
        return True, True
    return False, False
