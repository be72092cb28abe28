"""Thin Python wrapper over libq3's C ABI (include/q3.h).

torch provides device memory and the stream; every step of the forward pass
runs in libq3's HIP kernels.  This module only marshals arguments.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import Q3_BF16, Q3_F32, check, i32_array, load, q3_config, q3_tensor


def make_config(dims, *, max_slots: int, max_positions: int, max_prefill_tokens: int,
                kv_tokens: int, untied_lm_head: bool = False, weight_bits: int = 0) -> q3_config:
    """q3_config from a q3synth.ModelDims-like object plus capacities."""
    return q3_config(
        n_layers=dims.n_layers, hidden=dims.hidden, n_q_heads=dims.n_q_heads,
        n_kv_heads=dims.n_kv_heads, head_dim=dims.head_dim, ffn=dims.ffn, vocab=dims.vocab,
        rms_eps=dims.rms_eps, rope_theta=dims.rope_theta,
        dtype=Q3_BF16 if dims.dtype == "bf16" else Q3_F32, max_slots=max_slots,
        max_positions=max_positions, max_prefill_tokens=max_prefill_tokens, kv_tokens=kv_tokens,
        untied_lm_head=1 if untied_lm_head else 0, weight_bits=weight_bits)


def checkpoint_validate(cfg: q3_config, paths: Sequence[str]) -> None:
    """Check safetensors checkpoint headers against a config (host only)."""
    arr = (C.c_char_p * len(paths))(*[p.encode() for p in paths])
    check(load().q3_checkpoint_validate(C.byref(cfg), arr, len(paths)))


class Q3Model:
    """One libq3 model handle plus the device memory it borrows."""

    def __init__(self, dims, *, max_slots: int, max_positions: int, max_prefill_tokens: int,
                 kv_tokens: int, device: str = "cuda:0", stream: Optional[torch.cuda.Stream] = None,
                 untied_lm_head: bool = False, weight_bits: int = 0):
        self.lib = load()
        self.dims = dims
        self.device = torch.device(device)
        self.cfg = make_config(dims, max_slots=max_slots, max_positions=max_positions,
                               max_prefill_tokens=max_prefill_tokens, kv_tokens=kv_tokens,
                               untied_lm_head=untied_lm_head, weight_bits=weight_bits)
        self.handle = C.c_void_p()
        check(self.lib.q3_create(C.byref(self.cfg), C.byref(self.handle)))
        self.stream = stream if stream is not None else torch.cuda.Stream(self.device)
        self.sh = C.c_void_p(self.stream.cuda_stream)
        nb = [self.lib.q3_weights_bytes(C.byref(self.cfg)), self.lib.q3_kv_bytes(C.byref(self.cfg)),
              self.lib.q3_workspace_bytes(C.byref(self.cfg))]
        with torch.cuda.stream(self.stream):
            self.bufs = [torch.empty(n, dtype=torch.uint8, device=self.device) for n in nb]
        for b in self.bufs:
            if b.data_ptr() % 256:
                raise RuntimeError("device buffer not 256-byte aligned")
        self.nbytes = nb
        check(self.lib.q3_bind_memory(self.handle, self.bufs[0].data_ptr(), nb[0], self.bufs[1].data_ptr(),
                                      nb[1], self.bufs[2].data_ptr(), nb[2], self.sh))

    # ------------------------------------------------------------------ setup
    def load_safetensors(self, paths: Sequence[str]) -> None:
        """Load a safetensors checkpoint (one file or shards) into the model."""
        n = self.lib.q3_checkpoint_staging_bytes(C.byref(self.cfg))
        with torch.cuda.stream(self.stream):
            staging = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        arr = (C.c_char_p * len(paths))(*[p.encode() for p in paths])
        check(self.lib.q3_load_safetensors(self.handle, arr, len(paths), staging.data_ptr(), staging.numel(),
                                           self.sh))
        del staging

    def load_weights(self, weights: Dict[str, np.ndarray]) -> None:
        """Upload float32 arrays (bf16-valued for a bf16 model) by the page's names."""
        bf = self.cfg.dtype == Q3_BF16
        keep = []
        tens = (q3_tensor * len(weights))()
        names = []
        with torch.cuda.stream(self.stream):
            for i, (name, arr) in enumerate(weights.items()):
                a = np.ascontiguousarray(arr, dtype=np.float32)
                if bf:
                    u = a.view(np.uint32)
                    if np.any(u & 0xFFFF):
                        raise ValueError(f"{name}: values are not bf16-representable")
                    bits = (u >> 16).astype(np.uint16).view(np.int16)
                    t = torch.from_numpy(bits).to(self.device, non_blocking=False)
                else:
                    t = torch.from_numpy(a).to(self.device, non_blocking=False)
                keep.append(t)
                nm = name.encode()
                names.append(nm)
                tens[i].name = nm
                tens[i].data = t.data_ptr()
                tens[i].dtype = self.cfg.dtype
                tens[i].ndim = a.ndim
                tens[i].shape[0] = a.shape[0]
                tens[i].shape[1] = a.shape[1] if a.ndim == 2 else 0
        torch.cuda.synchronize(self.device)
        check(self.lib.q3_load_weights(self.handle, tens, len(weights), self.sh))
        del keep

    def seq_alloc(self, slot: int, capacity: int) -> None:
        check(self.lib.q3_seq_alloc(self.handle, slot, capacity, self.sh))

    def seq_reset(self, slots: Sequence[int]) -> None:
        arr = i32_array(slots)
        check(self.lib.q3_seq_reset(self.handle, len(slots), arr, self.sh))

    def kv_reset(self) -> None:
        check(self.lib.q3_kv_reset(self.handle, self.sh))

    def seq_length(self, slot: int) -> int:
        v = C.c_int64()
        check(self.lib.q3_seq_length(self.handle, slot, C.byref(v)))
        return v.value

    def set_graphs(self, on: bool) -> None:
        check(self.lib.q3_set_option(self.handle, _lib.Q3_OPT_DECODE_GRAPH, 1 if on else 0))

    def error_flags(self) -> int:
        v = C.c_uint32()
        check(self.lib.q3_error_flags(self.handle, C.byref(v), self.sh))
        return v.value

    # ------------------------------------------------------------------ calls
    def prefill_raw(self, slots, cu, d_tokens: torch.Tensor, d_logits: Optional[torch.Tensor],
                    d_next: torch.Tensor, flags: int = 0) -> None:
        s = i32_array(slots)
        c = i32_array(cu)
        check(self.lib.q3_prefill(self.handle, len(slots), s, c, d_tokens.data_ptr(),
                                  d_logits.data_ptr() if d_logits is not None else None,
                                  d_next.data_ptr(), flags, self.sh))

    def decode_raw(self, slots, d_tokens: torch.Tensor, d_logits: Optional[torch.Tensor],
                   d_next: torch.Tensor) -> None:
        s = i32_array(slots)
        check(self.lib.q3_decode_step(self.handle, len(slots), s, d_tokens.data_ptr(),
                                      d_logits.data_ptr() if d_logits is not None else None,
                                      d_next.data_ptr(), self.sh))

    def prefill(self, slots: Sequence[int], prompts: Sequence[Sequence[int]], all_logits: bool = False):
        """Prefill several slots (a slot holding tokens already is continued after
        them); returns (logits, next) device tensors."""
        lens = [len(p) for p in prompts]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        flat = np.ascontiguousarray(np.concatenate([np.asarray(p, dtype=np.int32) for p in prompts]))
        # the IDs are on the host here: check them before anything is queued
        check(self.lib.q3_check_tokens(self.handle, flat.ctypes.data_as(C.POINTER(C.c_int32)), flat.size))
        V = self.dims.vocab
        with torch.cuda.stream(self.stream):
            tok = torch.from_numpy(flat).to(self.device)
            rows = int(cu[-1]) if all_logits else len(slots)
            logits = torch.empty((rows, V), dtype=torch.float32, device=self.device)
            nxt = torch.empty(len(slots), dtype=torch.int32, device=self.device)
        self.prefill_raw(slots, cu, tok, logits, nxt, _lib.Q3_PREFILL_ALL_LOGITS if all_logits else 0)
        return logits, nxt

    def decode(self, slots: Sequence[int], tokens: torch.Tensor, want_logits: bool = True):
        with torch.cuda.stream(self.stream):
            logits = (torch.empty((len(slots), self.dims.vocab), dtype=torch.float32, device=self.device)
                      if want_logits else None)
            nxt = torch.empty(len(slots), dtype=torch.int32, device=self.device)
        self.decode_raw(slots, tokens, logits, nxt)
        return logits, nxt

    def sample(self, logits: torch.Tensor, temperature: float, top_p: float,
               uniform: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Temperature + top-p token per logit row (q3_sample); `uniform`
        holds one float32 in [0, 1) per row (unused at temperature 0)."""
        n = logits.shape[0]
        with torch.cuda.stream(self.stream):
            nxt = torch.empty(n, dtype=torch.int32, device=self.device)
        check(self.lib.q3_sample(self.handle, n, logits.data_ptr(), logits.stride(0), float(temperature),
                                 float(top_p), uniform.data_ptr() if uniform is not None else None,
                                 nxt.data_ptr(), self.sh))
        return nxt

    def decode_attention_kernel(self, layer: int, slots: Sequence[int]) -> None:
        """Queue one launch of the fused decode attention of `layer` on the
        slots' current state (q3op_model_decode_attention; no sync)."""
        check(self.lib.q3op_model_decode_attention(self.handle, layer, len(slots), i32_array(slots), self.sh))

    def synchronize(self) -> None:
        self.stream.synchronize()

    def close(self) -> None:
        if self.handle:
            self.stream.synchronize()
            self.lib.q3_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
