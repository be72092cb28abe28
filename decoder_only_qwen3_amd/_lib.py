"""ctypes declarations for libq3 (include/q3.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq3.so")

Q3_OK, Q3_E_ARG, Q3_E_STATE, Q3_E_CAPACITY, Q3_E_HIP, Q3_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
Q3_F32, Q3_BF16 = 0, 1
Q3_MAX_BATCH = 64
Q3_PREFILL_ALL_LOGITS = 1
Q3_OPT_DECODE_GRAPH = 1

STATUS_NAMES = {0: "Q3_OK", -1: "Q3_E_ARG", -2: "Q3_E_STATE", -3: "Q3_E_CAPACITY",
                -4: "Q3_E_HIP", -5: "Q3_E_UNSUPPORTED"}

# Every symbol include/q3.h declares.
EXPORTS = [
    "q3_create", "q3_destroy", "q3_weights_bytes", "q3_kv_bytes", "q3_workspace_bytes",
    "q3_bind_memory", "q3_load_weights", "q3_seq_alloc", "q3_seq_reset", "q3_kv_reset",
    "q3_seq_length", "q3_prefill", "q3_decode_step", "q3_set_option", "q3_error_flags",
    "q3_last_error", "q3_sample", "q3_checkpoint_validate", "q3_checkpoint_staging_bytes",
    "q3_load_safetensors", "q3_check_tokens",
    "q3op_embed", "q3op_rmsnorm", "q3op_linear_workspace_bytes", "q3op_linear", "q3op_norm_linear",
    "q3op_rope_workspace_bytes", "q3op_rope_append", "q3op_attention_workspace_bytes",
    "q3op_attention", "q3op_decode_attn_fused_workspace_bytes", "q3op_decode_attn_fused", "q3op_tune",
    "q3op_sample_workspace_bytes", "q3op_sample_top_p", "q3op_quantize", "q3op_dequantize", "q3op_qlinear",
    "q3op_qlinear_rows_workspace_bytes", "q3op_qlinear_rows", "q3op_model_decode_attention",
    "q3op_linear_noalloc",
]


class q3_config(C.Structure):
    _fields_ = [
        ("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
        ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
        ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_double),
        ("dtype", C.c_int32), ("max_slots", C.c_int32), ("max_positions", C.c_int64),
        ("max_prefill_tokens", C.c_int64), ("kv_tokens", C.c_int64), ("untied_lm_head", C.c_int32),
        ("weight_bits", C.c_int32),
    ]


class q3_tensor(C.Structure):
    _fields_ = [
        ("name", C.c_char_p), ("data", C.c_void_p), ("dtype", C.c_int32),
        ("ndim", C.c_int32), ("shape", C.c_int64 * 2),
    ]


class Q3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> C.CDLL:
    """Load the in-tree libq3.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -m decoder_only_qwen3_amd._build)")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, U32, SZ, VP = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_size_t, C.c_void_p
    cfgp = C.POINTER(q3_config)
    i32p = C.POINTER(C.c_int32)
    i64p = C.POINTER(C.c_int64)
    sig = {
        "q3_create": (I32, [cfgp, C.POINTER(P)]),
        "q3_destroy": (None, [P]),
        "q3_weights_bytes": (SZ, [cfgp]),
        "q3_kv_bytes": (SZ, [cfgp]),
        "q3_workspace_bytes": (SZ, [cfgp]),
        "q3_bind_memory": (I32, [P, VP, SZ, VP, SZ, VP, SZ, VP]),
        "q3_load_weights": (I32, [P, C.POINTER(q3_tensor), I32, VP]),
        "q3_seq_alloc": (I32, [P, I32, I64, VP]),
        "q3_seq_reset": (I32, [P, I32, i32p, VP]),
        "q3_kv_reset": (I32, [P, VP]),
        "q3_seq_length": (I32, [P, I32, C.POINTER(C.c_int64)]),
        "q3_prefill": (I32, [P, I32, i32p, i32p, VP, VP, VP, U32, VP]),
        "q3_decode_step": (I32, [P, I32, i32p, VP, VP, VP, VP]),
        "q3_set_option": (I32, [P, I32, I64]),
        "q3_error_flags": (I32, [P, C.POINTER(C.c_uint32), VP]),
        "q3_last_error": (C.c_char_p, []),
        "q3_sample": (I32, [P, I32, VP, I64, C.c_float, C.c_float, VP, VP, VP]),
        "q3_checkpoint_validate": (I32, [C.POINTER(q3_config), C.POINTER(C.c_char_p), I32]),
        "q3_checkpoint_staging_bytes": (SZ, [C.POINTER(q3_config)]),
        "q3_load_safetensors": (I32, [P, C.POINTER(C.c_char_p), I32, VP, SZ, VP]),
        "q3op_sample_workspace_bytes": (SZ, [I32]),
        "q3op_quantize": (I32, [VP, I32, I32, I32, VP, VP, VP]),
        "q3op_dequantize": (I32, [VP, VP, I32, I32, I32, VP, VP]),
        "q3op_qlinear": (I32, [I32, I32, VP, VP, VP, I32, I32, VP, C.c_float, VP, VP]),
        "q3op_qlinear_rows_workspace_bytes": (SZ, [I32, I32, I32]),
        "q3op_qlinear_rows": (I32, [I32, I32, VP, I32, VP, VP, I32, I32, VP, C.c_float, VP, I64, VP, SZ, VP]),
        "q3op_sample_top_p": (I32, [VP, I32, I32, I64, C.c_float, C.c_float, VP, VP, VP, VP, SZ, VP]),
        "q3op_embed": (I32, [I32, VP, I32, VP, I32, I32, VP, VP, VP]),
        "q3op_rmsnorm": (I32, [I32, VP, I32, VP, I32, C.c_float, VP, VP]),
        "q3op_linear_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
        "q3op_linear": (I32, [I32, I32, VP, I32, VP, I32, I32, VP, I64, VP, VP, SZ, VP]),
        "q3op_norm_linear": (I32, [I32, I32, VP, I32, VP, C.c_float, VP, I32, I32, VP, I64, VP, VP, SZ, VP]),
        "q3op_rope_workspace_bytes": (SZ, [I32, I32]),
        "q3op_rope_append": (I32, [I32, VP, I32, i32p, I32, i64p, i32p, i32p, VP, I32, I32, VP, VP,
                                   C.c_float, C.c_double, I32, VP, VP, SZ, VP]),
        "q3op_tune": (I32, [I32, I32]),
        "q3op_attention_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "q3op_decode_attn_fused_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "q3op_decode_attn_fused": (I32, [VP, I32, i64p, i32p, i32p, VP, I32, I32, VP, VP, C.c_float, C.c_double,
                                         I32, I32, VP, VP, SZ, VP]),
        "q3op_attention": (I32, [I32, VP, I32, i32p, I32, i64p, i32p, i32p, VP, I32, I32, I32, VP, VP,
                                 SZ, VP]),
        "q3op_model_decode_attention": (I32, [VP, I32, I32, i32p, VP]),
        "q3_check_tokens": (I32, [VP, i32p, I64]),
        "q3op_linear_noalloc": (I32, [I32, I32, VP, I32, VP, I32, I32, VP, I64, VP, VP]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != Q3_OK:
        msg = load().q3_last_error().decode(errors="replace")
        raise Q3Error(status, msg)


def i32_array(values):
    return (C.c_int32 * len(values))(*[int(v) for v in values])


def i64_array(values):
    return (C.c_int64 * len(values))(*[int(v) for v in values])
