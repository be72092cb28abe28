"""safetensors checkpoint headers checked against a model config (host only:
q3_checkpoint_validate reads no tensor data and needs no device)."""
import numpy as np
import pytest

import q3synth
from checkpoint_files import write_checkpoint, write_raw

D = q3synth.QWEN3_06B.replace(n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=2, ffn=512, vocab=256)


def _cfg(untied=False, dtype=None):
    from decoder_only_qwen3_amd import make_config
    d = D if dtype is None else D.replace(dtype=dtype)
    return make_config(d, max_slots=1, max_positions=64, max_prefill_tokens=64, kv_tokens=64,
                       untied_lm_head=untied)


def _weights(untied=False):
    w = q3synth.make_weights(D, seed=3)
    if untied:
        w["lm_head.weight"] = q3synth.round_to_bf16(
            np.random.default_rng(4).standard_normal((D.vocab, D.hidden)).astype(np.float32) * 0.02)
    return w


def _validate(cfg, paths):
    from decoder_only_qwen3_amd import _lib
    lib = _lib.load()
    import ctypes as C
    arr = (C.c_char_p * len(paths))(*[str(p).encode() for p in paths])
    st = lib.q3_checkpoint_validate(C.byref(cfg), arr, len(paths))
    return st, lib.q3_last_error().decode()


def test_valid_single_file_and_shards(tmp_path):
    from decoder_only_qwen3_amd import _lib
    w = _weights()
    one = [tmp_path / "model.safetensors"]
    write_checkpoint(w, [str(p) for p in one], metadata={"format": "pt"})
    assert _validate(_cfg(), one)[0] == _lib.Q3_OK
    shards = [tmp_path / f"model-{i}-of-3.safetensors" for i in range(3)]
    write_checkpoint(w, [str(p) for p in shards])
    assert _validate(_cfg(), shards)[0] == _lib.Q3_OK
    # float32 checkpoint for the float32 model
    f32 = [tmp_path / "f32.safetensors"]
    write_checkpoint(w, [str(p) for p in f32], dtype="f32")
    assert _validate(_cfg(dtype="f32"), f32)[0] == _lib.Q3_OK


def test_missing_wrong_shape_unknown_and_repeated(tmp_path):
    from decoder_only_qwen3_amd import _lib
    w = _weights()
    p = tmp_path / "a.safetensors"
    miss = dict(w)
    del miss["model.layers.1.mlp.up_proj.weight"]
    write_checkpoint(miss, [str(p)])
    st, msg = _validate(_cfg(), [p])
    assert st == _lib.Q3_E_ARG and "model.layers.1.mlp.up_proj.weight" in msg
    bad = dict(w, **{"model.layers.0.self_attn.k_proj.weight": np.zeros((128, 512), np.float32)})
    write_checkpoint(bad, [str(p)])
    st, msg = _validate(_cfg(), [p])
    assert st == _lib.Q3_E_ARG and "wrong shape" in msg
    extra = dict(w, **{"model.layers.0.mlp.bias": np.zeros(4, np.float32)})
    write_checkpoint(extra, [str(p)])
    st, msg = _validate(_cfg(), [p])
    assert st == _lib.Q3_E_ARG and "unknown tensor" in msg
    q = tmp_path / "b.safetensors"
    write_checkpoint({"model.norm.weight": w["model.norm.weight"]}, [str(q)])
    write_checkpoint(w, [str(p)])
    st, msg = _validate(_cfg(), [p, q])
    assert st == _lib.Q3_E_ARG and "twice" in msg


def test_dtype_must_match_the_model(tmp_path):
    from decoder_only_qwen3_amd import _lib
    p = tmp_path / "a.safetensors"
    write_checkpoint(_weights(), [str(p)], dtype="f32")
    st, msg = _validate(_cfg(), [p])
    assert st == _lib.Q3_E_UNSUPPORTED and "F32" in msg


def test_separate_head(tmp_path):
    from decoder_only_qwen3_amd import _lib
    p = tmp_path / "a.safetensors"
    write_checkpoint(_weights(untied=True), [str(p)])
    assert _validate(_cfg(untied=True), [p])[0] == _lib.Q3_OK
    st, msg = _validate(_cfg(untied=False), [p])
    assert st == _lib.Q3_E_ARG and "lm_head" in msg
    write_checkpoint(_weights(), [str(p)])
    st, msg = _validate(_cfg(untied=True), [p])
    assert st == _lib.Q3_E_ARG and "lacks lm_head.weight" in msg


@pytest.mark.parametrize("case", ["short", "json", "offsets", "range", "length", "missing_file", "dtype_name"])
def test_malformed_files(tmp_path, case):
    from decoder_only_qwen3_amd import _lib
    p = tmp_path / "bad.safetensors"
    hdr = {"model.norm.weight": {"dtype": "BF16", "shape": [512], "data_offsets": [0, 1024]}}
    if case == "short":
        p.write_bytes(b"\x05\x00")
    elif case == "json":  # header cut inside the JSON
        p.write_bytes(np.uint64(10).tobytes() + b"{\"a\": [1, ")
    elif case == "offsets":
        write_raw(p, hdr, b"\x00" * 100)  # data section shorter than the tensor
    elif case == "range":
        hdr["model.norm.weight"]["data_offsets"] = [0, 1000]  # not 512 x 2 bytes
        write_raw(p, hdr, b"\x00" * 1024)
    elif case == "length":
        write_raw(p, hdr, b"\x00" * 1024, header_len=1 << 40)
    elif case == "dtype_name":
        hdr["model.norm.weight"]["dtype"] = "Q4"
        write_raw(p, hdr, b"\x00" * 1024)
    paths = [tmp_path / "absent.safetensors"] if case == "missing_file" else [p]
    st, msg = _validate(_cfg(), paths)
    assert st == _lib.Q3_E_ARG, (case, st, msg)
