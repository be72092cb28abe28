"""AddressSanitizer + UndefinedBehaviorSanitizer build of libq3's safetensors
header reader (decoder_only_qwen3_amd/csrc/checkpoint.cpp), the host code that
parses untrusted files: compiled with the host compiler (no device code) and
run over valid checkpoints, hand-made malformed headers and seeded random
mutations of a valid header.  Any sanitizer report fails the test."""
import json
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import q3synth
from checkpoint_files import write_checkpoint, write_raw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_only_qwen3_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    out = str(tmp_path_factory.mktemp("san") / "st_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", CSRC, os.path.join(CSRC, "checkpoint.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "st_header_check.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(checker, paths):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([checker, *map(str, paths)], capture_output=True, text=True, errors="replace", env=env,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def _valid_header_file(tmp_path):
    d = q3synth.tiny_dims(dtype="bf16")
    w = q3synth.make_weights(d, seed=5)
    p = tmp_path / "valid.safetensors"
    write_checkpoint(w, [str(p)], metadata={"format": "pt"})
    return p


def test_valid_and_malformed_headers(checker, tmp_path):
    good = _valid_header_file(tmp_path)
    files = [good]
    blob = bytes(64)

    def raw(name, header, data=blob, header_len=None):
        p = tmp_path / name
        write_raw(str(p), header, data, header_len)
        files.append(p)

    t = {"dtype": "BF16", "shape": [4, 8], "data_offsets": [0, 64]}
    raw("ok_small.st", {"a": t})
    raw("past_end.st", {"a": dict(t, data_offsets=[0, 6400])})
    raw("range_mismatch.st", {"a": dict(t, data_offsets=[0, 62])})
    raw("reversed.st", {"a": dict(t, data_offsets=[64, 0])})
    raw("huge_offsets.st", {"a": dict(t, data_offsets=[2 ** 63, 2 ** 64 - 1])})
    raw("negative_shape.st", {"a": dict(t, shape=[-4, -16])})
    raw("overflow_shape.st", {"a": dict(t, shape=[2 ** 40, 2 ** 40, 2 ** 40])})
    raw("unknown_dtype.st", {"a": dict(t, dtype="Q7")})
    raw("not_object.st", [1, 2, 3])
    raw("huge_header_len.st", {"a": t}, header_len=2 ** 62)
    raw("zero_header_len.st", {"a": t}, header_len=0)
    raw("metadata_only.st", {"__metadata__": {"k": "v"}})
    # JSON cut short, unterminated strings, deep nesting, bad escapes
    for i, text in enumerate([b'{"a": {"dtype": "BF16", "shape": [4, 8', b'{"a', b'{"a": "\\u12', b'[' * 5000,
                              b'{"a": {"dtype": "BF16", "shape": [4, 8], "data_offsets": [0, 64]}}}}}',
                              b'{"a": {"dtype": "BF16", "shape": [1e999], "data_offsets": [0, 64]}}',
                              b'{"a": {"dtype": "BF16", "shape": [4, 8], "data_offsets": [0, 64], "x": [[[[{}]]]]}}',
                              b'{' + b'"k":1,' * 2000 + b'"z":0}', b'\xff\xfe\x00\x01', b'']):
        p = tmp_path / f"text{i}.st"
        with open(p, "wb") as f:
            f.write(struct.pack("<Q", len(text)) + text + blob)
        files.append(p)
    short = tmp_path / "short.st"
    short.write_bytes(b"\x05\x00\x00")
    files += [short, tmp_path / "missing.st"]
    out = _run(checker, files)
    accepted = {os.path.basename(line.split()[-1]) for line in out.splitlines() if line.startswith("ok ")}
    # the valid checkpoint, the small valid file, a header of metadata only (no
    # tensors) and a tensor entry with an extra key (ignored); nothing else
    assert accepted == {"valid.safetensors", "ok_small.st", "metadata_only.st", "text6.st"}, accepted


def test_random_mutations_of_a_valid_header(checker, tmp_path):
    good = _valid_header_file(tmp_path).read_bytes()
    (n,) = struct.unpack("<Q", good[:8])
    rng = np.random.default_rng(2024)
    files = []
    for i in range(400):
        b = bytearray(good[:8 + n + 256])
        kind = i % 4
        if kind == 0:          # flip bytes inside the JSON
            for pos in rng.integers(8, 8 + n, size=int(rng.integers(1, 6))):
                b[pos] = int(rng.integers(0, 256))
        elif kind == 1:        # cut the file
            b = b[:int(rng.integers(0, len(b)))]
        elif kind == 2:        # change the header length
            b[:8] = struct.pack("<Q", int(rng.integers(0, 2 * n)))
        else:                  # insert or delete bytes inside the JSON
            pos = int(rng.integers(8, 8 + n))
            if rng.integers(0, 2):
                b[pos:pos] = bytes(rng.integers(32, 127, size=int(rng.integers(1, 8))).astype(np.uint8))
            else:
                del b[pos:pos + int(rng.integers(1, 8))]
        p = tmp_path / f"mut{i}.st"
        p.write_bytes(bytes(b))
        files.append(p)
    out = _run(checker, files)
    assert out.splitlines()[-1].endswith(f"of {len(files)} accepted")
