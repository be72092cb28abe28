"""Writers of safetensors checkpoints for the tests (synthetic weights)."""
import json
import struct

import numpy as np
import torch
from safetensors.torch import save_file


def to_torch(arr: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def write_checkpoint(weights, paths, dtype="bf16", metadata=None):
    """Split `weights` (name -> float32 array) round-robin over `paths`."""
    names = sorted(weights)
    for k, path in enumerate(paths):
        part = {n: to_torch(weights[n], dtype) for n in names[k::len(paths)]}
        save_file(part, path, metadata=metadata)


def write_raw(path, header: dict, data: bytes, header_len=None):
    """A safetensors file from an explicit header object and data section."""
    h = json.dumps(header).encode()
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(h) if header_len is None else header_len))
        f.write(h)
        f.write(data)
