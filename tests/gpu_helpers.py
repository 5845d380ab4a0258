"""Helpers for the GPU tests: move exact storage bytes to the device and back.
No attention arithmetic here."""
import sys

import numpy as np

import attn_inputs as gen


def announce(what: str):
    """Name the case on stdout before a GPU step (flushed, so a run that dies
    still says which case it was in)."""
    print(f"\n[gpu case] {what}", flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_gpu(storage: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(storage).view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(storage, dtype=np.float32).copy())
    return t.to(dev())


def lens_gpu(L):
    import torch
    if L is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(L, dtype=np.int32)).to(dev())


def to_f64(t) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return gen.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


def max_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(gpu - ref).max()) if gpu.size else 0.0
