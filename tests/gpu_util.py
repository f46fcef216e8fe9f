"""Helpers for the GPU parity tests: move seeded inputs to the device and back."""
import numpy as np
import torch

import synth


def device_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda")


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return synth.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


TOL = {"bf16": {"o": 2e-2, "lse": 1e-3, "grad": 2e-2}, "f32": {"o": 1e-4, "lse": 1e-4, "grad": 1e-4}}
