"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device and
the error measures the tolerances are stated in."""

import numpy as np
import torch

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rms(x):
    x = np.asarray(x)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def max_err_over_rms(x, ref):
    """max |x - ref| / RMS(ref): the measure the tolerances are stated in."""
    ref = np.asarray(ref)
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(rms(ref), 1e-30)) if ref.size else 0.0


def bf16_rne(t32: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even of a float32 tensor to bfloat16 (torch's cast)."""
    return t32.to(torch.bfloat16)
