"""Exact widening of bfloat16 tensors to float64 numpy arrays (oracle input side).

TEST INFRASTRUCTURE ONLY.  Every bfloat16 value is exactly representable in
float64, so this conversion loses nothing.
"""

import numpy as np
import torch


def widen(x) -> np.ndarray:
    """bfloat16 (or any float) CPU tensor / array -> float64 numpy array, exactly."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)
