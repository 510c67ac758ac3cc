"""Helpers for the GPU tier: device buffers through PyTorch (plumbing only),
bf16 bit patterns, and the parity metrics."""
import sys

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefill_only_decision_amd as s1
    s1.load_library()   # raises when the HIP library is missing: never a silent skip
    return torch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bits(bits_u16):
    """uint16 bf16 bit patterns -> int16 device tensor (same bytes)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (n if n > 0 else 1.0))


def stream_ptr():
    import torch
    return torch.cuda.current_stream().cuda_stream
