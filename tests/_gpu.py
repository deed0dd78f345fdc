"""Helpers for the GPU parity tests: upload seeded host arrays, compare results."""
import numpy as np
import pytest
import torch

from synth import bf16_bits, bits_to_f32

needs_gpu = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bf16(a) -> torch.Tensor:
    """float32 array holding bf16-exact values -> bf16 device tensor (same bits)."""
    bits = bf16_bits(np.asarray(a, np.float32))
    return torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)


def u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def nan_bf16(shape) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev())


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output (unwritten element?)"
    m = np.max(np.abs(ref)) if ref.size else 0.0
    if m == 0.0:
        assert np.all(got == 0.0), "reference is zero but output is not"
        return 0.0
    return float(np.max(np.abs(got - ref)) / m)


TOL = 1e-2  # max|err| / max|ref| for bf16-in / fp32-accumulate outputs


def log(msg):
    print(msg, flush=True)
