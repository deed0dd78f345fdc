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


CANARY = 4096          # bf16 elements placed after every output buffer
CANARY_BITS = 0x5A5A   # their bit pattern (a finite value no kernel writes by chance)


CANARY_BITS32 = 0x5A5A5A5A  # the same for fp32 output buffers


def _check_canary(t: torch.Tensor):
    base = getattr(t, "_wide_canary", None)
    if base is not None:
        if base.dtype == torch.float32:
            tail = base[t.numel():].view(torch.int32).cpu().numpy().view(np.uint32)
            assert np.all(tail == CANARY_BITS32), "an output buffer was written past its end"
            return
        tail = base[t.numel():].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.all(tail == CANARY_BITS), "an output buffer was written past its end"


def host(t: torch.Tensor) -> np.ndarray:
    _check_canary(t)
    if t.dtype == torch.bfloat16:
        return bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def nan_bf16(shape) -> torch.Tensor:
    """An output buffer: NaN everywhere (an element the call leaves unwritten stays
    NaN), followed by a canary region that host() checks is untouched."""
    n = int(np.prod(shape))
    base = torch.empty(n + CANARY, dtype=torch.bfloat16, device=dev())
    base.view(torch.int16)[n:] = np.int16(np.uint16(CANARY_BITS).view(np.int16))
    base[:n] = float("nan")
    y = base[:n].view(shape)
    y._wide_canary = base
    return y


def nan_f32(shape) -> torch.Tensor:
    """nan_bf16 for an fp32 output buffer."""
    n = int(np.prod(shape))
    base = torch.empty(n + CANARY, dtype=torch.float32, device=dev())
    base.view(torch.int32)[n:] = np.int32(np.uint32(CANARY_BITS32).view(np.int32))
    base[:n] = float("nan")
    y = base[:n].view(shape)
    y._wide_canary = base
    return y


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
