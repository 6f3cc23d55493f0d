"""Helpers for the GPU parity tests: device upload of bf16 bit patterns and
the parity bars (written out here, per the method's tolerances)."""
import numpy as np
import torch

import oracle

# Parity bars: forward max|diff| <= 2e-2 and ||diff||/||ref|| <= 1e-2;
# gradients both <= 5e-2; LSE (fp32) max|diff| <= 1e-3; swaps bit-exact.
FWD_MAX_ABS, FWD_REL = 2e-2, 1e-2
GRAD_MAX_ABS, GRAD_REL = 5e-2, 5e-2
LSE_MAX_ABS = 1e-3


def dev(a: np.ndarray) -> torch.Tensor:
    """uint16 numpy bits -> int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """16-bit device tensor -> uint16 numpy bits."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(host(t))


def sentinel(shape, dtype=torch.int16) -> torch.Tensor:
    """Output buffer pre-filled with 0xFFFF (a NaN in bf16) to expose unwritten elements."""
    return torch.full(shape, -1, dtype=dtype, device="cuda")


def stats(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    nr = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nr) if nr > 0 else mx
    return mx, rel


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, max_abs: float, rel: float):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values (unwritten or overflow)" % name
    mx, rl = stats(got, ref)
    print("%s: max|diff|=%.3e rel_l2=%.3e (bars %.0e / %.0e)" % (name, mx, rl, max_abs, rel), flush=True)
    assert mx <= max_abs and rl <= rel, "%s: max|diff|=%.3e rel_l2=%.3e" % (name, mx, rl)
