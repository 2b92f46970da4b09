"""Device-side helpers for the GPU parity tests (not a test module)."""
import numpy as np
import pytest
import torch

DEV = torch.device("cuda:0")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def lib():
    import gradient_compression_error_amd as gc
    return gc


def to_dev(a: np.ndarray) -> torch.Tensor:
    """float32 array -> float32 device tensor; uint16 (bf16 bit patterns) -> bfloat16 device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def f32_bits(t) -> np.ndarray:
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


class TopkRunner:
    """Allocates outputs + workspace once for a (d, k) and runs encode/decode."""

    def __init__(self, d, k):
        gc = lib()
        self.d, self.k = d, k
        self.idx = torch.empty(k, dtype=torch.int32, device=DEV)
        self.val = torch.empty(k, dtype=torch.float32, device=DEV)
        self.out = torch.empty(d, dtype=torch.float32, device=DEV)
        self.ws = torch.empty(gc.gc_topk_workspace_bytes(d, k), dtype=torch.uint8, device=DEV)

    def encode(self, grad_t, mem_t, eta):
        lib().gc_topk_ef_encode(grad_t, mem_t, eta, self.k, self.idx, self.val, self.ws)

    def decode(self, accumulate=False):
        lib().gc_topk_decode(self.idx, self.val, self.out, accumulate=accumulate)


def rel_err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / den) if den > 0 else float(np.linalg.norm(got - want))
