"""Shared helpers of the GPU parity tests (device upload, error norms)."""
import numpy as np
import pytest


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(a, torch):
    """numpy -> device tensor with the same dtype and shape."""
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def say(*a):
    print(*a, flush=True)


def row_rel_l2(got, want) -> float:
    """Largest relative L2 error of any row (first axis; the other axes flattened), so
    that one wrong row or tile cannot hide inside a tensor-wide norm."""
    got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    want = np.asarray(want, dtype=np.float64).reshape(len(want), -1)
    num = np.linalg.norm(got - want, axis=1)
    den = np.maximum(np.linalg.norm(want, axis=1), 1e-300)
    return float(np.max(num / den))
