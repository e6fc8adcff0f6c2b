"""Helpers of the GPU parity tests: upload seeded host tensors, read results back, tolerances.

Tolerances (stated in the workloads' contract):
  fp32 inputs: max |O - O_ref| <= 1e-5 * max |O_ref|            (normwise)
  bf16 inputs: |O - O_ref| <= 2e-3 + 2e-2 * |O_ref|  elementwise (fp32 accumulation)
O_ref is the fp64 oracle on the exact stored input values.
"""
import sys

import numpy as np
import torch

import workloads as W


def say(*args):
    """Print and flush before each GPU step so a failing run names its case."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev(t: W.HostTensor) -> torch.Tensor:
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.data)).cuda()


def dev_idx(a, dtype) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dtype).cuda()


def host64(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def stacked_A(A: W.HostTensor) -> W.HostTensor:
    """[d_model, N*r] (the pages' A_k side by side) -> [N*r, d_model] (the ABI's stacked LoRA A weights)."""
    return W.HostTensor(np.ascontiguousarray(A.data.T), A.dtype)


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    stats = {"max_abs_err": float(err.max()), "normwise": float(err.max() / scale)}
    if dtype == "f32":
        assert stats["normwise"] <= 1e-5, f"{what}: normwise error {stats['normwise']:.3e} > 1e-5"
    else:
        bound = 2e-3 + 2e-2 * np.abs(ref)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 2e-3 + 2e-2|ref|; "
                               f"worst excess {float((err - bound).max()):.3e}")
    return stats
