"""Helpers for the GPU parity tests: device upload and the product tolerance."""
import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """Copy a host array to cuda:0 (allocations are at least 256-byte aligned)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_product_close(got, ref, mag, rel=1e-3, abs_=1e-5, what=""):
    """|got - ref| <= rel * sum|w x| + abs_, element by element."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = rel * mag + abs_
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r} err {err[i]:.3e} bound "
                             f"{bound[i]:.3e}")
    return float(np.max(err / bound)) if err.size else 0.0
