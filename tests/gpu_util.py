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


def assert_swiglu_close(h, g, mg, u, mu, what=""):
    """h = silu(g) u on the GPU, where its g and u are each within the product bar of the oracle's
    (g, mg) and (u, mu): |dh| <= |silu'| eg |u| + |silu(g)| eu + 1.1 eg eu with |silu'| <= 1.1,
    plus the SwiGLU bar on identical inputs (1e-5 |h| + 1e-5) for the fp32 evaluation itself."""
    import oracle

    eg, eu = 1e-3 * mg + 1e-5, 1e-3 * mu + 1e-5
    ref = oracle.swiglu(g, u)
    silu = g / (1.0 + np.exp(-np.clip(g, -700, 700)))
    bound = 1.1 * eg * np.abs(u) + np.abs(silu) * eu + 1.1 * eg * eu + 1e-5 * np.abs(ref) + 1e-5
    err = np.abs(np.asarray(h, np.float64) - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} of {err.size} outside the SwiGLU bound"
