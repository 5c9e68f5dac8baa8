"""Helpers shared by the GPU parity tests: device copies, progress lines and
the tolerance check."""
import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def empty(shape, dtype=torch.float32) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within(got, ref, tol, what: str) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    ratio = err / tol
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    bad = ~(err <= tol)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"worst err/tol {worst:.3g} at {np.unravel_index(np.nanargmax(ratio), ratio.shape)}")
    return worst
