"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch

RTOL = 1e-3   # elementwise |gpu - oracle| <= ATOL + RTOL * |oracle|
ATOL = 1e-4


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_close(got, ref, what: str, rtol: float = RTOL, atol: float = ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    lim = atol + rtol * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
                             f"gpu={got.flat[i]!r} oracle={ref.flat[i]!r} err={err.flat[i]:.3e} lim={lim.flat[i]:.3e}")
    return float((err / lim).max()) if err.size else 0.0


def say(msg: str):
    print(msg, flush=True)
