"""Helpers shared by the GPU parity tests (test code only)."""
import sys

import numpy as np

OUT_ATOL = 2e-3   # max-abs bar against the quantization-emulating oracle (unit-variance inputs)


def half_ulp_f16(x: np.ndarray) -> np.ndarray:
    """Half the fp16 spacing at |x|: the kernel stores fp16, so this much is format resolution."""
    return 0.5 * np.spacing(np.abs(np.asarray(x, dtype=np.float64)).astype(np.float16)).astype(np.float64)


def assert_output_parity(got: np.ndarray, ref: np.ndarray, atol: float = OUT_ATOL, what: str = "", extra=None):
    """|got - ref| <= atol + half an fp16 ulp of ref (+ `extra`, the oracle's allowance for
    quantization codes that floating point may round either way, where given)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    bound = atol + half_ulp_f16(ref)
    if extra is not None:
        used = int(np.sum(err > bound))
        bound = bound + np.asarray(extra, dtype=np.float64)
        if used:
            say(f"  {what}: {used} element(s) within the P-code flip allowance "
                f"(largest allowance {float(np.max(extra)):.2e})")
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements over tolerance; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}; max err {err.max():.3e}")
    return float(err.max())


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
