"""Helpers shared by the GPU parity tests (test code only)."""
import sys

import numpy as np

OUT_ATOL = 2e-3   # max-abs bar against the quantization-emulating oracle (unit-variance inputs)

# One record per output comparison of this session: (what, elements compared, max
# error, elements excused by the flip allowance, largest excess over the bar, the
# unit of that excess, largest ratio of an element's error to its own bound).
# tests/conftest.py prints them at the end of the run, whatever pytest captured.
RECORDS = []


def half_ulp_f16(x: np.ndarray) -> np.ndarray:
    """Half the fp16 spacing at |x|: the kernel stores fp16, so this much is format resolution."""
    return 0.5 * np.spacing(np.abs(np.asarray(x, dtype=np.float64)).astype(np.float16)).astype(np.float64)


def assert_output_parity(got: np.ndarray, ref: np.ndarray, atol: float = OUT_ATOL, what: str = "", extra=None):
    """|got - ref| <= atol + half an fp16 ulp of ref, element by element.

    `extra` is the oracle's first-order allowance for quantization codes of P that
    floating point may round either way (a P within a few ulps of a rounding
    boundary). It is capped at `atol`: an element whose error needs more than that
    fails even if the oracle's bound would excuse it. The number of elements that
    needed any allowance, and the largest allowance they used, are printed on
    every call that passes one.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    bound = atol + half_ulp_f16(ref)
    if extra is not None:
        extra = np.minimum(np.asarray(extra, dtype=np.float64), atol)
        excused = (err > bound) & (err <= bound + extra)
        n_exc = int(np.sum(excused))
        used = float(np.max(err - bound, where=excused, initial=0.0))
        say(f"  {what}: {n_exc} element(s) excused by the P-code flip allowance "
            f"(largest excess over the bar {used:.2e}; allowance capped at {atol:.0e})")
        bound = bound + extra
    bad = err > bound
    ratio = float(np.max(err / bound)) if err.size else 0.0
    RECORDS.append((what, err.size, float(err.max()) if err.size else 0.0,
                    n_exc if extra is not None else 0, used if extra is not None else 0.0, "", ratio))
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements over tolerance; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}; max err {err.max():.3e}")
    return float(err.max())


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
