"""Shared helpers for the test suite: tolerance check, device upload of seeded inputs."""
import os

import numpy as np

# Elementwise bar for floating outputs against the fp64 oracle: |gpu - oracle| <= ATOL + RTOL * |oracle|.
ATOL = 1e-3
RTOL = 1e-2


def tol_violations(got, ref, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad = ~(np.abs(got - ref) <= atol + rtol * np.abs(ref))
    return int(bad.sum()), bad


def assert_within_tol(got, ref, what="", atol=ATOL, rtol=RTOL):
    n, bad = tol_violations(got, ref, atol, rtol)
    if n:
        idx = np.flatnonzero(bad.reshape(-1))[:8]
        g = np.asarray(got, np.float64).reshape(-1)
        r = np.asarray(ref, np.float64).reshape(-1)
        detail = ", ".join(f"[{i}] gpu={g[i]:.6g} oracle={r[i]:.6g}" for i in idx)
        raise AssertionError(f"{what}: {n} of {g.size} outside |d| <= {atol} + {rtol}|oracle|: {detail}")


def gpu_present() -> bool:
    return os.path.exists("/dev/kfd")


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run still shows where it was."""
    print(f"[gpu-case] {msg}", flush=True)
