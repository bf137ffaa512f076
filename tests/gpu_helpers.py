"""Shared helpers of the GPU parity tests (comparison rules and case logging)."""
import sys

import numpy as np

# Attention outputs vs the oracle's identical fake-quant numerics: max-abs 2e-3
# and relative L2 1e-3 over the compared elements, on binary32 outputs.
ATOL = 2e-3
REL_L2 = 1e-3


def case(msg: str):
    """Name the case on stdout before a GPU step, so a fault is attributable."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def assert_close_attn(got, ref, what="attention"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= ATOL and rel <= REL_L2, f"{what}: max-abs {err.max():.3e} rel-L2 {rel:.3e}"
    return err.max(), rel
