"""Helpers for the GPU parity tests: seeded inputs, the library call, the
oracle, and the tolerance check."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import cache as OC

# Tolerances.  bf16 inputs with fp32 accumulation: max |err| <= 2e-2 and
# relative RMS <= 1e-2 on the output as the library returns it (rounded to
# the cache dtype).  fp32 inputs: the kernel rounds nothing but the order of
# fp32 sums, so 1e-3 / 1e-4.  Every case's raw errors are printed, and
# appended to the file DUO_ERRLOG names when that variable is set.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-3, 1e-4)}
_MANT_BITS = {"bf16": 7, "f32": 23}


def half_step(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the dtype's values at |ref| (its rounding error)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))  # a = m 2^e, 0.5 <= m < 1
    return np.where(a > 0, np.ldexp(1.0, e - 1 - _MANT_BITS[dtype] - 1), 0.0)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_kv_amd  # noqa: F401  (fails loudly if libduo.so is missing)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(x_f32: np.ndarray, dtype: str) -> torch.Tensor:
    return WL.to_torch(x_f32, dtype).cuda()


def stored(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """The float64 values the library actually sees after rounding."""
    return WL.round_to_dtype(x_f32, dtype)


def _log_errors(what: str, dtype: str, max_err: float, rel: float, ref_max: float) -> None:
    say(f"{what}: max|err| {max_err:.3e} rel-RMS {rel:.3e} (max|ref| {ref_max:.3g}, {dtype})")
    path = os.environ.get("DUO_ERRLOG")
    if path:
        with open(path, "a") as f:
            f.write(f"{what}\t{dtype}\t{max_err:.4e}\t{rel:.4e}\t{ref_max:.4g}\n")


def check_close(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str = ""):
    """max |got - ref| <= atol and ||got - ref|| / ||ref|| <= rel-RMS bound, on
    the output as returned (no allowance for its rounding)."""
    g = got.detach().float().cpu().double().numpy()
    atol, rrms = TOL[dtype]
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    max_err = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)) if err.size else 0.0
    _log_errors(what, dtype, max_err, rel, float(np.abs(ref).max()) if err.size else 0.0)
    assert max_err <= atol and rel <= rrms, (f"{what}: max|err| {max_err:.3e} (tol {atol}), "
                                            f"rel-RMS {rel:.3e} (tol {rrms})")
    return max_err, rel


def oracle_decode(q64, K64, V64, mask, S, W, scale):
    """q64 [B][n_q][d], K64/V64 [B][n_kv][T][d] -> [B][n_q][d] via the oracle's cache route."""
    return np.stack([OA.decode_step(q64[b], K64[b], V64[b], mask, S, W, scale) for b in range(q64.shape[0])])
