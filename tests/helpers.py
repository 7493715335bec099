"""Shared helpers of the GPU parity tests (comparison metrics and tolerances)."""
import numpy as np
import torch

# Parity bars, as max|gpu - oracle| / max|oracle| over a whole output tensor:
# fp32 paths 1e-4, bf16 paths 2e-2.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to_np(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (bf16 / fp32) tensor on the host."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    denom = np.abs(ref).max()
    err = np.abs(got - ref).max()
    if denom == 0:
        return float(err)
    return float(err / denom)


# every parity figure measured in this process (the session summary prints them)
PARITY = []


def record_parity(what: str, err: float, tol: float) -> None:
    """Keep a measured parity figure for the session summary, and append it to
    $GDN_PARITY_LOG (JSON lines) when that is set."""
    import json
    import os
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    rec = {"test": test, "what": what, "err": float(err), "tol": tol}
    PARITY.append(rec)
    path = os.environ.get("GDN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def assert_close(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    tol = TOL[dtype]
    record_parity(what, e, tol)
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{what}: non-finite output"
    assert e <= tol, f"{what}: max-abs-err/max-abs-ref = {e:.3e} > {tol:.0e}"
    return e


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest even), as float64."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(torch.bfloat16).to(
        torch.float64).numpy()
