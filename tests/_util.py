"""Helpers shared by the tests: moving seeded inputs to the device and comparing results."""
import numpy as np


def to_device(x, dtype, dev):
    """numpy array (float32, or uint16 bf16 bit patterns) -> torch tensor on dev."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.sqrt((a * a).sum()), np.sqrt((b * b).sum())
    if na == 0 or nb == 0:
        return 1.0 if na == nb else 0.0
    return float((a * b).sum() / (na * nb))


TOL = {"f32": dict(out=1e-4, lse=1e-4, cos=None), "bf16": dict(out=2e-2, lse=1e-3, cos=0.9999)}


def check_close(out, lse, o_ref, l_ref, dtype, what=""):
    """Element-wise gate: max |out - ref| and |lse - ref| within the dtype's tolerance, equal
    -inf pattern in lse, and (bf16) cosine over the compared outputs."""
    tol = TOL[dtype]
    out = np.asarray(out, np.float64)
    err = np.abs(out - o_ref).max() if out.size else 0.0
    assert err <= tol["out"], f"{what}: max|dO| = {err:.3e} > {tol['out']}"
    if tol["cos"] is not None and out.size and np.abs(o_ref).max() > 0:
        c = cosine(out, o_ref)
        assert c >= tol["cos"], f"{what}: cosine {c:.7f} < {tol['cos']}"
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        assert np.array_equal(np.isneginf(lse), np.isneginf(l_ref)), f"{what}: -inf pattern of lse differs"
        fin = np.isfinite(l_ref)
        if fin.any():
            el = np.abs(lse[fin] - l_ref[fin]).max()
            assert el <= tol["lse"], f"{what}: max|dlse| = {el:.3e} > {tol['lse']}"
    return err
