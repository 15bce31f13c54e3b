"""Tolerance checks shared by the GPU parity tests.

bf16 gate (stated for the method): max|T - T_ref| <= 2e-2 + 1e-2 * max|T_ref|
for O, dQ, dK, dV (and L).  A second, tighter gate catches outputs that are
small in magnitude and therefore pass the absolute term trivially (e.g. all
zeros): the relative Frobenius error ||T - T_ref|| / ||T_ref|| must stay below
REL_FRO.  Its value comes from the arithmetic: bf16 rounding of P or dS before
the products (2^-9 relative per element, averaging out over the sums) and of
the outputs (2^-9), so a correct kernel sits near 3e-3; 2e-2 leaves margin.
fp32 gate: max|T - T_ref| <= 1e-5.
"""
import numpy as np

BF16_ABS = 2e-2
BF16_REL_MAX = 1e-2
REL_FRO = 2e-2
F32_ABS = 1e-5


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def check_bf16(name, got, ref, rel_fro=REL_FRO):
    got, ref = _np(got), _np(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref).max() if got.size else 0.0
    ref_max = np.abs(ref).max() if ref.size else 0.0
    tol = BF16_ABS + BF16_REL_MAX * ref_max
    nrm = np.linalg.norm(ref)
    fro = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got - ref)
    msg = f"{name}: max_abs_err={err:.3e} tol={tol:.3e} rel_fro={fro:.3e} (max|ref|={ref_max:.3e})"
    assert err <= tol, msg
    assert fro <= rel_fro, msg
    return err, fro


def check_f32(name, got, ref):
    got, ref = _np(got), _np(ref)
    assert got.shape == ref.shape
    err = np.abs(got - ref).max()
    assert err <= F32_ABS, f"{name}: max_abs_err={err:.3e} > {F32_ABS}"
    return err
