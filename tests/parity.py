"""Comparison rule between the GPU results and the fp64 oracle.

Tolerances (stated for this method's bf16 path): on out, max|err| <= 2e-2 absolute
AND max|err| / max|ref| <= 1e-2 (a norm-wise relative error, since element-wise
relative error is meaningless near zero); on lse, max|err| <= 1e-3 absolute over
the finite entries, and the -inf entries (rows with no visible key) must match
exactly.  Rows with no visible key must also be exactly zero in out.
"""

import numpy as np

OUT_ABS = 2e-2
OUT_REL = 1e-2
LSE_ABS = 1e-3


def to_np(t):
    return t.detach().to("cpu", dtype=__import__("torch").float64).numpy() if hasattr(t, "detach") else np.asarray(t, np.float64)


def check_out(got, ref, what="out"):
    g, r = to_np(got), np.asarray(ref, np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite values (unwritten or NaN)"
    err = np.abs(g - r)
    max_err = float(err.max()) if err.size else 0.0
    scale = float(np.abs(r).max()) if r.size else 0.0
    assert max_err <= OUT_ABS, f"{what}: max abs err {max_err:.3e} > {OUT_ABS}"
    if scale > 0:
        assert max_err / scale <= OUT_REL, f"{what}: max err / max|ref| = {max_err / scale:.3e} > {OUT_REL}"
    return max_err


def check_lse(got, ref, what="lse"):
    g, r = to_np(got), np.asarray(ref, np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert not np.any(np.isnan(g)), f"{what}: NaN (unwritten?)"
    ninf_r, ninf_g = np.isneginf(r), np.isneginf(g)
    assert np.array_equal(ninf_r, ninf_g), f"{what}: -inf pattern differs ({ninf_r.sum()} vs {ninf_g.sum()})"
    fin = ~ninf_r
    if fin.any():
        assert np.all(np.isfinite(g[fin])), f"{what}: non-finite where the oracle is finite"
        err = float(np.abs(g[fin] - r[fin]).max())
        assert err <= LSE_ABS, f"{what}: max abs err {err:.3e} > {LSE_ABS}"
        return err
    return 0.0


def check_empty_rows_zero(out, lse_ref):
    """out [B,Sq,H,D]; rows whose oracle lse is -inf must be exactly 0."""
    o = to_np(out)
    l = np.asarray(lse_ref)
    b, h, i = np.nonzero(np.isneginf(l))
    if len(b):
        assert np.all(o[b, i, h, :] == 0.0), "rows with no visible key must be exactly zero"
