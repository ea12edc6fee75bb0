"""Shared helpers of the GPU parity tests: tolerances and comparisons."""
import numpy as np

import oracle

# fp32 path: max abs error <= 1e-4.  bf16 path (bf16 operands, fp32
# accumulation and softmax): max abs error <= 2e-2 and aggregate relative
# error sum|y - ref| / sum|ref| <= 5e-3.
TOL = {"f32": dict(max_abs=1e-4), "bf16": dict(max_abs=2e-2, mean_rel=5e-3)}


def gpu_to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma = oracle.max_abs_err(got, ref)
    mr = oracle.mean_rel_err(got, ref)
    tol = TOL[dtype]
    print(f"[parity] {what} dtype={dtype} max_abs={ma:.3e} mean_rel={mr:.3e} rms_ref={np.sqrt(np.mean(ref**2)):.3e}",
          flush=True)
    assert ma <= tol["max_abs"], f"{what}: max_abs {ma:.3e} > {tol['max_abs']}"
    if "mean_rel" in tol:
        assert mr <= tol["mean_rel"], f"{what}: mean_rel {mr:.3e} > {tol['mean_rel']}"
    return ma, mr
