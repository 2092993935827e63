"""Tolerance checks used by the parity tests.

Test infrastructure (see the package docstring); never used by the product path.

GEMM, per element:  |C_gpu - C_exact| <= ulp_bf16(|C_exact|) + 1e-4 * sum_k |a_k w_k|
Producer:           residual bit-exact; scale relative error <= 1e-6; e4m3
                    codes within 1 step of the value-ordered lattice on at most
                    0.1% of elements and never further.
"""
import numpy as np

from .codecs import decode_bf16, bf16_ulp, e4m3_step_index

GEMM_REL_ABS = 1e-4
SCALE_REL = 1e-6
CODE_FRAC = 1e-3


def gemm_violations(c_gpu_bits, c_exact, abs_sum):
    """Boolean mask of elements outside the GEMM tolerance, and the slack
    |delta| / bound (<= 1 means within)."""
    got = decode_bf16(c_gpu_bits)
    bound = bf16_ulp(c_exact) + GEMM_REL_ABS * np.asarray(abs_sum, np.float64)
    delta = np.abs(got - c_exact)
    bad = ~(delta <= bound)            # NaN in got counts as bad
    return bad, delta / bound


def assert_gemm_close(c_gpu_bits, c_exact, abs_sum, what=""):
    bad, ratio = gemm_violations(c_gpu_bits, c_exact, abs_sum)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        got = decode_bf16(c_gpu_bits)
        detail = [(tuple(i), float(got[tuple(i)]), float(np.asarray(c_exact)[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; "
                             f"max ratio {np.nanmax(ratio):.3g}; first {detail}")
    return float(np.max(ratio)) if ratio.size else 0.0


def producer_report(q_gpu, s_gpu, r_gpu, q_ref, s_ref, r_ref):
    """Return a dict of the producer's parity figures."""
    r_mismatch = int(np.count_nonzero(np.asarray(r_gpu, np.uint16) != np.asarray(r_ref, np.uint16)))
    s_ref64 = np.asarray(s_ref, np.float32).astype(np.float64)
    s_rel = np.abs(np.asarray(s_gpu, np.float32).astype(np.float64) - s_ref64) / s_ref64
    steps = np.abs(e4m3_step_index(q_gpu) - e4m3_step_index(q_ref))
    return {
        "residual_mismatch": r_mismatch,
        "scale_max_rel": float(np.max(s_rel)) if s_rel.size else 0.0,
        "codes_off_by_one": int(np.count_nonzero(steps == 1)),
        "codes_off_more": int(np.count_nonzero(steps > 1)),
        "codes_total": int(steps.size),
    }


def assert_producer_close(q_gpu, s_gpu, r_gpu, q_ref, s_ref, r_ref, what=""):
    rep = producer_report(q_gpu, s_gpu, r_gpu, q_ref, s_ref, r_ref)
    ok = (rep["residual_mismatch"] == 0 and rep["scale_max_rel"] <= SCALE_REL
          and rep["codes_off_more"] == 0
          and rep["codes_off_by_one"] <= CODE_FRAC * max(rep["codes_total"], 1))
    if not ok:
        raise AssertionError(f"{what}: producer parity failed: {rep}")
    return rep


def assert_codes_close(q_gpu, s_gpu, q_ref, s_ref, what=""):
    """Quantizer parity without a residual output (same scale / code bars)."""
    s_ref64 = np.asarray(s_ref, np.float32).astype(np.float64)
    s_rel = np.abs(np.asarray(s_gpu, np.float32).astype(np.float64) - s_ref64) / s_ref64
    steps = np.abs(e4m3_step_index(q_gpu) - e4m3_step_index(q_ref))
    rep = {"scale_max_rel": float(s_rel.max()) if s_rel.size else 0.0,
           "codes_off_by_one": int(np.count_nonzero(steps == 1)),
           "codes_off_more": int(np.count_nonzero(steps > 1)), "codes_total": int(steps.size)}
    if not (rep["scale_max_rel"] <= SCALE_REL and rep["codes_off_more"] == 0
            and rep["codes_off_by_one"] <= CODE_FRAC * max(rep["codes_total"], 1)):
        raise AssertionError(f"{what}: quantizer parity failed: {rep}")
    return rep
