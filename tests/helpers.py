"""Shared helpers for the GPU parity tests: device access, tensor
conversion, and the element-wise acceptance check against the oracle."""

import os

import numpy as np
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def mx():
    """The product binding, building the library first if it is missing."""
    import mxfp8_w8a8_quantized_amd as pkg

    if not os.path.exists(pkg.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return pkg


def dev():
    assert torch.cuda.is_available(), "GPU test needs a HIP device"
    return torch.device("cuda:0")


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def u8(t):
    return t.detach().to("cpu").numpy()


def assert_linear_close(y_gpu, y_ref, S, epilogue="none", what=""):
    """|y_gpu - y*| <= 1e-3 g S + ulp_bf16(y*) element-wise (NaN must match NaN)."""
    y = f64(y_gpu) if isinstance(y_gpu, torch.Tensor) else np.asarray(y_gpu)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y), nan_ref), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(y[ok] - y_ref[ok])
    tol = oracle.tolerance(S[ok], y_ref[ok], epilogue)
    bad = err > tol
    if bad.any():
        i = np.argmax(err / tol)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst err {err[i]:.4g} tol {tol[i]:.4g} "
            f"ref {y_ref[ok][i]:.6g}"
        )
    return float((err / tol).max()) if err.size else 0.0


def quant_ref(t):
    """Oracle codes and scales of a bf16/f32 torch tensor (exact float64 values)."""
    return oracle.quantize_mx(f64(t))


# Chained linears (ffn.net.0.proj feeding ffn.net.2 through a requantized
# intermediate). The oracle runs the whole chain from the seeded inputs; the
# GPU's intermediate may round differently where the oracle's value sits near
# a bf16 or E4M3 rounding boundary, and those elements are given both sides of
# the boundary.
#
# CHAIN_RADIUS bounds |fp32 result - exact| / (g S) for one linear of the
# library: the GEMM adds the K/64 block sums of its MFMAs to an fp32
# accumulator one after another, so an output goes through at most
# K/64 + 64 roundings of relative size 2**-24 (counting each MFMA's internal
# sum of 64 exact products as 64 more); for K <= 16384 that is under
# 2**-15.7. 2**-14 leaves a margin of three. The epilogue's own evaluation
# (bias add, GELU-tanh) adds 2**-20 |y| at most.
CHAIN_RADIUS = 2.0**-14


def requant_range(y_star, S, epilogue="none"):
    """What the oracle fixes about the MX quantization of the bf16 rounding
    of a linear's output, whose exact value is y_star (float64 [.., N], N a
    multiple of 32) with error scale S.

    Returns a dict: "codes", "scales": the oracle's quantization of
    bf16(y_star); "slo", "shi": per group the range of scale codes an output
    within the radius can take; "qlo", "qhi": per element the range of values
    its code can dequantize to; "fixed": elements whose code is the same for
    every output within the radius.
    """
    g = oracle.GELU_SLOPE_MAX if epilogue == "gelu_tanh" else 1.0
    r = CHAIN_RADIUS * g * S + 2.0**-20 * np.abs(y_star)
    center = oracle.bf16_round(y_star)
    lo, hi = oracle.bf16_round(y_star - r), oracle.bf16_round(y_star + r)
    codes, scales = oracle.quantize_mx(center)
    G = oracle.GROUP
    shp = y_star.shape[:-1] + (y_star.shape[-1] // G, G)
    m_lo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi))).reshape(shp)
    m_hi = np.maximum(np.abs(lo), np.abs(hi)).reshape(shp)
    slo = oracle.mx_scale_code(m_lo.max(axis=-1)).astype(np.int64)
    shi = oracle.mx_scale_code(m_hi.max(axis=-1)).astype(np.int64)
    lo_g, hi_g = lo.reshape(shp), hi.reshape(shp)
    qlo = np.full(shp, np.inf)
    qhi = np.full(shp, -np.inf)
    for d in range(int((shi - slo).max()) + 1):
        c = np.minimum(slo + d, shi)[..., None]  # every code in [slo, shi]
        step = np.ldexp(1.0, c - oracle.E8M0_BIAS)
        c_lo, c_hi = oracle.e4m3_encode(lo_g / step), oracle.e4m3_encode(hi_g / step)
        qlo = np.minimum(qlo, oracle.e4m3_decode(c_lo) * step)
        qhi = np.maximum(qhi, oracle.e4m3_decode(c_hi) * step)
        if d == 0:  # E4M3 rounding is monotone in |v|: equal end codes fix the code
            fixed = (slo == shi)[..., None] & (c_lo == c_hi)
    return {"codes": codes, "scales": scales, "slo": slo, "shi": shi, "qlo": qlo.reshape(y_star.shape),
            "qhi": qhi.reshape(y_star.shape), "fixed": fixed.reshape(y_star.shape)}


def assert_requant_valid(hq, hs, rng, what=""):
    """GPU codes hq and scales hs of the requantized intermediate against
    requant_range: equal wherever the range fixes them, inside it elsewhere.
    Returns the fraction of elements whose code was not fixed."""
    hq, hs = np.asarray(hq), np.asarray(hs).astype(np.int64)
    slo, shi, fixed = rng["slo"], rng["shi"], rng["fixed"]
    assert np.array_equal(hs[slo == shi], slo[slo == shi]), f"{what}: a scale the oracle fixes differs"
    assert ((hs >= slo) & (hs <= shi)).all(), f"{what}: a scale outside its range"
    n_bad = int((hq[fixed] != rng["codes"][fixed]).sum())
    assert n_bad == 0, f"{what}: {n_bad} codes the oracle fixes differ"
    v = oracle.dequantize_mx(hq, hs)
    bad = ~((v >= rng["qlo"]) & (v <= rng["qhi"]))
    assert not bad.any(), f"{what}: {int(bad.sum())} codes outside their range"
    return float(1.0 - fixed.mean())


def assert_chain_close(y_gpu, y_star_up, S_up, epilogue_up, w2q, w2s, b2, what=""):
    """Output of the second linear of a chain, y_gpu, against the oracle's
    chain: y2* from the oracle's codes of bf16(y_star_up) and the weights
    (w2q, w2s), within the usual tolerance plus, for every element whose
    intermediate code is not fixed (requant_range), its widest possible
    dequantized difference times |w2|."""
    rng = requant_range(y_star_up, S_up, epilogue_up)
    codes, scales, qlo, qhi = rng["codes"], rng["scales"], rng["qlo"], rng["qhi"]
    y2, S2 = oracle.linear_ref(codes, scales, w2q, w2s, bias=b2)
    qc = oracle.dequantize_mx(codes, scales)
    delta = np.maximum(qhi - qc, qc - qlo)
    allow = delta @ np.abs(oracle.dequantize_mx(w2q, w2s)).T
    y = f64(y_gpu) if isinstance(y_gpu, torch.Tensor) else np.asarray(y_gpu)
    err = np.abs(y - y2)
    # The GPU multiplies codes whose values differ from the oracle's by at
    # most delta, so its exact sum z is within `allow` of y2 and its error
    # scale is at most S2 + allow. The usual bound on the GPU's rounding of z,
    # 1e-3 (S2 + allow) + ulp(|z|), plus |z - y2| <= allow gives the
    # tolerance below: `allow` enters once as the shift of the exact value;
    # inside the tolerance it only widens S and the ulp's argument.
    tol = oracle.tolerance(S2 + allow, np.abs(y2) + allow) + allow
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst err {err[i]:.4g} "
                             f"tol {tol[i]:.4g} (allowance {allow[i]:.4g})")
    return float((allow / S2).mean())
