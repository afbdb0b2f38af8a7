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
