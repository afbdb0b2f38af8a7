"""Plain reference of the per-output-channel FP8 linear (the second FP8
scheme on the pages).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the bench's
``cpu_baseline`` leg, never by the product path; it imports nothing from the
product package.

What it computes, and where that is stated:

* "Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4", section
  "Conversion and compatibility": FP8 weights are E4M3 with one FP32 scale per
  output channel, rounded to nearest.
* "Model Quantization Techniques" (LightX2V), quantization mode table: FP8
  weights "channel symmetric", FP8 activations "channel dynamic symmetric"
  (one scale per token row, computed at run time); the fp8-f16-accum section
  states the dynamic row rule, scale = max(abs(x)) / qmax; the Conv3D mode
  table gives qmax 448 (the full E4M3 range) with FP32 accumulation.

Readings where the pages leave a step open (taken as the plainest ones):

* The scale is computed in FP32 (the pages' "FP32 scales"): s = fp32(amax) /
  fp32(448), and the element is encoded from the FP32 quotient fp32(x) / s,
  both divisions rounded to nearest even; the E4M3 encoding is the same as
  the MX path's (round to nearest, ties to even, saturate to +-448, sign of
  zero kept).
* A row whose scale is 0 (all zeros, or amax so small that amax / 448
  underflows) encodes every element as a signed zero; a row holding NaN or
  Inf gets scale NaN and every code 0x7F.
* The linear: y[m, n] = phi(s_x[m] * s_w[n] * sum_k dec(qx[m, k]) *
  dec(qw[n, k]) + bias[n]), accumulated in FP32 on the device, here in
  float64.

Every function is the definition written out with numpy.
"""

import numpy as np

from .mx_oracle import E4M3_MAX, E4M3_NAN, e4m3_decode, e4m3_encode, gelu_tanh

QMAX = np.float32(E4M3_MAX)  # 448: the FP32-accumulation qmax


def quantize_pc(x):
    """Per-row FP8 quantization along the last axis.

    x: array of float32-representable values [..., K]. Returns (codes uint8
    [..., K], scales float32 [...]) with scale = fp32(max |x|) / 448 and
    code = E4M3(fp32(x) / scale).
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        scale = (amax / QMAX).astype(np.float32)
        q = (x32 / scale[..., None]).astype(np.float32)
    zero = scale == 0
    q = np.where(zero[..., None], np.copysign(np.float32(0.0), x32), q)  # signed zeros
    codes = e4m3_encode(q.astype(np.float64))
    bad = ~np.isfinite(amax)
    codes[bad] = E4M3_NAN
    scale = np.where(bad, np.float32(np.nan), scale).astype(np.float32)
    return codes, scale


def dequantize_pc(codes, scales):
    """float64 value of per-row FP8 data: dec(code) * scale of its row."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def linear_pc_ref(xq, xs, wq, ws, bias=None, epilogue="none"):
    """Reference output of the per-channel FP8 linear and its error scale.

    xq [M, K] codes with row scales xs [M]; wq [N, K] codes with per-output-
    channel scales ws [N]; bias: float values [N] or None.
    y*[m, n] = phi(xs[m] ws[n] sum_k dec(xq[m, k]) dec(wq[n, k]) + bias[n]),
    S[m, n] = |xs[m] ws[n]| sum_k |dec(xq[m, k])| |dec(wq[n, k])|, float64.
    """
    xd = e4m3_decode(xq)
    wd = e4m3_decode(wq)
    sc = np.asarray(xs, dtype=np.float64)[:, None] * np.asarray(ws, dtype=np.float64)[None, :]
    y = sc * (xd @ wd.T)
    S = np.abs(sc) * (np.abs(xd) @ np.abs(wd).T)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if epilogue == "gelu_tanh":
        y = gelu_tanh(y)
    elif epilogue != "none":
        raise ValueError(f"unknown epilogue {epilogue!r}")
    return y, S
