"""Plain float64 reference of the MXFP8 W8A8 linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
bench's ``cpu_baseline`` leg, never by the product path, and it imports
nothing from the product package.

What the layer computes, and where that is stated:

* Model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)", section
  "Quantization Details": weights and activations are 8-bit of data type
  ``mx_fp`` with ``group_size`` 32 for both, symmetric, and the activation
  side is quantized on the fly; the checkpoint keeps E4M3 codes for the
  weights plus an E8M0 exponent for each run of 32 of them, and F16 biases.
* "Model Quantization Techniques" (LightX2V), section "MiniMax-H3 Video VAE
  Encoder Conv3D", mode table: the FP8 mode with FP32 accumulation uses the
  full E4M3 range, qmax 448 for weights and activations.

The pages name the formats but do not define their bit layouts, the shared
exponent rule or the rounding. The readings taken here are the OCP ones:
E4M3 "FN" (bias 7, no infinities, S.1111.111 is NaN, largest finite 448),
E8M0 (2**(c-127), 0xFF is NaN), shared exponent floor(log2 amax) - 8 clamped
to the E8M0 range, elements rounded to nearest with ties to even after
saturation to +-448, sign of zero kept, and a group holding NaN or Inf mapped
to scale 0xFF with every element 0x7F.

Every function is the definition written out with numpy; there is no
blocking, fusion or reordering beyond a matrix product.
"""

import numpy as np

GROUP = 32  # group_size and act_group_size of the quantization config
E4M3_MAX = 448.0  # largest finite E4M3 magnitude, 1.75 * 2**8
E4M3_EMAX = 8  # unbiased exponent of the top E4M3 binade
E8M0_BIAS = 127
E8M0_NAN = 0xFF
E4M3_NAN = 0x7F
GELU_SLOPE_MAX = 1.13  # bound on d/dv of GELU-tanh (its maximum is about 1.1290)


def e4m3_decode(codes):
    """Value of each FP8 E4M3 code as float64.

    Layout: bit 7 sign, bits 6..3 exponent E with bias 7, bits 2..0 mantissa
    m. E = 0 is subnormal, value m/8 * 2**-6. Otherwise (1 + m/8) * 2**(E-7).
    E = 15 with m = 7 is NaN; there are no infinities.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    E = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, E - 7)
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(E == 0, subnormal, normal)
    val = np.where(sign == 1, -mag, mag)
    return np.where((E == 15) & (m == 7), np.nan, val)


def e8m0_decode(codes):
    """Value of each E8M0 scale code: 2**(c - 127); code 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64)
    val = np.ldexp(np.ones(c.shape), c - E8M0_BIAS)
    return np.where(c == E8M0_NAN, np.nan, val)


# The 127 non-negative finite E4M3 magnitudes, codes 0x00..0x7E, ascending.
_MAGNITUDES = e4m3_decode(np.arange(0, 127))


def e4m3_encode(v):
    """FP8 E4M3 code of each float64 value.

    |v| is first saturated to 448, then rounded to the nearest of the 127
    non-negative finite magnitudes; an exact tie goes to the even code. The
    sign bit is copied from v, so -0.0 and negative values that round to zero
    give 0x80. NaN gives 0x7F.

    The distances below are exact in float64: adjacent magnitudes differ by
    at most a factor 2, so both subtractions are exact (Sterbenz).
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_MAGNITUDES, np.nan_to_num(a), side="left")
    hi = np.clip(hi, 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGNITUDES[lo]
    d_hi = _MAGNITUDES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo) | np.where(neg, 0x80, 0)
    code = np.where(np.isnan(v), E4M3_NAN, code)
    return code.astype(np.uint8)


def mx_scale_code(amax):
    """E8M0 code of the shared scale of a group whose largest |x| is amax.

    OCP MX: the scale is 2**(floor(log2 amax) - emax) with emax = 8, the
    exponent of the top E4M3 binade, clamped to the E8M0 range [-127, 127].
    amax = 0 has log2 = -inf and clamps to -127 (code 0x00). A group holding
    NaN or Inf (amax not finite) gets the NaN code 0xFF.
    """
    amax = np.asarray(amax, dtype=np.float64)
    # amax = f * 2**p with f in [0.5, 1): floor(log2 amax) = p - 1, exactly.
    _, p = np.frexp(np.nan_to_num(amax, nan=0.0, posinf=0.0))
    e = np.where(amax > 0, p - 1 - E4M3_EMAX, -E8M0_BIAS)
    e = np.clip(e, -127, 127)
    code = e + E8M0_BIAS
    code = np.where(np.isfinite(amax), code, E8M0_NAN)
    return code.astype(np.uint8)


def quantize_mx(x):
    """MXFP8 quantization of a float64 array along its last axis.

    Splits the last axis (length K, a multiple of 32) into groups of 32,
    takes each group's shared scale from its largest magnitude, and encodes
    x * 2**-e for every element. Returns (codes uint8 [..., K],
    scales uint8 [..., K/32]). The scaling by 2**-e is exact in float64 for
    every bf16 or fp32 input.
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (K // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)
    scales = mx_scale_code(amax)
    e = scales.astype(np.int64) - E8M0_BIAS
    scaled = np.ldexp(g, -e[..., None])
    codes = e4m3_encode(scaled)
    codes[scales == E8M0_NAN] = E4M3_NAN
    return codes.reshape(x.shape), scales


def dequantize_mx(codes, scales):
    """float64 value of MXFP8 data: decode(code) * 2**(scale - 127) per group."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (K // GROUP, GROUP))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def gelu_tanh(v):
    """GELU, tanh form: 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v**3)))."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v**3)))


def linear_ref(xq, xs, wq, ws, bias=None, epilogue="none"):
    """Reference output of the MXFP8 W8A8 linear, and its error scale.

    xq/xs: activation codes [M, K] and scales [M, K/32]; wq/ws: weight codes
    [N, K] and scales [N, K/32] (nn.Linear orientation); bias: the float
    values of the F16 bias [N], or None; epilogue: "none" or "gelu_tanh".

    y*[m, n] = phi(sum_k xhat[m, k] * what[n, k] + bias[n]) and
    S[m, n] = sum_k |xhat[m, k]| * |what[n, k]|, both in float64.
    """
    xh = dequantize_mx(xq, xs)
    wh = dequantize_mx(wq, ws)
    y = xh @ wh.T
    S = np.abs(xh) @ np.abs(wh).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if epilogue == "gelu_tanh":
        y = gelu_tanh(y)
    elif epilogue != "none":
        raise ValueError(f"unknown epilogue {epilogue!r}")
    return y, S


def bf16_ulp(y):
    """Spacing of bfloat16 numbers at |y| (8 significant bits; the
    subnormal spacing 2**-133 below 2**-126)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(np.nan_to_num(y, nan=0.0, posinf=0.0, neginf=0.0))
    _, p = np.frexp(a)  # a = f * 2**p, f in [0.5, 1): top bit is 2**(p-1)
    p = np.where(a > 0, p, -200)  # zero takes the subnormal spacing
    ulp = np.ldexp(np.ones(y.shape), np.maximum(p - 8, -133))
    return np.where(np.isfinite(y), ulp, np.nan)


def bf16_round(v):
    """Round float64 values to the nearest bfloat16, ties to even; values
    past the rounding boundary of the largest bf16 become +-inf."""
    v = np.asarray(v, dtype=np.float64)
    q = bf16_ulp(v)
    r = np.round(v / q) * q  # numpy rounds halves to even
    big = np.abs(r) > np.ldexp(2.0 - 2.0**-7, 127)
    return np.where(big, np.copysign(np.inf, v), r)


def tolerance(S, y_ref, epilogue="none"):
    """Allowed |y_gpu - y*|: 1e-3 * g * S plus one bf16 ulp of y*, with
    g = 1 for the identity epilogue and 1.13 (the largest slope of
    GELU-tanh) for gelu_tanh."""
    g = GELU_SLOPE_MAX if epilogue == "gelu_tanh" else 1.0
    return 1e-3 * g * np.asarray(S, dtype=np.float64) + bf16_ulp(y_ref)
