"""Non-finite inputs through every GEMM kind, against the oracle.

Reading (the pages leave it open; "Planned: Wan quantization and motion
parity", section "Current code reality", asks for guards that fail closed on
non-finite values): a 32-group holding NaN or +-Inf gets the E8M0 NaN scale
0xFF and every code 0x7F (E4M3 NaN), so it decodes to NaN. Every output that
reads such a group is then NaN, and every other output is unaffected. The
oracle's NaN rows and columns come from that rule alone; the GPU must put NaN
exactly there (``assert_linear_close`` compares the NaN pattern) and stay
within 1e-3 g sum|a||b| + one bf16 ulp everywhere else.

Covered: the slab GEMM, split-K, the few-token kernel (one and three K
ranges), the balanced GEMM with its split last round, the one-call
quantize + GEMM, the row-major and fused-prologue kernels, the requantizing
epilogue (NaN groups of the output requantize to 0xFF / 0x7F, finite groups
as the chain check allows) and the per-channel FP8 path (a row holding NaN
or Inf has scale NaN).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx, quant_ref, requant_range

pytestmark = pytest.mark.gpu

NAN, INF = float("nan"), float("inf")


def poisoned(M, K, N, seed, zero_row=None):
    """Seeded activations and weights with NaN, +Inf and -Inf in a few
    groups: token rows in the first tile, the second tile and the ragged
    tail; weight rows inside and at the end of the weight tiles."""
    x = synth.make_activation(M, K, seed)
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed)
    for r, c, v in ((3, 70, NAN), (5, K - 33, INF), (min(130, M - 2), 33, -INF), (M - 1, K - 1, NAN)):
        x[r, c] = v
    if zero_row is not None:
        x[zero_row] = 0
    for r, c, v in ((7, 9, INF), (N - 1, K // 2, NAN), (min(200, N - 2), 64, -INF)):
        w[r, c] = v
    return x, w, b


def oracle_ref(x, w, b, gelu):
    xq, xs = quant_ref(x)
    wq, ws = quant_ref(w)
    with np.errstate(invalid="ignore"):
        return oracle.linear_ref(xq, xs, wq, ws, bias=None if b is None else f64(b),
                                 epilogue="gelu_tanh" if gelu else "none")


def expect_nan_lines(yref, x, w):
    """The oracle's NaN outputs are exactly the poisoned token rows x all
    columns and all rows x the poisoned weight rows."""
    bad_m = ~np.isfinite(f64(x)).all(axis=1)
    bad_n = ~np.isfinite(f64(w)).all(axis=1)
    assert np.array_equal(np.isnan(yref), bad_m[:, None] | bad_n[None, :])


PLANS = [("slab", 1), ("splitk", 3), ("small", 1), ("small", 3), ("balanced", 1), ("slab_m128", 1)]


@pytest.mark.parametrize("plan", PLANS, ids=[f"{k}{s}" for k, s in PLANS])
@pytest.mark.parametrize("gelu", [False, True])
def test_nonfinite_groups_every_slab_kernel(plan, gelu):
    M, K, N = 300, 640, 272
    print(f"nonfinite {plan} gelu={gelu} M={M} K={K} N={N}", flush=True)
    d = dev()
    x, w, b = poisoned(M, K, N, seed=41, zero_row=9)
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    y = mx().mx_linear_slab_planned(plan, xs, ws, b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    yref, S = oracle_ref(x, w, b, gelu)
    expect_nan_lines(yref, x, w)
    assert_linear_close(y, yref, S, "gelu_tanh" if gelu else "none", what=f"{plan}")


def test_nonfinite_balanced_split_last_round():
    """17 x 16 = 272 tiles on 256 CUs: the last 16 tiles run split over K.
    One poisoned token row in every token tile and one poisoned weight row
    in every weight tile, so the split tiles see non-finite groups too."""
    M, K, N = 4352, 256, 4096
    print(f"nonfinite balanced M={M} K={K} N={N}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed=43)
    w = synth.make_weight(N, K, seed=43)
    b = synth.make_bias(N, seed=43)
    vals = (NAN, INF, -INF)
    for t in range(17):
        x[256 * t + (37 * t) % 256, (53 * t) % K] = vals[t % 3]
    for t in range(16):
        w[256 * t + (91 * t + 5) % 256, (29 * t) % K] = vals[(t + 1) % 3]
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    y = mx().mx_linear_slab_balanced(xs, ws, b.to(d))
    torch.cuda.synchronize()
    yref, S = oracle_ref(x, w, b, False)
    expect_nan_lines(yref, x, w)
    assert_linear_close(y, yref, S, what="balanced")


@pytest.mark.parametrize("path", ["onecall", "rowmajor", "fused"])
def test_nonfinite_groups_one_call_and_row_major(path):
    M, K, N = 300, 640, 272
    print(f"nonfinite {path} M={M} K={K} N={N}", flush=True)
    d = dev()
    x, w, b = poisoned(M, K, N, seed=47)
    xd, wd, bd = x.to(d), w.to(d), b.to(d)
    if path == "onecall":
        y = mx().mx_linear(xd, mx().mx_quantize_weight_slab(wd), bd)
    else:
        wq, wsc = mx().mx_quantize_weight(wd)
        if path == "fused":
            y = mx().mx_linear_fused(xd, wq, wsc, bd)
        else:
            xq, xsc = mx().mx_quantize_act(xd)
            y = mx().mx_linear_q(xq, xsc, wq, wsc, bd)
    torch.cuda.synchronize()
    yref, S = oracle_ref(x, w, b, False)
    expect_nan_lines(yref, x, w)
    assert_linear_close(y, yref, S, what=path)


def test_nonfinite_requant_epilogue():
    """The requantizing epilogue on outputs with NaN rows and columns: a
    32-group of the output holding a NaN must come out as scale 0xFF and 32
    codes 0x7F; finite groups as requant_range allows (exact where it fixes
    them)."""
    M, K, N = 300, 640, 320
    print(f"nonfinite requant M={M} K={K} N={N}", flush=True)
    d = dev()
    x, w, b = poisoned(M, K, N, seed=53)
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    h = mx().mx_linear_slab_requant(xs, ws, b.to(d), gelu=True)
    torch.cuda.synchronize()
    yref, S = oracle_ref(x, w, b, True)
    hq = h.q[:, :M].cpu().numpy().transpose(1, 0, 2).reshape(M, N)
    hs = h.s[:, :M].cpu().numpy().transpose(1, 0, 2).reshape(M, N // 32).astype(np.int64)
    nan_g = np.isnan(yref).reshape(M, N // 32, 32).any(axis=-1)
    assert nan_g.any() and (~nan_g).any()
    assert (hs[nan_g] == 0xFF).all(), "a group holding NaN did not get scale 0xFF"
    assert (hq.reshape(M, N // 32, 32)[nan_g] == 0x7F).all(), "a NaN group's codes are not 0x7F"
    rng = requant_range(np.nan_to_num(yref), np.nan_to_num(S), "gelu_tanh")
    fin = ~nan_g
    slo, shi = rng["slo"], rng["shi"]
    assert ((hs[fin] >= slo[fin]) & (hs[fin] <= shi[fin])).all(), "a finite group's scale is outside its range"
    fixed_s = fin & (slo == shi)
    assert np.array_equal(hs[fixed_s], slo[fixed_s])
    fin_e = np.repeat(fin, 32, axis=1)
    fixed = rng["fixed"] & fin_e
    assert np.array_equal(hq[fixed], rng["codes"][fixed]), "a code the oracle fixes differs"
    v = oracle.dequantize_mx(np.where(fin_e, hq, 0).astype(np.uint8), np.where(fin, hs, 0))
    ok = (v >= rng["qlo"]) & (v <= rng["qhi"])
    assert ok[fin_e].all(), "a finite group's code is outside its range"
    assert not h.q[:, M:].any() and not h.s[:, M:].any()  # pad rows stay zero


def test_nonfinite_per_channel_fp8():
    """Per-channel FP8: a row holding NaN or Inf has scale NaN and codes
    0x7F, so its whole output row (token) or column (weight) is NaN."""
    M, K, N = 300, 640, 272
    print(f"nonfinite per-channel M={M} K={K} N={N}", flush=True)
    d = dev()
    x, w, b = poisoned(M, K, N, seed=59)
    xp = mx().mx_pc_quantize_act_slab(x.to(d))
    wp = mx().mx_pc_quantize_weight_slab(w.to(d))
    y = mx().mx_pc_linear_slab(xp, wp, b.to(d), gelu=True)
    torch.cuda.synchronize()
    xq, xsc = oracle.quantize_pc(x.float().numpy())
    wq, wsc = oracle.quantize_pc(w.float().numpy())
    with np.errstate(invalid="ignore"):
        yref, S = oracle.linear_pc_ref(xq, xsc, wq, wsc, bias=f64(b), epilogue="gelu_tanh")
    expect_nan_lines(yref, x, w)
    assert_linear_close(y, yref, S, "gelu_tanh", what="per-channel")
