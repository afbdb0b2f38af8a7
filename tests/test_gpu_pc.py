"""GPU parity of the per-output-channel FP8 path (mx_pc_quantize_act_slab,
mx_pc_quantize_weight_slab, mx_pc_linear_slab) against the oracle
(oracle/pc_oracle.py): codes and f32 scales bit-exact on seeded inputs, the
linear within 1e-3 g S + one bf16 ulp with S = |s_x s_w| sum |dec| |dec|.

Sources: "Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4",
section "Conversion and compatibility"; "Model Quantization Techniques"
(LightX2V), quantization mode table and the row rule scale = max|x| / qmax,
qmax 448 with FP32 accumulation.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx

pytestmark = pytest.mark.gpu


def rows_of(sl, rows):
    """Row-major codes and scales of the given rows of a PCSlab (numpy)."""
    q = sl.q[:, rows].cpu().numpy()
    return q.transpose(1, 0, 2).reshape(len(rows), -1), sl.s[rows].cpu().numpy()


def same_f32(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.int32), np.asarray(b, np.float32).view(np.int32))


def check_quant(sl, x_host, rows=None):
    n = x_host.shape[0]
    rows = np.arange(n) if rows is None else rows
    q, s = rows_of(sl, torch.from_numpy(rows))
    rq, rs = oracle.quantize_pc(x_host[rows])
    assert np.array_equal(q, rq), f"{int((q != rq).sum())} codes differ"
    assert same_f32(s, rs), "scales differ"


@pytest.mark.parametrize("M,K", [(1, 64), (77, 192), (256, 128), (300, 5120), (513, 640), (5, 13824)])
def test_pc_act_quantizer_matches_oracle(M, K):
    x = synth.make_activation(M, K, seed=M + K)
    sl = mx().mx_pc_quantize_act_slab(x.to(dev()))
    torch.cuda.synchronize()
    check_quant(sl, x.float().numpy())
    assert not sl.q[:, M:].any() and not sl.s[M:].any()  # pad rows


def test_pc_act_quantizer_strided_and_special_rows():
    base = synth.make_activation(12, 384, seed=9)
    base[1] = 0
    base[2, 0] = -0.0
    base[3, 5] = float("nan")
    base[4, 7] = float("inf")
    base[5, 9] = -float("inf")
    base[6] = torch.tensor(2.0**-133, dtype=torch.bfloat16)  # bf16 subnormals: a subnormal f32 scale
    base[6, 3] = -base[6, 3]
    x = base[:, 64:320]  # pitch 384, K 256
    sl = mx().mx_pc_quantize_act_slab(x.to(dev()))
    torch.cuda.synchronize()
    check_quant(sl, x.float().numpy())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pc_weight_quantizer_matches_oracle(dtype):
    w = synth.make_weight(300, 1024, seed=4).to(dtype)
    sl = mx().mx_pc_quantize_weight_slab(w.to(dev()))
    torch.cuda.synchronize()
    check_quant(sl, w.float().numpy())


def test_pc_act_quantizer_full_size_sampled_rows():
    M, K = synth.VIDEO_TOKENS, synth.HIDDEN
    x = synth.make_activation(M, K, seed=21)
    sl = mx().mx_pc_quantize_act_slab(x.to(dev()))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(M - 84, M), rng.integers(0, M, 96)]))
    q, s = rows_of(sl, torch.from_numpy(rows))
    rq, rs = oracle.quantize_pc(x[rows].float().numpy())
    assert np.array_equal(q, rq) and same_f32(s, rs)
    assert not sl.q[:, M:].any() and not sl.s[M:].any()


def run_pc(M, K, N, seed, bias=True, gelu=False, x=None):
    d = dev()
    x = synth.make_activation(M, K, seed) if x is None else x
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed) if bias else None
    xs = mx().mx_pc_quantize_act_slab(x.to(d))
    ws = mx().mx_pc_quantize_weight_slab(w.to(d))
    y = mx().mx_pc_linear_slab(xs, ws, None if b is None else b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    return x, w, b, y


def oracle_pc(x, w, b, gelu):
    xq, xs = oracle.quantize_pc(x.float().numpy())
    wq, ws = oracle.quantize_pc(w.float().numpy())
    return oracle.linear_pc_ref(xq, xs, wq, ws, bias=None if b is None else f64(b),
                                epilogue="gelu_tanh" if gelu else "none")


@pytest.mark.parametrize(
    "M,K,N",
    [(1, 64, 16), (5, 64, 32), (77, 192, 256), (256, 128, 256), (300, 320, 512), (513, 512, 272), (70, 5120, 768)],
)
def test_pc_linear_small_shapes(M, K, N):
    print(f"pc linear M={M} K={K} N={N}", flush=True)
    x, w, b, y = run_pc(M, K, N, seed=M * 5 + K + N)
    yref, S = oracle_pc(x, w, b, False)
    assert_linear_close(y, yref, S, what=f"pc M{M} K{K} N{N}")


def test_pc_linear_gelu_no_bias():
    x, w, b, y = run_pc(300, 256, 512, seed=6, bias=False, gelu=True)
    yref, S = oracle_pc(x, w, None, True)
    assert_linear_close(y, yref, S, "gelu_tanh", what="pc gelu")


def test_pc_linear_zero_rows_give_bias_and_deterministic():
    ctx = synth.make_text_context(512, 5120, seed=3)
    x, w, b, y = run_pc(512, 5120, 1024, seed=3, x=ctx)
    want = f64(b.float().to(torch.bfloat16))  # bf16(f32(bias)): the zero rows' scale is 0
    assert np.array_equal(f64(y)[410:], np.broadcast_to(want, (102, 1024)))
    yref, S = oracle_pc(x, w, b, False)
    assert_linear_close(y, yref, S, what="pc text ctx")
    _, _, _, y2 = run_pc(512, 5120, 1024, seed=3, x=ctx)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_pc_linear_qkv_full_size():
    d = dev()
    shp = synth.CONFIGS["qkv_75348x5120x15360"][0]
    print(f"pc qkv {shp}", flush=True)
    x = synth.make_activation(shp.M, shp.K, 200)
    w = synth.make_weight(shp.N, shp.K, 200)
    b = synth.make_bias(shp.N, 200)
    xs = mx().mx_pc_quantize_act_slab(x.to(d))
    ws = mx().mx_pc_quantize_weight_slab(w.to(d))
    y = mx().mx_pc_linear_slab(xs, ws, b.to(d))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(shp.M - 84, shp.M), rng.integers(0, shp.M, 96)]))
    xq, xsr = oracle.quantize_pc(x[rows].float().numpy())
    wq, wsr = oracle.quantize_pc(w.numpy())
    yref, S = oracle.linear_pc_ref(xq, xsr, wq, wsr, bias=f64(b))
    assert_linear_close(y[rows], yref, S, what="pc qkv")


def test_pc_quantizer_quotients_at_rounding_ties():
    # Rows whose quotients x / s land on, and one or two float32 ulps around,
    # E4M3 rounding midpoints (ties go to the even code), under scales with
    # long significands: the quantizer's quotient must be the correctly
    # rounded one for the codes to match the oracle's.
    rng = np.random.default_rng(5)
    mags = oracle.e4m3_decode(np.arange(0, 127)).astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2  # E4M3 rounding boundaries, exact in float32
    rows = []
    for _ in range(64):
        amax = np.float32(rng.uniform(0.5, 64.0))
        s = np.float32(amax / np.float32(448.0))
        targets = rng.choice(mids, 255)
        vals = (targets * np.float64(s)).astype(np.float32)  # quotient within an ulp or two of a midpoint
        for d in (-2, -1, 1, 2):
            idx = rng.integers(0, 255, 32)
            for _ in range(abs(d)):
                vals[idx] = np.nextafter(vals[idx], np.float32(np.sign(d) * np.inf))
        vals = np.concatenate([[amax], np.minimum(np.abs(vals), amax) * rng.choice([-1, 1], 255)]).astype(np.float32)
        rows.append(vals)
    w = torch.from_numpy(np.stack(rows))  # [64, 256] f32: the weight path takes f32
    sl = mx().mx_pc_quantize_weight_slab(w.to(dev()))
    torch.cuda.synchronize()
    check_quant(sl, w.numpy())
    xb = w.to(torch.bfloat16)  # and the activation path, on the bf16-rounded rows
    sl = mx().mx_pc_quantize_act_slab(xb.to(dev()))
    torch.cuda.synchronize()
    check_quant(sl, xb.float().numpy())


def test_pc_offsets_past_4gib():
    # As the MX path's test: 2^20 + 77 rows of a repeated seeded block, the
    # per-channel code slab past 2^32 bytes; codes, scales and outputs of
    # sampled rows against the oracle.
    d = dev()
    M, K, N = (1 << 20) + 77, 5120, 256
    base = synth.make_activation(1000, K, seed=62)
    w, b = synth.make_weight(N, K, 62), synth.make_bias(N, 62)
    x = base.to(d).repeat((M + 999) // 1000, 1)[:M]
    xs = mx().mx_pc_quantize_act_slab(x)
    assert xs.q.numel() > 1 << 32
    ws = mx().mx_pc_quantize_weight_slab(w.to(d))
    y = mx().mx_pc_linear_slab(xs, ws, b.to(d))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([np.arange(3), np.arange(M - 80, M), rng.integers(0, M, 64),
                                     [(1 << 32) // K, (1 << 32) // K + 1]]))
    q, s = rows_of(xs, torch.from_numpy(rows))
    rq, rs = oracle.quantize_pc(base[rows % 1000].float().numpy())
    assert np.array_equal(q, rq) and same_f32(s, rs)
    yref, S = oracle_pc(base[rows % 1000], w, b, False)
    assert_linear_close(y[rows], yref, S, what="pc offsets past 4 GiB")
    del x, xs, y
    torch.cuda.empty_cache()
