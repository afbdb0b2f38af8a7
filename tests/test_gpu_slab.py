"""GPU parity of the slab-layout path (mx_quantize_act_slab,
mx_quantize_weight_slab, mx_slab_pack, mx_linear_slab,
mx_linear_slab_requant) against the oracle.

The slab layout only moves bytes: codes [K/64][R][64] and scales
[K/64][R][2] with R the row count rounded up to 256 and zero pad rows. The
oracle's row-major codes and scales are placed in that layout here, on the
host, and compared byte for byte; the GEMM is held to the same tolerance as
the row-major one (1e-3 g sum|a||b| + one bf16 ulp) and must equal
mx_linear_q bit for bit, since it performs the same MFMAs in the same order.

Source of the rule: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
OptRTN)", section "Quantization Details".
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (
    assert_chain_close,
    assert_linear_close,
    assert_requant_valid,
    dev,
    f64,
    mx,
    quant_ref,
    requant_range,
    u8,
)

pytestmark = pytest.mark.gpu


def to_slab(q, s):
    """Row-major numpy codes [rows, K] and scales [rows, K/32] in the slab layout."""
    rows, K = q.shape
    R = (rows + 255) // 256 * 256
    qs = np.zeros((K // 64, R, 64), dtype=np.uint8)
    ss = np.zeros((K // 64, R, 2), dtype=np.uint8)
    qs[:, :rows] = q.reshape(rows, K // 64, 64).transpose(1, 0, 2)
    ss[:, :rows] = s.reshape(rows, K // 64, 2).transpose(1, 0, 2)
    return qs, ss


def slab_rows_of(sl, rows):
    """Row-major codes and scales of the given rows of a Slab (numpy)."""
    q = u8(sl.q[:, rows])  # [K/64, n, 64]
    s = u8(sl.s[:, rows])
    n = len(rows)
    return q.transpose(1, 0, 2).reshape(n, -1), s.transpose(1, 0, 2).reshape(n, -1)


# The bf16 slab quantizer works on 8-row x 512-K tiles: shapes on and around
# those edges (partial last K tile, rows just under and over a tile, a pad
# region inside the last tile) are compared whole, pad rows included.
@pytest.mark.parametrize("M,K", [(1, 64), (77, 192), (256, 128), (300, 5120), (513, 640), (7, 512), (8, 448),
                                 (9, 576), (255, 1024), (257, 1088)])
def test_act_slab_quantizer_matches_oracle(M, K):
    x = synth.make_activation(M, K, seed=M + 3 * K)
    sl = mx().mx_quantize_act_slab(x.to(dev()))
    rq, rs = to_slab(*quant_ref(x))
    assert np.array_equal(u8(sl.s), rs)
    assert np.array_equal(u8(sl.q), rq)


def test_act_slab_quantizer_strided_rows_and_nonfinite():
    base = synth.make_activation(70, 384, seed=9)
    base[3, 70] = float("nan")
    base[5, 200] = float("-inf")
    x = base.to(dev())[:, 64:320]  # pitch 384, K 256
    sl = mx().mx_quantize_act_slab(x)
    rq, rs = to_slab(*quant_ref(base[:, 64:320]))
    assert np.array_equal(u8(sl.s), rs) and np.array_equal(u8(sl.q), rq)


def test_act_slab_quantizer_full_size_sampled_rows():
    M, K = synth.VIDEO_TOKENS, synth.HIDDEN
    x = synth.make_activation(M, K, seed=0)
    print(f"full-size slab act quantize {M}x{K}", flush=True)
    sl = mx().mx_quantize_act_slab(x.to(dev()))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 90, M), rng.integers(0, M, 512)]))
    q, s = slab_rows_of(sl, torch.from_numpy(rows))
    rq, rs = oracle.quantize_mx(f64(x[rows]))
    assert np.array_equal(s, rs) and np.array_equal(q, rq)
    R = sl.q.shape[1]
    assert R == 75520
    assert not sl.q[:, M:].any() and not sl.s[:, M:].any()  # pad rows are zero


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_weight_slab_quantizer_matches_oracle(dtype):
    w = synth.make_weight(272, 1024, seed=4).to(dtype)
    w[7, 9] = float("inf")
    sl = mx().mx_quantize_weight_slab(w.to(dev()))
    rq, rs = to_slab(*quant_ref(w))
    assert np.array_equal(u8(sl.s), rs) and np.array_equal(u8(sl.q), rq)


def test_slab_pack_matches_slab_quantizer():
    w = synth.make_weight(600, 640, seed=6).to(dev())
    q, s = mx().mx_quantize_weight(w)
    a = mx().mx_slab_pack(q, s)
    b = mx().mx_quantize_weight_slab(w)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.s, b.s)


def run_slab(M, K, N, seed, bias=True, gelu=False, x=None):
    d = dev()
    x = synth.make_activation(M, K, seed) if x is None else x
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed) if bias else None
    ws = mx().mx_quantize_weight_slab(w.to(d))
    xs = mx().mx_quantize_act_slab(x.to(d))
    y = mx().mx_linear_slab(xs, ws, None if b is None else b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    return x, w, b, y


def oracle_linear(x, w, b, gelu):
    xq, xs = quant_ref(x)
    wq, ws = quant_ref(w)
    return oracle.linear_ref(xq, xs, wq, ws, bias=None if b is None else f64(b),
                             epilogue="gelu_tanh" if gelu else "none")


@pytest.mark.parametrize(
    "M,K,N",
    [(1, 64, 16), (5, 64, 32), (77, 192, 256), (256, 128, 256), (300, 320, 512), (513, 512, 272), (70, 5120, 768)],
)
def test_linear_slab_small_shapes(M, K, N):
    print(f"linear_slab M={M} K={K} N={N}", flush=True)
    x, w, b, y = run_slab(M, K, N, seed=M * 5 + K + N)
    yref, S = oracle_linear(x, w, b, False)
    assert_linear_close(y, yref, S, what=f"M{M} K{K} N{N}")


def test_linear_slab_gelu_no_bias():
    x, w, b, y = run_slab(300, 448, 512, seed=12, bias=False, gelu=True)
    yref, S = oracle_linear(x, w, None, True)
    assert_linear_close(y, yref, S, "gelu_tanh", what="gelu")


@pytest.mark.parametrize("gelu", [False, True])
def test_linear_slab_equals_row_major_bitwise(gelu):
    d = dev()
    x = synth.make_activation(600, 1024, seed=31).to(d)
    w = synth.make_weight(512, 1024, seed=31).to(d)
    b = synth.make_bias(512, seed=31).to(d)
    wq, ws = mx().mx_quantize_weight(w)
    xq, xs = mx().mx_quantize_act(x)
    y1 = mx().mx_linear_q(xq, xs, wq, ws, b, gelu=gelu)
    y2 = mx().mx_linear_slab(mx().mx_slab_pack(xq, xs), mx().mx_slab_pack(wq, ws), b, gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_linear_slab_zero_rows_give_bias():
    ctx = synth.make_text_context(512, 5120, seed=2)
    x, w, b, y = run_slab(512, 5120, 1024, seed=2, x=ctx)
    want = f64(b.float().to(torch.bfloat16))
    assert np.array_equal(f64(y)[410:], np.broadcast_to(want, (102, 1024)))
    yref, S = oracle_linear(x, w, b, False)
    assert_linear_close(y, yref, S, what="text ctx")


def test_linear_slab_deterministic_and_fully_written():
    d = dev()
    xs = mx().mx_quantize_act_slab(synth.make_activation(333, 512, seed=21).to(d))
    ws = mx().mx_quantize_weight_slab(synth.make_weight(768, 512, seed=21).to(d))
    y1 = torch.full((333, 768), float("nan"), dtype=torch.bfloat16, device=d)
    y2 = torch.full((333, 768), float("nan"), dtype=torch.bfloat16, device=d)
    mx().mx_linear_slab(xs, ws, y=y1)
    mx().mx_linear_slab(xs, ws, y=y2)
    torch.cuda.synchronize()
    assert not torch.isnan(y1).any()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def sampled_rows(M, n=96, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(4), np.arange(M - 84, M), rng.integers(0, M, n)]))


def test_linear_slab_qkv_full_size():
    d = dev()
    shp = synth.CONFIGS["qkv_75348x5120x15360"][0]
    x = synth.make_activation(shp.M, shp.K, 100)
    w = synth.make_weight(shp.N, shp.K, 100)
    b = synth.make_bias(shp.N, 100)
    print(f"slab qkv {shp}", flush=True)
    xd, wd, bd = x.to(d), w.to(d), b.to(d)
    ws = mx().mx_quantize_weight_slab(wd)
    y = mx().mx_linear_slab(mx().mx_quantize_act_slab(xd), ws, bd)
    wq, wsr = mx().mx_quantize_weight(wd)
    xq, xsr = mx().mx_quantize_act(xd)
    y_rm = mx().mx_linear_q(xq, xsr, wq, wsr, bd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16))
    del y_rm, xq, xsr
    rows = sampled_rows(shp.M)
    yref, S = oracle.linear_ref(*quant_ref(x[rows]), *quant_ref(w), bias=f64(b))
    assert_linear_close(y[rows], yref, S, what="qkv slab")


def test_ffn_chain_full_size_slab():
    # ffn.net.0.proj (GELU) then ffn.net.2 over all 75348 tokens: the bf16
    # intermediate h [75348, 13824] is quantized again into a slab of 216
    # K-slabs (offsets past 2^30 bytes). h is held to the oracle's first
    # linear, its slab to what the oracle's chain fixes of it, and the
    # down-projection to the oracle's whole chain (assert_chain_close).
    d = dev()
    up, down = synth.CONFIGS["ffn_75348x5120x13824"]
    print(f"slab ffn {up} -> {down}", flush=True)
    x = synth.make_activation(up.M, up.K, 7)
    w1, b1 = synth.make_weight(up.N, up.K, 7), synth.make_bias(up.N, 7)
    w2, b2 = synth.make_weight(down.N, down.K, 8), synth.make_bias(down.N, 8)
    w1s = mx().mx_quantize_weight_slab(w1.to(d))
    w2s = mx().mx_quantize_weight_slab(w2.to(d))
    h = mx().mx_linear_slab(mx().mx_quantize_act_slab(x.to(d)), w1s, b1.to(d), gelu=True)
    hs = mx().mx_quantize_act_slab(h)
    y = mx().mx_linear_slab(hs, w2s, b2.to(d))
    torch.cuda.synchronize()
    rows = sampled_rows(up.M, 48, seed=3)
    href, S1 = oracle_linear(x[rows], w1, b1, True)
    assert_linear_close(h[rows], href, S1, "gelu_tanh", what="ffn up")
    assert_requant_valid(*slab_rows_of(hs, torch.from_numpy(rows)), requant_range(href, S1, "gelu_tanh"),
                         what="ffn intermediate slab")
    assert_chain_close(y[rows], href, S1, "gelu_tanh", *quant_ref(w2), f64(b2), what="ffn down")


@pytest.mark.parametrize("M,K,N,gelu", [(300, 256, 320, True), (513, 512, 256, False), (70, 5120, 768, True), (1, 64, 64, True)])
def test_requant_epilogue_equals_two_pass(M, K, N, gelu):
    # The fused output must be byte-identical to quantizing the bf16 output
    # of the same GEMM (same accumulation, same bf16 rounding, same rule),
    # pad rows included.
    d = dev()
    xs = mx().mx_quantize_act_slab(synth.make_activation(M, K, seed=M + N).to(d))
    ws = mx().mx_quantize_weight_slab(synth.make_weight(N, K, seed=M + N).to(d))
    b = synth.make_bias(N, seed=M + N).to(d)
    y = mx().mx_linear_slab(xs, ws, b, gelu=gelu)
    ref = mx().mx_quantize_act_slab(y)
    out = mx().mx_linear_slab_requant(xs, ws, b, gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(out.q, ref.q) and torch.equal(out.s, ref.s)
    assert not out.q[:, M:].any() and not out.s[:, M:].any()
    # and against what the oracle's linear fixes of the requantized output
    yref, S = oracle_linear(synth.make_activation(M, K, seed=M + N), synth.make_weight(N, K, seed=M + N),
                            synth.make_bias(N, seed=M + N), gelu)
    assert_requant_valid(*slab_rows_of(out, torch.arange(M)), requant_range(yref, S, "gelu_tanh" if gelu else "none"),
                         what="requantized output")


def test_ffn_chain_full_size_fused_requant():
    # ffn.net.0.proj with GELU writing the requantized intermediate directly,
    # then ffn.net.2: bit-identical to the two-pass chain, and sampled rows
    # against the oracle's chain from the seeded inputs.
    d = dev()
    up, down = synth.CONFIGS["ffn_75348x5120x13824"]
    print(f"slab ffn fused requant {up} -> {down}", flush=True)
    x = synth.make_activation(up.M, up.K, 17)
    w1, b1 = synth.make_weight(up.N, up.K, 17), synth.make_bias(up.N, 17)
    w2, b2 = synth.make_weight(down.N, down.K, 18), synth.make_bias(down.N, 18)
    w1s = mx().mx_quantize_weight_slab(w1.to(d))
    w2s = mx().mx_quantize_weight_slab(w2.to(d))
    xs = mx().mx_quantize_act_slab(x.to(d))
    hs = mx().mx_linear_slab_requant(xs, w1s, b1.to(d), gelu=True)
    y = mx().mx_linear_slab(hs, w2s, b2.to(d))
    h = mx().mx_linear_slab(xs, w1s, b1.to(d), gelu=True)
    hs2 = mx().mx_quantize_act_slab(h)
    torch.cuda.synchronize()
    assert torch.equal(hs.q, hs2.q) and torch.equal(hs.s, hs2.s)
    del hs2
    rows = sampled_rows(up.M, 48, seed=5)
    href, S1 = oracle_linear(x[rows], w1, b1, True)
    assert_linear_close(h[rows], href, S1, "gelu_tanh", what="ffn up")
    assert_requant_valid(*slab_rows_of(hs, torch.from_numpy(rows)), requant_range(href, S1, "gelu_tanh"),
                         what="ffn intermediate slab")
    assert_chain_close(y[rows], href, S1, "gelu_tanh", *quant_ref(w2), f64(b2), what="ffn down after fused requant")


@pytest.mark.parametrize("M,K,N,gelu", [(300, 512, 256, True), (77, 5120, 768, False)])
def test_linear_ws_one_call(M, K, N, gelu):
    # One call (quantize into the workspace, slab GEMM) equals the two calls
    # bit for bit, with strided activation rows, and the oracle within tolerance.
    d = dev()
    base = synth.make_activation(M, K + 64, seed=M + K)
    x = base[:, 32:32 + K]
    w = synth.make_weight(N, K, seed=M + K)
    b = synth.make_bias(N, seed=M + K)
    wsl = mx().mx_quantize_weight_slab(w.to(d))
    xd = base.to(d)[:, 32:32 + K]
    y1 = mx().mx_linear(xd, wsl, b.to(d), gelu=gelu)
    y2 = mx().mx_linear_slab(mx().mx_quantize_act_slab(xd), wsl, b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y1, yref, S, "gelu_tanh" if gelu else "none", what="linear_ws")


@pytest.mark.parametrize("M,K,N", [(128, 512, 512), (300, 320, 272), (1, 64, 16), (513, 256, 1024)])
def test_splitk_single_range_equals_slab(M, K, N):
    # One range: the same accumulation, reduction of one term, same epilogue.
    d = dev()
    xs = mx().mx_quantize_act_slab(synth.make_activation(M, K, seed=M + K).to(d))
    ws = mx().mx_quantize_weight_slab(synth.make_weight(N, K, seed=M + K).to(d))
    b = synth.make_bias(N, seed=M + K).to(d)
    for gelu in (False, True):
        y1 = mx().mx_linear_slab(xs, ws, b, gelu=gelu)
        y2 = mx().mx_linear_slab_splitk(xs, ws, b, gelu=gelu, splits=1)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize(
    "M,K,N,splits,gelu,bias",
    [(128, 512, 512, 8, False, True), (300, 320, 272, 5, True, True), (1, 64, 16, 1, False, False),
     (513, 256, 1024, 3, True, False), (77, 5120, 768, 80, False, True), (256, 1024, 256, 7, True, True)],
)
def test_splitk_matches_oracle(M, K, N, splits, gelu, bias):
    print(f"splitk M={M} K={K} N={N} splits={splits}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed=M * 3 + N)
    w = synth.make_weight(N, K, seed=M * 3 + N)
    b = synth.make_bias(N, seed=M * 3 + N) if bias else None
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    bd = None if b is None else b.to(d)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=d)
    mx().mx_linear_slab_splitk(xs, ws, bd, gelu=gelu, y=y, splits=splits)
    y2 = mx().mx_linear_slab_splitk(xs, ws, bd, gelu=gelu, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed reduction order
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y, yref, S, "gelu_tanh" if gelu else "none", what=f"splitk {splits}")


@pytest.mark.parametrize("cfg", ["single_128x5120x5120", "xattn_512x5120x10240"])
def test_splitk_small_token_configs(cfg):
    # The linears with few token tiles at their full sizes, with the chosen
    # split count; every output element against the oracle.
    d = dev()
    shp = synth.CONFIGS[cfg][0]
    assert shp.M <= 512
    x = synth.make_text_context(shp.M, shp.K, 31) if shp.M == synth.TEXT_TOKENS else synth.make_activation(shp.M, shp.K, 31)
    w, b = synth.make_weight(shp.N, shp.K, 31), synth.make_bias(shp.N, 31)
    splits = mx().mx_linear_splitk_choose(shp.M, shp.K, shp.N)
    print(f"splitk {cfg} {shp} splits={splits}", flush=True)
    assert splits > 1
    y = mx().mx_linear_slab_splitk(mx().mx_quantize_act_slab(x.to(d)), mx().mx_quantize_weight_slab(w.to(d)),
                                   b.to(d), gelu=shp.gelu)
    torch.cuda.synchronize()
    yref, S = oracle_linear(x, w, b, shp.gelu)
    assert_linear_close(y, yref, S, "gelu_tanh" if shp.gelu else "none", what=cfg)


def tile_coords(pid, tiles_m, tiles_n, gm=4):
    """The kernels' workgroup -> (token tile, weight tile) order: XCD ranges,
    then groups of 4 token tiles x all weight tiles."""
    nwg = tiles_m * tiles_n
    q, r = nwg >> 3, nwg & 7
    xcd, k = pid & 7, pid >> 3
    lid = xcd * q + min(xcd, r) + k
    group = lid // (gm * tiles_n)
    first_m = group * gm
    g = min(tiles_m - first_m, gm)
    in_group = lid - group * gm * tiles_n
    return first_m + in_group % g, in_group // g


def split_tile_mask(M, N, ncu=256):
    tm_, tn_ = (M + 255) // 256, (N + 255) // 256
    tiles = tm_ * tn_
    mask = np.zeros((M, N), dtype=bool)
    for pid in range(tiles - tiles % ncu, tiles):
        a, b = tile_coords(pid, tm_, tn_)
        mask[a * 256:(a + 1) * 256, b * 256:(b + 1) * 256] = True
    return mask


def test_tile_order_is_a_bijection():
    for tm_, tn_ in ((1, 20), (295, 20), (295, 60), (17, 16), (3, 5)):
        seen = {tile_coords(p, tm_, tn_) for p in range(tm_ * tn_)}
        assert seen == {(a, b) for a in range(tm_) for b in range(tn_)}


@pytest.mark.parametrize("M,K,N,gelu", [(4352, 512, 4096, False), (300, 256, 512, True), (128, 5120, 5120, False)])
def test_balanced_matches_slab_and_oracle(M, K, N, gelu):
    # Tiles of the full rounds equal mx_linear_slab bit for bit; the split
    # last round (and everything) is within the tolerance of the oracle.
    print(f"balanced M={M} K={K} N={N}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed=M + N + 1)
    w = synth.make_weight(N, K, seed=M + N + 1)
    b = synth.make_bias(N, seed=M + N + 1)
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    y1 = mx().mx_linear_slab(xs, ws, b.to(d), gelu=gelu)
    y2 = mx().mx_linear_slab_balanced(xs, ws, b.to(d), gelu=gelu)
    y3 = mx().mx_linear_slab_balanced(xs, ws, b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y3.view(torch.int16))
    props = torch.cuda.get_device_properties(d)
    mask = torch.from_numpy(split_tile_mask(M, N, props.multi_processor_count))
    if mx().mx_linear_balanced_ws_bytes(M, K, N) == 0:
        mask[:] = False
    keep = ~mask.to(d)
    assert torch.equal(y1.view(torch.int16)[keep], y2.view(torch.int16)[keep])
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y2, yref, S, "gelu_tanh" if gelu else "none", what="balanced")


def test_balanced_full_size_n5120():
    # 75348 x 5120 x 5120: 5900 tiles, the last 12 split; sampled rows of the
    # split tiles against the oracle, the rest bit-identical to the plain GEMM.
    d = dev()
    M, K, N = synth.VIDEO_TOKENS, synth.HIDDEN, synth.HIDDEN
    x = synth.make_activation(M, K, 41)
    w, b = synth.make_weight(N, K, 41), synth.make_bias(N, 41)
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    y1 = mx().mx_linear_slab(xs, ws, b.to(d))
    y2 = mx().mx_linear_slab_balanced(xs, ws, b.to(d))
    torch.cuda.synchronize()
    props = torch.cuda.get_device_properties(d)
    mask = split_tile_mask(M, N, props.multi_processor_count)
    keep = torch.from_numpy(~mask).to(d)
    assert torch.equal(y1.view(torch.int16)[keep], y2.view(torch.int16)[keep])
    rows = np.unique(np.nonzero(mask.any(axis=1))[0][::97])
    yref, S = oracle.linear_ref(*quant_ref(x[rows]), *quant_ref(w), bias=f64(b))
    assert_linear_close(y2[rows], yref, S, what="balanced full size")


def test_linear_ws_offsets_past_4gib():
    # 2^20 + 77 token rows at K = 5120: the activation slab is 5.4 GB, so the
    # quantizer takes its 64-bit index path and the GEMM's slab offsets pass
    # 2^32 bytes. The rows are a seeded block of 1000 rows repeated, so the
    # oracle knows every row; sampled rows across the whole range, the last
    # (ragged) tile included, are checked.
    d = dev()
    M, K, N = (1 << 20) + 77, 5120, 256
    base = synth.make_activation(1000, K, seed=61)
    w, b = synth.make_weight(N, K, 61), synth.make_bias(N, 61)
    x = base.to(d).repeat((M + 999) // 1000, 1)[:M]
    wsl = mx().mx_quantize_weight_slab(w.to(d))
    ws = torch.empty((mx().mx_linear_ws_bytes(M, K, N),), dtype=torch.uint8, device=d)
    assert ws.numel() > 1 << 32
    y = mx().mx_linear(x, wsl, b.to(d), workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(3), np.arange(M - 80, M), rng.integers(0, M, 64),
                                     [(1 << 31) // K, (1 << 32) // K, (1 << 32) // K + 1]]))
    yref, S = oracle_linear(base[rows % 1000], w, b, False)
    assert_linear_close(y[rows], yref, S, what="offsets past 4 GiB")
    del x, ws, y
    torch.cuda.empty_cache()
