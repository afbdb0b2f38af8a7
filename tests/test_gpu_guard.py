"""Output bounds of every kernel kind: each output is the leading part of a
larger device buffer pre-filled with a sentinel, at ragged sizes (rows and
columns off the tile grid). Every in-range bf16 element must be written (no
sentinel left), nothing past the output's end may change, and the values
must match the oracle (bf16 outputs) or the unguarded call (codes and
scales) bit for bit.

Source of the rule: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
OptRTN)", section "Quantization Details"; the ragged-row handling follows
"Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4", section
"Runtime setup" (masked tail loads, zero-filled ragged activation rows).
"""

import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx, quant_ref

pytestmark = pytest.mark.gpu

SENT16 = -1  # bf16 0xFFFF: a NaN with every mantissa bit set, which no kernel writes
SENT8 = 0xA5
TAIL = 4096  # elements past the output that must stay untouched


def guarded(shape, dtype):
    """(output view, whole buffer, sentinel) for an output of `shape`."""
    n = 1
    for s in shape:
        n *= s
    d = dev()
    if dtype == torch.bfloat16:
        big = torch.full((n + TAIL,), SENT16, dtype=torch.int16, device=d)
        return big[:n].view(torch.bfloat16).view(shape), big, SENT16
    fill = SENT8 if dtype == torch.uint8 else float("nan")
    big = torch.full((n + TAIL,), fill, dtype=dtype, device=d)
    return big[:n].view(shape), big, fill


def tail_untouched(big, n, fill):
    t = big[n:]
    if t.dtype.is_floating_point:
        return bool(torch.isnan(t).all())
    return bool((t == fill).all())


def check_bf16(y, big, yref, S, gelu, what):
    torch.cuda.synchronize()
    n = y.numel()
    assert tail_untouched(big, n, SENT16), f"{what}: wrote past the end of y"
    assert not bool((big[:n] == SENT16).any()), f"{what}: elements of y left unwritten"
    assert_linear_close(y, yref, S, "gelu_tanh" if gelu else "none", what=what)


M, K, N = 333, 320, 272  # ragged rows and columns; K spans five 64-K slabs


@pytest.fixture(scope="module")
def operands():
    x = synth.make_activation(M, K, 31)
    w = synth.make_weight(N, K, 32)
    b = synth.make_bias(N, 33)
    xq, xsc = quant_ref(x)
    wq, wsc = quant_ref(w)
    ref = {g: oracle.linear_ref(xq, xsc, wq, wsc, bias=f64(b), epilogue="gelu_tanh" if g else "none")
           for g in (False, True)}
    return x, w, b, ref


@pytest.mark.parametrize("plan", [("slab", 1), ("splitk", 3), ("small", 1), ("small", 4), ("balanced", 1), ("slab_m128", 1)])
@pytest.mark.parametrize("gelu", [False, True])
def test_slab_kernels_write_exactly_y(operands, plan, gelu):
    print(f"guard {plan} gelu={gelu}", flush=True)
    x, w, b, ref = operands
    d = dev()
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    y, big, _ = guarded((M, N), torch.bfloat16)
    mx().mx_linear_slab_planned(plan, xs, ws, b.to(d), gelu=gelu, y=y)
    check_bf16(y, big, *ref[gelu], gelu, f"{plan[0]}{plan[1]}")


@pytest.mark.parametrize("path", ["one_call", "fused", "row_major"])
def test_row_major_and_one_call_paths_write_exactly_y(operands, path):
    print(f"guard {path}", flush=True)
    x, w, b, ref = operands
    d = dev()
    y, big, _ = guarded((M, N), torch.bfloat16)
    if path == "one_call":
        mx().mx_linear(x.to(d), mx().mx_quantize_weight_slab(w.to(d)), b.to(d), gelu=True, y=y)
    else:
        wq, wsc = mx().mx_quantize_weight(w.to(d))
        if path == "fused":
            mx().mx_linear_fused(x.to(d), wq, wsc, b.to(d), gelu=True, y=y)
        else:
            xq, xsc = mx().mx_quantize_act(x.to(d))
            mx().mx_linear_q(xq, xsc, wq, wsc, b.to(d), gelu=True, y=y)
    check_bf16(y, big, *ref[True], True, path)


def test_per_channel_path_writes_exactly_y():
    print("guard per-channel", flush=True)
    d = dev()
    x = synth.make_activation(M, K, 34).to(d)
    w = synth.make_weight(N, K, 35).to(d)
    b = synth.make_bias(N, 36).to(d)
    xs = mx().mx_pc_quantize_act_slab(x)
    ws = mx().mx_pc_quantize_weight_slab(w)
    y, big, _ = guarded((M, N), torch.bfloat16)
    mx().mx_pc_linear_slab(xs, ws, b, gelu=True, y=y)
    y2 = mx().mx_pc_linear_slab(xs, ws, b, gelu=True)
    torch.cuda.synchronize()
    n = y.numel()
    assert tail_untouched(big, n, SENT16), "per-channel: wrote past the end of y"
    assert not bool((big[:n] == SENT16).any()), "per-channel: elements of y left unwritten"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_quantizers_write_exactly_their_outputs():
    print("guard quantizers", flush=True)
    d = dev()
    x = synth.make_activation(M, K, 37).to(d)
    w = synth.make_weight(N, K, 38).to(d)
    R = mx().mx_slab_rows(M)
    cases = []
    q, bq, fq = guarded((M, K), torch.uint8)
    s, bs, fs = guarded((M, K // 32), torch.uint8)
    mx().mx_quantize_act(x, q, s)
    cases.append(("act codes", q, bq, fq, mx().mx_quantize_act(x)[0]))
    cases.append(("act scales", s, bs, fs, mx().mx_quantize_act(x)[1]))
    q, bq, fq = guarded((N, K), torch.uint8)
    s, bs, fs = guarded((N, K // 32), torch.uint8)
    mx().mx_quantize_weight(w, q, s)
    cases.append(("weight codes", q, bq, fq, mx().mx_quantize_weight(w)[0]))
    cases.append(("weight scales", s, bs, fs, mx().mx_quantize_weight(w)[1]))
    sq, bq, fq = guarded((K // 64, R, 64), torch.uint8)
    ss, bs, fs = guarded((K // 64, R, 2), torch.uint8)
    ref = mx().mx_quantize_act_slab(x)
    mx().mx_quantize_act_slab(x, out=mx().Slab(sq, ss, M))
    cases.append(("act slab codes", sq, bq, fq, ref.q))
    cases.append(("act slab scales", ss, bs, fs, ref.s))
    pq, bq, fq = guarded((K // 64, R, 64), torch.uint8)
    ps, bs, fs = guarded((R,), torch.float32)
    pref = mx().mx_pc_quantize_act_slab(x)
    mx().mx_pc_quantize_act_slab(x, out=mx().PCSlab(pq, ps, M))
    cases.append(("per-channel slab codes", pq, bq, fq, pref.q))
    torch.cuda.synchronize()
    for what, out, big, fill, want in cases:
        assert tail_untouched(big, out.numel(), fill), f"{what}: wrote past the end"
        assert torch.equal(out, want), f"{what}: differs from the unguarded call"
    assert torch.equal(ps.view(torch.int32), pref.s.view(torch.int32)), "per-channel slab scales differ"
    assert tail_untouched(bs, ps.numel(), fs), "per-channel slab scales: wrote past the end"


def test_requant_epilogue_writes_exactly_its_slab():
    print("guard requant", flush=True)
    d = dev()
    N2 = 320  # the requantized output needs N % 64 == 0
    x = synth.make_activation(M, K, 39).to(d)
    w = synth.make_weight(N2, K, 40).to(d)
    b = synth.make_bias(N2, 41).to(d)
    xs = mx().mx_quantize_act_slab(x)
    ws = mx().mx_quantize_weight_slab(w)
    R = mx().mx_slab_rows(M)
    sq, bq, fq = guarded((N2 // 64, R, 64), torch.uint8)
    ss, bs, fs = guarded((N2 // 64, R, 2), torch.uint8)
    mx().mx_linear_slab_requant(xs, ws, b, gelu=True, out=mx().Slab(sq, ss, M))
    ref = mx().mx_quantize_act_slab(mx().mx_linear_slab(xs, ws, b, gelu=True))
    torch.cuda.synchronize()
    assert tail_untouched(bq, sq.numel(), fq), "requant codes: wrote past the end"
    assert tail_untouched(bs, ss.numel(), fs), "requant scales: wrote past the end"
    assert torch.equal(sq, ref.q) and torch.equal(ss, ref.s)
