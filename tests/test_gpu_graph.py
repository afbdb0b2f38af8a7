"""HIP-graph capture of the hot path: the activation quantizer into a slab
plus the GEMM through each kernel kind (slab GEMM, split-K, few-token kernel
with and without K ranges, the requantizing epilogue). Each graph is replayed
several times with eager work in between (the input rewritten in place), and
every replay must equal the eager result on the same input bit for bit: the
entry points launch kernels only (no allocation, no memset), so a captured
call is the same sequence of launches.
"""

import pytest
import torch

import synth
from helpers import dev, mx

pytestmark = pytest.mark.gpu


def _graph(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture (kernel attributes are set on first use)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize(
    "M,K,N,plan,gelu",
    [(512, 256, 1024, ("slab", 1), False), (300, 320, 272, ("splitk", 3), True), (128, 512, 512, ("small", 2), False),
     (77, 192, 256, ("small", 1), True), (300, 320, 528, ("slab_m128", 1), True)],
)
def test_graph_replays_match_eager(M, K, N, plan, gelu):
    print(f"graph M={M} K={K} N={N} plan={plan}", flush=True)
    d = dev()
    inputs = [synth.make_activation(M, K, seed=s).to(d) for s in (1, 2, 3)]
    w = mx().mx_quantize_weight_slab(synth.make_weight(N, K, seed=4).to(d))
    b = synth.make_bias(N, seed=4).to(d)
    x = inputs[0].clone()
    xs = mx().mx_quantize_act_slab(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    nb = mx().plan_ws_bytes(plan, M, N, K)
    ws = torch.empty((nb,), dtype=torch.uint8, device=d) if nb > 0 else None

    def step():
        mx().mx_quantize_act_slab(x, xs)
        mx().mx_linear_slab_planned(plan, xs, w, b, gelu=gelu, y=y, workspace=ws)

    g = _graph(step)
    for rep, xin in enumerate(inputs + inputs[:1]):
        x.copy_(xin)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        step()  # the same launches, eagerly
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), y.view(torch.int16)), f"replay {rep}"
    del g


def test_graph_requant_chain_matches_eager():
    # FFN-shaped chain at a small size: up-projection with GELU writing the
    # next linear's MX slab, then the down-projection.
    d = dev()
    M, K, H = 300, 256, 512
    x = synth.make_activation(M, K, seed=7).to(d)
    x2 = synth.make_activation(M, K, seed=8).to(d)
    w1 = mx().mx_quantize_weight_slab(synth.make_weight(H, K, seed=9).to(d))
    w2 = mx().mx_quantize_weight_slab(synth.make_weight(K, H, seed=10).to(d))
    b1, b2 = synth.make_bias(H, seed=9).to(d), synth.make_bias(K, seed=10).to(d)
    xs = mx().mx_quantize_act_slab(x)
    h = mx().mx_linear_slab_requant(xs, w1, b1, gelu=True)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=d)

    def step():
        mx().mx_quantize_act_slab(x, xs)
        mx().mx_linear_slab_requant(xs, w1, b1, gelu=True, out=h)
        mx().mx_linear_slab(h, w2, b2, y=y)

    g = _graph(step)
    for rep, xin in enumerate([x2, x.clone(), x2]):
        x.copy_(xin)
        g.replay()
        torch.cuda.synchronize()
        got_y, got_q = y.clone(), h.q.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got_q, h.q), f"replay {rep}: intermediate codes"
        assert torch.equal(got_y.view(torch.int16), y.view(torch.int16)), f"replay {rep}"
    del g
