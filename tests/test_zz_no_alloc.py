"""mx_linear_noalloc (the linear with the library's own scratch array as its
workspace) against mx_linear (the same call with a caller workspace),
through the C ABI: two calls in a row on the shared array, the second on a
smaller input (whose few-token plan needs zeroed tile counters where the
first call left partial sums), each bit-identical to mx_linear and within
the oracle's tolerance; a shape beyond the array is refused before anything
runs, and the next call still works.

For callers that cannot allocate (graph capture, serving loops).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx, quant_ref

pytestmark = pytest.mark.gpu


def one(M, K, N, seed, gelu):
    d = dev()
    x = synth.make_activation(M, K, seed)
    w = synth.make_weight(N, K, seed + 1)
    b = synth.make_bias(N, seed + 2)
    xd, bd = x.to(d), b.to(d)
    wsl = mx().mx_quantize_weight_slab(w.to(d))
    y_na = mx().mx_linear_noalloc(xd, wsl, bd, gelu=gelu)
    y_ws = mx().mx_linear(xd, wsl, bd, gelu=gelu)
    torch.cuda.synchronize()
    return x, w, b, y_na, y_ws


def test_noalloc_two_calls_second_smaller_match_mx_linear():
    mx().mx_linear_plan_clear()
    cases = [(512, 5120, 2560, 91, False), (128, 5120, 5120, 92, True)]
    assert mx().plan_linear(*cases[0][:3]) == ("splitk", 8)
    assert mx().plan_linear(*cases[1][:3]) == ("small", 3)
    for M, K, N, seed, gelu in cases:
        print(f"noalloc M={M} K={K} N={N} gelu={gelu}", flush=True)
        x, w, b, y_na, y_ws = one(M, K, N, seed, gelu)
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), f"{M}x{K}x{N}: differs from mx_linear"
        rows = np.unique(np.concatenate([np.arange(4), np.arange(M - 4, M), np.arange(0, M, 37)]))
        yref, S = oracle.linear_ref(*quant_ref(x[torch.from_numpy(rows)]), *quant_ref(w), bias=f64(b),
                                    epilogue="gelu_tanh" if gelu else "none")
        assert_linear_close(y_na[torch.from_numpy(rows).to(y_na.device)], yref, S, "gelu_tanh" if gelu else "none",
                            what=f"noalloc {M}x{K}x{N}")


def test_noalloc_refuses_shapes_beyond_the_array():
    d = dev()
    M, K, N = 20000, 5120, 256  # activation slab alone: 105 MB > 64 MiB
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=d)
    wsl = mx().mx_quantize_weight_slab(torch.zeros((N, K), dtype=torch.float32, device=d))
    with pytest.raises(mx().MXError) as e:
        mx().mx_linear_noalloc(x, wsl)
    assert e.value.status == mx().MX_ERR_UNSUPPORTED
    del x
    _, _, _, y_na, y_ws = one(77, 640, 272, 93, False)
    assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
