"""FFN chain on an intermediate that the oracle fixes completely.

ffn.net.0.proj feeds ffn.net.2 through its bf16 output requantized to MXFP8
(model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)", section
"Quantization Details": both are MXFP8 linears, so the second one's
activation is quantized at run time). On Gaussian weights the GPU's fp32
sums may round to the other side of a bf16 or E4M3 boundary than the exact
value, so the seeded-chain tests can pin only part of the intermediate's
codes. Here the first linear's weights select one input column per output,
scaled by +-2^p (p in [-3, 3]), with no bias and the identity epilogue:
each output is +-2^p times one quantized input, a value with at most four
significant bits, exact in fp32 and in bf16. The intermediate is then fixed
exactly, so:

* the requantizing epilogue and the two-pass path (bf16 output, then the
  activation quantizer) must both equal the oracle's codes and scales of the
  exact intermediate byte for byte, pad rows zero;
* ``requant_range`` must report every code as fixed (a pin of the chain
  check itself);
* ffn.net.2 on the requantized intermediate must match the oracle within the
  plain tolerance, with no allowance for intermediate rounding.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx, quant_ref, requant_range

pytestmark = pytest.mark.gpu


def selection_weight(N, K, seed):
    """fp32 [N, K]: row n is +-2^p_n at column c_n and zero elsewhere.
    Returns (w, c, scale) with scale = +-2^p_n."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, K, N)
    scale = rng.choice([-1.0, 1.0], N) * np.ldexp(1.0, rng.integers(-3, 4, N))
    w = torch.zeros((N, K), dtype=torch.float32)
    w[torch.arange(N), torch.from_numpy(c)] = torch.from_numpy(scale).float()
    return w, c, scale


def exact_intermediate(x_rows, c, scale):
    """The first linear's exact outputs for the given bf16 token rows:
    scale[n] * xhat[m, c[n]] (float64, exact). A zero sum is +0 (adding
    +0.0 clears the sign a single signed-zero product would carry; a sum
    of products that starts from +0 has no sign to keep)."""
    xq, xs = quant_ref(x_rows)
    xhat = oracle.dequantize_mx(xq, xs)
    return xhat[:, c] * scale[None, :] + 0.0


def slab_rows(sl, rows, K):
    q = sl.q[:, rows].cpu().numpy().transpose(1, 0, 2).reshape(len(rows), K)
    s = sl.s[:, rows].cpu().numpy().transpose(1, 0, 2).reshape(len(rows), K // 32)
    return q, s


@pytest.mark.parametrize("M,K,N,N2", [(300, 256, 512, 320), (77, 640, 1024, 128), (513, 128, 192, 64)])
def test_exact_chain_codes_byte_equal(M, K, N, N2):
    print(f"exact chain M={M} K={K} N={N} N2={N2}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed=M + N)
    w1, c, scale = selection_weight(N, K, seed=N + 1)
    w2 = synth.make_weight(N2, N, seed=N2 + 2)
    b2 = synth.make_bias(N2, seed=N2 + 3)
    xs = mx().mx_quantize_act_slab(x.to(d))
    w1s = mx().mx_quantize_weight_slab(w1.to(d))
    w2s = mx().mx_quantize_weight_slab(w2.to(d))
    h_fused = mx().mx_linear_slab_requant(xs, w1s, None)
    h_bf16 = mx().mx_linear_slab(xs, w1s, None)
    h_two = mx().mx_quantize_act_slab(h_bf16)
    y2 = mx().mx_linear_slab(h_fused, w2s, b2.to(d))
    torch.cuda.synchronize()

    h_star = exact_intermediate(x, c, scale)
    assert np.array_equal(f64(h_bf16), h_star), "first linear is not exact"
    # The weight quantizer keeps +-2^p exactly (code 0x78 or 0xF8 at scale
    # 2^(p-8), zero groups elsewhere).
    w1q, w1sc = quant_ref(w1)
    assert np.array_equal(oracle.dequantize_mx(w1q, w1sc), f64(w1))
    _, S1 = oracle.linear_ref(*quant_ref(x), w1q, w1sc)
    rng = requant_range(h_star, S1)
    assert rng["fixed"].all() and np.array_equal(rng["slo"], rng["shi"])
    hq, hs = oracle.quantize_mx(h_star)
    rows = np.arange(M)
    for name, h in (("requant epilogue", h_fused), ("two-pass", h_two)):
        q, s = slab_rows(h, torch.from_numpy(rows), N)
        assert np.array_equal(s, hs), f"{name}: scales differ from the oracle"
        assert np.array_equal(q, hq), f"{name}: {int((q != hq).sum())} codes differ from the oracle"
        assert not h.q[:, M:].any() and not h.s[:, M:].any(), f"{name}: pad rows not zero"
    w2q, w2sc = quant_ref(w2)
    y2ref, S2 = oracle.linear_ref(hq, hs, w2q, w2sc, bias=f64(b2))
    assert_linear_close(y2, y2ref, S2, what="ffn.net.2 on the exact intermediate")


def test_exact_chain_full_ffn_size_sampled_rows():
    """The same at the FFN's full size (75348 tokens, 5120 -> 13824 ->
    5120), in the launch configuration of the FFN workload: sampled token
    rows (the first 8, the ragged last 90 and 256 random) of the requantized
    intermediate byte-equal to the oracle, ffn.net.2 within tolerance."""
    M, K, N, N2 = synth.VIDEO_TOKENS, synth.HIDDEN, synth.FFN, synth.HIDDEN
    print(f"exact chain full size M={M} K={K} N={N} N2={N2}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed=5)
    w1, c, scale = selection_weight(N, K, seed=6)
    w2 = synth.make_weight(N2, N, seed=7)
    b2 = synth.make_bias(N2, seed=7)
    xs = mx().mx_quantize_act_slab(x.to(d))
    w1s = mx().mx_quantize_weight_slab(w1.to(d))
    w2s = mx().mx_quantize_weight_slab(w2.to(d))
    del w1
    h = mx().mx_linear_slab_requant(xs, w1s, None)
    y2 = mx().mx_linear_slab(h, w2s, b2.to(d))
    torch.cuda.synchronize()
    r = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 90, M), r.integers(0, M, 256)]))
    h_star = exact_intermediate(x[torch.from_numpy(rows)], c, scale)
    hq, hs = oracle.quantize_mx(h_star)
    q, s = slab_rows(h, torch.from_numpy(rows), N)
    assert np.array_equal(s, hs), "scales differ from the oracle"
    assert np.array_equal(q, hq), f"{int((q != hq).sum())} codes differ from the oracle"
    assert not h.q[:, M:].any() and not h.s[:, M:].any()
    w2q, w2sc = quant_ref(w2)
    y2ref, S2 = oracle.linear_ref(hq, hs, w2q, w2sc, bias=f64(b2))
    assert_linear_close(y2[torch.from_numpy(rows).to(d)], y2ref, S2, what="ffn.net.2 sampled rows")
