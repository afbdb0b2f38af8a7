"""GPU parity of one full denoise step's quantized linears: 40 transformer
blocks x 10 MXFP8 W8A8 linears (attn1 q/k/v/out, attn2 q/k/v/out, ffn up and
down) with independently seeded weights, 75348 video tokens and 512 text
tokens, each linear quantizing its input at run time, run back to back by
DenoiseStepLinears exactly as the bench times it.

Blocks 0 and 39 take weights drawn on the host; the oracle recomputes every
GEMM of those blocks on sampled token rows and output columns from the
seeded inputs (the feed-forward pair as a chain through the requantized
intermediate), right after the block ran. The other blocks' weights are drawn
on the GPU, so those blocks also show that the blocks do not share weights.

Source: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
section "Quantization Details" (the ten quantized linears per block, the
format); the token counts from its section "Running the Official Example".
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
)

pytestmark = pytest.mark.gpu

CHECKED_BLOCKS = (0, synth.DENOISE_BLOCKS - 1)


def sample(n_total, n, seed, tail):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(4), np.arange(n_total - tail, n_total), rng.integers(0, n_total, n)]))


def slab_rows_of(sl, rows):
    q = sl.q[:, rows].cpu().numpy()
    s = sl.s[:, rows].cpu().numpy()
    return q.transpose(1, 0, 2).reshape(len(rows), -1), s.transpose(1, 0, 2).reshape(len(rows), -1)


def check_block(block, step, inputs, weights, biases):
    from mxfp8_w8a8_quantized_amd.denoise import GEMMS

    M = synth.VIDEO_TOKENS
    rows = sample(M, 24, seed=block, tail=20)
    for gemm, role, names, gelu in GEMMS:
        w = torch.cat([weights[n] for n in names]) if len(names) > 1 else weights[names[0]]
        b = torch.cat([biases[n] for n in names]) if len(names) > 1 else biases[names[0]]
        N = w.shape[0]
        cols = sample(N, 160, seed=1000 + block, tail=48)
        epi = "gelu_tanh" if gelu else "none"
        what = f"block {block} {gemm}"
        print(f"check {what}", flush=True)
        if gemm == "ffn.net.0.proj":
            # the whole intermediate row is needed by ffn.net.2
            href, S1 = oracle.linear_ref(*quant_ref(inputs[role][rows]), *quant_ref(w), bias=f64(b), epilogue=epi)
            assert_requant_valid(*slab_rows_of(step.ffn_hidden, torch.from_numpy(rows)),
                                 requant_range(href, S1, epi), what=what)
            continue
        if gemm == "ffn.net.2":
            y = step.outputs[gemm][rows][:, cols]
            assert_chain_close(y, href, S1, "gelu_tanh", *quant_ref(w[cols]), f64(b[cols]), what=what)
            continue
        r = np.arange(synth.TEXT_TOKENS) if role == "text" else rows
        yref, S = oracle.linear_ref(*quant_ref(inputs[role][r]), *quant_ref(w[cols]), bias=f64(b[cols]), epilogue=epi)
        assert_linear_close(step.outputs[gemm][r][:, cols], yref, S, epi, what=what)


@pytest.mark.timeout(600)
def test_denoise_step_linears():
    from mxfp8_w8a8_quantized_amd.denoise import DenoiseStepLinears

    d = dev()
    mx()
    step = DenoiseStepLinears(synth.DENOISE_BLOCKS, synth.VIDEO_TOKENS, synth.TEXT_TOKENS, synth.HIDDEN, synth.FFN, d)
    host = {}
    for block in range(synth.DENOISE_BLOCKS):
        if block in CHECKED_BLOCKS:
            w, b = synth.make_denoise_block(block)
            host[block] = (w, b)
            step.set_block(block, {k: v.to(d) for k, v in w.items()}, {k: v.to(d) for k, v in b.items()})
        else:
            w, b = synth.make_denoise_block(block, d, on_device=True)
            step.set_block(block, w, b)
        del w, b
    print("weights quantized", flush=True)
    inputs = synth.make_denoise_inputs()
    inputs_d = {k: v.to(d) for k, v in inputs.items()}
    print("inputs drawn", flush=True)
    for block in range(synth.DENOISE_BLOCKS):
        step.run_block(block, inputs_d)
        if block in CHECKED_BLOCKS:
            torch.cuda.synchronize()
            check_block(block, step, inputs, *host[block])
    torch.cuda.synchronize()


def test_denoise_step_shapes_and_flop():
    from mxfp8_w8a8_quantized_amd.denoise import DenoiseStepLinears

    d = dev()
    step = DenoiseStepLinears(2, 300, 40, 256, 512, d)
    shapes = step.shapes()
    assert [s[0] for s in shapes] == ["attn1.qkv", "attn1.to_out.0", "attn2.to_q", "attn2.kv", "attn2.to_out.0",
                                      "ffn.net.0.proj", "ffn.net.2"]
    # the ten linears of the model, with q|k|v and k|v fused
    per_block = (3 * 300 * 256 * 256 + 300 * 256 * 256 * 3 + 2 * 40 * 256 * 256 + 2 * 300 * 256 * 512)
    assert step.flop() == 2 * 2.0 * per_block


@pytest.mark.parametrize("tuned", [False, True])
def test_denoise_step_small_against_oracle(tuned):
    # The same runner on a small model (2 blocks, 300 + 40 tokens, hidden
    # 256, ffn 512): every output element of both blocks against the oracle,
    # with the default plans and after warm-up tuning of block 0's shapes
    # (the plans tune() reports are the ones mx_linear then looks up).
    from mxfp8_w8a8_quantized_amd.denoise import GEMMS, DenoiseStepLinears

    mx().mx_linear_plan_clear()
    d = dev()
    M, T, H, F = 300, 40, 256, 512
    step = DenoiseStepLinears(2, M, T, H, F, d)
    blocks = []
    for block in range(2):
        w, b = {}, {}
        for slot, (shp, _) in enumerate(synth.DENOISE_LINEARS):
            N = {"ffn.net.0.proj": F}.get(shp.name, H)
            K = F if shp.name == "ffn.net.2" else H
            seed = synth.block_layer_seed(block, slot)
            w[shp.name], b[shp.name] = synth.make_weight(N, K, seed), synth.make_bias(N, seed)
        blocks.append((w, b))
        step.set_block(block, {k: v.to(d) for k, v in w.items()}, {k: v.to(d) for k, v in b.items()})
    inputs = {}
    for role, seed in synth.DENOISE_ROLE_SEEDS.items():
        inputs[role] = synth.make_text_context(T, H, seed) if role == "text" else synth.make_activation(M, H, seed)
    inputs_d = {k: v.to(d) for k, v in inputs.items()}
    if tuned:
        plans = step.tune(inputs_d)
        assert set(plans) == {g for g, _, _, _ in GEMMS} - {"ffn.net.0.proj"}
        assert plans == step.plans() and plans["attn2.kv"] == step.tuned["attn2.kv"]
        assert plans["ffn.net.2"] == step.tuned["ffn.net.2"]
    for block in range(2):
        step.run_block(block, inputs_d)
        torch.cuda.synchronize()
        w, b = blocks[block]
        for gemm, role, names, gelu in GEMMS:
            wc = torch.cat([w[n] for n in names])
            bc = torch.cat([b[n] for n in names])
            epi = "gelu_tanh" if gelu else "none"
            if gemm == "ffn.net.0.proj":
                href, S1 = oracle.linear_ref(*quant_ref(inputs[role]), *quant_ref(wc), bias=f64(bc), epilogue=epi)
                assert_requant_valid(*slab_rows_of(step.ffn_hidden, torch.arange(M)), requant_range(href, S1, epi),
                                     what=f"block {block} {gemm}")
            elif gemm == "ffn.net.2":
                assert_chain_close(step.outputs[gemm], href, S1, "gelu_tanh", *quant_ref(wc), f64(bc),
                                   what=f"block {block} {gemm}")
            else:
                yref, S = oracle.linear_ref(*quant_ref(inputs[role]), *quant_ref(wc), bias=f64(bc), epilogue=epi)
                assert_linear_close(step.outputs[gemm], yref, S, epi, what=f"block {block} {gemm}")


def test_denoise_step_rejects_bad_inputs():
    from mxfp8_w8a8_quantized_amd.denoise import DenoiseStepLinears

    d = dev()
    step = DenoiseStepLinears(1, 64, 8, 128, 256, d)
    with pytest.raises(RuntimeError):
        step.run_block(0, {})
    w, b = {}, {}
    for slot, (shp, _) in enumerate(synth.DENOISE_LINEARS):
        N = 256 if shp.name == "ffn.net.0.proj" else 128
        K = 256 if shp.name == "ffn.net.2" else 128
        w[shp.name] = torch.zeros((N, K), device=d)
        b[shp.name] = torch.zeros((N,), dtype=torch.float16, device=d)
    step.set_block(0, w, b)
    with pytest.raises(KeyError):
        step.run_block(0, {"attn1": torch.zeros((64, 128), dtype=torch.bfloat16, device=d)})
    bad = {r: torch.zeros((64 if r != "text" else 8, 128), dtype=torch.bfloat16, device=d) for r in
           ("attn1", "attn1.out", "attn2", "text", "attn2.out", "ffn")}
    bad["ffn"] = torch.zeros((64, 128), dtype=torch.float16, device=d)
    with pytest.raises(ValueError):
        step.run_block(0, bad)
    with pytest.raises(IndexError):
        step.set_block(1, w, b)
