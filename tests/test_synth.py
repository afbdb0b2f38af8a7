"""The seeded input generators: reproducible, right shapes and distributions,
and the workload geometry derived from the pages' official example."""

import hashlib
import json
import os

import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_constants.json")


def digest(t):
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def test_same_seed_same_bytes():
    assert digest(synth.make_activation(300, 256, 0)) == digest(synth.make_activation(300, 256, 0))
    assert digest(synth.make_activation(300, 256, 0)) != digest(synth.make_activation(300, 256, 1))
    assert digest(synth.make_weight(64, 256, 0)) == digest(synth.make_weight(64, 256, 0))
    assert digest(synth.make_bias(64, 0)) == digest(synth.make_bias(64, 0))


def test_row_chunks_regenerate_alone():
    a = synth.make_activation(70, 64, 5, chunk_rows=32)
    b = synth.make_activation(70, 64, 5, chunk_rows=32)
    assert torch.equal(a, b)


def test_dtypes_and_distributions():
    x = synth.make_activation(2048, 1024, 0)
    assert x.dtype == torch.bfloat16
    big = (x.float().abs() > 6).float().mean().item()
    assert 2e-4 < big < 2e-3  # the 0.1% outliers (x50), nearly all beyond 6 sigma
    w = synth.make_weight(512, 1024, 0)
    assert w.dtype == torch.float32 and abs(w.std().item() - 0.02) < 1e-3
    b = synth.make_bias(4096, 0)
    assert b.dtype == torch.float16 and abs(b.float().std().item() - 0.01) < 1e-3


def test_text_context_padding():
    c = synth.make_text_context(512, 256, 0)
    assert torch.all(c[410:] == 0)
    assert torch.all(c[:410].abs().sum(dim=1) > 0)
    assert 512 - 410 == int(0.2 * 512)


def test_video_token_count_from_official_example():
    ex = json.load(open(GOLDEN))["official_example"]
    M = synth.video_tokens(ex["width"], ex["height"], ex["frames"])
    assert M == 21 * 52 * 69 == 75348 == synth.VIDEO_TOKENS


def test_workload_shapes():
    c = synth.CONFIGS
    assert [(s.M, s.K, s.N) for s in c["single_128x5120x5120"]] == [(128, 5120, 5120)]
    assert [(s.M, s.K, s.N) for s in c["qkv_75348x5120x15360"]] == [(75348, 5120, 15360)]
    assert [(s.M, s.K, s.N, s.gelu) for s in c["ffn_75348x5120x13824"]] == [
        (75348, 5120, 13824, True),
        (75348, 13824, 5120, False),
    ]
    for shapes in c.values():
        for s in shapes:
            assert s.K % 32 == 0


def test_denoise_step_table():
    # Ten quantized linears per block, 40 blocks, as the model card lists
    # them; about 14 GiB of E4M3 codes + E8M0 scales in all.
    lin = synth.DENOISE_LINEARS
    assert synth.DENOISE_BLOCKS == 40 and len(lin) == 10
    assert [s.name for s, _ in lin] == [
        "attn1.to_q", "attn1.to_k", "attn1.to_v", "attn1.to_out.0",
        "attn2.to_q", "attn2.to_k", "attn2.to_v", "attn2.to_out.0",
        "ffn.net.0.proj", "ffn.net.2",
    ]
    assert {r for _, r in lin if r} == set(synth.DENOISE_ROLE_SEEDS)
    n_param = sum(s.N * s.K for s, _ in lin) * synth.DENOISE_BLOCKS
    gib = n_param * (1 + 1 / 32) / 2**30
    assert 13.0 < gib < 14.0
    flop = 2 * sum(s.M * s.N * s.K for s, _ in lin) * synth.DENOISE_BLOCKS
    assert abs(flop / 1.8035e15 - 1) < 1e-3
    seeds = {synth.block_layer_seed(b, i) for b in range(40) for i in range(10)}
    assert len(seeds) == 400


def test_denoise_block_weights_are_seeded_per_slot():
    w0, b0 = synth.make_denoise_block(0)
    w0b, _ = synth.make_denoise_block(0)
    assert all(torch.equal(w0[k], w0b[k]) for k in w0)
    w1, _ = synth.make_denoise_block(1)
    assert not torch.equal(w0["attn1.to_q"], w1["attn1.to_q"])
    assert not torch.equal(w0["attn1.to_q"][:16], w0["attn1.to_k"][:16])
    assert w0["ffn.net.2"].shape == (5120, 13824) and b0["ffn.net.0.proj"].dtype == torch.float16
