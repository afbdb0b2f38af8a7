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
