"""Seeded generators and the workload table (see the package docstring)."""

from dataclasses import dataclass

import torch

HIDDEN = 5120  # Wan2.2-A14B model width (K of q/k/v/out and ffn up)
FFN = 13824  # Wan2.2-A14B feed-forward width
TEXT_TOKENS = 512
TEXT_PAD_FRACTION = 0.2


def video_tokens(width=832, height=1104, frames=81, t_stride=4, s_stride=8, patch=2):
    """Token count of a Wan2.2 video latent after patchification.

    The VAE keeps the first frame and compresses the rest 4x in time, 8x in
    space; the transformer then takes 2x2 patches.
    """
    t = (frames - 1) // t_stride + 1
    h = height // (s_stride * patch)
    w = width // (s_stride * patch)
    return t * h * w


VIDEO_TOKENS = video_tokens()  # 21 * 69 * 52 = 75348

# Per-tensor stream offsets from the base seed.
SEED_X, SEED_W, SEED_B, SEED_MASK, SEED_W2, SEED_B2 = 1, 2, 3, 4, 5, 6


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def make_activation(M, K, seed, outlier_p=1e-3, outlier_scale=50.0, chunk_rows=4096):
    """bf16 [M, K]: fp32 N(0,1), entries under a Bernoulli(outlier_p) mask
    multiplied by outlier_scale, then cast to bf16 (round to nearest even).

    Drawn in row chunks (each chunk seeded from (seed, chunk index)) so the
    fp32 temporaries stay small at M = 75348 and any row block can be
    regenerated alone.
    """
    out = torch.empty((M, K), dtype=torch.bfloat16)
    for c0 in range(0, M, chunk_rows):
        rows = min(chunk_rows, M - c0)
        ci = c0 // chunk_rows
        v = torch.randn((rows, K), generator=_gen(seed * 1_000_003 + SEED_X * 7919 + ci))
        if outlier_p > 0:
            mask = torch.rand((rows, K), generator=_gen(seed * 1_000_003 + SEED_MASK * 7919 + ci)) < outlier_p
            v = torch.where(mask, v * outlier_scale, v)
        out[c0 : c0 + rows] = v.to(torch.bfloat16)
    return out


def make_activation_device(M, K, seed, device, outlier_p=1e-3, outlier_scale=50.0):
    """The recipe of make_activation drawn with a seeded generator on
    `device` (other values, same distribution): for timing runs whose inputs
    the oracle never sees, where drawing 1e9 values on the host is slow."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + SEED_X * 7919)
    v = torch.randn((M, K), device=device, generator=g)
    if outlier_p > 0:
        mask = torch.rand((M, K), device=device, generator=g) < outlier_p
        v = torch.where(mask, v * outlier_scale, v)
    return v.to(torch.bfloat16)


def make_weight_device(N, K, seed, device, std=0.02, stream=SEED_W):
    """make_weight's recipe drawn on `device` (see make_activation_device)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + stream * 7919)
    return torch.randn((N, K), device=device, generator=g) * std


def make_text_context(M, K, seed, pad_fraction=TEXT_PAD_FRACTION):
    """bf16 [M, K] ~ N(0,1) with its last floor(pad_fraction * M) rows zero."""
    x = make_activation(M, K, seed, outlier_p=0.0)
    n_pad = int(pad_fraction * M)
    if n_pad:
        x[M - n_pad :] = 0
    return x


def make_weight(N, K, seed, std=0.02, stream=SEED_W):
    """fp32 [N, K] ~ N(0, std) (nn.Linear orientation)."""
    return torch.randn((N, K), generator=_gen(seed * 1_000_003 + stream * 7919)) * std


def make_bias(N, seed, std=0.01, stream=SEED_B):
    """f16 [N]: fp32 N(0, std) cast to f16 (round to nearest even)."""
    return (torch.randn((N,), generator=_gen(seed * 1_000_003 + stream * 7919)) * std).to(torch.float16)


def block_layer_seed(block, slot):
    """Seed of the weights of layer `slot` (0..9) of transformer block `block`."""
    return 10000 + 10 * block + slot


@dataclass(frozen=True)
class LinearShape:
    name: str
    M: int
    K: int
    N: int
    gelu: bool = False


# The workloads: one entry per linear call, in call order.
CONFIGS = {
    # Single linear, 128 tokens.
    "single_128x5120x5120": [LinearShape("linear", 128, HIDDEN, HIDDEN)],
    # Fused self-attention q|k|v projection over the full video latent.
    "qkv_75348x5120x15360": [LinearShape("attn1.qkv", VIDEO_TOKENS, HIDDEN, 3 * HIDDEN)],
    # FFN pair: up-projection with GELU-tanh, then the down-projection on the
    # re-quantized intermediate.
    "ffn_75348x5120x13824": [
        LinearShape("ffn.net.0.proj", VIDEO_TOKENS, HIDDEN, FFN, gelu=True),
        LinearShape("ffn.net.2", VIDEO_TOKENS, FFN, HIDDEN),
    ],
    # Cross-attention: fused k|v on the text context, q and out on the video.
    "xattn_512x5120x10240": [
        LinearShape("attn2.kv", TEXT_TOKENS, HIDDEN, 2 * HIDDEN),
        LinearShape("attn2.q", VIDEO_TOKENS, HIDDEN, HIDDEN),
        LinearShape("attn2.out", VIDEO_TOKENS, HIDDEN, HIDDEN),
    ],
}
