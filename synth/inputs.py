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


# One denoise step: the ten quantized linears of each transformer block, in
# call order (slot i of block b draws its weight and bias from
# block_layer_seed(b, i)). Each linear reads the activation of one input
# role; the roles stand in for the tensors the unquantized parts of the block
# (norms, attention, residual adds) would hand over, so every video-side role
# is a bf16 [VIDEO_TOKENS, HIDDEN] activation of the usual recipe and the text
# role is the padded text context. ffn.net.2 reads the requantized output of
# ffn.net.0.proj instead of a role.
DENOISE_BLOCKS = 40
DENOISE_LINEARS = (
    (LinearShape("attn1.to_q", VIDEO_TOKENS, HIDDEN, HIDDEN), "attn1"),
    (LinearShape("attn1.to_k", VIDEO_TOKENS, HIDDEN, HIDDEN), "attn1"),
    (LinearShape("attn1.to_v", VIDEO_TOKENS, HIDDEN, HIDDEN), "attn1"),
    (LinearShape("attn1.to_out.0", VIDEO_TOKENS, HIDDEN, HIDDEN), "attn1.out"),
    (LinearShape("attn2.to_q", VIDEO_TOKENS, HIDDEN, HIDDEN), "attn2"),
    (LinearShape("attn2.to_k", TEXT_TOKENS, HIDDEN, HIDDEN), "text"),
    (LinearShape("attn2.to_v", TEXT_TOKENS, HIDDEN, HIDDEN), "text"),
    (LinearShape("attn2.to_out.0", VIDEO_TOKENS, HIDDEN, HIDDEN), "attn2.out"),
    (LinearShape("ffn.net.0.proj", VIDEO_TOKENS, HIDDEN, FFN, gelu=True), "ffn"),
    (LinearShape("ffn.net.2", VIDEO_TOKENS, FFN, HIDDEN), None),
)
DENOISE_ROLE_SEEDS = {"attn1": 101, "attn1.out": 102, "attn2": 103, "attn2.out": 104, "ffn": 105, "text": 106}


def make_denoise_inputs(device=None, on_device=False):
    """The activation of every input role of the denoise step (see
    DENOISE_LINEARS), seeded by DENOISE_ROLE_SEEDS. Drawn on the host and
    moved to `device`, or with on_device=True drawn there directly."""
    out = {}
    for role, seed in DENOISE_ROLE_SEEDS.items():
        if role == "text":
            x = make_text_context(TEXT_TOKENS, HIDDEN, seed)
        elif on_device:
            x = make_activation_device(VIDEO_TOKENS, HIDDEN, seed, device)
        else:
            x = make_activation(VIDEO_TOKENS, HIDDEN, seed)
        out[role] = x.to(device) if device is not None else x
    return out


def make_denoise_block(block, device=None, on_device=False):
    """Weights (fp32 [N, K]) and f16 biases of the ten linears of one block,
    keyed by linear name; on_device=True draws the weights on `device`."""
    weights, biases = {}, {}
    for slot, (shp, _) in enumerate(DENOISE_LINEARS):
        seed = block_layer_seed(block, slot)
        if on_device:
            w = make_weight_device(shp.N, shp.K, seed, device)
        else:
            w = make_weight(shp.N, shp.K, seed)
        b = make_bias(shp.N, seed)
        weights[shp.name] = w.to(device) if device is not None else w
        biases[shp.name] = b.to(device) if device is not None else b
    return weights, biases
