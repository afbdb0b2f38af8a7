"""Seeded synthetic inputs for the Wan2.2-A14B MXFP8 linear shapes.

This module holds no arithmetic of the quantization method: it only draws
random tensors with ``torch.Generator('cpu')`` (so every caller sees the same
bytes for the same seed) and casts them to the dtypes the layer takes. Both
the oracle's callers and the GPU path's callers use it; it imports neither.
The ``*_device`` variants draw the same recipe with a seeded generator on a
GPU, for timing runs whose inputs the oracle never sees.

Shapes (model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
sections "Quantization Details" and "Running the Official Example"):
the quantized linears are attn1/attn2 q, k, v, out and ffn.net.0.proj /
ffn.net.2 in each of 40 blocks; the official example is 832x1104, 81 frames.
With the Wan VAE's 4x temporal / 8x spatial compression and 2x2 patches that
is 21 x 52 x 69 = 75348 tokens. The hidden size 5120 and FFN size 13824 are
Wan2.2-A14B's. Text context is 512 tokens.

Value recipe: activations fp32 N(0, 1) with 0.1% of entries (Bernoulli mask)
multiplied by 50 as outliers, cast once to bf16; weights fp32 N(0, 0.02);
biases fp32 N(0, 0.01) cast to f16. Text context rows past 80% of the length
are zero (padding).
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    DENOISE_BLOCKS,
    DENOISE_LINEARS,
    DENOISE_ROLE_SEEDS,
    HIDDEN,
    FFN,
    TEXT_TOKENS,
    VIDEO_TOKENS,
    LinearShape,
    block_layer_seed,
    make_activation,
    make_activation_device,
    make_bias,
    make_denoise_block,
    make_denoise_inputs,
    make_text_context,
    make_weight,
    make_weight_device,
    video_tokens,
)
