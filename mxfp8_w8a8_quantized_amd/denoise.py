"""The quantized linears of one Wan2.2-A14B denoise step, run back to back.

Model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)", section
"Quantization Details": every transformer block carries ten MXFP8 W8A8
linears (self-attention attn1 q, k, v, out; cross-attention attn2 q, k, v,
out; the feed-forward ffn.net.0.proj with GELU-tanh and ffn.net.2), 40 blocks
in all, each with its own E4M3 weights, E8M0 scales and F16 bias, and each
quantizing its activation at run time.

This module only arranges library calls; every value is computed by the HIP
kernels behind the C ABI:

* attn1 q, k and v read the same hidden states, so they run as one GEMM on
  the row-concatenated weights (N = 3 * hidden); attn2 k and v likewise on the
  text tokens (N = 2 * hidden). An output column depends only on its own weight
  row, so the concatenation changes no value; the outputs are column blocks
  of one bf16 tensor.
* Each of those linears is one mx_linear call: the activation is quantized
  into the shared workspace slab, then multiplied by the slab weights through
  the shape's plan (tuned by ``tune()`` on the block's real operands, else
  the default rule: split-K for the 512 text tokens, whose 256 x 256 tiles
  are too few to occupy the GPU, the slab GEMM for the video tokens).
* The feed-forward pair quantizes its input into the workspace, runs
  ffn.net.0.proj with the requantizing epilogue (the MX slab of its bf16 GELU
  output, never written as bf16) and ffn.net.2 on that slab through its plan
  (mx_linear_slab_auto: tuned by ``tune()``, else the default rule).

The parts of a block that are not quantized linears (norms, modulation,
attention itself, residual adds) are not here: the caller hands in the
activation each linear reads, by input role (``ROLES``).
"""

import torch

from . import Slab, mx_linear, mx_linear_slab_auto, mx_linear_slab_requant, mx_linear_tune, mx_linear_tune_ws_bytes
from . import mx_linear_ws_bytes, mx_quantize_act_slab, mx_quantize_weight_slab, mx_slab_rows, plan_lookup

# Input role of each GEMM of a block, in call order, with the linears it
# fuses (names as in the Wan2.2 transformer's state dict).
GEMMS = (
    ("attn1.qkv", "attn1", ("attn1.to_q", "attn1.to_k", "attn1.to_v"), False),
    ("attn1.to_out.0", "attn1.out", ("attn1.to_out.0",), False),
    ("attn2.to_q", "attn2", ("attn2.to_q",), False),
    ("attn2.kv", "text", ("attn2.to_k", "attn2.to_v"), False),
    ("attn2.to_out.0", "attn2.out", ("attn2.to_out.0",), False),
    ("ffn.net.0.proj", "ffn", ("ffn.net.0.proj",), True),
    ("ffn.net.2", None, ("ffn.net.2",), False),
)
ROLES = ("attn1", "attn1.out", "attn2", "text", "attn2.out", "ffn")
LINEARS = tuple(name for _, _, names, _ in GEMMS for name in names)


class DenoiseStepLinears:
    """Slab weights of `blocks` transformer blocks and the buffers to run
    their 10 * blocks quantized linears on `tokens` video tokens and
    `text_tokens` text tokens.

    set_block() quantizes one block's weights; run_block() / run() enqueue the
    linears on the current stream of `device`. Outputs (bf16, overwritten by
    every block) are in ``outputs``, keyed by GEMM name; the feed-forward
    intermediate stays an MX slab (``ffn_hidden``).
    """

    def __init__(self, blocks, tokens, text_tokens, hidden, ffn, device):
        self.blocks, self.tokens, self.text_tokens = blocks, tokens, text_tokens
        self.hidden, self.ffn, self.device = hidden, ffn, torch.device(device)
        self.weights = [None] * blocks
        self.rows = {"attn1": tokens, "attn1.out": tokens, "attn2": tokens, "text": text_tokens,
                     "attn2.out": tokens, "ffn": tokens}
        n_out = {"attn1.qkv": 3 * hidden, "attn1.to_out.0": hidden, "attn2.to_q": hidden,
                 "attn2.kv": 2 * hidden, "attn2.to_out.0": hidden, "ffn.net.2": hidden}
        self.outputs = {}
        for gemm, role, _, _ in GEMMS:
            if gemm in n_out:
                M = tokens if role is None else self.rows[role]
                self.outputs[gemm] = torch.empty((M, n_out[gemm]), dtype=torch.bfloat16, device=self.device)
        self.ffn_hidden = Slab(
            torch.empty((ffn // 64, mx_slab_rows(tokens), 64), dtype=torch.uint8, device=self.device),
            torch.empty((ffn // 64, mx_slab_rows(tokens), 2), dtype=torch.uint8, device=self.device),
            tokens,
        )
        # One workspace for every one-call linear of a block: the activation
        # slab first (also the feed-forward input, viewed as a slab below),
        # then what the shape's plan needs.
        ws = max(mx_linear_ws_bytes(M, K, N) for gemm, M, K, N, _ in self.shapes() if gemm != "ffn.net.2")
        if ws < 0 or mx_linear_tune_ws_bytes(tokens, ffn, hidden) < 0:
            raise ValueError("hidden and ffn must be multiples of 64")
        # ffn.net.2 reads the intermediate slab, so any plan's partial sums
        # for it fit the whole workspace (the up-projection is done with the
        # activation slab at its start by then).
        ws = max(ws, mx_linear_tune_ws_bytes(tokens, ffn, hidden))
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=self.device)
        self.ffn_input = self._slab_view(tokens)
        self.tuned = {}

    def _slab_view(self, rows):
        R = mx_slab_rows(rows)
        nq = R * self.hidden
        return Slab(
            self.workspace[:nq].view(self.hidden // 64, R, 64),
            self.workspace[nq : nq + nq // 32].view(self.hidden // 64, R, 2),
            rows,
        )

    def shapes(self):
        """(gemm name, M, K, N, gelu) of the GEMMs of one block, in call order."""
        out = []
        for gemm, role, names, gelu in GEMMS:
            M = self.tokens if role is None else self.rows[role]
            K = self.ffn if gemm == "ffn.net.2" else self.hidden
            N = {"attn1.qkv": 3 * self.hidden, "attn2.kv": 2 * self.hidden, "ffn.net.0.proj": self.ffn}.get(
                gemm, self.hidden)
            out.append((gemm, M, K, N, gelu))
        return out

    def flop(self):
        """Multiply-adds x 2 of one whole step (all blocks)."""
        return self.blocks * sum(2.0 * M * K * N for _, M, K, N, _ in self.shapes())

    def set_block(self, block, weights, biases):
        """Quantize block `block`'s weights into slabs. weights: linear name ->
        fp32 or bf16 [N, K] on the device (nn.Linear orientation); biases:
        linear name -> f16 [N] on the device. The caller's tensors are not kept."""
        if not 0 <= block < self.blocks:
            raise IndexError(f"block {block} out of range [0, {self.blocks})")
        missing = [n for n in LINEARS if n not in weights or n not in biases]
        if missing:
            raise KeyError(f"missing weights or biases for {missing}")
        slabs = {}
        for gemm, _, names, _ in GEMMS:
            w = weights[names[0]] if len(names) == 1 else torch.cat([weights[n] for n in names], dim=0)
            b = biases[names[0]] if len(names) == 1 else torch.cat([biases[n] for n in names], dim=0)
            slabs[gemm] = (mx_quantize_weight_slab(w), b.contiguous())
        self.weights[block] = slabs

    def _check_inputs(self, inputs):
        for role in ROLES:
            x = inputs.get(role)
            if x is None:
                raise KeyError(f"missing input role {role!r}")
            if x.device != self.device or x.dtype != torch.bfloat16 or tuple(x.shape) != (self.rows[role], self.hidden):
                raise ValueError(f"input {role!r} must be bf16 [{self.rows[role]}, {self.hidden}] on {self.device}")

    def run_block(self, block, inputs, check=True):
        """Enqueue block `block`'s linears on the inputs (role -> bf16 tensor)."""
        slabs = self.weights[block]
        if slabs is None:
            raise RuntimeError(f"block {block} has no weights (set_block)")
        if check:
            self._check_inputs(inputs)
        for gemm, role, _, gelu in GEMMS:
            w, b = slabs[gemm]
            if gemm == "ffn.net.0.proj":
                mx_quantize_act_slab(inputs[role], self.ffn_input)
                mx_linear_slab_requant(self.ffn_input, w, b, gelu=gelu, out=self.ffn_hidden)
            elif gemm == "ffn.net.2":
                mx_linear_slab_auto(self.ffn_hidden, w, b, gelu=gelu, y=self.outputs[gemm], workspace=self.workspace)
            else:
                mx_linear(inputs[role], w, b, gelu=gelu, y=self.outputs[gemm], workspace=self.workspace)

    def tune(self, inputs, block=0, reps=5):
        """Warm-up tuning (mx_linear_tune) of the planned GEMMs of a block on
        block `block`'s weights and the given inputs (ffn.net.2 on the
        intermediate slab the up-projection writes from them): each shape's
        candidate kernels are timed once and the fastest is cached for the
        process, so every later run() takes it. Synchronizes; returns
        {gemm: plan} with the plan each GEMM runs from now on."""
        slabs = self.weights[block]
        if slabs is None:
            raise RuntimeError(f"block {block} has no weights (set_block)")
        self._check_inputs(inputs)
        tune_ws = None
        for gemm, role, _, gelu in GEMMS:
            if gemm == "ffn.net.0.proj":
                continue  # the requantizing epilogue runs the slab GEMM itself
            w, b = slabs[gemm]
            if gemm == "ffn.net.2":
                # on the intermediate slab that the up-projection writes
                w1, b1 = slabs["ffn.net.0.proj"]
                mx_quantize_act_slab(inputs["ffn"], self.ffn_input)
                mx_linear_slab_requant(self.ffn_input, w1, b1, gelu=True, out=self.ffn_hidden)
                xs, M, K = self.ffn_hidden, self.tokens, self.ffn
            else:
                M, K = self.rows[role], self.hidden
                xs = self._slab_view(M)
                mx_quantize_act_slab(inputs[role], xs)
            N = w.rows
            need = max(mx_linear_tune_ws_bytes(M, K, N), 1)
            if tune_ws is None or tune_ws.numel() < need:
                tune_ws = torch.empty((need,), dtype=torch.uint8, device=self.device)
            self.tuned[gemm] = mx_linear_tune(xs, w, b, gelu=gelu, y=self.outputs[gemm], workspace=tune_ws,
                                              reps=reps)
        del tune_ws
        return self.plans()

    def plans(self):
        """{gemm: (kind, splits)} each planned GEMM runs with (the plan
        lookup of mx_linear and mx_linear_slab_auto: tuned, else the default
        rule); ffn.net.0.proj always runs the slab kernel with the
        requantizing epilogue."""
        return {gemm: plan_lookup(M, K, N, gelu) for gemm, M, K, N, gelu in self.shapes()
                if gemm != "ffn.net.0.proj"}

    def run(self, inputs):
        """Enqueue the whole step: every block's linears, in block order."""
        self._check_inputs(inputs)
        for block in range(self.blocks):
            self.run_block(block, inputs, check=False)
