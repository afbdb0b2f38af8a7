#!/usr/bin/env python3
"""Benchmark of the MXFP8 W8A8 linear on one MI355X.

Workload: the fused self-attention q|k|v projection of Wan2.2-A14B over the
full video latent of the official example (832x1104, 81 frames): M = 75348
tokens, K = 5120, N = 15360. Activations bf16 (seeded synthetic, 0.1%
outliers), weights E4M3 + E8M0 (quantized once before timing, as stored
weights are), f16 bias, bf16 output.

One step = the whole hot path on one batch: dynamic MX quantization of the
activations straight into the GEMM's slab layout (mx_quantize_act_slab)
followed by the block-scaled GEMM with bias (mx_linear_slab). The weights are
stored quantized in the slab layout (mx_quantize_weight_slab, once, before
timing). Throughput counts the algorithmic 2*M*N*K FLOP per step.

Prints ONE JSON line. Besides the contract fields it carries
  roofline      the dominant kernel (the GEMM) against the dense MXFP8 MFMA
                peak, from its per-launch HIP-event times on the launch
                stream; `traffic` is the HBM bytes per launch from the
                committed rocprofv3 counter summary when that was taken on
                the current kernel sources, else null; `mfma_probe_TFLOPs`
                is the scaled MFMA's sustained rate from registers (no
                memory traffic) on this workload's codes and on zeros, and
                `frac_of_probe` the GEMM against the former;
  cpu_baseline  the float64 CPU oracle timed on a bounded row sample of the
                same inputs;
  extra         p10/p50/p90 of the step and GEMM times, the step with cold
                caches (a 1 GiB write before each rep), the activation
                quantizer's bandwidth, the same step on
                row-major operands (mx_quantize_act + mx_linear_q), the
                fused-prologue path (mx_linear), the weight quantizer, the
                other Wan2.2 linears, one whole denoise step's 400 linears
                (40 blocks) back to back, and one GPU's share of a two-way
                tensor-parallel split of four linears.

Modes for profiling: --profile step|quant|rowmajor|fused runs only those kernels
(steps times, no oracle); --profile single|ffn|xattn runs one of the other
workloads (the 128-token linear; the FFN pair as two one-call linears, then
with the requantizing epilogue; the cross-attention set); --profile workloads
runs all of them, the per-channel FP8 step and one whole denoise step twice
each; --profile-copy runs a 1 GiB device copy (its GB/s, and the calibration
of the HBM byte counters).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 W8A8 linear TFLOP/s incl. act-quant, M=75348 K=5120; % of MXFP8 peak"
WORKLOAD = "qkv_75348x5120x15360"
PEAK_MXFP8_TFLOPS = 5000.0  # MI355X dense MXFP8/FP8 MFMA peak
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_linear_qkv_75348x5120x15360.json")
GEMM_SOURCES = ["mx_gemm.hip", "mx_device.h"]
CPU_SAMPLE_ROWS = 8192
# The pages' own figures, quoted with their setups (context only: other
# hardware and software, not targets).
CONTEXT = {
    "quantized_weights_GiB_per_transformer": 13.99,
    "quantized_weights_source": "model card 'Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)', "
                                "Quantization Details (E4M3 weights + E8M0 scales of the 400 quantized linears; "
                                "the shape arithmetic here gives 13.49 GiB)",
    "mlx_gen_q8_s": 217.4,
    "mlx_gen_bf16_s": 95.48,
    "mlx_gen_setup": "'Planned: Wan quantization and motion parity', Current code reality: MLX-Gen q8 against "
                     "BF16, 704x384, 25 frames, 12 steps, on that project's local Apple-MLX machine (the q8 format "
                     "is not MXFP8)",
}


def kernel_source_hash():
    """Hash of the GEMM sources' code: comments dropped and whitespace runs
    folded (neither source puts // or /* in a string), so that a comment edit
    keeps the committed counters valid and any code edit voids them."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mxfp8_w8a8_quantized_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 30 warm-up steps: the GPU's clock settles over the first ~20 steps of
    # this GEMM (4.5 ms, then 4.32-4.35 ms per launch on MI355X).
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--profile", choices=["step", "rowmajor", "fused", "workloads", "quant", "single", "ffn", "xattn"],
                    help="run only these kernels")
    ap.add_argument("--profile-copy", action="store_true", help="run only a 1 GiB device copy")
    return ap.parse_args()


def timed_step(torch, fns, steps, warmup):
    """Runs the kernels fns[0], fns[1], ... as one step, warmup times then
    steps times, with a HIP event pair around each kernel on the current
    stream. Returns (total ms, [per-kernel list of per-launch ms])."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(steps):
        ev[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    per = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)] for i in range(len(fns))]
    return start.elapsed_time(end), per


def device_copy_gbps(torch, dev, steps=10, warmup=3):
    """GB/s of a plain 1 GiB device-to-device copy (torch's copy kernel):
    read + write bytes over time, the practical HBM rate that an HBM-bound
    kernel moving about as much as it reads can be held to on this GPU."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    total, _ = timed_step(torch, [lambda: b.copy_(a)], steps, warmup)
    del a, b
    torch.cuda.empty_cache()
    return round(2 * n / (total / steps * 1e-3) / 1e9, 1)


def graph_ms(torch, fn, reps, per_graph=5):
    """ms per call of fn replayed from a captured HIP graph (per_graph calls
    per graph), i.e. without the host's launch cost: what a serving loop
    that captures its launches would see."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * per_graph)
    del g
    return ms


def mean(v):
    return sum(v) / len(v)


def cpu_baseline(x_cpu, w_cpu, b_cpu, rows):
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    wq, ws = oracle.quantize_mx(w_cpu.double().numpy())  # offline, like the GPU's weights
    xr = x_cpu[:rows].double().numpy()
    b = b_cpu.double().numpy()
    t0 = time.perf_counter()
    xq, xs = oracle.quantize_mx(xr)
    y, S = oracle.linear_ref(xq, xs, wq, ws, bias=b)
    dt = time.perf_counter() - t0
    assert np.isfinite(y).all()
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": round(2.0 * rows * K * N / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {M} token rows x all {N} outputs (K={K}): float64 activation quantization + "
        f"dequantized GEMM with its sum|a||b| bound, {dt:.1f} s; FLOP counted as 2*rows*N*K",
    }


def percentiles(v):
    """p10, median and p90 of a list of per-launch times (ms)."""
    v = sorted(v)
    at = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]  # noqa: E731
    return [round(at(0.1), 4), round(at(0.5), 4), round(at(0.9), 4)]


def cold_steps(torch, dev, fns, reps):
    """The step with cold caches: before each rep a 1 GiB scratch write
    evicts the L2s and the 256 MB Infinity Cache, then the step's kernels
    run between HIP events. Returns per-step median ms and p10/p50/p90 of
    the step and of its last kernel (the GEMM)."""
    scratch = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    steps, last = [], []
    for r in range(reps + 1):
        scratch.fill_(r & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        ev[0].record()
        for i, f in enumerate(fns):
            f()
            ev[i + 1].record()
        torch.cuda.synchronize()
        if r == 0:
            continue  # the first rep warms the launch path
        steps.append(ev[0].elapsed_time(ev[-1]))
        last.append(ev[-2].elapsed_time(ev[-1]))
    del scratch
    return {"step_ms_p10_p50_p90": percentiles(steps), "gemm_ms_p10_p50_p90": percentiles(last), "reps": reps,
            "evict": "1 GiB device write before each rep"}


def mfma_probe(torch, mx, dev, a_codes, b_codes, iters=2000, reps=10):
    """The scaled FP8 MFMA's sustained rate with operands in registers and no
    memory traffic (mx_probe_mfma, one 4-wave workgroup per CU), on this
    workload's own activation and weight codes and on zero codes: the clock
    the chip holds depends on the operand bits, so this is the ceiling the
    GEMM's MFMAs face, next to the 5.0 PFLOP/s nominal peak."""
    n = 8 << 20  # bytes of codes each lane group draws from
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty((ncu * 256,), dtype=torch.float32, device=dev)
    out = {}
    for name, a, b in (("workload_codes", a_codes.view(-1)[:n], b_codes.view(-1)[:n]),
                       ("zero_codes", torch.zeros(n, dtype=torch.uint8, device=dev),
                        torch.zeros(n, dtype=torch.uint8, device=dev))):
        for _ in range(5):
            flop = mx.mx_probe_mfma(a, b, iters, ncu, sink)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            mx.mx_probe_mfma(a, b, iters, ncu, sink)
        ev[1].record()
        torch.cuda.synchronize()
        out[name] = round(flop * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12, 1)
    out["unit"] = "TFLOP/s"
    return out


def workload_roofline(layers, flop, ms):
    """Where a workload stands against its bound, per step at time ms:
    algorithmic HBM bytes (bf16 activations read, weight codes + scales, f16
    bias, bf16 output; the activation codes that the quantizer writes and the
    GEMM reads back are this implementation's, not the linear's, and are not
    counted) against 8 TB/s, and 2*M*N*K against the 5.0 PFLOP/s dense MXFP8
    peak. The bound is the one with the larger time at peak (HBM for the
    128-token linear, MFMA for the others)."""
    nbytes = 0
    for shp, _, _ in layers:
        nbytes += shp.M * shp.K * 2  # bf16 activations in
        nbytes += shp.N * shp.K + shp.N * shp.K // 32 + shp.N * 2 + shp.M * shp.N * 2
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    t_mfma = flop / (PEAK_MXFP8_TFLOPS * 1e12)
    if t_hbm > t_mfma:
        ach = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "bytes": nbytes}
    ach = flop / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_MXFP8_TFLOPS, 4), "bytes": nbytes}


def other_workloads(torch, mx, synth, dev, steps=10, warmup=3):
    """The other Wan2.2-A14B linears on the slab path, one step each: every
    linear quantizes its activation into a slab and runs the GEMM; the FFN's
    down-projection takes the up-projection's bf16 GELU output. Inputs are
    drawn on the GPU (same recipe as the headline's, other seed)."""
    res = {}
    for name, shapes in synth.CONFIGS.items():
        if name == WORKLOAD:
            continue
        layers = []
        for li, shp in enumerate(shapes):
            seed = 500 + li
            w = mx.mx_quantize_weight_slab(synth.make_weight_device(shp.N, shp.K, seed, dev))
            b = synth.make_bias(shp.N, seed).to(dev)
            layers.append((shp, w, b))
        acts = []
        for li, (shp, w, b) in enumerate(layers):
            if shp.name == "ffn.net.2":
                acts.append(None)  # the previous layer's output
                continue
            if shp.M == synth.TEXT_TOKENS:
                x = synth.make_text_context(shp.M, shp.K, 500 + li).to(dev)
            else:
                x = synth.make_activation_device(shp.M, shp.K, 500 + li, dev)
            acts.append(x)
        outs = [torch.empty((shp.M, shp.N), dtype=torch.bfloat16, device=dev) for shp, _, _ in layers]
        slabs = [mx.mx_quantize_act_slab(acts[li] if acts[li] is not None else outs[li - 1])
                 for li in range(len(layers))]
        # Each linear is one mx_linear call (quantizer + GEMM through the
        # shape's plan). Plans: the default rule (few-token kernel up to 256
        # tokens, split-K while the 256 x 256 tiles leave CUs idle, else the
        # slab GEMM), then warm-up tuning on the real operands of each linear
        # (mx_linear_tune times the candidate kernels on the quantized slab
        # and caches the fastest); the timed step runs the tuned plans.
        default_plans = [mx.plan_linear(shp.M, shp.K, shp.N) for shp, _, _ in layers]
        wss = [torch.empty((max(mx.mx_linear_ws_bytes(shp.M, shp.K, shp.N), 1),), dtype=torch.uint8, device=dev)
               for shp, _, _ in layers]

        def run():
            for li, (shp, w, b) in enumerate(layers):
                x = acts[li] if acts[li] is not None else outs[li - 1]
                mx.mx_linear(x, w, b, gelu=shp.gelu, y=outs[li], workspace=wss[li])

        for li, (shp, w, b) in enumerate(layers):
            x = acts[li] if acts[li] is not None else outs[li - 1]
            if li > 0 and acts[li] is None:
                run()  # the previous layer's output is this one's input
            mx.mx_quantize_act_slab(x, slabs[li])
            if shp.M <= 4096:  # the large shapes' plan is the slab GEMM; tuning them takes seconds
                tws = torch.empty((max(mx.mx_linear_tune_ws_bytes(shp.M, shp.K, shp.N), 1),), dtype=torch.uint8,
                                  device=dev)
                mx.mx_linear_tune(slabs[li], w, b, gelu=shp.gelu, y=outs[li], workspace=tws, reps=5)
                del tws
        plans = [mx.plan_lookup(shp.M, shp.K, shp.N, shp.gelu) for shp, _, _ in layers]
        run()

        total, _ = timed_step(torch, [run], steps, warmup)
        ms = total / steps
        g_ms = graph_ms(torch, run, steps)
        flop = sum(2.0 * shp.M * shp.N * shp.K for shp, _, _ in layers)
        res[name] = {
            "linears": [f"{shp.name} {shp.M}x{shp.K}x{shp.N}" + (" gelu" if shp.gelu else "")
                        + ("" if pl[0] == "slab" else f" {pl[0]}{pl[1]}")
                        + ("" if pl == d else f" (tuned; default {d[0]}{d[1]})")
                        for (shp, _, _), pl, d in zip(layers, plans, default_plans)],
            "ms": round(ms, 4),
            "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
            "pct_of_mxfp8_peak": round(100.0 * flop / (ms * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS, 2),
            "graph_ms": round(g_ms, 4),
            "graph_TFLOPs": round(flop / (g_ms * 1e-3) / 1e12, 2),
            "roofline": workload_roofline(layers, flop, g_ms),
        }
        if [shp.name for shp, _, _ in layers] == ["ffn.net.0.proj", "ffn.net.2"]:
            # The same pair with the requantization fused into the up-projection.
            (s1, w1, b1), (s2, w2, b2) = layers
            hs = [None]

            def run_fused():
                slabs[0] = mx.mx_quantize_act_slab(acts[0], slabs[0])
                hs[0] = mx.mx_linear_slab_requant(slabs[0], w1, b1, gelu=s1.gelu, out=hs[0])
                mx.mx_linear_slab(hs[0], w2, b2, gelu=s2.gelu, y=outs[1])

            total, _ = timed_step(torch, [run_fused], steps, warmup)
            ms = total / steps
            res[name]["fused_requant_ms"] = round(ms, 4)
            res[name]["fused_requant_TFLOPs"] = round(flop / (ms * 1e-3) / 1e12, 2)
            del hs
        del layers, acts, outs, slabs
        torch.cuda.empty_cache()
    return res


def profile_config(torch, mx, synth, dev, which, steps, warmup):
    """Runs one of the other workloads' linears alone (for kernel traces and
    counters): "single" the 128-token linear, "ffn" the FFN pair as two
    one-call linears and then with the requantizing epilogue, "xattn" the
    cross-attention set; each through mx_linear with the default plans."""
    name = {"single": "single_128x5120x5120", "ffn": "ffn_75348x5120x13824", "xattn": "xattn_512x5120x10240"}[which]
    layers = []
    for li, shp in enumerate(synth.CONFIGS[name]):
        w = mx.mx_quantize_weight_slab(synth.make_weight_device(shp.N, shp.K, 500 + li, dev))
        b = synth.make_bias(shp.N, 500 + li).to(dev)
        if shp.name == "ffn.net.2":
            x = None
        elif shp.M == synth.TEXT_TOKENS:
            x = synth.make_text_context(shp.M, shp.K, 500 + li).to(dev)
        else:
            x = synth.make_activation_device(shp.M, shp.K, 500 + li, dev)
        y = torch.empty((shp.M, shp.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((max(mx.mx_linear_ws_bytes(shp.M, shp.K, shp.N), 1),), dtype=torch.uint8, device=dev)
        layers.append((shp, w, b, x, y, ws))

    def run():
        for li, (shp, w, b, x, y, ws) in enumerate(layers):
            mx.mx_linear(x if x is not None else layers[li - 1][4], w, b, gelu=shp.gelu, y=y, workspace=ws)

    fns = [run]
    if which == "ffn":
        (s1, w1, b1, x1, _, ws1), (s2, w2, b2, _, y2, _) = layers
        xs = mx.mx_quantize_act_slab(x1)
        h = mx.mx_linear_slab_requant(xs, w1, b1, gelu=True)

        def run_requant():
            mx.mx_quantize_act_slab(x1, xs)
            mx.mx_linear_slab_requant(xs, w1, b1, gelu=True, out=h)
            mx.mx_linear_slab(h, w2, b2, y=y2)

        fns.append(run_requant)
    timed_step(torch, fns, steps, warmup)
    print(json.dumps({"profiled": which, "steps": steps,
                      "linears": [f"{shp.name} {shp.M}x{shp.K}x{shp.N} {mx.plan_lookup(shp.M, shp.K, shp.N, shp.gelu)}"
                                  for shp, *_ in layers]}), flush=True)


def denoise_step(torch, synth, dev, steps=2, warmup=1):
    """One full denoise step's quantized linears, back to back: 40 blocks x
    10 linears (q|k|v and the text k|v fused, 7 GEMMs a block), each with its
    own weights drawn on the GPU and quantized to slabs before timing, each
    quantizing its input (the FFN intermediate in the up-projection's
    epilogue)."""
    import mxfp8_w8a8_quantized_amd as mx
    from mxfp8_w8a8_quantized_amd.denoise import DenoiseStepLinears

    step = DenoiseStepLinears(synth.DENOISE_BLOCKS, synth.VIDEO_TOKENS, synth.TEXT_TOKENS, synth.HIDDEN, synth.FFN, dev)
    for block in range(synth.DENOISE_BLOCKS):
        w, b = synth.make_denoise_block(block, dev, on_device=True)
        step.set_block(block, w, b)
        del w, b
    inputs = synth.make_denoise_inputs(dev, on_device=True)
    # The default rule's plans (not plan_lookup: earlier workloads may have
    # cached tuned plans for the same shapes).
    defaults = {g: mx.plan_linear(M, K, N) for g, M, K, N, _ in step.shapes() if g in step.plans()}
    plans = step.tune(inputs)  # warm-up tuning of the block's one-call shapes, cached for the run
    total, _ = timed_step(torch, [lambda: step.run(inputs)], steps, warmup)
    ms = total / steps
    flop = step.flop()
    wbytes = sum(sl.q.numel() + sl.s.numel() for blk in step.weights for sl, _ in blk.values())
    res = {
        "blocks": step.blocks,
        "linears": 10 * step.blocks,
        "gemm_launches": len(step.shapes()) * step.blocks,
        "weight_GiB": round(wbytes / 2**30, 3),
        "ms": round(ms, 3),
        "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
        "pct_of_mxfp8_peak": round(100.0 * flop / (ms * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS, 2),
        "plans": {g: f"{k}{sp}" + ("" if (k, sp) == defaults[g] else f" (tuned; default {defaults[g][0]}{defaults[g][1]})")
                  for g, (k, sp) in plans.items()},
    }
    del step, inputs
    torch.cuda.empty_cache()
    return res


def per_channel_step(torch, mx, synth, dev, M, K, N, steps=10, warmup=3):
    """The per-output-channel FP8 scheme on the headline shape: per-token
    activation quantization (f32 row scales) + the GEMM with the row scales
    in its epilogue; weights quantized per output channel before timing."""
    x = synth.make_activation_device(M, K, 300, dev)
    w = mx.mx_pc_quantize_weight_slab(synth.make_weight_device(N, K, 300, dev))
    b = synth.make_bias(N, 300).to(dev)
    xs = mx.mx_pc_quantize_act_slab(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    total, (q_ms, g_ms) = timed_step(
        torch, [lambda: mx.mx_pc_quantize_act_slab(x, xs), lambda: mx.mx_pc_linear_slab(xs, w, b, y=y)], steps, warmup)
    ms = total / steps
    flop = 2.0 * M * N * K
    act_bytes = M * K * (2 + 1) + M * 4
    res = {
        "step_ms": round(ms, 4),
        "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
        "pct_of_mxfp8_peak": round(100.0 * flop / (ms * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS, 2),
        "gemm_ms": round(mean(g_ms), 4),
        "quantize_act_ms": round(mean(q_ms), 4),
        "quantize_act_GBps": round(act_bytes / (mean(q_ms) * 1e-3) / 1e9, 1),
    }
    del x, w, xs, y
    torch.cuda.empty_cache()
    return res


def tp2_shares(torch, mx, synth, dev, steps=10, warmup=3):
    """One GPU's share of a two-way tensor-parallel split, at its real shape:
    column-parallel halves of N (the q|k|v projection 75348x5120x7680 and the
    FFN up-projection 75348x5120x6912 with GELU) and row-parallel halves of K
    (attention out 75348x2560x5120 and FFN down 75348x6912x5120, bf16 partial
    sums without the bias, which the all-reduce's owner would add). Each
    share quantizes its own activations (rank-local) and runs the slab GEMM.
    The exchange itself (an all-reduce of the row-parallel partials over
    xGMI) is not measured: one GPU."""
    M = 75348
    shares = [("qkv column half", M, 5120, 7680, False, True), ("ffn up column half", M, 5120, 6912, True, True),
              ("attn out row half", M, 2560, 5120, False, False), ("ffn down row half", M, 6912, 5120, False, False)]
    res = {}
    for i, (name, m, k, n, gelu, has_bias) in enumerate(shares):
        x = synth.make_activation_device(m, k, 700 + i, dev)
        w = mx.mx_quantize_weight_slab(synth.make_weight_device(n, k, 700 + i, dev))
        b = synth.make_bias(n, 700 + i).to(dev) if has_bias else None
        xs = mx.mx_quantize_act_slab(x)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        total, (q_ms, g_ms) = timed_step(
            torch, [lambda: mx.mx_quantize_act_slab(x, xs), lambda: mx.mx_linear_slab(xs, w, b, gelu=gelu, y=y)],
            steps, warmup)
        ms = total / steps
        flop = 2.0 * m * n * k
        res[name] = {"shape": f"{m}x{k}x{n}" + (" gelu" if gelu else "") + ("" if has_bias else " no bias"),
                     "ms": round(ms, 4), "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
                     "gemm_TFLOPs": round(flop / (mean(g_ms) * 1e-3) / 1e12, 2)}
        del x, w, xs, y
        torch.cuda.empty_cache()
    return res


def main():
    args = parse_args()
    if args.gpus != 1:
        print(
            f"bench.py measures one GPU only (got --gpus {args.gpus}); the linear shards over tokens with no "
            "exchange, so several GPUs are not measured here.",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import mxfp8_w8a8_quantized_amd as mx
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.profile_copy:
        n = 1 << 30
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5,
                          "copy_GBps": device_copy_gbps(torch, dev, 3, 1)}))
        return

    if not os.path.exists(mx.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()

    shape = synth.CONFIGS[WORKLOAD][0]
    if args.profile in ("single", "ffn", "xattn"):
        profile_config(torch, mx, synth, dev, args.profile, args.steps, args.warmup)
        return
    if args.profile == "workloads":
        res = {
            "other_workloads": other_workloads(torch, mx, synth, dev, steps=2, warmup=1),
            "per_channel_fp8": per_channel_step(torch, mx, synth, dev, shape.M, shape.K, shape.N, steps=2, warmup=1),
            "denoise_step": denoise_step(torch, synth, dev, steps=1, warmup=1),
        }
        print(json.dumps({"profiled": "workloads", "results": res}), flush=True)
        return

    M, K, N = shape.M, shape.K, shape.N
    x_cpu = synth.make_activation(M, K, seed=0)
    w_cpu = synth.make_weight(N, K, seed=0)
    b_cpu = synth.make_bias(N, seed=0)
    x = x_cpu.to(dev)
    w = w_cpu.to(dev)
    bias = b_cpu.to(dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    # Weights are stored quantized: quantize once, outside the step.
    wsl = mx.mx_quantize_weight_slab(w)
    _, wq_per = timed_step(torch, [lambda: mx.mx_quantize_weight_slab(w, wsl)], 3, 1)
    xsl = mx.mx_quantize_act_slab(x)

    quant = lambda: mx.mx_quantize_act_slab(x, xsl)  # noqa: E731
    gemm = lambda: mx.mx_linear_slab(xsl, wsl, bias, y=y)  # noqa: E731

    rowmajor = None
    if args.profile in ("rowmajor", "fused") or (not args.profile and not args.no_extra):
        wq, ws = mx.mx_quantize_weight(w)
        xq, xs = mx.mx_quantize_act(x)
        rowmajor = [lambda: mx.mx_quantize_act(x, xq, xs), lambda: mx.mx_linear_q(xq, xs, wq, ws, bias, y=y)]
        fused = lambda: mx.mx_linear_fused(x, wq, ws, bias, y=y)  # noqa: E731
    del w

    if args.profile:
        fns = {"step": [quant, gemm], "quant": [quant], "rowmajor": rowmajor,
               "fused": [fused] if rowmajor else None}[args.profile]
        timed_step(torch, fns, args.steps, args.warmup)
        print(json.dumps({"profiled": args.profile, "steps": args.steps}), flush=True)
        return

    total_ms, (q_ms, g_ms) = timed_step(torch, [quant, gemm], args.steps, args.warmup)
    flop = 2.0 * M * N * K
    ms_per_step = total_ms / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    gemm_ms = mean(g_ms)
    achieved = flop / (gemm_ms * 1e-3) / 1e12

    probe = mfma_probe(torch, mx, dev, xsl.q, wsl.q)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("hbm_bytes_per_launch")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD,
            "M": M,
            "K": K,
            "N": N,
            "step": "mx_quantize_act_slab + mx_linear_slab (bias, bf16 out): the two kernels mx_linear runs for "
                    "this shape (its slab plan), timed one by one",
            "pct_of_mxfp8_peak": round(100.0 * value / PEAK_MXFP8_TFLOPS, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_MXFP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MXFP8_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "linear_slab_kernel (block-scaled GEMM)",
            "launch_ms": round(gemm_ms, 4),
            "mfma_probe_TFLOPs": probe,
            "frac_of_probe": round(achieved / probe["workload_codes"], 4),
            "kernel_source_hash": kernel_source_hash(),
        },
    }

    if not args.no_extra:
        qa = mean(q_ms)
        act_bytes = M * K * (2 + 1 + 1 / 32)
        w_bytes = N * K * (4 + 1 + 1 / 32)
        wqa = mean(wq_per[0])
        ws_buf = torch.empty((mx.mx_linear_ws_bytes(M, K, N),), dtype=torch.uint8, device=dev)
        one_call = lambda: mx.mx_linear(x, wsl, bias, y=y, workspace=ws_buf)  # noqa: E731
        oc_total, _ = timed_step(torch, [one_call], 30, 5)
        del ws_buf
        rm_total, (rq_ms, rg_ms) = timed_step(torch, rowmajor, 10, 2)
        _, (f_ms,) = timed_step(torch, [fused], 10, 2)
        fa = mean(f_ms)
        cold = cold_steps(torch, dev, [quant, gemm], 10)
        copy_gbps = device_copy_gbps(torch, dev)
        out["extra"] = {
            "quantize_act_ms": round(qa, 4),
            "quantize_act_GBps": round(act_bytes / (qa * 1e-3) / 1e9, 1),
            "quantize_act_hbm_frac": round(act_bytes / (qa * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "device_copy_GBps": copy_gbps,
            "quantize_act_copy_frac": round(act_bytes / (qa * 1e-3) / 1e9 / copy_gbps, 4),
            "gemm_ms": round(gemm_ms, 4),
            "gemm_ms_p10_p50_p90": percentiles(g_ms),
            "step_ms_p10_p50_p90": percentiles([a + b for a, b in zip(q_ms, g_ms)]),
            "cold": cold,
            "mx_linear_one_call_ms": round(oc_total / 30, 4),
            "rowmajor_step_ms": round(rm_total / 10, 4),
            "rowmajor_step_TFLOPs": round(flop / (rm_total / 10 * 1e-3) / 1e12, 2),
            "rowmajor_gemm_ms": round(mean(rg_ms), 4),
            "fused_prologue_ms": round(fa, 4),
            "fused_prologue_TFLOPs": round(flop / (fa * 1e-3) / 1e12, 2),
            "quantize_weight_f32_ms": round(wqa, 4),
            "quantize_weight_GBps": round(w_bytes / (wqa * 1e-3) / 1e9, 1),
        }

    if not args.no_extra:
        del y
        out["extra"]["context_from_pages"] = CONTEXT
        out["extra"]["other_workloads"] = other_workloads(torch, mx, synth, dev)
        out["extra"]["denoise_step"] = denoise_step(torch, synth, dev)
        out["extra"]["per_channel_fp8"] = per_channel_step(torch, mx, synth, dev, M, K, N)
        out["extra"]["tp2_shares"] = tp2_shares(torch, mx, synth, dev)

    if not args.no_cpu_baseline:
        del x, xsl, rowmajor
        out["cpu_baseline"] = cpu_baseline(x_cpu, w_cpu, b_cpu, CPU_SAMPLE_ROWS)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
