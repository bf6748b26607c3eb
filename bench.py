"""Benchmark: block-scaled GEMM TFLOP/s at FLUX DiT shapes on one MI355X.

One step = one pass of the hot path over one batch: selective dispatch,
dynamic MXFP8 quantization of the bf16 activations and the block-scaled GEMM
with its bf16 epilogue, i.e. one ``mxq_quant_gemm_fused`` call on the FLUX-dev
MLP up-projection at 1024x1024 (M = 4608 tokens, K = 3072, N = 12288).
Weights are quantized once before timing.  Inputs rotate through several
resident copies so the working set exceeds the 256 MB Infinity Cache; the
same loops with one copy are reported under "hot".  The metric's second
format is timed the same way on the FLUX single-stream linears in MXFP4
(4608 x 3072 -> 21504 and 4608 x 15360 -> 3072) under "mxfp4".

Timing: every loop is exactly K calls between one pair of HIP events on the
launch stream, after at least W warm-up calls and at least 1.5 s of warm GPU
time; per-call p10 / median / p90 come from a separate pass.  The roofline
figure is the GEMM-only loop; its HBM traffic, clock and MFMA-busy fraction
come from the committed rocprofv3 counter summary of the same kernel, when
that summary was taken on the current GEMM sources.  Quantizer figures are
GPU time per call over consecutive calls replayed from one HIP graph: an
eager loop of ~10 us kernels measures the Python binding's launch overhead
instead (reported beside it as "eager_ms").  ``--no-hot`` drops the
hot-cache loops (for counter runs).

Prints ONE JSON line.  ``--all`` adds the other FLUX-shaped workloads
(MXFP6, NVFP4 at 2048x2048, one double-stream block with selective bf16
fallback) under "extra", and the widened paths: producer-fused quantization
("producer_fused"), a block's linears eager vs HIP-graphed
("block_sequences"), block-scaled FP8 attention at the FLUX shape beside
torch's bf16 attention ("attention"), the single-stream block's concatenated
linear2 input built by the producers' epilogues ("single_block_concat") and
the quantizer under both shared-scale rules ("scale_rules").
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-scaled GEMM TFLOP/s at FLUX DiT shapes (MXFP8/MXFP4); % of MFMA peak"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"mxfp8": 5000.0, "mxfp4": 10100.0, "mxfp6_e2m3": 10100.0, "mxfp6_e3m2": 10100.0, "nvfp4": 2500.0,
               "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "microscaling_quantized_diffusion_amd", "csrc")
GEMM_SRCS = [os.path.join(CSRC, f) for f in ("gemm.hip", "gemm_mx.hip", "gemm_mx_kernel.h", "gemm_mx_requant.hip", "gemm_tile.h")]
# counter summary of the headline GEMM kernel (HBM traffic, clock and MFMA busy from rocprofv3 --pmc runs)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "mxe_gemm_mxfp8_flux_mlp_up_counters.txt")


def _src_sha() -> str:
    """Hash of the GEMM sources' code: every line with its // comment and surrounding blanks removed, blank lines
    skipped, so that comment edits keep a counter summary valid while any code change invalidates it."""
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def _profile_values(path=COUNTERS_FILE):
    """key: value pairs of a committed counter summary, if it was taken on the current GEMM sources."""
    if not os.path.exists(path):
        return {}
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("gemm_source_sha256_16") != _src_sha():
        return {}
    return vals


def _float_or_none(v):
    try:
        return float(v)
    except (TypeError, ValueError):
        return None


def _upload(bits, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


WARM_MS = 1500.0  # minimum GPU time of warm-up before any timed loop


def _time_loop(fn, iters, warmup, dist=None, warm_ms=None):
    """Average milliseconds per call over exactly `iters` calls, timed with one pair of HIP events on torch's
    current stream (the stream the library launches on) around the whole loop.

    Before it: `warmup` calls, continued until at least `warm_ms` of GPU time has passed since the first,
    because the first ~150 calls after an idle period run slower while clocks and power settle.  With `dist`,
    a separate pass of `iters` calls with an event after each fills dist with the p10 / median / p90 of the
    per-call times (per-call events perturb the average, so they stay out of the timed loop)."""
    import torch

    warm_ms = WARM_MS if warm_ms is None else warm_ms
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    done = 0
    while True:
        batch = max(1, warmup - done) if done < warmup else max(1, min(50, done))
        for _ in range(batch):
            fn(done)
            done += 1
        e1.record()
        e1.synchronize()
        if done >= warmup and e0.elapsed_time(e1) >= warm_ms:
            break
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / iters
    if dist is not None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record()
        for i in range(iters):
            fn(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])
        dist.update(p10=float(np.percentile(per, 10)), p50=float(np.percentile(per, 50)),
                    p90=float(np.percentile(per, 90)), warmup_calls=done)
    return ms


def _time_graph(fn, calls, reps=4, warm_ms=None):
    """Milliseconds per call of `calls` consecutive calls fn(0) .. fn(calls - 1) captured in one HIP graph.  The
    graph is replayed until `warm_ms` of GPU time has passed, then `reps` replays are timed with one event pair.
    This is the GPU time per call when the host does not pace the launches: for kernels of ~10 us the eager
    loop measures the Python binding's per-call overhead instead."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    warm_ms = WARM_MS if warm_ms is None else warm_ms
    state = {"i": 0}

    def body():
        for i in range(calls):
            fn(i)

    g = mxq.GraphedCall(body)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    while True:
        g()
        state["i"] += 1
        e1.record()
        e1.synchronize()
        if e0.elapsed_time(e1) >= warm_ms:
            break
    e0.record()
    for _ in range(reps):
        g()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / (reps * calls)


def run_layer(layer, dev, steps, warmup, rotate, seed=0):
    """Time fused / GEMM-only / quantize-only for one linear, as the library is called in production: weights
    pre-quantized once (MX scales in the packed layout), activations quantized per call.  Returns a dict."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    a_bits, w_bits = __import__("microscaling_quantized_diffusion_amd.inputs", fromlist=["x"]).make_layer_inputs(
        layer, seed=seed)
    M, K, N = layer.M, layer.K, layer.N
    flops = 2.0 * M * N * K
    quantized = mxq.should_quantize(M, K, N)
    a0 = _upload(a_bits, dev)
    w0 = _upload(w_bits, dev)
    As = [a0] + [a0.clone() for _ in range(rotate - 1)]
    res = {"layer": layer.name, "M": M, "K": K, "N": N, "gflop": flops / 1e9}
    if not quantized:
        Ws = [w0] + [w0.clone() for _ in range(rotate - 1)]
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ms = _time_loop(lambda i: mxq.gemm_bf16(As[i % rotate], Ws[i % rotate], None, out), steps, warmup)
        w_bytes = N * K * 2
        res.update(path="bf16", ms=ms, tflops=flops / ms / 1e9,
                   gbs=(w_bytes + M * K * 2 + M * N * 2) / ms / 1e6)
        return res
    fmt = layer.fmt
    # MX weights are pre-quantized with packed scales (whole-line scale fetches in the GEMM); the fused
    # call then writes the activation scales packed as well
    pk = fmt != "nvfp4"
    qw0 = mxq.quantize(fmt, w0, packed_scales=pk)
    Ws = [qw0] + [mxq.QTensor(fmt, qw0.codes.clone(), qw0.scales.clone(),
                              None if qw0.tensor_scale is None else qw0.tensor_scale.clone(), K, pk)
                  for _ in range(rotate - 1)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mxq.workspace_bytes(fmt, M, K, True), dtype=torch.uint8, device=dev)
    dist_fused, dist_gemm = {}, {}
    ms_fused = _time_loop(lambda i: mxq.quant_gemm_fused(As[i % rotate], Ws[i % rotate], None, out, ws), steps, warmup,
                          dist_fused)
    qa = [mxq.quantize(fmt, a, packed_scales=pk) for a in As]
    ms_gemm = _time_loop(lambda i: mxq.gemm(qa[i % rotate], Ws[i % rotate], None, out), steps, warmup, dist_gemm)
    qws = torch.empty(max(1, mxq.workspace_bytes(fmt, M, K, False)), dtype=torch.uint8, device=dev)
    ms_quant_eager = _time_loop(lambda i: mxq.quantize(fmt, As[i % rotate], qa[i % rotate], qws), steps, warmup)
    ms_quant = _time_graph(lambda i: mxq.quantize(fmt, As[i % rotate], qa[i % rotate], qws), 8 * rotate)
    # bytes the quantizer writes: MXFP6 stores each 24-byte block in a 32-byte slot
    code_b = M * K * (1.0 if fmt == "mxfp8" or fmt.startswith("mxfp6") else 0.5)
    scale_b = M * K / (16 if fmt == "nvfp4" else 32)
    quant_bytes = M * K * 2 + code_b + scale_b
    res.update(path=fmt, ms=ms_fused, ms_p10=dist_fused["p10"], ms_p50=dist_fused["p50"], ms_p90=dist_fused["p90"],
               warmup_calls=dist_fused["warmup_calls"],
               gemm_ms_p10=dist_gemm["p10"], gemm_ms_p50=dist_gemm["p50"], gemm_ms_p90=dist_gemm["p90"],
               tflops=flops / ms_fused / 1e9, gemm_ms=ms_gemm,
               gemm_tflops=flops / ms_gemm / 1e9, quant_ms=ms_quant, quant_gbs=quant_bytes / ms_quant / 1e6,
               quant_eager_ms=ms_quant_eager,
               pct_peak_fused=100.0 * flops / ms_fused / 1e9 / PEAK_TFLOPS[fmt],
               pct_peak_gemm=100.0 * flops / ms_gemm / 1e9 / PEAK_TFLOPS[fmt])
    del As, Ws, qa, out, ws, qws
    torch.cuda.empty_cache()
    return res


def run_sequence(workload, dev, steps, warmup):
    """One DiT block's linears back to back (selective rule included): eager calls vs one HIP-graph replay."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq
    from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, make_layer_inputs

    layers, inputs = [], []
    for i, ly in enumerate(WORKLOADS[workload].layers):
        a_bits, w_bits = make_layer_inputs(ly, seed=i)
        layers.append(mxq.QuantLinear.from_weight(ly.fmt, _upload(w_bits, dev)))
        inputs.append(_upload(a_bits, dev))
    seq = mxq.LinearSequence(layers, inputs)
    ms_eager = _time_loop(lambda i: seq(), steps, warmup)
    graphed = mxq.GraphedCall(seq)
    ms_graph = _time_loop(lambda i: graphed(), steps, warmup)
    flops = sum(2.0 * ly.M * ly.N * ly.K for ly in WORKLOADS[workload].layers)
    res = {"workload": workload, "sequence": [ly.name for ly in WORKLOADS[workload].layers],
           "ms_eager": ms_eager, "ms_graph": ms_graph, "tflops_eager": flops / ms_eager / 1e9,
           "tflops_graph": flops / ms_graph / 1e9}
    del seq, graphed, layers, inputs
    torch.cuda.empty_cache()
    return res


def run_producer_fused(dev, steps, warmup, rotate):
    """FLUX MLP at 1024x1024 (4608 tokens, 3072 -> 12288 -> 3072, MXFP8): the up-projection's output
    quantized for the down-projection by a separate quantizer pass vs inside the GEMM epilogue."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq
    from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, make_layer_inputs

    up = WORKLOADS["flux_mlp_up_mxfp8"].layers[0]
    M, D, H = up.M, up.K, up.N
    a_bits, w_bits = make_layer_inputs(up, seed=0)
    _, wd_bits = make_layer_inputs(up, seed=1, N=D, K=H)
    xs = [_upload(a_bits, dev)] + [None] * (rotate - 1)
    for i in range(1, rotate):
        xs[i] = xs[0].clone()
    qxs = [mxq.quantize("mxfp8", x) for x in xs]
    w_up = mxq.quantize("mxfp8", _upload(w_bits, dev))
    w_dn = mxq.quantize("mxfp8", _upload(wd_bits, dev))
    h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    qh = mxq.QTensor("mxfp8", torch.empty((M, H), dtype=torch.uint8, device=dev),
                     torch.empty((M, H // 32), dtype=torch.uint8, device=dev), None, H)
    y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    up_sep = _time_loop(lambda i: (mxq.gemm(qxs[i % rotate], w_up, None, h), mxq.quantize("mxfp8", h, qh)), steps,
                        warmup)
    up_fused = _time_loop(lambda i: mxq.gemm_requant(qxs[i % rotate], w_up, "mxfp8", None, "none", qh), steps,
                          warmup)
    up_fused_gelu = _time_loop(lambda i: mxq.gemm_requant(qxs[i % rotate], w_up, "mxfp8", None, "gelu_tanh", qh),
                               steps, warmup)
    chain_sep = _time_loop(lambda i: (mxq.gemm(qxs[i % rotate], w_up, None, h), mxq.quantize("mxfp8", h, qh),
                                      mxq.gemm(qh, w_dn, None, y)), steps, warmup)
    chain_fused = _time_loop(lambda i: (mxq.gemm_requant(qxs[i % rotate], w_up, "mxfp8", None, "none", qh),
                                        mxq.gemm(qh, w_dn, None, y)), steps, warmup)
    chain_fused_gelu = _time_loop(lambda i: (mxq.gemm_requant(qxs[i % rotate], w_up, "mxfp8", None, "gelu_tanh", qh),
                                             mxq.gemm(qh, w_dn, None, y)), steps, warmup)
    del xs, qxs, w_up, w_dn, h, qh, y
    torch.cuda.empty_cache()
    # the separate-quantizer rows carry no activation (there is no standalone GELU kernel), so they compare
    # with the fused rows without one; the *_gelu rows show what the fused activation adds
    return {"shape": f"{M}x{D} -> {H} -> {D}", "up_gemm_then_quantize_ms": up_sep, "up_requant_gemm_ms": up_fused,
            "up_requant_gemm_gelu_ms": up_fused_gelu, "mlp_chain_separate_quantizer_ms": chain_sep,
            "mlp_chain_producer_fused_ms": chain_fused, "mlp_chain_producer_fused_gelu_ms": chain_fused_gelu}


def run_attention(dev, steps, warmup, B=1, H=24, S=4608, D=128):
    """Block-scaled FP8 attention at the FLUX-dev 1024 x 1024 shape (24 heads, 4608 tokens = 4096 image +
    512 text, head dimension 128), one mxq_attention_fp8 call per step (Q, K, V quantization included);
    torch's bf16 scaled_dot_product_attention on the same inputs is timed beside it as context."""
    import torch
    import torch.nn.functional as F

    from microscaling_quantized_diffusion_amd import mxq

    g = torch.Generator(device=dev).manual_seed(0)
    q, k, v = (torch.randn((B, H, S, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    out = torch.empty_like(q)
    ws = torch.empty(mxq.attention_workspace_bytes(B, H, S, D), dtype=torch.uint8, device=dev)
    flops = 4.0 * B * H * S * S * D
    dist = {}
    ms = _time_loop(lambda i: mxq.attention_fp8(q, k, v, out, ws), steps, warmup, dist)
    ms_sdpa = _time_loop(lambda i: F.scaled_dot_product_attention(q, k, v), steps, warmup)
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return {"shape": f"B={B} H={H} S={S} D={D}", "ms": ms, "ms_p10_p50_p90": [dist["p10"], dist["p50"], dist["p90"]],
            "tflops": flops / ms / 1e9, "frac_of_fp8_mfma_peak": flops / ms / 1e9 / PEAK_TFLOPS["mxfp8"],
            "sdpa_bf16_ms": ms_sdpa, "sdpa_bf16_tflops": flops / ms_sdpa / 1e9, "speedup_vs_sdpa_bf16": ms_sdpa / ms}


def run_single_block_concat(dev, steps, warmup, H=24, S=4608, F=12288):
    """FLUX single-stream block at 1024 x 1024, MXFP4: the input of linear2 is [attention output (3072) |
    GELU of linear1's MLP part (12288)] for 4608 tokens.  Unfused: bf16 attention, the bf16 MLP GEMM and the
    standalone quantizer over the concatenation (the bf16 concatenation itself counted as free).  Fused:
    the attention and the MLP GEMM emit their MXFP4 codes straight into the concatenated matrix."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    D = H * 128
    g = torch.Generator(device=dev).manual_seed(0)
    q, k, v = (torch.randn((1, H, S, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    x = mxq.quantize("mxfp4", torch.randn((S, D), generator=g, device=dev).to(torch.bfloat16))
    w = mxq.quantize("mxfp4", (torch.randn((F, D), generator=g, device=dev) * 0.02).to(torch.bfloat16))
    ws = torch.empty(mxq.attention_workspace_bytes(1, H, S, 128), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    h = torch.empty((S, F), dtype=torch.bfloat16, device=dev)
    cat_bf16 = torch.zeros((S, D + F), dtype=torch.bfloat16, device=dev)
    cat = mxq.quantize("mxfp4", cat_bf16)
    att_part = mxq.QTensor("mxfp4", cat.codes[:, :D // 2], cat.scales[:, :D // 32], None, D)
    mlp_part = mxq.QTensor("mxfp4", cat.codes[:, D // 2:], cat.scales[:, D // 32:], None, F)
    t_att = _time_loop(lambda i: mxq.attention_fp8(q, k, v, o, ws), steps, warmup)
    t_mlp = _time_loop(lambda i: mxq.gemm(x, w, None, h), steps, warmup)
    t_quant = _time_loop(lambda i: mxq.quantize("mxfp4", cat_bf16, cat), steps, warmup)
    t_att_rq = _time_loop(lambda i: mxq.attention_fp8_requant(q, k, v, "mxfp4", att_part, ws), steps, warmup)
    t_mlp_rq = _time_loop(lambda i: mxq.gemm_requant(x, w, "mxfp4", None, "gelu_tanh", mlp_part), steps, warmup)
    unfused = _time_loop(lambda i: (mxq.attention_fp8(q, k, v, o, ws), mxq.gemm(x, w, None, h),
                                    mxq.quantize("mxfp4", cat_bf16, cat)), steps, warmup)
    fused = _time_loop(lambda i: (mxq.attention_fp8_requant(q, k, v, "mxfp4", att_part, ws),
                                  mxq.gemm_requant(x, w, "mxfp4", None, "gelu_tanh", mlp_part)), steps, warmup)
    del q, k, v, x, w, ws, o, h, cat_bf16, cat
    torch.cuda.empty_cache()
    return {"shape": f"{S} tokens, [{D} | {F}] -> MXFP4", "attention_bf16_ms": t_att, "mlp_gemm_bf16_ms": t_mlp,
            "concat_quantizer_ms": t_quant, "attention_requant_ms": t_att_rq, "mlp_gemm_gelu_requant_ms": t_mlp_rq,
            "unfused_ms": unfused, "producer_fused_ms": fused}


def run_scale_rules(dev, steps, warmup, rotate):
    """The MXFP8 quantizer on the FLUX MLP activation (4608 x 3072) with the OCP floor rule and the
    round-up rule."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq
    from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, make_layer_inputs

    layer = WORKLOADS["flux_mlp_up_mxfp8"].layers[0]
    a_bits, _ = make_layer_inputs(layer, seed=0)
    xs = [_upload(a_bits, dev)]
    xs += [xs[0].clone() for _ in range(rotate - 1)]
    qs = [mxq.quantize("mxfp8", x) for x in xs]
    res = {"shape": f"{layer.M}x{layer.K}"}
    nbytes = layer.M * layer.K * (2 + 1 + 1 / 32)
    for rule in ("floor", "rceil"):
        ms = _time_graph(lambda i: mxq.quantize("mxfp8", xs[i % rotate], qs[i % rotate], scale_rule=rule),
                         8 * rotate)
        res[f"{rule}_ms"] = ms
        res[f"{rule}_GB/s"] = nbytes / ms / 1e6
    del xs, qs
    torch.cuda.empty_cache()
    return res


def cpu_baseline(layer, sample_rows):
    """Time the CPU oracle (quantize A, dequantize both operands, fp64 GEMM) on the first `sample_rows`
    activation rows of the workload (all of them by default: about 10 s on 16 host cores)."""
    import oracle
    from microscaling_quantized_diffusion_amd.inputs import make_layer_inputs

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    a_bits, w_bits = make_layer_inputs(layer, seed=0)
    sample_rows = max(1, min(sample_rows, layer.M))
    a_s = np.ascontiguousarray(a_bits[:sample_rows])
    scheme = oracle.MXFP8 if layer.fmt == "mxfp8" else oracle.MXFP4
    t0 = time.perf_counter()
    ac, asc = oracle.quantize_mx(a_s, scheme)
    wc, wsc = oracle.quantize_mx(w_bits, scheme)
    ref = oracle.gemm_mx_ref(ac, asc, wc, wsc, scheme)
    dt = time.perf_counter() - t0
    flops = 2.0 * sample_rows * layer.N * layer.K
    del ref
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads,
        "kind": "oracle",
        "sample": (f"{sample_rows} of {layer.M} activation rows: oracle MX quantization of those rows and of all "
                   f"{layer.N}x{layer.K} weights, fp64 dequantized GEMM; {dt:.1f} s; os.cpu_count()={os.cpu_count()}, "
                   f"affinity={len(os.sched_getaffinity(0))}"),
    }


def main():
    global WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Every timed loop is preceded by at least --warmup calls and at least WARM_MS of GPU time (after an idle
    # period the first ~150 calls run 5-30 % slower while clocks and power settle).
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=8, help="resident input copies cycled through (cold L2/MALL)")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="minimum warm GPU time before each timed loop (counter runs pass 0: every dispatch is "
                         "then serialized and profiled)")
    ap.add_argument("--workload", default="flux_mlp_up_mxfp8")
    ap.add_argument("--all", action="store_true", help="also time the other FLUX-shaped workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the hot-cache timing (profiling runs: every GEMM dispatch is then one of the cold "
                         "timed loops)")
    ap.add_argument("--cpu-rows", type=int, default=4608, help="activation rows the CPU oracle runs (capped at M)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run three plain device-to-device copies of MIB MiB (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    WARM_MS = args.warm_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path runs on a single "
              "MI355X: tokens split across GPUs with no exchange, so one GPU's rate times N bounds the job)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from microscaling_quantized_diffusion_amd import mxq
    from microscaling_quantized_diffusion_amd.inputs import WORKLOADS

    mxq.lib()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    layer = WORKLOADS[args.workload].layers[0]
    print(f"# timing {args.workload} {layer.M}x{layer.K}x{layer.N} {layer.fmt}", file=sys.stderr, flush=True)
    r = run_layer(layer, dev, args.steps, args.warmup, args.rotate)

    flops = 2.0 * layer.M * layer.N * layer.K
    gemm_s = r["gemm_ms"] / 1e3
    prof = _profile_values()
    elem = {"mxfp8": "E4M3", "mxfp4": "E2M1"}.get(layer.fmt, layer.fmt)
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls_done": r["warmup_calls"],
        "ms_per_step": round(r["ms"], 5),
        "ms_per_step_p10_p50_p90": [round(r["ms_p10"], 5), round(r["ms_p50"], 5), round(r["ms_p90"], 5)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if layer.fmt == "mxfp8" else ("fp4_e2m1" if layer.fmt == "mxfp4" else "f16"),
        "data": "synthetic",
        "config": {"workload": args.workload, "M": layer.M, "K": layer.K, "N": layer.N, "format": layer.fmt,
                   "step": "mxq_quant_gemm_fused (dynamic activation quantization + block-scaled GEMM)",
                   "weights": "pre-quantized before timing (packed scale layout)", "rotating_copies": args.rotate},
        "pct_of_mfma_peak": round(r["pct_peak_fused"], 2),
        "roofline": {
            "bound": "mfma",
            "kernel": f"mxe_gemm_kernel<{elem}> (GEMM-only calls, one event pair around the timed loop)",
            "achieved": round(flops / gemm_s / 1e12, 2),
            "peak": PEAK_TFLOPS[layer.fmt],
            "unit": "TFLOP/s",
            "frac": round(flops / gemm_s / 1e12 / PEAK_TFLOPS[layer.fmt], 4),
            "traffic": _float_or_none(prof.get("hbm_bytes_per_launch")),
            "algorithmic_bytes": layer.M * layer.K + layer.N * layer.K + (layer.M + layer.N) * layer.K // 32
            + layer.M * layer.N * 2,
            "gemm_ms": round(r["gemm_ms"], 5),
            "gemm_ms_p10_p50_p90": [round(r["gemm_ms_p10"], 5), round(r["gemm_ms_p50"], 5),
                                    round(r["gemm_ms_p90"], 5)],
            "counters": ({k: _float_or_none(prof.get(k)) for k in ("clock_GHz", "mfma_busy_frac",
                                                                   "kernel_us_in_counter_run")}
                         | {"source": os.path.relpath(COUNTERS_FILE, ROOT)}) if prof else None,
        },
        "quantizer": {"ms": round(r["quant_ms"], 5), "GB/s": round(r["quant_gbs"], 1),
                      "frac_of_hbm": round(r["quant_gbs"] / PEAK_HBM_GBS, 4),
                      "timing": "GPU time per call over consecutive calls replayed from one HIP graph",
                      "eager_ms": round(r["quant_eager_ms"], 5)},
    }
    # the metric's second format: the FLUX single-stream linears in MXFP4 (config 3), same calls and timing
    line["mxfp4"] = []
    for i, ly in enumerate(WORKLOADS["flux_single_mxfp4"].layers):
        print(f"# timing flux_single_mxfp4/{ly.name} {ly.M}x{ly.K}x{ly.N}", file=sys.stderr, flush=True)
        e = run_layer(ly, dev, args.steps, args.warmup, min(args.rotate, 4), seed=i)
        line["mxfp4"].append({
            "layer": ly.name, "M": ly.M, "K": ly.K, "N": ly.N, "rotating_copies": min(args.rotate, 4),
            "fused_ms": round(e["ms"], 5), "fused_tflops": round(e["tflops"], 2),
            "gemm_ms": round(e["gemm_ms"], 5), "gemm_tflops": round(e["gemm_tflops"], 2),
            "gemm_frac_of_fp4_peak": round(e["gemm_tflops"] / PEAK_TFLOPS["mxfp4"], 4),
            "fused_frac_of_fp4_peak": round(e["tflops"] / PEAK_TFLOPS["mxfp4"], 4),
            "quant_ms": round(e["quant_ms"], 5), "quant_GB/s": round(e["quant_gbs"], 1)})
    if not args.no_hot:
        # the same loops with one resident input copy (weights and activations stay in L2 / MALL)
        print("# timing the hot-cache case (one input copy)", file=sys.stderr, flush=True)
        h = run_layer(layer, dev, args.steps, args.warmup, 1)
        line["hot"] = {"rotating_copies": 1, "ms_per_step": round(h["ms"], 5), "tflops": round(h["tflops"], 2),
                       "gemm_ms": round(h["gemm_ms"], 5), "gemm_tflops": round(h["gemm_tflops"], 2),
                       "quant_ms": round(h["quant_ms"], 5), "quant_GB/s": round(h["quant_gbs"], 1)}
    if args.all:
        leg_steps, leg_warm = max(10, args.steps // 2), max(3, args.warmup // 2)
        extra = []
        for name in ("flux_mlp_up_mxfp6", "flux_2048_nvfp4", "flux_double_block_b1", "flux_double_block_b4"):
            for i, ly in enumerate(WORKLOADS[name].layers):
                print(f"# timing {name}/{ly.name}", file=sys.stderr, flush=True)
                e = run_layer(ly, dev, leg_steps, leg_warm, min(args.rotate, 4), seed=i)
                e["workload"] = name
                extra.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in e.items()})
        line["extra"] = extra
        print("# timing producer-fused quantization on the FLUX MLP", file=sys.stderr, flush=True)
        pf = run_producer_fused(dev, leg_steps, leg_warm, min(args.rotate, 4))
        line["producer_fused"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in pf.items()}
        line["block_sequences"] = []
        for name in ("flux_double_block_b1", "flux_double_block_b4"):
            print(f"# timing the {name} linear sequence, eager and graphed", file=sys.stderr, flush=True)
            e = run_sequence(name, dev, leg_steps, leg_warm)
            line["block_sequences"].append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in e.items()})
        print("# timing FP8 attention at the FLUX shape", file=sys.stderr, flush=True)
        at = run_attention(dev, leg_steps, leg_warm)
        line["attention"] = {k: (round(v, 4) if isinstance(v, float) else
                                 [round(x, 4) for x in v] if isinstance(v, list) else v) for k, v in at.items()}
        print("# timing the single-stream block's concatenated linear2 input", file=sys.stderr, flush=True)
        sb = run_single_block_concat(dev, leg_steps, leg_warm)
        line["single_block_concat"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in sb.items()}
        print("# timing the MXFP8 quantizer with both scale rules", file=sys.stderr, flush=True)
        sr = run_scale_rules(dev, leg_steps, leg_warm, min(args.rotate, 4))
        line["scale_rules"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in sr.items()}
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copied {n} bytes three times", file=sys.stderr, flush=True)
        del src, dst
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(layer, args.cpu_rows)
        line["cpu_baseline"]["value"] = round(line["cpu_baseline"]["value"], 6)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
