#!/usr/bin/env python3
"""Benchmark of the KDA token-mixer hot path on one MI355X (gfx950).

A step is one KDA prefill of one layer over the single-sequence workload
(B=1, T=4096, H=64, dk=dv=128, bfloat16 q/k/v/g/beta, float32 state in and
out, float32 output, 64-token chunks): ``value`` is tokens per second for that
layer. The same run also times the batched decode step (B=256 sequences x 64
heads, 1 GiB float32 state updated in place) and reports its state bandwidth,
the decode-time convolution update, the packed variable-length prefill (8
sequences, ~135K tokens), the prefill with caches flushed before each call, and
(unless --skip-layer) the whole token-mixer layer at T=8192.

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize() on both sides, with HIP events recorded on the stream
the kernels are launched on. The headline prefill figure is the median of K
calls with the caches flushed (512 MiB written, untimed) before each call, each
call bracketed by its own events; the other paths are timed back to back.
Inputs are resident in device memory before the timed region starts. Prints
one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 MFMA, TFLOP/s
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 MFMA, TFLOP/s

# algorithmic bytes per token-layer of the prefill: q,k,v,g bf16 (4 x 64 x 128 x 2)
# + beta (64 x 2) + o float32 (64 x 128 x 4) + state in and out amortised over
# 4096 tokens (2 x 4 MiB / 4096)
PREFILL_BYTES_PER_TOKEN = 4 * 64 * 128 * 2 + 64 * 2 + 64 * 128 * 4 + 2 * 64 * 128 * 128 * 4 // 4096
# algorithmic flops per token-layer (chunk 64, triangles only): 4,468,736 MAC per
# chunk-head -> x2 / 64 tokens x 64 heads
PREFILL_FLOPS_PER_TOKEN = 2 * 4468736 * 64 // 64
# decode step: state read + write (2 x 1 GiB) + q,k,v,g bf16 + beta bf16 + o float32
DECODE_BYTES = 2 * 256 * 64 * 128 * 128 * 4 + 4 * 256 * 64 * 128 * 2 + 256 * 64 * 2 + 256 * 64 * 128 * 4
# conv update: x + state in + state out (shift) + weight + y, bf16
CONV_BYTES = (256 * 8192 + 2 * 256 * 3 * 8192 + 8192 * 4 + 256 * 8192) * 2

COUNTERS = os.path.join(ROOT, "profiles", "kda_prefill_t4096_h64_counters.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("kda_prefill_split.hip", "kda_chunk.h", "kda_device.h", "kda_api.cpp"):
        h.update(open(os.path.join(ROOT, "gated_delta_rule_02_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def dev(t, torch):
    import numpy as np
    if t.bits is not None:
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.vals)).cuda()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def settle(torch, fn, seconds=0.25):
    """Untimed calls for about `seconds` of wall time. The GPU raises its
    clocks only after some milliseconds of sustained load (the first calls
    of a fresh process ran about 13% slower than later ones), so every
    measurement starts from the steady state rather than from the ramp."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def timed(torch, fn, steps, warmup):
    """Average ms per call over `steps` calls after a settling period and
    `warmup` untimed calls."""
    stream = torch.cuda.current_stream()
    settle(torch, fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def graph_ms(torch, fn, n):
    """Per-call ms of `n` calls captured in one HIP graph and replayed: for a
    kernel of a few microseconds, back-to-back launches from the host time the
    dispatch gap as much as the kernel; a graph replays them without it. The
    graph is replayed several times with synchronizations between (an eager
    call first, as a warm-up)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(n):
                fn()
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / n
        best = t if best is None else min(best, t)
    return best


def timed_cold(torch, fn, steps, warmup, flush_bytes=512 << 20):
    """Per-call ms when, before every call, a 512 MiB buffer is written so that
    the 256 MB last-level cache (MALL) and L2 hold none of the call's inputs.
    Each call is bracketed by its own events on the launch stream; the flush
    is not timed. Returns (median, mean, wall seconds of the timed loop)."""
    stream = torch.cuda.current_stream()
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    settle(torch, fn)
    for i in range(warmup):
        buf.fill_(float(i))
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        buf.fill_(float(i))
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = sorted(a.elapsed_time(b) for a, b in ev)
    med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
    return med, sum(t) / len(t), wall


def bench_prefill(torch, K, steps, warmup):
    from gated_delta_rule_02_amd import synth
    d = synth.workload_prefill()
    q, k, v, g, b = (dev(d[x], torch) for x in ("q", "k", "v", "g", "beta"))
    T, H, D = q.shape
    s0 = torch.zeros((1, H, D, D), dtype=torch.float32, device="cuda")
    sT = torch.empty_like(s0)
    o = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    fn = lambda: K.kda_prefill(q, k, v, g, b, o, initial_state=s0, final_state=sT)
    ms_cold, ms_cold_mean, wall = timed_cold(torch, fn, steps, warmup)
    ms, _ = timed(torch, fn, steps, warmup)
    snaps = torch.empty((1, 4, H, D, D), dtype=torch.float32, device="cuda")
    fs = lambda: K.kda_prefill(q, k, v, g, b, o, initial_state=s0, final_state=sT, snapshots=snaps,
                               snapshot_interval=1024)
    ms_snap, _ = timed(torch, fs, max(5, steps // 2), 2)
    return ms, wall, d, (ms_cold, ms_cold_mean), ms_snap


def bench_varlen(torch, K, steps, warmup):
    """The packed variable-length prefill: 8 sequences whose lengths are the
    seeded draw U[1024, 32768] of the varlen parity workload, H=64, bf16
    inputs with that workload's distributions (drawn on the device here: the
    kernels' timing does not depend on the values), random fp32 initial
    states, final states written."""
    import numpy as np
    from gated_delta_rule_02_amd import synth
    lengths = synth.varlen_lengths(np.random.default_rng(1003), 8, 1024, 32768)
    cu = synth.cu_from_lengths(lengths)
    T, H, D = int(cu[-1]), 64, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1003)
    rn = lambda *shape: torch.randn(*shape, device="cuda", generator=gen, dtype=torch.float32)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    q = unit(rn(T, H, D)).to(torch.bfloat16)
    k = unit(rn(T, H, D)).to(torch.bfloat16)
    v = rn(T, H, D).to(torch.bfloat16)
    g = torch.clamp(-torch.nn.functional.softplus(rn(T, H, D)), min=-5.0).to(torch.bfloat16)
    b = torch.sigmoid(rn(T, H)).to(torch.bfloat16)
    s0 = rn(len(lengths), H, D, D) * 0.02
    sT = torch.empty_like(s0)
    o = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    cu_d = torch.from_numpy(cu).cuda()
    cu_h = torch.from_numpy(cu)
    fn = lambda: K.kda_prefill(q, k, v, g, b, o, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=len(lengths),
                               initial_state=s0, final_state=sT)
    ms, _ = timed(torch, fn, max(3, steps // 4), max(1, warmup // 2))
    return ms, T, [int(x) for x in lengths]


def bench_seqpar(torch, K, steps, warmup, P=4):
    """The prefill workload cut into P equal segments and stitched with the
    segment maps (what P ranks of a sequence-parallel prefill would each do
    on their share, here all on one GPU): every segment's map at once, P - 1
    chained map applications, then every segment's outputs at once from its
    incoming state. Also the per-rank share alone: one segment's map and its
    prefill (T / P tokens, 64 heads)."""
    import numpy as np
    from gated_delta_rule_02_amd import synth
    d = synth.workload_prefill()
    q, k, v, g, b = (dev(d[x], torch) for x in ("q", "k", "v", "g", "beta"))
    T, H, D = q.shape
    cuts = np.linspace(0, T, P + 1).astype(np.int32)
    cu_d, cu_h = torch.from_numpy(cuts).cuda(), torch.from_numpy(cuts)
    M = torch.empty((P, H, D, D), dtype=torch.float32, device="cuda")
    Nm = torch.empty_like(M)
    S = torch.zeros_like(M)
    sT = torch.empty_like(M)
    o = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    maps = lambda: K.kda_prefill_segment_maps(k, v, g, b, M, Nm, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=P)

    def chain():
        for i in range(1, P):
            K.kda_affine_apply(M[i - 1], S[i - 1], S[i], N=Nm[i - 1])

    seg = lambda: K.kda_prefill(q, k, v, g, b, o, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=P,
                                initial_state=S, final_state=sT)

    def whole():
        maps()
        chain()
        seg()

    L = T // P
    q1, k1, v1, g1, b1 = (x[:L] for x in (q, k, v, g, b))
    M1, N1, S1, sT1 = M[:1], Nm[:1], S[:1], sT[:1]
    o1 = o[:L]
    rank_maps = lambda: K.kda_prefill_segment_maps(k1, v1, g1, b1, M1, N1)
    rank_seg = lambda: K.kda_prefill(q1, k1, v1, g1, b1, o1, initial_state=S1, final_state=sT1)
    n = max(5, steps // 2)
    return {"workload": "the prefill workload (T=4096, H=64) cut into %d segments of %d tokens" % (P, L),
            "ms_total": timed(torch, whole, n, 2)[0], "ms_segment_maps": timed(torch, maps, n, 2)[0],
            "ms_chain": timed(torch, chain, n, 2)[0], "ms_segment_prefill": timed(torch, seg, n, 2)[0],
            "per_rank_share": {"workload": "one segment: %d tokens x 64 heads" % L,
                               "ms_segment_map": timed(torch, rank_maps, n, 2)[0],
                               "ms_prefill_from_incoming_state": timed(torch, rank_seg, n, 2)[0]}}


def bench_decode(torch, K, steps, warmup):
    from gated_delta_rule_02_amd import synth
    d = synth.workload_decode()
    q, k, v, g, b = (dev(d[x], torch) for x in ("q", "k", "v", "g", "beta"))
    st = torch.from_numpy(d["state"]).cuda()
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ms, _ = timed(torch, lambda: K.kda_decode_step(q, k, v, g, b, st, o), steps, warmup)
    x, cst, w = dev(d["conv_x"], torch), dev(d["conv_state"], torch), dev(d["conv_w"], torch)
    y = torch.empty_like(x)
    ms_conv, _ = timed(torch, lambda: K.kda_conv_state_update(x, cst, w, y), steps, warmup)
    ms_conv_graph = graph_ms(torch, lambda: K.kda_conv_state_update(x, cst, w, y), steps)
    # reference: a plain in-place read-modify-write of a buffer the size of the
    # state (torch's elementwise kernel), the access pattern decode cannot avoid
    ms_ref, _ = timed(torch, lambda: st.mul_(1.0), max(5, steps // 2), 2)
    return ms, (ms_conv, ms_conv_graph), ms_ref


def bench_decode_multi(torch, K, steps, warmup):
    """Draft verification: B=256 sequences x 4 tokens x 64 heads, the state
    after every token kept (4 GiB), the input state only read."""
    from gated_delta_rule_02_amd import synth
    d = synth.workload_decode_multi()
    B, Tq, H = 256, d["Tq"], 64
    q, k, v, g = (dev(d[x], torch).view(B, Tq, H, 128) for x in ("q", "k", "v", "g"))
    b = dev(d["beta"], torch).view(B, Tq, H)
    st = torch.from_numpy(d["state"]).cuda()
    ts = torch.empty((B, Tq, H, 128, 128), dtype=torch.float32, device="cuda")
    o = torch.empty((B, Tq, H, 128), dtype=torch.float32, device="cuda")
    ms, _ = timed(torch, lambda: K.kda_decode_multi(q, k, v, g, b, st, o, token_states=ts), steps, warmup)
    nbytes = (B * H * 128 * 128 * 4 * (1 + Tq) + 4 * B * Tq * H * 128 * 2 + B * Tq * H * 2
              + B * Tq * H * 128 * 4)
    return ms, nbytes


def bench_decode_bf16_state(torch, K, steps, warmup):
    """The decode step with the state stored in bfloat16 (512 MiB read and
    written; float32 arithmetic), on the decode workload's inputs."""
    from gated_delta_rule_02_amd import synth
    d = synth.workload_decode()
    B, H = 256, 64
    q, k, v, g = (dev(d[x], torch).view(B, 1, H, 128) for x in ("q", "k", "v", "g"))
    b = dev(d["beta"], torch).view(B, 1, H)
    st = torch.from_numpy(d["state"]).cuda().to(torch.bfloat16)
    o = torch.empty((B, 1, H, 128), dtype=torch.float32, device="cuda")
    ms, _ = timed(torch, lambda: K.kda_decode_multi(q, k, v, g, b, st, o), steps, warmup)
    nbytes = 2 * B * H * 128 * 128 * 2 + 4 * B * H * 128 * 2 + B * H * 2 + B * H * 128 * 4
    return ms, nbytes


def bench_gemv_fp8(torch, K, steps, warmup):
    """One decode token through the layer's input projection with block-FP8
    weights (41,024 x 4,096 E4M3 codes + 128 x 128 block scales): HBM-bound
    on the 168 MB of codes."""
    N, Kd = 5 * 8192 + 64, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    codes = torch.randint(0, 126, (N, Kd), device="cuda", generator=g, dtype=torch.int32).to(torch.uint8)
    scales = torch.rand(((N + 127) // 128, Kd // 128), device="cuda", generator=g) * 0.01
    x = torch.randn(1, Kd, device="cuda", generator=g).to(torch.bfloat16)
    y = torch.empty(1, N, dtype=torch.float32, device="cuda")
    ms, _ = timed(torch, lambda: K.kda_gemv_fp8(x, codes, scales, y), steps, warmup)
    nbytes = N * Kd + scales.numel() * 4 + Kd * 2 + N * 4
    return ms, nbytes


def bench_w8a8(torch, K, steps, warmup):
    """Block-FP8 W8A8 on the layer's input projection (41,024 x 4,096 E4M3
    weights, 128 x 128 scales): the activations quantized per token and
    128-column group, then the FP8 product; for one decode token (weight
    streaming) and for the 8,192-token prefill (matrix cores)."""
    N, Kd, M = 5 * 8192 + 64, 4096, 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    wc = torch.randint(0, 126, (N, Kd), device="cuda", generator=g, dtype=torch.int32).to(torch.uint8)
    ws = torch.rand(((N + 127) // 128, Kd // 128), device="cuda", generator=g) * 0.01
    x = torch.randn(M, Kd, device="cuda", generator=g).to(torch.bfloat16)
    xc = torch.empty(M, Kd, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, Kd // 128, dtype=torch.float32, device="cuda")
    y1 = torch.empty(1, N, dtype=torch.float32, device="cuda")
    ms_q1, _ = timed(torch, lambda: K.kda_quantize_fp8(x[:1], xc[:1], xs[:1]), steps, warmup)
    ms_d, _ = timed(torch, lambda: K.kda_gemm_fp8(xc[:1], xs[:1], wc, ws, y1), steps, warmup)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ms_q, _ = timed(torch, lambda: K.kda_quantize_fp8(x, xc, xs), steps, warmup)
    ms_g, _ = timed(torch, lambda: K.kda_gemm_fp8(xc, xs, wc, ws, y), max(3, steps // 2), 2)
    return {"decode": (ms_q1, ms_d, N * Kd + ws.numel() * 4 + Kd + Kd // 128 * 4 + N * 4),
            "prefill": (ms_q, ms_g, 2.0 * M * N * Kd, M * Kd * 2 + M * Kd + M * Kd // 128 * 4)}


def bench_layer(torch, steps, warmup):
    from gated_delta_rule_02_amd import layer, synth
    d = synth.workload_layer()
    mixer = layer.KDAMixer.from_host(d)
    x = dev(d["x"], torch)
    fn = lambda: mixer.forward(x)
    ms, _ = timed(torch, fn, max(1, steps // 4), max(1, warmup // 2))
    return ms, mixer.flops_per_token() * x.shape[0]


def bench_layer_fp8(torch, steps, warmup):
    """The same layer with block-FP8 (W8A8) projections."""
    from gated_delta_rule_02_amd import layer, synth
    d = synth.workload_layer_fp8()
    mixer = layer.KDAMixerFP8.from_host(d)
    x = dev(d["x"], torch)
    ms, _ = timed(torch, lambda: mixer.forward(x), max(1, steps // 4), max(1, warmup // 2))
    return ms, mixer.flops_per_token() * x.shape[0]


def bench_decode_layer_fp8(torch, steps, warmup, B=1):
    """One decode step of the W8A8 layer for B sequences (hidden 4096, H=64):
    launched eagerly from the host, and replayed from one HIP graph."""
    from gated_delta_rule_02_amd import layer, synth
    d = synth.workload_layer_fp8(T=8)
    mixer = layer.KDAMixerFP8.from_host(d)
    H, W = d["H"], d["H"] * 128
    x = dev(d["x"], torch)[:1].repeat(B, 1).contiguous()
    st = torch.zeros((B, H, 128, 128), device="cuda")
    cs = torch.zeros((3, B, 3, W), dtype=torch.bfloat16, device="cuda")
    ms_e, _ = timed(torch, lambda: mixer.decode(x, st, cs), steps, warmup)
    g = layer.DecodeGraph(mixer, B, st, cs)
    ms_g, _ = timed(torch, lambda: g.step(x), steps, warmup)
    wbytes = mixer.W_in.numel() + mixer.Wo.numel()
    return ms_e, ms_g, wbytes


def bench_gemm(torch, K, steps, warmup):
    """The layer's input projection alone (M = 8192 tokens, K = 4096,
    N = 5 x 8192 + 64, bf16 in and out) with the library's GEMM, and the same
    product with torch.mm (the vendor BLAS) on a pre-transposed weight as a
    reference."""
    M, N, Kd = 8192, 5 * 8192 + 64, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    A = torch.randn(M, Kd, device="cuda", generator=g).to(torch.bfloat16)
    B = (torch.randn(N, Kd, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ms, _ = timed(torch, lambda: K.kda_gemm(A, B, C), max(3, steps // 2), 2)
    Bt = B.t().contiguous()
    C2 = torch.empty_like(C)
    ms_ref, _ = timed(torch, lambda: torch.mm(A, Bt, out=C2), max(3, steps // 2), 2)
    return ms, ms_ref, 2.0 * M * N * Kd


def cpu_baseline(d, min_seconds=10.0):
    """The FP64 oracle (token-serial, threads over heads) on the prefill
    workload, timed on this host: the whole 4096-token sequence is run again
    until at least `min_seconds` of wall time have passed."""
    from oracle import reference as R
    threads = R.default_threads()
    T = d["q"].shape[0]
    reps = 0
    t0 = time.perf_counter()
    while True:
        R.kda_serial(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals, nthreads=threads)
        reps += 1
        t = time.perf_counter() - t0
        if t >= min_seconds:
            break
    return {"value": reps * T / t, "unit": "tokens/s/layer", "cores": threads, "kind": "oracle",
            "sample": "the prefill workload (4096 tokens x 64 heads, d=128, zero initial state) run %d times "
                      "back to back, fp64 token-serial, %.1f s wall on %d threads" % (reps, t, threads)}


def bench_copy(torch, steps, warmup):
    """A plain device-to-device copy of 256 MiB: the known-size kernel that
    calibrates the HBM byte counters."""
    n = 64 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms, _ = timed(torch, lambda: dst.copy_(src), steps, warmup)
    return {"workload": "torch copy_ of 256 MiB float32", "read_bytes_per_launch": n * 4,
            "write_bytes_per_launch": n * 4, "ms_per_step": ms, "GB/s": 2 * n * 4 / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-layer", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only", choices=["prefill", "seqpar", "varlen", "decode", "decode_step", "layer", "fp8", "copy"],
                    default=None,
                    help="time one path only (for profiler runs); 'copy' times the plain copy that calibrates byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_02_amd import kda as K
    K.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    out = {}
    if args.only in (None, "prefill"):
        log("prefill T=4096 H=64")
        ms_warm, wall, d, (ms, ms_cold_mean), ms_snap = bench_prefill(torch, K, args.steps, args.warmup)
        log("prefill %.3f ms/step median with the caches flushed before each call (%.3f ms warm, back to back)"
            % (ms, ms_warm))
        T = 4096
        achieved = PREFILL_BYTES_PER_TOKEN * T / (ms * 1e-3) / 1e9
        traffic = None
        if os.path.exists(COUNTERS):
            c = json.load(open(COUNTERS))
            if c.get("source_hash") == kernel_source_hash():
                traffic = c.get("hbm_bytes_per_launch")
        out.update({
            "metric": "KDA prefill tokens/s/layer (T=4096,H=64,d=128); decode state GB/s",
            "value": T / (ms * 1e-3), "unit": "tokens/s/layer", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "KDA prefill, one layer: B=1 T=4096 H=64 dk=dv=128, bf16 q/k/v/g/beta, "
                                   "fp32 state in/out, fp32 o, chunk 64",
                       "global_batch": 1, "seq_len": T, "heads": 64, "head_dim": 128, "chunk": 64},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                         "kernel": "kda_prefill call (two-pass form: intra_kernel + state_roles_kernel per window, 2 windows of 32 chunks)",
                         "algorithmic_bytes_per_launch": PREFILL_BYTES_PER_TOKEN * T,
                         "mfma_tflops": PREFILL_FLOPS_PER_TOKEN * T / (ms * 1e-3) / 1e12,
                         "mfma_frac_of_bf16_peak": PREFILL_FLOPS_PER_TOKEN * T / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
            "timing": "median of the timed calls, each bracketed by its own HIP events on the launch stream, "
                      "with 512 MiB written before every call (untimed) so that no input is cached",
            "prefill_cold_cache_mean_ms": ms_cold_mean,
            "prefill_warm": {"ms_per_step": ms_warm, "tokens/s/layer": T / (ms_warm * 1e-3),
                             "method": "the same call back to back, caches warm: mean over the timed calls"},
            "prefill_snapshots": {"workload": "the same prefill saving the state every 1024 tokens (4 x 4 MiB)",
                                  "ms_per_step": ms_snap, "tokens/s/layer": T / (ms_snap * 1e-3)},
        })
        if not args.skip_cpu:
            log("cpu baseline (fp64 oracle)")
            out["cpu_baseline"] = cpu_baseline(d)
    if args.only in (None, "seqpar"):
        log("sequence-parallel prefill pieces, 4 segments")
        out["sequence_parallel"] = bench_seqpar(torch, K, args.steps, args.warmup)
        log("sequence-parallel total %.3f ms" % out["sequence_parallel"]["ms_total"])
    if args.only in (None, "varlen"):
        log("varlen prefill, 8 packed sequences")
        ms_v, T_v, lens = bench_varlen(torch, K, args.steps, args.warmup)
        log("varlen %.3f ms/step for %d tokens" % (ms_v, T_v))
        out["varlen"] = {"workload": "packed varlen prefill: 8 sequences, lengths %s (%d tokens), H=64 "
                                     "dk=dv=128, bf16 inputs, fp32 initial and final states, fp32 o" % (lens, T_v),
                         "ms_per_step": ms_v, "tokens/s/layer": T_v / (ms_v * 1e-3),
                         "algorithmic_GB/s": (T_v * (4 * 64 * 128 * 2 + 64 * 2 + 64 * 128 * 4)
                                              + 2 * 8 * 64 * 128 * 128 * 4) / (ms_v * 1e-3) / 1e9}
    if args.only == "decode_step":
        # the decode step and the conv update alone (a profile of this run
        # holds no other decode_kernel instantiation)
        log("decode step only, B=256 H=64")
        ms, (ms_conv, ms_cg), ms_ref = bench_decode(torch, K, args.steps, args.warmup)
        out["decode"] = {"ms_per_step": ms, "GB/s": DECODE_BYTES / (ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": DECODE_BYTES / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        out["conv_update"] = {"ms_per_step": ms_conv, "GB/s": CONV_BYTES / (ms_conv * 1e-3) / 1e9,
                              "graph_ms_per_step": ms_cg, "graph_frac_of_hbm_peak": CONV_BYTES / (ms_cg * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if args.only in (None, "decode"):
        log("decode B=256 H=64")
        ms, (ms_conv, ms_cg), ms_ref = bench_decode(torch, K, args.steps, args.warmup)
        log("decode %.3f ms/step, conv %.4f ms (%.4f ms in a graph), in-place stream %.3f ms" % (ms, ms_conv, ms_cg, ms_ref))
        ref_gbs = 2 * 2 ** 30 / (ms_ref * 1e-3) / 1e9
        out["decode"] = {"workload": "decode step B=256 H=64 dk=dv=128, bf16 inputs, fp32 state [256,64,128,128] in place, fp32 o",
                         "ms_per_step": ms, "GB/s": DECODE_BYTES / (ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": DECODE_BYTES / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_step": DECODE_BYTES, "state_GB/s": 2 * 2 ** 30 / (ms * 1e-3) / 1e9,
                         "inplace_stream_reference_GB/s": ref_gbs,
                         "inplace_stream_reference": "torch mul_ in place on the 1 GiB state buffer (read + write)"}
        out["conv_update"] = {"workload": "x [256,8192] bf16, state [256,3,8192] bf16 in place",
                              "ms_per_step": ms_conv, "GB/s": CONV_BYTES / (ms_conv * 1e-3) / 1e9,
                              "frac_of_hbm_peak": CONV_BYTES / (ms_conv * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "graph_ms_per_step": ms_cg,
                              "graph_frac_of_hbm_peak": CONV_BYTES / (ms_cg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "note": "ms_per_step: back-to-back launches, which for a kernel of a few microseconds "
                                      "include the dispatch gap; graph_ms_per_step: 20 calls replayed from one HIP graph"}
        log("decode B=256 H=64, bf16 state")
        ms_b, nb = bench_decode_bf16_state(torch, K, args.steps, args.warmup)
        out["decode_bf16_state"] = {"workload": "decode step B=256 H=64, bf16 inputs, state stored in bf16 "
                                                "[256,64,128,128] (512 MiB) in place, fp32 arithmetic, fp32 o",
                                    "ms_per_step": ms_b, "bytes_per_step": nb, "GB/s": nb / (ms_b * 1e-3) / 1e9,
                                    "frac_of_hbm_peak": nb / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "speedup_vs_fp32_state": ms / ms_b}
        log("fp8 GEMV 41024 x 4096")
        ms_f, nbf = bench_gemv_fp8(torch, K, args.steps, args.warmup)
        out["gemv_fp8"] = {"workload": "one decode token through the input projection, block-FP8 weights "
                                       "41,024 x 4,096 E4M3 + 128x128 fp32 scales, bf16 x, fp32 y",
                           "ms_per_step": ms_f, "bytes_per_step": nbf, "GB/s": nbf / (ms_f * 1e-3) / 1e9,
                           "frac_of_hbm_peak": nbf / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log("decode multi-token B=256 x 4 tokens")
        ms_m, nbytes = bench_decode_multi(torch, K, args.steps, args.warmup)
        log("decode multi %.3f ms/step" % ms_m)
        out["decode_multi"] = {"workload": "draft verification B=256 x 4 tokens x H=64, bf16 inputs, fp32 state "
                                           "read once, the state after every token written (4 GiB), fp32 o",
                               "ms_per_step": ms_m, "bytes_per_step": nbytes, "GB/s": nbytes / (ms_m * 1e-3) / 1e9,
                               "frac_of_hbm_peak": nbytes / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if args.only == "layer" or (args.only is None and not args.skip_layer):
        log("layer T=8192 hidden=4096")
        ms, flops = bench_layer(torch, args.steps, args.warmup)
        log("layer %.3f ms/step" % ms)
        out["layer"] = {"workload": "full token-mixer layer T=8192 hidden=4096 H=64: projections, conv, gate, "
                                    "KDA core, norm x gate, output projection",
                        "ms_per_step": ms, "tokens/s": 8192 / (ms * 1e-3), "TFLOP/s": flops / (ms * 1e-3) / 1e12}
        log("layer T=8192 hidden=4096, block-FP8 W8A8 projections")
        ms8, flops8 = bench_layer_fp8(torch, args.steps, args.warmup)
        log("layer fp8 %.3f ms/step" % ms8)
        out["layer_fp8"] = {"workload": "the same layer with E4M3 weights in 128x128 blocks (fp32 block scales) and "
                                        "activations quantized per (token, 128 channels): kda_quantize_fp8, "
                                        "kda_gemm_fp8, kda_output_norm_gate_fp8",
                            "ms_per_step": ms8, "tokens/s": 8192 / (ms8 * 1e-3), "TFLOP/s": flops8 / (ms8 * 1e-3) / 1e12,
                            "speedup_vs_bf16_layer": ms / ms8}
        for Bd in (1, 8):
            log("W8A8 layer decode step B=%d: eager and HIP graph" % Bd)
            ms_e, ms_g, wb = bench_decode_layer_fp8(torch, args.steps, args.warmup, B=Bd)
            log("decode B=%d eager %.4f ms, graph %.4f ms" % (Bd, ms_e, ms_g))
            out["layer_fp8_decode_b%d" % Bd] = {
                "workload": "one decode token for %d sequence(s) through the W8A8 layer (hidden 4096, H=64): "
                            "quantize, FP8 GEMV, 3 conv updates, gate, decode step, quantized epilogue, FP8 GEMV" % Bd,
                "ms_eager": ms_e, "ms_graph": ms_g, "weight_bytes": wb,
                "weight_GB/s_graph": wb / (ms_g * 1e-3) / 1e9}
        log("input projection GEMM 8192 x 41024 x 4096")
        ms_g, ms_r, fl = bench_gemm(torch, K, args.steps, args.warmup)
        out["gemm"] = {"workload": "input projection 8192 x 41024 x 4096, bf16 in and out, fp32 accumulate",
                       "ms_per_step": ms_g, "TFLOP/s": fl / (ms_g * 1e-3) / 1e12,
                       "frac_of_bf16_peak": fl / (ms_g * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                       "vendor_blas_reference_TFLOP/s": fl / (ms_r * 1e-3) / 1e12,
                       "vendor_blas_reference": "torch.mm on the same bf16 operands (weight pre-transposed)"}
    if args.only in (None, "fp8"):
        log("block-FP8 W8A8 input projection (decode token and 8192-token prefill)")
        r = bench_w8a8(torch, K, args.steps, args.warmup)
        q1, d1, nb1 = r["decode"]
        qp, gp, fl, nbq = r["prefill"]
        log("w8a8 decode %.4f ms (+ quantize %.4f), prefill gemm %.3f ms (+ quantize %.3f)" % (d1, q1, gp, qp))
        out["w8a8"] = {
            "workload": "input projection 41,024 x 4,096 with E4M3 weights in 128x128 blocks and activations "
                        "quantized per (token, 128 channels); bf16 x quantized by kda_quantize_fp8",
            "decode_token": {"ms_gemm": d1, "ms_quantize": q1, "bytes_per_step": nb1,
                             "GB/s": nb1 / (d1 * 1e-3) / 1e9, "frac_of_hbm_peak": nb1 / (d1 * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "prefill_8192": {"ms_gemm": gp, "ms_quantize": qp, "TFLOP/s": fl / (gp * 1e-3) / 1e12,
                             "frac_of_fp8_peak": fl / (gp * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
                             "quantize_GB/s": nbq / (qp * 1e-3) / 1e9}}
    if args.only == "copy":
        log("copy 256 MiB")
        out["copy"] = bench_copy(torch, args.steps, args.warmup)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
