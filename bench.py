#!/usr/bin/env python3
"""Benchmark of the BitLinear hot path on one MI355X.

Default workload: the 70B-shaped ternary stack (80 layers x q 8192x8192, k/v 1024x8192,
o 8192x8192, gate/up 28672x8192, down 8192x28672, 2-bit packed T2-PN-64, 17,112,760,320
bytes) decoded at M=1 token. One step = one pass over all 80 layers; each layer runs four
dependent linear groups in model order (stacked q|k|v, o, stacked gate|up, down), each one
launch of the fused quantise + add-only GEMV (int32 accumulation by select + popcount, no
multiplies); the pass is replayed from a HIP graph. The metric is effective HBM GB/s =
algorithmic bytes of the pass / pass time.

The same JSON line carries the other measured workloads under "extra": the same pass on the
int8 matrix cores from T2-MF64 weights (bl_bitlinear_forward_mf) and as one persistent
launch; the stack at M = 8, 32, 64 (tokens/s); the 3B-shaped prefill at M = 512 (int8
TOPS); the 7B-shaped decode set, the OneBit and residual 4096x4096 layers and SVID; a
"roofline" object for the dominant kernel and a "cpu_baseline" object for the CPU oracle.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-extra] [--only NAME]
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

METRIC = "BitLinear GEMV effective HBM GB/s (% peak); int8 TOPS at M=512 (% peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode70b_m1_traffic.json")
# the dominant kernel's sources: its file and the device helpers it includes
KERNEL_SOURCES = [os.path.join(ROOT, "ternary_weight_linear_amd", "csrc", f)
                  for f in ("gemv.hip", "bl_internal.h")]
CEIL_LIB = os.path.join(ROOT, "ternary_weight_linear_amd", "libblceil.so")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--skip-extra", action="store_true", help="only the default workload")
    p.add_argument("--skip-cpu", action="store_true", help="no CPU-oracle baseline")
    p.add_argument("--only", default="", help="run one extra workload by name (profiling)")
    p.add_argument("--no-graph", action="store_true", help="launch the pass eagerly (profilers)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run a plain 1 GiB device copy (HBM counter calibration) and exit")
    p.add_argument("--ceilings", action="store_true",
                   help="measure the streaming-read and int8 matrix-core ceilings only")
    return p.parse_args()


# ------------------------------------------------------------------------------------------
# timing helpers: HIP events on the stream the kernels are launched on
# ------------------------------------------------------------------------------------------
def timed(torch, fn, steps, warmup):
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps          # ms per call of fn


# ------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------
def build_stack70b(torch, tw, sgpu, synth, dev):
    """80 layers of packed ternary weights, stacked per dependent group (N-concatenation of
    T2-PN-64 buffers is the packed form of the stacked matrix)."""
    return build_stack(torch, tw, sgpu, synth, dev, synth.LLAMA70B_LINEARS, synth.LLAMA70B_LAYERS, 5)


def build_stack(torch, tw, sgpu, synth, dev, linears, nlayers, key_id):
    """nlayers layers of the given linears, packed and stacked per dependent group: q|k|v and
    gate|up share their input, so each pair or triple is one matrix of stacked rows."""
    shapes = dict((n, (N, K)) for n, N, K in linears)
    groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gateup", ["gate", "up"]), ("down", ["down"])]
    tmp = torch.empty(max(N * K for N, K in shapes.values()), dtype=torch.int8, device=dev)
    layers = []
    for layer in range(nlayers):
        lg = []
        for gname, members in groups:
            K = shapes[members[0]][1]
            Ntot = sum(shapes[m][0] for m in members)
            buf = torch.empty(Ntot * K // 4, dtype=torch.uint8, device=dev)
            off = 0
            for m in members:
                N = shapes[m][0]
                mid = [n for n, _, _ in linears].index(m)
                key = synth.matrix_key(0, key_id, layer, mid)
                codes = tmp[: N * K].view(N, K)
                sgpu.ternary_codes(key, N, K, dev, out=codes)
                st = tw._lib.bl_pack_ternary(tw._ptr(codes), N, K, tw.ctypes.c_void_p(buf.data_ptr() + off),
                                             None, tw._stream(torch.device(dev)))
                assert st == 0
                off += N * K // 4
            lg.append((gname, buf, Ntot, K))
        layers.append(lg)
    torch.cuda.synchronize()
    del tmp
    return layers


def stack_bytes(layers):
    return sum(buf.numel() for lg in layers for _, buf, _, _ in lg)


def decode_pass(torch, tw, synth, dev, layers, M):
    """Per-(layer, group) activations and output buffers, and the pass closure.

    M <= 2: one launch per group, the fused quantise + add-only GEMV (bl_bitlinear_forward,
    GEMV path). M > 2: quantiser launch + int8-MFMA GEMM launch per group."""
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=dev)
    items = []
    for li, lg in enumerate(layers):
        for gi, (gname, buf, N, K) in enumerate(lg):
            x = torch.from_numpy(synth.normal_fp16((M, K), 0, 5, 1000 + li, gi)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            items.append(dict(x=x, w=buf, N=N, K=K, y=y))
    use_gemv = M <= 2
    ws_need = max(tw.bl_workspace_bytes(M, it["N"], it["K"]) for it in items)
    ws = tw.workspace(dev, ws_need)
    wsp, wsb = tw.ctypes.c_void_p(ws.data_ptr()), ws.numel()
    lib, P = tw._lib, tw.ctypes.c_void_p
    for it in items:
        if not use_gemv:
            it["q"] = torch.empty((M, it["K"]), dtype=torch.int8, device=dev)
            it["gamma"] = torch.empty(M, dtype=torch.float32, device=dev)
    bp = P(beta.data_ptr())
    args = []
    for it in items:
        a = dict(x=P(it["x"].data_ptr()), w=P(it["w"].data_ptr()), y=P(it["y"].data_ptr()), N=it["N"], K=it["K"])
        if not use_gemv:
            a["q"], a["g"] = P(it["q"].data_ptr()), P(it["gamma"].data_ptr())
        args.append(a)

    def full_pass():
        stream = P(torch.cuda.current_stream().cuda_stream)    # the capture stream inside a graph
        for a in args:
            if use_gemv:
                st = lib.bl_bitlinear_forward(a["x"], M, a["K"], a["w"], bp, 1, a["N"], a["y"],
                                              tw.BL_PATH_GEMV, wsp, wsb, stream)
            else:
                st = lib.bl_quant_act_int8(a["x"], M, a["K"], a["q"], a["g"], None, None, stream)
                assert st == 0
                st = lib.bl_bitlinear_gemm(a["q"], a["g"], M, a["K"], a["w"], bp, 1, a["N"], a["y"],
                                           wsp, wsb, stream)
            assert st == 0

    algo_bytes = sum(it["w"].numel() + 2 * M * it["K"] + 4 * M * it["N"] for it in items)
    weight_bytes = sum(it["w"].numel() for it in items)
    launches = len(items) * (1 if use_gemv else 2)
    return items, full_pass, algo_bytes, weight_bytes, launches


def repack_stack_mf(torch, tw, dev, layers):
    """The same 80 layers in T2-MF64, the matrix-core layout of the batched path."""
    out = []
    for lg in layers:
        out.append([(gname, tw.bl_repack_ternary_mf(buf, N, K), N, K) for gname, buf, N, K in lg])
    torch.cuda.synchronize()
    return out


def decode_pass_mf(torch, tw, synth, dev, layers_mf, M):
    """Decode over T2-MF64 weights: per group one bl_bitlinear_forward_mf call (M <= 16: one
    fused launch; above: quantiser + matrix-core product; same activations as decode_pass)."""
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=dev)
    items = []
    for li, lg in enumerate(layers_mf):
        for gi, (gname, buf, N, K) in enumerate(lg):
            x = torch.from_numpy(synth.normal_fp16((M, K), 0, 5, 1000 + li, gi)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            items.append(dict(x=x, w=buf, N=N, K=K, y=y))
    ws = tw.workspace(dev, max(tw.bl_workspace_bytes(M, it["N"], it["K"]) for it in items))
    wsp, wsb = tw.ctypes.c_void_p(ws.data_ptr()), ws.numel()
    lib, P = tw._lib, tw.ctypes.c_void_p
    bp = P(beta.data_ptr())
    args = [(P(it["x"].data_ptr()), it["K"], P(it["w"].data_ptr()), it["N"], P(it["y"].data_ptr()))
            for it in items]

    def full_pass():
        stream = P(torch.cuda.current_stream().cuda_stream)
        for x, K, w, N, y in args:
            st = lib.bl_bitlinear_forward_mf(x, M, K, w, bp, 1, N, y, wsp, wsb, stream)
            assert st == 0

    algo_bytes = sum(it["w"].numel() + 2 * M * it["K"] + 4 * M * it["N"] for it in items)
    weight_bytes = sum(it["w"].numel() for it in items)
    # launches per linear, as the header states for bl_bitlinear_forward_mf: one fused launch
    # at M <= 4, and at M <= 16 for K <= 8192 over fewer than 512 bands; else two
    def launches(N, K):
        return 1 if M <= 4 or (M <= 16 and K <= 8192 and N // 64 < 512) else 2
    return (items, full_pass, algo_bytes, weight_bytes,
            sum(launches(it["N"], it["K"]) for it in items))


def bench_decode70b_mf(torch, tw, synth, dev, layers_mf, M, steps, warmup, use_graph=True):
    items, full_pass, algo, wbytes, launches = decode_pass_mf(torch, tw, synth, dev, layers_mf, M)
    ms_eager = timed(torch, full_pass, max(1, steps // 4), 1 if warmup else 0)
    run, keep = (graphed(torch, full_pass) if use_graph else (full_pass, None))
    ms = timed(torch, run, steps, warmup)
    return dict(ms_per_pass=ms, ms_per_pass_eager=ms_eager, launches_per_pass=launches,
                groups=len(items), algo_bytes=algo, weight_bytes=wbytes,
                tokens_per_s=M / (ms / 1e3), gbs=algo / (ms / 1e3) / 1e9,
                weight_gbs=wbytes / (ms / 1e3) / 1e9, graph=use_graph)


def graphed(torch, fn):
    """Capture one call of fn into a HIP graph (after a warm-up call) and return its replay."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g.replay, g


def read_floor_pass(torch, dev, layers, steps, warmup):
    """The decode pass with every GEMV launch replaced by a streaming read of the same packed
    weight buffer, launched in the same order and replayed from a HIP graph like the timed
    pass: what the pass's dependent launches over these sizes cost with no arithmetic."""
    return read_floor(torch, dev, [buf for lg in layers for (_, buf, _, _) in lg], steps, warmup)


def read_floor(torch, dev, buffers, steps, warmup):
    """One streaming read per buffer (one contiguous slice per workgroup with non-temporal
    loads, or grid-strided reads), in order, replayed from a HIP graph. The read and its grid
    are the fastest of a few per buffer size."""
    import ctypes
    lib = ctypes.CDLL(CEIL_LIB)
    P = ctypes.c_void_p
    for fn in (lib.bl_ceil_stream_read, lib.bl_ceil_stream_read_slices):
        fn.argtypes = [P, ctypes.c_int64, P, ctypes.c_int, P]
    out = torch.zeros(4096, dtype=torch.int32, device=dev)
    bufs = [(buf, buf.numel()) for buf in buffers]
    kinds = {"slices": lib.bl_ceil_stream_read_slices, "strided": lib.bl_ceil_stream_read}
    best_by = {}
    for nb in sorted({n for _, n in bufs}):
        # slices where the size divides into whole 32 KiB pieces per workgroup, grid-strided
        # reads (any size) otherwise or where faster
        cands = [("slices", g) for g in (32, 64, 128, 160, 256, 320, 448, 512, 640, 896, 1024, 1792, 2048)
                 if nb % (g * 32768) == 0]
        cands += [("strided", g) for g in (512, 1024, 2048, 4096)]
        same = [b for b, n in bufs if n == nb]
        best = None
        for kind, g in cands:
            def sweep(kind=kind, g=g):
                st = P(torch.cuda.current_stream().cuda_stream)
                for b in same:
                    assert kinds[kind](P(b.data_ptr()), nb, P(out.data_ptr()), g, st) == 0
            run, keep = graphed(torch, sweep)
            t = timed(torch, run, 3, 1) / len(same)
            del run, keep
            if best is None or t < best[0]:
                best = (t, kind, g)
        best_by[nb] = best

    def full_pass():
        st = P(torch.cuda.current_stream().cuda_stream)
        for b, nb in bufs:
            _, kind, g = best_by[nb]
            assert kinds[kind](P(b.data_ptr()), nb, P(out.data_ptr()), g, st) == 0

    run, keep = graphed(torch, full_pass)
    ms = timed(torch, run, steps, warmup)
    del run, keep
    return {"ms_per_pass": ms, "launches_per_pass": len(bufs),
            "us_per_launch_by_bytes": {str(nb): round(t * 1e3, 3) for nb, (t, k, g) in best_by.items()},
            "read_by_bytes": {str(nb): f"{k}, {g} workgroups" for nb, (t, k, g) in best_by.items()},
            "kernel": "stream_read_slices_kernel / stream_read_kernel (ceilings.hip)"}


def bench_decode70b(torch, tw, synth, dev, layers, M, steps, warmup, use_graph=True):
    items, full_pass, algo, wbytes, launches = decode_pass(torch, tw, synth, dev, layers, M)
    ms_eager = timed(torch, full_pass, max(1, steps // 4), 1 if warmup else 0)
    res = dict(ms_per_pass_eager=ms_eager)
    run, keep = (graphed(torch, full_pass) if use_graph else (full_pass, None))
    ms = timed(torch, run, steps, warmup)
    res.update(ms_per_pass=ms, launches_per_pass=launches, groups=len(items), algo_bytes=algo,
               weight_bytes=wbytes, tokens_per_s=M / (ms / 1e3), gbs=algo / (ms / 1e3) / 1e9,
               weight_gbs=wbytes / (ms / 1e3) / 1e9, graph=use_graph)
    return res


def bench_prefill3b(torch, tw, synth, dev, steps, warmup):
    """3B-shaped linears at M = 512: W ~ N(0, 0.02^2) -> absmean ternary on the GPU; x fp16 ~
    N(0,1) with 1% outlier channels x20. Groups stacked as in the decode pass. Measured with
    the weights in T2-MF64 (the matrix-core layout, repacked once on the GPU; quantiser with
    row sums + bl_bitlinear_gemm_mf) and, for comparison, in T2-PN-64 (bl_bitlinear_gemm)."""
    shapes = dict((n, (N, K)) for n, N, K in synth.LLAMA3B_LINEARS)
    groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gateup", ["gate", "up"]), ("down", ["down"])]
    M = 512
    items = []
    for gi, (gname, members) in enumerate(groups):
        K = shapes[members[0]][1]
        parts, betas = [], []
        for m in members:
            N = shapes[m][0]
            mid = [n for n, _, _ in synth.LLAMA3B_LINEARS].index(m)
            W = torch.from_numpy(synth.normal_fp32((N, K), 0, 4, 0, mid, std=0.02)).to(dev)
            packed, beta, _ = tw.bl_ternarize_absmean(W)
            parts.append(packed)
            betas.append(beta.expand(N))
            del W
        w = torch.cat(parts)
        beta = torch.cat(betas).contiguous()
        Ntot = sum(shapes[m][0] for m in members)
        x16, _ = synth.with_outlier_channels(synth.normal_fp16((M, K), 0, 4, 100, gi), 0.01, 20.0, 0, 4, 200 + gi)
        items.append(dict(x=torch.from_numpy(x16).to(dev), w=w, wmf=tw.bl_repack_ternary_mf(w, Ntot, K),
                          beta=beta, N=Ntot, K=K,
                          y=torch.empty((M, Ntot), dtype=torch.float32, device=dev),
                          q=torch.empty((M, K), dtype=torch.int8, device=dev),
                          gamma=torch.empty(M, dtype=torch.float32, device=dev),
                          rowsum=torch.empty(M, dtype=torch.int32, device=dev)))
    ws = tw.workspace(dev, max(tw.bl_workspace_bytes(M, it["N"], it["K"]) for it in items))
    wsp, wsb = tw.ctypes.c_void_p(ws.data_ptr()), ws.numel()
    stream = tw._stream(torch.device(dev))
    lib, P = tw._lib, tw.ctypes.c_void_p

    def quant(it):
        assert lib.bl_quant_act_int8(P(it["x"].data_ptr()), M, it["K"], P(it["q"].data_ptr()),
                                     P(it["gamma"].data_ptr()), P(it["rowsum"].data_ptr()), None,
                                     stream) == 0

    def gemm_mf(it):
        assert lib.bl_bitlinear_gemm_mf(P(it["q"].data_ptr()), P(it["gamma"].data_ptr()),
                                        P(it["rowsum"].data_ptr()), M, it["K"], P(it["wmf"].data_ptr()),
                                        P(it["beta"].data_ptr()), it["N"], it["N"], P(it["y"].data_ptr()),
                                        None, wsp, wsb, stream) == 0

    def gemm_pn(it):
        assert lib.bl_bitlinear_gemm(P(it["q"].data_ptr()), P(it["gamma"].data_ptr()), M, it["K"],
                                     P(it["w"].data_ptr()), P(it["beta"].data_ptr()), it["N"], it["N"],
                                     P(it["y"].data_ptr()), wsp, wsb, stream) == 0

    ops = sum(2 * M * it["N"] * it["K"] for it in items)

    def measure(gemm):
        ms = timed(torch, lambda: [f(it) for it in items for f in (quant, gemm)], steps, warmup)
        ms_g = timed(torch, lambda: [gemm(it) for it in items], steps, warmup)
        per_shape = {}
        for it in items:
            t = timed(torch, lambda it=it: gemm(it), steps, warmup)
            per_shape[f"{M}x{it['N']}x{it['K']}"] = dict(ms=t, tops=2 * M * it["N"] * it["K"] / (t / 1e3) / 1e12)
        return dict(ms_per_pass=ms, ms_gemms_only=ms_g, int8_ops=ops, tops_pass=ops / (ms / 1e3) / 1e12,
                    tops_gemms=ops / (ms_g / 1e3) / 1e12,
                    frac_peak_gemms=ops / (ms_g / 1e3) / 1e12 / INT8_PEAK_TOPS, per_shape=per_shape)

    res = measure(gemm_mf)
    res["weights"] = "T2-MF64"
    pn = measure(gemm_pn)
    res["t2pn"] = {k: pn[k] for k in ("ms_per_pass", "ms_gemms_only", "tops_gemms", "frac_peak_gemms")}
    res["library_int8"] = library_int8_gemms(torch, dev, items, M, steps, warmup)
    return res


def library_int8_gemms(torch, dev, items, M, steps, warmup):
    """Context for the prefill figure: the vendor BLAS int8 GEMM (torch._int_mm) on the same
    shapes, with the weights as dense int8 codes (4x the packed bytes), int32 outputs and no
    epilogue; the faster of the two weight layouts per shape. Not part of the path."""
    per_shape, ms_total, ops = {}, 0.0, 0
    for it in items:
        N, K = it["N"], it["K"]
        best = None
        for layout in ("KxN column-major", "KxN row-major"):
            if layout.endswith("column-major"):
                b = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev).t()
            else:
                b = torch.randint(-1, 2, (K, N), dtype=torch.int8, device=dev)
            t = timed(torch, lambda: torch._int_mm(it["q"], b), steps, warmup)
            if best is None or t < best[0]:
                best = (t, layout)
            del b
        per_shape[f"{M}x{N}x{K}"] = dict(ms=best[0], tops=2 * M * N * K / (best[0] / 1e3) / 1e12,
                                         weights=best[1])
        ms_total += best[0]
        ops += 2 * M * N * K
    return dict(op="torch._int_mm (vendor BLAS), int8 x int8 -> int32", per_shape=per_shape,
                ms_gemms=ms_total, tops_gemms=ops / (ms_total / 1e3) / 1e12)


def bench_decode7b_stack(torch, tw, sgpu, synth, dev, steps, warmup):
    """The LLaMA-7B-shaped model decoded at M = 1: 32 layers (1.62 GB packed, > the 256 MB
    MALL) in model order, q|k|v and gate|up stacked, one fused launch per group replayed
    from a HIP graph: the T2-MF64 decode kernel (the same pass as the 70B line) and, for
    comparison, the add-only GEMV from T2-PN-64."""
    layers = build_stack(torch, tw, sgpu, synth, dev, synth.LLAMA7B_LINEARS, 32, 3)
    layers_mf = repack_stack_mf(torch, tw, dev, layers)
    r = bench_decode70b_mf(torch, tw, synth, dev, layers_mf, 1, steps, warmup)
    del layers_mf
    out = {k: r[k] for k in ("ms_per_pass", "tokens_per_s", "gbs", "launches_per_pass", "weight_bytes")}
    out["weights"] = "T2-MF64"
    r = bench_decode70b(torch, tw, synth, dev, layers, 1, steps, warmup)
    out["t2pn_gemv"] = {k: r[k] for k in ("ms_per_pass", "tokens_per_s", "gbs")}
    # the same 128 launches reading their weights and nothing else
    rf = read_floor_pass(torch, dev, layers, steps, warmup)
    out["launch_read_floor_ms"] = rf["ms_per_pass"]
    out["frac_launch_read_floor"] = rf["ms_per_pass"] / out["ms_per_pass"]
    del layers
    return out


def bench_decode7b(torch, tw, sgpu, synth, dev, steps, warmup, pool=32):
    """7B-shaped set of 7 linears at M = 1, a pool of `pool` distinct sets (> the 256 MB MALL),
    each its own bl_bitlinear_gemv launch on bit planes quantised beforehand (the standalone
    GEMV entry point, no stacking)."""
    M = 1
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=dev)
    items = []
    tmp = torch.empty(11008 * 4096, dtype=torch.int8, device=dev)
    for s in range(pool):
        for mid, (name, N, K) in enumerate(synth.LLAMA7B_LINEARS):
            codes = tmp[: N * K].view(N, K)
            sgpu.ternary_codes(synth.matrix_key(0, 3, s, mid), N, K, dev, out=codes)
            w = tw.bl_pack_ternary(codes)
            x = torch.from_numpy(synth.normal_fp16((M, K), 0, 3, s, mid)).to(dev)
            q, gamma, _, planes = tw.bl_quant_act_int8(x, want_q=False, want_rowsum=False)
            items.append(dict(w=w, N=N, K=K, planes=planes, gamma=gamma,
                              y=torch.empty((M, N), dtype=torch.float32, device=dev)))
    del tmp
    ws = tw.workspace(dev, max(tw.bl_workspace_bytes(M, it["N"], it["K"]) for it in items))
    wsp, wsb = tw.ctypes.c_void_p(ws.data_ptr()), ws.numel()
    stream = tw._stream(torch.device(dev))
    lib, P = tw._lib, tw.ctypes.c_void_p
    bp = P(beta.data_ptr())

    def sweep():
        for it in items:
            assert lib.bl_bitlinear_gemv(P(it["planes"].data_ptr()), P(it["gamma"].data_ptr()), M, it["K"],
                                         P(it["w"].data_ptr()), bp, 1, it["N"], P(it["y"].data_ptr()),
                                         wsp, wsb, stream) == 0

    ms = timed(torch, sweep, steps, warmup)
    wbytes = sum(it["w"].numel() for it in items)
    return dict(pool_sets=pool, ms_per_sweep=ms, gemv_launches=len(items), weight_bytes=wbytes,
                gbs=wbytes / (ms / 1e3) / 1e9, us_per_set=ms * 1e3 / pool)


def bench_svid(torch, tw, synth, dev, steps, warmup):
    """SVID initialisation (signs + 20 rounds of power iteration) of a 4096x4096 fp32 weight."""
    N = K = 4096
    W = torch.from_numpy(synth.normal_fp32((N, K), 0, 2, 4, 0)).to(dev)
    ms = timed(torch, lambda: tw.bl_svid_rank1(W, iters=20), max(2, steps // 4), 1)
    return dict(ms=ms, iters=20, weight_bytes_read_per_iter=2 * N * K * 4,
                gbs=(2 * 20 + 1) * N * K * 4 / (ms / 1e3) / 1e9)


def bench_onebit(torch, tw, synth, dev, steps, warmup, pool=256):
    """OneBit 4096x4096 at M = 1 and 16 over a pool of 256 distinct sign matrices (512 MiB)."""
    N = K = 4096
    out = {}
    spool = []
    for s in range(pool):
        W = torch.from_numpy(synth.normal_fp32((N, K), 0, 2, 4, s)).to(dev) if s < 4 else None
        if W is not None:
            spool.append(tw.bl_pack_sign(W))
        else:   # distinct matrices without host generation: bit-rotate the four drawn ones
            spool.append(torch.roll(spool[s % 4], shifts=s))
    g = torch.from_numpy(synth.uniform_fp16((K,), 0.5, 1.5, 0, 2, 2)).to(dev)
    h = torch.from_numpy(synth.uniform_fp16((N,), 0.5, 1.5, 0, 2, 3)).to(dev)
    lib, P = tw._lib, tw.ctypes.c_void_p
    for M in (1, 16):
        x = torch.from_numpy(synth.normal_fp16((M, K), 0, 2, 1)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = tw.workspace(dev, tw.bl_workspace_bytes(M, N, K))
        wsp, wsb = P(ws.data_ptr()), ws.numel()

        def sweep():
            stream = P(torch.cuda.current_stream().cuda_stream)   # the capture stream in a graph
            for sp in spool:
                assert lib.bl_onebit_linear(P(x.data_ptr()), P(g.data_ptr()), P(sp.data_ptr()),
                                            P(h.data_ptr()), M, N, K, P(y.data_ptr()), wsp, wsb, stream) == 0

        ms_eager = timed(torch, sweep, max(2, steps // 4), 1)
        run, keep = graphed(torch, sweep)
        ms = timed(torch, run, max(2, steps // 4), 1)
        out[f"M{M}"] = dict(us_per_layer=ms * 1e3 / pool, us_per_layer_eager=ms_eager * 1e3 / pool,
                            gbs_signs=pool * N * K / 8 / (ms / 1e3) / 1e9,
                            stored_bits_per_layer=8 * spool[0].numel() + 16 * (N + K), graph=True)
    # the same launches reading their sign matrices and nothing else
    out["launch_read_floor_us_per_layer"] = read_floor(torch, dev, spool, max(2, steps // 4), 1)["ms_per_pass"] * 1e3 / pool
    # a 70B-sized matrix (28672 x 8192, 29 MiB of signs) at M = 1, pool of 16
    N2, K2, pool2 = 28672, 8192, 16
    W = torch.from_numpy(synth.normal_fp32((N2, K2), 0, 2, 5, 0)).to(dev)
    base = tw.bl_pack_sign(W)
    del W
    spool2 = [base] + [torch.roll(base, shifts=s) for s in range(1, pool2)]
    g2 = torch.from_numpy(synth.uniform_fp16((K2,), 0.5, 1.5, 0, 2, 6)).to(dev)
    h2 = torch.from_numpy(synth.uniform_fp16((N2,), 0.5, 1.5, 0, 2, 7)).to(dev)
    x2 = torch.from_numpy(synth.normal_fp16((1, K2), 0, 2, 8)).to(dev)
    y2 = torch.empty((1, N2), dtype=torch.float32, device=dev)
    ws2 = tw.workspace(dev, tw.bl_workspace_bytes(1, N2, K2))

    def sweep2():
        stream = P(torch.cuda.current_stream().cuda_stream)
        for sp in spool2:
            assert lib.bl_onebit_linear(P(x2.data_ptr()), P(g2.data_ptr()), P(sp.data_ptr()),
                                        P(h2.data_ptr()), 1, N2, K2, P(y2.data_ptr()),
                                        P(ws2.data_ptr()), ws2.numel(), stream) == 0

    run, keep = graphed(torch, sweep2)
    ms = timed(torch, run, max(2, steps // 4), 1)
    out["28672x8192_M1"] = dict(us_per_layer=ms * 1e3 / pool2,
                                gbs_signs=pool2 * N2 * K2 / 8 / (ms / 1e3) / 1e9, graph=True,
                                launch_read_floor_us=read_floor(torch, dev, spool2, max(2, steps // 4), 1)["ms_per_pass"] * 1e3 / pool2)
    return out


def bench_residual(torch, tw, synth, dev, steps, warmup, pool=128):
    """Residual-binarised 4096x4096 layers at M = 1 and 16 over a pool of 128 distinct
    layers (two sign planes + two fp32 scale arrays each: 5 MiB, 640 MiB in all)."""
    N = K = 4096
    out = {}
    layers = []
    for s in range(pool):
        if s < 4:
            W = torch.from_numpy(synth.normal_fp32((N, K), 0, 15, s, std=0.02)).to(dev)
            layers.append(tw.bl_residual_binarize(W))
        else:   # distinct layers without host generation: rotate the four binarised ones
            layers.append(tuple(torch.roll(t, shifts=s) for t in layers[s % 4]))
    lib, P = tw._lib, tw.ctypes.c_void_p
    layer_bytes = sum(t.numel() * t.element_size() for t in layers[0])
    for M in (1, 16):
        x = torch.from_numpy(synth.normal_fp16((M, K), 0, 15, 100 + M)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = tw.workspace(dev, tw.bl_workspace_bytes(M, N, K))
        wsp, wsb = P(ws.data_ptr()), ws.numel()
        ptrs = [[P(t.data_ptr()) for t in L] for L in layers]

        def sweep():
            stream = P(torch.cuda.current_stream().cuda_stream)   # the capture stream in a graph
            for po, ao, pr, ar in ptrs:
                assert lib.bl_residual_linear(P(x.data_ptr()), po, ao, pr, ar, M, N, K,
                                              P(y.data_ptr()), wsp, wsb, stream) == 0

        ms_eager = timed(torch, sweep, max(2, steps // 4), 1)
        run, keep = graphed(torch, sweep)
        ms = timed(torch, run, max(2, steps // 4), 1)
        out[f"M{M}"] = dict(us_per_layer=ms * 1e3 / pool, us_per_layer_eager=ms_eager * 1e3 / pool,
                            gbs=pool * layer_bytes / (ms / 1e3) / 1e9, bytes_per_layer=layer_bytes,
                            graph=True)
    return out


# ------------------------------------------------------------------------------------------
# measured ceilings (ternary_weight_linear_amd/csrc/ceilings.hip)
# ------------------------------------------------------------------------------------------
def measured_ceilings(torch, dev):
    """Streaming HBM read of a 4 GiB buffer (16 x the 256 MB MALL) and an int8 matrix-core
    loop, both timed with HIP events on the launch stream; best of a few launch shapes."""
    import ctypes
    lib = ctypes.CDLL(CEIL_LIB)
    lib.bl_ceil_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.bl_ceil_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bl_ceil_mfma_i8_ops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.bl_ceil_mfma_i8_ops.restype = ctypes.c_double
    P = ctypes.c_void_p
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    lib.bl_ceil_stream_read_slices.argtypes = lib.bl_ceil_stream_read.argtypes
    best_read = 0.0
    read_grid = None
    # grid-strided reads, and one contiguous slice per workgroup with non-temporal loads
    shapes = [("grid-strided", lib.bl_ceil_stream_read, g) for g in (1024, 2048, 4096, 8192)]
    shapes += [("slices, nt", lib.bl_ceil_stream_read_slices, g) for g in (256, 512, 1024, 2048)]
    for kind, fn, grid in shapes:
        out = torch.zeros(grid, dtype=torch.int32, device=dev)
        stream = P(torch.cuda.current_stream().cuda_stream)
        ms = timed(torch, lambda: fn(P(buf.data_ptr()), nbytes, P(out.data_ptr()), grid, stream), 5, 2)
        gbs = nbytes / (ms / 1e3) / 1e9
        if gbs > best_read:
            best_read, read_grid = gbs, f"{kind}, {grid} workgroups"
    del buf
    best_mfma = 0.0
    mfma_grid = None
    iters = 4000
    for grid in (512, 1024, 2048):
        out = torch.empty(grid * 256 * 4, dtype=torch.int32, device=dev)
        stream = P(torch.cuda.current_stream().cuda_stream)
        ms = timed(torch, lambda: lib.bl_ceil_mfma_i8(iters, grid, P(out.data_ptr()), stream), 5, 2)
        tops = lib.bl_ceil_mfma_i8_ops(iters, grid) / (ms / 1e3) / 1e12
        if tops > best_mfma:
            best_mfma, mfma_grid = tops, grid
    return {"hbm_read_gbs": round(best_read, 1), "hbm_read_frac_spec": round(best_read / HBM_PEAK_GBS, 4),
            "hbm_read_kernel": f"stream_read_kernel / stream_read_slices_kernel, 4 GiB read once, best: {read_grid}",
            "int8_mfma_tops": round(best_mfma, 1), "int8_mfma_frac_spec": round(best_mfma / INT8_PEAK_TOPS, 4),
            "int8_mfma_kernel": f"mfma_i8_kernel (v_mfma_i32_16x16x64_i8, 8 independent accumulators "
                                f"per wave), {mfma_grid} workgroups of 4 waves"}


# ------------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ------------------------------------------------------------------------------------------
def _oracle_leg(synth, mats, budget_s):
    """Time the oracle's quantise + exact accumulate + rescale over (codes, x) pairs for about
    budget_s seconds; returns (repetitions, seconds)."""
    import oracle
    t0 = time.perf_counter()
    reps = 0
    while True:
        for codes, x in mats:
            q, gamma, _ = oracle.quant_act_int8(x)
            acc = oracle.acc_exact(q, codes)
            oracle.bitlinear_output(acc, gamma, synth.BETA_DIRECT)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            return reps, time.perf_counter() - t0


def cpu_baseline(synth, budget_s=6.0):
    """The CPU oracle as it stands, on bounded samples of three workloads: the headline leg
    (70B layer 0, first 512 rows of each linear, M = 1) with all host threads and with one,
    the 7B decode set (first 512 rows of each linear, M = 1) and the 3B prefill set (first
    64 rows of each linear, M = 512 tokens)."""
    import threadpoolctl
    def sample(linears, key_cfg, rows, M, x_keys):
        mats = []
        for mid, (name, N, K) in enumerate(linears):
            codes = synth.ternary_codes(synth.matrix_key(0, key_cfg, 0, mid), N, K, rows=np.arange(rows))
            mats.append((codes, synth.normal_fp16((M, K), *x_keys, mid)))
        return mats
    legs = {}
    threads_all = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    m70 = sample(synth.LLAMA70B_LINEARS, 5, 512, 1, (0, 5, 1000))
    for name, limit in (("70b_m1_all_threads", None), ("70b_m1_1_thread", 1)):
        with threadpoolctl.threadpool_limits(limits=limit):
            reps, dt = _oracle_leg(synth, m70, budget_s)
        legs[name] = {"gbs_packed": reps * sum(c.size for c, _ in m70) / 4 / dt / 1e9,
                      "threads": limit or int(threads_all), "reps": reps, "s": round(dt, 2)}
    m7 = sample(synth.LLAMA7B_LINEARS, 3, 512, 1, (0, 3, 2000))
    reps, dt = _oracle_leg(synth, m7, budget_s / 2)
    legs["7b_m1_all_threads"] = {"gbs_packed": reps * sum(c.size for c, _ in m7) / 4 / dt / 1e9,
                                 "threads": int(threads_all), "reps": reps, "s": round(dt, 2)}
    m3 = sample(synth.LLAMA3B_LINEARS, 4, 64, 512, (0, 4, 3000))
    reps, dt = _oracle_leg(synth, m3, budget_s / 2)
    legs["3b_m512_all_threads"] = {"tops": reps * sum(2 * 512 * c.size for c, _ in m3) / dt / 1e12,
                                   "threads": int(threads_all), "reps": reps, "s": round(dt, 2)}
    main = legs["70b_m1_all_threads"]
    return {"value": main["gbs_packed"], "unit": "GB/s", "cores": main["threads"], "kind": "oracle",
            "sample": "70B-shaped layer 0, first 512 rows of each of the 7 linears, M=1; oracle "
                      "quantise + exact accumulate + rescale, repeated for ~6 s; GB/s counts the 2-bit "
                      "packed bytes those rows would occupy. Legs: the same with one thread; 7B decode "
                      "set (512 rows per linear, M=1); 3B prefill set (64 rows per linear, M=512, int8 TOPS)",
            "legs": legs, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def bench_decode70b_stack(torch, tw, synth, dev, layers, M, steps, warmup):
    """The same pass (M <= 4) as ONE persistent launch over all 320 linears
    (bl_bitlinear_forward_stack): same activations, outputs and order as decode_pass, with a
    grid-wide wait between consecutive linears."""
    items, _, algo, wbytes, _ = decode_pass(torch, tw, synth, dev, layers, M)
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=dev)
    plan = tw.bl_stack_prepare([(it["x"], it["w"], beta, it["y"]) for it in items], M)
    count = len(items)
    ws = tw.workspace(dev, tw.bl_workspace_bytes(M, 64, 128))
    wsp, wsb = tw.ctypes.c_void_p(ws.data_ptr()), ws.numel()
    pp = tw.ctypes.c_void_p(plan.data_ptr())
    lib = tw._lib

    def full_pass():
        st = lib.bl_bitlinear_forward_stack(pp, count, M, wsp, wsb,
                                            tw.ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, tw._lib.bl_last_error()

    ms = timed(torch, full_pass, steps, warmup)
    status = tw.bl_stack_status(plan)
    assert status == 0, f"stack status {status}"
    return dict(ms_per_pass=ms, launches_per_pass=1, groups=count, algo_bytes=algo,
                weight_bytes=wbytes, tokens_per_s=M / (ms / 1e3), gbs=algo / (ms / 1e3) / 1e9,
                weight_gbs=wbytes / (ms / 1e3) / 1e9, graph=False, _plan=plan, _items=items)


def kernel_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, or None if it is missing or was taken from a different kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_prefill3b_m512_mfma.json")
GEMM_SOURCES = [os.path.join(ROOT, "ternary_weight_linear_amd", "csrc", f)
                for f in ("tern_mfma.hip", "bl_internal.h")]


def mfma_counters():
    """Matrix-core utilisation of the prefill GEMM from the committed rocprofv3 counter
    summary, or None if it is missing or was taken from different kernel sources."""
    try:
        t = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    if t.get("source_sha256") != h.hexdigest():
        return None
    return t.get("summary")


def kernel_source_hash():
    """sha256 over the dominant kernel's source files, in order."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path's multi-GPU "
                                   "sharding is a design note, not a measured configuration",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import synth
    import synth.gpu as sgpu
    import ternary_weight_linear_amd as tw

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        a.fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": a.numel()}))
        return

    if args.ceilings:
        print(json.dumps({"measured_ceilings": measured_ceilings(torch, dev)}))
        return

    if args.only in ("prefill3b", "decode7b", "decode7b_stack", "onebit", "residual"):
        fn = {"prefill3b": lambda: bench_prefill3b(torch, tw, synth, dev, args.steps, args.warmup),
              "decode7b": lambda: bench_decode7b(torch, tw, sgpu, synth, dev, args.steps, args.warmup),
              "decode7b_stack": lambda: bench_decode7b_stack(torch, tw, sgpu, synth, dev, args.steps, args.warmup),
              "onebit": lambda: bench_onebit(torch, tw, synth, dev, args.steps, args.warmup),
              "residual": lambda: bench_residual(torch, tw, synth, dev, args.steps, args.warmup)}[args.only]
        print(json.dumps({args.only: fn()}))
        return

    ceilings = None
    if not args.skip_extra:
        ceilings = measured_ceilings(torch, dev)
        log("measured ceilings:", json.dumps(ceilings))
    t0 = time.time()
    log("building the 70B-shaped packed stack (17.1 GB) ...")
    layers = build_stack70b(torch, tw, sgpu, synth, dev)
    log(f"stack ready: {stack_bytes(layers)} bytes in {time.time() - t0:.1f} s")
    extra = {}
    if args.only:
        res = {}
        if args.only.startswith("decode70b_m"):
            M = int(args.only.split("_m")[1])
            res = bench_decode70b(torch, tw, synth, dev, layers, M, args.steps, args.warmup,
                                  use_graph=not args.no_graph)
        elif args.only.startswith("mf_m"):
            M = int(args.only.split("_m")[1])
            layers_mf = repack_stack_mf(torch, tw, dev, layers)
            res = bench_decode70b_mf(torch, tw, synth, dev, layers_mf, M, args.steps, args.warmup,
                                     use_graph=not args.no_graph)
        elif args.only == "read_floor":
            res = read_floor_pass(torch, dev, layers, args.steps, args.warmup)
        elif args.only.startswith("stack_m"):
            M = int(args.only.split("_m")[1])
            res = bench_decode70b_stack(torch, tw, synth, dev, layers, M, args.steps, args.warmup)
            res = {k: v for k, v in res.items() if not k.startswith("_")}
        print(json.dumps({args.only: res}))
        return

    main_res = bench_decode70b(torch, tw, synth, dev, layers, 1, args.steps, args.warmup,
                               use_graph=not args.no_graph)
    log("decode70b M=1:", json.dumps(main_res))
    read_floor = None
    if not args.skip_extra:
        read_floor = read_floor_pass(torch, dev, layers, args.steps, args.warmup)
        log("the same pass as streaming reads only:", json.dumps(read_floor))
    if not args.skip_extra:
        layers_mf = repack_stack_mf(torch, tw, dev, layers)
        r = bench_decode70b_mf(torch, tw, synth, dev, layers_mf, 1, args.steps, args.warmup)
        extra["decode70b_m1_mfma"] = {k: r[k] for k in ("ms_per_pass", "ms_per_pass_eager", "tokens_per_s", "gbs")}
        extra["decode70b_m1_mfma"]["weights"] = "T2-MF64"
        log("decode70b M=1, int8 matrix cores (T2-MF64 weights):", json.dumps(extra["decode70b_m1_mfma"]))
        r = bench_decode70b_stack(torch, tw, synth, dev, layers, 1, args.steps, args.warmup)
        extra["decode70b_m1_stack"] = {k: r[k] for k in ("ms_per_pass", "tokens_per_s", "gbs", "launches_per_pass")}
        del r
        log("decode70b M=1, one persistent launch:", json.dumps(extra["decode70b_m1_stack"]))
        for M in (8, 32, 64):
            r = bench_decode70b(torch, tw, synth, dev, layers, M, max(3, args.steps // 4), 1,
                                use_graph=not args.no_graph)
            extra[f"decode70b_m{M}_t2pn"] = {k: r[k] for k in ("ms_per_pass", "ms_per_pass_eager", "tokens_per_s", "gbs")}
            log(f"decode70b M={M} (T2-PN-64 weights):", json.dumps(extra[f'decode70b_m{M}_t2pn']))
        for M in (8, 32, 64):
            r = bench_decode70b_mf(torch, tw, synth, dev, layers_mf, M, max(3, args.steps // 4), 1)
            extra[f"decode70b_m{M}"] = {k: r[k] for k in ("ms_per_pass", "tokens_per_s", "gbs")}
            extra[f"decode70b_m{M}"]["weights"] = "T2-MF64"
            log(f"decode70b M={M} (T2-MF64 weights):", json.dumps(extra[f'decode70b_m{M}']))
        del layers_mf
    del layers
    torch.cuda.empty_cache()
    if not args.skip_extra:
        extra["prefill3b_m512"] = bench_prefill3b(torch, tw, synth, dev, args.steps, args.warmup)
        log("prefill3b:", json.dumps(extra["prefill3b_m512"]))
        extra["decode7b_m1"] = bench_decode7b_stack(torch, tw, sgpu, synth, dev, args.steps, args.warmup)
        log("decode7b (32 layers, stacked, fused launches):", json.dumps(extra["decode7b_m1"]))
        extra["decode7b_m1_pool32"] = bench_decode7b(torch, tw, sgpu, synth, dev, args.steps, args.warmup)
        log("decode7b (7 GEMV launches per layer):", json.dumps(extra["decode7b_m1_pool32"]))
        extra["onebit4096_pool256"] = bench_onebit(torch, tw, synth, dev, args.steps, args.warmup)
        extra["residual4096_pool128"] = bench_residual(torch, tw, synth, dev, args.steps, args.warmup)
        log("onebit:", json.dumps(extra["onebit4096_pool256"]))
        extra["svid4096"] = bench_svid(torch, tw, synth, dev, args.steps, args.warmup)
        log("svid:", json.dumps(extra["svid4096"]))

    ms = main_res["ms_per_pass"]
    launches = main_res["launches_per_pass"]
    # algorithmic bytes per launch: packed weights + fp16 x + fp32 y, averaged over the pass;
    # the launch duration is the pass time (HIP events on the launch stream) per launch, so
    # it includes the gap between consecutive graph launches
    per_launch_bytes = main_res["algo_bytes"] / launches
    avg_launch_s = ms / 1e3 / launches
    achieved = per_launch_bytes / avg_launch_s / 1e9
    traffic = kernel_traffic()
    roofline_gemm = None
    if "prefill3b_m512" in extra:
        pf = extra["prefill3b_m512"]
        roofline_gemm = {"bound": "mfma", "kernel": "tern_mfq_kernel<FM, 4> (staged-q int8 MFMA, T2-MF64, four bands per workgroup)",
                         "workload": "3B-shaped prefill, M=512: q|k|v 512x9600x3200, o 512x3200x3200, "
                                     "gate|up 512x17280x3200, down 512x3200x8640",
                         "achieved": round(pf["tops_gemms"], 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(pf["tops_gemms"] / INT8_PEAK_TOPS, 4),
                         "int8_ops_per_pass": pf["int8_ops"], "ms_gemms": round(pf["ms_gemms_only"], 4),
                         "mfma_counters": mfma_counters()}
        if ceilings:
            roofline_gemm["frac_measured_peak"] = round(pf["tops_gemms"] / ceilings["int8_mfma_tops"], 4)
    out = {
        "metric": METRIC,
        "value": round(main_res["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 activations x ternary weights, int32 accumulate, fp32 out",
        "data": "synthetic: seeded counter-based ternary codes (P(0)=P(+-1)=1/3), fp16 N(0,1) activations",
        "config": {"workload": "b1.58 70B-shaped full stack decode, M=1 token, 80 layers x "
                               "(qkv 10240x8192, o 8192x8192, gate|up 57344x8192, down 8192x28672)",
                   "weights": "T2-PN-64 (2 bits per weight)",
                   "weight_bytes_per_pass": main_res["weight_bytes"],
                   "algorithmic_bytes_per_pass": main_res["algo_bytes"],
                   "launches_per_pass": main_res["launches_per_pass"],
                   "tokens_per_s": round(main_res["tokens_per_s"], 2),
                   "frac_hbm_peak": round(main_res["gbs"] / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm",
                     "kernel": "gemv_fused_kernel<1, GL> (quantise + add-only GEMV, T2-PN-64)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": round(per_launch_bytes, 1),
                     "frac_measured_peak": (round(achieved / ceilings["hbm_read_gbs"], 4)
                                            if ceilings else None),
                     # the pass against the same launches doing nothing but read their weights
                     "launch_read_floor_ms": round(read_floor["ms_per_pass"], 4) if read_floor else None,
                     "frac_launch_read_floor": (round(read_floor["ms_per_pass"] / ms, 4)
                                                if read_floor else None)},
        "roofline_gemm": roofline_gemm,
        "measured_ceilings": ceilings,
        "launch_read_floor": read_floor,
        "extra": extra,
    }
    if not args.skip_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
