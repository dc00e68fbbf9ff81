"""Full-size parity for the 70B-shaped stack (80 layers x q 8192x8192, k/v 1024x8192,
o 8192x8192, gate/up 28672x8192, down 8192x28672), in the launch configurations the
benchmark times.

The stack is built exactly as bench.py builds it (GPU counter-based codes, packed into
stacked q|k|v and gate|up T2-PN-64 buffers, repacked into T2-MF64 where the matrix-core
lines need it). The checks follow the stack's parity budget:

* layers 0 and 79 in full: every row of all seven matrices at M = 1, 8, 32 and 64, the
  int32 accumulators bit-exact against the oracle (acc-returning entry points on the same
  weights) and the fp32 outputs of the benchmark's own launches within 1e-3 of the oracle
  on every element;
* every layer: 128 seeded rows per matrix at M = 1, 8, 32 and 64 through a graph-replayed
  pass of the benchmark's launches, int32 and fp32 as above;
* the persistent whole-stack launch, graph replays against eager launches.

The oracle regenerates every code it uses on the host (synth.ternary_codes, the host twin
of the GPU generator)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sgpu
import ternary_weight_linear_amd as tw
from tests.gpu_util import DEV, assert_rel, dev, host, say

pytestmark = pytest.mark.gpu

GROUPS = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gateup", ["gate", "up"]), ("down", ["down"])]
SHAPES = {n: (N, K) for n, N, K in synth.LLAMA70B_LINEARS}
MIDS = {n: i for i, (n, _, _) in enumerate(synth.LLAMA70B_LINEARS)}


def _layer(layer):
    out = []
    for gname, members in GROUPS:
        K = SHAPES[members[0]][1]
        Ntot = sum(SHAPES[m][0] for m in members)
        buf = torch.empty(Ntot * K // 4, dtype=torch.uint8, device=DEV)
        off = 0
        parts = []
        for m in members:
            N = SHAPES[m][0]
            key = synth.matrix_key(0, 5, layer, MIDS[m])
            codes = sgpu.ternary_codes(key, N, K, DEV)
            packed = tw.bl_pack_ternary(codes)
            buf[off: off + packed.numel()].copy_(packed)
            parts.append((m, key, N, off // (K // 4)))     # name, key, rows, first stacked row
            off += packed.numel()
            del codes
        out.append((gname, buf, Ntot, K, parts))
    torch.cuda.synchronize()
    return out


def _sampled_reference(x16, parts, K, rows_per_member, seed):
    """Oracle outputs for sampled stacked rows: returns (stacked row ids, y_ref [M, rows])."""
    rg = synth.rng(seed, 7)
    q, gamma, _ = oracle.quant_act_int8(x16)
    ids, refs = [], []
    for name, key, N, first in parts:
        rows = np.sort(rg.choice(N, size=min(rows_per_member, N), replace=False))
        codes = synth.ternary_codes(key, N, K, rows=rows)
        acc = oracle.acc_exact(q, codes)
        refs.append(oracle.bitlinear_output(acc, gamma, synth.BETA_DIRECT))
        ids.append(first + rows)
    return np.concatenate(ids), np.concatenate(refs, axis=1)


@pytest.fixture(scope="module")
def stack70b():
    say("fullsize: building the 80-layer 70B-shaped stack (17.1 GB)")
    layers = []
    for layer in range(synth.LLAMA70B_LAYERS):
        layers.append(_layer(layer))
        if layer % 20 == 19:
            say("fullsize: built", layer + 1, "layers")
    return layers


@pytest.fixture(scope="module")
def layer0(stack70b):
    return stack70b[0]


BENCH_M = [1, 8, 32, 64]
ACC_CHUNK = 4096            # oracle rows per fp64 product (bounds host memory)


def _bench_x(layer, gi, M):
    """The benchmark's activations for (layer, group) at M tokens."""
    return synth.normal_fp16((M, K_OF[gi]), 0, 5, 1000 + layer, gi)


K_OF = [SHAPES[members[0]][1] for _, members in GROUPS]


def _gpu_bench_launch(x, buf, wmf, beta, N, M, out=None):
    """The launch the benchmark times for one group: the fused quantise + add-only GEMV at
    M <= 2 (T2-PN-64), bl_bitlinear_forward_mf (T2-MF64) above."""
    if M <= 2:
        return tw.bl_bitlinear_forward(x, buf, beta, N, path=tw.BL_PATH_GEMV, out=out)
    return tw.bl_bitlinear_forward_mf(x, wmf, beta, N, out=out)


def _gpu_acc(x, buf, wmf, N, K, M):
    """int32 accumulators for the same weights from an acc-returning entry point: the
    add-only GEMV (X8-64 planes) at M <= 2, the T2-MF64 matrix-core product above; the
    quantiser's outputs are returned for the bit-exact check."""
    q, gamma, rowsum, planes = tw.bl_quant_act_int8(x, want_planes=M <= 2)
    if M <= 2:
        acc = tw.bl_bitlinear_acc_i32(buf, N, K, planes=planes, path=tw.BL_PATH_GEMV)
    else:
        _, acc = tw.bl_bitlinear_gemm_mf(q, gamma, rowsum, wmf, None, N, want_y=False, want_acc=True)
    return acc, q, gamma, rowsum


@pytest.mark.parametrize("layer", [0, 79])
@pytest.mark.parametrize("gi", [0, 1, 2, 3])
def test_full_layer_every_row(stack70b, layer, gi):
    """Every row of the group's matrices, M = 1, 8, 32, 64: q, gamma and row sums bit-exact,
    int32 accumulators bit-exact (and the T2-PN-64 matrix-core product's too), fp32 outputs
    of the benchmark's launch within 1e-3 everywhere."""
    gname, buf, N, K, parts = stack70b[layer][gi]
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    say("fullsize every row: layer", layer, gname, N, "x", K, "(host codes)")
    codes = np.concatenate([synth.ternary_codes(key, Nm, K) for _, key, Nm, _ in parts])
    xs = {M: _bench_x(layer, gi, M) for M in BENCH_M}
    qs = {M: oracle.quant_act_int8(xs[M]) for M in BENCH_M}
    qall = np.concatenate([qs[M][0] for M in BENCH_M])
    ref_all = np.concatenate([oracle.acc_exact(qall, codes[r:r + ACC_CHUNK])
                              for r in range(0, N, ACC_CHUNK)], axis=1)
    del codes
    wmf = tw.bl_repack_ternary_mf(buf, N, K)
    r0 = 0
    for M in BENCH_M:
        say("fullsize every row: layer", layer, gname, "M", M)
        rq, rg, rrow = qs[M]
        ref_acc = ref_all[r0:r0 + M]
        r0 += M
        x = dev(xs[M])
        acc, q, gamma, rowsum = _gpu_acc(x, buf, wmf, N, K, M)
        assert np.array_equal(host(q), rq) and np.array_equal(host(rowsum), rrow)
        assert np.array_equal(host(gamma).view(np.uint32), rg.view(np.uint32))
        assert np.array_equal(host(acc), ref_acc), f"int32 accumulators, M = {M}"
        if M > 2:
            acc_pn = tw.bl_bitlinear_acc_i32(buf, N, K, q=q, path=tw.BL_PATH_GEMM)
            assert np.array_equal(host(acc_pn), ref_acc), f"T2-PN-64 product, M = {M}"
        y = _gpu_bench_launch(x, buf, wmf, beta, N, M)
        assert_rel(host(y), oracle.bitlinear_output(ref_acc, rg, synth.BETA_DIRECT))
    del wmf


_SAMPLED = {}


def _sampled_codes(layer, parts, K):
    """128 seeded rows of every matrix of a group: (stacked row ids, host codes)."""
    key0 = (layer, parts[0][0])
    if key0 not in _SAMPLED:
        ids, cs = [], []
        for name, key, N, first in parts:
            rows = np.sort(synth.rng(0, 8, layer, MIDS[name]).choice(N, size=min(128, N), replace=False))
            cs.append(synth.ternary_codes(key, N, K, rows=rows))
            ids.append(first + rows)
        _SAMPLED[key0] = (np.concatenate(ids), np.concatenate(cs))
    return _SAMPLED[key0]


@pytest.mark.parametrize("M", BENCH_M)
def test_all_layers_sampled_rows(stack70b, M):
    """All 80 layers through one graph-replayed pass of the benchmark's launches (the
    configuration it times), then 128 seeded rows of every matrix: int32 accumulators
    bit-exact and fp32 outputs within 1e-3 of the oracle."""
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    items = []
    for layer, lg in enumerate(stack70b):
        for gi, (gname, buf, N, K, parts) in enumerate(lg):
            x16 = _bench_x(layer, gi, M)
            wmf = tw.bl_repack_ternary_mf(buf, N, K) if M > 2 else None
            y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
            items.append((layer, gi, x16, dev(x16), buf, wmf, N, K, parts, y))
    say("fullsize all layers M", M, "launches", len(items))

    def run():
        for layer, gi, x16, x, buf, wmf, N, K, parts, y in items:
            _gpu_bench_launch(x, buf, wmf, beta, N, M, out=y)

    run()                                   # allocates the workspace outside the capture
    torch.cuda.synchronize()
    for it in items:
        it[-1].fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    for layer, gi, x16, x, buf, wmf, N, K, parts, y in items:
        if gi == 0 and layer % 16 == 0:
            say("fullsize all layers M", M, "checking layer", layer)
        ids, codes = _sampled_codes(layer, parts, K)
        rq, rg, _ = oracle.quant_act_int8(x16)
        ref_acc = oracle.acc_exact(rq, codes)
        acc, _, _, _ = _gpu_acc(x, buf, wmf, N, K, M)
        assert np.array_equal(host(acc)[:, ids], ref_acc), (layer, gi, M)
        assert_rel(host(y)[:, ids], oracle.bitlinear_output(ref_acc, rg, synth.BETA_DIRECT))
    del g, items


def test_stack_layer_graph_replays_match_eager(layer0):
    """Capture the layer's four fused launches in a HIP graph; every replay, with eager
    work and synchronisations between replays, must reproduce the eager outputs bitwise."""
    say("fullsize: graph replay")
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    xs = [torch.from_numpy(synth.normal_fp16((1, K), 0, 5, 2000, gi)).to(DEV)
          for gi, (_, _, _, K, _) in enumerate(layer0)]
    ys = [torch.empty((1, N), dtype=torch.float32, device=DEV) for (_, _, N, _, _) in layer0]

    def run():
        for (gname, buf, N, K, parts), x, y in zip(layer0, xs, ys):
            tw.bl_bitlinear_forward(x, buf, beta, N, path=tw.BL_PATH_GEMV, out=y)

    run()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int32), e.view(torch.int32)), f"replay {rep} differs"
        tmp = torch.randn(1 << 20, device=DEV).sum()       # eager work between replays
        torch.cuda.synchronize()
        del tmp


@pytest.mark.parametrize("M", [1, 2])
def test_stack_kernel_full_size(layer0, M):
    """The persistent whole-stack launch (the benchmark's launch configuration) on the 70B
    layer's four groups three times over (12 linears): every output bitwise equal to one
    bl_bitlinear_forward call per linear, sampled rows against the oracle."""
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    lins = []
    for rep in range(3):
        for gi, (gname, buf, N, K, parts) in enumerate(layer0):
            x16 = synth.normal_fp16((M, K), 0, 5, 3000 + rep, gi)
            y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
            lins.append((gname, x16, torch.from_numpy(x16).to(DEV), buf, N, K, parts, y))
    say("fullsize stack kernel M", M, "linears", len(lins))
    plan = tw.bl_stack_prepare([(x, buf, beta, y) for _, _, x, buf, _, _, _, y in lins], M)
    tw.bl_bitlinear_forward_stack(plan, len(lins), M)
    assert tw.bl_stack_status(plan) == 0
    for i, (gname, x16, x, buf, N, K, parts, y) in enumerate(lins):
        ref = tw.bl_bitlinear_forward(x, buf, beta, N, path=tw.BL_PATH_GEMV)
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), f"linear {i} ({gname})"
        if i < 4:
            ids, yref = _sampled_reference(x16, parts, K, 16, seed=100 + i + 10 * M)
            assert_rel(host(y)[:, ids], yref)


@pytest.mark.parametrize("M", [1, 2, 8, 64])
def test_mf_layer_sampled_rows(layer0, M):
    """The 70B layer repacked into T2-MF64 (the benchmark's matrix-core decode line at M = 1,
    its batched decode at M = 8, 64): sampled rows against the oracle; at M <= 2 every output
    bitwise equal to the add-only GEMV from T2-PN-64 (same integers, same epilogue)."""
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    for gi, (gname, buf, N, K, parts) in enumerate(layer0):
        say("fullsize mf", gname, "M", M)
        wmf = tw.bl_repack_ternary_mf(buf, N, K)
        x16 = synth.normal_fp16((M, K), 0, 5, 4000, gi)
        x = torch.from_numpy(x16).to(DEV)
        y = tw.bl_bitlinear_forward_mf(x, wmf, beta, N)
        ids, yref = _sampled_reference(x16, parts, K, 32, seed=200 + gi + 10 * M)
        assert_rel(host(y)[:, ids], yref)
        if M <= 2:
            ref = tw.bl_bitlinear_forward(x, buf, beta, N, path=tw.BL_PATH_GEMV)
            assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), gname
        del wmf


def test_mf_layer_graph_replays_match_eager(layer0):
    """The benchmark's matrix-core decode line for one layer: four fused T2-MF64 decode
    launches captured in a HIP graph; every replay, with eager work and synchronisations
    between replays, must reproduce the eager outputs bitwise."""
    say("fullsize: mf graph replay")
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    wmfs = [tw.bl_repack_ternary_mf(buf, N, K) for (_, buf, N, K, _) in layer0]
    xs = [torch.from_numpy(synth.normal_fp16((1, K), 0, 5, 5000, gi)).to(DEV)
          for gi, (_, _, _, K, _) in enumerate(layer0)]
    ys = [torch.empty((1, N), dtype=torch.float32, device=DEV) for (_, _, N, _, _) in layer0]

    def run():
        for (gname, buf, N, K, parts), w, x, y in zip(layer0, wmfs, xs, ys):
            tw.bl_bitlinear_forward_mf(x, w, beta, N, out=y)

    run()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int32), e.view(torch.int32)), f"replay {rep} differs"
        tmp = torch.randn(1 << 20, device=DEV).sum()       # eager work between replays
        torch.cuda.synchronize()
        del tmp
    del wmfs
