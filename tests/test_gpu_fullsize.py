"""Full-size parity in the launch configuration the benchmark times.

One layer of the 70B-shaped stack is built exactly as bench.py builds it (GPU counter-based
codes, packed into stacked q|k|v and gate|up buffers, repacked into T2-MF64) and run through
the same entry points (the fused quantise + add-only GEMV at M = 1, the benchmark's default
pass; the fused T2-MF64 matrix-core decode at M = 1, 2, its comparison line; quantiser +
int8-MFMA products at M = 8 and 64). Sampled output rows are recomputed by the oracle from
codes regenerated on the host. Graph-replayed passes are checked bit-for-bit against eager
launches over several replays."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sgpu
import ternary_weight_linear_amd as tw
from tests.gpu_util import DEV, assert_rel, host, say

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
def layer0():
    say("fullsize: building layer 0 of the 70B-shaped stack")
    return _layer(0)


@pytest.mark.parametrize("M", [1, 8, 64])
def test_stack_layer_sampled_rows(layer0, M):
    beta = torch.tensor([float(synth.BETA_DIRECT)], dtype=torch.float32, device=DEV)
    for gi, (gname, buf, N, K, parts) in enumerate(layer0):
        say("fullsize", gname, "M", M, "N", N, "K", K)
        x16 = synth.normal_fp16((M, K), 0, 5, 1000, gi)
        x = torch.from_numpy(x16).to(DEV)
        if M <= 2:
            y = tw.bl_bitlinear_forward(x, buf, beta, N, path=tw.BL_PATH_GEMV)
        else:
            q, gamma, _, _ = tw.bl_quant_act_int8(x, want_rowsum=False, want_planes=False)
            y = tw.bl_bitlinear_gemm(q, gamma, buf, beta, N)
        ids, yref = _sampled_reference(x16, parts, K, 48, seed=gi + 10 * M)
        assert_rel(host(y)[:, ids], yref)


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
