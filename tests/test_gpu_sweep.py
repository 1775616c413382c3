"""The mixed-precision sweep forward as a whole against the oracle: the 150 linears of
one forward at M = 4096 (30 blocks x {qkv, out, w1, w3, w2}; the "Ultra" variant of the
blog page "Z-Image NVFP4 ...", variant table, keeps qkv/out and blocks 0-4 and 25-29 in
bf16, the other 60 linears are SVDQuant W4A4 NVFP4), built exactly as the sweep benchmark
builds them (device-drawn seeded inputs), run eagerly and as one captured HIP graph with one
shared workspace, as the benchmark runs it.

Checks:
- the graph replay equals the eager forward bit for bit on every layer;
- every layer's output on a sample of rows x columns (first and last of each, plus seeded
  picks) against the oracle: linear_bf16 for the bf16 layers, linear_w4a4 for the W4A4
  layers, whose NVFP4 weight rows the oracle quantises itself from the pre-quantisation bf16
  weight (and which must equal the device's codes and scales for those rows bit for bit);
- normwise relative error <= 5e-3 on the sample, and every sampled element within the
  per-element bound of its arithmetic (as in the per-layer tests).
"""

import numpy as np
import pytest
import torch

import bench
import workloads
from oracle import formats as F
from oracle import repack as P
from oracle import svdq as S
from tests.gpu_util import host_bits, ulp_bf16

pytestmark = pytest.mark.gpu

M, R = workloads.SWEEP_M, workloads.SWEEP_R
N_ROWS, N_COLS = 6, 24


def _bits(t):
    return host_bits(t.contiguous())


@pytest.fixture(scope="module")
def sweep(gpu_lib):
    ops = gpu_lib
    dev = torch.device("cuda:0")
    built, acts = bench.sweep_build(dev, 1, keep_prequant=True)
    xs = acts[0]
    ys = [torch.empty((M, e["N"]), dtype=torch.bfloat16, device=dev) for e in built]
    ws = torch.empty(max(ops.linear_workspace_bytes(M, e["N"], e["K"], R) for e in built
                         if e["precision"] == "w4a4"), dtype=torch.uint8, device=dev)

    def forward():
        for li, e in enumerate(built):
            if e["precision"] == "bf16":
                ops.linear_bf16(xs[li], e["W"], e["b"], y=ys[li])
            else:
                ops.linear_w4a4(xs[li], e["layer"], y=ys[li], workspace=ws)

    forward()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward()
    torch.cuda.synchronize()
    for y in ys:
        y.fill_(0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    same = [torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ys, eager)]
    del eager
    return dict(built=built, xs=xs, ys=ys, same=same)


def _sample(li, n, size):
    rng = np.random.default_rng(9100 + li)
    picks = rng.choice(size, size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, size - 1], picks]))


def test_graph_replay_equals_eager(sweep):
    bad = [i for i, ok in enumerate(sweep["same"]) if not ok]
    assert not bad, f"layers {bad} differ between the graph replay and the eager forward"


@pytest.mark.parametrize("block", range(workloads.SWEEP_BLOCKS))
def test_block_against_oracle(sweep, block):
    built = sweep["built"]
    for li, e in enumerate(built):
        if e["block"] != block:
            continue
        K, N = e["K"], e["N"]
        rows, cols = _sample(li, N_ROWS, M), _sample(li + 500, N_COLS, N)
        x = _bits(sweep["xs"][li][torch.from_numpy(rows).cuda()])
        got = F.bf16_to_f64(_bits(sweep["ys"][li])[rows][:, cols])
        where = f"block {block} {e['name']} ({e['precision']}, K={K}, N={N})"
        if e["precision"] == "bf16":
            W = _bits(e["W"][torch.from_numpy(cols).cuda()])
            b = _bits(e["b"])[cols]
            y64, _ = S.linear_bf16(x, W, b)
            xa, wa = np.abs(F.bf16_to_f64(x)), np.abs(F.bf16_to_f64(W))
            bound = ulp_bf16(y64) + 2 * (K + 2) * 2.0 ** -24 * (xa @ wa.T + np.abs(F.bf16_to_f64(b)))
        else:
            lay = e["layer"]
            idx = torch.from_numpy(cols).cuda()
            Wp = _bits(e["Wp"][idx])
            qw, sw = S.quantize_act(Wp, F.f64_to_bf16(np.ones(K)))
            # the device's codes and scales of those weight rows, from the packed buffer
            dq, ds = P.unpack(lay.weight.cpu().numpy(), N, K)
            assert np.array_equal(dq[cols], qw) and np.array_equal(ds[:, cols], sw), f"{where}: weight codes"
            sm = _bits(lay.smooth)
            wc, wt = _bits(lay.wcscales)[cols], _bits(lay.wtscale)
            pd, pu, b = _bits(lay.proj_down), _bits(lay.proj_up)[cols], _bits(lay.bias)[cols]
            y64, _, qa, sa = S.linear_w4a4(x, sm, qw, sw, wc, wt, pd, pu, b)
            alpha = np.abs(F.bf16_to_f64(wt)[0] * F.bf16_to_f64(wc))
            main_abs = np.abs(S.dequant(qa, sa)) @ np.abs(S.dequant(qw, sw)).T * alpha
            pu_abs = np.abs(F.bf16_to_f64(pu)).T
            bound = (ulp_bf16(y64) + (K / 16 + 3) * 2.0 ** -24 * main_abs
                     + 2.0 ** -8 * (np.abs(S.lowrank_down(x, pd)) @ pu_abs)
                     + (K + R + 2) * 2.0 ** -24 * ((np.abs(F.bf16_to_f64(x)) @ np.abs(F.bf16_to_f64(pd))) @ pu_abs))
        err = S.normwise_rel_err(got, y64)
        assert err <= 5e-3, f"{where}: normwise {err}"
        bad = np.argwhere(np.abs(got - y64) > bound)
        assert bad.size == 0, f"{where}: {len(bad)} sampled elements beyond the bound, first {bad[:3].tolist()}"
