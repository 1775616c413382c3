"""The library's launches under HIP graph capture (torch.cuda.graph): a captured
forward of one bf16 linear and one packed W4A4 linear is replayed several times,
with eager work and synchronisations in between, and every replay must equal the
eager results bit for bit; the replayed outputs are also checked against the
oracle (the bf16 layer's per-element bound and the W4A4 layer's 5e-3 gate). The
entry points make no allocation and no attribute call while capturing once the
kernels have run eagerly."""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, make_layer, ulp_bf16

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    ops = gpu_lib
    d_bf = workloads.make_bf16_linear(300, 256, 200, kind="dit", seed=11)
    x_bf, w_bf, b_bf = dev_bf16(d_bf["x"]), dev_bf16(d_bf["W"]), dev_bf16(d_bf["bias"])
    d_q, layer = make_layer(dict(M=300, K=256, N=192, R=32, kind="dit", seed=12))
    layer = layer.packed()
    x_q = dev_bf16(d_q["x"])
    M = 300
    y_bf = torch.empty((M, 200), dtype=torch.bfloat16, device="cuda")
    y_q = torch.empty((M, 192), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, ops.linear_workspace_bytes(M, 192, 256, 32)), dtype=torch.uint8, device="cuda")

    def forward():
        ops.linear_bf16(x_bf, w_bf, b_bf, y=y_bf)
        ops.linear_w4a4(x_q, layer, y=y_q, workspace=ws)

    forward()
    torch.cuda.synchronize()
    ref_bf = y_bf.clone()
    ref_q = y_q.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward()
    torch.cuda.synchronize()

    other = workloads.make_bf16_linear(300, 256, 200, kind="dit", seed=13)
    x_other = dev_bf16(other["x"])
    for rep in range(4):
        y_bf.fill_(0)
        y_q.fill_(0)
        ws.fill_(0x5A)
        ops.linear_bf16(x_other, w_bf, None, y=torch.empty_like(y_bf))   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_bf.view(torch.int16), ref_bf.view(torch.int16)), f"bf16 output, replay {rep}"
        assert torch.equal(y_q.view(torch.int16), ref_q.view(torch.int16)), f"W4A4 output, replay {rep}"
    # the replayed outputs against the oracle
    y64_bf, _ = S.linear_bf16(d_bf["x"], d_bf["W"], d_bf["bias"])
    got_bf = F.bf16_to_f64(host_bits(y_bf))
    xa, wa = np.abs(F.bf16_to_f64(d_bf["x"])), np.abs(F.bf16_to_f64(d_bf["W"]))
    bound = ulp_bf16(y64_bf) + 2 * (256 + 2) * 2.0 ** -24 * (xa @ wa.T + np.abs(F.bf16_to_f64(d_bf["bias"])))
    assert np.all(np.abs(got_bf - y64_bf) <= bound), "bf16 replay beyond the oracle bound"
    y64_q, _, _, _ = S.linear_w4a4(d_q["x"], d_q["smooth"], d_q["qweight"], d_q["wscales"], d_q["wcscales"],
                                   d_q["wtscale"], d_q["proj_down"], d_q["proj_up"], d_q["bias"])
    assert S.normwise_rel_err(F.bf16_to_f64(host_bits(y_q)), y64_q) <= 5e-3
