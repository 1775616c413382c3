"""GPU parity of svdq_linear_bf16 (the linears a mixed-precision NVFP4 model keeps in
bf16; blog page "Z-Image NVFP4 ...", variant table) against the oracle's float64
y = x @ W^T + bias.

Gate: normwise relative error <= 5e-3 on the bf16 output. Also asserted, for every
element, the bound that follows from the arithmetic: one bf16 ulp of output
rounding (the fp32 value may cross a binade) plus 2 (K + 2) 2^-24 of
|x| @ |W|^T + |bias| (fp32 accumulation of exact products, the bias add); and at
least 99% of the elements equal the oracle's correctly rounded bf16 value (only
values within the fp32 error of a rounding midpoint may differ, by one ulp).
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, ulp_bf16

pytestmark = pytest.mark.gpu


def check_rows(d, y_bits, rows):
    x = d["x"][rows]
    y64, yb = S.linear_bf16(x, d["W"], d["bias"])
    got = F.bf16_to_f64(y_bits[rows])
    err = S.normwise_rel_err(got, y64)
    assert err <= 5e-3, err
    mag = np.abs(F.bf16_to_f64(x)) @ np.abs(F.bf16_to_f64(d["W"])).T
    if d["bias"] is not None:
        mag = mag + np.abs(F.bf16_to_f64(d["bias"]))[None, :]
    bound = ulp_bf16(y64) + 2 * (d["K"] + 2) * 2.0 ** -24 * mag
    bad = np.argwhere(np.abs(got - y64) > bound)
    assert bad.size == 0, f"{len(bad)} elements beyond the arithmetic bound, first {bad[:3].tolist()}"
    exact = float(np.mean(y_bits[rows] == yb))
    assert exact >= 0.99, exact
    return err, exact


def run(gpu_lib, d):
    x = dev_bf16(d["x"])
    w = dev_bf16(d["W"])
    b = dev_bf16(d["bias"]) if d["bias"] is not None else None
    y = gpu_lib.linear_bf16(x, w, b)
    torch.cuda.synchronize()
    return host_bits(y)


@pytest.mark.parametrize("M,K,N,bias", [
    (64, 256, 128, True),
    (300, 336, 200, True),      # K % 64 = 16: zero-filled last panel; ragged M and N
    (257, 64, 321, True),       # one K panel; N % 8 != 0 (scalar stores)
    (513, 1024, 520, False),    # no bias; 3 row blocks
    (1, 16, 1, True),           # smallest problem
    (5, 48, 13, True),
    (40, 3840, 8, True),
    (130, 128, 200, True),      # two K panels: one pass of the pipelined loop
    (70, 80, 96, False),        # two panels, the second zero-filled past K
    (33, 192, 264, True),       # three panels; ragged N
])
def test_bf16_linear_small(gpu_lib, M, K, N, bias):
    d = workloads.make_bf16_linear(M, K, N, kind="dit", seed=M * 7 + N, with_bias=bias)
    y_bits = run(gpu_lib, d)
    check_rows(d, y_bits, np.arange(M))


@pytest.mark.parametrize("backend", ["hip", "blaslt", "auto"])
@pytest.mark.parametrize("K,N", [(3840, 11520), (3840, 3840), (3840, 10240), (10240, 3840)])
def test_bf16_linear_dit_shapes_sampled(gpu_lib, K, N, backend, monkeypatch):
    """The sweep's bf16 layer shapes at M = 4096 (qkv, out, w1/w3, w2): sampled rows
    from every row block, including tile edges and the last row; with the
    hand-written kernel forced, hipBLASLt forced, and the library's own choice."""
    if backend != "auto":
        monkeypatch.setenv("SVDQ_BF16_GEMM", backend)
    M = 4096
    d = workloads.make_bf16_linear(M, K, N, kind="dit", seed=5000 + K + N)
    y_bits = run(gpu_lib, d)
    rng = np.random.default_rng(K + N)
    rows = np.unique(np.concatenate([[0, 255, 256, 1023, M - 1], rng.choice(M, 11, replace=False)]))
    check_rows(d, y_bits, rows)


def test_bf16_linear_2048px_sampled(gpu_lib):
    """M = 16896 (2048px image + text tokens), out projection, ragged last row block."""
    M, K, N = workloads.M_2048, 3840, 3840
    d = workloads.make_bf16_linear(M, K, N, kind="dit", seed=77)
    y_bits = run(gpu_lib, d)
    rows = np.array([0, 4095, 16383, 16384, M - 2, M - 1])
    check_rows(d, y_bits, rows)


def test_bf16_linear_wide_tile_ragged_sampled(gpu_lib):
    """M = 4000, N = 4200, K = 336: 224 tiles of 256 x 320 (one round on 256 CUs) against
    272 of 256 x 256, so the launcher takes the 320-wide tile with its plain loop; both
    edges are ragged (160 rows, 40 columns past the last full tile) and the last K
    panel is zero-filled past K."""
    M, K, N = 4000, 336, 4200
    d = workloads.make_bf16_linear(M, K, N, kind="dit", seed=4242)
    y_bits = run(gpu_lib, d)
    rows = np.array([0, 255, 256, 3839, 3840, 3998, 3999])
    check_rows(d, y_bits, rows)


def test_bf16_linear_into_given_output_is_deterministic(gpu_lib):
    d = workloads.make_bf16_linear(256, 512, 384, kind="dit", seed=3)
    x, w, b = dev_bf16(d["x"]), dev_bf16(d["W"]), dev_bf16(d["bias"])
    y = torch.full((256, 384), 7.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.linear_bf16(x, w, b, y=y)
    y2 = gpu_lib.linear_bf16(x, w, b)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    check_rows(d, host_bits(y), np.arange(256))


def test_bf16_linear_empty(gpu_lib):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    y = gpu_lib.linear_bf16(x, w)
    assert y.shape == (0, 32)


def test_bf16_linear_rounding_bit_exact(gpu_lib):
    """x and W of small dyadic values and biases of 256, 1024, -512 or 0: every fp32
    partial sum is exact and many results sit on bf16 rounding ties, so the output must
    equal the oracle's round-to-nearest-even of its float64 value bit for bit."""
    rng = np.random.default_rng(4200)
    M, K, N = 70, 208, 90
    d = dict(M=M, K=K, N=N,
             x=F.f64_to_bf16(rng.choice([0.0, 0.5, -1.0, 1.5, 2.0, -0.25], size=(M, K))),
             W=F.f64_to_bf16(rng.choice([0.0, 1.0, -0.5, 0.75, -2.0], size=(N, K))),
             bias=F.f64_to_bf16(rng.choice([256.0, 1024.0, -512.0, 0.0], size=N)))
    y64, yb = S.linear_bf16(d["x"], d["W"], d["bias"])
    ties = np.sum(np.abs(y64 / ulp_bf16(y64) % 1 - 0.5) < 1e-12)
    assert ties > 50, ties
    assert np.array_equal(run(gpu_lib, d), yb)


@pytest.mark.parametrize("M,K,N,bias", [(300, 336, 200, True), (257, 64, 321, False), (1, 16, 1, True)])
def test_bf16_linear_blaslt_small(gpu_lib, M, K, N, bias, monkeypatch):
    """hipBLASLt forced on ragged shapes, with and without bias: the operand
    transposition and the bias epilogue give the same checks as the kernel."""
    monkeypatch.setenv("SVDQ_BF16_GEMM", "blaslt")
    d = workloads.make_bf16_linear(M, K, N, kind="dit", seed=M * 11 + N, with_bias=bias)
    y_bits = run(gpu_lib, d)
    check_rows(d, y_bits, np.arange(M))


def test_bf16_linear_blaslt_graph_replays(gpu_lib, monkeypatch):
    """hipBLASLt's product captured in a graph after an eager call made its plan:
    every replay (with other eager work between) equals the eager output bit for
    bit, and a shape first seen under capture falls back to the kernel and is
    still within the parity checks."""
    monkeypatch.setenv("SVDQ_BF16_GEMM", "blaslt")
    d = workloads.make_bf16_linear(300, 256, 200, kind="dit", seed=17)
    d2 = workloads.make_bf16_linear(96, 128, 72, kind="dit", seed=18)
    x, w, b = dev_bf16(d["x"]), dev_bf16(d["W"]), dev_bf16(d["bias"])
    x2, w2, b2 = dev_bf16(d2["x"]), dev_bf16(d2["W"]), dev_bf16(d2["bias"])
    y = torch.empty((300, 200), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((96, 72), dtype=torch.bfloat16, device="cuda")
    gpu_lib.linear_bf16(x, w, b, y=y)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.linear_bf16(x, w, b, y=y)
        gpu_lib.linear_bf16(x2, w2, b2, y=y2)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        y2.zero_()
        gpu_lib.linear_bf16(x2, w2, None, y=torch.empty_like(y2))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
        check_rows(d2, host_bits(y2), np.arange(96))
