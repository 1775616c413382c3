"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module is the only code shared by the oracle's tests and the GPU path's
tests and benchmark. It draws inputs and holds none of the layer's
arithmetic: no quantisation, no scale rule, no contraction.

No trained weights or datasets are available, so the tensors stand in for a
quantised diffusion transformer's linears with the shapes and value
distributions of the pages' 1024^2 and 2048px workloads (a DiT of width 3840
with fused QKV, FFN w1/w3/w2 of width 10240, rank-128 residual; model card
"nunchaku-z-image-turbo-svdq", tensor table, and the NVFP4 blog's layer
tables).

Recipe (numpy Generator(PCG64(seed)); draw order x, outlier channels, smooth,
W, wcscales, proj_down, proj_up, bias; W stays float32, everything else is
rounded to bf16 with round-to-nearest-even):

* "tiny": x ~ N(0,1); smooth ~ U(0.5, 2); W ~ N(0, 0.02); wcscales ~ U(0.5, 1.5);
  wtscale = 1; proj_down, proj_up ~ N(0, 0.02); bias ~ N(0, 0.01).
* "dit": x ~ N(0,1) with floor(1% of K) channels (drawn without replacement)
  scaled by 20 before rounding; smooth = bf16(1 / sqrt(max(absmax_k(x), 1e-6)))
  from the rounded x; W ~ N(0, 0.02); wtscale = 1;
  wcscales[n] = bf16(max_k |W[n, k]| / (6 * 448)), which places the per-block
  weight scales in e4m3's normal range; proj and bias as above.
* "swiglu": like "dit" but x = silu(a) * b with a, b ~ N(0, (0.02 sqrt(3840))^2),
  the input of an FFN down projection (w2), then the same outlier channels.

bf16 tensors are returned as uint16 bit patterns; W as float32.
"""

import math

import numpy as np

# Shapes of the workloads (M tokens, K in, N out, R rank).
TINY = dict(M=64, K=256, N=128, R=16, kind="tiny", seed=1001)
QKV_1024 = dict(M=4096, K=3840, N=11520, R=128, kind="dit", seed=1002)
FFN_W1_1024 = dict(M=4096, K=3840, N=10240, R=128, kind="dit", seed=1003)
FFN_W3_1024 = dict(M=4096, K=3840, N=10240, R=128, kind="dit", seed=1013)
FFN_W2_1024 = dict(M=4096, K=10240, N=3840, R=128, kind="swiglu", seed=1023)
# 2048px: 16384 image tokens + 512 text tokens.
M_2048 = 16384 + 512
LAYERS_2048 = {
    "qkv": dict(M=M_2048, K=3840, N=11520, R=128, kind="dit", seed=1004),
    "out": dict(M=M_2048, K=3840, N=3840, R=128, kind="dit", seed=1014),
    "w1": dict(M=M_2048, K=3840, N=10240, R=128, kind="dit", seed=1024),
    "w3": dict(M=M_2048, K=3840, N=10240, R=128, kind="dit", seed=1034),
    "w2": dict(M=M_2048, K=10240, N=3840, R=128, kind="swiglu", seed=1044),
}
# One GPU's share of the 1024^2 layers under 8-way tensor parallelism: qkv and w1 split by
# output columns (N / 8), w2 by input rows (K / 8, 1280 = 80 whole 16-blocks).
SHARDS_TP8_1024 = {
    "qkv": dict(M=4096, K=3840, N=11520 // 8, R=128, kind="dit", seed=1052),
    "w1": dict(M=4096, K=3840, N=10240 // 8, R=128, kind="dit", seed=1053),
    "w2": dict(M=4096, K=10240 // 8, N=3840, R=128, kind="swiglu", seed=1054),
}


def f32_to_bf16_bits(a):
    """float32/float64 array -> bf16 bit patterns (uint16), round to nearest even.

    Goes through float32 first; the inputs drawn here are float32-exact
    or only need a bf16 value, so this is the ordinary dtype cast.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _outliers(rng, x, K):
    n_out = int(math.floor(0.01 * K))
    idx = rng.choice(K, size=n_out, replace=False) if n_out > 0 else np.zeros(0, np.int64)
    x[:, idx] *= 20.0
    return idx


def make_linear(M, K, N, R, kind="dit", seed=0, with_bias=True):
    """Draw one linear layer's inputs. Returns a dict of numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "swiglu":
        sd = 0.02 * math.sqrt(3840.0)
        a = rng.standard_normal((M, K), dtype=np.float32) * np.float32(sd)
        b = rng.standard_normal((M, K), dtype=np.float32) * np.float32(sd)
        x = (a / (1.0 + np.exp(-a))) * b
    else:
        x = rng.standard_normal((M, K), dtype=np.float32)
    if kind in ("dit", "swiglu"):
        _outliers(rng, x, K)
    x_bits = f32_to_bf16_bits(x)
    if kind == "tiny":
        smooth = rng.uniform(0.5, 2.0, size=K).astype(np.float32)
    else:
        absmax = np.abs(bf16_bits_to_f32(x_bits)).max(axis=0)
        smooth = 1.0 / np.sqrt(np.maximum(absmax, 1e-6))
    smooth_bits = f32_to_bf16_bits(smooth)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if kind == "tiny":
        wcscales = rng.uniform(0.5, 1.5, size=N)
    else:
        wcscales = np.abs(W).max(axis=1).astype(np.float64) / (6.0 * 448.0)
    wcscales_bits = f32_to_bf16_bits(wcscales)
    wtscale_bits = f32_to_bf16_bits(np.array([1.0]))
    proj_down = rng.standard_normal((K, R), dtype=np.float32) * np.float32(0.02)
    proj_up = rng.standard_normal((N, R), dtype=np.float32) * np.float32(0.02)
    bias = rng.standard_normal(N, dtype=np.float32) * np.float32(0.01)
    return dict(
        M=M, K=K, N=N, R=R,
        x=x_bits, smooth=smooth_bits, W=W,
        wcscales=wcscales_bits, wtscale=wtscale_bits,
        proj_down=f32_to_bf16_bits(proj_down), proj_up=f32_to_bf16_bits(proj_up),
        bias=f32_to_bf16_bits(bias) if with_bias else None,
    )


def make_activation(M, K, kind="dit", seed=0):
    """Only x and smooth, for activation-quantisation cases (same recipe)."""
    d = make_linear(M, K, 16, 0, kind=kind, seed=seed, with_bias=False)
    return d["x"], d["smooth"]


def make_bf16_linear(M, K, N, kind="dit", seed=0, with_bias=True):
    """Inputs of a linear kept in bf16: x (same recipe as make_linear, so
    "dit" has the outlier channels), W ~ N(0, 0.02) and bias ~ N(0, 0.01),
    all rounded to bf16. Draw order x, outlier channels, W, bias."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    if kind in ("dit", "swiglu"):
        _outliers(rng, x, K)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    bias = rng.standard_normal(N, dtype=np.float32) * np.float32(0.01)
    return dict(M=M, K=K, N=N, x=f32_to_bf16_bits(x), W=f32_to_bf16_bits(W),
                bias=f32_to_bf16_bits(bias) if with_bias else None)


# The mixed-precision linear sweep of a 30-block DiT at 1024^2 (M = 4096
# tokens), 8 denoising forwards. The blog page's variant table: the "Ultra"
# variant keeps attention (qkv, out) and blocks 0-4 and 25-29 in bf16 and
# quantises 60 linears to NVFP4; 60 = 20 blocks x the 3 FFN linears w1, w3, w2.
SWEEP_M = 4096
SWEEP_BLOCKS = 30
SWEEP_STEPS = 8
SWEEP_LAYERS = (("qkv", 3840, 11520), ("out", 3840, 3840),
                ("w1", 3840, 10240), ("w3", 3840, 10240), ("w2", 10240, 3840))
SWEEP_R = 128


def sweep_precision(block, name):
    """"bf16" or "w4a4" for one linear of the sweep (Ultra variant)."""
    if name in ("qkv", "out") or block < 5 or block >= 25:
        return "bf16"
    return "w4a4"


def sweep_layers():
    """The sweep's linears in execution order: dicts with block, name, K, N,
    precision and the weight seed 5000 + 10 * block + layer index."""
    out = []
    for b in range(SWEEP_BLOCKS):
        for li, (name, K, N) in enumerate(SWEEP_LAYERS):
            out.append(dict(block=b, name=name, K=K, N=N, precision=sweep_precision(b, name),
                            seed=5000 + 10 * b + li))
    return out


def sweep_activation_seed(step, layer_index):
    """Seed of the fresh activations of one (forward step, linear) pair."""
    return 6000 + 1000 * step + layer_index


def make_omega(K, R, seed):
    """Gaussian test matrix [K, R] (float32, N(0, 1)) for the randomized rank-R
    split of weight preparation."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((K, R), dtype=np.float32)


def make_prep_weight(N, K, seed, strong=8):
    """A bf16 weight [N, K] ~ N(0, 0.02) plus `strong` directions of decaying
    strength (trained weights have a few large singular values; SVDQuant's
    low-rank branch targets them), and a smooth factor from an outlier
    activation (same recipe as "dit"). Returns (W bits, smooth bits, x bits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    if strong:
        A = rng.standard_normal((N, strong), dtype=np.float32) * np.geomspace(1.0, 0.3, strong).astype(np.float32)
        B = rng.standard_normal((strong, K), dtype=np.float32) * np.float32(0.02)
        W = W + A @ B
    x, smooth = make_activation(64, K, kind="dit", seed=seed + 1)
    return f32_to_bf16_bits(W), smooth, x
