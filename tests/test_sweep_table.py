"""The mixed-precision sweep's layer table against the blog page's variant table
("Ultra": attention qkv/out and blocks 0-4 and 25-29 stay bf16; 60 linears are
NVFP4, which with 30 blocks is blocks 5-24 times the FFN linears w1, w3, w2), and
its flop count per forward."""

import workloads


def test_ultra_policy():
    layers = workloads.sweep_layers()
    assert len(layers) == 30 * 5
    q = [(L["block"], L["name"]) for L in layers if L["precision"] == "w4a4"]
    assert len(q) == 60
    assert set(q) == {(b, n) for b in range(5, 25) for n in ("w1", "w3", "w2")}
    assert all(L["precision"] == "bf16" for L in layers if L["name"] in ("qkv", "out"))
    assert len({L["seed"] for L in layers}) == 150
    seeds = {workloads.sweep_activation_seed(f, li) for f in range(8) for li in range(150)}
    assert len(seeds) == 8 * 150


def test_flops_per_forward():
    M, R = workloads.SWEEP_M, workloads.SWEEP_R
    bf = sum(2 * M * L["K"] * L["N"] for L in workloads.sweep_layers() if L["precision"] == "bf16")
    q = sum(2 * M * L["K"] * L["N"] + 2 * M * R * (L["K"] + L["N"])
            for L in workloads.sweep_layers() if L["precision"] == "w4a4")
    assert bf == 24_159_191_040_000
    assert q == 20_213_189_836_800
    assert abs((bf + q) / 1e12 - 44.37) < 0.01
