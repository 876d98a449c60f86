"""The seeded input generator: published SplitMix64 values, determinism, and
the workload shapes (no GPU)."""
import os

import numpy as np
import pytest
import torch

from convolution_int8_implicit_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_splitmix64_published_sequence():
    vals = []
    with open(os.path.join(HERE, "golden", "splitmix64_seed0.txt")) as f:
        vals = [int(line, 16) for line in f.read().splitlines() if line.startswith("0x")]
    state = 0
    for v in vals:
        state = (state + synth.GAMMA) & synth.MASK64
        assert synth.mix64_int(state) == v
    # the tensor path computes the same function with wrapping int64 arithmetic
    z = torch.tensor([synth._s64(synth.GAMMA * (i + 1)) for i in range(3)], dtype=torch.int64)
    got = [(int(t) & synth.MASK64) for t in synth._mix(z)]
    assert got == vals


def test_uniform_matches_pure_python_definition():
    seed, tid, lo, hi = 3, synth.tensor_id(5, synth.ROLE_W), -127, 127
    got = synth.uniform(seed, tid, (1000,), lo, hi, dtype=torch.int64)
    key = synth.stream_key(seed, tid)
    for i in (0, 1, 2, 511, 999):
        x = synth.mix64_int(key + (i + 1) * synth.GAMMA)
        assert int(got[i]) == lo + ((x >> 32) % (hi - lo + 1))
    assert int(got.min()) >= lo and int(got.max()) <= hi


def test_uniform_is_deterministic_and_row_addressable():
    wl = synth.workload(3, n=4)
    full = synth.input_tensor(wl)
    again = synth.input_tensor(wl)
    assert torch.equal(full, again)
    rows = synth.input_tensor(wl, rows=[3, 1])
    assert torch.equal(rows[0], full[3]) and torch.equal(rows[1], full[1])
    # different seeds or tensor ids give different streams
    a = synth.uniform(0, 1, (64,), 0, 127)
    b = synth.uniform(1, 1, (64,), 0, 127)
    c = synth.uniform(0, 2, (64,), 0, 127)
    assert not torch.equal(a, b) and not torch.equal(a, c)


def test_value_ranges_cover_the_distribution():
    p = synth.conv_params(0, synth.workload(0).convs[0])
    assert p["w"].dtype == torch.int8 and p["w"].shape == (512, 1, 1, 128)
    assert int(p["w"].min()) == -127 and int(p["w"].max()) == 127
    assert int(p["mult"].min()) >= 1 << 30 and int(p["mult"].max()) <= (1 << 31) - 1
    assert int(p["shift"].min()) == 8 and int(p["shift"].max()) == 16
    assert int(p["bias"].abs().max()) <= 1 << 16
    x = synth.input_tensor(synth.workload(0))
    assert x.shape == (1, 28, 28, 128) and int(x.min()) == 0 and int(x.max()) == 127


def test_resnet50_spec_counts():
    net = synth.resnet50_spec()
    assert len(net.blocks) == 16
    main = 3 * len(net.blocks)
    proj = sum(1 for b in net.blocks if b.proj is not None)
    # the Inspur conv-merge article: 48 convolutions in the 4 residual groups
    assert main == 48 and proj == 4 and main + proj + 1 == 53
    layers = [net.stem.layer] + [c.layer for b in net.blocks for c in (b.proj, b.c1, b.c2, b.c3) if c]
    assert layers == list(range(53)) and net.fc_layer == 53
    # MACs per image (2 ops per MAC) of the backbone + FC
    h = w = 224
    macs = net.stem.macs(1, h, w)
    h = w = 56
    for b in net.blocks:
        macs += b.c1.macs(1, h, w)
        macs += b.c2.macs(1, h, w)
        h2, w2 = b.c2.out_hw(h, w)
        macs += b.c3.macs(1, h2, w2)
        if b.proj:
            macs += b.proj.macs(1, h, w)
        h, w = h2, w2
    macs += net.fc_in * net.fc_out
    assert (h, w) == (7, 7)
    assert abs(2 * macs / 1e9 - 8.1785) < 0.01


@pytest.mark.parametrize("idx", range(5))
def test_workload_table(idx):
    wl = synth.workloads()[idx]
    assert wl.index == idx
    assert wl.n == [1, 2048, 256, 128, 2048][idx]
    shp = synth.input_shape(wl)
    assert shp[1:3] == ((28, 28) if idx < 3 else (224, 224))


def test_resnet26_spec_counts():
    from convolution_int8_implicit_amd import synth
    net = synth.resnet26_spec()
    assert len(net.blocks) == 8
    assert sum(b.proj is not None for b in net.blocks) == 4
    # 26 weighted layers: stem + 8 x 3 bottleneck convs + FC (projections extra)
    assert 1 + 3 * len(net.blocks) + 1 == 26
    assert net.fc_in == 2048 and net.fc_out == 1000
    wl = synth.latency_workload()
    assert (wl.index, wl.n, wl.h, wl.w) == (5, 1, 224, 224)
