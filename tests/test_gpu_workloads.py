"""GPU parity on the five synthetic workloads at their full sizes.

The GPU runs each workload whole, in the launch configuration the benchmark
times; the oracle recomputes a seeded sample of images (always including the
first and the last) and the sampled outputs must match byte for byte.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ifx():
    import convolution_int8_implicit_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def sample_rows(n, k=4, seed=0):
    rng = np.random.default_rng(seed + n)
    rows = {0, n - 1}
    while len(rows) < min(k, n):
        rows.add(int(rng.integers(0, n)))
    return sorted(rows)


def oracle_conv(orc, synth, spec, seed):
    p = synth.conv_params(seed, spec)
    from oracle.ref import ConvParams
    return ConvParams(p["w"].numpy(), p["bias"].numpy(), p["mult"].numpy(), p["shift"].numpy(), spec.stride,
                      spec.pad)


def test_workload0_full(ifx, orc):
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(0)
    note(wl.name)
    spec = wl.convs[0]
    dc = model.device_conv(spec, wl.index, wl.n, wl.h, wl.w)
    x = synth.input_tensor(wl)
    r = synth.residual_tensor(wl)
    y = model.empty_act(wl.n, 28, 28, 512)
    dc.run(ifx.pack_act(x.cuda()), y, ifx.pack_act(r.cuda()))
    got = ifx.unpack_act(y, 512).cpu().numpy()
    cp = oracle_conv(orc, synth, spec, wl.index)
    exp = orc.conv_layer(x.numpy(), cp, spec.flags, residual=r.numpy())
    np.testing.assert_array_equal(got, exp)
    # sanity: the workload is not degenerate (some zeros, some saturation, many values)
    assert 0 < np.mean(exp == 0) < 0.5 and np.mean(exp == 127) < 0.5 and len(np.unique(exp)) > 64


def test_workload1_full_batch_sampled(ifx, orc):
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(1)
    note(wl.name)
    spec = wl.convs[0]
    dc = model.device_conv(spec, wl.index, wl.n, wl.h, wl.w)
    xb = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
    rb = ifx.pack_act(synth.residual_tensor(wl, device="cuda"))
    y = model.empty_act(wl.n, 28, 28, 512)
    dc.run(xb, y, rb)
    rows = sample_rows(wl.n)
    got = ifx.unpack_act(y[rows].contiguous(), 512).cpu().numpy()
    cp = oracle_conv(orc, synth, spec, wl.index)
    exp = orc.conv_layer(synth.input_tensor(wl, rows=rows).numpy(), cp, spec.flags,
                         residual=synth.residual_tensor(wl, rows=rows).numpy())
    np.testing.assert_array_equal(got, exp)


def test_workload2_block_sampled(ifx, orc):
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(2)
    note(wl.name)
    c1, c2, c3 = wl.convs
    dcs = [model.device_conv(c1, wl.index, wl.n, 28, 28), model.device_conv(c2, wl.index, wl.n, 28, 28),
           model.device_conv(c3, wl.index, wl.n, 28, 28)]
    blk = model.DeviceBlock(dcs, None)
    ws = torch.empty(blk.workspace_bytes(), dtype=torch.int8, device="cuda")
    xb = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
    y = model.empty_act(wl.n, 28, 28, 512)
    blk.forward(xb, y, ws)
    rows = sample_rows(wl.n)
    got = ifx.unpack_act(y[rows].contiguous(), 512).cpu().numpy()
    x = synth.input_tensor(wl, rows=rows).numpy()
    cps = [oracle_conv(orc, synth, s, wl.index) for s in (c1, c2, c3)]
    exp = orc.block(x, *cps)
    np.testing.assert_array_equal(got, exp)


def test_workload3_stem_sampled(ifx, orc):
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(3)
    note(wl.name)
    spec = wl.convs[0]
    dc = model.device_conv(spec, wl.index, wl.n, wl.h, wl.w)
    xb = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
    y = model.empty_act(wl.n, 56, 56, 64)
    dc.run(xb, y)
    rows = sample_rows(wl.n)
    got = ifx.unpack_act(y[rows].contiguous(), 64).cpu().numpy()
    cp = oracle_conv(orc, synth, spec, wl.index)
    exp = orc.conv_layer(synth.input_tensor(wl, rows=rows).numpy(), cp, spec.flags)
    np.testing.assert_array_equal(got, exp)
    # the same layer reading the compact NHWC image gives the same whole tensor
    note(wl.name + " nhwc input")
    dn = model.device_conv(spec, wl.index, wl.n, wl.h, wl.w)
    dn.desc.flags |= ifx.INPUT_NHWC
    y2 = model.empty_act(wl.n, 56, 56, 64)
    dn.run(synth.input_tensor(wl, device="cuda"), y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def _oracle_net(orc, synth, wl, rows):
    from oracle.ref import BlockParams
    net = wl.net
    stem = oracle_conv(orc, synth, net.stem, wl.index)
    blocks = [BlockParams(oracle_conv(orc, synth, b.c1, wl.index), oracle_conv(orc, synth, b.c2, wl.index),
                          oracle_conv(orc, synth, b.c3, wl.index),
                          oracle_conv(orc, synth, b.proj, wl.index) if b.proj is not None else None)
              for b in net.blocks]
    fcp = synth.fc_params(wl.index, net)
    x = synth.input_tensor(wl, rows=rows).numpy()
    return orc.net(x, stem, blocks, fcp["w"].numpy(), fcp["bias"].numpy())


def test_workload4_net_sampled_and_sub_batch_invariant(ifx, orc):
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(4)
    note(wl.name)
    net = model.DeviceNet(wl.net, wl.index, sub_batch=model.DEFAULT_SUB_BATCH)
    xb = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
    ws = torch.empty(net.workspace_bytes(wl.n), dtype=torch.int8, device="cuda")
    logits = torch.empty((wl.n, 1000), dtype=torch.int32, device="cuda")
    net.forward(xb, logits, wl.n, ws)
    torch.cuda.synchronize()
    rows = sample_rows(wl.n)
    note(f"oracle net on images {rows}")
    exp = _oracle_net(orc, synth, wl, rows)
    got = logits[rows].cpu().numpy()
    np.testing.assert_array_equal(got, exp)
    # results do not depend on how the batch is split into passes
    for sb in (0, 160):
        if sb == model.DEFAULT_SUB_BATCH:
            continue
        note(f"sub_batch {sb}")
        net.set_sub_batch(sb)
        ws2 = torch.empty(net.workspace_bytes(wl.n), dtype=torch.int8, device="cuda")
        l2 = torch.empty_like(logits)
        net.forward(xb, l2, wl.n, ws2)
        torch.cuda.synchronize()
        assert torch.equal(l2, logits)
        del ws2
    # the network fed the compact NHWC image (stem reads it directly)
    for sb in (0, 160):
        note(f"nhwc input, sub_batch {sb}")
        nn_ = model.DeviceNet(wl.net, wl.index, sub_batch=sb, nhwc_input=True)
        ws3 = torch.empty(nn_.workspace_bytes(wl.n), dtype=torch.int8, device="cuda")
        l3 = torch.empty_like(logits)
        nn_.forward(synth.input_tensor(wl, device="cuda"), l3, wl.n, ws3)
        torch.cuda.synchronize()
        assert torch.equal(l3, logits)
        del ws3, nn_


@pytest.mark.parametrize("n", [1, 3])
def test_latency_net26_graph_replays(ifx, orc, n):
    """The ResNet-26-shaped network (batch-1 latency setting): eager forward equals the
    oracle; the same forward recorded as one HIP graph gives the same logits on every
    replay, with other device work and synchronisations between replays."""
    from convolution_int8_implicit_amd import model, synth
    wl = synth.latency_workload(n)
    note(wl.name)
    net = model.DeviceNet(wl.net, wl.index, nhwc_input=True)
    x = synth.input_tensor(wl, device="cuda")
    ws = torch.empty(net.workspace_bytes(n), dtype=torch.int8, device="cuda")
    logits = torch.empty((n, 1000), dtype=torch.int32, device="cuda")
    net.forward(x, logits, n, ws)
    torch.cuda.synchronize()
    eager = logits.clone()
    exp = _oracle_net(orc, synth, wl, list(range(n)))
    np.testing.assert_array_equal(eager.cpu().numpy(), exp)
    g = net.graph(x, logits, n, ws)
    for rep in range(3):
        note(f"graph replay {rep}")
        logits.fill_(-7)                      # eager work between replays
        ws.fill_(rep)
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(logits, eager), rep
    g.close()
