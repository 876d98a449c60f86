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


def _oracle_net(orc, synth, wl, rows, trace=None):
    from oracle.ref import BlockParams
    net = wl.net
    stem = oracle_conv(orc, synth, net.stem, wl.index)
    blocks = [BlockParams(oracle_conv(orc, synth, b.c1, wl.index), oracle_conv(orc, synth, b.c2, wl.index),
                          oracle_conv(orc, synth, b.c3, wl.index),
                          oracle_conv(orc, synth, b.proj, wl.index) if b.proj is not None else None)
              for b in net.blocks]
    fcp = synth.fc_params(wl.index, net)
    x = synth.input_tensor(wl, rows=rows).numpy()
    return orc.net(x, stem, blocks, fcp["w"].numpy(), fcp["bias"].numpy(), trace=trace)


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


def test_workload4_every_layer_sampled(ifx, orc):
    """Every layer of the batch-2048 network for sampled images, against the oracle's trace.

    ifx_net_forward runs a batch of 2048 as two concurrent passes of 1024 images.  Here the
    driver's launches are issued pass by pass through the C ABI, with the same kernels and
    grids: the fused stem reading the NHWC images; per bottleneck conv1 (unless the previous
    block chained it), conv2, then conv3 fused with its projection, or chained with the next
    block's conv1 where the library reports that pair as chainable (conv3 with its projection
    too), or alone.  conv1 of a block whose conv2 has stride 2 stores its output phase-split
    (IFX_OUT_PHASE, also through the chained launch) for conv2 (IFX_IN_PHASE).  A chained block
    output whose next reader is a stride-2 projection is stored at its even pixels only
    (IFX_OUT_EVEN), and that projection then runs with stride 1 on the subsampled tensor; an
    unchained block output with such a reader is stored whole and its even pixels a second time
    (ifx_conv_fused_even), and the projection reads that copy with stride 1.  After
    each layer the sampled images (the first and last of the batch, one in each pass, and two
    more) are compared byte for byte with the oracle: the pooled stem output and all 16 block
    outputs (the stored pixels of the subsampled one)."""
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(4)
    net = model.DeviceNet(wl.net, wl.index, nhwc_input=True)
    rows = sample_rows(wl.n)
    note(f"oracle trace on images {rows}")
    trace = []
    _oracle_net(orc, synth, wl, rows, trace=trace)
    half = wl.n // 2

    def at(dc, n):
        d = ifx.ConvDesc.from_buffer_copy(dc.desc)
        d.n = n
        return d

    def with_flag(d, f):
        q = ifx.ConvDesc.from_buffer_copy(d)
        q.flags |= f
        return q

    def phase_in_ok(d):  # a stride-2 3x3 that reads the phase-split layout (the driver's rule)
        return (d.kh == 3 and d.stride == 2 and d.pad == 1 and d.h % 2 == 0 and d.w % 2 == 0
                and ifx.conv_validate(with_flag(d, ifx.IN_PHASE)) == 0)

    chained = phases = evens = 0
    for p0 in (0, half):
        mine = [i for i, r in enumerate(rows) if p0 <= r < p0 + half]
        local = [rows[i] - p0 for i in mine]
        note(f"pass of images {p0}..{p0 + half - 1}: sampled {[rows[i] for i in mine]}")
        x = synth.input_tensor(wl, device="cuda", rows=list(range(p0, p0 + half)))
        t = model.empty_act(half, 56, 56, 64)
        ifx.conv_fused(at(net.stem, half), x, net.stem.w_blk, net.stem.bias, net.stem.mult, net.stem.shift, None, t)
        del x
        torch.cuda.synchronize()
        got = ifx.unpack_act(t[local].contiguous(), 64).cpu().numpy()
        np.testing.assert_array_equal(got, trace[0][mine], err_msg="stem")
        t1 = None  # the block's conv1 output when the previous block chained it
        t1_ps = False  # ... stored phase-split
        t_even = False  # t holds only the even pixels of the block input
        t_xe = None  # or: the block input's even pixels, a second copy
        for bi, blk in enumerate(net.blocks):
            c1, c2, c3 = blk.convs
            d2 = at(c2, half)
            if t1 is None:
                d1o = at(c1, half)
                t1_ps = phase_in_ok(d2) and ifx.conv_validate(with_flag(d1o, ifx.OUT_PHASE)) == 0
                t1 = model.empty_act(half, *c1.out_hw, c1.spec.c_out)
                ifx.conv_fused(with_flag(d1o, ifx.OUT_PHASE) if t1_ps else d1o, t, c1.w_blk, c1.bias, c1.mult,
                               c1.shift, None, t1)
            phases += t1_ps
            t2 = model.empty_act(half, *c2.out_hw, c2.spec.c_out)
            ifx.conv_fused(with_flag(d2, ifx.IN_PHASE) if t1_ps else d2, t1, c2.w_blk, c2.bias, c2.mult, c2.shift,
                           None, t2)
            nb_ = net.blocks[bi + 1] if bi + 1 < len(net.blocks) else None
            nxt = nb_.convs[0] if nb_ is not None else None
            # the next block's conv1 as a chained launch writes phase-split for a stride-2 conv2
            d1n = None
            if nxt is not None:
                d1n = at(nxt, half)
                if phase_in_ok(at(nb_.convs[1], half)):
                    d1n = with_flag(d1n, ifx.OUT_PHASE)
            t1, t1_ps = None, False
            y_even, ye = False, None
            d3 = at(c3, half)
            if blk.proj is not None:
                pj = blk.proj
                dp = at(pj, half)
                if t_even or t_xe is not None:  # the projection's stride-2 pixels, already subsampled
                    dp.stride, dp.h, dp.w = 1, (dp.h + 1) // 2, (dp.w + 1) // 2
                px = t_xe if t_xe is not None else t
                y = model.empty_act(half, *c3.out_hw, c3.spec.c_out)
                if nxt is not None and ifx.conv_proj_chain_kernel_name(d3, dp, d1n) is not None:
                    t1 = model.empty_act(half, *nxt.out_hw, nxt.spec.c_out)
                    t1_ps = bool(d1n.flags & ifx.OUT_PHASE)
                    ifx.conv_proj_chain_fused(d3, t2, c3.w_blk, c3.bias, c3.mult, c3.shift, dp, px, pj.w_blk,
                                              pj.bias, pj.mult, pj.shift, y, d1n, nxt.w_blk, nxt.bias,
                                              nxt.mult, nxt.shift, t1)
                    chained += 1
                else:
                    ifx.conv_proj_fused(d3, t2, c3.w_blk, c3.bias, c3.mult, c3.shift, dp, px,
                                        pj.w_blk, pj.bias, pj.mult, pj.shift, y)
            elif nxt is not None and ifx.conv_chain_kernel_name(d3, d1n) is not None:
                pn = nb_.proj
                y_even = pn is not None and pn.spec.k == 1 and pn.spec.stride == 2
                if y_even:
                    d3.flags |= ifx.OUT_EVEN
                    y = model.empty_act(half, (c3.out_hw[0] + 1) // 2, (c3.out_hw[1] + 1) // 2, c3.spec.c_out)
                else:
                    y = model.empty_act(half, *c3.out_hw, c3.spec.c_out)
                t1 = model.empty_act(half, *nxt.out_hw, nxt.spec.c_out)
                t1_ps = bool(d1n.flags & ifx.OUT_PHASE)
                ifx.conv_chain_fused(d3, t2, c3.w_blk, c3.bias, c3.mult, c3.shift, t, y, d1n,
                                     nxt.w_blk, nxt.bias, nxt.mult, nxt.shift, t1)
                chained += 1
            else:
                y = model.empty_act(half, *c3.out_hw, c3.spec.c_out)
                pn = nb_.proj if nb_ is not None else None
                if pn is not None and pn.spec.k == 1 and pn.spec.stride == 2 and ifx.conv_even_supported(d3):
                    ye = model.empty_act(half, (c3.out_hw[0] + 1) // 2, (c3.out_hw[1] + 1) // 2, c3.spec.c_out)
                    ifx.conv_fused_even(d3, t2, c3.w_blk, c3.bias, c3.mult, c3.shift, t, y, ye)
                    evens += 1
                else:
                    ifx.conv_fused(d3, t2, c3.w_blk, c3.bias, c3.mult, c3.shift, t, y)
            torch.cuda.synchronize()
            del t2, t
            got = ifx.unpack_act(y[local].contiguous(), c3.spec.c_out).cpu().numpy()
            exp = trace[1 + bi][mine]
            np.testing.assert_array_equal(got, exp[:, ::2, ::2] if y_even else exp, err_msg=f"block {bi}")
            if ye is not None:
                got = ifx.unpack_act(ye[local].contiguous(), c3.spec.c_out).cpu().numpy()
                np.testing.assert_array_equal(got, exp[:, ::2, ::2], err_msg=f"block {bi} even copy")
            t, t_even, t_xe = y, y_even, ye
        del t
        torch.cuda.synchronize()
    # res2.1 -> res2.2 (with its projection), res2.2 -> res2.3, res2.3 -> res3.1, res3.2 -> res3.3,
    # res3.3 -> res3.4; both passes
    assert chained == 10
    assert phases == 6   # res3.1, res4.1, res5.1 conv2 read a phase-split conv1 output; both passes
    assert evens == 4    # res3.4 and res4.6 also store their outputs' even pixels; both passes


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
