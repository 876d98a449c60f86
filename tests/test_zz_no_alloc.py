"""ifx_block_forward_noalloc: the bottleneck with library-held scratch instead of a caller
workspace, called through the C ABI and compared byte for byte with ifx_block_forward."""
import ctypes
import sys

import pytest
import torch

import convolution_int8_implicit_amd as ifx


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _with_batch(blk, n):
    bp = ifx.BlockParams.from_buffer_copy(blk.params)
    for i in range(4):
        bp.d[i].n = n
    return bp


def _fake_block(n, h, c_in, c_mid, c_out, stride, proj):
    """Block parameters with valid shapes and non-null aligned (never dereferenced) pointers."""
    bp = ifx.BlockParams()
    layers = [(h, c_in, c_mid, 1, 1, 0, ifx.RELU), (h, c_mid, c_mid, 3, stride, 1, ifx.RELU),
              ((h - 1) // stride + 1, c_mid, c_out, 1, 1, 0, ifx.RESIDUAL | ifx.RELU), (h, c_in, c_out, 1, stride, 0, 0)]
    for i, (hh, ci, co, k, s, p, f) in enumerate(layers):
        bp.d[i] = ifx.conv_desc(n, hh, hh, ci, co, k, k, s, p, f)
        bp.w_blk[i] = bp.bias[i] = bp.mult[i] = bp.shift[i] = 0x10000 * (i + 1)
    bp.has_proj = 1 if proj else 0
    return bp


def test_noalloc_validation_needs_no_device():
    """Errors come from host-side validation before any device use: a block whose workspace
    exceeds the scratch (res2 bottleneck at batch 256: 2 x 51 MB), null and misaligned tensors."""
    L = ifx.lib()
    fake = ctypes.c_void_p(0x20000)
    big = _fake_block(256, 56, 256, 64, 256, 1, False)
    assert ifx.block_workspace_bytes(big) > ifx.BLOCK_SCRATCH_BYTES
    assert L.ifx_block_forward_noalloc(ctypes.byref(big), fake, fake, None) == 5
    small = _fake_block(2, 28, 512, 128, 512, 1, False)
    assert 0 < ifx.block_workspace_bytes(small) <= ifx.BLOCK_SCRATCH_BYTES
    assert L.ifx_block_forward_noalloc(ctypes.byref(small), None, fake, None) == 1
    assert L.ifx_block_forward_noalloc(ctypes.byref(small), fake, ctypes.c_void_p(0x20004), None) == 4
    assert L.ifx_block_forward_noalloc(None, fake, fake, None) == 1


@pytest.mark.gpu
def test_noalloc_block_matches_workspace_block():
    from convolution_int8_implicit_amd import model, synth
    assert torch.cuda.is_available()
    ifx.lib()
    # the res3 bottleneck (512 -> 128 -> 128 -> 512, 28x28) at batch 256 uses 51 MB of the scratch
    wl = synth.workload(2)
    dcs = [model.device_conv(s, wl.index, wl.n, 28, 28) for s in wl.convs]
    blk = model.DeviceBlock(dcs, None)
    xb = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
    for n in (256, 3):  # the second call is smaller: the scratch still holds the first call's data
        note(f"res3 bottleneck batch {n}")
        bp = _with_batch(blk, n)
        x = xb[:n].contiguous()
        ws = torch.empty(ifx.block_workspace_bytes(bp), dtype=torch.int8, device="cuda")
        ref = model.empty_act(n, 28, 28, 512)
        ifx.block_forward(bp, x, ref, ws)
        got = torch.full_like(ref, 0x5A)
        ifx.block_forward_noalloc(bp, x, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
        del ws
    # res5.1 (1024 -> 512 -> 512/s2 -> 2048 with the fused projection) at batch 1: c1 and c2
    # split over K, so the partial sums live in the scratch too
    net = synth.workload(4).net
    bs = net.blocks[13]
    note("res5.1 projection block batch 1 (split K)")
    pblk = model.device_block(bs, 4, 1, 14, 14)
    x = ifx.pack_act(synth.uniform(4, 999, (1, 14, 14, 1024), 0, 127, device="cuda"))
    ws = torch.empty(ifx.block_workspace_bytes(pblk.params), dtype=torch.int8, device="cuda")
    ref = model.empty_act(1, 7, 7, 2048)
    pblk.forward(x, ref, ws)
    for rep in range(2):
        got = torch.full_like(ref, 0x5A)
        ifx.block_forward_noalloc(pblk.params, x, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), rep
    # over the limit: an error, and nothing is written
    note("over the scratch limit")
    big = _with_batch(blk, 2048)
    assert ifx.block_workspace_bytes(big) > ifx.BLOCK_SCRATCH_BYTES
    y = torch.full((16,), 7, dtype=torch.int8, device="cuda")
    with pytest.raises(ifx.IfxError):
        ifx.block_forward_noalloc(big, y, y)
    torch.cuda.synchronize()
    assert torch.all(y == 7)
