"""GPU parity: libifx.so (through its C ABI) against the CPU oracle, byte for byte.

Every step of the path is integer, so the bar is bit-exactness: int8 outputs,
int32 accumulators and int32 logits must equal the oracle's on the same seeded
inputs.  Outputs are written into sentinel-filled buffers with guard bands, and
runs are repeated to catch races.
"""
import ctypes
import itertools
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SENT = 0x5A
GUARD = 4096


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ifx():
    import convolution_int8_implicit_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def guarded(nbytes, dtype=torch.int8):
    """A device buffer of nbytes inside sentinel guard bands; returns (view, whole)."""
    whole = torch.full((nbytes + 2 * GUARD,), SENT, dtype=torch.int8, device="cuda")
    view = whole[GUARD:GUARD + nbytes]
    if dtype != torch.int8:
        view = view.view(dtype)
    return view, whole


def check_guards(whole):
    w = whole.cpu().numpy()
    assert np.all(w[:GUARD] == SENT) and np.all(w[-GUARD:] == SENT), "write outside the output buffer"


def rand(rng, shape, lo, hi, dtype=np.int8):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(dtype)


def cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_conv(ifx, x, w, bias, mult, shift, k, s, p, flags, residual=None, check_pad=True):
    """Run ifx_conv_fused on NHWC/OHWI numpy inputs; returns NHWC numpy output."""
    n, h, wd, c = x.shape
    oc = w.shape[0]
    d = ifx.conv_desc(n, h, wd, c, oc, k, k, s, p, flags)
    xb = cu(x) if flags & ifx.INPUT_NHWC else ifx.pack_act(cu(x))
    wb = ifx.pack_weights(d, cu(w))
    ho, wo = ifx.conv_out_dims(d)
    rb = ifx.pack_act(cu(residual)) if residual is not None else None
    if flags & ifx.OUT_I32:
        y, whole = guarded(n * ho * wo * oc * 4, torch.int32)
        y = y.view(n, ho, wo, oc)
    else:
        nbytes = ifx.act_bytes(n, ho, wo, oc)
        y, whole = guarded(nbytes)
        y = y.view(n, (oc + 31) // 32, ho, wo, 32)
    ifx.conv_fused(d, xb, wb, cu(bias), cu(mult) if mult is not None else None,
                   cu(shift) if shift is not None else None, rb, y)
    torch.cuda.synchronize()
    check_guards(whole)
    if flags & ifx.OUT_I32:
        return y.cpu().numpy()
    if check_pad and oc % 32:
        tail = y[:, -1, :, :, oc % 32:].cpu().numpy()
        assert np.all(tail == 0), "padding channels of the packed output must be zero"
    return ifx.unpack_act(y, oc).cpu().numpy()


def to_phase(t):
    """Packed [n, c1, h, w, 32] -> phase-split [n, c1, 2, 2, h/2, w/2, 32] (ifx.h's permutation)."""
    n, c1, h, w, _ = t.shape
    return t.view(n, c1, h // 2, 2, w // 2, 2, 32).permute(0, 1, 3, 5, 2, 4, 6).contiguous()


def from_phase(t, n, c1, h, w):
    """Phase-split bytes -> packed [n, c1, h, w, 32]."""
    return t.view(n, c1, 2, 2, h // 2, w // 2, 32).permute(0, 1, 4, 2, 5, 3, 6).reshape(n, c1, h, w, 32)


def params(rng, oc, shift_lo=8, shift_hi=16):
    return (rand(rng, oc, -(1 << 16), 1 << 16, np.int32), rand(rng, oc, 1 << 30, (1 << 31) - 1, np.int32),
            rand(rng, oc, shift_lo, shift_hi, np.int32))


# ------------------------------------------------------------------ packers
@pytest.mark.parametrize("c", [3, 32, 64, 96, 130])
def test_pack_unpack_act(ifx, orc, c):
    note(f"pack_act c={c}")
    rng = np.random.default_rng(c)
    x = rand(rng, (3, 7, 9, c), -128, 127)
    xb = ifx.pack_act(cu(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xb.cpu().numpy(), orc.pack_act(x))
    np.testing.assert_array_equal(ifx.unpack_act(xb, c).cpu().numpy(), x)


@pytest.mark.parametrize("oc,k,ic", [(512, 1, 128), (64, 3, 64), (1000, 1, 2048), (96, 3, 40), (128, 3, 128)])
def test_pack_weights(ifx, orc, oc, k, ic):
    note(f"pack_weights oc={oc} k={k} ic={ic}")
    rng = np.random.default_rng(oc + k + ic)
    w = rand(rng, (oc, k, k, ic), -127, 127)
    d = ifx.conv_desc(1, 8, 8, ic, oc, k, k, 1, k // 2, 0)
    wb = ifx.pack_weights(d, cu(w))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wb.cpu().numpy(), orc.pack_weights(w).reshape(-1))


def test_pack_weights_stem(ifx, orc):
    note("pack_weights stem")
    rng = np.random.default_rng(77)
    w = rand(rng, (64, 7, 7, 3), -127, 127)
    d = ifx.conv_desc(1, 224, 224, 3, 64, 7, 7, 2, 3, ifx.RELU | ifx.MAXPOOL)
    wb = ifx.pack_weights(d, cu(w))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wb.cpu().numpy(), orc.pack_weights_stem(w).reshape(-1))


# ------------------------------------------------------------------ raw accumulators
ACC_CASES = [
    # n, h, w, c, oc, k, s, p
    (1, 28, 28, 128, 512, 1, 1, 0),
    (2, 9, 11, 96, 64, 1, 1, 0),
    (3, 14, 13, 64, 256, 1, 2, 0),
    (2, 9, 9, 64, 64, 3, 1, 1),
    (1, 15, 14, 128, 128, 3, 2, 1),
    (2, 7, 7, 32, 96, 3, 1, 1),
    (1, 5, 6, 3, 40, 3, 1, 1),
    (4, 1, 1, 2048, 1000, 1, 1, 0),
    (1, 3, 3, 33, 200, 3, 2, 1),
]


@pytest.mark.parametrize("case", ACC_CASES)
def test_int32_accumulators(ifx, orc, case):
    n, h, w, c, oc, k, s, p = case
    note(f"acc {case}")
    rng = np.random.default_rng(sum(case))
    x = rand(rng, (n, h, w, c), -128, 127)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    zero = np.zeros(oc, np.int32)
    got = gpu_conv(ifx, x, wt, zero, None, None, k, s, p, ifx.OUT_I32)
    np.testing.assert_array_equal(got, orc.conv_acc(x, wt, s, p))
    # with a bias: acc + bias
    bias = rand(rng, oc, -(1 << 16), 1 << 16, np.int32)
    got = gpu_conv(ifx, x, wt, bias, None, None, k, s, p, ifx.OUT_I32)
    np.testing.assert_array_equal(got, orc.conv_acc(x, wt, s, p) + bias)


# ------------------------------------------------------------------ fused int8 epilogue
FUSED_SHAPES = [
    (1, 28, 28, 128, 512, 1, 1, 0),
    (2, 9, 11, 96, 64, 1, 1, 0),
    (3, 14, 13, 64, 256, 1, 2, 0),
    (2, 9, 9, 64, 64, 3, 1, 1),
    (1, 15, 14, 128, 128, 3, 2, 1),
    (1, 5, 6, 3, 40, 3, 1, 1),
    (3, 7, 7, 512, 2048, 1, 1, 0),
    # wide 1x1 without a shortcut: 256x128 tiles on a three-stage ring
    (2, 9, 7, 160, 200, 1, 1, 0),    # 5 channel blocks: 3 K-steps, all requested up front, odd tail
    (1, 11, 10, 192, 136, 1, 2, 0),  # strided, exactly 3 K-steps, ragged output channels
    (1, 6, 7, 256, 384, 1, 1, 0),    # 4 K-steps through the ring
    (2, 5, 5, 320, 256, 1, 1, 0),    # 5 K-steps through the ring
    # strided 3x3 with >= 256 output channels on the plain layout: 128x256 tiles of eight waves
    (2, 9, 11, 64, 256, 3, 2, 1),
    (1, 8, 7, 96, 288, 3, 2, 1),     # ragged output channels, odd channel-block count
    # stride-1 3x3, <= 64 input channels, 48 <= W <= 62: the haloed-window kernel (flags 0 and 1;
    # with a shortcut the general kernel runs)
    (2, 56, 56, 64, 64, 3, 1, 1),    # the res2 shape: 14 row bands of 8 rows, one per workgroup
    (3, 13, 50, 40, 96, 3, 1, 1),    # ragged last band (13 rows), two channel blocks, padded channels
    (1, 7, 62, 32, 64, 3, 1, 1),     # widest window (pitch 64), one channel block
    (2, 5, 48, 64, 200, 3, 1, 1),    # narrowest, four output-channel tiles, padding in the last
    # 3x3 with >= 512 output channels (flags 0 and 1): four waves of 64x128 sub-tiles on a
    # three-stage ring; with a shortcut the general kernel runs
    (2, 9, 11, 64, 512, 3, 1, 1),    # two 128x256 tiles across images, a ragged pixel tile
    (1, 7, 7, 96, 520, 3, 1, 1),     # ragged output channels: a partial 64-channel half
]


@pytest.mark.parametrize("shape", FUSED_SHAPES)
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_fused_conv(ifx, orc, shape, flags):
    n, h, w, c, oc, k, s, p = shape
    note(f"fused {shape} flags={flags}")
    rng = np.random.default_rng(sum(shape) * 7 + flags)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    bias, mult, shift = params(rng, oc)
    ho, wo = orc.out_dim(h, k, s, p), orc.out_dim(w, k, s, p)
    res = rand(rng, (n, ho, wo, oc), -128, 127) if flags & ifx.RESIDUAL else None
    got = gpu_conv(ifx, x, wt, bias, mult, shift, k, s, p, flags, res)
    exp = orc.conv_fused(x, wt, bias, mult, shift, s, p, flags, res)
    np.testing.assert_array_equal(got, exp)


# The haloed-window kernel is persistent: one workgroup per CU per 64-channel tile, each walking a
# contiguous run of 8-row bands with the next band's window fetched into the second buffer while
# the current one computes.  With 256 CUs a run holds two or more bands from 37 images of 56 rows
# on (7 bands each), so these batches drive the double-buffered loop: 37 images leave a last
# workgroup with a single band (ragged), 75 give three bands to every workgroup, and 128 output
# channels halve the workgroups per tile (three bands each).
@pytest.mark.parametrize("n,oc", [(37, 64), (75, 64), (37, 128)])
@pytest.mark.parametrize("flags", [0, 1])
def test_halo_window_multi_band(ifx, orc, n, oc, flags):
    note(f"halo window multi-band n={n} oc={oc} flags={flags}")
    rng = np.random.default_rng(n * 3 + oc + flags)
    x = rand(rng, (n, 56, 56, 64), 0, 127)
    wt = rand(rng, (oc, 3, 3, 64), -127, 127)
    bias, mult, shift = params(rng, oc)
    got = gpu_conv(ifx, x, wt, bias, mult, shift, 3, 1, 1, flags)
    np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, 1, 1, flags))


# Unit-stride 3x3 layers over a multiple of 128 input channels, with 128-channel output tiles, on
# 14- or 28-wide images, run the haloed-window kernel: tiles of 224 pixels in whole rows (8 of a
# 28-wide image, 16 of a 14-wide one), whose windows take one halo row above and below every
# image a tile touches (a 16-row tile of 14-row images touches up to three), the reduction in
# 64-channel chunks, and a ragged last tile.  Sampled images are compared, among them the first
# two (the first tile that spans an image boundary) and the last two.
WIN_SHAPES = [
    (80, 28, 28, 128, 128),   # res3 conv2: 280 tiles, one pair of chunks
    (150, 14, 14, 256, 256),  # res4 conv2: 132 pixel tiles (the last one quarter full) x 2
    (74, 28, 28, 512, 128),   # four pairs of chunks
    (300, 14, 14, 128, 384),  # three output-channel tiles, a half-full last pixel tile
]


@pytest.mark.parametrize("shape", WIN_SHAPES)
@pytest.mark.parametrize("flags", [0, 1])
def test_window_3x3(ifx, orc, shape, flags):
    n, h, w, c, oc = shape
    note(f"window 3x3 {shape} flags={flags}")
    rng = np.random.default_rng(sum(shape) * 11 + flags)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, 3, 3, c), -127, 127)
    # shifts 0-20 take the general requantisation, 8-16 the fast forms
    bias, mult, shift = params(rng, oc, 0, 20) if flags == 0 else params(rng, oc)
    d = ifx.conv_desc(n, h, w, c, oc, 3, 3, 1, 1, flags)
    assert ifx.conv_kernel_name(d).startswith("conv3x3_win_kernel<")
    got = gpu_conv(ifx, x, wt, bias, mult, shift, 3, 1, 1, flags)
    idx = sorted({0, 1, 2, n // 2, n - 2, n - 1})
    exp = orc.conv_fused(x[idx], wt, bias, mult, shift, 1, 1, flags)
    np.testing.assert_array_equal(got[idx], exp)


def test_window_3x3_even_copy(ifx, orc):
    """The haloed-window kernel also writes the even-pixel copy when asked."""
    n, h, w, c, oc = 80, 28, 28, 128, 128
    note("window 3x3 even copy")
    rng = np.random.default_rng(2024)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, 3, 3, c), -127, 127)
    bias, mult, shift = params(rng, oc)
    d = ifx.conv_desc(n, h, w, c, oc, 3, 3, 1, 1, ifx.RELU)
    assert ifx.conv_kernel_name(d).startswith("conv3x3_win_kernel<")
    assert ifx.conv_even_supported(d)
    y, yw = guarded(ifx.act_bytes(n, h, w, oc))
    ye, ew = guarded(ifx.act_bytes(n, h // 2, w // 2, oc))
    ifx.conv_fused_even(d, ifx.pack_act(cu(x)), ifx.pack_weights(d, cu(wt)), cu(bias), cu(mult), cu(shift), None,
                        y, ye)
    torch.cuda.synchronize()
    check_guards(yw)
    check_guards(ew)
    idx = [0, 1, n - 1]
    exp = orc.conv_fused(x[idx], wt, bias, mult, shift, 1, 1, ifx.RELU)
    got = ifx.unpack_act(y.view(n, oc // 32, h, w, 32), oc).cpu().numpy()
    np.testing.assert_array_equal(got[idx], exp)
    got_e = ifx.unpack_act(ye.view(n, oc // 32, h // 2, w // 2, 32), oc).cpu().numpy()
    np.testing.assert_array_equal(got_e[idx], exp[:, ::2, ::2])


# 1x1 layers with a shortcut, unit stride and 256 or 512 output channels run on persistent
# workgroups (two per CU for 256 channels, one for 512) that walk 64-pixel tiles through a ring
# of 3-4 LDS buffers.  These batches give every workgroup several tiles, more than the ring holds,
# so the ring wraps; the small shapes leave ragged tiles spanning images.  Sampled images are
# compared (each image's outputs depend on that image alone).
RING_SHAPES = [
    (100, 28, 28, 128, 512),  # the res3 conv3 shape: 1225 tiles over 256 workgroups
    (200, 28, 28, 64, 256),   # K = 64: 2450 tiles over 512 workgroups, four-deep ring
    (40, 56, 56, 96, 256),    # K = 96 (two K-steps, the second half zero): three-deep ring
    (3, 7, 7, 128, 512),      # 147 pixels: tiles spanning images, a ragged last tile
    (1, 5, 5, 32, 256),       # one partial tile, K = 32
    # K of 160..256 and 512 / 1024 / 1536 output channels: weights of four K-steps in registers,
    # workgroups in slices of 512 channels (at least 512 tiles)
    (168, 14, 14, 256, 1024),  # the res4 conv3 shape: two slices
    (700, 7, 7, 224, 512),     # seven channel blocks (the last K-step half empty), ragged last tile
    (33, 32, 32, 160, 1536),   # three slices, five channel blocks
]


@pytest.mark.parametrize("shape", RING_SHAPES)
@pytest.mark.parametrize("flags", [2, 3])  # shortcut, shortcut + ReLU
def test_ring_1x1_shortcut(ifx, orc, shape, flags):
    n, h, w, c, oc = shape
    note(f"ring 1x1 {shape} flags={flags}")
    rng = np.random.default_rng(sum(shape) * 5 + flags)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, 1, 1, c), -127, 127)
    bias, mult, shift = params(rng, oc, 0, 20)  # shifts 0-1 take the general requantisation
    res = rand(rng, (n, h, w, oc), -128, 127)
    d = ifx.conv_desc(n, h, w, c, oc, 1, 1, 1, 0, flags)
    assert ifx.conv_kernel_name(d).startswith("conv1x1_ring_kernel<")
    got = gpu_conv(ifx, x, wt, bias, mult, shift, 1, 1, 0, flags, res)
    idx = sorted({0, n // 2, n - 1})
    exp = orc.conv_fused(x[idx], wt, bias, mult, shift, 1, 0, flags, res[idx])
    np.testing.assert_array_equal(got[idx], exp)


# The phase-split layout between a bottleneck's conv1 and its stride-2 conv2: conv1 (the general
# kernel: 1x1 with K > 128, or a 3x3) stores its output as four parity planes, and the stride-2 3x3
# reads them, each tap a run of consecutive pixels.  Outputs are compared after undoing the
# permutation; inputs are permuted from the plain packed tensor.
PHASE_OUT_SHAPES = [
    (2, 28, 28, 512, 256, 1, 1, 0),   # res4.1 conv1
    (3, 14, 14, 1024, 512, 1, 1, 0),  # res5.1 conv1, 3 images of 196 pixels across tiles
    (2, 10, 6, 160, 200, 1, 1, 0),    # ragged channels, 5 input blocks
    (1, 12, 8, 96, 64, 3, 1, 1),      # a 3x3 producer (256x64 tiles)
]
PHASE_IN_SHAPES = [
    (2, 28, 28, 256, 256, 3, 2, 1),   # res4.1 conv2 (128x256 tiles of 64x128 sub-tiles)
    (2, 56, 56, 128, 128, 3, 2, 1),   # res3.1 conv2
    (3, 14, 14, 512, 512, 3, 2, 1),   # res5.1 conv2: 7x7 outputs
    (1, 10, 6, 96, 72, 3, 2, 1),      # odd output width, ragged channels
]


@pytest.mark.parametrize("shape", PHASE_OUT_SHAPES)
@pytest.mark.parametrize("flags", [0, 1])
def test_phase_split_output(ifx, orc, shape, flags):
    n, h, w, c, oc, k, s, p = shape
    note(f"phase-split output {shape} flags={flags}")
    rng = np.random.default_rng(sum(shape) + 3 * flags)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    bias, mult, shift = params(rng, oc)
    d = ifx.conv_desc(n, h, w, c, oc, k, k, s, p, flags | ifx.OUT_PHASE)
    ho, wo = ifx.conv_out_dims(d)
    c1 = (oc + 31) // 32
    y, whole = guarded(ifx.act_bytes(n, ho, wo, oc))
    dp = ifx.conv_desc(n, h, w, c, oc, k, k, s, p, flags)  # the plain descriptor packs the weights
    ifx.conv_fused(d, ifx.pack_act(cu(x)), ifx.pack_weights(dp, cu(wt)), cu(bias), cu(mult), cu(shift), None, y)
    torch.cuda.synchronize()
    check_guards(whole)
    got = ifx.unpack_act(from_phase(y, n, c1, ho, wo).contiguous(), oc).cpu().numpy()
    np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, s, p, flags))


@pytest.mark.parametrize("shape", PHASE_IN_SHAPES)
@pytest.mark.parametrize("flags", [0, 1])
def test_phase_split_input(ifx, orc, shape, flags):
    n, h, w, c, oc, k, s, p = shape
    note(f"phase-split input {shape} flags={flags}")
    rng = np.random.default_rng(sum(shape) + 5 * flags)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    bias, mult, shift = params(rng, oc)
    d = ifx.conv_desc(n, h, w, c, oc, k, k, s, p, flags | ifx.IN_PHASE)
    dp = ifx.conv_desc(n, h, w, c, oc, k, k, s, p, flags)
    ho, wo = ifx.conv_out_dims(d)
    xb = ifx.pack_act(cu(x)).view(n, (c + 31) // 32, h, w, 32)
    y, whole = guarded(ifx.act_bytes(n, ho, wo, oc))
    ifx.conv_fused(d, to_phase(xb), ifx.pack_weights(dp, cu(wt)), cu(bias), cu(mult), cu(shift), None, y)
    torch.cuda.synchronize()
    check_guards(whole)
    got = ifx.unpack_act(y.view(n, (oc + 31) // 32, ho, wo, 32), oc).cpu().numpy()
    np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, s, p, flags))


def test_requant_edges(ifx, orc):
    """shift 0 and 1 (general path), mult 0 and 2^31-1, exact ties, negative values."""
    note("requant edges")
    rng = np.random.default_rng(5)
    n, h, w, c, oc = 2, 6, 5, 64, 128
    x = rand(rng, (n, h, w, c), -128, 127)
    wt = rand(rng, (oc, 1, 1, c), -127, 127)
    bias = rand(rng, oc, -(1 << 16), 1 << 16, np.int32)
    shift = np.tile(np.array([0, 1, 2, 3, 31, 30, 16, 8], np.int32), oc // 8)
    mult = np.tile(np.array([1 << 30, (1 << 31) - 1, 0, 1, (1 << 31) - 1, 1 << 29, 12345, 1 << 30], np.int32), oc // 8)
    for flags in (0, ifx.RELU):
        got = gpu_conv(ifx, x, wt, bias, mult, shift, 1, 1, 0, flags)
        np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, 1, 0, flags))
    # all channels on the fast path but with ties: mult = 2^30, shift = 2 -> y/8, ties at y = 8j+4
    mult2 = np.full(oc, 1 << 30, np.int32)
    shift2 = np.full(oc, 2, np.int32)
    got = gpu_conv(ifx, x, wt, bias, mult2, shift2, 1, 1, 0, 0)
    np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult2, shift2, 1, 0, 0))


@pytest.mark.parametrize("k", [1, 3])
def test_requant_ties_with_shortcut(ifx, orc, k):
    """The requantisation modes with a shortcut: channel groups whose multipliers can tie
    (2^30, 3*2^28, shift 2-4: the tie-correcting path) beside tie-free ones (odd multipliers:
    the one-multiply path); negative sums near halfway, through the small-K and general kernels."""
    note(f"requant ties with shortcut k={k}")
    rng = np.random.default_rng(17 + k)
    n, h, w, c, oc = 2, 9, 7, 64 if k == 1 else 96, 128
    x = rand(rng, (n, h, w, c), -128, 127)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    bias = rand(rng, oc, -(1 << 12), 1 << 12, np.int32)
    # 64-channel groups (one wave each): tie-prone, tie-free, then mixed within the group
    mult = np.empty(oc, np.int32)
    mult[:64] = np.tile(np.array([1 << 30, 3 << 28], np.int32), 32)
    mult[64:] = rand(rng, 64, 1 << 30, (1 << 31) - 1, np.int32) | 1
    mult[96:100] = 1 << 30
    shift = np.tile(np.array([2, 3, 4, 2], np.int32), oc // 4)
    ho, wo = orc.out_dim(h, k, 1, k // 2), orc.out_dim(w, k, 1, k // 2)
    res = rand(rng, (n, ho, wo, oc), -128, 127)
    for flags in (ifx.RESIDUAL, ifx.RESIDUAL | ifx.RELU):
        got = gpu_conv(ifx, x, wt, bias, mult, shift, k, 1, k // 2, flags, res)
        np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, 1, k // 2, flags, res))


@pytest.mark.parametrize("c,k", [(64, 1), (256, 1), (64, 3)])
def test_requant_int32_min_sum(ifx, orc, c, k):
    """acc + bias = -2^31 exactly (zero input, bias INT32_MIN, which the BN folding emits when it
    clamps): with a multiplier of exactly shift - 1 trailing zero bits the value is a rounding
    tie, so the tie-correcting requantisation must run.  Small-K 1x1 (c = 64), general 1x1
    (c = 256) and 3x3 kernels; with and without a shortcut."""
    note(f"requant int32-min sum c={c} k={k}")
    rng = np.random.default_rng(31 + c + k)
    n, h, w, oc = 2, 6, 5, 128
    x = np.zeros((n, h, w, c), np.int8)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    bias = np.full(oc, -(1 << 31), np.int32)
    # y * m / 2^(31+s) = -m / 2^s: -1/2, -3/2, -255/2 (ties) and -1/2 - 2^-31 (no tie)
    mult = np.tile(np.array([128, 3 << 14, 255 << 7, (1 << 30) | 1], np.int32), oc // 4)
    shift = np.tile(np.array([8, 15, 8, 31], np.int32), oc // 4)
    res = rand(rng, (n, h, w, oc), -128, 127)
    for flags in (0, ifx.RESIDUAL, ifx.RESIDUAL | ifx.RELU):
        r = res if flags & ifx.RESIDUAL else None
        got = gpu_conv(ifx, x, wt, bias, mult, shift, k, 1, k // 2, flags, r)
        exp = orc.conv_fused(x, wt, bias, mult, shift, 1, k // 2, flags, r)
        np.testing.assert_array_equal(got, exp)
    # the values themselves, rounded away from zero: -1, -2, -128, -1
    exp = orc.conv_fused(x, wt, bias, mult, shift, 1, k // 2, 0)
    assert np.all(exp[..., 0::4] == -1) and np.all(exp[..., 1::4] == -2)
    assert np.all(exp[..., 2::4] == -128) and np.all(exp[..., 3::4] == -1)


def test_identity_halves(ifx, orc):
    """The golden identity case on the GPU: out = round_half_away(x / 2)."""
    note("identity halves")
    vals = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    c = 256
    x = vals.reshape(1, 1, 1, c)
    wt = np.zeros((c, 1, 1, c), np.int8)
    wt[np.arange(c), 0, 0, np.arange(c)] = 1
    z = np.zeros(c, np.int32)
    got = gpu_conv(ifx, x, wt, z, np.full(c, 1 << 30, np.int32), z, 1, 1, 0, 0).reshape(-1)
    exp = np.sign(vals.astype(np.int64)) * ((np.abs(vals.astype(np.int64)) + 1) // 2)
    np.testing.assert_array_equal(got.astype(np.int64), exp)


def test_fuzz_small_shapes(ifx, orc):
    rng = np.random.default_rng(2024)
    ksp = [(1, 1, 0), (1, 2, 0), (3, 1, 1), (3, 2, 1)]
    for it in range(24):
        k, s, p = ksp[it % 4]
        n = int(rng.integers(1, 4))
        h, w = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        c = int(rng.choice([3, 32, 64, 96, 17]))
        oc = int(rng.choice([32, 64, 96, 40, 160, 256]))
        flags = int(rng.integers(0, 4))
        note(f"fuzz it={it} n={n} h={h} w={w} c={c} oc={oc} k={k} s={s} flags={flags}")
        x = rand(rng, (n, h, w, c), -128, 127)
        wt = rand(rng, (oc, k, k, c), -127, 127)
        bias, mult, shift = params(rng, oc, 0, 20)
        ho, wo = orc.out_dim(h, k, s, p), orc.out_dim(w, k, s, p)
        res = rand(rng, (n, ho, wo, oc), -128, 127) if flags & ifx.RESIDUAL else None
        got = gpu_conv(ifx, x, wt, bias, mult, shift, k, s, p, flags, res)
        np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, s, p, flags, res))


# ------------------------------------------------------------------ bottleneck with projection
# (n, h, w, c_in, c_mid, c_out, stride, c3 kernel): conv3 and the projection run as one kernel
# when both are 1x1 (the shortcut tile never reaches HBM); a 3x3 conv3 takes the unfused path.
PROJ_BLOCKS = [
    (3, 9, 9, 96, 48, 160, 2, 1),    # strided, two output-channel tiles, padded channels
    (2, 13, 11, 64, 32, 96, 1, 1),   # unit stride, ragged pixel tile
    (1, 7, 7, 256, 64, 64, 1, 1),    # 64 output channels: the tall tile shape
    (5, 11, 6, 40, 24, 200, 2, 1),   # odd channel-block counts (32-channel blocks 2 and 1)
    (2, 8, 8, 64, 32, 128, 1, 3),    # 3x3 conv3: projection and conv3 launched separately
    (1, 14, 14, 1024, 256, 1024, 2, 1),  # batch 1, long K: c1 (8 parts) and c2 (18 parts) split K
    (1, 9, 9, 96, 200, 96, 1, 3),    # 63 blocks in 16 parts (odd tail), 200 channels (padding
                                     # groups); the split 3x3 conv3 adds the shortcut
]


@pytest.mark.parametrize("shape", PROJ_BLOCKS)
def test_projection_block(ifx, orc, shape):
    from oracle.ref import ConvParams
    n, h, w, c_in, c_mid, c_out, s, k3 = shape
    note(f"projection block {shape}")
    rng = np.random.default_rng(sum(shape) * 13)
    x = rand(rng, (n, h, w, c_in), 0, 127)
    # (c_in, c_out, k, stride, pad, flags) of c1, c2, c3 and the projection
    layers = [(c_in, c_mid, 1, 1, 0, ifx.RELU), (c_mid, c_mid, 3, s, 1, ifx.RELU),
              (c_mid, c_out, k3, 1, k3 // 2, ifx.RESIDUAL | ifx.RELU), (c_in, c_out, 1, s, 0, 0)]
    hs = [(h, w), (h, w)]
    ho, wo = orc.out_dim(h, 3, s, 1), orc.out_dim(w, 3, s, 1)
    hs += [(ho, wo), (h, w)]
    bp = ifx.BlockParams()
    keep, cps = [], []
    for i, ((ci, co, k, st, pd, fl), (hh, ww)) in enumerate(zip(layers, hs)):
        wt = rand(rng, (co, k, k, ci), -127, 127)
        bias, mult, shift = params(rng, co, 0, 20)
        d = ifx.conv_desc(n, hh, ww, ci, co, k, k, st, pd, fl)
        tensors = [ifx.pack_weights(d, cu(wt)), cu(bias), cu(mult), cu(shift)]
        keep += tensors
        bp.d[i] = d
        bp.w_blk[i], bp.bias[i], bp.mult[i], bp.shift[i] = (t.data_ptr() for t in tensors)
        cps.append(ConvParams(wt, bias, mult, shift, st, pd))
    bp.has_proj = 1
    if k3 == 1:
        # the same conv3 + projection through the public one-launch entry point
        t = rand(rng, (n, ho, wo, c_mid), 0, 127)
        y, whole = guarded(ifx.act_bytes(n, ho, wo, c_out))
        ifx.conv_proj_fused(bp.d[2], ifx.pack_act(cu(t)), *keep[8:12], bp.d[3], ifx.pack_act(cu(x)), *keep[12:16], y)
        torch.cuda.synchronize()
        check_guards(whole)
        got = ifx.unpack_act(y.view(n, (c_out + 31) // 32, ho, wo, 32), c_out).cpu().numpy()
        sc = orc.conv_layer(x, cps[3], 0)
        np.testing.assert_array_equal(got, orc.conv_layer(t, cps[2], ifx.RESIDUAL | ifx.RELU, residual=sc))
    ws = torch.empty(ifx.block_workspace_bytes(bp), dtype=torch.int8, device="cuda")
    nbytes = ifx.act_bytes(n, ho, wo, c_out)
    for rep in range(2):
        y, whole = guarded(nbytes)
        ifx.block_forward(bp, ifx.pack_act(cu(x)), y, ws)
        torch.cuda.synchronize()
        check_guards(whole)
        got = ifx.unpack_act(y.view(n, (c_out + 31) // 32, ho, wo, 32), c_out).cpu().numpy()
        exp = orc.block(x, cps[0], cps[1], cps[2], cps[3])
        np.testing.assert_array_equal(got, exp)


# conv3 + projection with 256 or more output channels over at least 2048 tiles of 128x256 runs
# the wide-tile form that keeps the requantised projection in registers: (n, ho, c_mid, c_in,
# c_out, projection stride).  Sampled images are compared.
PROJ_WIDE_SHAPES = [
    (340, 14, 256, 512, 1024, 2),  # res4.1: stride-2 projection on 28x28, a ragged last tile
    (672, 7, 512, 1024, 2048, 1),  # res5.1 on the even-pixel copy (stride 1)
]


@pytest.mark.parametrize("shape", PROJ_WIDE_SHAPES)
def test_projection_wide_tiles(ifx, orc, shape):
    from oracle.ref import ConvParams
    n, ho, c_mid, c_in, c_out, s = shape
    note(f"projection wide tiles {shape}")
    rng = np.random.default_rng(sum(shape) * 17)
    hi = ho * s
    t = rand(rng, (n, ho, ho, c_mid), 0, 127)
    x = rand(rng, (n, hi, hi, c_in), 0, 127)
    w3 = rand(rng, (c_out, 1, 1, c_mid), -127, 127)
    wp = rand(rng, (c_out, 1, 1, c_in), -127, 127)
    p3 = params(rng, c_out, 0, 20) if s == 2 else params(rng, c_out)
    pp = params(rng, c_out, 0, 20) if s == 2 else params(rng, c_out)
    d3 = ifx.conv_desc(n, ho, ho, c_mid, c_out, 1, 1, 1, 0, ifx.RESIDUAL | ifx.RELU)
    dp = ifx.conv_desc(n, hi, hi, c_in, c_out, 1, 1, s, 0, 0)
    assert ifx.conv_kernel_name(d3, dp) == "igemm_kernel<1, 1, 128, 256, 2, 128, true, true, true>"
    y, whole = guarded(ifx.act_bytes(n, ho, ho, c_out))
    ifx.conv_proj_fused(d3, ifx.pack_act(cu(t)), ifx.pack_weights(d3, cu(w3)), *(cu(v) for v in p3), dp,
                        ifx.pack_act(cu(x)), ifx.pack_weights(dp, cu(wp)), *(cu(v) for v in pp), y)
    torch.cuda.synchronize()
    check_guards(whole)
    idx = sorted({0, 1, n // 2, n - 1})
    got = ifx.unpack_act(y.view(n, c_out // 32, ho, ho, 32), c_out).cpu().numpy()[idx]
    sc = orc.conv_layer(x[idx], ConvParams(wp, *pp, s, 0), 0)
    exp = orc.conv_layer(t[idx], ConvParams(w3, *p3, 1, 0), ifx.RESIDUAL | ifx.RELU, residual=sc)
    np.testing.assert_array_equal(got, exp)


# A conv3 with shortcut that also stores its output's even pixels (ifx_conv_fused_even):
# (n, h, w, c_in, c_out, k): the ring kernel (K <= 128, 256 / 512 channels) and the general kernel
EVEN_COPY_SHAPES = [
    (3, 28, 28, 128, 512, 1),  # res3.4 conv3 (ring kernel), 2352 pixels across images
    (2, 14, 14, 256, 1024, 1),  # res4.6 conv3 shape at batch 2 (general kernel)
    (168, 14, 14, 256, 1024, 1),  # ... at a batch of 512+ tiles (ring kernel, two channel slices)
    (3, 7, 7, 512, 2048, 1),   # odd sizes: a 4x4 copy of a 7x7 output
    (2, 9, 11, 96, 256, 1),    # ring kernel with odd height, ragged last tile
    (1, 9, 9, 64, 128, 3),     # a 3x3 general-kernel conv3
]


@pytest.mark.parametrize("shape", EVEN_COPY_SHAPES)
@pytest.mark.parametrize("flags", [2, 3])
def test_conv_fused_even_copy(ifx, orc, shape, flags):
    n, h, w, c, oc, k = shape
    note(f"even copy {shape} flags={flags}")
    rng = np.random.default_rng(sum(shape) * 19 + flags)
    x = rand(rng, (n, h, w, c), 0, 127)
    wt = rand(rng, (oc, k, k, c), -127, 127)
    bias, mult, shift = params(rng, oc)
    r = rand(rng, (n, h, w, oc), -128, 127)
    d = ifx.conv_desc(n, h, w, c, oc, k, k, 1, k // 2, flags)
    assert ifx.conv_even_supported(d)
    he, we = (h + 1) // 2, (w + 1) // 2
    y, yw = guarded(ifx.act_bytes(n, h, w, oc))
    ye, ew = guarded(ifx.act_bytes(n, he, we, oc))
    ifx.conv_fused_even(d, ifx.pack_act(cu(x)), ifx.pack_weights(d, cu(wt)), cu(bias), cu(mult), cu(shift),
                        ifx.pack_act(cu(r)), y, ye)
    torch.cuda.synchronize()
    check_guards(yw)
    check_guards(ew)
    exp = orc.conv_fused(x, wt, bias, mult, shift, 1, k // 2, flags, r)
    got = ifx.unpack_act(y.view(n, (oc + 31) // 32, h, w, 32), oc).cpu().numpy()
    np.testing.assert_array_equal(got, exp)
    got_e = ifx.unpack_act(ye.view(n, (oc + 31) // 32, he, we, 32), oc).cpu().numpy()
    np.testing.assert_array_equal(got_e, exp[:, ::2, ::2])


def test_conv_fused_even_unsupported(ifx):
    """A kernel that does not write the copy refuses the call and launches nothing."""
    d = ifx.conv_desc(2, 6, 6, 64, 128, 1, 1, 1, 0, ifx.RELU)  # the small-K 1x1 kernel
    assert not ifx.conv_even_supported(d)
    x = torch.zeros(ifx.act_bytes(2, 6, 6, 64), dtype=torch.int8, device="cuda")
    w = ifx.pack_weights(d, torch.zeros((128, 1, 1, 64), dtype=torch.int8, device="cuda"))
    p = torch.zeros(128, dtype=torch.int32, device="cuda")
    y = torch.full((ifx.act_bytes(2, 6, 6, 128),), 5, dtype=torch.int8, device="cuda")
    ye = torch.full((ifx.act_bytes(2, 3, 3, 128),), 5, dtype=torch.int8, device="cuda")
    with pytest.raises(ifx.IfxError):
        ifx.conv_fused_even(d, x, w, p, p, p, None, y, ye)
    torch.cuda.synchronize()
    assert bool((y == 5).all()) and bool((ye == 5).all())


# conv3 (64 < K <= 128, 512 output channels) with a unit-stride 1x1 projection (128 < K <= 256) in
# the persistent ring kernel: (n, h, w, conv3 input channels, projection input channels)
RING_PROJ_SHAPES = [
    (4, 28, 28, 128, 256),   # res3.1 after its input was stored subsampled
    (3, 9, 7, 100, 200),     # ragged last tile, padded channel blocks on both inputs
    (1, 5, 6, 96, 160),      # one partial tile, three and five K-blocks
]


@pytest.mark.parametrize("shape", RING_PROJ_SHAPES)
def test_ring_projection(ifx, orc, shape):
    from oracle.ref import ConvParams
    n, h, w, c3in, cpin = shape
    note(f"ring projection {shape}")
    rng = np.random.default_rng(sum(shape) * 17)
    t = rand(rng, (n, h, w, c3in), 0, 127)
    x = rand(rng, (n, h, w, cpin), 0, 127)
    w3 = rand(rng, (512, 1, 1, c3in), -127, 127)
    wp = rand(rng, (512, 1, 1, cpin), -127, 127)
    b3, m3, s3 = params(rng, 512, 0, 20)
    bp, mp, sp = params(rng, 512, 0, 20)
    d3 = ifx.conv_desc(n, h, w, c3in, 512, 1, 1, 1, 0, ifx.RESIDUAL | ifx.RELU)
    dp = ifx.conv_desc(n, h, w, cpin, 512, 1, 1, 1, 0, 0)
    assert ifx.conv_kernel_name(d3, dp).startswith("conv1x1_ring_kernel<8, 2, 4, 64, true>")
    y, yw = guarded(ifx.act_bytes(n, h, w, 512))
    ifx.conv_proj_fused(d3, ifx.pack_act(cu(t)), ifx.pack_weights(d3, cu(w3)), cu(b3), cu(m3), cu(s3),
                        dp, ifx.pack_act(cu(x)), ifx.pack_weights(dp, cu(wp)), cu(bp), cu(mp), cu(sp), y)
    torch.cuda.synchronize()
    check_guards(yw)
    got = ifx.unpack_act(y.view(n, 16, h, w, 32), 512).cpu().numpy()
    sc = orc.conv_layer(x, ConvParams(wp, bp, mp, sp, 1, 0), 0)
    exp = orc.conv_layer(t, ConvParams(w3, b3, m3, s3, 1, 0), ifx.RESIDUAL | ifx.RELU, residual=sc)
    np.testing.assert_array_equal(got, exp)


# ------------------------------------------------------------------ conv3 chained with the next conv1
# (n, h, w, c_in of conv3, conv1 output channels, conv1 flags): conv3 is 1x1 c_in -> 256 with
# shortcut and ReLU, conv1 1x1 256 -> N1; pixel counts that are and are not multiples of the
# 64-pixel tile, a padded channel block in conv3's input
# conv3 + its projection shortcut + the next conv1 (64 channels) in one launch:
# (n, h, w, conv3 input channels, projection input channels, conv1 flags)
PROJ_CHAIN_SHAPES = [
    (2, 56, 56, 64, 64, 1),    # the res2.1 -> res2.2 shape
    (3, 9, 7, 40, 32, 0),      # ragged last tile, one-block projection input, conv1 without ReLU
    (1, 5, 6, 64, 48, 1),      # one partial tile
]


@pytest.mark.parametrize("shape", PROJ_CHAIN_SHAPES)
def test_conv_proj_chain_fused(ifx, orc, shape):
    n, h, w, c3in, cpin, f1 = shape
    note(f"proj chain {shape}")
    rng = np.random.default_rng(sum(shape) * 13)
    t2 = rand(rng, (n, h, w, c3in), 0, 127)
    x = rand(rng, (n, h, w, cpin), 0, 127)
    w3 = rand(rng, (256, 1, 1, c3in), -127, 127)
    wp = rand(rng, (256, 1, 1, cpin), -127, 127)
    w1 = rand(rng, (64, 1, 1, 256), -127, 127)
    b3, m3, s3 = params(rng, 256, 0, 20)
    bp, mp, sp = params(rng, 256, 0, 20)
    b1, m1, s1 = params(rng, 64, 0, 20)
    d3 = ifx.conv_desc(n, h, w, c3in, 256, 1, 1, 1, 0, ifx.RESIDUAL | ifx.RELU)
    dp = ifx.conv_desc(n, h, w, cpin, 256, 1, 1, 1, 0, 0)
    d1 = ifx.conv_desc(n, h, w, 256, 64, 1, 1, 1, 0, f1)
    assert ifx.conv_proj_chain_kernel_name(d3, dp, d1).endswith(", true>")
    y, yw = guarded(ifx.act_bytes(n, h, w, 256))
    t1, tw = guarded(ifx.act_bytes(n, h, w, 64))
    ifx.conv_proj_chain_fused(d3, ifx.pack_act(cu(t2)), ifx.pack_weights(d3, cu(w3)), cu(b3), cu(m3), cu(s3),
                              dp, ifx.pack_act(cu(x)), ifx.pack_weights(dp, cu(wp)), cu(bp), cu(mp), cu(sp),
                              y, d1, ifx.pack_weights(d1, cu(w1)), cu(b1), cu(m1), cu(s1), t1)
    torch.cuda.synchronize()
    check_guards(yw)
    check_guards(tw)
    sc = orc.conv_fused(x, wp, bp, mp, sp, 1, 0, 0)
    exp_y = orc.conv_fused(t2, w3, b3, m3, s3, 1, 0, ifx.RESIDUAL | ifx.RELU, sc)
    exp_t1 = orc.conv_fused(exp_y, w1, b1, m1, s1, 1, 0, f1)
    np.testing.assert_array_equal(ifx.unpack_act(y.view(n, 8, h, w, 32), 256).cpu().numpy(), exp_y)
    np.testing.assert_array_equal(ifx.unpack_act(t1.view(n, 2, h, w, 32), 64).cpu().numpy(), exp_t1)


# (n, h, w, conv3 input channels, block-output channels, conv1 output channels, conv1 flags,
#  y at even pixels only, t1 phase-split)
CHAIN_SHAPES = [
    (2, 56, 56, 64, 256, 64, 1, False, False),    # the res2.2 -> res2.3 shape
    (1, 56, 56, 64, 256, 128, 1, True, True),     # res2.3 -> res3.1 (a stride-2 projection and conv2 follow)
    (1, 56, 56, 64, 256, 128, 1, False, False),
    (3, 9, 7, 40, 256, 64, 0, False, False),      # 189 pixels: a ragged last tile; conv1 without ReLU
    (3, 9, 7, 40, 256, 128, 1, True, False),      # odd height and width: the last row and column are even
    (1, 6, 6, 32, 256, 128, 0, False, True),      # one partial tile
    (2, 6, 10, 64, 256, 64, 0, True, False),      # even sizes, tiles spanning images
    (3, 28, 28, 128, 512, 128, 1, False, False),  # the res3.2 -> res3.3 shape (eight waves, K = 128)
    (2, 7, 9, 96, 512, 128, 0, False, False),     # K = 96 (second K-step half zero), ragged tiles
]


@pytest.mark.parametrize("shape", CHAIN_SHAPES)
def test_conv_chain_fused(ifx, orc, shape):
    n, h, w, c3in, cb, n1, f1, even, ps = shape
    note(f"chain {shape}")
    rng = np.random.default_rng(sum(shape) * 11)
    t2 = rand(rng, (n, h, w, c3in), 0, 127)
    res = rand(rng, (n, h, w, cb), -128, 127)
    w3 = rand(rng, (cb, 1, 1, c3in), -127, 127)
    w1 = rand(rng, (n1, 1, 1, cb), -127, 127)
    b3, m3, s3 = params(rng, cb, 0, 20)
    b1, m1, s1 = params(rng, n1, 0, 20)
    d3p = ifx.conv_desc(n, h, w, c3in, cb, 1, 1, 1, 0, ifx.RESIDUAL | ifx.RELU)  # for the weight packs
    d1p = ifx.conv_desc(n, h, w, cb, n1, 1, 1, 1, 0, f1)
    d3 = ifx.conv_desc(n, h, w, c3in, cb, 1, 1, 1, 0, ifx.RESIDUAL | ifx.RELU | (ifx.OUT_EVEN if even else 0))
    d1 = ifx.conv_desc(n, h, w, cb, n1, 1, 1, 1, 0, f1 | (ifx.OUT_PHASE if ps else 0))
    assert ifx.conv_chain_kernel_name(d3, d1).endswith(", true, false>" if even else ", false, false>")
    hy, wy = ((h + 1) // 2, (w + 1) // 2) if even else (h, w)
    y, yw = guarded(ifx.act_bytes(n, hy, wy, cb))
    t1, tw = guarded(ifx.act_bytes(n, h, w, n1))
    ifx.conv_chain_fused(d3, ifx.pack_act(cu(t2)), ifx.pack_weights(d3p, cu(w3)), cu(b3), cu(m3), cu(s3),
                         ifx.pack_act(cu(res)), y, d1, ifx.pack_weights(d1p, cu(w1)), cu(b1), cu(m1), cu(s1), t1)
    torch.cuda.synchronize()
    check_guards(yw)
    check_guards(tw)
    exp_y = orc.conv_fused(t2, w3, b3, m3, s3, 1, 0, ifx.RESIDUAL | ifx.RELU, res)
    exp_t1 = orc.conv_fused(exp_y, w1, b1, m1, s1, 1, 0, f1)
    got_y = ifx.unpack_act(y.view(n, cb // 32, hy, wy, 32), cb).cpu().numpy()
    np.testing.assert_array_equal(got_y, exp_y[:, ::2, ::2] if even else exp_y)
    t1p = from_phase(t1, n, n1 // 32, h, w).contiguous() if ps else t1.view(n, n1 // 32, h, w, 32)
    np.testing.assert_array_equal(ifx.unpack_act(t1p, n1).cpu().numpy(), exp_t1)


# ------------------------------------------------------------------ stem
@pytest.mark.parametrize("n,h,w,c", [(2, 224, 224, 3), (1, 37, 45, 3), (3, 16, 16, 4), (1, 2, 3, 1)])
def test_stem(ifx, orc, n, h, w, c):
    note(f"stem n={n} h={h} w={w} c={c}")
    rng = np.random.default_rng(h + w + c)
    x = rand(rng, (n, h, w, c), -128, 127)
    wt = rand(rng, (64, 7, 7, c), -127, 127)
    bias, mult, shift = params(rng, 64)
    for flags in (ifx.RELU | ifx.MAXPOOL, ifx.MAXPOOL):
        got = gpu_conv(ifx, x, wt, bias, mult, shift, 7, 2, 3, flags)
        np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, 2, 3, flags))


@pytest.mark.parametrize("n,h,w,c", [(2, 224, 224, 3), (1, 37, 45, 3), (2, 40, 44, 3), (1, 9, 12, 3),
                                     (3, 16, 16, 4), (1, 2, 3, 1), (2, 30, 28, 2)])
def test_stem_nhwc_input(ifx, orc, n, h, w, c):
    """The stem reading the compact NHWC image (aligned 3-channel path when
    w % 4 == 0, byte path otherwise) gives the packed-input stem's result."""
    note(f"stem nhwc n={n} h={h} w={w} c={c}")
    rng = np.random.default_rng(7 * h + w + c)
    x = rand(rng, (n, h, w, c), -128, 127)
    wt = rand(rng, (64, 7, 7, c), -127, 127)
    bias, mult, shift = params(rng, 64)
    for flags in (ifx.RELU | ifx.MAXPOOL, ifx.MAXPOOL):
        got = gpu_conv(ifx, x, wt, bias, mult, shift, 7, 2, 3, flags | ifx.INPUT_NHWC)
        np.testing.assert_array_equal(got, orc.conv_fused(x, wt, bias, mult, shift, 2, 3, flags))


@pytest.mark.parametrize("nhwc", [False, True])
def test_stem_requant_edges(ifx, orc, nhwc):
    """The stem's three requantisation forms on pooled accumulators: shifts 0 and 1 (the general
    form), the tie-correcting form without ReLU (mult 2^30, shift 2: ties at y = 8j + 4), mult 0,
    1 and 2^31 - 1, through the packed and the compact NHWC input paths.  The pooled maximum is
    what gets requantised, which the epilogue allows for mult >= 0 only, so no mult is negative."""
    note(f"stem requant edges nhwc={nhwc}")
    rng = np.random.default_rng(31 + nhwc)
    n, h, w, c = 2, 40, 44, 3
    x = rand(rng, (n, h, w, c), -128, 127)
    wt = rand(rng, (64, 7, 7, c), -8, 8)  # small weights: many pooled sums near the tie points
    bias = rand(rng, 64, -(1 << 10), 1 << 10, np.int32)
    shift = np.tile(np.array([0, 1, 2, 3, 31, 30, 16, 8], np.int32), 8)
    mult = np.tile(np.array([1 << 30, (1 << 31) - 1, 0, 1, (1 << 31) - 1, 1 << 29, 12345, 1 << 30], np.int32), 8)
    # the tie case with a negative bias: about 2 % of the pooled sums are negative exact ties inside the
    # int8 range, where rounding half away from zero and half up differ
    ties = (rand(rng, 64, -9000, -5000, np.int32), np.full(64, 1 << 30, np.int32), np.full(64, 2, np.int32))
    extra = ifx.INPUT_NHWC if nhwc else 0
    for b_, m_, s_ in ((bias, mult, shift), ties):
        for flags in (ifx.RELU | ifx.MAXPOOL, ifx.MAXPOOL):
            got = gpu_conv(ifx, x, wt, b_, m_, s_, 7, 2, 3, flags | extra)
            np.testing.assert_array_equal(got, orc.conv_fused(x, wt, b_, m_, s_, 2, 3, flags))


# ------------------------------------------------------------------ small networks: pool and head
@pytest.mark.parametrize("n,h,w,nblk", [(2, 40, 44, 0), (1, 224, 224, 0), (3, 16, 16, 1), (1, 9, 12, 1),
                                        (515, 16, 16, 1), (4097, 9, 12, 0)])
def test_small_net_pool_and_head(ifx, orc, n, h, w, nblk):
    """Stem -> 0 or 1 bottleneck -> average pool -> FC through ifx_net_forward: the pool over
    9 to 3136 pixels per plane (pixel groups of the wave left partly empty) and the int32
    logits equal the oracle's; a batch run in single-image passes gives the same logits.
    515 images run as two concurrent halves (258 + 257) on two streams, eagerly and recorded
    as one graph (fork and join inside the capture), replayed with other work between.  4097
    images give halves of 4098 and 4096 pooled planes: the pool's eight-planes-per-wave
    mapping, with a partly filled last wave."""
    from oracle.ref import BlockParams as OracleBlock, ConvParams
    note(f"small net n={n} h={h} w={w} blocks={nblk}")
    rng = np.random.default_rng(n * 1000 + h + w + nblk)
    x = rand(rng, (n, h, w, 3), -128, 127)
    keep = []

    def conv(ci, co, k, st, pd, fl, hh, ww):
        wt = rand(rng, (co, k, k, ci), -127, 127)
        bias, mult, shift = params(rng, co, 0, 20)
        d = ifx.conv_desc(n, hh, ww, ci, co, k, k, st, pd, fl)
        t = [ifx.pack_weights(d, cu(wt)), cu(bias), cu(mult), cu(shift)]
        keep.extend(t)
        return d, t, ConvParams(wt, bias, mult, shift, st, pd)

    sd, st_, sp = conv(3, 64, 7, 2, 3, ifx.RELU | ifx.MAXPOOL | ifx.INPUT_NHWC, h, w)
    ph, pw = ifx.conv_out_dims(sd)
    p = ifx.NetParams()
    p.stem = sd
    p.stem_w, p.stem_bias, p.stem_mult, p.stem_shift = (t.data_ptr() for t in st_)
    blocks, c = [], 64
    if nblk:
        bp = ifx.BlockParams()
        layers = [(64, 32, 1, ifx.RELU), (32, 32, 3, ifx.RELU), (32, 128, 1, ifx.RESIDUAL | ifx.RELU), (64, 128, 1, 0)]
        cps = []
        for i, (ci, co, k, fl) in enumerate(layers):
            d, t, cp = conv(ci, co, k, 1, k // 2, fl, ph, pw)
            bp.d[i] = d
            bp.w_blk[i], bp.bias[i], bp.mult[i], bp.shift[i] = (q.data_ptr() for q in t)
            cps.append(cp)
        bp.has_proj = 1
        arr = (ifx.BlockParams * 1)(bp)
        keep.append(arr)
        p.blocks = ctypes.cast(arr, ctypes.POINTER(ifx.BlockParams))
        blocks.append(OracleBlock(*cps))
        c = 128
    p.n_blocks = nblk
    fc_out = 1000
    fw = rand(rng, (fc_out, c), -127, 127)
    fb = rand(rng, fc_out, -(1 << 20), 1 << 20, np.int32)
    fd = ifx.conv_desc(n, 1, 1, c, fc_out, 1, 1, 1, 0, ifx.OUT_I32)
    fwb, fbb = ifx.pack_weights(fd, cu(fw.reshape(fc_out, 1, 1, c))), cu(fb)
    keep += [fwb, fbb]
    p.fc_w_blk, p.fc_bias = fwb.data_ptr(), fbb.data_ptr()
    p.fc_in, p.fc_out = c, fc_out
    exp = orc.net(x, sp, blocks, fw, fb)
    xd = cu(x)
    for sub in (0, 1) if n < 64 else (0, 100):
        p.sub_batch = sub
        ws = torch.empty(ifx.net_workspace_bytes(p, n), dtype=torch.int8, device="cuda")
        logits, whole = guarded(n * fc_out * 4, torch.int32)
        ifx.net_forward(p, xd, logits, n, ws)
        torch.cuda.synchronize()
        check_guards(whole)
        np.testing.assert_array_equal(logits.view(n, fc_out).cpu().numpy(), exp)
    if n >= 192:
        p.sub_batch = 0
        ws = torch.empty(ifx.net_workspace_bytes(p, n), dtype=torch.int8, device="cuda")
        logits, whole = guarded(n * fc_out * 4, torch.int32)
        g = ifx.NetGraph(p, xd, logits, n, ws)
        for rep in range(3):
            note(f"two-lane graph replay {rep}")
            logits.fill_(-7)
            ws.fill_(rep)
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            check_guards(whole)
            np.testing.assert_array_equal(logits.view(n, fc_out).cpu().numpy(), exp)
        g.close()


# ------------------------------------------------------------------ determinism
def test_repeat_runs_identical(ifx):
    note("determinism res3 conv3 batch 64")
    from convolution_int8_implicit_amd import model, synth
    wl = synth.workload(1, n=64)
    spec = wl.convs[0]
    dc = model.device_conv(spec, wl.index, wl.n, wl.h, wl.w)
    xb = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
    rb = ifx.pack_act(synth.residual_tensor(wl, device="cuda"))
    outs = []
    for _ in range(3):
        y = torch.full((ifx.act_bytes(wl.n, 28, 28, 512),), SENT, dtype=torch.int8, device="cuda")
        dc.run(xb, y, rb)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ------------------------------------------------------------------ BN folding
def _fold_inputs(rng, n):
    g = rng.uniform(0.05, 4.0, n).astype(np.float32)
    g[::17] = -g[::17]                          # some channels not representable (status 2)
    be = rng.uniform(-3, 3, n).astype(np.float32)
    mu = rng.uniform(-2, 2, n).astype(np.float32)
    var = rng.uniform(0.0, 9.0, n).astype(np.float32)
    sw = (2.0 ** rng.uniform(-40, 2, n)).astype(np.float32)  # tiny, normal and >= 1 scales
    cb = rng.uniform(-1, 1, n).astype(np.float32)
    cb[::29] = 3e9                               # bias outside int32 (status 3)
    return sw, g, be, mu, var, cb


@pytest.mark.parametrize("n,per_channel,with_bias", [(1, True, False), (64, True, True), (1000, True, True),
                                                     (300, False, True), (2048, False, False)])
def test_fold_bn_matches_oracle(ifx, orc, n, per_channel, with_bias):
    note(f"fold_bn n={n} per_channel={per_channel} bias={with_bias}")
    rng = np.random.default_rng(n + per_channel)
    sw, g, be, mu, var, cb = _fold_inputs(rng, n)
    if not per_channel:
        sw = sw[:1]
    xs, ys, eps = 0.0173, 0.0411, 1e-5
    got = ifx.fold_bn(xs, ys, eps, cu(sw), cu(g), cu(be), cu(mu), cu(var), cu(cb) if with_bias else None)
    torch.cuda.synchronize()
    exp = orc.fold_bn(xs, ys, eps, sw, g, be, mu, var, conv_bias=cb if with_bias else None)
    for name, a, b in zip(("bias", "mult", "shift", "status"), got, exp):
        np.testing.assert_array_equal(a.cpu().numpy(), b, err_msg=name)


def test_fold_bn_feeds_the_fused_conv(ifx, orc):
    """Parameters derived on the device drive ifx_conv_fused to the oracle's result."""
    note("fold_bn -> conv_fused")
    rng = np.random.default_rng(77)
    oc, c = 64, 96
    g = rng.uniform(0.2, 2.0, oc).astype(np.float32)
    be, mu = rng.uniform(-1, 1, oc).astype(np.float32), rng.uniform(-1, 1, oc).astype(np.float32)
    var = rng.uniform(0.2, 3.0, oc).astype(np.float32)
    sw = (2.0 ** rng.uniform(-9, -6, oc)).astype(np.float32)
    bias, mult, shift, st = ifx.fold_bn(0.02, 0.05, 1e-5, cu(sw), cu(g), cu(be), cu(mu), cu(var))
    assert int(st.abs().sum()) == 0
    x = rand(rng, (2, 9, 11, c), 0, 127)
    wt = rand(rng, (oc, 3, 3, c), -127, 127)
    b_, m_, s_ = bias.cpu().numpy(), mult.cpu().numpy(), shift.cpu().numpy()
    got = gpu_conv(ifx, x, wt, b_, m_, s_, 3, 1, 1, ifx.RELU)
    np.testing.assert_array_equal(got, orc.conv_fused(x, wt, b_, m_, s_, 1, 1, ifx.RELU))


# ------------------------------------------------------------------ input quantisation, logits
def _round_up16(n):
    return (n + 15) // 16 * 16


@pytest.mark.parametrize("shape", [(2, 224, 224, 3), (1, 7, 5, 3), (3, 1, 1, 1), (1, 3, 3, 5), (1, 1, 1, 6)])
def test_quantize_f32(ifx, orc, shape):
    """fp32 NHWC image -> int8 codes, element by element against the oracle: random values, exact
    ties (channel 0 has mult 1), saturation, +-inf and NaN; counts with a ragged tail (count % 4)
    written inside guard bands."""
    note(f"quantize_f32 {shape}")
    rng = np.random.default_rng(sum(shape) + 11)
    c = shape[-1]
    x = rng.normal(0, 60, shape).astype(np.float32)
    mult = rng.uniform(0.5, 2.0, c).astype(np.float32)
    mult[0] = 1.0
    flat = x.reshape(-1)
    ch0 = flat[0::c]
    k = min(ch0.size, 64)
    ch0[:k] = np.arange(k) - k // 2 + 0.5            # exact ties at mult 1
    flat[0::c] = ch0
    specials = np.array([np.nan, np.inf, -np.inf, 1e30, -1e30, 127.5, -128.5], np.float32)
    m = min(specials.size, flat.size)
    flat[flat.size - m:] = specials[:m]
    q, whole = guarded(_round_up16(flat.size))
    ifx.quantize_f32(cu(x), cu(mult), out=q[:flat.size].view(shape))
    torch.cuda.synchronize()
    check_guards(whole)
    np.testing.assert_array_equal(q[:flat.size].cpu().numpy().reshape(shape), orc.quantize_f32(x, mult))


@pytest.mark.parametrize("shape", [(2, 224, 224, 3), (1, 9, 7, 3), (2, 1, 1, 1), (1, 2, 3, 5)])
def test_quantize_u8(ifx, orc, shape):
    """uint8 NHWC image -> int8 codes with ImageNet-style float32 means and 1 / (std * s_x)
    multipliers, and a channel with mean 127.5 and mult 1 (every code an exact tie)."""
    note(f"quantize_u8 {shape}")
    rng = np.random.default_rng(sum(shape) + 23)
    c = shape[-1]
    x = rand(rng, shape, 0, 255, np.uint8)
    mean = np.resize(np.array([123.675, 116.28, 103.53], np.float32), c)
    mult = np.resize((1.0 / (np.array([58.395, 57.12, 57.375]) * 0.02)).astype(np.float32), c)
    mean[0], mult[0] = 127.5, 1.0
    n = x.size
    q, whole = guarded(_round_up16(n))
    ifx.quantize_u8(cu(x), cu(mean), cu(mult), out=q[:n].view(shape))
    torch.cuda.synchronize()
    check_guards(whole)
    np.testing.assert_array_equal(q[:n].cpu().numpy().reshape(shape), orc.quantize_u8(x, mean, mult))


@pytest.mark.parametrize("shape", [(2048, 1000), (37, 1000), (1, 3), (5, 1)])
def test_dequantize_logits(ifx, orc, shape):
    """int32 logits -> float32: full-range values (conversions that round beyond 2^24) and a scale
    that is not a power of two, compared bit for bit."""
    note(f"dequantize {shape}")
    rng = np.random.default_rng(shape[0] + shape[1])
    q = rand(rng, shape, -(1 << 31), (1 << 31) - 1, np.int32)
    flat = q.reshape(-1)
    edge = np.array([(1 << 24) + 1, -((1 << 24) + 3), (1 << 31) - 1, -(1 << 31), 0], np.int32)
    flat[:min(edge.size, flat.size)] = edge[:flat.size]
    scale = np.float32(0.0123)
    n = q.size
    y, whole = guarded(_round_up16(4 * n), torch.float32)
    ifx.dequantize_i32(cu(q), float(scale), out=y[:n].view(shape))
    torch.cuda.synchronize()
    check_guards(whole)
    got = y[:n].cpu().numpy().reshape(shape)
    want = orc.dequantize_i32(q, scale)
    np.testing.assert_array_equal(got.view(np.int32), want.view(np.int32))


@pytest.mark.parametrize("u8", [False, True])
def test_quantized_image_feeds_the_stem(ifx, orc, u8):
    """The pre-processing and the stem chained on the device: an fp32 (or uint8) NHWC image quantised
    by ifx_quantize_* and read by the fused stem (IFX_INPUT_NHWC) equals the oracle's quantisation
    followed by the oracle's stem."""
    note(f"quantize -> stem u8={u8}")
    rng = np.random.default_rng(41 + u8)
    n, h, w, c = 2, 64, 64, 3
    mult = np.array([0.9, 1.1, 0.75], np.float32)
    if u8:
        x = rand(rng, (n, h, w, c), 0, 255, np.uint8)
        mean = np.array([123.675, 116.28, 103.53], np.float32)
        q = ifx.quantize_u8(cu(x), cu(mean), cu(mult))
        q_ref = orc.quantize_u8(x, mean, mult)
    else:
        x = rng.normal(0, 70, (n, h, w, c)).astype(np.float32)
        q = ifx.quantize_f32(cu(x), cu(mult))
        q_ref = orc.quantize_f32(x, mult)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    wt = rand(rng, (64, 7, 7, c), -127, 127)
    bias, mult_s, shift = params(rng, 64)
    flags = ifx.RELU | ifx.MAXPOOL
    got = gpu_conv(ifx, q.cpu().numpy(), wt, bias, mult_s, shift, 7, 2, 3, flags | ifx.INPUT_NHWC)
    np.testing.assert_array_equal(got, orc.conv_fused(q_ref, wt, bias, mult_s, shift, 2, 3, flags))
