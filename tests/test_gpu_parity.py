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
    # strided 3x3 with >= 256 output channels: 128x256 tiles of eight waves
    (2, 9, 11, 64, 256, 3, 2, 1),
    (1, 8, 7, 96, 288, 3, 2, 1),     # ragged output channels, odd channel-block count
    # stride-1 3x3, <= 64 input channels, 48 <= W <= 62: the haloed-window kernel (flags 0 and 1;
    # with a shortcut the general kernel runs)
    (2, 56, 56, 64, 64, 3, 1, 1),    # the res2 shape: 14 row bands of 4 rows
    (3, 13, 50, 40, 96, 3, 1, 1),    # ragged last band (13 rows), two channel blocks, padded channels
    (1, 7, 62, 32, 64, 3, 1, 1),     # widest window (pitch 64), one channel block
    (2, 5, 48, 64, 200, 3, 1, 1),    # narrowest, four output-channel tiles, padding in the last
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


# ------------------------------------------------------------------ small networks: pool and head
@pytest.mark.parametrize("n,h,w,nblk", [(2, 40, 44, 0), (1, 224, 224, 0), (3, 16, 16, 1), (1, 9, 12, 1),
                                        (515, 16, 16, 1)])
def test_small_net_pool_and_head(ifx, orc, n, h, w, nblk):
    """Stem -> 0 or 1 bottleneck -> average pool -> FC through ifx_net_forward: the pool over
    9 to 3136 pixels per plane (pixel groups of the wave left partly empty) and the int32
    logits equal the oracle's; a batch run in single-image passes gives the same logits.
    515 images run as two concurrent halves (258 + 257) on two streams, eagerly and recorded
    as one graph (fork and join inside the capture), replayed with other work between."""
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
