"""The C-ABI library loads, exports every entry point of include/ifx.h, and its
host-side validation rejects bad arguments before any device work (no GPU)."""
import ctypes
import os
import re

import pytest

import convolution_int8_implicit_amd as ifx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, f)).read(), flags=re.S)
            names |= set(re.findall(r"\b(ifx_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_entry_point():
    L = ifx.lib()
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert ifx.version() == 100
    assert ifx.status_string(0) == "ok" and "workspace" in ifx.status_string(5)
    assert ifx.last_hip_error() == 0


def D(n=1, h=28, w=28, ci=128, co=512, k=1, s=1, p=0, f=ifx.RELU | ifx.RESIDUAL):
    return ifx.conv_desc(n, h, w, ci, co, k, k, s, p, f)


@pytest.mark.parametrize("d,st", [
    (D(), 0),
    (D(k=3, p=1), 0), (D(k=3, s=2, p=1), 0), (D(k=1, s=2), 0),
    (D(n=0), 2), (D(h=-1), 2), (D(ci=0), 2), (D(co=0), 2),
    (D(k=5, p=2), 3), (D(k=3, p=0), 3), (D(k=1, p=1), 3), (D(s=3), 3),
    (D(f=ifx.MAXPOOL), 3), (D(f=ifx.OUT_I32 | ifx.RELU), 3), (D(f=0x40), 3),
    (D(h=224, w=224, ci=3, co=64, k=7, s=2, p=3, f=ifx.RELU | ifx.MAXPOOL), 0),
    (D(h=224, w=224, ci=3, co=64, k=7, s=2, p=3, f=ifx.RELU), 3),
    (D(h=224, w=224, ci=8, co=64, k=7, s=2, p=3, f=ifx.MAXPOOL), 3),
    (D(h=224, w=224, ci=3, co=32, k=7, s=2, p=3, f=ifx.MAXPOOL), 3),
    (D(h=1, w=1, k=3, s=1, p=1), 0), (D(h=2, w=2, ci=3, co=64, k=7, s=2, p=3, f=ifx.MAXPOOL), 0),
    (D(n=1 << 20, h=4096, w=4096), 2), (D(co=42), 3), (D(co=44), 0),
    (D(h=224, w=224, ci=3, co=64, k=7, s=2, p=3, f=ifx.RELU | ifx.MAXPOOL | ifx.INPUT_NHWC), 0),
    (D(f=ifx.RELU | ifx.INPUT_NHWC), 3), (D(k=3, p=1, f=ifx.INPUT_NHWC), 3),
    (D(f=ifx.RELU | ifx.RESIDUAL | ifx.OUT_EVEN), 3),  # a flag of the chained call only
    # phase-split layouts: the general kernel only, even sizes, never with int32 output
    (D(ci=512, co=256, f=ifx.RELU | ifx.OUT_PHASE), 0), (D(ci=128, f=ifx.RELU | ifx.OUT_PHASE), 3),
    (D(ci=512, h=27, w=28, f=ifx.OUT_PHASE), 3), (D(ci=512, f=ifx.OUT_I32 | ifx.OUT_PHASE), 3),
    (D(ci=256, co=256, k=3, s=2, p=1, f=ifx.IN_PHASE), 0), (D(ci=256, k=3, s=1, p=1, f=ifx.IN_PHASE), 3),
    (D(ci=256, h=27, k=3, s=2, p=1, f=ifx.IN_PHASE), 3), (D(ci=256, k=1, s=2, f=ifx.IN_PHASE), 3),
    (D(ci=64, co=64, h=56, w=56, k=3, s=1, p=1, f=ifx.OUT_PHASE), 3),  # the haloed 3x3
])
def test_descriptor_validation(d, st):
    assert ifx.conv_validate(d) == st


def test_out_dims_and_sizes(orc):
    for (h, k, s, p) in [(28, 1, 1, 0), (56, 1, 2, 0), (56, 3, 2, 1), (7, 3, 1, 1), (9, 3, 2, 1)]:
        ho, wo = ifx.conv_out_dims(D(h=h, w=h + 1, k=k, s=s, p=p))
        assert (ho, wo) == (orc.out_dim(h, k, s, p), orc.out_dim(h + 1, k, s, p))
    ho, wo = ifx.conv_out_dims(D(h=224, w=224, ci=3, co=64, k=7, s=2, p=3, f=ifx.MAXPOOL))
    assert (ho, wo) == (56, 56)
    assert ifx.act_bytes(2, 5, 6, 33) == 2 * 2 * 5 * 6 * 32
    assert ifx.act_bytes(0, 5, 6, 33) == 0
    for co, k, ci in [(512, 1, 128), (64, 3, 64), (1000, 1, 2048), (96, 3, 40)]:
        o2 = orc.wgroup(co)
        assert ifx.wpack_bytes(D(ci=ci, co=co, k=k, p=k // 2)) == (co + o2 - 1) // o2 * o2 * k * k * ((ci + 31) // 32) * 32
    assert ifx.wpack_bytes(D(h=224, w=224, ci=3, co=64, k=7, s=2, p=3, f=ifx.MAXPOOL)) == 64 * 256
    assert ifx.wpack_bytes(D(k=5, p=2)) == 0


def test_errors_return_before_any_launch():
    L = ifx.lib()
    d = D()
    fake = ctypes.c_void_p(0x100000)          # aligned, never dereferenced
    odd = ctypes.c_void_p(0x100001)           # misaligned
    args = [fake] * 7
    # null input
    assert L.ifx_conv_fused(ctypes.byref(d), None, *args[:5], fake, None) == 1
    # residual required
    assert L.ifx_conv_fused(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, None) == 1
    # mult/shift required unless OUT_I32
    assert L.ifx_conv_fused(ctypes.byref(d), fake, fake, fake, None, fake, fake, fake, None) == 1
    # misaligned output
    assert L.ifx_conv_fused(ctypes.byref(d), fake, fake, fake, fake, fake, fake, odd, None) == 4
    # unsupported descriptor reported before pointer checks
    bad = D(k=5, p=2)
    assert L.ifx_conv_fused(ctypes.byref(bad), None, None, None, None, None, None, None, None) == 3
    assert L.ifx_pack_act(None, fake, 1, 2, 2, 3, None) == 1
    assert L.ifx_pack_act(fake, odd, 1, 2, 2, 3, None) == 4
    assert L.ifx_pack_act(fake, fake, 0, 2, 2, 3, None) == 2
    assert L.ifx_unpack_act(fake, fake, 1, 2, -2, 3, None) == 2
    assert L.ifx_pack_weights(ctypes.byref(bad), fake, fake, None) == 3
    assert L.ifx_conv_out_dims(ctypes.byref(d), None, None) == 1
    assert L.ifx_conv_validate(None) == 1


def test_conv_proj_fused_validation():
    """conv3 + projection in one launch: descriptors, pairing and pointers are checked on the
    host and nothing is launched on an error."""
    L = ifx.lib()
    fake = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100001)
    d3 = D(n=2, h=14, w=14, ci=64, co=256)
    dp = D(n=2, h=28, w=28, ci=128, co=256, s=2, f=0)
    four = [fake] * 4  # weights, bias, mult, shift

    def call(a3, ap, t=fake, y=fake):
        return L.ifx_conv_proj_fused(ctypes.byref(a3), t, *four, ctypes.byref(ap), fake, *four, y, None)

    assert L.ifx_conv_proj_fused(None, fake, *four, ctypes.byref(dp), fake, *four, fake, None) == 1
    assert call(d3, dp, t=None) == 1
    assert call(d3, dp, y=odd) == 4
    assert call(D(n=2, h=14, w=14, ci=64, co=256, k=3, p=1), dp) == 3           # conv3 must be 1x1
    assert call(d3, D(n=2, h=28, w=28, ci=128, co=256, s=2, f=ifx.RELU)) == 3    # projection without ReLU
    assert call(D(n=2, h=14, w=14, ci=64, co=256, f=ifx.RELU), dp) == 3         # conv3 adds the shortcut
    assert call(d3, D(n=2, h=28, w=28, ci=128, co=128, s=2, f=0)) == 2          # channel counts differ
    assert call(d3, D(n=2, h=28, w=28, ci=128, co=256, s=1, f=0)) == 2          # output sizes differ
    assert call(d3, D(n=3, h=28, w=28, ci=128, co=256, s=2, f=0)) == 2          # batches differ
    assert call(D(k=5, p=2), dp) == 3


def test_conv_fused_even_validation():
    """The even-pixel copy: pointers, alignment and the kernel's support are checked on the host,
    and nothing is launched on an error."""
    L = ifx.lib()
    fake = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100001)
    R = ifx.RESIDUAL | ifx.RELU
    d = D(n=2, h=28, w=28, ci=128, co=512, f=R)  # a res3 conv3 (ring kernel)

    def call(dd, ye=fake, y=fake, res=fake):
        return L.ifx_conv_fused_even(ctypes.byref(dd), fake, fake, fake, fake, fake, res, y, ye, None)

    assert L.ifx_conv_even_supported(ctypes.byref(d)) == 1
    assert L.ifx_conv_even_supported(ctypes.byref(D(n=2, h=14, w=14, ci=256, co=1024, f=R))) == 1  # general kernel
    assert L.ifx_conv_even_supported(ctypes.byref(D(n=2, h=6, w=6, ci=64, co=128, f=ifx.RELU))) == 0  # small-K 1x1
    assert L.ifx_conv_even_supported(ctypes.byref(D(n=2, h=6, w=6, ci=256, co=128, f=ifx.OUT_I32))) == 0
    assert L.ifx_conv_even_supported(ctypes.byref(D(k=5, p=2))) == 0  # invalid descriptor
    assert L.ifx_conv_even_supported(None) == 0
    assert call(d, ye=None) == 1
    assert call(d, res=None) == 1
    assert call(d, ye=odd) == 4
    assert call(D(n=2, h=6, w=6, ci=64, co=128, f=ifx.RELU)) == 3
    assert call(D(k=5, p=2)) == 3


def _block(n=2, proj=True, c3_flags=ifx.RESIDUAL | ifx.RELU, c2_cin=64):
    p = ifx.BlockParams()
    p.d[0] = D(n=n, h=8, w=8, ci=256, co=64, f=ifx.RELU)
    p.d[1] = D(n=n, h=8, w=8, ci=c2_cin, co=64, k=3, s=2, p=1, f=ifx.RELU)
    p.d[2] = D(n=n, h=4, w=4, ci=64, co=256, f=c3_flags)
    p.d[3] = D(n=n, h=8, w=8, ci=256, co=256, s=2, f=0)
    p.has_proj = 1 if proj else 0
    for i in range(4):
        p.w_blk[i] = p.bias[i] = p.mult[i] = p.shift[i] = 0x100000
    return p


def _split_bytes(n, ho, wo, ci, co, k, stride, pad=0, out_i32=False):
    """Partial-sum bytes of a split-K launch: a launch of fewer than 64 output tiles and at least
    16 K-steps (two 32-channel blocks each) is split into at most 16 parts of an even number of
    blocks, at least two steps each, aiming at 256 workgroups, while the int32 partials fit in
    8 MB (and Oc is a multiple of 4)."""
    i1, oc1 = -(-ci // 32), -(-co // 32)
    if (k == 1 and pad == 0 and not out_i32 and i1 <= 4) or co % 4:
        return 0                                     # the small-K 1x1 kernel: one pass, no split
    m, nkb = n * ho * wo, k * k * i1
    wide = oc1 * 32 > 64
    bm, bn = (128, 128) if wide else (256, 64)
    if k == 1 and wide:
        bm, bn = 256, 128
    elif k == 3 and stride == 2 and oc1 * 32 >= 256:
        bm, bn = 128, 256
    tiles = -(-m // bm) * -(-(oc1 * 32) // bn)
    steps = (nkb + 1) // 2
    if tiles >= 64 or steps < 16:
        return 0
    parts = min(-(-256 // tiles), steps // 2, 16)
    if parts < 2:
        return 0
    per = 2 * -(-steps // parts)
    nparts = -(-nkb // per)
    if nparts < 2 or nparts * m * co * 4 > 8 << 20:
        return 0
    return -(-(nparts * m * co * 4) // 256) * 256


def test_split_rule_examples():
    # 3x3/s2 of 64 channels on 8x8: 18 blocks are too short a reduction to split
    assert _split_bytes(2, 4, 4, 64, 64, 3, 2, 1) == 0
    # 28x28x256 3x3 at batch 8: 72 blocks, 25 tiles -> 9 parts would need 14.5 MB -> no split
    assert _split_bytes(8, 28, 28, 256, 64, 3, 1, 1) == 0
    # the classifier at batch 1: 2048 -> 1000, 8 tiles, 64 blocks -> 16 parts of 4 blocks
    assert _split_bytes(1, 1, 1, 2048, 1000, 1, 1, out_i32=True) == 16 * 1000 * 4
    # 7x7x512 3x3 at batch 1: 4 tiles, 144 blocks -> 15 parts of 10 blocks (the last 4)
    assert _split_bytes(1, 7, 7, 512, 512, 3, 1, 1) == 15 * 49 * 512 * 4
    # Oc not a multiple of 4: never split
    assert _split_bytes(1, 7, 7, 512, 510, 3, 1, 1) == 0


def test_block_validation_and_workspace():
    L = ifx.lib()
    p = _block()
    ws = ifx.block_workspace_bytes(p)
    exp = 2 * 2 * 8 * 8 * 32 + 2 * 2 * 4 * 4 * 32 + 2 * 8 * 4 * 4 * 32
    exp += _split_bytes(2, 4, 4, 64, 64, 3, 2, 1)    # 0: every K is short; c3 runs fused
    assert ws == exp
    fake = ctypes.c_void_p(0x200000)
    assert L.ifx_block_forward(ctypes.byref(p), fake, fake, fake, ws - 1, None) == 5
    assert L.ifx_block_forward(ctypes.byref(p), None, fake, fake, ws, None) == 1
    assert ifx.block_workspace_bytes(_block(proj=False)) == 0          # identity shortcut needs c3 out == input
    assert ifx.block_workspace_bytes(_block(c3_flags=ifx.RELU)) == 0   # c3 must add the shortcut
    assert ifx.block_workspace_bytes(_block(c2_cin=32)) == 0           # channel chain broken
    q = _block()
    q.w_blk[3] = None
    assert L.ifx_block_forward(ctypes.byref(q), fake, fake, fake, ws, None) == 1


def test_net_validation_and_workspace():
    L = ifx.lib()
    blk = _block(n=1)
    blk.d[0] = D(n=1, h=56, w=56, ci=64, co=64, f=ifx.RELU)
    blk.d[1] = D(n=1, h=56, w=56, ci=64, co=64, k=3, s=1, p=1, f=ifx.RELU)
    blk.d[2] = D(n=1, h=56, w=56, ci=64, co=256, f=ifx.RESIDUAL | ifx.RELU)
    blk.d[3] = D(n=1, h=56, w=56, ci=64, co=256, s=1, f=0)
    arr = (ifx.BlockParams * 1)(blk)
    p = ifx.NetParams()
    p.stem = D(n=1, h=224, w=224, ci=3, co=64, k=7, s=2, p=3, f=ifx.RELU | ifx.MAXPOOL)
    p.stem_w = p.stem_bias = p.stem_mult = p.stem_shift = 0x100000
    p.n_blocks = 1
    p.blocks = ctypes.cast(arr, ctypes.POINTER(ifx.BlockParams))
    p.fc_w_blk = p.fc_bias = 0x100000
    p.fc_in, p.fc_out = 256, 1000
    ws = ifx.net_workspace_bytes(p, 4)
    act = 4 * 8 * 56 * 56 * 32
    t = 4 * 2 * 56 * 56 * 32
    assert ws == 2 * act + 2 * t + act + 4 * 8 * 32
    p.sub_batch = 2
    assert ifx.net_workspace_bytes(p, 4) == ws // 2 + _split_bytes(2, 56, 56, 64, 64, 3, 1, 1)
    fake = ctypes.c_void_p(0x200000)
    assert L.ifx_net_forward(ctypes.byref(p), fake, fake, 4, fake, ws // 2 - 1, None) == 5
    # a whole batch of >= 192 images runs as two concurrent halves, each with its own workspace
    p.sub_batch = 256
    half = ifx.net_workspace_bytes(p, 256)                  # one pass of 256 images
    assert ifx.net_workspace_bytes(p, 512) == half          # consecutive passes share one workspace
    p.sub_batch = 0
    assert ifx.net_workspace_bytes(p, 512) == 2 * half
    p.sub_batch = 96
    lane96 = ifx.net_workspace_bytes(p, 96)
    p.sub_batch = 0
    assert ifx.net_workspace_bytes(p, 192) == 2 * lane96
    p.sub_batch = 191
    one = ifx.net_workspace_bytes(p, 191)
    p.sub_batch = 0
    assert ifx.net_workspace_bytes(p, 191) == one           # below 192: one pass
    p.fc_in = 255
    assert ifx.net_workspace_bytes(p, 4) == 0


def test_fold_bn_validation_before_any_launch():
    L = ifx.lib()
    fake = 0x100000                      # aligned, never dereferenced
    good = dict(c_out=8, x_scale=0.1, y_scale=0.2, eps=1e-5, w_per_channel=1, w_scale=fake, conv_bias=None,
                gamma=fake, beta=fake, mean=fake, var=fake)
    outs = [ctypes.c_void_p(fake)] * 4
    assert L.ifx_fold_bn(None, *outs, None) == 1
    f = ifx.BnFold(**{**good, "c_out": 0})
    assert L.ifx_fold_bn(ctypes.byref(f), *outs, None) == 2
    f = ifx.BnFold(**{**good, "gamma": None})
    assert L.ifx_fold_bn(ctypes.byref(f), *outs, None) == 1
    f = ifx.BnFold(**good)
    assert L.ifx_fold_bn(ctypes.byref(f), None, *outs[1:], None) == 1
    f = ifx.BnFold(**{**good, "var": fake + 2})
    assert L.ifx_fold_bn(ctypes.byref(f), *outs, None) == 4
    f = ifx.BnFold(**good)
    assert L.ifx_fold_bn(ctypes.byref(f), ctypes.c_void_p(fake + 4), *outs[1:], None) == 4


def test_graph_entry_points_validate_before_recording():
    L = ifx.lib()
    h = ctypes.c_void_p(123)
    assert L.ifx_net_graph_create(None, None, None, 1, None, 0, None) == 1       # no handle pointer
    assert L.ifx_net_graph_create(None, None, None, 1, None, 0, ctypes.byref(h)) == 1
    assert h.value is None                                                        # cleared on error
    assert L.ifx_graph_launch(None, None) == 1
    assert L.ifx_graph_destroy(None) == 0


def test_dispatch_of_the_network_shapes():
    """The kernel instance each ResNet-50 layer shape launches at 1024 images (one pass of a batch
    of 2048), as the host-only name query reports it without a GPU, and the boundaries of the
    haloed-window 3x3 and of the wide-tile fused projection."""
    R, RR = ifx.RELU, ifx.RESIDUAL | ifx.RELU

    def name(n, h, w, c, oc, k, s, p, flags):
        return ifx.conv_kernel_name(ifx.conv_desc(n, h, w, c, oc, k, k, s, p, flags))

    win = "conv3x3_win_kernel<"
    # unit-stride 3x3 over a multiple of 128 channels on 28- and 14-wide images, enough tiles
    assert name(1024, 28, 28, 128, 128, 3, 1, 1, R) == win + "32, true>"
    assert name(1024, 14, 14, 256, 256, 3, 1, 1, R) == win + "16, true>"
    assert name(1024, 14, 14, 256, 256, 3, 1, 1, 0) == win + "16, false>"
    # not on 7-wide images (the window would exceed 384 pixels), not below one tile per CU, not
    # with 64 channels (the res2 kernel), a shortcut, stride 2 or 96 channels
    assert not name(1024, 7, 7, 512, 512, 3, 1, 1, R).startswith(win)
    assert not name(64, 28, 28, 128, 128, 3, 1, 1, R).startswith(win)
    assert name(1024, 56, 56, 64, 64, 3, 1, 1, R) == "conv3x3_halo_kernel<true>"
    assert not name(1024, 28, 28, 128, 128, 3, 1, 1, RR).startswith(win)
    assert not name(1024, 28, 28, 128, 128, 3, 2, 1, R).startswith(win)
    assert not name(1024, 28, 28, 96, 128, 3, 1, 1, R).startswith(win)

    def proj_name(n, ho, cmid, cin, cout, s):
        d3 = ifx.conv_desc(n, ho, ho, cmid, cout, 1, 1, 1, 0, RR)
        dp = ifx.conv_desc(n, ho * s, ho * s, cin, cout, 1, 1, s, 0, 0)
        return ifx.conv_kernel_name(d3, dp)

    wide = "igemm_kernel<1, 1, 128, 256, 2, 128, true, true, true>"
    assert proj_name(1024, 14, 256, 512, 1024, 1) == wide  # res4.1 on the even-pixel copy
    assert proj_name(1024, 7, 512, 1024, 2048, 1) == wide  # res5.1
    assert proj_name(97, 14, 256, 512, 1024, 1) == "igemm_kernel<1, 1, 128, 128, 2, 64, true, true, true>"


def test_quantisation_validation():
    """ifx_quantize_f32 / ifx_quantize_u8 / ifx_dequantize_i32 reject null, shape and alignment
    errors before any launch (an empty tensor is a no-op)."""
    import convolution_int8_implicit_amd as ifx
    L = ifx.lib()
    fake = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100001)
    word = ctypes.c_void_p(0x100004)      # 4-byte aligned: fine for mean/mult, not for x, q or y
    assert L.ifx_quantize_f32(None, fake, 12, 3, fake, None) == 1
    assert L.ifx_quantize_f32(fake, fake, 12, 3, None, None) == 1
    assert L.ifx_quantize_f32(fake, fake, 13, 3, fake, None) == 2      # not a multiple of c
    assert L.ifx_quantize_f32(fake, fake, 12, 0, fake, None) == 2
    assert L.ifx_quantize_f32(fake, fake, -3, 3, fake, None) == 2
    assert L.ifx_quantize_f32(fake, fake, 1 << 31, 1, fake, None) == 2
    assert L.ifx_quantize_f32(word, fake, 12, 3, fake, None) == 4
    assert L.ifx_quantize_f32(fake, odd, 12, 3, fake, None) == 4
    assert L.ifx_quantize_f32(fake, fake, 12, 3, odd, None) == 4
    assert L.ifx_quantize_f32(fake, fake, 0, 3, word, None) == 0
    assert L.ifx_quantize_u8(fake, fake, 12, 3, None, fake, None) == 1
    assert L.ifx_quantize_u8(fake, fake, 12, 5, fake, fake, None) == 2
    assert L.ifx_quantize_u8(fake, fake, 12, 3, odd, fake, None) == 4
    assert L.ifx_quantize_u8(odd, fake, 12, 3, fake, fake, None) == 4
    assert L.ifx_dequantize_i32(None, fake, 4, 1.0, None) == 1
    assert L.ifx_dequantize_i32(fake, fake, -1, 1.0, None) == 2
    assert L.ifx_dequantize_i32(fake, word, 4, 1.0, None) == 4
    assert L.ifx_dequantize_i32(fake, fake, 0, 1.0, None) == 0
