"""MI355X-native fused int8 ResNet convolution: Python binding of libifx.so.

The compute path is the C-ABI library built from csrc/ (hand-written gfx950
HIP kernels); this module only marshals arguments.  Tensors are torch device
tensors (torch supplies memory and streams); every step of the path runs in
the library's kernels.  There is no fallback: if the library is not built the
first call raises.

Entry points mirror include/ifx.h:
    conv_validate, conv_out_dims, act_bytes, wpack_bytes,
    pack_act, unpack_act, pack_weights, conv_fused,
    block_workspace_bytes, block_forward, net_workspace_bytes, net_forward,
    fold_bn, status_string, last_hip_error, version
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "RELU", "RESIDUAL", "MAXPOOL", "OUT_I32", "INPUT_NHWC", "OUT_EVEN", "OUT_PHASE", "IN_PHASE", "IfxError", "ConvDesc", "BlockParams", "NetParams", "lib",
    "conv_desc", "conv_validate", "conv_out_dims", "act_bytes", "wpack_bytes", "pack_act", "unpack_act",
    "pack_weights", "conv_fused", "conv_fused_even", "conv_even_supported", "conv_chain_fused", "conv_chain_kernel_name", "conv_proj_chain_fused",
    "conv_proj_chain_kernel_name", "conv_kernel_name",
    "block_workspace_bytes", "block_forward", "block_forward_noalloc",
    "BLOCK_SCRATCH_BYTES", "net_workspace_bytes",
    "net_forward", "NetGraph", "fold_bn", "BnFold", "status_string", "last_hip_error", "version", "LIB_PATH",
]

RELU, RESIDUAL, MAXPOOL, OUT_I32, INPUT_NHWC, OUT_EVEN, OUT_PHASE, IN_PHASE = 1, 2, 4, 8, 16, 32, 64, 128
STATUS = {0: "IFX_OK", 1: "IFX_E_NULL", 2: "IFX_E_SHAPE", 3: "IFX_E_UNSUPPORTED", 4: "IFX_E_ALIGN",
          5: "IFX_E_WORKSPACE", 6: "IFX_E_HIP"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libifx.so")


class IfxError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = STATUS.get(status, str(status))
        extra = ""
        if status == 6:
            extra = f" (hipError {last_hip_error()})"
        super().__init__(f"{what}: {name}{extra}")


class ConvDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32), ("c_in", ctypes.c_int32),
                ("c_out", ctypes.c_int32), ("kh", ctypes.c_int32), ("kw", ctypes.c_int32),
                ("stride", ctypes.c_int32), ("pad", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class BlockParams(ctypes.Structure):
    _fields_ = [("d", ConvDesc * 4), ("has_proj", ctypes.c_int32), ("w_blk", ctypes.c_void_p * 4),
                ("bias", ctypes.c_void_p * 4), ("mult", ctypes.c_void_p * 4), ("shift", ctypes.c_void_p * 4)]


class NetParams(ctypes.Structure):
    _fields_ = [("stem", ConvDesc), ("stem_w", ctypes.c_void_p), ("stem_bias", ctypes.c_void_p),
                ("stem_mult", ctypes.c_void_p), ("stem_shift", ctypes.c_void_p), ("n_blocks", ctypes.c_int32),
                ("blocks", ctypes.POINTER(BlockParams)), ("fc_w_blk", ctypes.c_void_p),
                ("fc_bias", ctypes.c_void_p), ("fc_in", ctypes.c_int32), ("fc_out", ctypes.c_int32),
                ("sub_batch", ctypes.c_int32)]


class BnFold(ctypes.Structure):
    _fields_ = [("c_out", ctypes.c_int32), ("x_scale", ctypes.c_float), ("y_scale", ctypes.c_float),
                ("eps", ctypes.c_float), ("w_per_channel", ctypes.c_int32), ("w_scale", ctypes.c_void_p),
                ("conv_bias", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("mean", ctypes.c_void_p), ("var", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libifx.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libifx.so not built ({LIB_PATH}); run python -m convolution_int8_implicit_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    i64 = ctypes.c_int64
    D = ctypes.POINTER(ConvDesc)
    sigs = {
        "ifx_conv_validate": ([D], i32),
        "ifx_conv_out_dims": ([D, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "ifx_act_bytes": ([i32, i32, i32, i32], sz),
        "ifx_wpack_bytes": ([D], sz),
        "ifx_pack_act": ([vp, vp, i32, i32, i32, i32, vp], i32),
        "ifx_quantize_f32": ([vp, vp, i64, i32, vp, vp], i32),
        "ifx_quantize_u8": ([vp, vp, i64, i32, vp, vp, vp], i32),
        "ifx_dequantize_i32": ([vp, vp, i64, ctypes.c_float, vp], i32),
        "ifx_unpack_act": ([vp, vp, i32, i32, i32, i32, vp], i32),
        "ifx_pack_weights": ([D, vp, vp, vp], i32),
        "ifx_conv_fused": ([D, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "ifx_conv_fused_even": ([D, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "ifx_conv_even_supported": ([D], i32),
        "ifx_conv_proj_fused": ([D, vp, vp, vp, vp, vp, D, vp, vp, vp, vp, vp, vp, vp], i32),
        "ifx_block_workspace_bytes": ([ctypes.POINTER(BlockParams)], sz),
        "ifx_block_forward": ([ctypes.POINTER(BlockParams), vp, vp, vp, sz, vp], i32),
        "ifx_block_forward_noalloc": ([ctypes.POINTER(BlockParams), vp, vp, vp], i32),
        "ifx_net_workspace_bytes": ([ctypes.POINTER(NetParams), i32], sz),
        "ifx_net_forward": ([ctypes.POINTER(NetParams), vp, vp, i32, vp, sz, vp], i32),
        "ifx_fold_bn": ([ctypes.POINTER(BnFold), vp, vp, vp, vp, vp], i32),
        "ifx_net_graph_create": ([ctypes.POINTER(NetParams), vp, vp, i32, vp, sz, ctypes.POINTER(vp)], i32),
        "ifx_graph_launch": ([vp, vp], i32),
        "ifx_graph_destroy": ([vp], i32),
        "ifx_conv_kernel_name": ([D, ctypes.c_char_p, sz], i32),
        "ifx_conv_proj_kernel_name": ([D, D, ctypes.c_char_p, sz], i32),
        "ifx_conv_chain_kernel_name": ([D, D, ctypes.c_char_p, sz], i32),
        "ifx_conv_chain_fused": ([D, vp, vp, vp, vp, vp, vp, vp, D, vp, vp, vp, vp, vp, vp], i32),
        "ifx_conv_proj_chain_kernel_name": ([D, D, D, ctypes.c_char_p, sz], i32),
        "ifx_conv_proj_chain_fused": ([D, vp, vp, vp, vp, vp, D, vp, vp, vp, vp, vp, vp, D, vp, vp, vp, vp, vp,
                                       vp], i32),
        "ifx_status_string": ([i32], ctypes.c_char_p),
        "ifx_probe_copy": ([vp, vp, sz, vp], i32),
        "ifx_probe_mfma_i8": ([vp, i32, i32, vp], i32),
        "ifx_probe_mfma_i8_data": ([vp, i32, i32, vp], i32),
        "ifx_probe_dma_lds": ([vp, sz, i32, i32, vp, vp], i32),
        "ifx_probe_lds_read": ([vp, i32, i32, vp, vp], i32),
        "ifx_probe_valu": ([i32, vp, i32, i32, vp], i32),
        "ifx_last_hip_error": ([], i32),
        "ifx_version": ([], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = L
    return L


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc: int, what: str):
    if rc != 0:
        raise IfxError(rc, what)


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libifx takes contiguous device tensors")


def conv_desc(n, h, w, c_in, c_out, kh, kw, stride, pad, flags) -> ConvDesc:
    return ConvDesc(n, h, w, c_in, c_out, kh, kw, stride, pad, flags)


def conv_validate(d: ConvDesc) -> int:
    return lib().ifx_conv_validate(ctypes.byref(d))


def conv_out_dims(d: ConvDesc):
    ho, wo = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ifx_conv_out_dims(ctypes.byref(d), ctypes.byref(ho), ctypes.byref(wo)), "ifx_conv_out_dims")
    return ho.value, wo.value


def act_bytes(n, h, w, c) -> int:
    return lib().ifx_act_bytes(n, h, w, c)


def wpack_bytes(d: ConvDesc) -> int:
    return lib().ifx_wpack_bytes(ctypes.byref(d))


def pack_act(x_nhwc: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """NHWC int8 -> packed NC/32HW32 [n, ceil(c/32), h, w, 32]."""
    _dev(x_nhwc, out)
    n, h, w, c = x_nhwc.shape
    if out is None:
        out = torch.empty((n, (c + 31) // 32, h, w, 32), dtype=torch.int8, device=x_nhwc.device)
    _check(lib().ifx_pack_act(_ptr(x_nhwc), _ptr(out), n, h, w, c, _stream(stream)), "ifx_pack_act")
    return out


def quantize_f32(x: torch.Tensor, mult: torch.Tensor, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """float32 NHWC image -> int8 codes (ifx_quantize_f32); mult: float32 [c], c the last axis."""
    _dev(x, mult, out)
    assert x.dtype == torch.float32 and mult.dtype == torch.float32
    if out is None:
        out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    _check(lib().ifx_quantize_f32(_ptr(x), _ptr(out), x.numel(), mult.numel(), _ptr(mult), _stream(stream)),
           "ifx_quantize_f32")
    return out


def quantize_u8(x: torch.Tensor, mean: torch.Tensor, mult: torch.Tensor, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """uint8 NHWC image -> int8 codes (ifx_quantize_u8); mean, mult: float32 [c], c the last axis."""
    _dev(x, mean, mult, out)
    assert x.dtype == torch.uint8 and mean.dtype == torch.float32 and mult.dtype == torch.float32
    assert mean.numel() == mult.numel()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    _check(lib().ifx_quantize_u8(_ptr(x), _ptr(out), x.numel(), mult.numel(), _ptr(mean), _ptr(mult),
                                 _stream(stream)), "ifx_quantize_u8")
    return out


def dequantize_i32(q: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int32 results (the logits) -> float32 (ifx_dequantize_i32): (float)q * scale."""
    _dev(q, out)
    assert q.dtype == torch.int32
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib().ifx_dequantize_i32(_ptr(q), _ptr(out), q.numel(), float(scale), _stream(stream)),
           "ifx_dequantize_i32")
    return out


def unpack_act(x_blk: torch.Tensor, c: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Packed [n, c1, h, w, 32] -> NHWC [n, h, w, c]."""
    _dev(x_blk, out)
    n, _, h, w, _ = x_blk.shape
    if out is None:
        out = torch.empty((n, h, w, c), dtype=torch.int8, device=x_blk.device)
    _check(lib().ifx_unpack_act(_ptr(x_blk), _ptr(out), n, h, w, c, _stream(stream)), "ifx_unpack_act")
    return out


def pack_weights(d: ConvDesc, w_ohwi: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """OHWI int8 -> the packed weight layout of d (flat int8 tensor)."""
    _dev(w_ohwi, out)
    nbytes = wpack_bytes(d)
    if nbytes == 0:
        raise IfxError(conv_validate(d) or 2, "ifx_wpack_bytes")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.int8, device=w_ohwi.device)
    _check(lib().ifx_pack_weights(ctypes.byref(d), _ptr(w_ohwi), _ptr(out), _stream(stream)), "ifx_pack_weights")
    return out


def conv_fused(d: ConvDesc, x_blk, w_blk, bias, mult, shift, residual, y, stream=None) -> None:
    _dev(x_blk, w_blk, bias, mult, shift, residual, y)
    _check(lib().ifx_conv_fused(ctypes.byref(d), _ptr(x_blk), _ptr(w_blk), _ptr(bias), _ptr(mult), _ptr(shift),
                                _ptr(residual), _ptr(y), _stream(stream)), "ifx_conv_fused")


def conv_fused_even(d: ConvDesc, x_blk, w_blk, bias, mult, shift, residual, y, y_even, stream=None) -> None:
    """ifx_conv_fused that also writes the output's even pixels densely to y_even (ifx_conv_fused_even)."""
    _dev(x_blk, w_blk, bias, mult, shift, residual, y, y_even)
    _check(lib().ifx_conv_fused_even(ctypes.byref(d), _ptr(x_blk), _ptr(w_blk), _ptr(bias), _ptr(mult), _ptr(shift),
                                     _ptr(residual), _ptr(y), _ptr(y_even), _stream(stream)), "ifx_conv_fused_even")


def conv_even_supported(d: ConvDesc) -> bool:
    """Whether ifx_conv_fused_even(d, ...) runs (host-only query)."""
    return bool(lib().ifx_conv_even_supported(ctypes.byref(d)))


def conv_proj_fused(d3: ConvDesc, t_blk, w3_blk, bias3, mult3, shift3, dp: ConvDesc, x_blk, wp_blk, biasp, multp,
                    shiftp, y, stream=None) -> None:
    """conv3 of a bottleneck with its 1x1 projection shortcut in one launch (ifx_conv_proj_fused)."""
    _dev(t_blk, w3_blk, bias3, mult3, shift3, x_blk, wp_blk, biasp, multp, shiftp, y)
    _check(lib().ifx_conv_proj_fused(ctypes.byref(d3), _ptr(t_blk), _ptr(w3_blk), _ptr(bias3), _ptr(mult3),
                                     _ptr(shift3), ctypes.byref(dp), _ptr(x_blk), _ptr(wp_blk), _ptr(biasp),
                                     _ptr(multp), _ptr(shiftp), _ptr(y), _stream(stream)), "ifx_conv_proj_fused")


def block_workspace_bytes(p: BlockParams) -> int:
    return lib().ifx_block_workspace_bytes(ctypes.byref(p))


def block_forward(p: BlockParams, x_blk, y_blk, ws: torch.Tensor, stream=None) -> None:
    _dev(x_blk, y_blk, ws)
    _check(lib().ifx_block_forward(ctypes.byref(p), _ptr(x_blk), _ptr(y_blk), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "ifx_block_forward")


def conv_chain_fused(d3: ConvDesc, t_blk, w3_blk, bias3, mult3, shift3, residual, y, d1: ConvDesc, w1_blk, bias1,
                     mult1, shift1, t1, stream=None) -> None:
    """conv3 (with its shortcut) and the next block's conv1 as one launch (ifx_conv_chain_fused)."""
    ts = (t_blk, w3_blk, bias3, mult3, shift3, residual, y, w1_blk, bias1, mult1, shift1, t1)
    _dev(*ts)
    _check(lib().ifx_conv_chain_fused(ctypes.byref(d3), *[_ptr(t) for t in ts[:7]], ctypes.byref(d1),
                                      *[_ptr(t) for t in ts[7:]], _stream(stream)), "ifx_conv_chain_fused")


def conv_chain_kernel_name(d3: ConvDesc, d1: ConvDesc):
    """The kernel ifx_conv_chain_fused(d3, d1) launches, or None when the pair does not chain."""
    buf = ctypes.create_string_buffer(256)
    rc = lib().ifx_conv_chain_kernel_name(ctypes.byref(d3), ctypes.byref(d1), buf, len(buf))
    if rc == 3:
        return None
    _check(rc, "ifx_conv_chain_kernel_name")
    return buf.value.decode()


def conv_proj_chain_fused(d3: ConvDesc, t_blk, w3_blk, bias3, mult3, shift3, dp: ConvDesc, x_blk, wp_blk, biasp,
                          multp, shiftp, y, d1: ConvDesc, w1_blk, bias1, mult1, shift1, t1, stream=None) -> None:
    """conv3 with its projection shortcut and the next block's conv1 as one launch
    (ifx_conv_proj_chain_fused)."""
    a = (t_blk, w3_blk, bias3, mult3, shift3)
    b = (x_blk, wp_blk, biasp, multp, shiftp, y)
    c = (w1_blk, bias1, mult1, shift1, t1)
    _dev(*a, *b, *c)
    _check(lib().ifx_conv_proj_chain_fused(ctypes.byref(d3), *[_ptr(t) for t in a], ctypes.byref(dp),
                                           *[_ptr(t) for t in b], ctypes.byref(d1), *[_ptr(t) for t in c],
                                           _stream(stream)), "ifx_conv_proj_chain_fused")


def conv_proj_chain_kernel_name(d3: ConvDesc, dp: ConvDesc, d1: ConvDesc):
    """The kernel ifx_conv_proj_chain_fused(d3, dp, d1) launches, or None when they do not chain."""
    buf = ctypes.create_string_buffer(256)
    rc = lib().ifx_conv_proj_chain_kernel_name(ctypes.byref(d3), ctypes.byref(dp), ctypes.byref(d1), buf, len(buf))
    if rc == 3:
        return None
    _check(rc, "ifx_conv_proj_chain_kernel_name")
    return buf.value.decode()


def conv_kernel_name(d: ConvDesc, proj: Optional[ConvDesc] = None) -> str:
    """The kernel instance ifx_conv_fused(d) (or ifx_conv_proj_fused(d, proj)) launches, as
    profilers print it (host-only query)."""
    buf = ctypes.create_string_buffer(256)
    if proj is None:
        _check(lib().ifx_conv_kernel_name(ctypes.byref(d), buf, len(buf)), "ifx_conv_kernel_name")
    else:
        _check(lib().ifx_conv_proj_kernel_name(ctypes.byref(d), ctypes.byref(proj), buf, len(buf)),
               "ifx_conv_proj_kernel_name")
    return buf.value.decode()


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Streaming-copy ceiling probe (ifx_probe.h): dst = src, 16-byte non-temporal chunks."""
    _dev(src, dst)
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    _check(lib().ifx_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "ifx_probe_copy")


def probe_mfma_i8(out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """int8 MFMA ceiling probe (ifx_probe.h); returns the ops it performs."""
    _dev(out)
    assert out.dtype == torch.int32 and out.numel() >= 4 * blocks
    _check(lib().ifx_probe_mfma_i8(_ptr(out), blocks, iters, _stream(stream)), "ifx_probe_mfma_i8")
    return blocks * 4 * iters * 16 * 32768


def probe_mfma_i8_data(out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """int8 MFMA rate probe with operands that change every instruction (ifx_probe.h); returns its ops."""
    _dev(out)
    assert out.dtype == torch.int32 and out.numel() >= 4 * blocks
    _check(lib().ifx_probe_mfma_i8_data(_ptr(out), blocks, iters, _stream(stream)), "ifx_probe_mfma_i8_data")
    return blocks * 4 * iters * 4 * 16 * 32768


def probe_dma_lds(src: torch.Tensor, out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """Buffer->LDS DMA rate probe (ifx_probe.h) over the bytes of src; returns the bytes it moves."""
    _dev(src, out)
    nbytes = src.numel() * src.element_size()
    assert out.dtype == torch.int32 and out.numel() >= 4 * blocks
    _check(lib().ifx_probe_dma_lds(_ptr(src), nbytes, blocks, iters, _ptr(out), _stream(stream)),
           "ifx_probe_dma_lds")
    return blocks * 4 * iters * 8192


def probe_lds_read(offsets: torch.Tensor, out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """ds_read_b128 rate probe (ifx_probe.h) for the lane byte offsets (64 int32); returns the bytes it reads."""
    _dev(offsets, out)
    assert offsets.dtype == torch.int32 and offsets.numel() == 64
    assert out.dtype == torch.int32 and out.numel() >= blocks
    _check(lib().ifx_probe_lds_read(_ptr(offsets), blocks, iters, _ptr(out), _stream(stream)), "ifx_probe_lds_read")
    return blocks * 4 * iters * 8 * 1024


def probe_valu(kind: int, out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """VALU issue-rate probe (ifx_probe.h) of one operation pair (kind 0: requantisation core,
    1: integer add + xor, 2: the f64 form); returns the wave-level chain steps it runs."""
    _dev(out)
    assert out.dtype == torch.int32 and out.numel() >= blocks
    _check(lib().ifx_probe_valu(kind, _ptr(out), blocks, iters, _stream(stream)), "ifx_probe_valu")
    return blocks * 4 * iters * 8


# Bytes of the library-held scratch ifx_block_forward_noalloc uses (IFX_BLOCK_SCRATCH_BYTES).
BLOCK_SCRATCH_BYTES = 64 << 20


def block_forward_noalloc(p: BlockParams, x_blk, y_blk, stream=None) -> None:
    _dev(x_blk, y_blk)
    _check(lib().ifx_block_forward_noalloc(ctypes.byref(p), _ptr(x_blk), _ptr(y_blk), _stream(stream)),
           "ifx_block_forward_noalloc")


def net_workspace_bytes(p: NetParams, n: int) -> int:
    return lib().ifx_net_workspace_bytes(ctypes.byref(p), n)


def net_forward(p: NetParams, x_blk, logits, n: int, ws: torch.Tensor, stream=None) -> None:
    _dev(x_blk, logits, ws)
    _check(lib().ifx_net_forward(ctypes.byref(p), _ptr(x_blk), _ptr(logits), n, _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "ifx_net_forward")


def fold_bn(x_scale: float, y_scale: float, eps: float, w_scale: torch.Tensor, gamma: torch.Tensor,
            beta: torch.Tensor, mean: torch.Tensor, var: torch.Tensor, conv_bias: Optional[torch.Tensor] = None,
            stream=None):
    """BN folding on the device (ifx_fold_bn): float32 device tensors [c_out] (w_scale
    may have one element) -> (bias, mult, shift, status) int32 device tensors."""
    _dev(w_scale, gamma, beta, mean, var, conv_bias)
    n = gamma.numel()
    f = BnFold(n, float(x_scale), float(y_scale), float(eps), 0 if w_scale.numel() == 1 else 1,
               w_scale.data_ptr(), conv_bias.data_ptr() if conv_bias is not None else None, gamma.data_ptr(),
               beta.data_ptr(), mean.data_ptr(), var.data_ptr())
    outs = [torch.empty(n, dtype=torch.int32, device=gamma.device) for _ in range(4)]
    _check(lib().ifx_fold_bn(ctypes.byref(f), *[_ptr(o) for o in outs], _stream(stream)), "ifx_fold_bn")
    return tuple(outs)


class NetGraph:
    """ifx_net_forward for fixed buffers recorded once as a HIP graph (ifx_net_graph_create);
    launch() enqueues the whole network with one call.  Keeps the buffers alive."""

    def __init__(self, p: NetParams, x, logits, n: int, ws: torch.Tensor, keep=()):
        _dev(x, logits, ws)
        self._keep = (p, x, logits, ws, *keep)
        h = ctypes.c_void_p()
        _check(lib().ifx_net_graph_create(ctypes.byref(p), _ptr(x), _ptr(logits), n, _ptr(ws),
                                          ws.numel() * ws.element_size(), ctypes.byref(h)), "ifx_net_graph_create")
        self._h = h

    def launch(self, stream=None) -> None:
        if self._h is None:
            raise RuntimeError("graph destroyed")
        _check(lib().ifx_graph_launch(self._h, _stream(stream)), "ifx_graph_launch")

    def close(self) -> None:
        if self._h is not None:
            _check(lib().ifx_graph_destroy(self._h), "ifx_graph_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def status_string(s: int) -> str:
    return lib().ifx_status_string(s).decode()


def last_hip_error() -> int:
    return lib().ifx_last_hip_error()


def version() -> int:
    return lib().ifx_version()


def exported_symbols() -> Sequence[str]:
    return [n for n in dir(lib()) if n.startswith("ifx_")]
