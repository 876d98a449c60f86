"""Python face of the CPU oracle (test infrastructure only).

Only the test suite, `__graft_entry__.smoke()` and the benchmark's CPU-baseline
leg may import this module; the GPU library never does.  Arrays are numpy, in
logical layouts: activations NHWC int8, weights OHWI int8, per-channel
parameters int32.

The arithmetic of one fused convolution lives in oracle.c; this file only
marshals arrays and composes convolutions into the bottleneck block and the
ResNet-50-shaped network exactly as the pages describe:
  * Inspur conv-merge article, section 2.2: a residual block is Conv1+BN+ReLU,
    Conv2+BN+ReLU, Conv3+BN, then Sum with the block input, then ReLU.
  * DiDi IFX DAWNBench blog, inference section: the stem is one fused
    CONV+BN+RELU+MAXPOOL.
Readings where the pages are silent: the stride of a downsampling block sits
on its 3x3 conv and on the projection; the projection has no ReLU; the head is
an integer average pool (mean rounded half away from zero) and an int8 FC with
int32 logits.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
RELU, RESIDUAL, MAXPOOL = 1, 2, 4
OK, E_OVERFLOW, E_ARG, E_NOMEM = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


def _load():
    from . import build as _build  # noqa: WPS433 (local import keeps build optional)

    lib_path = _build.build(force=False)
    lib = ctypes.CDLL(lib_path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.orc_out_dim.argtypes = [i32, i32, i32, i32]
    lib.orc_out_dim.restype = i32
    lib.orc_conv_acc.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, i32, i32, i32, vp]
    lib.orc_conv_acc.restype = i32
    lib.orc_round_shift.argtypes = [i64, i32]
    lib.orc_round_shift.restype = i64
    lib.orc_requant.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i64)]
    lib.orc_requant.restype = i32
    lib.orc_epilogue.argtypes = [vp, i64, i32, vp, vp, vp, vp, i32, vp]
    lib.orc_epilogue.restype = i32
    lib.orc_maxpool3s2p1.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.orc_maxpool3s2p1.restype = i32
    lib.orc_conv_fused.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, i32, i32, i32,
                                   vp, vp, vp, vp, i32, vp]
    lib.orc_conv_fused.restype = i32
    lib.orc_avgpool.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.orc_avgpool.restype = i32
    lib.orc_fc.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    lib.orc_fc.restype = i32
    lib.orc_pack_act.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.orc_pack_act.restype = i32
    lib.orc_unpack_act.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.orc_unpack_act.restype = i32
    lib.orc_wgroup.argtypes = [i32]
    lib.orc_wgroup.restype = i32
    lib.orc_pack_weights.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.orc_pack_weights.restype = i32
    lib.orc_pack_weights_stem.argtypes = [vp, i32, i32, vp]
    lib.orc_pack_weights_stem.restype = i32
    f64 = ctypes.c_double
    lib.orc_quantize_f32.argtypes = [vp, i64, i32, vp, vp]
    lib.orc_quantize_f32.restype = i32
    lib.orc_quantize_u8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.orc_quantize_u8.restype = i32
    lib.orc_dequantize_i32.argtypes = [vp, i64, ctypes.c_float, vp]
    lib.orc_dequantize_i32.restype = i32
    lib.orc_fold_bn.argtypes = [i32, f64, f64, f64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_fold_bn.restype = i32
    return lib


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc == E_OVERFLOW:
        raise OverflowError(f"oracle {what}: int32 overflow")
    if rc != OK:
        raise OracleError(f"oracle {what}: status {rc}")


def out_dim(n_in: int, k: int, s: int, p: int) -> int:
    return lib().orc_out_dim(n_in, k, s, p)


def conv_acc(x, w, stride: int, pad: int) -> np.ndarray:
    """int32 accumulators [N,Ho,Wo,Oc] of x (NHWC int8) with w (OHWI int8)."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    n, h, wd, c = x.shape
    oc, kh, kw, ic = w.shape
    assert ic == c, (ic, c)
    ho, wo = out_dim(h, kh, stride, pad), out_dim(wd, kw, stride, pad)
    acc = np.empty((n, ho, wo, oc), np.int32)
    _check(lib().orc_conv_acc(_ptr(x), n, h, wd, c, _ptr(w), oc, kh, kw, stride, pad, _ptr(acc)),
           "conv_acc")
    return acc


def round_shift(p: int, s: int) -> int:
    return int(lib().orc_round_shift(int(p), int(s)))


def requant(acc: int, bias: int, mult: int, shift: int) -> int:
    q = ctypes.c_int64(0)
    _check(lib().orc_requant(int(acc), int(bias), int(mult), int(shift), ctypes.byref(q)), "requant")
    return int(q.value)


def epilogue(acc, bias, mult, shift, residual=None, flags: int = 0) -> np.ndarray:
    acc = _c(acc, np.int32)
    oc = acc.shape[-1]
    npix = acc.size // oc
    res = None if residual is None else _c(residual, np.int8)
    if res is not None:
        assert res.shape == acc.shape
    out = np.empty(acc.shape, np.int8)
    _check(lib().orc_epilogue(_ptr(acc), npix, oc, _ptr(_c(bias, np.int32)), _ptr(_c(mult, np.int32)),
                              _ptr(_c(shift, np.int32)), _ptr(res), flags, _ptr(out)), "epilogue")
    return out


def maxpool3s2p1(x) -> np.ndarray:
    x = _c(x, np.int8)
    n, h, w, c = x.shape
    out = np.empty((n, out_dim(h, 3, 2, 1), out_dim(w, 3, 2, 1), c), np.int8)
    _check(lib().orc_maxpool3s2p1(_ptr(x), n, h, w, c, _ptr(out)), "maxpool")
    return out


def conv_fused(x, w, bias, mult, shift, stride: int, pad: int, flags: int,
               residual=None) -> np.ndarray:
    """One fused convolution; NHWC int8 in and out (pooled shape with MAXPOOL)."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    n, h, wd, c = x.shape
    oc, kh, kw, ic = w.shape
    assert ic == c, (ic, c)
    ho, wo = out_dim(h, kh, stride, pad), out_dim(wd, kw, stride, pad)
    if flags & MAXPOOL:
        ho, wo = out_dim(ho, 3, 2, 1), out_dim(wo, 3, 2, 1)
    res = None if residual is None else _c(residual, np.int8)
    if flags & RESIDUAL:
        assert res is not None and res.shape == (n, ho, wo, oc)
    out = np.empty((n, ho, wo, oc), np.int8)
    _check(lib().orc_conv_fused(_ptr(x), n, h, wd, c, _ptr(w), oc, kh, kw, stride, pad,
                                _ptr(_c(bias, np.int32)), _ptr(_c(mult, np.int32)),
                                _ptr(_c(shift, np.int32)), _ptr(res), flags, _ptr(out)),
           "conv_fused")
    return out


def avgpool(x) -> np.ndarray:
    x = _c(x, np.int8)
    n, h, w, c = x.shape
    out = np.empty((n, c), np.int8)
    _check(lib().orc_avgpool(_ptr(x), n, h, w, c, _ptr(out)), "avgpool")
    return out


def fc(a, w, bias) -> np.ndarray:
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    n, k = a.shape
    o, k2 = w.shape
    assert k == k2
    out = np.empty((n, o), np.int32)
    _check(lib().orc_fc(_ptr(a), n, k, _ptr(w), o, _ptr(_c(bias, np.int32)), _ptr(out)), "fc")
    return out


def pack_act(x) -> np.ndarray:
    x = _c(x, np.int8)
    n, h, w, c = x.shape
    out = np.empty((n, (c + 31) // 32, h, w, 32), np.int8)
    lib().orc_pack_act(_ptr(x), n, h, w, c, _ptr(out))
    return out


def unpack_act(blk, c: int) -> np.ndarray:
    blk = _c(blk, np.int8)
    n, c1, h, w, _ = blk.shape
    out = np.empty((n, h, w, c), np.int8)
    lib().orc_unpack_act(_ptr(blk), n, h, w, c, _ptr(out))
    return out


def wgroup(oc: int) -> int:
    return lib().orc_wgroup(oc)


def pack_weights(w) -> np.ndarray:
    w = _c(w, np.int8)
    oc, kh, kw, ic = w.shape
    o2 = wgroup(oc)
    o1 = (oc + o2 - 1) // o2
    out = np.empty((o1, kh, kw, (ic + 31) // 32, o2, 32), np.int8)
    lib().orc_pack_weights(_ptr(w), oc, kh, kw, ic, _ptr(out))
    return out


def pack_weights_stem(w) -> np.ndarray:
    w = _c(w, np.int8)
    oc, kh, kw, ic = w.shape
    assert (kh, kw) == (7, 7) and ic <= 4
    out = np.empty((oc, 8, 8, 4), np.int8)
    _check(lib().orc_pack_weights_stem(_ptr(w), oc, ic, _ptr(out)), "pack_weights_stem")
    return out


# ---------------------------------------------------------------------------
# Composition: bottleneck block and ResNet-50-shaped network.
# ---------------------------------------------------------------------------

@dataclass
class ConvParams:
    """One conv layer: OHWI int8 weights, per-channel int32 bias/mult/shift."""
    w: np.ndarray
    bias: np.ndarray
    mult: np.ndarray
    shift: np.ndarray
    stride: int
    pad: int


def conv_layer(x, p: ConvParams, flags: int, residual=None) -> np.ndarray:
    return conv_fused(x, p.w, p.bias, p.mult, p.shift, p.stride, p.pad, flags, residual)


def block(x, c1: ConvParams, c2: ConvParams, c3: ConvParams,
          proj: Optional[ConvParams] = None, intermediates: Optional[dict] = None) -> np.ndarray:
    """Bottleneck (Inspur conv-merge article, section 2.2):
    t1 = Conv1+BN+ReLU(x); t2 = Conv2+BN+ReLU(t1); sc = x or projection(x)
    (1x1, strided, BN, no ReLU); y = ReLU(Conv3+BN(t2) + sc)."""
    t1 = conv_layer(x, c1, RELU)
    t2 = conv_layer(t1, c2, RELU)
    sc = x if proj is None else conv_layer(x, proj, 0)
    y = conv_layer(t2, c3, RESIDUAL | RELU, residual=sc)
    if intermediates is not None:
        intermediates.update(t1=t1, t2=t2, sc=sc, y=y)
    return y


@dataclass
class BlockParams:
    c1: ConvParams
    c2: ConvParams
    c3: ConvParams
    proj: Optional[ConvParams]


def net(x, stem: ConvParams, blocks: Sequence[BlockParams], fc_w, fc_bias,
        trace: Optional[list] = None) -> np.ndarray:
    """Stem (CONV+BN+RELU+MAXPOOL) -> bottlenecks -> average pool -> FC (int32 logits)."""
    t = conv_layer(x, stem, RELU | MAXPOOL)
    if trace is not None:
        trace.append(t)
    for bp in blocks:
        t = block(t, bp.c1, bp.c2, bp.c3, bp.proj)
        if trace is not None:
            trace.append(t)
    a = avgpool(t)
    if trace is not None:
        trace.append(a)
    return fc(a, fc_w, fc_bias)


def fold_bn(x_scale, y_scale, eps, w_scale, gamma, beta, mean, var, conv_bias=None):
    """BN folding to (bias, mult, shift, status) int32 arrays (orc_fold_bn).  Scales and
    eps are float32 values (as the library takes them); arrays are float32 [c_out]
    (w_scale may have one element: per-tensor)."""
    L = lib()
    f32 = lambda a: np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    gamma, beta, mean, var, w_scale = f32(gamma), f32(beta), f32(mean), f32(var), f32(w_scale)
    n = gamma.size
    cb = f32(conv_bias) if conv_bias is not None else None
    outs = [np.zeros(n, np.int32) for _ in range(4)]
    rc = L.orc_fold_bn(n, float(np.float32(x_scale)), float(np.float32(y_scale)), float(np.float32(eps)),
                       0 if w_scale.size == 1 else 1, _ptr(w_scale), _ptr(cb), _ptr(gamma), _ptr(beta),
                       _ptr(mean), _ptr(var), *[_ptr(o) for o in outs])
    _check(rc, "fold_bn")
    return tuple(outs)


def quantize_f32(x, mult) -> np.ndarray:
    """fp32 NHWC image -> int8 codes (orc_quantize_f32): code = sat8(round_half_away(x * mult[ch])),
    one float32 multiply; ch is the last axis.  mult: float32 [c]."""
    x = _c(x, np.float32)
    mult = _c(mult, np.float32).ravel()
    q = np.empty(x.shape, np.int8)
    _check(lib().orc_quantize_f32(_ptr(x), x.size, mult.size, _ptr(mult), _ptr(q)), "quantize_f32")
    return q


def quantize_u8(x, mean, mult) -> np.ndarray:
    """uint8 NHWC image -> int8 codes (orc_quantize_u8): code = sat8(round_half_away(((float)u -
    mean[ch]) * mult[ch])), float32 operations; ch is the last axis."""
    x = _c(x, np.uint8)
    mean = _c(mean, np.float32).ravel()
    mult = _c(mult, np.float32).ravel()
    assert mean.size == mult.size
    q = np.empty(x.shape, np.int8)
    _check(lib().orc_quantize_u8(_ptr(x), x.size, mult.size, _ptr(mean), _ptr(mult), _ptr(q)), "quantize_u8")
    return q


def dequantize_i32(q, scale) -> np.ndarray:
    """int32 codes (the logits) -> float32 (orc_dequantize_i32): y = (float)q * scale."""
    q = _c(q, np.int32)
    y = np.empty(q.shape, np.float32)
    _check(lib().orc_dequantize_i32(_ptr(q), q.size, float(np.float32(scale)), _ptr(y)), "dequantize_i32")
    return y
