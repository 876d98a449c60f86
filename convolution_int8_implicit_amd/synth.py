"""Seeded synthetic workloads for the fused int8 convolution path.

This module holds no step of the method's arithmetic: it only describes the
workload shapes and draws seeded integers, so that the GPU library and the CPU
oracle can be fed identical inputs.

Random numbers: a counter-based generator built on the SplitMix64 output
function of Steele, Lea and Flood ("Fast splittable pseudorandom number
generators", OOPSLA 2014).  Element `i` of the tensor with id `tid` under
`seed` is

    stream = mix64((seed << 32) | tid)
    x_i    = mix64(stream + (i + 1) * GAMMA)            (mod 2^64)
    value  = lo + ((x_i >> 32) mod (hi - lo + 1))

so any element (an image, a layer) can be regenerated on its own.  Tensor ids
are 16 * layer_index + role, with roles below; layers are numbered in network
order (stem 0, then for each bottleneck [projection], c1, c2, c3; FC last).
All arithmetic is on int64 torch tensors (wrapping multiply), so the same
values come out on the CPU and on the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

ROLE_INPUT, ROLE_W, ROLE_BIAS, ROLE_MULT, ROLE_SHIFT, ROLE_RESIDUAL = range(6)

RELU, RESIDUAL, MAXPOOL = 1, 2, 4

# Value ranges of the synthetic workloads.
W_RANGE = (-127, 127)
BIAS_RANGE = (-(1 << 16), 1 << 16)
MULT_RANGE = (1 << 30, (1 << 31) - 1)
SHIFT_RANGE = (8, 16)
POST_RELU_RANGE = (0, 127)
IMAGE_RANGE = (-128, 127)


def _s64(u: int) -> int:
    u &= MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _lsr(z, 30)
    z = z * _s64(MIX1)
    z = z ^ _lsr(z, 27)
    z = z * _s64(MIX2)
    return z ^ _lsr(z, 31)


def mix64_int(z: int) -> int:
    """Pure-Python SplitMix64 output function on unsigned 64-bit integers."""
    z &= MASK64
    z = (z ^ (z >> 30)) * MIX1 & MASK64
    z = (z ^ (z >> 27)) * MIX2 & MASK64
    return z ^ (z >> 31)


def tensor_id(layer: int, role: int) -> int:
    return 16 * layer + role


def stream_key(seed: int, tid: int) -> int:
    return mix64_int(((seed & 0xFFFFFFFF) << 32) | (tid & 0xFFFFFFFF))


def uniform_flat(seed: int, tid: int, index: torch.Tensor, lo: int, hi: int) -> torch.Tensor:
    """Values for the given flat element indices (int64 tensor, any device)."""
    span = hi - lo + 1
    assert 0 < span <= (1 << 32)
    z = index.to(torch.int64) + 1
    z = z * _s64(GAMMA) + _s64(stream_key(seed, tid))
    x = _lsr(_mix(z), 32)
    return x.remainder(span) + lo


def uniform(seed: int, tid: int, shape: Sequence[int], lo: int, hi: int,
            dtype=torch.int8, device="cpu", chunk: int = 1 << 26) -> torch.Tensor:
    """A full tensor of seeded uniform integers in [lo, hi], C order."""
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=dtype, device=device)
    for start in range(0, numel, chunk):
        stop = min(numel, start + chunk)
        idx = torch.arange(start, stop, dtype=torch.int64, device=device)
        out[start:stop] = uniform_flat(seed, tid, idx, lo, hi).to(dtype)
    return out.view(*shape)


def uniform_rows(seed: int, tid: int, shape: Sequence[int], rows: Sequence[int], lo: int, hi: int,
                 dtype=torch.int8, device="cpu") -> torch.Tensor:
    """Only the listed leading-dimension rows (e.g. images) of a seeded tensor."""
    per = 1
    for s in shape[1:]:
        per *= int(s)
    r = torch.as_tensor(list(rows), dtype=torch.int64, device=device)
    idx = (r[:, None] * per + torch.arange(per, dtype=torch.int64, device=device)[None, :]).reshape(-1)
    return uniform_flat(seed, tid, idx, lo, hi).to(dtype).view(len(rows), *shape[1:])


# ---------------------------------------------------------------------------
# Workload description.
# ---------------------------------------------------------------------------

@dataclass
class ConvSpec:
    """One convolution layer of a workload (logical shapes)."""
    layer: int          # layer index (tensor-id namespace)
    c_in: int
    c_out: int
    k: int
    stride: int
    pad: int
    flags: int
    name: str = ""

    def out_hw(self, h: int, w: int) -> Tuple[int, int]:
        ho = (h + 2 * self.pad - self.k) // self.stride + 1
        wo = (w + 2 * self.pad - self.k) // self.stride + 1
        if self.flags & MAXPOOL:
            ho = (ho + 2 - 3) // 2 + 1
            wo = (wo + 2 - 3) // 2 + 1
        return ho, wo

    def macs(self, n: int, h: int, w: int) -> int:
        ho = (h + 2 * self.pad - self.k) // self.stride + 1
        wo = (w + 2 * self.pad - self.k) // self.stride + 1
        return n * ho * wo * self.c_out * self.k * self.k * self.c_in


@dataclass
class BlockSpec:
    c1: ConvSpec
    c2: ConvSpec
    c3: ConvSpec
    proj: Optional[ConvSpec] = None


@dataclass
class NetSpec:
    stem: ConvSpec
    blocks: List[BlockSpec] = field(default_factory=list)
    fc_layer: int = 0
    fc_in: int = 2048
    fc_out: int = 1000


def resnet50_spec(stages=(3, 4, 6, 3), widths=(64, 128, 256, 512), expansion: int = 4) -> NetSpec:
    """ResNet-50-shaped backbone: 7x7/s2 stem with fused 3x3/s2 max-pool, then
    bottlenecks whose first block per stage carries the stride on its 3x3 conv
    and on a 1x1 projection shortcut."""
    layer = 0
    stem = ConvSpec(layer, 3, 64, 7, 2, 3, RELU | MAXPOOL, "stem")
    layer += 1
    blocks = []
    c_in = 64
    for si, (nb, wdt) in enumerate(zip(stages, widths)):
        for bi in range(nb):
            stride = 2 if (si > 0 and bi == 0) else 1
            proj = None
            if bi == 0:
                proj = ConvSpec(layer, c_in, wdt * expansion, 1, stride, 0, 0, f"res{si + 2}.{bi + 1}.proj")
                layer += 1
            c1 = ConvSpec(layer, c_in, wdt, 1, 1, 0, RELU, f"res{si + 2}.{bi + 1}.c1")
            c2 = ConvSpec(layer + 1, wdt, wdt, 3, stride, 1, RELU, f"res{si + 2}.{bi + 1}.c2")
            c3 = ConvSpec(layer + 2, wdt, wdt * expansion, 1, 1, 0, RESIDUAL | RELU,
                          f"res{si + 2}.{bi + 1}.c3")
            layer += 3
            blocks.append(BlockSpec(c1, c2, c3, proj))
            c_in = wdt * expansion
    return NetSpec(stem, blocks, fc_layer=layer, fc_in=c_in, fc_out=1000)


def resnet26_spec() -> NetSpec:
    """ResNet-26-shaped backbone (the DAWNBench inference model of the DiDi IFX
    blog, read as the ResNet-50 layout with two bottlenecks per stage): 26
    weighted layers = stem + 8 x 3 bottleneck convs + FC, plus 4 projections."""
    return resnet50_spec(stages=(2, 2, 2, 2))


@dataclass
class Workload:
    """One of the five synthetic workloads (seed = its index)."""
    index: int
    name: str
    kind: str            # "conv", "block", "stem" or "net"
    n: int
    h: int
    w: int
    convs: List[ConvSpec] = field(default_factory=list)
    input_range: Tuple[int, int] = POST_RELU_RANGE
    net: Optional[NetSpec] = None


def res3_conv3(index: int, n: int) -> Workload:
    spec = ConvSpec(0, 128, 512, 1, 1, 0, RESIDUAL | RELU, "res3.x.conv3")
    return Workload(index, f"res3.x conv3 1x1 128->512 +BN+Sum+ReLU, 28x28, batch {n}", "conv",
                    n, 28, 28, [spec], POST_RELU_RANGE)


def res3_bottleneck(index: int, n: int) -> Workload:
    convs = [ConvSpec(0, 512, 128, 1, 1, 0, RELU, "c1"),
             ConvSpec(1, 128, 128, 3, 1, 1, RELU, "c2"),
             ConvSpec(2, 128, 512, 1, 1, 0, RESIDUAL | RELU, "c3")]
    return Workload(index, f"res3 bottleneck 512->128->128->512, 28x28, batch {n}", "block",
                    n, 28, 28, convs, POST_RELU_RANGE)


def stem_workload(index: int, n: int) -> Workload:
    spec = ConvSpec(0, 3, 64, 7, 2, 3, RELU | MAXPOOL, "stem")
    return Workload(index, f"stem 7x7/s2 3->64 +BN+ReLU+maxpool3x3/s2, 224x224, batch {n}", "stem",
                    n, 224, 224, [spec], IMAGE_RANGE)


def net_workload(index: int, n: int) -> Workload:
    return Workload(index, f"ResNet-50-shaped int8 backbone + avgpool + FC, 224x224, batch {n}", "net",
                    n, 224, 224, [], IMAGE_RANGE, resnet50_spec())


def latency_workload(n: int = 1) -> Workload:
    """The batch-1 latency setting: ResNet-26-shaped network on 224x224x3 images (seed 5)."""
    return Workload(5, f"ResNet-26-shaped int8 backbone + avgpool + FC, 224x224, batch {n}", "net",
                    n, 224, 224, [], IMAGE_RANGE, resnet26_spec())


def workloads() -> List[Workload]:
    """The five workloads, in seed order."""
    return [res3_conv3(0, 1), res3_conv3(1, 2048), res3_bottleneck(2, 256), stem_workload(3, 128),
            net_workload(4, 2048)]


def workload(index: int, n: Optional[int] = None) -> Workload:
    base = workloads()[index]
    if n is None or n == base.n:
        return base
    maker = {0: res3_conv3, 1: res3_conv3, 2: res3_bottleneck, 3: stem_workload, 4: net_workload}[index]
    return maker(index, n)


# ---------------------------------------------------------------------------
# Parameter and tensor draws.
# ---------------------------------------------------------------------------

def conv_params(seed: int, spec: ConvSpec, device="cpu") -> dict:
    """Seeded parameters of one conv: OHWI int8 weights and int32 bias/mult/shift."""
    L = spec.layer
    return {
        "w": uniform(seed, tensor_id(L, ROLE_W), (spec.c_out, spec.k, spec.k, spec.c_in), *W_RANGE,
                     dtype=torch.int8, device=device),
        "bias": uniform(seed, tensor_id(L, ROLE_BIAS), (spec.c_out,), *BIAS_RANGE, dtype=torch.int32,
                        device=device),
        "mult": uniform(seed, tensor_id(L, ROLE_MULT), (spec.c_out,), *MULT_RANGE, dtype=torch.int32,
                        device=device),
        "shift": uniform(seed, tensor_id(L, ROLE_SHIFT), (spec.c_out,), *SHIFT_RANGE, dtype=torch.int32,
                         device=device),
    }


def fc_params(seed: int, spec: NetSpec, device="cpu") -> dict:
    L = spec.fc_layer
    return {
        "w": uniform(seed, tensor_id(L, ROLE_W), (spec.fc_out, spec.fc_in), *W_RANGE, dtype=torch.int8,
                     device=device),
        "bias": uniform(seed, tensor_id(L, ROLE_BIAS), (spec.fc_out,), *BIAS_RANGE, dtype=torch.int32,
                        device=device),
    }


def input_shape(wl: Workload) -> Tuple[int, int, int, int]:
    c = wl.convs[0].c_in if wl.convs else wl.net.stem.c_in
    return (wl.n, wl.h, wl.w, c)


def input_tensor(wl: Workload, device="cpu", rows: Optional[Sequence[int]] = None) -> torch.Tensor:
    """NHWC int8 input of a workload (all images, or only `rows`)."""
    shape = input_shape(wl)
    tid = tensor_id(0, ROLE_INPUT)
    if rows is None:
        return uniform(wl.index, tid, shape, *wl.input_range, dtype=torch.int8, device=device)
    return uniform_rows(wl.index, tid, shape, rows, *wl.input_range, dtype=torch.int8, device=device)


def residual_tensor(wl: Workload, device="cpu", rows: Optional[Sequence[int]] = None) -> torch.Tensor:
    """NHWC int8 shortcut input of a single-conv workload with RESIDUAL."""
    spec = wl.convs[0]
    ho, wo = spec.out_hw(wl.h, wl.w)
    shape = (wl.n, ho, wo, spec.c_out)
    tid = tensor_id(0, ROLE_RESIDUAL)
    if rows is None:
        return uniform(wl.index, tid, shape, *POST_RELU_RANGE, dtype=torch.int8, device=device)
    return uniform_rows(wl.index, tid, shape, rows, *POST_RELU_RANGE, dtype=torch.int8, device=device)
