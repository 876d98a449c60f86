"""Device-side assembly of the synthetic workloads for libifx.so.

Builds packed weights and the ctypes parameter structs of ifx_block_forward /
ifx_net_forward from the seeded workload description in `synth`, keeping the
torch device tensors alive for as long as the structs point at them.  All
packing runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional

import torch

# Images per pass of ifx_net_forward used by the benchmark (0 = whole batch).
DEFAULT_SUB_BATCH = 0

from . import (INPUT_NHWC, BlockParams, ConvDesc, NetGraph, NetParams, block_forward, block_workspace_bytes, conv_desc, conv_fused,
               conv_out_dims, net_forward, net_workspace_bytes, pack_act, pack_weights, synth)


@dataclass
class DeviceConv:
    """One conv layer on the device: descriptor (batch n), packed weights, per-channel params."""
    spec: synth.ConvSpec
    desc: ConvDesc
    w_blk: torch.Tensor
    bias: torch.Tensor
    mult: torch.Tensor
    shift: torch.Tensor
    out_hw: tuple

    def run(self, x_blk, y, residual=None, stream=None):
        conv_fused(self.desc, x_blk, self.w_blk, self.bias, self.mult, self.shift, residual, y, stream)


def device_conv(spec: synth.ConvSpec, seed: int, n: int, h: int, w: int, device="cuda",
                params: Optional[dict] = None, stream=None) -> DeviceConv:
    d = conv_desc(n, h, w, spec.c_in, spec.c_out, spec.k, spec.k, spec.stride, spec.pad, spec.flags)
    p = params if params is not None else synth.conv_params(seed, spec, device=device)
    p = {k: v.to(device).contiguous() for k, v in p.items()}
    w_blk = pack_weights(d, p["w"], stream=stream)
    return DeviceConv(spec, d, w_blk, p["bias"], p["mult"], p["shift"], conv_out_dims(d))


def empty_act(n, h, w, c, device="cuda") -> torch.Tensor:
    return torch.empty((n, (c + 31) // 32, h, w, 32), dtype=torch.int8, device=device)


class DeviceBlock:
    """A bottleneck (c1, c2, c3, optional projection) as one ifx_block_params."""

    def __init__(self, convs: List[DeviceConv], proj: Optional[DeviceConv]):
        self.convs = convs
        self.proj = proj
        self.params = BlockParams()
        layers = convs + ([proj] if proj is not None else [])
        for i, dc in enumerate(layers):
            self.params.d[i] = dc.desc
            self.params.w_blk[i] = dc.w_blk.data_ptr()
            self.params.bias[i] = dc.bias.data_ptr()
            self.params.mult[i] = dc.mult.data_ptr()
            self.params.shift[i] = dc.shift.data_ptr()
        self.params.has_proj = 1 if proj is not None else 0

    def workspace_bytes(self) -> int:
        return block_workspace_bytes(self.params)

    def forward(self, x_blk, y_blk, ws, stream=None):
        block_forward(self.params, x_blk, y_blk, ws, stream)


def device_block(bs: synth.BlockSpec, seed: int, n: int, h: int, w: int, device="cuda") -> DeviceBlock:
    c1 = device_conv(bs.c1, seed, n, h, w, device)
    c2 = device_conv(bs.c2, seed, n, *c1.out_hw, device)
    c3 = device_conv(bs.c3, seed, n, *c2.out_hw, device)
    proj = device_conv(bs.proj, seed, n, h, w, device) if bs.proj is not None else None
    return DeviceBlock([c1, c2, c3], proj)


class DeviceNet:
    """The ResNet-50-shaped network as one ifx_net_params (weights for batch-independent use).

    nhwc_input: forward() takes the compact NHWC image [n, h, w, c] and the stem
    reads it directly; otherwise it takes the packed [n, 1, h, w, 32] tensor.
    """

    def __init__(self, spec: synth.NetSpec, seed: int, h: int = 224, w: int = 224, device="cuda",
                 sub_batch: int = 0, nhwc_input: bool = False):
        self.spec = spec
        self.seed = seed
        self.nhwc_input = nhwc_input
        self.stem = device_conv(spec.stem, seed, 1, h, w, device)
        if nhwc_input:
            self.stem.desc.flags |= INPUT_NHWC
        hh, ww = self.stem.out_hw
        self.blocks: List[DeviceBlock] = []
        for bs in spec.blocks:
            blk = device_block(bs, seed, 1, hh, ww, device)
            self.blocks.append(blk)
            hh, ww = blk.convs[2].out_hw
        fcp = synth.fc_params(seed, spec, device=device)
        fd = conv_desc(1, 1, 1, spec.fc_in, spec.fc_out, 1, 1, 1, 0, 8)
        self.fc_w_blk = pack_weights(fd, fcp["w"].reshape(spec.fc_out, 1, 1, spec.fc_in).contiguous())
        self.fc_bias = fcp["bias"].contiguous()
        self._barr = (BlockParams * len(self.blocks))(*[b.params for b in self.blocks])
        p = NetParams()
        p.stem = self.stem.desc
        p.stem_w = self.stem.w_blk.data_ptr()
        p.stem_bias = self.stem.bias.data_ptr()
        p.stem_mult = self.stem.mult.data_ptr()
        p.stem_shift = self.stem.shift.data_ptr()
        p.n_blocks = len(self.blocks)
        p.blocks = ctypes.cast(self._barr, ctypes.POINTER(BlockParams))
        p.fc_w_blk = self.fc_w_blk.data_ptr()
        p.fc_bias = self.fc_bias.data_ptr()
        p.fc_in = spec.fc_in
        p.fc_out = spec.fc_out
        p.sub_batch = sub_batch
        self.params = p

    def set_sub_batch(self, sb: int):
        self.params.sub_batch = sb

    def workspace_bytes(self, n: int) -> int:
        return net_workspace_bytes(self.params, n)

    def forward(self, x, logits, n, ws, stream=None):
        net_forward(self.params, x, logits, n, ws, stream)

    def graph(self, x, logits, n, ws) -> NetGraph:
        """The forward pass over these buffers recorded as one HIP graph."""
        return NetGraph(self.params, x, logits, n, ws, keep=(self,))


def pack_input(x_nhwc: torch.Tensor, stream=None) -> torch.Tensor:
    return pack_act(x_nhwc.contiguous(), stream=stream)
