#!/usr/bin/env python3
"""Benchmark of the fused int8 ResNet convolution path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload net|conv1x1|conv1x1_b1|block|stem]

Default workload: the ResNet-50-shaped int8 backbone + average pool + int8 FC
at batch 2048 on 224x224x3 images (synthetic, seeded).  One step is the whole
hot path over the batch: fused stem reading the NHWC int8 images directly
(conv 7x7/s2 + BN + ReLU + max-pool, written as NC/32HW32), 16 bottlenecks of fused convolutions
(BN + requant + shortcut + ReLU in the epilogue), average pool and FC to int32
logits.  Weights are packed once beforehand (offline reblocking).

Prints ONE JSON line with the throughput (images/s), int8 TOPS, a roofline
object for the dominant kernel (HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_I8 = 5.0e15      # MI355X dense int8 MFMA, ops/s
PEAK_HBM = 8.0e12     # MI355X HBM3E, bytes/s
RIDGE = PEAK_I8 / PEAK_HBM
METRIC = "int8 TOPS + images/s (fused conv stack), % of int8 MFMA peak / HBM BW"


def kernel_name(spec, nhwc_input=True, proj=None, w=None) -> str:
    """The kernel template instance a conv layer dispatches to, spelled as rocprofv3
    prints it (mirrors the library's host dispatch).  proj: the projection shortcut's
    spec when `spec` is a conv3 fused with it (ifx_conv_proj_fused); w: the input width."""
    if spec.k == 7:
        return f"stem_kernel<{1 if nhwc_input else 0}>"
    oc_pad = (spec.c_out + 31) // 32 * 32
    bm, bn = (128, 128) if oc_pad > 64 else (256, 64)
    res = "true" if spec.flags & 2 else "false"
    relu = "true" if spec.flags & 1 else "false"
    i1 = (spec.c_in + 31) // 32
    if proj is not None and spec.k == 1 and spec.stride == 1 and i1 <= 4 and (proj.c_in + 31) // 32 <= 4:
        # both contractions short: the small-K fused kernel, shortcut kept in registers
        return f"conv1x1_proj_kernel<{bm}, {bn}, {((proj.c_in + 31) // 32 + 1) // 2}, {(i1 + 1) // 2}, {relu}>"
    if spec.k == 3 and spec.stride == 1 and i1 <= 2 and w is not None and 48 <= w <= 62 and res == "false" \
            and proj is None:
        return f"conv3x3_halo_kernel<{relu}>"  # stride-1 3x3, <= 64 input channels: haloed window
    if spec.k == 1 and spec.pad == 0 and i1 <= 4 and proj is None:
        return f"conv1x1_kernel<{bm}, {bn}, {(i1 + 1) // 2}, {res}, {relu}>"
    st = 2
    if spec.k == 1 and oc_pad > 64 and res == "false":
        bm, bn, st = 256, 128, 3  # wide 1x1 convolutions without a shortcut
    if spec.k == 3 and spec.stride == 2 and oc_pad >= 256 and res == "false":
        bm, bn = 128, 256  # strided 3x3 with >= 256 output channels
    return f"igemm_kernel<{spec.k}, {spec.k}, {bm}, {bn}, {st}, {res}, {relu}, {'false' if proj is None else 'true'}>"


# Sources each kernel family is built from: HBM traffic taken from counters is only
# reported while these files are unchanged.
KERNEL_SOURCES = {
    "igemm_kernel": ["igemm.hip", "device_common.h", "ifx_internal.h"],
    "conv1x1_kernel": ["conv1x1.hip", "device_common.h", "ifx_internal.h"],
    "conv1x1_proj_kernel": ["conv1x1.hip", "device_common.h", "ifx_internal.h"],
    "conv3x3_halo_kernel": ["igemm.hip", "device_common.h", "ifx_internal.h"],
    "stem_kernel": ["stem.hip", "device_common.h", "ifx_internal.h"],
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(ROOT, "convolution_int8_implicit_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary of this
    workload (profiles/hbm_traffic_<workload>.txt), or None when there is none or
    the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if not line.startswith("kernel: "):
                continue
            fields = dict(kv.split("=", 1) for kv in line.strip()[len("kernel: "):].split(" | ")[1:])
            name = line[len("kernel: "):].split(" | ")[0].strip()
            if name == kernel and fields.get("digest") == source_digest(kernel):
                return int(fields["hbm_bytes_per_launch"])
    return None


def summarize_pmc(fetch_csv: str, write_csv: str, calib_bytes: int, out: str, workload: str, note: str):
    """Turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE;
    KiB per dispatch) into per-launch HBM bytes per kernel instance, scaled by what the
    same counters read for a plain copy of calib_bytes (torch bitwise_not, int32)."""
    import csv
    import re
    from collections import defaultdict

    def short(name):
        m = re.search(r"((?:conv1x1_proj|conv1x1|conv3x3_halo|igemm|stem)_kernel<[^>]*>)", name)
        if m:
            return m.group(1)
        return "copy" if "bitwise_not" in name else None

    def read(path, counter):
        per = defaultdict(list)
        with open(path) as fh:
            rows = [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        # only the per-launch replays, which follow the network's last average-pool dispatch:
        # they are the launches the roofline times (the forward's concurrent passes are not)
        last_pool = max((int(r["Dispatch_Id"]) for r in rows if "avgpool_kernel" in r["Kernel_Name"]), default=-1)
        for r in rows:
            k = short(r["Kernel_Name"])
            if k and (k == "copy" or int(r["Dispatch_Id"]) > last_pool):
                per[k].append((int(r["Dispatch_Id"]), float(r["Counter_Value"]) * 1024.0))
        # the calibration copies are the process's last three bitwise_not dispatches
        per["copy"] = sorted(per["copy"])[-3:]
        return {k: [v for _, v in sorted(lst)] for k, lst in per.items()}

    fe, wr = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    med = lambda v: sorted(v)[len(v) // 2]
    cf, cw = med(fe["copy"]), med(wr["copy"])
    fs, ws = calib_bytes / cf, calib_bytes / cw
    lines = [f"# HBM traffic per dispatch, workload {workload}, from rocprofv3 counters",
             "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two separate --pmc runs, each",
             "# scaled by what the counter reads for a plain copy kernel of known size run in the",
             "# same process (torch bitwise_not over int32: reads and writes calib_bytes).",
             "# Dispatches: the per-launch replays bench.py times for the roofline (those after the",
             "# network's last average-pool dispatch).", f"# {note}",
             f"copy_calibration: calib_bytes={calib_bytes} | fetch_read={cf:.0f} | write_read={cw:.0f} | "
             f"fetch_scale={fs:.4f} | write_scale={ws:.4f}"]
    for k in sorted(set(fe) & set(wr)):
        if k == "copy":
            continue
        f_avg = sum(fe[k]) / len(fe[k]) * fs
        w_avg = sum(wr[k]) / len(wr[k]) * ws
        lines.append(f"kernel: {k} | digest={source_digest(k)} | dispatches={len(fe[k])} | "
                     f"fetch_bytes_per_launch={f_avg:.0f} | write_bytes_per_launch={w_avg:.0f} | "
                     f"hbm_bytes_per_launch={f_avg + w_avg:.0f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_csv: str, stats_csv: str, out: str, workload: str, note: str):
    """The rocprofv3 --kernel-trace --stats summary of a bench.py run: the --stats table (all
    dispatches), then per kernel instance the average of the per-launch replays alone (the
    dispatches after the network's last average-pool dispatch), which is what the roofline's
    avg_launch_us measures with HIP events."""
    import csv
    import re
    from collections import defaultdict

    def clean(nm):
        nm = nm.replace("void ifx::(anonymous namespace)::", "").replace("ifx::(anonymous namespace)::", "")
        return nm if len(nm) <= 100 or nm.startswith(("igemm", "conv1x1", "stem", "avgpool", "splitk")) else nm[:100] + "..."

    lines = [f"# rocprofv3 kernel statistics, workload {workload}", f"# {note}", "#",
             "# all dispatches (rocprofv3 --stats):",
             "# name | calls | average ns | total ns | percent | min ns | max ns"]
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            lines.append(f'{clean(r["Name"])} | {r["Calls"]} | {float(r["AverageNs"]):.0f} | '
                         f'{float(r["TotalDurationNs"]):.0f} | {float(r["Percentage"]):.2f} | '
                         f'{float(r["MinNs"]):.0f} | {float(r["MaxNs"]):.0f}')
    with open(trace_csv) as fh:
        rows = list(csv.DictReader(fh))
    last_pool = max((int(r["Dispatch_Id"]) for r in rows if "avgpool_kernel" in r["Kernel_Name"]), default=-1)
    rep = defaultdict(list)
    for r in rows:
        m = re.search(r"((?:conv1x1_proj|conv1x1|conv3x3_halo|igemm|stem)_kernel<[^>]*>)", r["Kernel_Name"])
        if m and int(r["Dispatch_Id"]) > last_pool:
            rep[m.group(1)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["#", "# per-launch replays only (one conv launch at a time on one stream; bench.py's",
              "# roofline avg_launch_us is the HIP-event average of these launches):",
              "# name | replays | average ns | min ns | max ns"]
    for k, v in sorted(rep.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"replay: {k} | {len(v)} | {sum(v) / len(v):.0f} | {min(v)} | {max(v)}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def layer_work(spec, n, h, w):
    """(ops, algorithmic bytes, output h, w) of one conv at batch n on an h x w input.
    ops = 2 per real MAC; bytes = each distinct tensor crossing HBM once: real input
    channels (only sampled pixels for a strided 1x1), weights, 12 B/channel of
    bias/mult/shift, the shortcut, and the output (pooled for the stem)."""
    ho = (h + 2 * spec.pad - spec.k) // spec.stride + 1
    wo = (w + 2 * spec.pad - spec.k) // spec.stride + 1
    ops = 2 * n * ho * wo * spec.c_out * spec.k * spec.k * spec.c_in
    in_px = n * ho * wo if (spec.k == 1 and spec.stride > 1) else n * h * w
    byts = in_px * spec.c_in + spec.c_out * spec.k * spec.k * spec.c_in + 12 * spec.c_out
    oh, ow = ho, wo
    if spec.flags & 4:
        oh, ow = (ho - 1) // 2 + 1, (wo - 1) // 2 + 1
    byts += n * oh * ow * spec.c_out
    if spec.flags & 2:
        byts += n * ho * wo * spec.c_out
    return ops, byts, oh, ow


def net_layers(net, n):
    """[(spec, n, h, w)] for every conv launch of the network, in order."""
    out = [(net.stem, n, 224, 224)]
    h = w = 56
    for b in net.blocks:
        out.append((b.c1, n, h, w))
        h2 = (h + 2 - 3) // b.c2.stride + 1
        out.append((b.c2, n, h, w))
        if b.proj is not None:
            out.append((b.proj, n, h, w))
        out.append((b.c3, n, h2, h2))
        h = w = h2
    return out


def cpu_baseline(workload: str, budget_s: float = 20.0):
    """The CPU oracle, untuned, on a bounded sample of the same workload."""
    import numpy as np

    from convolution_int8_implicit_amd import synth
    from oracle import ref as orc
    from oracle.ref import BlockParams, ConvParams

    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

    def cp(wl, spec):
        p = synth.conv_params(wl.index, spec)
        return ConvParams(p["w"].numpy(), p["bias"].numpy(), p["mult"].numpy(), p["shift"].numpy(), spec.stride,
                          spec.pad)

    if workload in ("net", "net26_b1"):
        wl = synth.workload(4) if workload == "net" else synth.latency_workload(64)
        stem = cp(wl, wl.net.stem)
        blocks = [BlockParams(cp(wl, b.c1), cp(wl, b.c2), cp(wl, b.c3), cp(wl, b.proj) if b.proj else None)
                  for b in wl.net.blocks]
        fcp = synth.fc_params(wl.index, wl.net)
        fw, fb = fcp["w"].numpy(), fcp["bias"].numpy()

        def run(rows):
            x = synth.input_tensor(wl, rows=rows).numpy()
            t0 = time.perf_counter()
            orc.net(x, stem, blocks, fw, fb)
            return time.perf_counter() - t0
        per_img_ops = sum(layer_work(sp, 1, hh, ww)[0] for sp, _, hh, ww in net_layers(wl.net, 1)) + \
            2 * wl.net.fc_in * wl.net.fc_out
    else:
        idx = {"conv1x1": 1, "conv1x1_b1": 0, "block": 2, "stem": 3}[workload]
        wl = synth.workload(idx)
        cps = [cp(wl, s) for s in wl.convs]

        def run(rows):
            x = synth.input_tensor(wl, rows=rows).numpy()
            r = synth.residual_tensor(wl, rows=rows).numpy() if wl.kind == "conv" else None
            t0 = time.perf_counter()
            if wl.kind == "block":
                orc.block(x, *cps)
            else:
                orc.conv_layer(x, cps[0], wl.convs[0].flags, residual=r)
            return time.perf_counter() - t0
        per_img_ops = sum(2 * s.macs(1, wl.h, wl.w) for s in wl.convs)
    run([0])         # warm-up (first-call costs)
    t1 = run([0])    # one image, warm
    k = int(max(1, min(wl.n - 1, budget_s / max(t1, 1e-3))))
    rows = list(range(1, 1 + k))
    tk = run(rows)
    return {"value": round(k / tk, 3), "unit": "images/s", "cores": cores, "kind": "oracle",
            "sample": f"{k} of {wl.n} images of the same workload (after 2 untimed single-image runs), "
                      f"{tk:.1f} s, {k * per_img_ops / tk / 1e9:.2f} GOPS int8"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="net",
                    choices=["net", "net26_b1", "conv1x1", "conv1x1_b1", "block", "stem"])
    ap.add_argument("--sub-batch", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy this many MiB with a plain elementwise kernel (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic_<workload>.txt from two counter runs and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "STATS_CSV"),
                    help="write profiles/kernel_stats_<workload>.txt from a --kernel-trace --stats run and exit")
    ap.add_argument("--note", default="", help="command lines recorded in the --summarize-* output")
    ap.add_argument("--packed-input", action="store_true",
                    help="feed the stem a packed NC/32HW32 input made by a separate pack kernel in the step")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1],
                        os.path.join(ROOT, "profiles", f"kernel_stats_{args.workload}.txt"), args.workload, args.note)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_calibration_mib << 20,
                      os.path.join(ROOT, "profiles", f"hbm_traffic_{args.workload}.txt"), args.workload, args.note)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (images are independent, so a "
              "batch shards over GPUs with no exchange step); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import convolution_int8_implicit_amd as ifx
    from convolution_int8_implicit_amd import model, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    ifx.lib()
    stream = torch.cuda.current_stream()
    sub_batch = model.DEFAULT_SUB_BATCH if args.sub_batch is None else args.sub_batch

    # ---------------- workload setup (untimed) ----------------
    if args.workload in ("net", "net26_b1"):
        wl = synth.workload(4) if args.workload == "net" else synth.latency_workload(1)
        n = wl.n
        net = model.DeviceNet(wl.net, wl.index, sub_batch=sub_batch, nhwc_input=not args.packed_input)
        x_nhwc = synth.input_tensor(wl, device="cuda")
        ws = torch.empty(net.workspace_bytes(n), dtype=torch.int8, device="cuda")
        logits = torch.empty((n, wl.net.fc_out), dtype=torch.int32, device="cuda")
        if args.packed_input:
            x_blk = model.empty_act(n, 224, 224, 3)

            def step():
                ifx.pack_act(x_nhwc, out=x_blk, stream=stream)
                net.forward(x_blk, logits, n, ws, stream)
        elif args.workload == "net26_b1":
            x_blk = x_nhwc
            net.forward(x_nhwc, logits, n, ws, stream)  # eager once: one-time device queries
            graph = net.graph(x_nhwc, logits, n, ws)

            def step():
                graph.launch(stream)
        else:
            x_blk = x_nhwc

            def step():
                net.forward(x_nhwc, logits, n, ws, stream)
        layers = net_layers(wl.net, n)
        total_ops = sum(layer_work(s, nn, h, w)[0] for s, nn, h, w in layers) + 2 * n * wl.net.fc_in * wl.net.fc_out
        config = {"workload": wl.name, "batch": n, "image": "224x224x3 int8 NHWC",
                  "convs": 1 + sum(3 + (b.proj is not None) for b in wl.net.blocks),
                  "head": "avgpool + FC 2048->1000 int32 logits", "sub_batch": sub_batch,
                  "step": ("input pack + " if args.packed_input else "") +
                  ("ifx_graph_launch of the recorded ifx_net_forward" if args.workload == "net26_b1"
                   else "ifx_net_forward")}
    else:
        idx = {"conv1x1": 1, "conv1x1_b1": 0, "block": 2, "stem": 3}[args.workload]
        wl = synth.workload(idx)
        n = wl.n
        dcs = [model.device_conv(s, wl.index, n, wl.h, wl.w) if i == 0 else None for i, s in enumerate(wl.convs)]
        x_blk = ifx.pack_act(synth.input_tensor(wl, device="cuda"))
        if wl.convs[0].k == 7 and not args.packed_input:
            dcs[0].desc.flags |= ifx.INPUT_NHWC
            x_blk = synth.input_tensor(wl, device="cuda")
        if wl.kind == "block":
            dcs = [model.device_conv(s, wl.index, n, 28, 28) for s in wl.convs]
            blk = model.DeviceBlock(dcs, None)
            ws = torch.empty(blk.workspace_bytes(), dtype=torch.int8, device="cuda")
            y = model.empty_act(n, 28, 28, 512)

            def step():
                blk.forward(x_blk, y, ws, stream)
            layers = [(s, n, 28, 28) for s in wl.convs]
        else:
            spec = wl.convs[0]
            ho, wo = spec.out_hw(wl.h, wl.w)
            y = model.empty_act(n, ho, wo, spec.c_out)
            res = ifx.pack_act(synth.residual_tensor(wl, device="cuda")) if spec.flags & 2 else None

            def step():
                dcs[0].run(x_blk, y, res, stream)
            layers = [(spec, n, wl.h, wl.w)]
        total_ops = sum(layer_work(s, nn, h, w)[0] for s, nn, h, w in layers)
        config = {"workload": wl.name, "batch": n}

    # ---------------- timed region ----------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sec_per_step = max(ev0.elapsed_time(ev1) * 1e-3, 0.0) / args.steps
    extra = {}
    if args.workload == "net26_b1":
        # the same forward launched kernel by kernel from the host, for comparison
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            net.forward(x_nhwc, logits, n, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        extra = {"latency_us": round(sec_per_step * 1e6, 1),
                 "eager_latency_us": round(e0.elapsed_time(e1) * 1e3 / args.steps, 1)}
    img_s = n / sec_per_step
    tops = total_ops / sec_per_step / 1e12

    # ---------------- per-kernel durations (HIP events on the launch stream) ----------------
    # The convolutions of a step are replayed one launch at a time through ifx_conv_fused on
    # the same stream and the same data flow as the drivers (real activations), each launch
    # bracketed by HIP events; durations are grouped by kernel instance.
    def with_batch(dc, nb):
        d = ifx.ConvDesc.from_buffer_copy(dc.desc)
        d.n = nb
        return model.DeviceConv(dc.spec, d, dc.w_blk, dc.bias, dc.mult, dc.shift, dc.out_hw)

    launches = []  # (kernel instance, ops, algorithmic bytes, fn); fn only, for bookkeeping steps
    nhwc = not args.packed_input

    def conv_launch(spec, nb_, h, w, fn):
        ops, byts, _, _ = layer_work(spec, nb_, h, w)
        return (kernel_name(spec, nhwc, w=w), ops, byts, fn)

    def proj_launch(c3spec, pspec, nb_, h3, w3, hp, wp, fn):
        # conv3 + projection in one kernel: both contractions; the shortcut is not a tensor
        o3, b3, oh, ow = layer_work(c3spec, nb_, h3, w3)
        op, bp, _, _ = layer_work(pspec, nb_, hp, wp)
        shortcut = nb_ * oh * ow * c3spec.c_out
        return (kernel_name(c3spec, nhwc, proj=pspec), o3 + op, b3 + bp - 2 * shortcut, fn)

    if args.workload in ("net", "net26_b1"):
        # the forward's passes: a whole batch of >= 192 images runs as two concurrent halves
        if sub_batch == 0 and n >= 192:
            nb = (n + 1) // 2
        else:
            nb = sub_batch if 0 < sub_batch < n else n
        passes = (n + nb - 1) // nb
        big = max(ifx.act_bytes(nb, h, w, s.c_out if s.k != 7 else 64) for s, _, h, w in layers)
        big = max(big, ifx.act_bytes(nb, 56, 56, 256))
        bufs = [torch.empty(big, dtype=torch.int8, device="cuda") for _ in range(4)]
        cur, nxt, t1, t2 = bufs
        stem = with_batch(net.stem, nb)
        launches.append(conv_launch(wl.net.stem, nb, 224, 224, lambda: stem.run(x_blk[:nb], cur, None, stream)))
        h = w = 56
        state = {"cur": cur, "nxt": nxt}
        for bs, db in zip(wl.net.blocks, net.blocks):
            c1, c2, c3 = (with_batch(d, nb) for d in db.convs)
            pj = with_batch(db.proj, nb) if db.proj is not None else None
            h2 = c2.out_hw[0]

            def mk(c, xin_key, out, res_key=None):
                def f():
                    xin = state[xin_key] if isinstance(xin_key, str) else xin_key
                    res = None if res_key is None else (state[res_key] if isinstance(res_key, str) else res_key)
                    o = state[out] if isinstance(out, str) else out
                    c.run(xin, o, res, stream)
                return f

            def mk_proj(c3_, pj_):
                def f():
                    ifx.conv_proj_fused(c3_.desc, t2, c3_.w_blk, c3_.bias, c3_.mult, c3_.shift, pj_.desc,
                                        state["cur"], pj_.w_blk, pj_.bias, pj_.mult, pj_.shift, state["nxt"], stream)
                return f
            launches.append(conv_launch(bs.c1, nb, h, w, mk(c1, "cur", t1)))
            launches.append(conv_launch(bs.c2, nb, h, w, mk(c2, t1, t2)))
            if pj is not None:
                launches.append(proj_launch(bs.c3, bs.proj, nb, h2, h2, h, w, mk_proj(c3, pj)))
            else:
                launches.append(conv_launch(bs.c3, nb, h2, h2, mk(c3, t2, "nxt", "cur")))

            def swap():
                state["cur"], state["nxt"] = state["nxt"], state["cur"]
            launches.append((None, 0, 0, swap))
            h = w = h2
    else:
        nb, passes = n, 1
        if wl.kind == "block":
            t1b = model.empty_act(n, 28, 28, 128)
            t2b = model.empty_act(n, 28, 28, 128)
            c1, c2, c3 = dcs
            launches = [conv_launch(wl.convs[0], n, 28, 28, lambda: c1.run(x_blk, t1b, None, stream)),
                        conv_launch(wl.convs[1], n, 28, 28, lambda: c2.run(t1b, t2b, None, stream)),
                        conv_launch(wl.convs[2], n, 28, 28, lambda: c3.run(t2b, y, x_blk, stream))]
        else:
            launches = [conv_launch(wl.convs[0], n, wl.h, wl.w, step)]
    reps = max(1, min(args.steps, 5) if args.workload == "net" else args.steps)
    evs = []
    torch.cuda.synchronize()
    for _ in range(reps):
        for name, ops, byts, fn in launches:
            if name is None:
                fn()
                continue
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((name, ops, byts, a, b))
    torch.cuda.synchronize()
    per_kernel = {}
    for name, ops, byts, a, b in evs:
        d = per_kernel.setdefault(name, {"time": 0.0, "ops": 0, "bytes": 0, "launches": 0})
        d["time"] += a.elapsed_time(b) * 1e-3
        d["ops"] += ops
        d["bytes"] += byts
        d["launches"] += 1
    dom_name, dom = max(per_kernel.items(), key=lambda kv: kv[1]["time"])
    ai = dom["ops"] / dom["bytes"]
    avg_t = dom["time"] / dom["launches"]
    if ai >= RIDGE:
        achieved = dom["ops"] / dom["launches"] / avg_t / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_I8 / 1e12, "unit": "TFLOP/s"}
    else:
        achieved = dom["bytes"] / dom["launches"] / avg_t / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = round(achieved / roof["peak"], 4)
    traffic = profiled_traffic(dom_name, args.workload)
    roof["traffic"] = None if traffic is None else round(traffic / avg_t / 1e9, 1)
    roof["traffic_unit"] = "GB/s of HBM bytes (counters) per launch time"
    roof["traffic_bytes_per_launch"] = traffic
    roof["kernel"] = dom_name
    roof["launches_per_step"] = dom["launches"] // reps * passes
    roof["avg_launch_us"] = round(avg_t * 1e6, 2)
    roof["work_per_launch"] = {"ops": dom["ops"] // dom["launches"], "bytes": dom["bytes"] // dom["launches"]}
    kernel_share = {k: round(v["time"] / reps * passes * 1e3, 3) for k, v in per_kernel.items()}

    line = {
        "metric": METRIC,
        "value": round(img_s, 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded SplitMix64, uniform int8 images/weights)",
        "config": config,
        "tops": round(tops, 2),
        "frac_int8_peak": round(tops * 1e12 / PEAK_I8, 4),
        "kernel_ms_per_step": kernel_share,
        "roofline": roof,
        **extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)
    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nb // 4,), dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
