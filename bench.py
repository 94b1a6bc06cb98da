"""Benchmark of the tile-sparse incremental conv hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--seed S] [--no-cpu]

One step is one incremental update of one layer for one edit, on the
U-Net-shaped workload (3x3 stride-1 conv, bf16 NHWC 1x256x256x128 -> 128,
6x6 output blocks, block-grid dilation 1, seeded 3-ellipse blob edit covering
1.2% of the pixels):
    sige_diff_mask_bits -> sige_reduce_bits_copy -> sige_sparse_conv_layer (copy_cached=0)
whose result is the spec-literal one (the cached output with the listed blocks
recomputed): the change mask is written one bit per pixel (the reduce's single
workgroup reads 8 KiB instead of 64 KiB), and the full copy of the cache into
the output runs on the idle workgroups of the single-workgroup reduce launch.  Every input is already
resident in device memory.  K steps run back to back
as replays of a HIP graph of 10 captured steps, between two HIP events;
`value` is the mean time per step in microseconds (lower is better).  The
latency of one step launched alone (one graph replay, and eager launches from
Python) is reported beside it.

Prints ONE JSON line on stdout.  Also reported: each kernel's mean duration
(HIP events around replays of a graph of 20 back-to-back launches of that call
alone), its algorithmic bytes / flops and its fraction of the MI355X peak; the
same step launched eagerly from Python; the three-call path; the copy-free
path; the dense conv on the same GPU (MIOpen through torch, and this library
with every block active); and the CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
METRIC = "sparse-conv layer latency & speedup vs dense at 1.2% edit; MFMA util, HBM GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU baseline sample length")
    ap.add_argument("--no-comparators", action="store_true",
                    help="time the step and its kernels only (for profiler runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: the block size and dilation sweep (a line per point, then a table)")
    ap.add_argument("--cold-kernels", type=int, default=0, metavar="R",
                    help="R rounds of every kernel of the step and of the three-call path, each launched after "
                         "512 MiB of writes, then R rounds each after 512 MiB of reads, that evict the MALL (for a "
                         "profiler's kernel trace and counters)")
    ap.add_argument("--attention", action="store_true",
                    help="instead of the step: only the query-pruned attention comparator (one JSON line)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU split of the block list is a design note, not built.", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        run_sweep(args)
        return
    if args.attention:
        run_attention(args)
        return

    import numpy as np
    import torch
    import torch.nn.functional as F

    import spatially_sparse_incremental_amd as ssi
    import synth
    from spatially_sparse_incremental_amd import comparators as cmp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = synth.workload("unet_256x256x128_bf16")
    L = wl.layers[0]
    dt = synth.DTYPES[L.dtype]
    es = torch.tensor([], dtype=dt).element_size()
    seed = args.seed
    shape = synth.edit_shape(wl, seed)
    mask_np = shape.raster(L.h, L.w)
    a_o_cpu = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
    a_e_cpu = synth.make_edit(a_o_cpu, mask_np, wl.edit_kind, seed)
    w_cpu, b_cpu = synth.make_layer_tensors(L, seed)

    a_o, a_e = a_o_cpu.to(dev), a_e_cpu.to(dev)
    w_krsc = ssi.weight_to_krsc(w_cpu).to(dev)
    bias = b_cpu.to(dev)
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    d = ssi.sige_geom_derive(g)
    cap = d.cap
    # the layer's weights packed once in the fused kernel's load order (a per-layer
    # preparation like the OIHW -> KRSC permute, outside every timing); the fused
    # layer calls below read them (sige_sparse_conv_layer_packed)
    w_packed = ssi.sige_pack_weights(w_krsc, g)

    # cache = conv(A_o), computed once (untimed) by the library with every block active
    idx_all = torch.arange(cap, dtype=torch.int32, device=dev)
    cnt_all = torch.tensor([cap], dtype=torch.int32, device=dev)
    cache = torch.empty((1, d.ho, d.wo, L.c_out), dtype=dt, device=dev)
    ssi.sige_sparse_conv_layer(a_o, w_krsc, bias, None, idx_all, cnt_all, g, out=cache, copy_cached=False,
                               w_packed=w_packed)

    mask = torch.empty((1, L.h, L.w), dtype=torch.uint8, device=dev)
    mbits = torch.empty((L.h * L.w // 32,), dtype=torch.int32, device=dev)  # the mask, one bit per pixel
    idx = torch.empty((cap,), dtype=torch.int32, device=dev)
    count = torch.empty((1,), dtype=torch.int32, device=dev)
    out = torch.empty_like(cache)

    def step(st=None):
        # out = cache outside the listed blocks (a full copy), conv inside: the copy
        # runs on the idle workgroups of the single-workgroup reduce
        ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits, stream=st)
        ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out, idx=idx, count=count, stream=st)
        ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx, count, g, out=out, copy_cached=False, stream=st,
                                   w_packed=w_packed)

    K, W = args.steps, args.warmup
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    active = int(count.item())
    edit_frac = float(mask_np.mean())

    ev, capture, graph_time = _timers(torch)

    # ---- timed region: K steps back to back, as replays of a graph of S steps
    S = 10
    K = max(S, K // S * S)
    gsteps = capture(step, S)
    cur = torch.cuda.current_stream()
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(cur)
    for _ in range(K // S):
        gsteps.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / K
    assert int(count.item()) == active
    print(f"[bench] step {step_ms * 1e3:.2f} us (graphs of {S} steps), {wall / K * 1e6:.2f} us wall, "
          f"active blocks {active}", file=sys.stderr, flush=True)

    # one step per graph replay (includes the graph launch)
    gstep = capture(step, 1)
    e0, e1 = ev(), ev()
    e0.record(cur)
    for _ in range(K):
        gstep.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    t_single = e0.elapsed_time(e1) / K * 1e3

    # spread: each replay of the 10-step graph timed alone (per-step mean of each)
    spread = []
    for _ in range(60):
        a, b = ev(), ev()
        a.record(cur)
        gsteps.replay()
        b.record(cur)
        b.synchronize()
        spread.append(a.elapsed_time(b) / S * 1e3)
    # cold: the 256 MB MALL (and the L2s) evicted by reading 512 MiB before every
    # step (outside the events; reads leave clean lines, so no write-back of the
    # eviction competes with the step); one step per replay, events around it
    evict = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(40):
        torch.amax(evict)
        a, b = ev(), ev()
        a.record(cur)
        gstep.replay()
        b.record(cur)
        b.synchronize()
        cold.append(a.elapsed_time(b) * 1e3)
    del evict

    def pct(v, q):
        v = sorted(v)
        return round(v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))], 3)

    distribution = {"warm_per_step_us": {"p10": pct(spread, 0.1), "p50": pct(spread, 0.5), "p90": pct(spread, 0.9),
                                         "replays": len(spread), "note": "each replay of a 10-step graph"},
                    "cold_step_us": {"p10": pct(cold, 0.1), "p50": pct(cold, 0.5), "p90": pct(cold, 0.9),
                                     "runs": len(cold),
                                     "note": "512 MiB read before each step to evict the MALL; one step "
                                             "per graph replay, HIP events around it (includes the graph launch)"}}

    # the same step launched eagerly from Python
    t_eager = None
    e0, e1 = ev(), ev()
    e0.record(cur)
    for _ in range(K):
        step()
    e1.record(cur)
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) / K * 1e3

    # ---- per-kernel durations: graphs of 20 back-to-back launches of one call
    kt = {  # the three calls of the step
        "diff": graph_time(lambda: ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)),
        "reduce_copy": graph_time(lambda: ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out,
                                                                    idx=idx, count=count)),
        "fused_layer": graph_time(lambda: ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx, count, g,
                                                                     out=out, copy_cached=False, w_packed=w_packed)),
    }
    # the three-call path's kernels on the same list (separate launches, block tensors in HBM)
    blocks = torch.empty((cap, d.ib, d.ib, L.c_in), dtype=dt, device=dev)
    oblocks = torch.empty((cap, L.block, L.block, L.c_out), dtype=dt, device=dev)
    out3 = torch.empty_like(cache)
    t_gather = graph_time(lambda: ssi.sige_gather(a_e, g, idx, count, blocks=blocks))
    t_convb = graph_time(lambda: ssi.sige_conv_blocks(blocks, w_krsc, bias, g, count, out_blocks=oblocks,
                                                      w_packed=w_packed))
    t_scatter = graph_time(lambda: ssi.sige_scatter(oblocks, idx, count, g, cache, out=out3, copy_cached=True))
    print(f"[bench] kernels {kt} gather {t_gather:.2f} conv_blocks {t_convb:.2f} scatter {t_scatter:.2f}",
          file=sys.stderr, flush=True)
    if args.cold_kernels:
        # each call alone on cold caches: 512 MiB written first, so its reads come from HBM
        calls = [lambda: ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits),
                 lambda: ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out, idx=idx,
                                                   count=count),
                 lambda: ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx, count, g, out=out,
                                                    copy_cached=False, w_packed=w_packed),
                 lambda: ssi.sige_gather(a_e, g, idx, count, blocks=blocks),
                 lambda: ssi.sige_conv_blocks(blocks, w_krsc, bias, g, count, out_blocks=oblocks,
                                              w_packed=w_packed),
                 lambda: ssi.sige_scatter(oblocks, idx, count, g, cache, out=out3, copy_cached=True)]
        evict = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
        for r in range(args.cold_kernels):  # evicted by writes: the MALL is left full of dirty lines
            for f in calls:
                evict.fill_(r & 0xFF)
                f()
        evict.zero_()
        for r in range(args.cold_kernels):  # evicted by reads: the MALL is left full of clean lines
            for f in calls:
                torch.amax(evict)
                f()
        torch.cuda.synchronize()
        del evict
        print(f"[bench] cold kernels: {args.cold_kernels} rounds of {len(calls)} calls, after writes and after "
              "reads of 512 MiB", file=sys.stderr, flush=True)

    t_nocopy = t_three = t_fused_copy = t_dense_ours = t_dense_miopen = None
    t_reduce = t_step_conv_copy = t_step_bytes = t_reduce_bytes = None
    t_seq = t_seq2 = t_restore = t_bbox = t_bbox_tiles = attention = ldm_split = t_layer = None
    chain = gaugan = None
    bbox_flops = bbox_blocks = rect = None
    if not args.no_comparators:
        # the step with the copy inside the conv launch instead of the reduce launch
        out_c = torch.empty_like(cache)

        def step_conv_copy():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            ssi.sige_reduce_bits(mbits, L.h, L.w, g, L.dilate, idx=idx, count=count)
            ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, cache, idx, count, g, out=out_c, copy_cached=True,
                                       w_packed=w_packed)

        t_step_conv_copy = graph_time(step_conv_copy, 5, 40)

        def layer_only():  # the per-layer part of the step: reduce (with the copy) and the fused layer
            ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out, idx=idx, count=count)
            ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx, count, g, out=out, copy_cached=False,
                                       w_packed=w_packed)

        t_layer = graph_time(layer_only, 5, 40)
        t_reduce = graph_time(lambda: ssi.sige_reduce_bits(mbits, L.h, L.w, g, L.dilate, idx=idx, count=count))

        def step_bytes():  # the step with the change mask as bytes
            ssi.sige_diff_mask(a_o, a_e, wl.tau, mask=mask)
            ssi.sige_reduce_mask_copy(mask, g, L.dilate, cache, out=out, idx=idx, count=count)
            ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx, count, g, out=out, copy_cached=False,
                                       w_packed=w_packed)

        t_step_bytes = graph_time(step_bytes, 5, 40)
        t_reduce_bytes = graph_time(lambda: ssi.sige_reduce_mask(mask, g, L.dilate, idx=idx, count=count))
        t_fused_copy = graph_time(lambda: ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, cache, idx, count, g,
                                                                     out=out_c, copy_cached=True, w_packed=w_packed))

        # the step without the cache copy (persistent output buffer)
        out_persist = cache.clone()

        def step_nocopy():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            ssi.sige_reduce_bits(mbits, L.h, L.w, g, L.dilate, idx=idx, count=count)
            ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx, count, g, out=out_persist, copy_cached=False,
                                       w_packed=w_packed)

        # the three-call path
        def step_three():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            ssi.sige_reduce_bits(mbits, L.h, L.w, g, L.dilate, idx=idx, count=count)
            ssi.sige_gather(a_e, g, idx, count, blocks=blocks)
            ssi.sige_conv_blocks(blocks, w_krsc, bias, g, count, out_blocks=oblocks, w_packed=w_packed)
            ssi.sige_scatter(oblocks, idx, count, g, cache, out=out3, copy_cached=True)

        t_nocopy = graph_time(step_nocopy, 5, 40)
        t_three = graph_time(step_three, 5, 40)
        # dense comparators on the same GPU
        dense_all = torch.empty_like(cache)
        t_dense_ours = graph_time(lambda: ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, None, idx_all, cnt_all, g,
                                                                     out=dense_all, copy_cached=False,
                                                                     w_packed=w_packed), 5, 10)

        def timed_eager(fn, reps):
            for _ in range(min(10, reps)):
                fn()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record(cur)
            for _ in range(reps):
                fn()
            b.record(cur)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps * 1e3  # us

        t_dense_miopen = None
        try:
            x_cl = a_e.permute(0, 3, 1, 2)  # NCHW view with channels_last strides
            w_cl = w_cpu.to(dev).contiguous(memory_format=torch.channels_last)
            with torch.no_grad():
                t_dense_miopen = timed_eager(lambda: F.conv2d(x_cl, w_cl, bias.to(dt), padding=L.pad), max(20, K // 5))
        except Exception as exc:  # noqa: BLE001 - report, do not hide
            print(f"[bench] MIOpen dense conv failed: {exc}", file=sys.stderr)

        # sequential edits: two blob edits alternate through one persistent
        # buffer; each step restores the previous edit's blocks that the new
        # edit does not list, instead of copying the whole cache
        a_e2 = synth.make_edit(a_o_cpu, synth.edit_shape(wl, seed + 1).raster(L.h, L.w), wl.edit_kind,
                               seed + 1).to(dev)
        seq_edits = [a_e, a_e2]
        seq_idx = [torch.empty((cap,), dtype=torch.int32, device=dev) for _ in range(2)]
        seq_cnt = [torch.zeros((1,), dtype=torch.int32, device=dev) for _ in range(2)]
        seq_out = cache.clone()
        seq_bits = torch.empty_like(mbits)

        def seq_step(k, one_call):
            cur, prv = k % 2, (k + 1) % 2
            ssi.sige_diff_mask_bits(a_o, seq_edits[cur], wl.tau, bits=seq_bits)
            ssi.sige_reduce_bits(seq_bits, L.h, L.w, g, L.dilate, idx=seq_idx[cur], count=seq_cnt[cur])
            if one_call:  # restore and conv in one launch
                ssi.sige_sparse_conv_layer_restore(seq_edits[cur], w_krsc, bias, cache, seq_idx[prv], seq_cnt[prv],
                                                   seq_idx[cur], seq_cnt[cur], g, seq_out)
            else:
                ssi.sige_restore_blocks(seq_idx[prv], seq_cnt[prv], seq_idx[cur], seq_cnt[cur], g, cache, seq_out)
                ssi.sige_sparse_conv_layer(seq_edits[cur], w_krsc, bias, None, seq_idx[cur], seq_cnt[cur], g,
                                           out=seq_out, copy_cached=False)  # KRSC, as the one-launch restore

        # both edits per call, so that graph replays keep the alternation
        t_seq = graph_time(lambda: (seq_step(0, True), seq_step(1, True)), 5, 40) / 2
        t_seq2 = graph_time(lambda: (seq_step(0, False), seq_step(1, False)), 5, 40) / 2
        t_restore = graph_time(lambda: ssi.sige_restore_blocks(seq_idx[1], seq_cnt[1], seq_idx[0], seq_cnt[0], g,
                                                               cache, seq_out))

        # the bounding-box crop that the pages set aside: a dense conv (torch,
        # i.e. MIOpen) of the output rectangle the edit's bounding box reaches,
        # written into a copy of the cache; and the same rectangle as a block
        # list through this library.  The box is found once, outside the timing.
        rect = cmp.bbox_out_rect(cmp.edit_bbox(mask), L.h, L.w, L.k, L.stride, L.pad)
        bbox_rows, bbox_cols = rect[1] - rect[0] + 1, rect[3] - rect[2] + 1
        bbox_flops = 2 * bbox_rows * bbox_cols * L.c_out * L.c_in * L.k * L.k
        bbox_out = torch.empty_like(cache)
        w_cl2 = w_cpu.to(dev).contiguous(memory_format=torch.channels_last)

        def step_bbox():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            bbox_out.copy_(cache)
            cmp.bbox_crop_conv(a_e, w_cl2, bias, cache, rect, L.k, L.stride, L.pad, out=bbox_out)

        try:
            with torch.no_grad():
                t_bbox = timed_eager(step_bbox, max(20, K // 5))
        except Exception as exc:  # noqa: BLE001 - report, do not hide
            print(f"[bench] bounding-box comparator failed: {exc}", file=sys.stderr)
        bbox_idx, bbox_cnt = cmp.bbox_block_list(rect, L.block, d.nby, d.nbx, device=dev)
        bbox_blocks = int(bbox_cnt.item())

        def step_bbox_tiles():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            ssi.sige_sparse_conv_layer(a_e, w_krsc, bias, cache, bbox_idx, bbox_cnt, g, out=bbox_out,
                                       copy_cached=True, w_packed=w_packed)

        t_bbox_tiles = graph_time(step_bbox_tiles, 5, 40)

        attention = _attention_comparator(torch, F, ssi, synth, graph_time, timed_eager, seed)
        ldm_split = _ldm_split_comparator(torch, F, ssi, synth, graph_time, timed_eager, seed)
        try:
            chain = _chain_comparator(torch, F, ssi, synth, graph_time, seed)
        except Exception as exc:  # noqa: BLE001 - report, do not hide
            print(f"[bench] chain comparator failed: {exc}", file=sys.stderr)
        try:
            gaugan = _gaugan_comparator(torch, F, ssi, synth, graph_time, timed_eager, seed)
        except Exception as exc:  # noqa: BLE001 - report, do not hide
            print(f"[bench] GauGAN comparator failed: {exc}", file=sys.stderr)

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # ---- algorithmic work: flops and bytes per listed block, per layer and per edit
    npix_in, npix_out = L.h * L.w, d.ho * d.wo
    b2 = L.block * L.block
    act_pix = int(_active_pixels(idx[:active].cpu().numpy(), d, L.block))
    w_bytes = L.c_out * L.k * L.k * L.c_in * es
    diff_bytes = 2 * npix_in * L.c_in * es + npix_in // 8    # the mask written one bit per pixel
    reduce_bytes = npix_in // 8 + 4 * active + 4
    blk_bytes = active * (d.ib * d.ib * L.c_in * es + b2 * L.c_out * es)
    copy_bytes = 2 * (npix_out - act_pix) * L.c_out * es
    conv_flops = 2.0 * active * b2 * L.c_in * L.c_out * L.k * L.k
    dense_flops = 2.0 * npix_out * L.c_in * L.c_out * L.k * L.k
    peak_tf = PEAK_MFMA_TFLOPS[L.dtype]

    def hbm(nbytes, us):
        # warm: every tensor of this workload is resident in the 256 MB MALL, so this rate is not
        # an HBM rate (HBM fractions come from the cold pass below)
        gbps = nbytes / (us * 1e-6) / 1e9
        return dict(us=round(us, 3), bytes=int(nbytes), gbps_warm_mall=round(gbps, 1))

    conv_bytes = blk_bytes + w_bytes + 4 * L.c_out             # the conv without the copy
    full_copy_bytes = 2 * npix_out * L.c_out * es               # out = cache, every pixel
    reduce_copy_bytes = reduce_bytes + full_copy_bytes

    def mfma(us):
        tf = conv_flops / (us * 1e-6) / 1e12
        return dict(flops=int(conv_flops), tflops=round(tf, 2), frac_mfma=round(tf / peak_tf, 5))

    kernels = {  # the step's three launches
        "diff": hbm(diff_bytes, kt["diff"]),
        "reduce_copy": dict(hbm(reduce_copy_bytes, kt["reduce_copy"]), note="reduce on one workgroup, the full "
                            "cache copy on the others"),
        "fused_layer": dict(hbm(conv_bytes, kt["fused_layer"]), **mfma(kt["fused_layer"])),
        "gather": hbm(active * d.ib * d.ib * L.c_in * es * 2, t_gather),
        "conv_blocks": dict(hbm(blk_bytes + w_bytes, t_convb), **mfma(t_convb)),
        "scatter": hbm(active * b2 * L.c_out * es + act_pix * L.c_out * es + copy_bytes, t_scatter),
    }
    if not args.no_comparators:
        kernels.update({
            "reduce": dict(us=round(t_reduce, 3), bytes=int(reduce_bytes), bound="latency"),
            "fused_layer_with_copy": dict(hbm(conv_bytes + copy_bytes, t_fused_copy), **mfma(t_fused_copy)),
        })
    # HBM bytes per launch read from the rocprofv3 counters (FETCH_SIZE and WRITE_SIZE,
    # calibrated on a plain copy), while the sources they were taken on are unchanged
    for name, tb in _measured_kernel_traffic().items():
        if name in kernels:
            us = kernels[name]["us"]
            kernels[name]["traffic_bytes"] = tb
            kernels[name]["traffic_gbps_warm_mall"] = round(tb / (us * 1e-6) / 1e9, 1)
    # HBM rates per kernel with the MALL evicted first (the committed cold-cache summary,
    # while the sources it was taken on are unchanged)
    for name, cold in _measured_cold_kernels().items():
        if name in kernels:
            kernels[name]["cold"] = dict(cold, frac_hbm=round(cold["gbps"] / PEAK_HBM_GBPS, 4))
    # the whole step against its roofline: t_roof = max(flops / MFMA peak, bytes / HBM peak)
    # over the algorithmic work of the three launches, without and with the spec-literal copy
    step_bytes = diff_bytes + reduce_bytes + conv_bytes

    def step_roof(nbytes):
        t_roof = max(conv_flops / (peak_tf * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9)) * 1e6
        return dict(bytes=int(nbytes), flops=int(conv_flops), t_roof_us=round(t_roof, 3),
                    frac=round(t_roof / (step_ms * 1e3), 4))

    step_roofline = {"t_measured_us": round(step_ms * 1e3, 3), "no_copy": step_roof(step_bytes),
                     "with_copy": step_roof(step_bytes + full_copy_bytes),
                     "note": "bytes: diff reads both activations and writes the packed mask, the reduce reads the "
                             "mask, the layer reads the listed windows, the weights and bias and writes the listed "
                             "blocks; with_copy adds reading and writing the whole cache"}
    # the roofline of the step's longest launch: the conv against the MFMA peak (it
    # is the contraction), the others against HBM
    dom = max(kt, key=lambda k: kt[k])
    if dom == "fused_layer":
        tf = conv_flops / (kt[dom] * 1e-6) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(tf, 2), "peak": peak_tf, "unit": "TFLOP/s",
                    "frac": round(tf / peak_tf, 4), "traffic": _measured_kernel_traffic().get("fused_layer")}
    else:
        droof = kernels[dom]
        roofline = {"kernel": dom, "bound": "hbm", "achieved": droof["gbps_warm_mall"], "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(droof["gbps_warm_mall"] / PEAK_HBM_GBPS, 4), "traffic": None}

    cpu = None
    if not args.no_cpu:
        cpu = _cpu_baseline(a_o_cpu, a_e_cpu, w_cpu, b_cpu, cache.cpu(), L, wl.tau, args.cpu_seconds)

    step_us = step_ms * 1e3
    res = {
        "metric": METRIC,
        "value": round(step_us, 3),
        "unit": "us per incremental layer update (diff + reduce with the cache copy + fused sparse conv)",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(step_ms, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": L.dtype,
        "data": "synthetic: seeded 3-ellipse blob edit, N(0,1) activations, He-normal weights (packed once per "
                "layer in the fused kernel's load order by sige_pack_weights, outside the timed region)",
        "config": {"workload": "unet_256x256x128_bf16_3x3s1_b6_d1_blob1.2pct", "n": 1, "h": L.h, "w": L.w,
                   "c_in": L.c_in, "c_out": L.c_out, "k": L.k, "stride": L.stride, "block": L.block,
                   "dilate": L.dilate, "seed": seed, "edit_fraction": round(edit_frac, 5),
                   "active_blocks": active, "block_capacity": cap},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "cpu_baseline": cpu,
        "distribution": distribution,
        "kernels": kernels,
        "comparators": None if args.no_comparators else {
            "dense_conv_miopen_us": None if t_dense_miopen is None else round(t_dense_miopen, 3),
            "dense_conv_ours_all_blocks_us": round(t_dense_ours, 3),
            "speedup_vs_dense_miopen": None if t_dense_miopen is None else round(t_dense_miopen / step_us, 3),
            "speedup_vs_dense_ours": round(t_dense_ours / step_us, 3),
            "speedup_vs_best_dense": round(min(t for t in (t_dense_miopen, t_dense_ours) if t is not None) / step_us,
                                           3),
            "dense_ours_tflops": round(dense_flops / (t_dense_ours * 1e-6) / 1e12, 1),
            "step_no_copy_us": round(t_nocopy, 3),
            "step_byte_mask_us": round(t_step_bytes, 3),
            "reduce_byte_mask_us": round(t_reduce_bytes, 3),
            "step_copy_in_conv_us": round(t_step_conv_copy, 3),
            "step_three_call_us": round(t_three, 3),
            "step_sequential_edits_us": round(t_seq, 3),
            "step_sequential_edits_two_calls_us": round(t_seq2, 3),
            "restore_blocks_us": round(t_restore, 3),
            "bbox_crop_dense_step_us": None if t_bbox is None else round(t_bbox, 3),
            "bbox_tiles_step_us": round(t_bbox_tiles, 3),
            "bbox_output_rect": list(rect),
            "bbox_blocks": bbox_blocks,
            "bbox_mac_reduction": round(dense_flops / bbox_flops, 2),
            "attention_ldm_64x64x5x64_f16": attention,
            "ldm_16x16x1280_f16_split": ldm_split,
            "layer_reduce_and_fused_us": round(t_layer, 3),
            "speedup_layer_vs_dense_miopen": None if t_dense_miopen is None else round(t_dense_miopen / t_layer, 3),
            "chain_unet_12conv_bf16": chain,
            "gaugan_convs_bf16": gaugan,
            "speedup_no_copy_vs_dense_miopen": None if t_dense_miopen is None else round(t_dense_miopen / t_nocopy, 3),
        },
        "latency": {
            "step_eager_launch_us": round(t_eager, 3),
            "step_single_graph_replay_us": round(t_single, 3),
            "step_wall_us": round(wall / K * 1e6, 3),
        },
        "mac_reduction": round(dense_flops / conv_flops, 2) if conv_flops else None,
    }
    print(json.dumps(res), flush=True)


def _timers(torch):
    """HIP-event timing helpers: ev(), capture(fn, n_in) -> graph, graph_time(fn, n_in, replays) -> us."""
    def ev():
        return torch.cuda.Event(enable_timing=True)

    def capture(fn, n_in):
        """A HIP graph of n_in back-to-back calls of fn (launches only; no memsets inside)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(n_in):
                fn()
        gr.replay()
        torch.cuda.synchronize()
        return gr

    def graph_time(fn, n_in=20, replays=25):
        """Mean duration of one fn call: events around `replays` replays of a graph of n_in calls."""
        gr = capture(fn, n_in)
        cur = torch.cuda.current_stream()
        e0, e1 = ev(), ev()
        e0.record(cur)
        for _ in range(replays):
            gr.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n_in * replays) * 1e3  # us

    return ev, capture, graph_time


def run_attention(args):
    """Only the query-pruned attention comparator, as one JSON line (for profiler runs)."""
    import torch
    import torch.nn.functional as F

    import spatially_sparse_incremental_amd as ssi
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    ev, _, graph_time = _timers(torch)

    def timed_eager(fn, reps):
        for _ in range(min(10, reps)):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        cur = torch.cuda.current_stream()
        a.record(cur)
        for _ in range(reps):
            fn()
        b.record(cur)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3  # us

    res = _attention_comparator(torch, F, ssi, synth, graph_time, timed_eager, args.seed)
    print(json.dumps({"attention_ldm_64x64x5x64_f16": res}), flush=True)


def run_sweep(args):
    """Block size and dilation sweep (one JSON line per point, then a markdown
    table): blocks listed, MAC reduction, reduce and fused-layer times with and
    without the cache copy, the same for the layer split over input channels,
    the library's choice between the two (sige_sparse_conv_layer_auto), and the
    dense conv (torch/MIOpen) of the layer."""
    import torch
    import torch.nn.functional as F

    import spatially_sparse_incremental_amd as ssi
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ev, capture, graph_time = _timers(torch)
    rows, dense_t = [], {}
    for wname, L in synth.SWEEP:
        wl = synth.workload(wname)
        seed = args.seed
        m = synth.edit_shape(wl, seed).raster(L.h, L.w)
        a_o_cpu = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
        a_o = a_o_cpu.to(dev)
        a_e = synth.make_edit(a_o_cpu, m, wl.edit_kind, seed).to(dev)
        w_cpu, b_cpu = synth.make_layer_tensors(L, seed)
        wk, bias = ssi.weight_to_krsc(w_cpu).to(dev), b_cpu.to(dev)
        g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
        d = ssi.sige_geom_derive(g)
        cache = synth.make_activation(1, d.ho, d.wo, L.c_out, L.dtype, seed + 50).to(dev)
        out, persist = torch.empty_like(cache), cache.clone()
        mask = ssi.sige_diff_mask(a_o, a_e, wl.tau)
        idx, cnt = ssi.sige_reduce_mask(mask, g, L.dilate)
        torch.cuda.synchronize()
        blocks = int(cnt.item())
        t_red = graph_time(lambda: ssi.sige_reduce_mask(mask, g, L.dilate, idx=idx, count=cnt))
        t_copy = graph_time(lambda: ssi.sige_sparse_conv_layer(a_e, wk, bias, cache, idx, cnt, g, out=out))
        t_nocopy = graph_time(lambda: ssi.sige_sparse_conv_layer(a_e, wk, bias, None, idx, cnt, g, out=persist,
                                                                 copy_cached=False))
        ws = torch.empty(ssi.sige_sparse_conv_layer_split_workspace(g, a_e.dtype), dtype=torch.uint8, device=dev)
        t_split_copy = graph_time(lambda: ssi.sige_sparse_conv_layer_split(a_e, wk, bias, cache, idx, cnt, g, out=out,
                                                                           workspace=ws))
        t_split_nocopy = graph_time(lambda: ssi.sige_sparse_conv_layer_split(a_e, wk, bias, None, idx, cnt, g,
                                                                             out=persist, copy_cached=False,
                                                                             workspace=ws))
        plan = ssi.sige_sparse_conv_layer_plan(g, a_e.dtype)
        ws_auto = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
        t_auto_nocopy = graph_time(lambda: ssi.sige_sparse_conv_layer_auto(a_e, wk, bias, None, idx, cnt, g,
                                                                           out=persist, copy_cached=False,
                                                                           workspace=ws_auto))
        key = (wname, L.h, L.c_in)
        if key not in dense_t:
            x_cl = a_e.permute(0, 3, 1, 2)
            w_cl = w_cpu.to(dev).contiguous(memory_format=torch.channels_last)
            with torch.no_grad():
                for _ in range(10):
                    F.conv2d(x_cl, w_cl, bias.to(a_e.dtype), padding=L.pad)
                torch.cuda.synchronize()
                e0, e1 = ev(), ev()
                e0.record()
                for _ in range(50):
                    F.conv2d(x_cl, w_cl, bias.to(a_e.dtype), padding=L.pad)
                e1.record()
                torch.cuda.synchronize()
            dense_t[key] = e0.elapsed_time(e1) / 50 * 1e3
        act_pix = _active_pixels(idx[:blocks].cpu().numpy(), d, L.block)
        row = {"layer": L.name, "h": L.h, "w": L.w, "c_in": L.c_in, "c_out": L.c_out, "dtype": L.dtype,
               "block": L.block, "dilate": L.dilate, "blocks": blocks, "capacity": d.cap,
               "edit_fraction": round(float(m.mean()), 5),
               "mac_reduction": round(d.ho * d.wo / act_pix, 2) if act_pix else None,
               "reduce_us": round(t_red, 3), "fused_copy_us": round(t_copy, 3),
               "fused_nocopy_us": round(t_nocopy, 3), "split_copy_us": round(t_split_copy, 3),
               "split_nocopy_us": round(t_split_nocopy, 3), "auto_nocopy_us": round(t_auto_nocopy, 3),
               "auto_path": _auto_path(plan, blocks),
               "dense_miopen_us": round(dense_t[key], 3),
               "speedup_auto_nocopy_vs_dense": round(dense_t[key] / t_auto_nocopy, 2)}
        rows.append(row)
        print(json.dumps(row), flush=True)
    cols = ["layer", "block", "dilate", "blocks", "capacity", "mac_reduction", "reduce_us", "fused_copy_us",
            "fused_nocopy_us", "split_copy_us", "split_nocopy_us", "auto_nocopy_us", "auto_path", "dense_miopen_us",
            "speedup_auto_nocopy_vs_dense"]
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for r in rows:
        print("| " + " | ".join(str(r[c]) for c in cols) + " |")


def _attention_comparator(torch, F, ssi, synth, graph_time, timed_eager, seed):
    """Query-pruned self-attention at the latent-diffusion shape (64x64 tokens,
    5 heads of 64, fp16): query blocks of 4x4 tokens from a blob edit's diff
    (k = 1 geometry, dilation 1) at 1.2% and 10% of the frame, against dense
    attention over all 4096 queries (torch scaled_dot_product_attention)."""
    dev = torch.device("cuda:0")
    wl = synth.workload("ldm_64x64x320_f16")
    h = w = 64
    heads, d, b = 5, 64, 4
    g = ssi.geom(1, h, w, heads * d, heads * d, 1, 1, 0, b)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q, k, v = ((torch.randn((1, h, w, heads * d), generator=gen) * 0.5).to(torch.float16).to(dev) for _ in range(3))
    cache = torch.randn((1, h, w, heads * d), generator=gen).to(torch.float16).to(dev)
    out = torch.empty_like(cache)
    ws = torch.empty(ssi.sige_sparse_attention_workspace(1, h, w, heads, d, b), dtype=torch.uint8, device=dev)
    x_o = synth.make_activation(1, h, w, 320, "f16", seed).to(dev)
    res = {}
    for area in (0.012, 0.10):
        m = synth.edit_shape(wl, seed, area).raster(h, w)
        x_e = synth.make_edit(x_o.cpu(), m, "replace", seed).to(dev)
        mask = ssi.sige_diff_mask(x_o, x_e, wl.tau)
        idx, cnt = ssi.sige_reduce_mask(mask, g, 1)
        torch.cuda.synchronize()
        blocks = int(cnt.item())
        t = graph_time(lambda: ssi.sige_sparse_attention(q, k, v, idx, cnt, heads, b, cached=cache, out=out,
                                                         workspace=ws))
        t_nocopy = graph_time(lambda: ssi.sige_sparse_attention(q, k, v, idx, cnt, heads, b, out=out,
                                                                copy_cached=False, workspace=ws))
        flops = 4.0 * blocks * b * b * heads * d * h * w
        key = f"area_{area:g}"
        res[key] = {"query_blocks": blocks, "sparse_us": round(t, 3), "sparse_nocopy_us": round(t_nocopy, 3),
                    "tflops_nocopy": round(flops / (t_nocopy * 1e-6) / 1e12, 2)}
    qh, kh, vh = (x.reshape(1, h * w, heads, d).transpose(1, 2).contiguous() for x in (q, k, v))
    try:
        with torch.no_grad():
            t_dense = timed_eager(lambda: F.scaled_dot_product_attention(qh, kh, vh), 50)
        res["dense_sdpa_us"] = round(t_dense, 3)
        res["dense_tflops"] = round(4.0 * h * w * heads * d * h * w / (t_dense * 1e-6) / 1e12, 2)
    except Exception as exc:  # noqa: BLE001 - report, do not hide
        print(f"[bench] dense attention failed: {exc}", file=sys.stderr)
    return res


def _ldm_split_comparator(torch, F, ssi, synth, graph_time, timed_eager, seed):
    """The latent-diffusion 16x16x1280 fp16 3x3 layer (b = 2, dilation 1) with the
    blob edit: the library's choice (sige_sparse_conv_layer_auto) and the
    single-range fused layer on the packed weights, the layer split over input
    channels (KRSC weights, its own entry point) and the dense conv
    (torch/MIOpen), each with the cache copy."""
    dev = torch.device("cuda:0")
    wl = synth.workload("ldm_64x64x320_f16")
    L = [x for x in wl.layers if x.name == "l16_3x3"][0]
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
    a_e = synth.make_edit(a_o, synth.edit_shape(wl, seed).raster(L.h, L.w), wl.edit_kind, seed).to(dev)
    a_o = a_o.to(dev)
    w_cpu, b_cpu = synth.make_layer_tensors(L, seed)
    wk, bias = ssi.weight_to_krsc(w_cpu).to(dev), b_cpu.to(dev)
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + 50).to(dev)
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    idx, cnt = ssi.sige_reduce_mask(ssi.sige_diff_mask(a_o, a_e, wl.tau), g, L.dilate)
    out = torch.empty_like(cache)
    ws = torch.empty(ssi.sige_sparse_conv_layer_split_workspace(g, a_e.dtype), dtype=torch.uint8, device=dev)
    wpk = ssi.sige_pack_weights(wk, g)  # packed once, outside the timing
    t_plain = graph_time(lambda: ssi.sige_sparse_conv_layer(a_e, wk, bias, cache, idx, cnt, g, out=out, w_packed=wpk))
    t_split = graph_time(lambda: ssi.sige_sparse_conv_layer_split(a_e, wk, bias, cache, idx, cnt, g, out=out,
                                                                  workspace=ws))
    plan = ssi.sige_sparse_conv_layer_plan(g, a_e.dtype)
    ws_auto = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    t_auto = graph_time(lambda: ssi.sige_sparse_conv_layer_auto(a_e, wk, bias, cache, idx, cnt, g, out=out,
                                                                workspace=ws_auto, w_packed=wpk))
    res = {"blocks": int(cnt.item()), "auto_us": round(t_auto, 3),
           "auto_path": _auto_path(plan, int(cnt.item())), "split_max": plan.split_max,
           "single_range_us": round(t_plain, 3), "split_us": round(t_split, 3)}
    try:
        x_cl = a_e.permute(0, 3, 1, 2)
        w_cl = w_cpu.to(dev).contiguous(memory_format=torch.channels_last)
        with torch.no_grad():
            t_dense = timed_eager(lambda: F.conv2d(x_cl, w_cl, bias.to(a_e.dtype), padding=L.pad), 50)
        res["dense_miopen_us"] = round(t_dense, 3)
        res["speedup_auto_vs_dense"] = round(t_dense / t_auto, 2)
        res["speedup_split_vs_dense"] = round(t_dense / t_split, 2)
    except Exception as exc:  # noqa: BLE001 - report, do not hide
        print(f"[bench] dense 16x16x1280 conv failed: {exc}", file=sys.stderr)
    return res


def _chain_comparator(torch, F, ssi, synth, graph_time, seed):
    """The 12-conv U-Net chain (256 to 32 pixels, 128 to 512 channels) at the 1.2% blob edit, as HIP graphs: one
    diff at 256x256 (the mask one bit per pixel), then per layer the reduce of
    the mask pooled to the layer's input with the cache copy on its idle
    workgroups, and the fused layer, layer l+1 reading layer l's output;
    against the same 12 convs dense through torch/MIOpen."""
    dev = torch.device("cuda:0")
    wl = synth.workload("unet_chain_12conv_bf16")
    first = wl.layers[0]
    m = synth.edit_shape(wl, seed).raster(first.h, first.w)
    a_o = synth.make_activation(1, first.h, first.w, first.c_in, first.dtype, seed).to(dev)
    a_e = synth.make_edit(a_o.cpu(), m, wl.edit_kind, seed).to(dev)
    mbits = torch.empty((first.h * first.w // 32,), dtype=torch.int32, device=dev)
    layers = []
    x_dense = [a_e.permute(0, 3, 1, 2)]
    for li, L in enumerate(wl.layers):
        w_cpu, b_cpu = synth.make_layer_tensors(L, seed * 100 + li)
        g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
        d = ssi.sige_geom_derive(g)
        cache = synth.make_activation(1, d.ho, d.wo, L.c_out, L.dtype, seed * 100 + li + 50).to(dev)
        layers.append(dict(L=L, g=g, wk=ssi.weight_to_krsc(w_cpu).to(dev), bias=b_cpu.to(dev), cache=cache,
                           out=torch.empty_like(cache), idx=torch.empty((d.cap,), dtype=torch.int32, device=dev),
                           cnt=torch.empty((1,), dtype=torch.int32, device=dev),
                           w_cl=w_cpu.to(dev).contiguous(memory_format=torch.channels_last),
                           b16=b_cpu.to(dev).to(a_e.dtype), mbits=mbits))
        ly = layers[-1]
        ly["wp"] = ssi.sige_pack_weights(ly["wk"], g)
    blocks = []

    def sparse_chain():
        ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
        x = a_e
        for ly in layers:
            ssi.sige_reduce_bits_copy(mbits, first.h, first.w, ly["g"], ly["L"].dilate, ly["cache"], out=ly["out"],
                                      idx=ly["idx"], count=ly["cnt"])
            ssi.sige_sparse_conv_layer(x, ly["wk"], ly["bias"], None, ly["idx"], ly["cnt"], ly["g"], out=ly["out"],
                                       copy_cached=False)
            x = ly["out"]

    def dense_chain():
        x = x_dense[0]
        for ly in layers:
            x = F.conv2d(x, ly["w_cl"], ly["b16"], stride=ly["L"].stride, padding=ly["L"].pad)

    sparse_chain()
    torch.cuda.synchronize()
    blocks = [int(ly["cnt"].item()) for ly in layers]
    t_single = graph_time(sparse_chain, 2, 25)
    xs = [a_e] + [ly["out"] for ly in layers[:-1]]
    for ly, x in zip(layers, xs):
        plan = ssi.sige_sparse_conv_layer_plan(ly["g"], a_e.dtype)
        ly["ws"] = torch.empty(max(ssi.sige_sparse_conv_layer_split_workspace(ly["g"], a_e.dtype),
                                   plan.workspace_bytes), dtype=torch.uint8, device=dev)
        ly["auto_path"] = _auto_path(plan, int(ly["cnt"].item()))
        # the bound: per layer, the faster of the two kernels timed on this very edit
        ly["mode"] = "single"
        t1 = graph_time(lambda: _chain_layer(ssi, ly, x, first), 5, 20)
        ly["mode"] = "split"
        t2 = graph_time(lambda: _chain_layer(ssi, ly, x, first), 5, 20)
        ly["best"] = "split" if t2 < t1 else "single"

    def chain_with(mode):
        for ly in layers:
            ly["mode"] = ly["best"] if mode == "best" else mode

        def run():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            x = a_e
            for ly in layers:
                _chain_layer(ssi, ly, x, first)
                x = ly["out"]
        return run

    t_per_layer = graph_time(chain_with("auto"), 2, 25)
    # every layer's list depends on the one mask only: all twelve lists and cache
    # copies in one launch, then the twelve layers
    geoms, dils = [ly["g"] for ly in layers], [ly["L"].dilate for ly in layers]
    idxs, cnts = [ly["idx"] for ly in layers], [ly["cnt"] for ly in layers]
    caches, outs = [ly["cache"] for ly in layers], [ly["out"] for ly in layers]

    def batched_with(mode):
        def run():
            ssi.sige_diff_mask_bits(a_o, a_e, wl.tau, bits=mbits)
            ssi.sige_reduce_bits_layers(mbits, first.h, first.w, geoms, dils, idxs, cnts, caches, outs)
            x = a_e
            for ly in layers:
                ly["mode"] = ly["best"] if mode == "best" else mode
                _chain_conv(ssi, ly, x)
                x = ly["out"]
        return run

    t_sparse = graph_time(batched_with("auto"), 2, 25)
    t_best = graph_time(batched_with("best"), 2, 25)
    with torch.no_grad():
        t_dense = graph_time(dense_chain, 1, 10)
    return {"sparse_us": round(t_sparse, 3), "dense_miopen_us": round(t_dense, 3),
            "speedup": round(t_dense / t_sparse, 2), "blocks_per_layer": blocks,
            "path_per_layer": [ly["auto_path"] for ly in layers],
            "best_of_two_bound_us": round(t_best, 3),
            "best_of_two_path_per_layer": [ly["best"] for ly in layers],
            "sparse_per_layer_reduce_us": round(t_per_layer, 3),
            "sparse_single_range_only_us": round(t_single, 3),
            "note": "one diff + one launch building all 12 lists with the 12 cache copies + 12 layers through "
                    "sige_sparse_conv_layer_auto (the kernel the library picks from the list length; "
                    "path_per_layer is its choice: split, single (64 x 32 tiles) or wide (256 x 128 tiles)); "
                    "best_of_two_bound: the faster of the single-range and split kernels per layer (the two with "
                    "entry points of their own), timed on this edit (not available to a caller); "
                    "per_layer_reduce: a reduce with its copy "
                    "before each layer; dense: 12 x F.conv2d; HIP graphs"}


def _auto_path(plan, n):
    """The kernel sige_sparse_conv_layer_auto runs for a list of n blocks."""
    if n <= plan.split_max:
        return "split"
    return "wide" if plan.wide_min <= n <= plan.wide_max else "single"


def _chain_layer(ssi, ly, x, first):
    """One layer of the chain: the reduce with the cache copy, then the layer."""
    mbits = ly["mbits"]
    ssi.sige_reduce_bits_copy(mbits, first.h, first.w, ly["g"], ly["L"].dilate, ly["cache"], out=ly["out"],
                              idx=ly["idx"], count=ly["cnt"])
    _chain_conv(ssi, ly, x)


def _chain_conv(ssi, ly, x):
    """The layer of the chain on its list, into its output (which holds the cache
    copy), by ly["mode"]: the library's choice, or one kernel."""
    if ly["mode"] == "auto":
        ssi.sige_sparse_conv_layer_auto(x, ly["wk"], ly["bias"], None, ly["idx"], ly["cnt"], ly["g"],
                                        out=ly["out"], copy_cached=False, workspace=ly["ws"], w_packed=ly["wp"])
    elif ly["mode"] == "split":
        ssi.sige_sparse_conv_layer_split(x, ly["wk"], ly["bias"], None, ly["idx"], ly["cnt"], ly["g"],
                                         out=ly["out"], copy_cached=False, workspace=ly["ws"])
    else:
        ssi.sige_sparse_conv_layer(x, ly["wk"], ly["bias"], None, ly["idx"], ly["cnt"], ly["g"], out=ly["out"],
                                   copy_cached=False)


def _gaugan_comparator(torch, F, ssi, synth, graph_time, timed_eager, seed):
    """The four GauGAN-shaped bf16 convs (32x64x1024 to 256x512x256) under the seeded star polygon at
    0.5 / 1.2 / 5 / 15 / 30% of the frame: the reduce (mask one bit per pixel,
    the cache copy on its idle workgroups) + sige_sparse_conv_layer_auto (the
    kernel the library picks; `path`: split, single (64 x 32 tiles) or wide
    (256 x 128 tiles); the weights packed once per layer by
    sige_pack_weights, outside the timing), against the dense conv through
    torch/MIOpen;
    best_of_two_bound: the faster of the single-range and split kernels (the
    two with entry points of their own) timed on the very edit, which a caller
    cannot do."""
    dev = torch.device("cuda:0")
    wl = synth.workload("gaugan_4conv_bf16")
    res, dense = {}, {}
    prep = []
    for li, L in enumerate(wl.layers):
        w_cpu, b_cpu = synth.make_layer_tensors(L, seed + li)
        a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed + li).to(dev)
        g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
        cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + li + 50).to(dev)
        wk = ssi.weight_to_krsc(w_cpu).to(dev)
        ww = ssi.sige_pack_weights(wk, g)
        prep.append((L, g, a_o, wk, b_cpu.to(dev), cache,
                     w_cpu.to(dev).contiguous(memory_format=torch.channels_last), ww))
        with torch.no_grad():
            x = a_o.permute(0, 3, 1, 2)
            dense[L.name] = round(timed_eager(lambda: F.conv2d(x, prep[-1][6], prep[-1][4].to(a_o.dtype),
                                                               padding=L.pad), 20), 3)
    for area in (0.005, 0.012, 0.05, 0.15, 0.30):
        shape = synth.edit_shape(wl, seed, area)
        row = {}
        for li, (L, g, a_o, wk, bias, cache, _, ww) in enumerate(prep):
            a_e = synth.make_edit(a_o.cpu(), shape.raster(L.h, L.w), wl.edit_kind, seed + li).to(dev)
            mbits = ssi.sige_diff_mask_bits(a_o, a_e, wl.tau)
            idx, cnt = ssi.sige_reduce_bits(mbits, L.h, L.w, g, L.dilate)
            out = torch.empty_like(cache)
            ws = torch.empty(ssi.sige_sparse_conv_layer_split_workspace(g, a_e.dtype), dtype=torch.uint8,
                             device=dev)
            plan = ssi.sige_sparse_conv_layer_plan(g, a_e.dtype)
            ws_auto = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)

            def auto():
                ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out, idx=idx, count=cnt)
                ssi.sige_sparse_conv_layer_auto(a_e, wk, bias, None, idx, cnt, g, out=out, copy_cached=False,
                                                workspace=ws_auto, w_packed=ww)

            def one():
                ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out, idx=idx, count=cnt)
                ssi.sige_sparse_conv_layer(a_e, wk, bias, None, idx, cnt, g, out=out, copy_cached=False)

            def split():
                ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cache, out=out, idx=idx, count=cnt)
                ssi.sige_sparse_conv_layer_split(a_e, wk, bias, None, idx, cnt, g, out=out, copy_cached=False,
                                                 workspace=ws)

            t0, t1, t2 = graph_time(auto, 5, 20), graph_time(one, 5, 20), graph_time(split, 5, 20)
            n = int(cnt.item())
            row[L.name] = {"blocks": n, "sparse_us": round(t0, 3),
                           "path": _auto_path(plan, n), "dense_miopen_us": dense[L.name],
                           "speedup": round(dense[L.name] / t0, 2),
                           "best_of_two_bound_us": round(min(t1, t2), 3),
                           "best_of_two_path": "split" if t2 < t1 else "single"}
        res[f"area_{area:g}"] = row
    return res


def _csrc_hash():
    """sha256 over every file of the HIP sources, in name order."""
    import hashlib

    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "spatially_sparse_incremental_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def _measured_kernel_traffic():
    """HBM bytes per launch of each kernel of the step and of the three-call path,
    from the committed counter summary; empty when any HIP source has changed
    since the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(here, "profiles", "step_kernels_unet256_pmc_traffic.md")
    try:
        fields = dict(line.split(": ", 1) for line in open(summary).read().splitlines() if ": " in line)
        if fields.get("csrc_sha256", "").strip() != _csrc_hash():
            return {}
        return {k[len("traffic_bytes."):]: int(v) for k, v in fields.items() if k.startswith("traffic_bytes.")}
    except (OSError, ValueError):
        return {}


def _measured_cold_kernels():
    """Per-kernel duration and HBM rate with the MALL evicted by reads, from the committed
    cold-cache summary; empty when any HIP source has changed since it was taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(here, "profiles", "step_kernels_unet256_cold_hbm.md")
    try:
        fields = dict(line.split(": ", 1) for line in open(summary).read().splitlines()
                      if ": " in line and "|" not in line)
        if fields.get("csrc_sha256", "").strip() != _csrc_hash():
            return {}
        out = {}
        for k, v in fields.items():
            if k.startswith("cold_us."):
                name = k[len("cold_us."):]
                nbytes = int(fields["cold_bytes." + name])
                us = float(v)
                out[name] = dict(us=us, bytes=nbytes, gbps=round(nbytes / (us * 1e-6) / 1e9, 1))
        return out
    except (OSError, ValueError, KeyError):
        return {}


def _active_pixels(idx, d, b):
    """Output pixels covered by the listed blocks (edge blocks clipped)."""
    tot = 0
    for lin in idx.tolist():
        r = lin % (d.nby * d.nbx)
        by, bx = r // d.nbx, r % d.nbx
        tot += min(b, d.ho - by * b) * min(b, d.wo - bx * b)
    return tot


def _cpu_baseline(a_o, a_e, w, bias, cache, L, tau, seconds):
    """The oracle, as it is, on the host cores: diff + reduce + edited layer output."""
    import oracle

    def once():
        m = oracle.diff_mask(a_o, a_e, tau)
        act = oracle.block_activity(m, L.h, L.w, L.k, L.stride, L.pad, L.block, L.dilate)
        oracle.index_list(act)
        oracle.sparse_layer(a_e, w, bias, L.k, L.stride, L.pad, L.block, act, cache)

    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < seconds and len(times) < 50):
        t0 = time.perf_counter()
        once()
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    threads = oracle.num_threads()
    # one thread, and the dense CPU conv of the same layer (every block), each timed once
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        once()
        single = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    t0 = time.perf_counter()
    oracle.dense_conv(a_e, w, bias, L.k, L.stride, L.pad)
    dense = time.perf_counter() - t0
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(med * 1e6, 1), "unit": "us per incremental layer update", "cores": threads,
            "kind": "oracle",
            "sample": f"the full workload (diff + reduce + edited layer incl. cache copy), median of {len(times)} "
                      f"runs, {len(os.sched_getaffinity(0))} host CPUs visible",
            "single_thread_us": round(single * 1e6, 1), "dense_conv_us": round(dense * 1e6, 1),
            "cpu_model": model}


if __name__ == "__main__":
    main()
