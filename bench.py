"""Benchmark of the routed-expert MoE FFN on one MI355X.

Default workload: one Hy4-shaped MoE layer in batch-1 decode (hidden 6144, intermediate
2048, 256 STQ1_0 routed experts, top-8, one bf16 shared expert).  A step is one pass of
the whole hot path -- route, permute, expert FFN, combine -- on one token, with the inputs
resident in HBM.  Steps rotate over several independently generated copies of the layer
(and fresh tokens) so that no step finds its weights in the 256 MB Infinity Cache left by
the previous one.

Printed: one JSON line.  `value` = expert-weight GB/s = (bytes of the 8 routed experts the
token touches + the shared expert) / step time.  Also reported: whole-layer algorithmic
GB/s, per-stage times from HIP events, the roofline of the dominant kernel, the CPU oracle
timed on a bounded sample, a prefill line (4096 tokens, MXFP4 x FP8) in TFLOP/s with and
without the shared expert, and the other format x regime pairs: STQ1_0 prefill (4096
tokens) and MXFP4 decode (one token, fused entry point).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
FP16_PEAK_TFLOPS = 2500.0
STQ_MAT_BYTES = 2048 * 6144 // 256 * 42          # one Hy4 STQ1_0 expert matrix
MX_MAT_BYTES = 2048 * 6144 // 2 + 2048 * 6144 // 32


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=8, help="layer copies the decode steps rotate over")
    p.add_argument("--prefill-steps", type=int, default=5)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the STQ1_0 prefill and MXFP4 decode lines")
    p.add_argument("--counter-run", action="store_true",
                   help="byte-counter runs: skip the work whose kernels share names with another "
                        "line's (the 29-layer chain, the MXFP4 64-token line's four-call comparison)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="first run a plain copy kernel (torch.neg) over this many MiB, three times, "
                        "as the reference dispatch for the HBM byte counters")
    p.add_argument("--trace-summary", metavar="TRACE_DIR",
                   help="print the per-kernel time table of a rocprofv3 --kernel-trace run and exit")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: summarise two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) "
                        "of this script into a markdown table with the per-launch HBM traffic")
    return p.parse_args()


def dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def make_decode_copy(c, copy):
    """Device tensors of one layer copy (its own seed)."""
    import synth
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import bf16_experts
    seed = c.seed * 1000 + copy
    routed = [synth.stq1_family(seed, 0, m, c.E, c.I * c.H) for m in range(3)]
    routed_t = [(dev(cd), dev(sc)) for cd, sc in routed]
    del routed
    sh = [dev(w) for w in synth.shared_weights(seed, 0, c.I, c.H)]
    return dict(routed=M.Experts(M.MOE_W_STQ1_0, *routed_t), shared=bf16_experts(*sh),
                wr=dev(synth.router_weights(seed, 0, c.E, c.H)),
                x=dev(synth.activations(seed, 0, 64, c.H)))


def decode_bench(args):
    import numpy as np
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M

    c = synth.cfg(1)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    copies = []
    for i in range(args.copies):
        t0 = time.perf_counter()
        copies.append(make_decode_copy(c, i))
        log(f"layer copy {i} ready in {time.perf_counter() - t0:.1f} s")
    f32, i32 = torch.float32, torch.int32
    logits = torch.empty((c.T, c.E), dtype=f32, device="cuda")
    ids = torch.empty((c.T, c.k), dtype=i32, device="cuda")
    w = torch.empty((c.T, c.k), dtype=f32, device="cuda")
    sp = torch.empty(d.P, dtype=i32, device="cuda")
    off = torch.empty(c.E + 1, dtype=i32, device="cuda")
    pp = torch.empty(d.P, dtype=i32, device="cuda")
    yp = torch.empty((d.P, c.H), dtype=f32, device="cuda")
    ysh = torch.empty((c.T, c.H), dtype=f32, device="cuda")
    out = torch.empty((c.T, c.H), dtype=f32, device="cuda")
    ws = torch.zeros(M.moe_layer_decode_workspace_size(d, True), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def step(i, st=None):
        L = copies[i % len(copies)]
        x = L["x"][(i // len(copies)) % 64].reshape(1, -1)
        M.moe_layer_decode(d, L["routed"], L["shared"], x, L["wr"], None, logits, ids, w, sp, off,
                           pp, yp, ysh, None, out, None, ws, s if st is None else st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps
    # the same steps replayed from one captured HIP graph (one step per layer copy)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream().cuda_stream
        for i in range(len(copies)):
            step(i, cs)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // len(copies))
    start.record(stream)
    for _ in range(reps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / (reps * len(copies))
    del graph
    # second pass with the library's per-kernel HIP events (same steps, same stream)
    M.moe_profile_enable(True)
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    prof = M.moe_profile_read()
    M.moe_profile_enable(False)
    # the four separate entry points on the same workload, for reference
    from bit_quantized_moe_softmax_amd.layer import LayerBuffers
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    n4 = min(args.steps, 50)
    ev0.record(stream)
    for i in range(n4):
        L = copies[i % len(copies)]
        x = L["x"][(i // len(copies)) % 64].reshape(1, -1)
        M.moe_route(d, x, L["wr"], None, None, bufs.logits, bufs.topk_ids, bufs.topk_w, s)
        M.moe_permute(d, bufs.topk_ids, bufs.sorted_pair, bufs.offsets, bufs.pair_pos, s)
        M.moe_expert_ffn(d, L["routed"], L["shared"], x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs,
                         bufs.y_shared, bufs.ws, s)
        M.moe_combine(d, bufs.y_pairs, bufs.topk_w, bufs.pair_pos, bufs.y_shared, None, bufs.out, None, s)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms4 = ev0.elapsed_time(ev1) / n4
    routed_gu_b = c.k * 2 * STQ_MAT_BYTES
    routed_dn_b = c.k * STQ_MAT_BYTES
    shared_gu_b = 2 * c.I * c.H * 2
    shared_dn_b = c.I * c.H * 2
    router_b = c.E * c.H * 2
    x_b = c.H * 2
    # algorithmic bytes per launch of each kernel: weights + activations read + results written
    P = c.T * c.k
    kb = {
        # router GEMV partials beside the shared gate/up: router and shared gate/up weights, x,
        # the shared h out (bf16 hi + lo)
        "decode_k1_route": router_b + shared_gu_b + x_b + c.T * c.I * 4,
        # routing, routed gate/up beside the shared down: the touched experts' gate/up, the
        # shared down weights, x and shared h in, routing outputs, routed h and y_shared out
        "decode_k2_gateup": routed_gu_b + shared_dn_b + x_b + c.T * c.I * 4 + c.T * c.E * 4
                            + (2 * c.k + c.E + 1) * 4 + P * c.I * 4 + c.T * c.H * 4,
        # routed down + combine: the touched experts' down weights, routed h and y_shared in,
        # y_pairs and out written
        "decode_k3_down_combine": routed_dn_b + P * c.I * 4 + c.T * c.H * 4 + P * c.H * 4 + c.T * c.H * 4,
    }
    expert_b = routed_gu_b + routed_dn_b + shared_gu_b + shared_dn_b
    layer_b = expert_b + router_b + x_b + c.H * 4
    return dict(c=c, ms=ms, ms4=ms4, graph_ms=graph_ms, t_wall=t_wall, expert_b=expert_b, layer_b=layer_b, prof=prof,
                kbytes=kb, routed_b=routed_gu_b + routed_dn_b, shared_b=shared_gu_b + shared_dn_b,
                router_b=router_b)


def prefill_bench(args):
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import LayerBuffers

    c = synth.cfg(3)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    t0 = time.perf_counter()
    sh = [(c.I, c.H), (c.I, c.H), (c.H, c.I)]
    routed = []
    for m in range(3):
        cd, sc = synth.mxfp4_family(c.seed, 0, m, c.E, *sh[m])
        dc, ds = dev(cd), dev(sc)
        # one-time weight preparation: repack into the tiled layout the GEMMs stream
        tc, ts = torch.empty_like(dc), torch.empty_like(ds)
        M.moe_mxfp4_pack_tiles(dc, ds, c.E * sh[m][0], sh[m][1], tc, ts)
        torch.cuda.synchronize()
        routed.append((tc, ts))
        del cd, sc, dc, ds
    R = M.Experts(M.MOE_W_MXFP4_TILED, *routed)
    x = dev(synth.activations(c.seed, 0, c.T, c.H))
    logits = dev(synth.prefill_logits(c.seed, 0, c.T, c.E))
    log(f"prefill inputs ready in {time.perf_counter() - t0:.1f} s")
    bufs = LayerBuffers(d, M.MOE_W_MXFP4_TILED, True)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    M.moe_route(d, None, None, None, logits, bufs.logits, bufs.topk_ids, bufs.topk_w, s)
    M.moe_permute(d, bufs.topk_ids, bufs.sorted_pair, bufs.offsets, bufs.pair_pos, s)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    M.moe_expert_ffn(d, R, None, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, None, bufs.ws, s)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.prefill_steps):
        M.moe_expert_ffn(d, R, None, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, None, bufs.ws, s)
    ev[1].record(stream)
    torch.cuda.synchronize()
    r_ms = ev[0].elapsed_time(ev[1]) / args.prefill_steps
    M.moe_profile_enable(True)
    for i in range(args.prefill_steps):
        M.moe_expert_ffn(d, R, None, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, None, bufs.ws, s)
    torch.cuda.synchronize()
    prof = M.moe_profile_read()
    M.moe_profile_enable(False)
    flops = 2.0 * c.T * c.k * 3 * c.I * c.H
    # the same layer with its bf16 shared expert (prefill grouped GEMMs on the bf16 MFMA)
    from bit_quantized_moe_softmax_amd.layer import bf16_experts
    sh = bf16_experts(*[dev(w) for w in synth.shared_weights(c.seed, 0, c.I, c.H)])
    M.moe_expert_ffn(d, R, sh, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, bufs.y_shared, bufs.ws, s)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.prefill_steps):
        M.moe_expert_ffn(d, R, sh, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, bufs.y_shared, bufs.ws, s)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ws_ms = ev[0].elapsed_time(ev[1]) / args.prefill_steps
    # and with the recipe's own shared-expert format: MXFP8 W8A8 group 32
    sh8 = M.Experts(M.MOE_W_MXFP8, *[(dev(cd), dev(sc)) for cd, sc in
                                     synth.shared_weights_mxfp8(c.seed, 0, c.I, c.H)])
    M.moe_expert_ffn(d, R, sh8, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, bufs.y_shared, bufs.ws, s)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.prefill_steps):
        M.moe_expert_ffn(d, R, sh8, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs, bufs.y_shared, bufs.ws, s)
    ev[1].record(stream)
    torch.cuda.synchronize()
    w8_ms = ev[0].elapsed_time(ev[1]) / args.prefill_steps
    return dict(c=c, routed_ms=r_ms, flops=flops, tflops=flops / (r_ms * 1e-3) / 1e12, prof=prof,
                with_shared_ms=ws_ms, with_mxfp8_shared_ms=w8_ms, shared_flops=2.0 * c.T * 3 * c.I * c.H)


def stq_prefill_bench(args):
    """Hy4 STQ1_0 layer at 4096 tokens through moe_expert_ffn: routed experts on the fp16-MFMA
    grouped GEMMs (weights decoded in registers) and the bf16 shared expert."""
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import LayerBuffers, bf16_experts

    c = synth.cfg(3)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    routed = [synth.stq1_family(c.seed, 0, m, c.E, c.I * c.H) for m in range(3)]
    R = M.Experts(M.MOE_W_STQ1_0, *[(dev(cd), dev(sc)) for cd, sc in routed])
    del routed
    sh = bf16_experts(*[dev(w) for w in synth.shared_weights(c.seed, 0, c.I, c.H)])
    x = dev(synth.activations(c.seed, 0, c.T, c.H))
    logits = dev(synth.prefill_logits(c.seed, 0, c.T, c.E))
    bufs = LayerBuffers(d, M.MOE_W_STQ1_0, True)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    M.moe_route(d, None, None, None, logits, bufs.logits, bufs.topk_ids, bufs.topk_w, s)
    M.moe_permute(d, bufs.topk_ids, bufs.sorted_pair, bufs.offsets, bufs.pair_pos, s)

    def run(n, shared):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(n):
            M.moe_expert_ffn(d, R, sh if shared else None, x, bufs.sorted_pair, bufs.offsets, bufs.y_pairs,
                             bufs.y_shared if shared else None, bufs.ws, s)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    run(1, True)
    r_ms = run(args.prefill_steps, False)
    ws_ms = run(args.prefill_steps, True)
    M.moe_profile_enable(True)
    run(args.prefill_steps, True)
    prof = M.moe_profile_read()
    M.moe_profile_enable(False)
    flops = 2.0 * c.T * c.k * 3 * c.I * c.H
    return dict(c=c, routed_ms=r_ms, with_shared_ms=ws_ms, flops=flops, prof=prof)


def slot_bank_bench(args, slots):
    """Hy4 STQ1_0 layer, one token, with the 256 routed experts in pinned host memory and an
    S-slot device bank: per step route, copy the ids to the host, plan, fetch the misses
    (host -> device), remap ids, permute, expert FFN over the slots, combine.  Host-to-device
    traffic is part of the step (context for models larger than HBM, not the headline)."""
    import numpy as np
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import LayerBuffers, bf16_experts

    c = synth.cfg(1)
    d = M.Dims(1, c.H, c.I, c.E, c.k)
    dS = M.Dims(1, c.H, c.I, slots, c.k)
    fams = [synth.stq1_family(c.seed, 0, m, c.E, c.I * c.H) for m in range(3)]
    host = [tuple(torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).pin_memory() for a in f) for f in fams]
    del fams
    per = []
    for cd, sc in host:
        per += [cd.numel() // c.E, sc.numel() // c.E]
    slot_t = [(torch.empty(slots * per[2 * i], dtype=torch.uint8, device="cuda"),
               torch.empty(slots * per[2 * i + 1], dtype=torch.uint8, device="cuda")) for i in range(3)]
    host_src = M.Experts(M.MOE_W_STQ1_0, *host)
    dev_slots = M.Experts(M.MOE_W_STQ1_0, *slot_t)
    shared = bf16_experts(*[dev(w) for w in synth.shared_weights(c.seed, 0, c.I, c.H)])
    wr = dev(synth.router_weights(c.seed, 0, c.E, c.H))
    xs = dev(synth.activations(c.seed, 3, 256, c.H))
    bank = M.SlotBank(c.E, slots, per, io_split=4)
    b = LayerBuffers(dS, M.MOE_W_STQ1_0, True)
    slot_of_dev = torch.empty(c.E, dtype=torch.int32, device="cuda")
    slot_ids = torch.empty((1, c.k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def step(i):
        x = xs[i % 256].reshape(1, -1)
        M.moe_route(d, x, wr, None, None, b.logits, b.topk_ids, b.topk_w, s)
        slot_of, _ = bank.plan(b.topk_ids.cpu().numpy())
        slot_of_dev.copy_(torch.from_numpy(slot_of), non_blocking=False)
        bank.fetch(host_src, dev_slots, s)
        M.moe_remap_ids(b.topk_ids, d.P, slot_of_dev, slot_ids, s)
        M.moe_permute(dS, slot_ids, b.sorted_pair, b.offsets, b.pair_pos, s)
        M.moe_expert_ffn(dS, dev_slots, shared, x, b.sorted_pair, b.offsets, b.y_pairs, b.y_shared, b.ws, s)
        M.moe_combine(dS, b.y_pairs, b.topk_w, b.pair_pos, b.y_shared, None, b.out, None, s)

    for i in range(8):
        step(i)
    torch.cuda.synchronize()
    h0, m0 = bank.stats()
    n = 48
    t0 = time.perf_counter()
    for i in range(8, 8 + n):
        step(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    h1, m1 = bank.stats()
    hits, misses = h1 - h0, m1 - m0
    moved = misses * sum(per)
    return {"slots": slots, "us_per_step": round(dt * 1e6, 1), "hit_rate": round(hits / max(1, hits + misses), 3),
            "host_to_device_gbs": round(moved / (dt * n) / 1e9, 1)}


def mx_decode_bench(args):
    """Hy4 layer with MXFP4 (tiled) routed experts, one token, through moe_layer_decode;
    steps rotate over three layer copies so the weights are not cache-resident."""
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import bf16_experts

    c = synth.cfg(1)
    d = M.Dims(1, c.H, c.I, c.E, c.k)
    shapes = [(c.I, c.H), (c.I, c.H), (c.H, c.I)]
    copies = []
    for cp in range(3):
        seed = c.seed * 1000 + 500 + cp
        fams = []
        for m in range(3):
            cd, sc = synth.mxfp4_family(seed, 0, m, c.E, *shapes[m])
            dc, ds = dev(cd), dev(sc)
            tc, ts = torch.empty_like(dc), torch.empty_like(ds)
            M.moe_mxfp4_pack_tiles(dc, ds, c.E * shapes[m][0], shapes[m][1], tc, ts)
            torch.cuda.synchronize()
            fams.append((tc, ts))
            del cd, sc, dc, ds
        copies.append(dict(R=M.Experts(M.MOE_W_MXFP4_TILED, *fams),
                           sh=bf16_experts(*[dev(w) for w in synth.shared_weights(seed, 0, c.I, c.H)]),
                           wr=dev(synth.router_weights(seed, 0, c.E, c.H)),
                           x=dev(synth.activations(seed, 0, 64, c.H))))
    f32, i32 = torch.float32, torch.int32
    bufs = [torch.empty((1, c.E), dtype=f32, device="cuda"), torch.empty((1, c.k), dtype=i32, device="cuda"),
            torch.empty((1, c.k), dtype=f32, device="cuda"), torch.empty(d.P, dtype=i32, device="cuda"),
            torch.empty(c.E + 1, dtype=i32, device="cuda"), torch.empty(d.P, dtype=i32, device="cuda"),
            torch.empty((d.P, c.H), dtype=f32, device="cuda"), torch.empty((1, c.H), dtype=f32, device="cuda")]
    out = torch.empty((1, c.H), dtype=f32, device="cuda")
    ws = torch.zeros(M.moe_layer_decode_workspace_size(d, True), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def step(i):
        L = copies[i % 3]
        M.moe_layer_decode(d, L["R"], L["sh"], L["x"][(i // 3) % 64].reshape(1, -1), L["wr"], None, *bufs,
                           None, out, None, ws, s)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    M.moe_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = M.moe_profile_read()
    M.moe_profile_enable(False)
    mat = c.I * c.H * 17 // 32                     # one MXFP4 expert matrix: E2M1 codes + UE8M0 scales
    # K1 router + x quantisation + shared gate/up; K2 routed gate/up + shared down; K3 routed
    # down + combine (+ y_shared)
    kb = {"decode_k1_route": c.E * c.H * 2 + c.H * 2 + c.H + c.H // 32 + 2 * c.I * c.H * 2 + c.I * 4,
          "decode_k2_gateup": c.k * 2 * mat + c.I * c.H * 2 + c.H + c.H // 32 + c.I * 4
                              + c.k * c.I * 33 // 32 + c.H * 4,
          "decode_k3_down_combine": c.k * mat + c.k * c.I * 33 // 32 + c.k * c.H * 4 + 2 * c.H * 4}
    expert_b = 3 * c.k * mat + 3 * c.I * c.H * 2
    return dict(c=c, ms=ms, prof=prof, kbytes=kb, expert_b=expert_b)


def gpu_stq_layer(c, seed):
    """One STQ1_0 Hy4 layer generated on the GPU from a seeded torch generator, with the
    distributions of the synthetic workloads: uniform code bytes (= uniform over the 32
    patterns), fp16 scales |N(0, 0.02)|, bf16 N(0, 0.02) router and shared expert."""
    import torch
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import bf16_experts
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    n_blk = c.I * c.H // 256
    fam = []
    for _ in range(3):
        codes = torch.randint(0, 256, (c.E, n_blk * 40), dtype=torch.uint8, device="cuda", generator=g)
        scales = (torch.randn((c.E, n_blk), device="cuda", generator=g).abs_() * 0.02).half().view(torch.int16)
        fam.append((codes, scales))

    def bf16(shape):
        return (torch.randn(shape, device="cuda", generator=g) * 0.02).bfloat16().view(torch.int16)

    return dict(routed=M.Experts(M.MOE_W_STQ1_0, *fam),
                shared=bf16_experts(bf16((c.I, c.H)), bf16((c.I, c.H)), bf16((c.H, c.I))),
                wr=bf16((c.E, c.H)))


def decode_bufs(d, c, shared=True):
    import torch
    f32, i32 = torch.float32, torch.int32
    import bit_quantized_moe_softmax_amd as M
    return dict(logits=torch.empty((c.T, c.E), dtype=f32, device="cuda"),
                ids=torch.empty((c.T, c.k), dtype=i32, device="cuda"),
                w=torch.empty((c.T, c.k), dtype=f32, device="cuda"),
                sp=torch.empty(d.P, dtype=i32, device="cuda"),
                off=torch.empty(c.E + 1, dtype=i32, device="cuda"),
                pp=torch.empty(d.P, dtype=i32, device="cuda"),
                yp=torch.empty((d.P, c.H), dtype=f32, device="cuda"),
                ysh=torch.empty((c.T, c.H), dtype=f32, device="cuda"),
                ws=torch.zeros(M.moe_layer_decode_workspace_size(d, shared), dtype=torch.uint8, device="cuda"))


def decode_call(M, d, L, x, bias, b, residual, out, stream):
    M.moe_layer_decode(d, L["routed"], L["shared"], x, L["wr"], bias, b["logits"], b["ids"], b["w"],
                       b["sp"], b["off"], b["pp"], b["yp"], b["ysh"], residual, out, None, b["ws"], stream)


def decode_t64_bench(args):
    """64-token decode with Zipf(1.1)-skewed routing (the batch-64 workload): one fused
    moe_layer_decode per step over 3 GPU-generated layer copies (the step's unique experts,
    about 0.7 GB, do not fit the 256 MB Infinity Cache, and the copies keep the shared expert
    and router cold too).  Reports U (unique experts per step), the unique-expert bytes and
    the whole step's algorithmic bytes as GB/s."""
    import numpy as np
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    c = synth.cfg(2)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    copies = [gpu_stq_layer(c, 2000 + i) for i in range(3)]
    xs = [dev(synth.activations(c.seed, 1 + i, c.T, c.H)) for i in range(2)]
    bias = dev(synth.zipf_bias(c.seed, 0, c.E))
    b = decode_bufs(d, c)
    out = torch.empty((c.T, c.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    # unique experts of every (copy, batch) combination the steps use
    U = {}
    for i in range(len(copies)):
        for j in range(len(xs)):
            decode_call(M, d, copies[i], xs[j], bias, b, None, out, s)
            torch.cuda.synchronize()
            U[(i, j)] = len(np.unique(b["ids"].cpu().numpy()))

    def step(i):
        decode_call(M, d, copies[i % 3], xs[(i // 3) % 2], bias, b, None, out, s)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    M.moe_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = M.moe_profile_read()
    M.moe_profile_enable(False)
    u_avg = float(np.mean([U[(i % 3, (i // 3) % 2)] for i in range(args.steps)]))
    expert_b = 3 * STQ_MAT_BYTES
    shared_b = 3 * c.I * c.H * 2
    router_b = c.E * c.H * 2
    act_b = c.T * c.H * 2 + c.T * c.H * 4 + d.P * c.H * 4 + c.T * c.H * 4   # x, out, y_pairs, y_shared
    unique_b = u_avg * expert_b
    step_b = unique_b + shared_b + router_b + act_b
    # beyond 4 tokens: K1 = router + routing beside the shared gate/up; K2 = routed gate/up;
    # K3 = shared and routed down (writes y_shared, y_pairs); K4 = combine
    kb = {"decode_k1_route": router_b + c.T * c.H * 2 + c.T * c.E * 4 + 2 * c.I * c.H * 2 + c.T * c.I * 4,
          "decode_k2_gateup": u_avg * 2 * STQ_MAT_BYTES + c.T * c.H * 2 + d.P * c.I * 4,
          "decode_k3_down_combine": u_avg * STQ_MAT_BYTES + c.I * c.H * 2 + (d.P + c.T) * c.I * 4
                                    + d.P * c.H * 4 + c.T * c.H * 4,
          "decode_k4_combine": d.P * c.H * 4 + 2 * c.T * c.H * 4}
    return dict(c=c, ms=ms, U=u_avg, unique_b=unique_b, step_b=step_b, prof=prof, kbytes=kb)


def gpu_mx_layer(c, seed):
    """One Hy4 layer with MXFP4 routed experts in the tiled layout, generated on the GPU from a
    seeded torch generator with the synthetic workloads' distributions: uniform E2M1 code bytes,
    UE8M0 scale bytes uniform over 127 + {-8 .. -4}, bf16 N(0, 0.02) router and shared expert."""
    import torch
    import bit_quantized_moe_softmax_amd as M
    from bit_quantized_moe_softmax_amd.layer import bf16_experts
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    fam = []
    for rows, K in ((c.I, c.H), (c.I, c.H), (c.H, c.I)):
        codes = torch.randint(0, 256, (c.E * rows, K // 2), dtype=torch.uint8, device="cuda", generator=g)
        scales = torch.randint(119, 124, (c.E * rows, K // 32), dtype=torch.uint8, device="cuda", generator=g)
        tc, ts = torch.empty_like(codes), torch.empty_like(scales)
        M.moe_mxfp4_pack_tiles(codes, scales, c.E * rows, K, tc, ts)
        torch.cuda.synchronize()
        del codes, scales
        fam.append((tc, ts))

    def bf16(shape):
        return (torch.randn(shape, device="cuda", generator=g) * 0.02).bfloat16().view(torch.int16)

    return dict(routed=M.Experts(M.MOE_W_MXFP4_TILED, *fam),
                shared=bf16_experts(bf16((c.I, c.H)), bf16((c.I, c.H)), bf16((c.H, c.I))),
                wr=bf16((c.E, c.H)))


def mx_decode_t64_bench(args):
    """64-token decode with Zipf(1.1) routing and MXFP4 (tiled) routed experts: the fused
    moe_layer_decode over 3 GPU-generated layer copies (about 2 GB of unique experts per step),
    and the same steps through the four separate calls (route, permute, expert FFN on the
    grouped GEMMs, combine) for comparison."""
    import numpy as np
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    c = synth.cfg(2)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    copies = [gpu_mx_layer(c, 5000 + i) for i in range(3)]
    xs = [dev(synth.activations(c.seed, 1 + i, c.T, c.H)) for i in range(2)]
    bias = dev(synth.zipf_bias(c.seed, 0, c.E))
    b = decode_bufs(d, c)
    out = torch.empty((c.T, c.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    U = {}
    for i in range(len(copies)):
        for j in range(len(xs)):
            decode_call(M, d, copies[i], xs[j], bias, b, None, out, s)
            torch.cuda.synchronize()
            U[(i, j)] = len(np.unique(b["ids"].cpu().numpy()))

    def step(i):
        decode_call(M, d, copies[i % 3], xs[(i // 3) % 2], bias, b, None, out, s)

    def timed(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(n):
            fn(i)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms = timed(step, args.steps)
    M.moe_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = M.moe_profile_read()
    M.moe_profile_enable(False)
    # the four separate calls on the same inputs
    ws4 = torch.zeros(M.moe_workspace_size(d, M.MOE_W_MXFP4_TILED, True), dtype=torch.uint8, device="cuda")

    def step4(i):
        L, x = copies[i % 3], xs[(i // 3) % 2]
        M.moe_route(d, x, L["wr"], bias, None, b["logits"], b["ids"], b["w"], s)
        M.moe_permute(d, b["ids"], b["sp"], b["off"], b["pp"], s)
        M.moe_expert_ffn(d, L["routed"], L["shared"], x, b["sp"], b["off"], b["yp"], b["ysh"], ws4, s)
        M.moe_combine(d, b["yp"], b["w"], b["pp"], b["ysh"], None, out, None, s)

    ms4 = float("nan")
    if not getattr(args, "counter_run", False):
        n4 = max(3, args.steps // 4)
        for i in range(3):
            step4(i)
        torch.cuda.synchronize()
        ms4 = timed(step4, n4)
    u_avg = float(np.mean([U[(i % 3, (i // 3) % 2)] for i in range(args.steps)]))
    P = d.P
    xq_b = c.T * (c.H + c.H // 32)
    hq_b = P * (c.I + c.I // 32)
    shared_b = 3 * c.I * c.H * 2
    router_b = c.E * c.H * 2
    unique_b = u_avg * 3 * MX_MAT_BYTES
    step_b = unique_b + shared_b + router_b + c.T * c.H * 2 + c.T * c.H * 4 + P * c.H * 4 + c.T * c.H * 4
    kb = {"decode_k1_route": router_b + c.T * c.H * 2 + c.T * c.E * 4 + 2 * c.I * c.H * 2 + c.T * c.I * 4 + xq_b,
          "decode_k2_gateup": u_avg * 2 * MX_MAT_BYTES + xq_b + hq_b,
          "decode_k3_down_combine": u_avg * MX_MAT_BYTES + c.I * c.H * 2 + c.T * c.I * 4 + hq_b
                                    + P * c.H * 4 + c.T * c.H * 4,
          "decode_k4_combine": P * c.H * 4 + 2 * c.T * c.H * 4}
    del copies
    torch.cuda.empty_cache()
    return dict(c=c, ms=ms, ms4=ms4, U=u_avg, unique_b=unique_b, step_b=step_b, prof=prof, kbytes=kb)


def chain_bench(args):
    """The 29-layer STQ1_0 stack at 16 tokens (about 46 GB of packed experts resident):
    a step runs, for every layer, RMSNorm (bf16 out) and the fused moe_layer_decode with the
    residual add, on Zipf-skewed routing.  Every step starts from the same hidden state, so
    every step touches the same experts; U per layer is read from the ids of an untimed pass."""
    import numpy as np
    import torch
    import synth
    import bit_quantized_moe_softmax_amd as M
    c = synth.cfg(4)
    d = M.Dims(c.T, c.H, c.I, c.E, c.k)
    t0 = time.perf_counter()
    layers = [gpu_stq_layer(c, 7000 + l) for l in range(c.layers)]
    biases = [dev(synth.zipf_bias(c.seed, l, c.E)) for l in range(c.layers)]
    torch.cuda.synchronize()
    log(f"29 layers generated on the GPU in {time.perf_counter() - t0:.1f} s")
    b = decode_bufs(d, c)
    r0 = dev(O_bf16_to_f32(synth.activations(c.seed, 0, c.T, c.H)))
    r = torch.empty_like(r0)
    r2 = torch.empty_like(r0)
    a = torch.empty((c.T, c.H), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    U = []

    def step(record=False):
        r.copy_(r0)
        cur, nxt = r, r2
        for l in range(c.layers):
            M.moe_rmsnorm_bf16(c.T, c.H, 1e-6, cur, a, s)
            decode_call(M, d, layers[l], a, biases[l], b, cur, nxt, s)
            if record:
                torch.cuda.synchronize()
                U.append(len(np.unique(b["ids"].cpu().numpy())))
            cur, nxt = nxt, cur

    step(record=True)
    for _ in range(max(1, args.warmup // 2)):
        step()
    torch.cuda.synchronize()
    n = max(3, args.steps // 2)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(n):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / n
    expert_b = 3 * STQ_MAT_BYTES
    # shared expert, router, and the activations: RMSNorm reads r and writes a; the layer reads
    # a and the residual, writes out, y_shared and y_pairs
    per_layer_fixed = 3 * c.I * c.H * 2 + c.E * c.H * 2 + c.T * c.H * (4 + 2 + 2 + 4 + 4 + 4) + d.P * c.H * 4
    step_b = sum(u * expert_b for u in U) + c.layers * per_layer_fixed
    del layers
    torch.cuda.empty_cache()
    return dict(c=c, ms=ms, U=U, step_b=step_b, steps=n)


def O_bf16_to_f32(bits):
    """bf16 bit patterns -> float32 (a plain reinterpretation, no arithmetic)."""
    import numpy as np
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


TRAFFIC_KERNELS = {  # profile slot -> substring of the HIP kernel name
    "decode_k1_route": "k1s_router<", "decode_k2_gateup": "k2s_gateup<",
    "decode_k3_down_combine": "k3_down_combine<", "mx_gateup": "mx_gemm_kernel<true, true, 8>",
    "mx_down": "mx_gemm_kernel<false, true, 8>", "stq_gateup": "g16_kernel<0, true, 1>",
    "stq_down": "g16_kernel<0, false, 2>", "mxdec_k2_gateup": "k2s_gateup_mx<",
    "mxdec_k3_down_combine": "k3_down_combine_mx<",
    # the 64-token decode (its K2 / K3 kernels are also the 16-token chain's, and its K1 the
    # MXFP4 64-token layer's: byte-counter runs pass --counter-run, which skips the chain)
    "t64_decode_k1_route": "k1_route<24, 8, 4,", "t64_decode_k2_gateup": "k2l_gateup<24, 8>",
    "t64_decode_k3_down_combine": "k3l_down<24, 8>", "mx64_decode_k2_gateup": "k2l_gateup_mx<24, 8, true>",
    "mx64_decode_k3_down_combine": "k3l_down_mx<24, 8, true>", "copy": "neg_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hy4_layer_hbm_traffic_per_kernel.md")
_DEC_SRC = "bit_quantized_moe_softmax_amd/csrc/decode_fused.hip"
_MX_SRC = "bit_quantized_moe_softmax_amd/csrc/mx_gemm.hip"
_G16_SRC = "bit_quantized_moe_softmax_amd/csrc/gemm16.hip"
TRAFFIC_SOURCES = {"decode_k1_route": _DEC_SRC, "decode_k2_gateup": _DEC_SRC,
                   "decode_k3_down_combine": _DEC_SRC, "mx_gateup": _MX_SRC, "mx_down": _MX_SRC,
                   "stq_gateup": _G16_SRC, "stq_down": _G16_SRC, "mxdec_k2_gateup": _DEC_SRC,
                   "mxdec_k3_down_combine": _DEC_SRC, "t64_decode_k1_route": _DEC_SRC,
                   "t64_decode_k2_gateup": _DEC_SRC, "t64_decode_k3_down_combine": _DEC_SRC,
                   "mx64_decode_k2_gateup": _DEC_SRC, "mx64_decode_k3_down_combine": _DEC_SRC}


def source_hash(slot):
    """First 16 hex digits of the sha256 of the source file that holds the slot's kernel, with
    its comments and blank lines removed (an edit of a comment does not change the kernel)."""
    import hashlib
    import re
    src = open(os.path.join(ROOT, TRAFFIC_SOURCES[slot]), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def pmc_summary(fetch_dir, write_dir, copy_mib):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled by what the same
    counters read for a plain copy of known size."""
    import csv
    import glob

    def load(d, counter):
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                for slot, sub in TRAFFIC_KERNELS.items():
                    if sub in r["Kernel_Name"]:
                        acc.setdefault(slot, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    fe, nf = load(fetch_dir, "FETCH_SIZE")
    wr, nw = load(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_fac = fe["copy"] / copy_kib
    w_fac = wr["copy"] / copy_kib
    rows = {}
    for slot in TRAFFIC_KERNELS:
        if slot == "copy" or slot not in fe or slot not in wr:
            continue
        b = (fe[slot] / f_fac + wr[slot] / w_fac) * 1024.0
        rows[slot] = {"fetch_kib": round(fe[slot], 1), "write_kib": round(wr[slot], 1),
                      "dispatches": [nf[slot], nw[slot]], "traffic_bytes": round(b),
                      "source_sha256_16": source_hash(slot)}
    data = {"copy_mib": copy_mib,
            "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4), "kernels": rows}
    print("| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches | HBM traffic B/launch (scaled) |")
    print("|---|---|---|---|---|")
    for slot, r in rows.items():
        print(f"| {slot} | {r['fetch_kib']} | {r['write_kib']} | {r['dispatches'][0]} / {r['dispatches'][1]} "
              f"| {r['traffic_bytes']} |")
    print(f"\nCopy calibration: {copy_mib} MiB read and written by torch.neg; FETCH_SIZE reads "
          f"{f_fac:.4f}x and WRITE_SIZE {w_fac:.4f}x the bytes moved.\n")
    print("traffic-json: " + json.dumps(data))


def trace_summary(trace_dir):
    """Per-kernel dispatch times (microseconds) from the kernel_trace.csv of a rocprofv3
    --kernel-trace run of this script.  Kernel names keep their template arguments; torch's own
    kernels are shown by their base name.  The MX grouped GEMMs and x quantisation that the
    64-token MXFP4 line runs through the separate entry points (an x quantisation over 64
    tokens precedes them) are listed apart, and the large-T decode kernels are also split by
    the k1_route instantiation that precedes them (one per workload)."""
    import csv
    import glob
    import re
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    def short(name):
        n = re.sub(r"^void ", "", name)
        n = re.sub(r"\(anonymous namespace\)::", "", n)
        if n.startswith("at::") or "native::" in n:
            return re.sub(r"<.*", "", n.split("(")[0]) + " (torch)"
        return re.sub(r"\(.*\)$", "", n).strip()

    stats, by_wl = {}, {}
    small_mx, k1 = False, None
    total = 0.0
    for r in rows:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        total += us
        n = short(r["Kernel_Name"])
        if n.startswith("mx_quant_kernel"):
            small_mx = int(r["Grid_Size_X"]) < 65536
        label = n
        if (n.startswith("mx_gemm_kernel") or n.startswith("mx_quant_kernel")) and small_mx:
            label = n + " [64-token four-call comparison]"
        stats.setdefault(label, []).append(us)
        if n.startswith("k1_route"):
            k1 = n
        if k1 and re.match(r"(k1_route|k2l_gateup|k3l_down|combine_kernel)", n):
            by_wl.setdefault((k1, n), []).append(us)
        if not re.match(r"(k1_route|k2l_gateup|k3l_down|combine_kernel|rmsnorm_kernel)", n):
            k1 = None
    print("| kernel | calls | avg us | min us | max us | % of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
              f"{100.0 * sum(v) / total:.2f} |")
    print("\nLarge-T kernels by workload (the k1_route instantiation that precedes them):\n")
    print("| after | kernel | calls | avg us | min us |")
    print("|---|---|---:|---:|---:|")
    for (a, k), v in sorted(by_wl.items()):
        print(f"| {a} | {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} |")


def load_traffic():
    """Per-launch HBM traffic from the committed counter summary, or {} when the kernels' sources
    changed after the counters were taken."""
    try:
        for line in open(TRAFFIC_FILE):
            if line.startswith("traffic-json: "):
                data = json.loads(line[len("traffic-json: "):])
                return {k: v["traffic_bytes"] for k, v in data["kernels"].items()
                        if k in TRAFFIC_SOURCES and v["source_sha256_16"] == source_hash(k)}
    except OSError:
        pass
    return {}


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _threads(n):
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except ImportError:  # pragma: no cover
        return contextlib.nullcontext()


def cpu_baseline(args, threads=None, budget_s=10.0, max_calls=16):
    """The oracle as it stands on batch-1 Hy4 STQ1_0 layer calls (fresh tokens) on the host's
    cores (all BLAS threads, or `threads`), bounded to about budget_s of work."""
    import synth
    from oracle import moe_oracle as O
    c = synth.cfg(1)
    x = synth.activations(c.seed, 0, 1, c.H)
    wr = synth.router_weights(c.seed, 0, c.E, c.H)
    sh = synth.shared_weights(c.seed, 0, c.I, c.H)
    shapes = [(c.I, c.H), (c.I, c.H), (c.H, c.I)]
    gen_s = [0.0]   # time spent generating the synthetic packed weights (not oracle work)

    def get_w(e, m):
        n = shapes[m][0] * shapes[m][1]
        t = time.perf_counter()
        codes, scales = synth.stq1_matrix(c.seed, 0, e, m, n)
        gen_s[0] += time.perf_counter() - t
        return O.stq1_matrix(codes, scales, *shapes[m])

    cores = threads or _cores()
    xs = synth.activations(c.seed, 1, 16, c.H)
    n = 0
    with _threads(cores):
        t0 = time.perf_counter()
        while n < max_calls and (n == 0 or time.perf_counter() - t0 - gen_s[0] < budget_s):
            O.moe_layer(x if n == 0 else xs[n:n + 1], c.k, get_w, "stq1", wr_bits=wr, shared=sh)
            n += 1
        dt = (time.perf_counter() - t0 - gen_s[0]) / n
    expert_b = c.k * 3 * STQ_MAT_BYTES + 3 * c.I * c.H * 2
    return dict(value=expert_b / dt / 1e9, unit="GB/s", cores=cores, kind="oracle",
                sample=f"{n} batch-1 Hy4 STQ1_0 layer calls on fresh tokens (route, 8 routed experts "
                       f"decoded and applied in float64, shared expert, combine), {cores} BLAS "
                       f"thread{'s' if cores > 1 else ''}, {dt:.2f} s per call without the synthetic "
                       f"weight generation; value = expert-weight bytes per call / time per call")


def cpu_baselines_extra():
    """Bounded samples of the oracle on the other workloads (host cores, all BLAS threads;
    synthetic weight generation excluded): 2 tokens of the 64-token Zipf batch, a few experts
    of the 4096-token MXFP4 prefill with all their pairs (float32 BLAS for the matmuls, as a
    timing stand-in; parity runs in float64), and the 2 sampled tokens of the 29-layer chain
    through one layer.  Each in the unit of its GPU line."""
    import numpy as np
    import synth
    from oracle import moe_oracle as O
    cores = _cores()
    out = {}
    sh = [(2048, 6144), (2048, 6144), (6144, 2048)]
    with _threads(cores):
        # 64-token Zipf decode: 2 tokens of the batch, GB/s of their unique experts' bytes
        c = synth.cfg(2)
        x = synth.activations(c.seed, 0, 2, c.H)
        wr = synth.router_weights(c.seed, 0, c.E, c.H)
        bias = synth.zipf_bias(c.seed, 0, c.E)
        shw = synth.shared_weights(c.seed, 0, c.I, c.H)
        gen = [0.0]

        def stq_w(seed, layer):
            def get_w(e, m):
                t = time.perf_counter()
                cd, sc = synth.stq1_matrix(seed, layer, e, m, sh[m][0] * sh[m][1])
                gen[0] += time.perf_counter() - t
                return O.stq1_matrix(cd, sc, *sh[m])
            return get_w

        t0 = time.perf_counter()
        ref = O.moe_layer(x, c.k, stq_w(c.seed, 0), "stq1", wr_bits=wr, bias=bias, shared=shw)
        dt = time.perf_counter() - t0 - gen[0]
        U = len(np.unique(ref["ids"]))
        b = U * 3 * STQ_MAT_BYTES + 3 * c.I * c.H * 2 + c.E * c.H * 2
        out["decode_t64_zipf"] = dict(value=b / dt / 1e9, unit="GB/s", cores=cores, kind="oracle",
                                      sample=f"2 of the 64 tokens ({U} unique experts) through the whole "
                                             f"layer in {dt:.2f} s; value = their unique-expert + shared + "
                                             f"router bytes / time")
        # 4096-token MXFP4 prefill: experts 0, 1 with all their pairs, fp32 matmuls
        c = synth.cfg(3)
        logits = synth.prefill_logits(c.seed, 0, c.T, c.E)
        _, ids, _ = O.route(c.k, logits_in=logits)
        sp, off, _ = O.permute(ids, c.E)
        xall = synth.activations(c.seed, 0, c.T, c.H)
        flop = 0.0
        gen[0] = 0.0
        t0 = time.perf_counter()
        for e in (0, 1):
            toks = sp[off[e]:off[e + 1]] // c.k
            tg = time.perf_counter()
            mats = [synth.mxfp4_matrix(c.seed, 0, e, m, *sh[m]) for m in range(3)]
            gen[0] += time.perf_counter() - tg
            W = [O.mxfp4_matrix(cd, sc, *sh[m]).astype(np.float32) for m, (cd, sc) in enumerate(mats)]
            a = O.mx_dequantize_e4m3(*O.mx_quantize_e4m3(O.bf16_to_f64(xall[toks]))).astype(np.float32)
            h = O.silu(a @ W[0].T) * (a @ W[1].T)
            hq = O.mx_dequantize_e4m3(*O.mx_quantize_e4m3(h)).astype(np.float32)
            _ = hq @ W[2].T
            flop += 2.0 * len(toks) * 3 * c.I * c.H
        dt = time.perf_counter() - t0 - gen[0]
        out["mxfp4_prefill_t4096"] = dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                                          sample=f"experts 0 and 1 with all their pairs ({int(flop / (2 * 3 * c.I * c.H))} "
                                                 f"pairs) of the 4096-token batch: MX quantisation, E2M1 decode, "
                                                 f"float32 matmuls, in {dt:.2f} s")
        # 29-layer chain: the 2 sampled tokens through layer 0
        c = synth.cfg(4)
        toks = synth.sample_tokens(c.seed, c.T, 2)
        xr = O.bf16_to_f64(synth.activations(c.seed, 0, c.T, c.H))[toks]
        gen[0] = 0.0
        t0 = time.perf_counter()
        a = O.rmsnorm_bf16(xr)
        ref = O.moe_layer(a, c.k, stq_w(c.seed, 0), "stq1", wr_bits=synth.router_weights(c.seed, 0, c.E, c.H),
                          bias=synth.zipf_bias(c.seed, 0, c.E), shared=synth.shared_weights(c.seed, 0, c.I, c.H),
                          residual=xr)
        dt = time.perf_counter() - t0 - gen[0]
        U = len(np.unique(ref["ids"]))
        b = U * 3 * STQ_MAT_BYTES + 3 * c.I * c.H * 2 + c.E * c.H * 2
        out["chain_29_layers"] = dict(value=b / dt / 1e9, unit="GB/s", cores=cores, kind="oracle",
                                      sample=f"the 2 sampled tokens through layer 0 of 29 (RMSNorm, {U} unique "
                                             f"experts, shared expert, residual) in {dt:.2f} s")
    return out


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.calibrate_copy_mib)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU expert-parallel path is a design, not code)"}))
        sys.exit(2)
    import torch
    import bit_quantized_moe_softmax_amd as M
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    M.lib()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    traffic = load_traffic()
    dec = decode_bench(args)
    c = dec["c"]
    value = dec["expert_b"] / (dec["ms"] * 1e-3) / 1e9
    kern = {}
    for name, nbytes in dec["kbytes"].items():
        us, n = dec["prof"][name]
        if n == 0:
            continue   # a kernel of the other decode structure
        kern[name] = {"avg_us": round(us, 3), "launches": n, "algorithmic_bytes": nbytes,
                      "gbs": round(nbytes / (us * 1e-6) / 1e9, 1) if us > 0 else None}
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    dk = kern[dom]
    out = {
        "metric": "MoE FFN expert-weight GB/s (decode) + TFLOP/s (prefill), % of roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hy4-stq1_0-decode-t1", "tokens": c.T, "hidden": c.H,
                   "intermediate": c.I, "experts": c.E, "top_k": c.k, "shared_expert": "bf16",
                   "routed_format": "STQ1_0", "layer_copies": args.copies,
                   "entry_point": "moe_layer_decode"},
        "whole_layer_gbs": round(dec["layer_b"] / (dec["ms"] * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "four_call_ms_per_step": round(dec["ms4"], 5),
        "graph_ms_per_step": round(dec["graph_ms"], 5),
        "graph_value": round(dec["expert_b"] / (dec["graph_ms"] * 1e-3) / 1e9, 1),
        "kernels": kern,
        "bytes_per_step": {"routed": dec["routed_b"], "shared": dec["shared_b"],
                           "router": dec["router_b"], "layer_total": dec["layer_b"]},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": dk["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dk["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic.get(dom), "algorithmic_bytes": dk["algorithmic_bytes"]},
    }
    if not args.no_prefill:
        try:
            pre = prefill_bench(args)
            pc = pre["c"]
            gu_flop = 2.0 * pc.T * pc.k * 2 * pc.I * pc.H
            dn_flop = 2.0 * pc.T * pc.k * pc.I * pc.H
            pk = {}
            for name, fl in (("mx_gateup", gu_flop), ("mx_down", dn_flop), ("mx_quant", None)):
                us, n = pre["prof"][name]
                pk[name] = {"avg_us": round(us, 2), "launches": n,
                            "tflops": round(fl / (us * 1e-6) / 1e12, 1) if (fl and us > 0) else None}
            out["prefill"] = {"workload": "hy4-mxfp4xfp8-prefill-t4096", "routed_ms": round(pre["routed_ms"], 4),
                              "tflops": round(pre["tflops"], 1), "peak_tflops_fp8": FP8_PEAK_TFLOPS,
                              "frac": round(pre["tflops"] / FP8_PEAK_TFLOPS, 4),
                              "routed_flop": pre["flops"], "kernels": pk,
                              "roofline": {"bound": "mfma", "kernel": "mx_gateup",
                                           "achieved": pk["mx_gateup"]["tflops"], "peak": FP8_PEAK_TFLOPS,
                                           "unit": "TFLOP/s",
                                           "frac": round((pk["mx_gateup"]["tflops"] or 0) / FP8_PEAK_TFLOPS, 4),
                                           "traffic": traffic.get("mx_gateup")}}
            sh_ms = pre["with_shared_ms"] - pre["routed_ms"]
            out["prefill"]["with_shared_expert"] = {
                "layer_ms": round(pre["with_shared_ms"], 4),
                "shared_ms": round(sh_ms, 4),
                "shared_tflops_bf16": round(pre["shared_flops"] / (sh_ms * 1e-3) / 1e12, 1) if sh_ms > 0 else None,
                "kernels": {n: round(pre["prof"][n][0], 2) for n in ("shared_gateup", "shared_down", "act_prep")
                            if pre["prof"][n][1]}}
            s8_ms = pre["with_mxfp8_shared_ms"] - pre["routed_ms"]
            out["prefill"]["with_mxfp8_shared_expert"] = {
                "layer_ms": round(pre["with_mxfp8_shared_ms"], 4), "shared_ms": round(s8_ms, 4),
                "note": "the WFP4AFP8 recipe's formats: MXFP4 routed experts, MXFP8 W8A8 shared expert"}
        except Exception as e:  # the decode line must still print
            out["prefill"] = {"error": repr(e)}
    if not args.no_extra:
        # the other format x regime pairs: STQ1_0 prefill, MXFP4 decode
        try:
            sp = stq_prefill_bench(args)
            pk = {n: round(sp["prof"][n][0], 2) for n in ("stq_gateup", "stq_down", "shared_gateup",
                                                          "shared_down", "act_prep") if sp["prof"][n][1]}
            gu = 2.0 * sp["c"].T * sp["c"].k * 2 * sp["c"].I * sp["c"].H
            gu_tf = round(gu / (pk["stq_gateup"] * 1e-6) / 1e12, 1) if pk.get("stq_gateup") else None
            out["stq1_0_prefill"] = {
                "workload": "hy4-stq1_0-prefill-t4096", "routed_ms": round(sp["routed_ms"], 4),
                "layer_ms": round(sp["with_shared_ms"], 4),
                "tflops": round(sp["flops"] / (sp["routed_ms"] * 1e-3) / 1e12, 1),
                "peak_tflops_fp16": FP16_PEAK_TFLOPS,
                "frac": round(sp["flops"] / (sp["routed_ms"] * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
                "kernels_us": pk,
                "roofline": {"bound": "mfma", "kernel": "stq_gateup", "achieved": gu_tf,
                             "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round((gu_tf or 0) / FP16_PEAK_TFLOPS, 4),
                             "traffic": traffic.get("stq_gateup")}}
        except Exception as e:
            out["stq1_0_prefill"] = {"error": repr(e)}
        try:
            md = mx_decode_bench(args)
            kern = {}
            for name, nbytes in md["kbytes"].items():
                us, n = md["prof"][name]
                kern[name] = {"avg_us": round(us, 3), "algorithmic_bytes": nbytes,
                              "gbs": round(nbytes / (us * 1e-6) / 1e9, 1) if us > 0 else None}
            gbs = md["expert_b"] / (md["ms"] * 1e-3) / 1e9
            k2 = kern["decode_k2_gateup"]
            out["mxfp4_decode"] = {"workload": "hy4-mxfp4xfp8-decode-t1", "entry_point": "moe_layer_decode",
                                   "us_per_step": round(md["ms"] * 1e3, 2), "expert_weight_gbs": round(gbs, 1),
                                   "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "kernels": kern,
                                   "roofline": {"bound": "hbm", "kernel": "decode_k2_gateup (MXFP4)",
                                                "achieved": k2["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                "frac": round((k2["gbs"] or 0) / HBM_PEAK_GBS, 4),
                                                "traffic": traffic.get("mxdec_k2_gateup"),
                                                "algorithmic_bytes": k2["algorithmic_bytes"]}}
        except Exception as e:
            out["mxfp4_decode"] = {"error": repr(e)}
        try:
            out["slot_bank_decode"] = {
                "workload": "hy4-stq1_0-decode-t1, routed experts in pinned host memory",
                "note": "host-to-device copies inside the step (PCIe-inclusive); random tokens, so hits "
                        "come only from the bank holding a slot's expert by chance",
                "runs": [slot_bank_bench(args, S) for S in (8, 96)]}
        except Exception as e:
            out["slot_bank_decode"] = {"error": repr(e)}
    if not args.no_extra:
        try:
            t64 = decode_t64_bench(args)
            kern = {}
            for name, nbytes in t64["kbytes"].items():
                us, n = t64["prof"][name]
                if n == 0:
                    continue
                kern[name] = {"avg_us": round(us, 3), "launches": n, "algorithmic_bytes": round(nbytes),
                              "gbs": round(nbytes / (us * 1e-6) / 1e9, 1) if us > 0 else None}
            dom = max(kern, key=lambda k: kern[k]["avg_us"])
            gbs = t64["step_b"] / (t64["ms"] * 1e-3) / 1e9
            out["decode_t64_zipf"] = {
                "workload": "hy4-stq1_0-decode-t64-zipf1.1", "entry_point": "moe_layer_decode",
                "us_per_step": round(t64["ms"] * 1e3, 2), "unique_experts": round(t64["U"], 2),
                "unique_expert_bytes": round(t64["unique_b"]), "step_bytes": round(t64["step_b"]),
                "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "unique_expert_gbs": round(t64["unique_b"] / (t64["ms"] * 1e-3) / 1e9, 1),
                "kernels": kern,
                "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["gbs"], "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round((kern[dom]["gbs"] or 0) / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get("t64_" + dom), "algorithmic_bytes": kern[dom]["algorithmic_bytes"]}}
        except Exception as e:
            out["decode_t64_zipf"] = {"error": repr(e)}
    if not args.no_extra:
        try:
            m64 = mx_decode_t64_bench(args)
            kern = {}
            for name, nbytes in m64["kbytes"].items():
                us, n = m64["prof"][name]
                if n == 0:
                    continue
                kern[name] = {"avg_us": round(us, 3), "launches": n, "algorithmic_bytes": round(nbytes),
                              "gbs": round(nbytes / (us * 1e-6) / 1e9, 1) if us > 0 else None}
            dom = max(kern, key=lambda k: kern[k]["avg_us"])
            gbs = m64["step_b"] / (m64["ms"] * 1e-3) / 1e9
            out["mxfp4_decode_t64_zipf"] = {
                "workload": "hy4-mxfp4xfp8-decode-t64-zipf1.1", "entry_point": "moe_layer_decode",
                "us_per_step": round(m64["ms"] * 1e3, 2), "unique_experts": round(m64["U"], 2),
                "unique_expert_bytes": round(m64["unique_b"]), "step_bytes": round(m64["step_b"]),
                "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "four_call_us_per_step": round(m64["ms4"] * 1e3, 2) if m64["ms4"] == m64["ms4"] else None,
                "kernels": kern,
                "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["gbs"], "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round((kern[dom]["gbs"] or 0) / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get("mx64_" + dom), "algorithmic_bytes": kern[dom]["algorithmic_bytes"]}}
        except Exception as e:
            out["mxfp4_decode_t64_zipf"] = {"error": repr(e)}
    if not args.no_extra and not args.counter_run:
        try:
            ch = chain_bench(args)
            gbs = ch["step_b"] / (ch["ms"] * 1e-3) / 1e9
            out["chain_29_layers"] = {
                "workload": "hy4-stq1_0-stack29-t16-zipf1.1", "layers": ch["c"].layers, "tokens": ch["c"].T,
                "resident_expert_bytes": ch["c"].layers * ch["c"].E * 3 * STQ_MAT_BYTES,
                "ms_per_step": round(ch["ms"], 4), "steps": ch["steps"], "step_bytes": round(ch["step_b"]),
                "unique_experts_per_layer": ch["U"], "gbs": round(gbs, 1),
                "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "note": "a step = 29 x (RMSNorm + fused layer with residual) from the same hidden state"}
        except Exception as e:
            out["chain_29_layers"] = {"error": repr(e)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args)
        out["cpu_baseline_1thread"] = cpu_baseline(args, threads=1, budget_s=4.0, max_calls=1)
        try:
            out["cpu_baseline_other_workloads"] = cpu_baselines_extra()
        except Exception as e:
            out["cpu_baseline_other_workloads"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
