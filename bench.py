#!/usr/bin/env python3
"""Benchmark of the MoE-layer hot path on one MI355X.

Headline (the JSON line's `value`): prefill throughput in tokens/s of one MoE
layer at T=2048 tokens with Zipf-skewed routing (H=2048, I=512, 256 experts,
top-8 + shared expert, 4-bit affine g=64 weights), one step = moe_route +
moe_expert_ffn_q4 (both expert GEMMs in one persistent launch, then the
combine) on a batch already resident in HBM.  Consecutive steps rotate over
independently seeded weight sets (distinct layers) so that no step finds its
weights in the 256 MB last-level cache.

Also reported: the one-launch GEMM kernel's MFMA roofline fraction (HIP events
around its launch, timed per step), the same steps with the two GEMMs as two
launches (moe_expert_gemm_q4 + moe_down_combine), the batch-1 decode path's HBM
bandwidth (40 independently weighted layers, one call each) and the per-layer
latency of the same 40 layers chained through the residual add and RMSNorm (one
HIP graph, no host synchronisation), decode calls of 2, 4 and 8 tokens, a
16384-token prompt through one layer in chunks of 2048 tokens (workspace bounded
by the chunk) next to the single call, the T=512 layer with uniform-ish routing (every expert active: HBM
bandwidth over the weights read), a stack of 40 layers at T=4096 with the
residual add and RMSNorm between layers (tokens/s, no host synchronisation in
the pass), and the CPU oracle's throughput on a bounded token sample.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer prefill tokens/s @T=2048 (MFMA %); T=1 decode HBM GB/s (% of peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (dense fp16 is the same figure)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

T, H, I, E, K_TOP = 2048, 2048, 512, 256, 8
ZIPF_S = 1.1
SEED_PREFILL = 4000
SEED_DECODE = 2000
SEED_UNIFORM = 3000
SEED_EP_SHARE = 6000
SEED_STACK = 5000
MIN_WARMUP = 60                # steps of sustained load before the clocks settle (measured)


# HBM traffic of the one-launch GEMM kernel (q4_ffn_kernel) on this workload, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, mean
# over the dispatches), each scaled by what the same counter reports for a plain 256 MiB
# device-to-device copy (bench.py --copy-calibration 256: FETCH_SIZE reads 131085.4 KiB ->
# x2.0, WRITE_SIZE 262144 KiB -> x1.0).  Valid only for the GEMM source these counters were
# taken on; otherwise (or before they are taken) the JSON reports null.
FFN_TRAFFIC = {
    "gemm_src_sha256": "94aec9054e878f00509ce45aba73d258f3395060b565913175d1f27a70a7ea43",
    "fetch_kib": 265492.1042, "fetch_scale": 2.0,
    "write_kib": 102882.0104, "write_scale": 1.0,
    "profile": "profiles/moe_layer_prefill2048_zipf_hbm_traffic.md",
}


def ffn_traffic_bytes():
    import hashlib
    t = FFN_TRAFFIC
    if t is None:
        return None
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                       "bit_quantized_expert_top_amd", "csrc", "gemm.hip")
    try:
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if h != t["gemm_src_sha256"]:
        return None
    return round((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024)


def expert_bytes(H, I):
    """Packed bytes of one expert: codes (0.5 B/weight) + bf16 scale and bias per 64 weights."""
    return 3 * H * I // 2 + 3 * H * (I // 64) * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=120,
                    help="untimed steps replayed back to back right before the timed ones; at "
                         "least MIN_WARMUP are run (the clocks take about 60 steps of sustained "
                         "load to settle), and the JSON reports the number run")
    ap.add_argument("--sets", type=int, default=6, help="weight sets rotated in the prefill loop")
    ap.add_argument("--decode-sets", type=int, default=40,
                    help="T=1 layers (independent weights): decode calls and the chained stack")
    ap.add_argument("--decode-steps", type=int, default=400)
    ap.add_argument("--ep-share-sets", type=int, default=4,
                    help="weight sets of the T=2048 leg whose picks stay on one GPU's expert-parallel "
                         "share (32 of 256 experts); 0 skips it")
    ap.add_argument("--uniform-sets", type=int, default=4,
                    help="weight sets of the T=512 uniform-routing leg (0: skip it)")
    ap.add_argument("--stack-layers", type=int, default=40,
                    help="layers of the T=4096 stack leg (0: skip it)")
    ap.add_argument("--chunked-tokens", type=int, default=16384,
                    help="prompt length of the chunked-prefill leg (0 skips it)")
    ap.add_argument("--affine-sets", type=int, default=4,
                    help="weight sets of the affine-bias prefill leg (0: skip it)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the MoE layer on one GPU only; the expert-parallel "
              "split across GPUs is a design note, not implemented. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_expert_top_amd as moe
    from synth.device import make_layer_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return
    shape = moe.Shape(T=T, H=H, I=I, E=E, top_k=K_TOP)

    def device_layer(d):
        proj = {n: d[n] for n in moe.DeviceLayer.NAMES}
        # packed into the tile layout once, like a weight load; row copies dropped
        return moe.DeviceLayer(proj, d["router_wt"], d["router_bias"], device=dev, keep_rows=False)

    # ---------------- prefill: T=2048, Zipf-skewed routing ----------------
    print(f"[bench] generating {args.sets} prefill weight sets", file=sys.stderr, flush=True)
    raw0 = make_layer_device(SEED_PREFILL, T, H, I, E, zipf_s=ZIPF_S, device=dev)
    x = raw0["x"]
    sets = [device_layer(raw0)]
    for s in range(1, args.sets):
        sets.append(device_layer(make_layer_device(SEED_PREFILL + 100 * s, T, H, I, E,
                                                   zipf_s=ZIPF_S, device=dev, with_x=False)))
    r = moe.Routing(shape, dev, with_logits=False)
    ws = moe.workspace(shape, dev)
    h = torch.empty((T * K_TOP + T, I), dtype=torch.int16, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step(w):
        moe.moe_route(shape, x, w, r, ws)
        moe.moe_expert_ffn_q4(shape, x, w, r, h, y, ws)

    def phases(step_inputs, xs, r_, ws_, h_, y_):
        """Eager steps with HIP events on the launch stream between the routing, the one-launch
        GEMM kernel (moe_expert_ffn_q4 without its combine) and the combine: mean ms of each."""
        ev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in step_inputs]
        for (w, shp), e in zip(step_inputs, ev_):
            e[0].record()
            moe.moe_route(shp, xs, w, r_, ws_)
            e[1].record()
            moe.moe_expert_ffn_q4(shp, xs, w, r_, h_, y_, ws_, combine=False)
            e[2].record()
            moe.moe_combine(shp, r_, y_, ws_)
            e[3].record()
        torch.cuda.synchronize()
        n_ = len(ev_)
        return [sum(e[i].elapsed_time(e[i + 1]) for e in ev_) / n_ for i in range(3)]

    for w in sets:                                  # first touch of every set and buffer
        step(w)
    torch.cuda.synchronize()

    K = args.steps
    route_ms, ffn_ms, comb_ms = phases([(sets[s % len(sets)], shape) for s in range(K)], x, r, ws,
                                       h, y)

    # throughput: the layer steps captured in HIP graphs (one step per weight set, and
    # the K mod sets remaining steps), replayed so that exactly K steps run between the
    # first and the last event; an event between replays gives each replay's time
    def capture(ws_):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for w in ws_:
                step(w)
        g.replay()
        return g

    graph = capture(sets)
    reps, rem = divmod(K, len(sets))
    graph_rem = capture(sets[:rem]) if rem else None
    # the W warmup steps (at least MIN_WARMUP, rounded up to whole replays), back to back as
    # the timed ones
    warm_reps = -(-max(args.warmup, MIN_WARMUP) // len(sets))
    warm_steps = warm_reps * len(sets)
    for _ in range(warm_reps):
        graph.replay()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
    wall0 = time.perf_counter()
    evs[0].record()
    for i in range(reps):
        graph.replay()
        evs[i + 1].record()
    if graph_rem is not None:
        graph_rem.replay()
    evs[-1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_step = total_ms / K
    rep_step_us = sorted(evs[i].elapsed_time(evs[i + 1]) / len(sets) * 1e3 for i in range(reps))
    step_stats = ({"mean": round(ms_step * 1e3, 2), "median": round(rep_step_us[len(rep_step_us) // 2], 2),
                   "min": round(rep_step_us[0], 2), "replays": reps, "steps_per_replay": len(sets)}
                  if reps else {"mean": round(ms_step * 1e3, 2)})
    del graph, graph_rem

    print(f"[bench] prefill {ms_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    rows = T * K_TOP + T
    flops_gateup = 2.0 * rows * (2 * I) * H
    flops_down = 2.0 * rows * I * H
    flops_ffn = flops_gateup + flops_down
    tok_s = T / (ms_step * 1e-3)
    ffn_tflops = flops_ffn / (ffn_ms * 1e-3) / 1e12
    layer_mfma_frac = flops_ffn / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)

    # the same steps with the GEMMs as two launches (moe_expert_gemm_q4, moe_down_combine)
    def step2(w):
        moe.moe_route(shape, x, w, r, ws)
        moe.moe_expert_gemm_q4(shape, x, w, r, h, ws)
        moe.moe_down_combine(shape, h, w, r, y, ws)

    K2 = min(K, 2 * len(sets))
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K2)]
    for s_ in range(K2):
        w = sets[s_ % len(sets)]
        moe.moe_route(shape, x, w, r, ws)
        ev2[s_][0].record()
        moe.moe_expert_gemm_q4(shape, x, w, r, h, ws)
        ev2[s_][1].record()
        moe.moe_down_combine(shape, h, w, r, y, ws)
        ev2[s_][2].record()
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        for w in sets:
            step2(w)
    for _ in range(warm_reps + 1):                  # the same warmup as the timed steps
        g2.replay()
    t2a = torch.cuda.Event(enable_timing=True)
    t2b = torch.cuda.Event(enable_timing=True)
    reps2 = max(1, reps)
    t2a.record()
    for _ in range(reps2):
        g2.replay()
    t2b.record()
    torch.cuda.synchronize()
    two_launch = {"us_per_step": round(t2a.elapsed_time(t2b) / (reps2 * len(sets)) * 1e3, 2),
                  "gateup_us": round(sum(e[0].elapsed_time(e[1]) for e in ev2) / K2 * 1e3, 2),
                  "down_combine_us": round(sum(e[1].elapsed_time(e[2]) for e in ev2) / K2 * 1e3, 2)}
    del g2

    # ---------------- the same workload with biases b != -8 s in every group ----------------
    # (the general affine format: the GEMMs add the rank-G bias term in every item)
    affine = None
    if args.affine_sets:
        print(f"[bench] affine biases, {args.affine_sets} weight sets", file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
        asets = [device_layer(make_layer_device(SEED_PREFILL + 100 * s, T, H, I, E, zipf_s=ZIPF_S,
                                                device=dev, with_x=False, affine=True))
                 for s in range(args.affine_sets)]
        for w in asets:
            step(w)
        torch.cuda.synchronize()
        a_ffn_us = phases([(w, shape) for w in asets], x, r, ws, h, y)[1] * 1e3
        ag = capture(asets)
        for _ in range(-(-MIN_WARMUP // len(asets))):  # MIN_WARMUP steps of warmup, back to back
            ag.replay()
        areps = 4
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(areps):
            ag.replay()
        a1.record()
        torch.cuda.synchronize()
        a_us = a0.elapsed_time(a1) / (areps * len(asets)) * 1e3
        affine = {"workload": "prefill2048_zipf_affine: the headline layer with every group's bias "
                              "b = -8 s + d, d ~ U(-2 s, 2 s) (rank-G bias term in every GEMM item)",
                  "us_per_step": round(a_us, 2), "tokens_per_s": round(T / (a_us * 1e-6), 1),
                  "ffn_kernel_us": round(a_ffn_us, 2),
                  "ffn_mfma_frac": round(flops_ffn / (a_ffn_us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12), 4),
                  "weight_sets": len(asets)}
        del ag, asets
        torch.cuda.empty_cache()
    else:
        del sets

    # ---------------- decode: T=1 ----------------
    # One weight set per layer of a 40-layer decode stack.  (i) decode-path bandwidth: one
    # moe_decode per layer on that layer's own token, independent calls in one HIP graph;
    # (ii) the chained stack: every layer decodes the previous layer's output after the
    # residual add and RMSNorm, 40 layers in one HIP graph with no host synchronisation.
    print(f"[bench] decode with {args.decode_sets} weight sets", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    dshape = moe.Shape(T=1, H=H, I=I, E=E, top_k=K_TOP)
    dsets = []
    for s in range(args.decode_sets):
        d = make_layer_device(SEED_DECODE + s, 1, H, I, E, zipf_s=None, device=dev)
        dsets.append((d["x"], device_layer(d)))
    dws = moe.workspace(dshape, dev)
    ids = torch.empty(K_TOP, dtype=torch.int32, device=dev)
    tw = torch.empty(K_TOP, dtype=torch.float32, device=dev)
    yd = torch.empty(H, dtype=torch.float32, device=dev)
    for i in range(10):
        xd, wd = dsets[i % len(dsets)]
        moe.moe_decode(dshape, xd, wd, ids, tw, yd, dws)
    torch.cuda.synchronize()

    def graph_us_per_layer(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / (reps * len(dsets)) * 1e3

    def independent():
        for xd, wd in dsets:
            moe.moe_decode(dshape, xd, wd, ids, tw, yd, dws)

    dreps = max(1, args.decode_steps // len(dsets))
    dec_us = graph_us_per_layer(independent, dreps)
    dec_bytes = 9 * expert_bytes(H, I) + E * H * 2 + H * 2 + H * 4 + K_TOP * 8
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9

    dres = torch.empty(H, dtype=torch.float32, device=dev)
    du = torch.empty(H, dtype=torch.int16, device=dev)
    dx0 = dsets[0][0].view(H)

    def chained_separate():
        # r_0 = x, u_0 = x; every layer: y = MoE(u); r += y; u = bf16(RMSNorm(r))
        dres.copy_(dx0.view(torch.bfloat16))
        du.copy_(dx0)
        for _, wd in dsets:
            moe.moe_decode(dshape, du, wd, ids, tw, yd, dws)
            moe.moe_rmsnorm_residual(1, H, 1e-6, dres, yd, du)

    def chained():
        # the same recurrence with the residual add and RMSNorm folded into each later
        # layer's router pass (moe_decode_residual); the last add + norm ends the pass
        dres.copy_(dx0.view(torch.bfloat16))
        moe.moe_decode(dshape, dx0, dsets[0][1], ids, tw, yd, dws)
        for _, wd in dsets[1:]:
            moe.moe_decode_residual(dshape, dres, yd, 1e-6, du, wd, ids, tw, yd, dws)
        moe.moe_rmsnorm_residual(1, H, 1e-6, dres, yd, du)

    dsep_us = graph_us_per_layer(chained_separate, dreps)
    dstack_us = graph_us_per_layer(chained, dreps)
    dstack = {"workload": f"decode_stack{len(dsets)}: {len(dsets)} MoE layers at T=1 chained "
                          f"through the residual add + RMSNorm (folded into each later layer's "
                          f"router pass), independent weights per layer",
              "us_per_layer": round(dstack_us, 2),
              "us_per_layer_separate_norm_kernel": round(dsep_us, 2),
              "hbm_gbs": round(dec_bytes / (dstack_us * 1e-6) / 1e9, 1),
              "hbm_frac": round(dec_bytes / (dstack_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
              "tokens_per_s": round(1.0 / (dstack_us * 1e-6 * len(dsets)), 1),
              "host_syncs_per_pass": 0}

    # small decode batches (T = 2, 4, 8 tokens per call, e.g. a verify step): one call per
    # layer, independent calls in one HIP graph.  Bandwidth is counted over the union of the
    # experts the call's tokens picked (each read once), the shared expert, the router rows,
    # x and y.
    dbatch = {}
    gx = torch.Generator(device=dev)
    gx.manual_seed(SEED_DECODE + 999)
    xb = torch.randn((8, H), generator=gx, device=dev).to(torch.bfloat16).view(torch.int16)
    for Tb in (2, 4, 8):
        bshape = moe.Shape(T=Tb, H=H, I=I, E=E, top_k=K_TOP)
        bws = moe.workspace(bshape, dev)
        bids = torch.empty((len(dsets), Tb, K_TOP), dtype=torch.int32, device=dev)
        btw = torch.empty((Tb, K_TOP), dtype=torch.float32, device=dev)
        by = torch.empty((Tb, H), dtype=torch.float32, device=dev)
        xT = xb[:Tb].contiguous()

        def batched():
            for li, (_, wd) in enumerate(dsets):
                moe.moe_decode(bshape, xT, wd, bids[li], btw, by, bws)

        b_us = graph_us_per_layer(batched, dreps)
        uniq = [len(set(bids[li].flatten().tolist())) for li in range(len(dsets))]
        b_bytes = ((sum(uniq) / len(uniq) + 1) * expert_bytes(H, I) + E * H * 2 + Tb * H * 2
                   + Tb * H * 4 + Tb * K_TOP * 8)
        dbatch[f"T{Tb}"] = {"us_per_call": round(b_us, 2), "tokens_per_s": round(Tb / (b_us * 1e-6), 1),
                            "distinct_experts_mean": round(sum(uniq) / len(uniq), 2),
                            "bytes_per_call": round(b_bytes),
                            "hbm_gbs": round(b_bytes / (b_us * 1e-6) / 1e9, 1),
                            "hbm_frac": round(b_bytes / (b_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del bws, bids, btw, by
    del dsets, dres, du
    torch.cuda.empty_cache()

    # ---------------- prefill T=2048 on one GPU's expert-parallel share ----------------
    # Under expert parallelism over 8 GPUs each GPU owns 32 experts and, after the dispatch
    # all-to-all, runs their rows: 8 GPUs x 2048 tokens x 8 picks x 32/256 = 16384 rows, 512 per
    # expert.  Here 2048 tokens pick among 32 experts only (router bias), which gives each of
    # them the same 512 rows; the shared expert runs the GPU's own 2048 tokens, as it would.
    ep = None
    if args.ep_share_sets:
        print(f"[bench] T={T} expert-parallel share (32 experts), {args.ep_share_sets} weight sets",
              file=sys.stderr, flush=True)
        raw = make_layer_device(SEED_EP_SHARE, T, H, I, E, device=dev, ep_share=8)
        xe = raw["x"]
        esets = [device_layer(raw)]
        del raw
        for s_ in range(1, args.ep_share_sets):
            esets.append(device_layer(make_layer_device(SEED_EP_SHARE + 100 * s_, T, H, I, E, device=dev,
                                                        with_x=False, ep_share=8)))

        def estep(w):
            moe.moe_route(shape, xe, w, r, ws)
            moe.moe_expert_ffn_q4(shape, xe, w, r, h, y, ws)

        for w in esets:
            estep(w)
        torch.cuda.synchronize()
        e_active = int((r.counts > 0).sum().item())
        e_max = int(r.counts.max().item())
        EK = 12
        _, e_ffn_ms, e_comb_ms = phases([(esets[s_ % len(esets)], shape) for s_ in range(EK)], xe, r,
                                        ws, h, y)
        eg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(eg):
            for w in esets:
                estep(w)
        for _ in range(-(-MIN_WARMUP // len(esets))):  # MIN_WARMUP steps of warmup, back to back
            eg.replay()
        ereps = max(1, 24 // len(esets))
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a_.record()
        for _ in range(ereps):
            eg.replay()
        b_.record()
        torch.cuda.synchronize()
        e_us = a_.elapsed_time(b_) / (ereps * len(esets)) * 1e3
        erows = T * K_TOP + T
        e_fl_gu = 2.0 * erows * (2 * I) * H
        e_fl_dn = 2.0 * erows * I * H
        ep = {"workload": f"prefill{T}_ep8_share: one GPU's share under expert parallelism over 8 GPUs, "
                          f"T={T} tokens picking among 32 experts (router bias), {erows - T} routed rows, "
                          f"{e_active} experts active, at most {e_max} rows per expert",
              "us_per_step": round(e_us, 2), "tokens_per_s": round(T / (e_us * 1e-6), 1),
              "ffn_kernel_us": round(e_ffn_ms * 1e3, 2),
              "ffn_mfma_frac": round((e_fl_gu + e_fl_dn) / (e_ffn_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
              "combine_us": round(e_comb_ms * 1e3, 2),
              "layer_mfma_frac": round((e_fl_gu + e_fl_dn) / (e_us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12), 4),
              "weight_sets": len(esets)}
        del eg, esets, xe
        torch.cuda.empty_cache()

    # ---------------- prefill T=512, uniform-ish routing: every expert is active ----------------
    uni = None
    if args.uniform_sets:
        Tu = 512
        print(f"[bench] T={Tu} uniform routing, {args.uniform_sets} weight sets", file=sys.stderr,
              flush=True)
        ushape = moe.Shape(T=Tu, H=H, I=I, E=E, top_k=K_TOP)
        raw = make_layer_device(SEED_UNIFORM, Tu, H, I, E, zipf_s=None, device=dev)
        xu = raw["x"]
        usets = [device_layer(raw)]
        del raw
        for s in range(1, args.uniform_sets):
            usets.append(device_layer(make_layer_device(SEED_UNIFORM + 100 * s, Tu, H, I, E,
                                                        zipf_s=None, device=dev, with_x=False)))
        ur = moe.Routing(ushape, dev, with_logits=False)
        uws = moe.workspace(ushape, dev)
        uh = torch.empty((Tu * K_TOP + Tu, I), dtype=torch.int16, device=dev)
        uy = torch.empty((Tu, H), dtype=torch.float32, device=dev)

        def ustep(w):
            moe.moe_route(ushape, xu, w, ur, uws)
            moe.moe_expert_ffn_q4(ushape, xu, w, ur, uh, uy, uws)

        for w in usets:
            ustep(w)
        torch.cuda.synchronize()
        active = int((ur.counts > 0).sum().item())
        ug = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ug):
            for w in usets:
                ustep(w)
        for _ in range(-(-MIN_WARMUP // len(usets))):  # MIN_WARMUP steps of warmup, back to back
            ug.replay()
        ureps = max(1, 24 // len(usets))
        u0 = torch.cuda.Event(enable_timing=True)
        u1 = torch.cuda.Event(enable_timing=True)
        u0.record()
        for _ in range(ureps):
            ug.replay()
        u1.record()
        torch.cuda.synchronize()
        u_us = u0.elapsed_time(u1) / (ureps * len(usets)) * 1e3
        # algorithmic bytes: the active experts' and the shared expert's packed weights,
        # the router weights, x (bf16) and y (fp32)
        u_bytes = (active + 1) * expert_bytes(H, I) + E * H * 2 + Tu * H * 2 + Tu * H * 4
        u_gbs = u_bytes / (u_us * 1e-6) / 1e9
        uni = {"workload": f"prefill{Tu}_uniform: one MoE layer, T={Tu}, random router, "
                           f"{active} of {E} experts active",
               "us_per_step": round(u_us, 2), "tokens_per_s": round(Tu / (u_us * 1e-6), 1),
               "bytes_per_step": u_bytes, "hbm_gbs": round(u_gbs, 1),
               "hbm_frac": round(u_gbs / PEAK_HBM_GBS, 4), "weight_sets": len(usets)}
        del ug, usets, ur, uws, uh, uy, xu
        torch.cuda.empty_cache()

    # ---------------- long prompt: chunked prefill vs one call ----------------
    chunked = None
    if args.chunked_tokens:
        Tl, Cl = args.chunked_tokens, 2048
        print(f"[bench] T={Tl} prompt in chunks of {Cl}", file=sys.stderr, flush=True)
        lshape = moe.Shape(T=Tl, H=H, I=I, E=E, top_k=K_TOP)
        raw = make_layer_device(SEED_UNIFORM + 7, Tl, H, I, E, zipf_s=None, device=dev)
        xl = raw["x"]
        wl = device_layer(raw)
        del raw
        yl = torch.empty((Tl, H), dtype=torch.float32, device=dev)
        cws = moe.workspace_chunked(lshape, Cl, dev)

        def timed(fn, reps=4):
            fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        c_ms = timed(lambda: moe.moe_layer_chunked(lshape, xl, wl, yl, Cl, cws))
        lr = moe.Routing(lshape, dev, with_logits=False)
        lws = moe.workspace(lshape, dev)
        lh = torch.empty((Tl * K_TOP + Tl, I), dtype=torch.int16, device=dev)
        f_ms = timed(lambda: moe.moe_layer(lshape, xl, wl, lr, lh, yl, lws))
        whole_bytes = lws.numel() + sum(t.numel() * t.element_size() for t in
                                        (lh, lr.topk_ids, lr.topk_w, lr.counts, lr.offsets,
                                         lr.row_token, lr.tok_row, lr.row_w, lr.blocks))
        chunked = {"workload": f"prefill{Tl}: one MoE layer over a {Tl}-token prompt, random "
                               f"router, in chunks of {Cl} tokens",
                   "chunk": Cl, "ms": round(c_ms, 3), "tokens_per_s": round(Tl / (c_ms * 1e-3), 1),
                   "workspace_bytes": cws.numel(),
                   "single_call_ms": round(f_ms, 3),
                   "single_call_tokens_per_s": round(Tl / (f_ms * 1e-3), 1),
                   "single_call_scratch_bytes": whole_bytes}
        del wl, xl, yl, cws, lr, lws, lh
        torch.cuda.empty_cache()

    # ---------------- 40-layer stack at T=4096: residual + RMSNorm between layers ----------------
    stack = None
    if args.stack_layers:
        Ts, L = 4096, args.stack_layers
        print(f"[bench] stack of {L} layers at T={Ts}", file=sys.stderr, flush=True)
        sshape = moe.Shape(T=Ts, H=H, I=I, E=E, top_k=K_TOP)
        x0 = make_layer_device(SEED_STACK, Ts, H, I, E, device=dev)["x"]
        layers = [device_layer(make_layer_device(SEED_STACK + l, Ts, H, I, E, device=dev,
                                                 with_x=False)) for l in range(L)]
        sr = moe.Routing(sshape, dev, with_logits=False)
        sws = moe.workspace(sshape, dev)
        sh_ = torch.empty((Ts * K_TOP + Ts, I), dtype=torch.int16, device=dev)
        sy = torch.empty((Ts, H), dtype=torch.float32, device=dev)
        res = torch.empty((Ts, H), dtype=torch.float32, device=dev)
        u = torch.empty_like(x0)

        def stack_pass():
            # r_0 = x, u_0 = x; every layer: y = MoE(u); r += y; u = bf16(RMSNorm(r))
            res.copy_(x0.view(torch.bfloat16))
            u.copy_(x0)
            for w in layers:
                moe.moe_route(sshape, u, w, sr, sws)
                # both GEMMs in one launch (y: the shared expert's part), then the combine with
                # the residual add and RMSNorm: the combined rows are added to the residual as
                # they are formed
                moe.moe_expert_ffn_q4(sshape, u, w, sr, sh_, sy, sws, combine=False)
                moe.moe_combine_residual(sshape, sr, sy, res, 1e-6, u, sws)

        stack_pass()
        torch.cuda.synchronize()
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg):
            stack_pass()
        sg.replay()
        torch.cuda.synchronize()
        sg.replay()                                    # a pass of warmup, back to back
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        sreps = 3
        s0.record()
        for _ in range(sreps):
            sg.replay()
        s1.record()
        torch.cuda.synchronize()
        s_ms = s0.elapsed_time(s1) / sreps
        srows = Ts * K_TOP + Ts
        s_flops = L * 2.0 * srows * 3 * I * H
        stack = {"workload": f"stack{L}_T{Ts}: {L} MoE layers with residual add + RMSNorm between "
                             f"them, T={Ts}, random routers, independent weights per layer",
                 "ms_per_pass": round(s_ms, 3), "us_per_layer": round(s_ms * 1e3 / L, 2),
                 "tokens_per_s": round(Ts / (s_ms * 1e-3), 1),
                 "layer_mfma_frac": round(s_flops / (s_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                 "host_syncs_per_pass": 0}
        del sg, layers, sr, sws, sh_, sy, res, u, x0
        torch.cuda.empty_cache()

    # ---------------- CPU oracle baseline (rank 0, N=1) ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        from synth.device import to_host_inputs
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        inp = to_host_inputs(raw0, T, H, I, E, K_TOP)
        L = oracle.Layer(inp)
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        L.tokens(list(range(cores)))                       # calibration
        per_tok = (time.perf_counter() - t0) / cores
        n = int(max(cores, min(T, args.cpu_seconds / max(per_tok, 1e-6))))
        rng = np.random.default_rng(0)
        toks = sorted(rng.choice(T, size=n, replace=False).tolist())
        t0 = time.perf_counter()
        L.tokens(toks)
        dt = time.perf_counter() - t0
        # one thread, on a sample of about a sixth of that time
        oracle.set_threads(1)
        n1 = max(1, min(n, int(n / cores * 2)))
        t0 = time.perf_counter()
        L.tokens(toks[:n1])
        dt1 = time.perf_counter() - t0
        oracle.set_threads(cores)
        cpu = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} of the {T} tokens of the same layer (weight set 0), full per-token "
                         f"path: router over 256 experts, top-8, 9 SwiGLU experts in float64; "
                         f"{dt:.1f} s wall",
               "single_thread": {"value": round(n1 / dt1, 3), "unit": "tokens/s", "cores": 1,
                                 "sample": f"the first {n1} of those tokens, {dt1:.1f} s wall"}}

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm_steps,
        "warmup_requested": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_us": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the expert GEMMs run on fp16 MFMA (weights rebuilt exactly as (q-8)*s in fp16, bf16
        # activations converted exactly) with fp32 accumulation; inputs and the router are bf16
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "prefill2048_zipf: one MoE layer, T=2048 tokens, H=2048, I=512, "
                               "256 experts top-8 + shared expert, 4-bit affine g=64 weights, "
                               "Zipf(1.1) router bias",
                   "T": T, "H": H, "I": I, "E": E, "top_k": K_TOP, "weight_sets": args.sets,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma",
                     "kernel": "q4_ffn_kernel (gate/up + SwiGLU + down in one persistent launch, "
                               "fp16 MFMA)",
                     "achieved": round(ffn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ffn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": ffn_traffic_bytes(), "avg_launch_us": round(ffn_ms * 1e3, 2),
                     "flops_per_launch": flops_ffn},
        "layer_mfma_frac": round(layer_mfma_frac, 4),
        "phase_us": {"route": round(route_ms * 1e3, 2), "ffn_kernel": round(ffn_ms * 1e3, 2),
                     "combine": round(comb_ms * 1e3, 2)},
        "two_launch": two_launch,
        "wall_s": round(wall, 3),
        "prefill2048_zipf_affine": affine,
        "prefill2048_ep8_share": ep,
        "decode": {"metric": "T=1 decode HBM GB/s", "value": round(dec_gbs, 1), "unit": "GB/s",
                   "frac_of_peak": round(dec_gbs / PEAK_HBM_GBS, 4), "us_per_call": round(dec_us, 2),
                   "bytes_per_call": dec_bytes, "weight_sets": args.decode_sets},
        "decode_stack": dstack,
        "decode_batch": dbatch,
        "prefill512_uniform": uni,
        "stack": stack,
        "prefill_chunked": chunked,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
