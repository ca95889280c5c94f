#!/usr/bin/env python
"""Benchmark of the FlowCache per-step hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs
already resident in HBM (the two parts are independent and run on two
streams):
  * fc_kv_compress on the long-video workload (24 heads, d=128, 8100
    denoising queries, 129600 clean keys = 16 chunks of 4 x 45 x 45 tokens,
    keep 32400 per head, lambda 0.5, pool window 7, bf16; the smooth-field
    keys of the generator with frames 48-63 copied from frames 16-31):
    importance (two MFMA passes, the redundancy fused into them), pool +
    score + top-B, K/V compaction;
  * fc_chunk_rel_l1_decide on 16 concurrent chunks of 64x8x90x160 bf16
    latents (steady state, all chunks active at staggered local steps).

Beside the step it times the stages on the same inputs, the lambda sweep
{0.3, 0.5, 0.7}, the MAGI-like and SkyReels-like compressions, a MAGI-like run
of the KV cache manager, and the oracle on the host cores (CPU baseline).

Prints one JSON line.  `value` is clean-KV token-heads scored and selected per
second over whole steps (the chunk decision included).  The roofline entry is
the importance stage (its three launches, timed with HIP events on the stream
they run on), with Q K^T counted once over both passes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "clean KV tokens scored+selected/sec/head; L1 GB/s; % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "importance_long_traffic.json")
CSRC = os.path.join(ROOT, "kv_cache_compression_fc_amd", "csrc")
TRAFFIC_SOURCES = ("importance.hip", "red_rows.hpp", "common.hpp")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the sources of the importance stage's kernels."""
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def time_events(fn, reps: int) -> float:
    """Average ms per call of fn over reps, HIP events on the current stream."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def time_paired_diff(fa, fb, pairs: int) -> float:
    """Median over pairs of (ms of one fa call - ms of the fb call right after
    it), HIP events around each call on the current stream: the clock drifts
    of a power-capped chip cancel inside a pair, which a difference of two
    separately timed averages does not."""
    import torch
    fa()
    fb()
    torch.cuda.synchronize()
    diffs = []
    for _ in range(pairs):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        fa()
        ev[1].record()
        fb()
        ev[2].record()
        ev[2].synchronize()
        diffs.append(ev[0].elapsed_time(ev[1]) - ev[1].elapsed_time(ev[2]))
    return statistics.median(diffs)


def time_cold(fn, reps: int, scratch):
    """Median ms per call with the 256 MB MALL (Infinity Cache) flushed first:
    before each call a 512 MB scratch buffer is read (a sum), which leaves only
    clean scratch lines in the MALL, so the call's own misses cost no
    write-back of the flush; then the call alone runs between two events.
    Eager launches: the host queues the call's kernels while the GPU is still
    reading the scratch buffer (about 80 us), so they start back to back; a
    graph replay would add its own launch latency inside the interval."""
    import torch
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    sink = torch.empty((), dtype=torch.float32, device=scratch.device)
    for s, e in evs:
        torch.sum(scratch, 0, out=sink)
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in evs), "eager"


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def cpu_info() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            return next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "unknown")
    except OSError:
        return "unknown"


def cpu_baseline(cfg, ccfg, min_seconds: float):
    """The oracle (never tuned) on a bounded sample of the same step: the
    whole fp64 compression of sampled heads of the long-video workload (the
    generator's values; importance in C + OpenMP, the rest in numpy), and the
    relative-L1 decision of all 16 chunks (numpy).  Heads are independent and
    equally sized, so a step costs H x (mean time per head) + the decision."""
    import oracle
    from kv_cache_compression_fc_amd import synth
    tr = synth.ChunkTrajectory(ccfg, seed=0)
    xt, xtm1, steps = tr.pair(ccfg.n_chunks - 1)
    offs = [i * ccfg.chunk_elems for i in range(ccfg.n_chunks + 1)]
    t0 = time.perf_counter()
    l1 = oracle.chunk_l1_rel(xt, xtm1, offs)
    f = [0.0] * ccfg.n_chunks
    for i, n in enumerate(steps):
        if n >= 0:
            _, f[i] = oracle.decide(n, f[i], l1[i], ccfg.m, ccfg.eps[0])
    t_dec = time.perf_counter() - t0
    del xt, xtm1, tr
    head_times = []
    h = 0
    while not head_times or sum(head_times) + t_dec < min_seconds:
        Q, K, V = synth.kv_inputs(cfg, seed=0, heads=[h])
        t0 = time.perf_counter()
        oracle.kv_compress(Q, K, V, cfg.B, 0.5, cfg.w)
        head_times.append(time.perf_counter() - t0)
        h = (h + 1) % cfg.H
    t_step = cfg.H * statistics.mean(head_times) + t_dec
    return {"value": cfg.H * cfg.Lk / t_step, "unit": "token-heads/s", "cores": oracle.num_threads(),
            "cpu": cpu_info(), "kind": "oracle", "seconds": sum(head_times) + t_dec,
            "step_seconds_estimated": t_step,
            "sample": f"{len(head_times)} of {cfg.H} long-video heads compressed whole in fp64 "
                      f"(L_q={cfg.Lq}, L_k={cfg.Lk}, B={cfg.B}, lambda 0.5; mean {statistics.mean(head_times):.2f} s "
                      f"per head, scaled by H={cfg.H}) plus the relative-L1 decision of {ccfg.n_chunks} chunks "
                      f"({t_dec:.2f} s)"}


def cache_run(fc, synth, dev, reps: int):
    """The MAGI-like cache run: chunks of 3600 tokens commit into a cache of
    7200 per head, each compression scored by 3600 queries.  Each chunk is
    first written into the active rows of the cache's current region (the
    producer's store, outside the timing), then committed in place; the run
    goes through once untimed, then again with every commit timed on the
    stream (HIP events), and the compressing commits (third chunk on) are
    averaged.  The same run with the chunk handed over from its own buffer
    (the commit copies it in first) is timed beside it, and the append-only
    commit (copy of one chunk behind the clean rows) on its own for the copy
    kernel's bandwidth."""
    import torch
    cfg = synth.CACHE_CONFIGS["magi"]
    log(f"generating the cache run: {cfg.n_chunks} chunks of {cfg.tokens_per_chunk} tokens, {cfg.H} heads")
    Q, K, V = synth.cache_inputs(cfg, seed=0)
    Q, K, V = Q.to(dev), K.to(dev), V.to(dev)
    T = cfg.tokens_per_chunk
    chunks = [(K[:, c * T:(c + 1) * T].contiguous(), V[:, c * T:(c + 1) * T].contiguous()) for c in range(cfg.n_chunks)]
    del K, V
    kv = fc.KvCache(cfg.H, cfg.d, cfg.B_budget, cfg.B_active, cfg.Lq, cfg.lam, cfg.w, torch.bfloat16, device=dev)

    def run(in_place: bool):
        times = []
        for _ in range(2):  # untimed pass, then the timed one (events only; the host runs ahead)
            kv.length, kv.next_pos, kv.cur = 0, 0, 0
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(cfg.n_chunks)]
            for c, (Kc, Vc) in enumerate(chunks):
                if in_place:
                    Ka, Va = kv.active(T)
                    Ka.copy_(Kc)
                    Va.copy_(Vc)
                ev[c][0].record()
                if in_place:
                    kv.commit(None, None, Q[c], L_c=T)
                else:
                    kv.commit(Kc, Vc, Q[c])
                ev[c][1].record()
            torch.cuda.synchronize()
            times = [a.elapsed_time(b) for a, b in ev]
        return [t for c, t in enumerate(times) if (c + 1) * T > cfg.B_budget]

    comp = run(True)
    comp_copy = run(False)
    merged = cfg.B_budget + T
    commit_ms = statistics.mean(comp)
    Kc, Vc = chunks[0]
    Bt = cfg.B_budget + cfg.B_active

    def append():
        fc.fc_cache_commit(kv.p, 0, Kc, Vc, 0, None, kv._K[0], kv._V[0], kv._pos[0], kv._K[1], kv._V[1], kv._pos[1],
                           kv.workspace)
    t_app = time_events(append, reps)
    app_bytes = 2 * 2 * cfg.H * T * cfg.d * 2 + cfg.H * T * 4      # K and V rows read + written, positions
    return {
        "workload": f"MAGI-like cache run: {cfg.H} heads, d={cfg.d}, {cfg.n_chunks} chunks of {T} tokens, "
                    f"budget {cfg.B_budget}, {cfg.Lq} queries per compression, lambda {cfg.lam}, bf16",
        "compressing_commits": len(comp), "commit_ms": commit_ms, "commit_ms_max": max(comp),
        "merged_token_heads_per_s": cfg.H * merged / (commit_ms * 1e-3),
        "commit_with_chunk_copy_ms": statistics.mean(comp_copy),
        "region_bytes": 2 * cfg.H * Bt * cfg.d * 2 + cfg.H * Bt * 4,
        "workspace_bytes": int(kv.workspace.numel()),
        "append_commit_ms": t_app, "append_gbps": app_bytes / (t_app * 1e-3) / 1e9,
    }


def other_shapes(fc, synth, dev, reps: int):
    """fc_kv_compress alone on the MAGI-like shape (the generator's values)
    and the SkyReels-like shape (seeded N(0,1) bf16 drawn on the device; its
    parity at this size is the tests' business): token-heads/s and the
    importance rate."""
    import torch
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for name in ("magi", "skyreels"):
        cfg = synth.KV_CONFIGS[name]
        H, Lq, Lk, d, B = cfg.H, cfg.Lq, cfg.Lk, cfg.d, cfg.B
        if name == "magi":
            Q, K, V = (x.to(dev) for x in synth.kv_inputs(cfg, seed=0, workers=workers()))
            data = "generator (smooth-field keys)"
        else:
            Q = torch.randn((H, Lq, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            K = torch.randn((H, Lk, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            V = torch.randn((H, Lk, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            data = "device-seeded N(0,1) bf16"
        lam = 0.5
        p = fc.kv_params(Q, K, B, lam, cfg.w)
        ws = torch.empty(fc.fc_kv_compress_workspace_bytes(p), dtype=torch.uint8, device=dev)
        o = {"K_out": torch.empty((H, B, d), dtype=K.dtype, device=dev),
             "V_out": torch.empty((H, B, d), dtype=V.dtype, device=dev),
             "idx": torch.empty((H, B), dtype=torch.int32, device=dev)}
        comp = lambda: fc.fc_kv_compress(Q, K, V, B, lam, cfg.w, out=o, workspace=ws)
        imp_o, r_o = (torch.empty((H, Lk), dtype=torch.float32, device=dev) for _ in range(2))
        imp_only = lambda: fc.fc_kv_importance_redundancy(Q, K, imp_out=imp_o, r_out=r_o, workspace=ws)
        t = time_events(comp, reps)
        t_imp = time_events(imp_only, reps)
        t_sel = time_paired_diff(comp, imp_only, max(reps, 10))
        flops = 2.0 * H * Lq * Lk * d   # Q K^T once
        out[name] = {"H": H, "L_q": Lq, "L_k": Lk, "B_budget": B, "compress_ms": t,
                     "token_heads_per_s": H * Lk / (t * 1e-3), "tokens_per_s_per_head": Lk / (t * 1e-3),
                     "importance_stage_ms": t_imp,
                     "importance_algorithmic_tflops": flops / (t_imp * 1e-3) / 1e12,
                     "select_gather_in_compress_ms": t_sel, "data": data}
        del Q, K, V, ws, o
        torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="minimum host time of the CPU-baseline (oracle) leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other shapes and the KV-cache run")
    ap.add_argument("--profile-importance", type=int, default=0, metavar="N",
                    help="only run the importance stage N times on the long-video inputs (for counter runs)")
    ap.add_argument("--loop-lse", type=float, default=0.0, metavar="SECONDS",
                    help="only run importance pass 1 on the long-video shape back to back for SECONDS "
                         "(to read the board's power and clocks meanwhile)")
    ap.add_argument("--profile-streaming", type=int, default=0, metavar="N",
                    help="only run the HBM-bound stages (stand-alone redundancy, chunk decision, select + "
                         "gather) N times each, the MALL flushed before every call (for kernel traces and "
                         "HBM counters)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) to calibrate HBM counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "the path shards by head with no exchange, so run one process per GPU.", file=sys.stderr)
        return 2

    import torch
    from kv_cache_compression_fc_amd import binding as fc
    from kv_cache_compression_fc_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    if args.calib_copy:
        n = 1 << 30
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 3}), flush=True)
        return 0

    cfg = synth.KV_CONFIGS["long"]
    ccfg = synth.CHUNK_CONFIGS["scale"]
    H, Lq, Lk, d, B, w = cfg.H, cfg.Lq, cfg.Lk, cfg.d, cfg.B, cfg.w
    lam = 0.5
    Bp = min(B, Lk)
    log(f"generating inputs: {cfg.name} KV workload ({workers()} threads)")
    t0 = time.perf_counter()
    Q, K, V = synth.kv_inputs(cfg, seed=0, workers=workers())
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    del Q, K, V
    log(f"  {time.perf_counter() - t0:.1f} s")
    p = fc.kv_params(Qd, Kd, B, lam, w)
    ws = torch.empty(fc.fc_kv_compress_workspace_bytes(p), dtype=torch.uint8, device=dev)

    if args.profile_importance > 0:
        imp = torch.empty((H, Lk), dtype=torch.float32, device=dev)
        r = torch.empty((H, Lk), dtype=torch.float32, device=dev)
        for _ in range(args.profile_importance):
            fc.fc_kv_importance_redundancy(Qd, Kd, imp_out=imp, r_out=r, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile_importance_calls": args.profile_importance}), flush=True)
        return 0
    if args.loop_lse > 0:
        lse = fc.fc_kv_importance_lse(Qd, Kd, workspace=ws)
        torch.cuda.synchronize()
        log("loop start")
        t0, calls = time.perf_counter(), 0
        while time.perf_counter() - t0 < args.loop_lse:
            for _ in range(5):
                fc.fc_kv_importance_lse(Qd, Kd, lse_out=lse, workspace=ws)
            torch.cuda.synchronize()
            calls += 5
        dt = time.perf_counter() - t0
        print(json.dumps({"loop_lse_calls": calls, "ms_per_call": 1e3 * dt / calls}), flush=True)
        return 0

    log(f"generating {ccfg.n_chunks} chunk states")
    tr = synth.ChunkTrajectory(ccfg, seed=0)
    g_steady = ccfg.n_chunks - 1  # every chunk active, local steps 15..0
    xt, xtm1, steps = tr.pair(g_steady)
    xt_d, xtm1_d = xt.to(dev), xtm1.to(dev)
    del xt, xtm1, tr
    offs_c = [i * ccfg.chunk_elems for i in range(ccfg.n_chunks + 1)]
    dec = fc.ChunkDecider(offs_c, ccfg.m, ccfg.eps[0], torch.bfloat16, dev)
    dec.step.copy_(torch.tensor(steps, dtype=torch.int32))
    if args.profile_streaming > 0:
        scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MB, read before each call
        sink = torch.empty((), dtype=torch.float32, device=dev)
        r = torch.empty((H, Lk), dtype=torch.float32, device=dev)
        imp, r_sel = fc.fc_kv_importance_redundancy(Qd, Kd, workspace=ws)
        for _ in range(args.profile_streaming):
            torch.sum(scratch, 0, out=sink)
            fc.fc_kv_redundancy(Kd, r_out=r, workspace=ws)
            torch.sum(scratch, 0, out=sink)
            dec.decide(xt_d, xtm1_d)
            torch.sum(scratch, 0, out=sink)
            fc.fc_kv_select(imp, r_sel, B, lam, w, Kd, Vd, want_scores=False, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile_streaming_calls": args.profile_streaming}), flush=True)
        return 0

    out = {"K_out": torch.empty((H, Bp, d), dtype=Kd.dtype, device=dev),
           "V_out": torch.empty((H, Bp, d), dtype=Vd.dtype, device=dev),
           "idx": torch.empty((H, Bp), dtype=torch.int32, device=dev)}

    # The two parts of a step are independent (the cache's keys vs the chunks'
    # latents): the decision runs on a second stream (default priority),
    # forked at the start of the step and joined at its end, so its HBM
    # traffic overlaps the compression's compute.
    side = torch.cuda.Stream(device=dev)
    main_s = torch.cuda.current_stream()

    def step():
        side.wait_stream(main_s)
        with torch.cuda.stream(side):
            dec.decide(xt_d, xtm1_d, stream=side)
        fc.fc_kv_compress(Qd, Kd, Vd, B, lam, w, out=out, workspace=ws)
        main_s.wait_stream(side)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log(f"ms/step {ms_per_step:.4f} (wall {1e3 * wall / args.steps:.4f})")

    # Stages on the same inputs, same stream, HIP events.
    reps = args.kernel_reps
    imp = torch.empty((H, Lk), dtype=torch.float32, device=dev)
    r = torch.empty((H, Lk), dtype=torch.float32, device=dev)
    lse = torch.empty((H, Lq), dtype=torch.float32, device=dev)
    # the importance stage exactly as the step runs it: pass 1 with redundancy
    # pass A, the merge, pass 2 with redundancy pass B
    t_imp = time_events(lambda: fc.fc_kv_importance_redundancy(Qd, Kd, imp_out=imp, r_out=r, workspace=ws), reps)
    # the two passes alone (without the redundancy), for the per-pass rates
    t_lse = time_events(lambda: fc.fc_kv_importance_lse(Qd, Kd, lse_out=lse, workspace=ws), reps)
    t_colsum = time_events(lambda: fc.fc_kv_importance_colsum(Qd, Kd, lse, imp_out=imp, workspace=ws), reps)
    # what the redundancy adds inside the importance stage (pass A in pass 1's
    # launch, pass B in pass 2's): the stage minus the two passes without it,
    # timed in alternating pairs
    imp_plain = torch.empty_like(imp)

    def passes_alone():
        fc.fc_kv_importance_lse(Qd, Kd, lse_out=lse, workspace=ws)
        fc.fc_kv_importance_colsum(Qd, Kd, lse, imp_out=imp_plain, workspace=ws)
    t_red_in = time_paired_diff(lambda: fc.fc_kv_importance_redundancy(Qd, Kd, imp_out=imp, r_out=r, workspace=ws),
                                passes_alone, max(reps, 10))
    fc.fc_kv_importance_redundancy(Qd, Kd, imp_out=imp, r_out=r, workspace=ws)
    t_red = time_events(lambda: fc.fc_kv_redundancy(Kd, r_out=torch.empty_like(r), workspace=ws), reps)
    t_sel = time_events(lambda: fc.fc_kv_select(imp, r, B, lam, w, Kd, Vd, want_scores=False, workspace=ws), reps)
    t_sel_idx = time_events(lambda: fc.fc_kv_select(imp, r, B, lam, w, want_scores=False, workspace=ws), reps)
    sweep = {}
    for lam_s in cfg.lam:
        t_c = time_events(lambda: fc.fc_kv_compress(Qd, Kd, Vd, B, lam_s, w, out=out, workspace=ws), reps)
        sweep[str(lam_s)] = {"compress_ms": t_c, "token_heads_per_s": H * Lk / (t_c * 1e-3)}
    t_compress = sweep[str(lam)]["compress_ms"]
    t_l1 = time_events(lambda: dec.decide(xt_d, xtm1_d), reps)
    n_ch = ccfg.n_chunks
    p_pol = fc.fc_l1_params(n_ch, ccfg.m, ccfg.eps[0], fc.FC_BF16)
    cstep = torch.tensor(steps, dtype=torch.int32, device=dev)
    st_na, f_na = cstep.clone(), torch.zeros(n_ch, device=dev)
    rec_na = torch.zeros(n_ch, dtype=torch.uint8, device=dev)
    t_noalloc = time_events(lambda: fc.fc_chunk_rel_l1_decide_noalloc(p_pol, offs_c, xt_d, xtm1_d, st_na, f_na, rec_na),
                            reps)
    ws_pol = torch.empty(fc.fc_chunk_rel_l1_workspace_bytes(p_pol, offs_c), dtype=torch.uint8, device=dev)
    gstep = torch.zeros(1, dtype=torch.int32, device=dev)
    f_u, l1_u = torch.zeros(1, device=dev), torch.zeros(1, device=dev)
    rec_u = torch.zeros(n_ch, dtype=torch.uint8, device=dev)
    t_uni = time_events(lambda: fc.fc_uniform_rel_l1_decide(p_pol, offs_c, xt_d, xtm1_d, cstep, gstep, f_u, rec_u,
                                                            l1_u, ws_pol), reps)
    hstep = torch.tensor(steps, dtype=torch.int32, device=dev)
    acc_h, dev_h = torch.zeros(n_ch, device=dev), torch.zeros(n_ch, device=dev)
    ref_h = torch.zeros(n_ch, dtype=torch.uint8, device=dev)
    t_hist = time_events(lambda: fc.fc_history_rel_l1_decide(p_pol, offs_c, xt_d, xtm1_d, hstep, acc_h, ref_h,
                                                             dev_h, ws_pol), reps)
    # the HBM-bound stages again with the MALL flushed before every call
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MB
    t_red_c, _ = time_cold(lambda: fc.fc_kv_redundancy(Kd, r_out=torch.empty_like(r), workspace=ws), reps, scratch)
    t_sel_c, _ = time_cold(lambda: fc.fc_kv_select(imp, r, B, lam, w, Kd, Vd, want_scores=False, workspace=ws),
                           reps, scratch)
    t_l1_c, how_cold = time_cold(lambda: dec.decide(xt_d, xtm1_d), reps, scratch)
    del scratch
    # the fused variant: Euler update X_{t-1} = X_t + v dt and the decision in
    # one pass, in place, on the same 16 chunks (velocity: the path's own)
    v_d = synth.ChunkTrajectory(ccfg, seed=0).velocity().to(dev)
    x_work = xt_d.clone()
    dts = torch.full((ccfg.n_chunks,), -1e-4, dtype=torch.float32, device=dev)
    dec_fused = fc.ChunkDecider(offs_c, ccfg.m, ccfg.eps[0], torch.bfloat16, dev)
    dec_fused.step.copy_(torch.tensor(steps, dtype=torch.int32))   # every chunk active; the counters advance
    t_fused = time_events(lambda: dec_fused.euler_step(x_work, v_d, dts, x_work), reps)
    del v_d, x_work
    torch.cuda.synchronize()

    qk_flops = 2.0 * H * Lq * Lk * d              # one Q K^T product (the method's own work)
    red_bytes = H * Lk * (d * 2 + 4)              # read K once, write r
    red_exec_bytes = H * Lk * (2 * d * 2 + 4)     # the two passes: K read twice, r written
    sel_bytes = 8 * H * Lk + 4 * H * Bp + 2 * 2 * H * Bp * d * 2   # imp + r, idx, K/V rows read + written
    l1_bytes = 2 * ccfg.n_chunks * ccfg.chunk_elems * 2             # both states, bf16
    fused_bytes = 3 * ccfg.n_chunks * ccfg.chunk_elems * 2          # X_t and v read, X_{t-1} written
    imp_tflops = qk_flops / (t_imp * 1e-3) / 1e12
    # the selection and gather inside the compression: the compression minus
    # its importance stage, timed in alternating pairs
    sel_in_step = time_paired_diff(lambda: fc.fc_kv_compress(Qd, Kd, Vd, B, lam, w, out=out, workspace=ws),
                                   lambda: fc.fc_kv_importance_redundancy(Qd, Kd, imp_out=imp, r_out=r, workspace=ws),
                                   max(reps, 10))
    stages = {
        "importance_stage_ms": t_imp, "importance_algorithmic_tflops": imp_tflops,
        "importance_executed_tflops": 2 * imp_tflops,
        "importance_pass1_ms": t_lse, "importance_pass1_tflops": qk_flops / (t_lse * 1e-3) / 1e12,
        "importance_pass2_ms": t_colsum, "importance_pass2_tflops": qk_flops / (t_colsum * 1e-3) / 1e12,
        "select_gather_in_compress_ms": sel_in_step,
        "select_gather_in_compress_gbps": sel_bytes / (sel_in_step * 1e-3) / 1e9,
        "select_gather_ms": t_sel, "select_gather_gbps": sel_bytes / (t_sel * 1e-3) / 1e9,
        "select_indices_only_ms": t_sel_idx,
        "redundancy_standalone_ms": t_red, "redundancy_standalone_gbps": red_bytes / (t_red * 1e-3) / 1e9,
        "redundancy_standalone_executed_gbps": red_exec_bytes / (t_red * 1e-3) / 1e9,
        "redundancy_in_importance_ms": t_red_in,
        "redundancy_in_importance_gbps": red_bytes / (t_red_in * 1e-3) / 1e9 if t_red_in > 0 else None,
        "compress_ms": t_compress, "chunk_l1_ms": t_l1, "chunk_l1_gbps": l1_bytes / (t_l1 * 1e-3) / 1e9,
        "chunk_l1_noalloc_ms": t_noalloc, "chunk_l1_noalloc_gbps": l1_bytes / (t_noalloc * 1e-3) / 1e9,
        "euler_l1_fused_ms": t_fused, "euler_l1_fused_gbps": fused_bytes / (t_fused * 1e-3) / 1e9,
        "uniform_l1_ms": t_uni, "uniform_l1_gbps": l1_bytes / (t_uni * 1e-3) / 1e9,
        "history_l1_ms": t_hist, "history_l1_gbps": l1_bytes / (t_hist * 1e-3) / 1e9,
        "mall_flushed": {
            "redundancy_standalone_ms": t_red_c, "redundancy_standalone_gbps": red_bytes / (t_red_c * 1e-3) / 1e9,
            "redundancy_standalone_executed_gbps": red_exec_bytes / (t_red_c * 1e-3) / 1e9,
            "per_pass": "profiles/streaming_long_kernel_trace.md (bench.py --profile-streaming under a kernel trace)",
            "select_gather_ms": t_sel_c, "select_gather_gbps": sel_bytes / (t_sel_c * 1e-3) / 1e9,
            "chunk_l1_ms": t_l1_c, "chunk_l1_gbps": l1_bytes / (t_l1_c * 1e-3) / 1e9,
        },
        "lambda_sweep": sweep,
        "timing": f"HIP events on the launch stream, {reps} calls each; mall_flushed: 512 MB read before each "
                  f"call, {how_cold} launches, median; select_gather includes the redundancy softmax "
                  f"statistics kernel that fc_kv_compress takes from pass 2 instead; "
                  f"select_gather_in_compress: median over alternating pairs of (compression - its "
                  f"importance stage); redundancy_in_importance: likewise (importance stage - its two passes "
                  f"without the redundancy)",
    }
    for k, v in stages.items():
        log(f"  {k}: {v}")

    others = cache = None
    if not args.no_extras:
        del Qd, Kd, Vd, ws, out, imp, r, lse
        torch.cuda.empty_cache()
        others = other_shapes(fc, synth, dev, reps)
        for k, v in others.items():
            log(f"  {k}: {v}")
        cache = cache_run(fc, synth, dev, reps)
        for k, v in cache.items():
            log(f"  cache {k}: {v}")

    traffic = traffic_rec = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("kernel_source_sha256_16") == source_hash():
            traffic = rec.get("hbm_bytes_per_stage")
            traffic_rec = {k: rec[k] for k in ("per_kernel", "fetch_factor", "write_factor") if k in rec}

    result = {
        "metric": METRIC,
        "value": H * Lk / (ms_per_step * 1e-3),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth-field keys with repeated chunks, N(0,1) queries/values; "
                "flow-matching chunk trajectories)",
        "config": {
            "workload": "long-video KV compression + chunk relative-L1 decision",
            "H": H, "d": d, "L_q": Lq, "L_k": Lk, "B_budget": B, "lambda": lam, "pool_window": w,
            "duplicated_frames": [list(cfg.dup[1]), "copied from", list(cfg.dup[0])],
            "chunks": ccfg.n_chunks, "chunk_shape": [64, 8, 90, 160], "m": ccfg.m, "eps": ccfg.eps[0],
        },
        "tokens_per_s_per_head": Lk / (ms_per_step * 1e-3),
        "l1_gbps": l1_bytes / (t_l1 * 1e-3) / 1e9,
        "roofline": {
            "kernel": "importance stage: imp_lse_kernel (pass 1 + redundancy pass A) + imp_lse_merge_kernel + "
                      "imp_colsum_kernel (pass 2 + redundancy pass B)",
            "bound": "mfma", "achieved": imp_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": imp_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
            "executed_frac": 2 * imp_tflops / PEAK_BF16_TFLOPS,
            "avg_launch_ms": t_imp, "algorithmic_per_launch": qk_flops,
            "algorithmic_definition": "2*H*L_q*L_k*d flops: Q K^T counted once; the two-pass method executes it "
                                      "twice (executed_frac)",
            "traffic_detail": traffic_rec,
        },
        "stages": stages,
    }
    if others is not None:
        result["other_shapes"] = others
    if cache is not None:
        result["cache"] = cache
    # Context only: the FlowCache page's main table (section on key
    # experimental data) gives whole-video generation times with the models
    # on an A800; they include the transformer forwards this library does not
    # run, so they are not a target for this per-step metric.
    result["context"] = {
        "source": "Flow Caching for Autoregressive Video Generation (papernotes digest), main table, A800",
        "whole_video_latency_s": {"MAGI-1": {"vanilla": 2873, "flowcache_fast": 1209},
                                  "SkyReels-V2": {"vanilla": 1540, "flowcache_fast": 230}},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample of the step")
        result["cpu_baseline"] = cpu_baseline(cfg, ccfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
