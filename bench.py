"""Throughput of the block-sparse multi-draft verification hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stack64k]

A step is one verification pass over the whole workload: on every selecting layer
sv_select_and_attend (scoring, budget, top-k, sparse multi-draft attention, merge),
on every reuse layer sv_sparse_verify_attn over the previous layer's index buffers
(inter-layer reuse without a copy). Inputs are seeded synthetic tensors already
resident in HBM (the paged KV pools are built with sv_block_repr before timing). The
step is captured once in a HIP graph and replayed.

Prints one JSON line. `value` is verified draft-token-heads per second (rows of
(draft token, query head) per layer, summed over layers and sequences).
`roofline` refers to the attention entry point (the dominant cost; the merge of its
split partials runs inside the same launch when the grid is resident at once, else
in a merge kernel right after it): algorithmic bytes (selected K/V of one layer)
over its average duration, timed with HIP events on the stream it runs on.
`traffic` is the HBM traffic per launch from the committed profiler counter summary
of the attention kernel, reported only while that summary was taken from the
current kernel source. `dense_vs_sparse` times the same attention entry point with
every block selected at the same context lengths (the dense verification the sparse
path stands in for). `cpu_baseline` times the fp64 oracle on a bounded sample of the
same workload on the host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "verify-attn draft-token-heads/s and % HBM peak at 32K-128K ctx, 1 GPU"
ATTN_SRC = os.path.join(ROOT, "block_sparse_speculative_amd", "csrc", "attn.hip")
COUNTERS = os.path.join(ROOT, "profiles", "attn_kernel_{workload}_counters.txt")


def counter_field(workload: str, name: str):
    """A figure of the committed counter summary of the attention kernel, or None when
    there is none or it was taken from another version of the kernel source."""
    import hashlib
    path = COUNTERS.format(workload=workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if fields.get("source_sha256") != sha or name not in fields:
        return None
    return float(fields[name].split()[0])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stack64k")
    ap.add_argument("--instances", type=int, default=0,
                    help="rotated resident copies (0: enough to exceed the 256 MB last-level cache)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip timing the dense (every block selected) attention")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--separate", action="store_true",
                    help="run the separate-call path (select / reuse copy / attend) instead")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--draft-tree", default="chain", choices=["chain", "random", "star"],
                    help="draft structure: a chain (the workload's own) or a seeded draft tree")
    ap.add_argument("--launch-curve", action="store_true",
                    help="also time the attention entry point against the number of selected "
                         "blocks per unit (fixed cost and streaming rate of one launch)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the qwen128k block that follows the headline workload")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ffn-only", action="store_true",
                    help="only time the sparse FFN (its JSON record alone, for profiling)")
    ap.add_argument("--append-only", action="store_true",
                    help="only time the decode-step KV append of the workload (its JSON "
                         "record alone, for profiling)")
    return ap.parse_args()


def copy_calibration(mib: int, reps: int):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) read by the profiler."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_mib": mib, "reps": reps, "bytes_read_per_copy": n * 4,
                      "bytes_written_per_copy": n * 4, "gbs": 2 * n * 4 / dt / 1e9}), flush=True)


def cpu_baseline(inst, budget_s: float):
    """Oracle draft-token-heads/s on host cores over whole layers of the same workload
    (sequence 0 first, then the next sequences), until about `budget_s` seconds of
    oracle work. Representatives are computed outside the timed region (they exist
    before verification), as are the device-to-host copies and the fp64 widening."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    w = inst.w
    G, bs, T = w.group, w.block_size, w.num_draft
    dense, mn, frac, kf, kl = w.budget
    timed, rows, units_done = 0.0, 0, 0
    done = []                              # (sequence, layers) covered
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        for b in range(w.num_seqs):
            ctx = inst.ctx_lens[b]
            prev = None
            layers_done = 0
            for l in range(len(inst.layers)):
                x = inst.logical(l)
                q = x["q"][b].float().cpu().numpy()
                kc = x["k_ctx"][b, :ctx].float().cpu().numpy()
                vc = x["v_ctx"][b, :ctx].float().cpu().numpy()
                kd = x["k_draft"][b].float().cpu().numpy()
                vd = x["v_draft"][b].float().cpu().numpy()
                del x
                reuse = inst.layers[l].reuse
                sels = []
                for g in range(w.num_kv_heads):
                    sl = slice(g, g + 1)
                    qg = q[:, g * G:(g + 1) * G]
                    if not reuse:
                        reps = O.block_representatives(kc[:, sl], bs)          # untimed
                    t0 = time.perf_counter()
                    if reuse:
                        sel = prev[g]
                    else:
                        sc = O.block_scores(qg[0], reps, G)[0]
                        k = O.budget_blocks(ctx, bs, dense, mn, frac)
                        sel = O.select_blocks(sc, k, bool(kf), bool(kl))
                    O.verify_attention(qg, kc[:, sl], vc[:, sl], kd[:, sl], vd[:, sl], [sel],
                                       bs, inst.scale,
                                       parents=None if inst.parents is None else inst.parents[b])
                    timed += time.perf_counter() - t0
                    sels.append(sel)
                    rows += T * G
                    units_done += 1
                prev = sels
                layers_done += 1
                if timed >= budget_s and (not w.reuse_odd_layers or layers_done % 2 == 0):
                    break
            done.append((b, layers_done))
            if timed >= budget_s:
                break
    desc = ", ".join(f"sequence {b} (ctx {inst.ctx_lens[b]}) layers 0..{n - 1}" for b, n in done)
    return {
        "value": rows / timed,
        "unit": "draft-token-heads/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{desc} of {len(inst.layers)} layers, all {w.num_kv_heads} KV heads: "
                   f"{units_done} units, {rows} draft-token-heads, {timed:.1f} s of numpy fp64 "
                   f"with BLAS on {cores} host threads (scores, budget, top-k, attention; "
                   f"representatives precomputed)"),
    }


def dense_vs_sparse(inst, sparse_us: float, reps: int):
    """The same attention entry point at the same context lengths with every block of
    every sequence selected (the dense verification the sparse path replaces), on
    layer 0 of `inst`: its average launch time, its bandwidth over the K/V it reads,
    and its ratio to the sparse launch time."""
    import torch
    from block_sparse_speculative_amd import _lib as L
    from block_sparse_speculative_amd import pipeline as PL

    w = inst.w
    B, Hkv = w.num_seqs, w.num_kv_heads
    nbs = [-(-c // w.block_size) for c in inst.ctx_lens]
    k_max = max(nbs)
    idx = torch.full((B, Hkv, k_max), -1, dtype=torch.int32)
    for b, n in enumerate(nbs):
        idx[b, :, :n] = torch.arange(n, dtype=torch.int32)
    idx = idx.to(inst.device)
    cnt = torch.tensor(nbs, dtype=torch.int32)[:, None].expand(B, Hkv).contiguous().to(inst.device)
    ws = PL.Workspaces(inst.shape, k_max, 0, inst.device)
    ly = inst.layers[0]
    out = torch.empty_like(ly.out)

    def call():
        L.sparse_verify_attn(inst.shape, ly.q, ly.k_draft, ly.v_draft, ly.pool.k, ly.pool.v,
                             inst.table, inst.ctx, idx, cnt, k_max, inst.scale, out, ws=ws.attn,
                             draft_mask=inst.draft_mask)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(4):
            call()
    stream = torch.cuda.current_stream()
    graph.replay()
    stream.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        graph.replay()
    ev1.record(stream)
    ev1.synchronize()
    dense_us = ev0.elapsed_time(ev1) * 1e3 / (4 * reps)
    elem = 4 if w.dtype == "fp32" else 2
    dense_bytes = sum(inst.ctx_lens) * Hkv * w.head_dim * 2 * elem
    return {
        "ctx": inst.ctx_lens if len(set(inst.ctx_lens)) > 1 else inst.ctx_lens[0],
        "dense_blocks_per_seq": k_max,
        "dense_us": dense_us,
        "sparse_us": sparse_us,
        "ratio": dense_us / sparse_us,
        "dense_kv_bytes": dense_bytes,
        "dense_gbs": dense_bytes / (dense_us * 1e-6) / 1e9,
        "dense_frac": dense_bytes / (dense_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
    }


def launch_curve(inst, reps: int):
    """Average time of one attention launch against k, the blocks selected per unit
    (a seeded random sorted subset per sequence and KV head, distinct per launch), over
    8 launches replayed in a graph (cycling over the layers of `inst`, so a one-layer
    workload does not carry a whole graph launch per attention launch). k runs from 0
    to the workload's k_max
    at its own split layout, then doubles with k_max = k up to every block. A least-
    squares line through the points with k >= k_max gives the launch's fixed cost
    (intercept) and its streaming rate (slope)."""
    import torch
    from block_sparse_speculative_amd import _lib as L
    from block_sparse_speculative_amd import pipeline as PL

    w = inst.w
    B, Hkv = w.num_seqs, w.num_kv_heads
    nbs = [-(-c // w.block_size) for c in inst.ctx_lens]
    nl = len(inst.layers)
    nlaunch = 8
    elem = 4 if w.dtype == "fp32" else 2
    gen = torch.Generator().manual_seed(12345)
    ks = sorted({0, max(1, inst.k_max // 8), max(1, inst.k_max // 4), max(1, inst.k_max // 2),
                 inst.k_max})
    k = inst.k_max * 2
    while k < max(nbs):
        ks.append(k)
        k *= 2
    ks.append(max(nbs))
    points = []
    for k in ks:
        k_max = max(k, inst.k_max)
        idxs = []
        for _ in range(nlaunch):
            idx = torch.full((B, Hkv, k_max), -1, dtype=torch.int32)
            for b, n in enumerate(nbs):
                for g in range(Hkv):
                    kk = min(k, n)
                    idx[b, g, :kk] = torch.randperm(n, generator=gen)[:kk].sort().values.to(torch.int32)
            idxs.append(idx.to(inst.device))
        cnt = torch.tensor([min(k, n) for n in nbs], dtype=torch.int32)[:, None].expand(
            B, Hkv).contiguous().to(inst.device)
        ws = PL.Workspaces(inst.shape, k_max, 0, inst.device)
        outs = [torch.empty_like(inst.layers[i % nl].out) for i in range(nlaunch)]

        def call(i):
            ly = inst.layers[i % nl]
            L.sparse_verify_attn(inst.shape, ly.q, ly.k_draft, ly.v_draft, ly.pool.k, ly.pool.v,
                                 inst.table, inst.ctx, idxs[i], cnt, k_max, inst.scale, outs[i],
                                 ws=ws.attn, draft_mask=inst.draft_mask)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(nlaunch):
                call(i)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(nlaunch):
                call(i)
        stream = torch.cuda.current_stream()
        graph.replay()
        stream.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            graph.replay()
        ev1.record(stream)
        ev1.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / (reps * nlaunch)
        kv = sum(min(k, n) * w.block_size for n in nbs) * Hkv * w.head_dim * 2 * elem
        points.append({"k": k, "k_max": k_max, "splits": L.attn_num_splits(inst.shape, k_max, 0),
                       "us": round(us, 2), "kv_bytes": kv, "gbs": round(kv / us / 1e3, 1)})
        print(f"[bench]   launch curve k={k}: {us:.2f} us", file=sys.stderr, flush=True)
    fixed_us, stream_gbs = fit_launch_line(points, inst.k_max)
    return {"points": points, "fixed_us": fixed_us, "stream_gbs": stream_gbs}


def fit_launch_line(points, k_min: int):
    """Least-squares line us = fixed + kv_bytes / rate through the points with
    k >= k_min. Returns (fixed cost in us, streaming rate in GB/s, or None when the
    slope is not positive)."""
    fit = [pt for pt in points if pt["k"] >= k_min]
    n = len(fit)
    mx = sum(pt["kv_bytes"] for pt in fit) / n
    my = sum(pt["us"] for pt in fit) / n
    sxx = sum((pt["kv_bytes"] - mx) ** 2 for pt in fit)
    slope = sum((pt["kv_bytes"] - mx) * (pt["us"] - my) for pt in fit) / sxx if sxx > 0 else 0.0
    return my - slope * mx, ((1e-3 / slope) if slope > 0 else None)


def build_instances(w, args, reps_total: int, progress=None):
    from block_sparse_speculative_amd.workload import Instance
    return [Instance(w, seed=args.seed + r, num_splits=args.num_splits, with_lse=False,
                     progress=progress, fused=not args.separate) for r in range(reps_total)]


def capture(fn):
    """A HIP graph of fn() (one eager warm-up on a side stream first)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def event_time_us(replay, reps: int) -> float:
    """Average time of one replay(), from HIP events on the current stream."""
    import torch
    stream = torch.cuda.current_stream()
    replay()
    stream.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        replay()
    ev1.record(stream)
    ev1.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / reps


def measure(w, args, steps: int, warmup: int, label: str):
    """One pass of the hot path over the workload, graph-replayed `steps` times after
    `warmup` replays (resident instances rotated past the last-level cache), and the
    attention launch alone. Returns (instances, figures)."""
    import torch
    from block_sparse_speculative_amd import synth
    from block_sparse_speculative_amd import workload as WL

    bytes_per_pass = WL.algorithmic_bytes(w, synth.context_lengths(w, args.seed), w.num_layers)
    # Rotate resident copies so one rotation touches more than 2 x 256 MB of selected
    # data and representatives (the MI355X last-level cache).
    reps_total = args.instances or max(1, -(-2 * 256 * 2 ** 20 // bytes_per_pass))
    print(f"[bench] {label} {w.name}: {bytes_per_pass / 1e6:.1f} MB algorithmic per pass, "
          f"{reps_total} resident instance(s)", file=sys.stderr, flush=True)

    def progress(done, total):
        if done == total or done % 8 == 0:
            print(f"[bench]   built layer {done}/{total}", file=sys.stderr, flush=True)

    insts = build_instances(w, args, reps_total, progress)
    inst0 = insts[0]
    torch.cuda.synchronize()

    def step():
        for it in insts:
            it.step()

    use_graph = not args.no_graph
    run = capture(step).replay if use_graph else step
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s_per_pass = wall / (steps * reps_total)      # the graph covers reps_total passes

    # ---- roofline of the attention entry point: a graph of only the attention calls
    # of every layer (indices from the passes above), replayed between HIP events on the
    # stream it runs on
    def attend_all():
        for it in insts:
            for l in range(len(it.layers)):
                it.attend(l)

    g_attn = capture(attend_all)
    attn_us = event_time_us(g_attn.replay, max(3, steps)) / (reps_total * len(inst0.layers))
    elem = 4 if w.dtype == "fp32" else 2
    kv_bytes_per_launch = (inst0.selected_tokens() // len(inst0.layers)) * w.head_dim * 2 * elem
    achieved = kv_bytes_per_launch / (attn_us * 1e-6) / 1e9
    all_bytes = WL.all_bytes(w, inst0.ctx_lens, len(inst0.layers), inst0.k_max, inst0.num_splits)
    fig = dict(s_per_pass=s_per_pass, units=inst0.units(), bytes_per_pass=bytes_per_pass,
               all_bytes_per_pass=all_bytes,
               attn_us=attn_us, kv_bytes_per_launch=kv_bytes_per_launch, achieved=achieved,
               reps_total=reps_total, graph=use_graph)
    return insts, fig


def full_verification_schedule(inst, sparse_pass_us: float, period: int, reps: int):
    """Periodic full verification: every `period`-th verification pass attends over
    every block on every layer (through the same attention entry point, no selection),
    the others are the sparse pass. Times one full pass (graph-replayed, HIP events) and
    reports the schedule's mean pass time."""
    import torch
    from block_sparse_speculative_amd import _lib as L
    from block_sparse_speculative_amd import pipeline as PL

    w = inst.w
    B, Hkv = w.num_seqs, w.num_kv_heads
    nbs = [-(-c // w.block_size) for c in inst.ctx_lens]
    k_max = max(nbs)
    idx = torch.full((B, Hkv, k_max), -1, dtype=torch.int32)
    for b, n in enumerate(nbs):
        idx[b, :, :n] = torch.arange(n, dtype=torch.int32)
    idx = idx.to(inst.device)
    cnt = torch.tensor(nbs, dtype=torch.int32)[:, None].expand(B, Hkv).contiguous().to(inst.device)
    ws = PL.Workspaces(inst.shape, k_max, 0, inst.device)
    outs = [torch.empty_like(ly.out) for ly in inst.layers]

    def full_pass():
        for ly, out in zip(inst.layers, outs):
            L.sparse_verify_attn(inst.shape, ly.q, ly.k_draft, ly.v_draft, ly.pool.k, ly.pool.v,
                                 inst.table, inst.ctx, idx, cnt, k_max, inst.scale, out,
                                 ws=ws.attn, draft_mask=inst.draft_mask)

    full_us = event_time_us(capture(full_pass).replay, reps)
    mean_us = ((period - 1) * sparse_pass_us + full_us) / period
    return {"period": period, "full_pass_us": full_us, "sparse_pass_us": sparse_pass_us,
            "mean_pass_us": mean_us, "full_over_sparse": full_us / sparse_pass_us,
            "mean_over_sparse": mean_us / sparse_pass_us,
            "what": "one full verification (every block, every layer) per period passes; the "
                    "others sparse"}


def decode_append(inst, reps: int):
    """One decode step's KV append on every layer: sv_block_repr writing T tokens per
    sequence (the last T positions of each context, rewritten in place with ctx_after =
    the context, so the touched blocks are full) and re-deriving the representatives of
    the blocks they land in. Graph-replayed, HIP events."""
    import torch
    from block_sparse_speculative_amd import pipeline as PL

    w = inst.w
    B, T = w.num_seqs, w.num_draft
    dev = inst.device
    ctx = torch.tensor(inst.ctx_lens, dtype=torch.int32, device=dev)
    before = (ctx - T).clamp(min=0).to(torch.int32)
    n_new = (ctx - before).to(torch.int32)

    def append_all():
        for ly in inst.layers:
            PL.append(inst.shape, ly.pool, ly.k_draft, ly.v_draft, n_new, before, inst.table,
                      ctx_after=ctx)

    us = event_time_us(capture(append_all).replay, reps)
    per_layer = us / len(inst.layers)
    return {"tokens_per_seq": T, "layers": len(inst.layers), "us_per_step": us,
            "us_per_layer": per_layer}


def sparse_ffn_bench(reps: int, seed: int = 0, graph: bool = True):
    """The threshold-pruned FFN of one verification pass (f4): 8 draft tokens through a
    Llama-3.1-8B-shaped FFN (4096 x 14336), two layers' weights rotated so a replay reads
    past the 256 MB last-level cache. Algorithmic bytes: all of W_gate plus the W_up and
    W_down rows of the channels some token keeps. The same call with tau = 0 (every
    channel kept, the dense FFN) is timed beside it."""
    import torch
    from block_sparse_speculative_amd import _lib as L
    from block_sparse_speculative_amd import synth

    w = synth.FFN_WORKLOADS["ffn_llama8b"]
    dev = torch.device("cuda")
    layers = [synth.make_ffn(w, seed + i, dev) for i in range(2)]
    shape = L.make_ffn_shape(w.num_tokens, w.d_model, w.d_ffn)
    ws = torch.empty(L.sparse_ffn_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    ys = [torch.empty((w.num_tokens, w.d_model), dtype=torch.bfloat16, device=dev) for _ in layers]
    keeps = [torch.zeros((w.d_ffn,), dtype=torch.int32, device=dev) for _ in layers]

    def run(tau):
        def fn():
            for inp, y, k in zip(layers, ys, keeps):
                L.sparse_ffn(shape, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down_t"], tau, y,
                             keep_bits=k, ws=ws)
        return fn

    def timed(fn):
        return event_time_us(capture(fn).replay if graph else fn, reps) / len(layers)

    sparse_us = timed(run(w.tau))
    torch.cuda.synchronize()
    kept_any = sum(float((k != 0).float().mean()) for k in keeps) / len(keeps)
    bits = torch.stack(keeps).cpu().to(torch.int64) & 0xFFFFFFFF
    per_token = float(sum(((bits >> t) & 1).float().mean() for t in range(w.num_tokens))) / w.num_tokens
    dense_us = timed(run(0.0))
    row = w.d_model * 2
    sparse_bytes = w.d_ffn * row * (1 + 2 * kept_any)
    dense_bytes = 3 * w.d_ffn * row
    return {
        "workload": w.name, "tokens": w.num_tokens, "d_model": w.d_model, "d_ffn": w.d_ffn,
        "tau": w.tau, "kept_per_token": per_token, "channels_any_token_keeps": kept_any,
        "sparse_us": sparse_us, "dense_us": dense_us, "speedup": dense_us / sparse_us,
        "algorithmic_bytes": sparse_bytes,
        "achieved_gbs": sparse_bytes / (sparse_us * 1e-6) / 1e9,
        "frac": sparse_bytes / (sparse_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "dense_frac": dense_bytes / (dense_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the per-GPU "
              f"share of a sharded deployment is the single-GPU workload measured here.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_mib:
        copy_calibration(args.copy_mib, max(1, args.steps))
        return
    if args.ffn_only:
        print(json.dumps(sparse_ffn_bench(max(1, args.steps), args.seed, graph=not args.no_graph)),
              flush=True)
        return
    if args.append_only:
        from block_sparse_speculative_amd import synth as _synth
        w = _synth.WORKLOADS[args.workload]
        inst = build_instances(w, args, 1)[0]
        rec = decode_append(inst, max(1, args.steps))
        rec["workload"] = w.name
        print(json.dumps(rec), flush=True)
        return

    from block_sparse_speculative_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = synth.WORKLOADS[args.workload].with_(draft_tree=args.draft_tree)
    insts, fig = measure(w, args, args.steps, args.warmup, "headline")
    inst0 = insts[0]
    s_per_pass = fig["s_per_pass"]
    step_gbs = fig["bytes_per_pass"] / s_per_pass / 1e9
    result = {
        "metric": METRIC,
        "value": fig["units"] / s_per_pass,
        "unit": "draft-token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s_per_pass * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian K/V/Q with planted heavy blocks; random-init, no weights)",
        "config": {
            "workload": w.name, "layers": len(inst0.layers), "num_seqs": w.num_seqs,
            "ctx": inst0.ctx_lens if len(set(inst0.ctx_lens)) > 1 else inst0.ctx_lens[0],
            "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "draft_tokens": w.num_draft,
            "draft_structure": w.draft_tree, "k_max": inst0.k_max,
            "reuse": "odd layers reuse" if w.reuse_odd_layers else "none",
            "splits": inst0.num_splits, "graph": fig["graph"],
            "resident_instances": fig["reps_total"],
            "path": ("separate calls: sv_select_blocks / sv_reuse_indices, sv_sparse_verify_attn"
                     if args.separate else
                     "sv_select_and_attend on selecting layers; sv_sparse_verify_attn on the "
                     "previous layer's index buffers on reuse layers"),
        },
        "hbm_frac_step": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": fig["bytes_per_pass"],
        # every byte the pass reads or writes once (queries, drafts, outputs, tables,
        # indices, scores, split partials besides the algorithmic bytes): secondary
        "all_bytes_per_step": fig["all_bytes_per_pass"],
        "roofline": {
            "kernel": "sv_sparse_verify_attn (attn_kernel; split partials merged inside the "
                      "launch)",
            "bound": "hbm",
            "achieved": fig["achieved"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": fig["achieved"] / HBM_PEAK_GBS,
            "traffic": counter_field(w.name, "traffic_bytes_per_launch"),
            "mfma_busy_pct": counter_field(w.name, "mfma_busy_pct"),
            "avg_launch_us": fig["attn_us"],
            "algorithmic_bytes_per_launch": fig["kv_bytes_per_launch"],
        },
    }
    reps = max(3, args.steps)
    if not args.no_dense:
        print("[bench] dense verification at the same context", file=sys.stderr, flush=True)
        result["dense_vs_sparse"] = dense_vs_sparse(inst0, fig["attn_us"], reps)
        print("[bench] periodic full verification", file=sys.stderr, flush=True)
        result["full_verification_schedule"] = full_verification_schedule(
            inst0, s_per_pass * 1e6, 8, max(3, min(reps, 10)))
    if args.launch_curve:
        print("[bench] attention launch time against selected blocks", file=sys.stderr, flush=True)
        result["launch_curve"] = launch_curve(inst0, reps)
    print("[bench] decode-step KV append", file=sys.stderr, flush=True)
    result["decode_append"] = decode_append(inst0, reps)
    del insts
    torch.cuda.empty_cache()
    if not args.no_secondary and args.workload != "qwen128k":
        # the other graded context length (128K), in the same run
        wq = synth.WORKLOADS["qwen128k"].with_(draft_tree=args.draft_tree)
        qi, qf = measure(wq, args, min(args.steps, 10), min(args.warmup, 3), "secondary")
        result["secondary"] = {
            "workload": wq.name, "ms_per_step": qf["s_per_pass"] * 1e3,
            "value": qf["units"] / qf["s_per_pass"], "unit": "draft-token-heads/s",
            "hbm_frac_step": qf["bytes_per_pass"] / qf["s_per_pass"] / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_step": qf["bytes_per_pass"],
            "avg_launch_us": qf["attn_us"], "achieved": qf["achieved"],
            "frac": qf["achieved"] / HBM_PEAK_GBS,
            "traffic": counter_field(wq.name, "traffic_bytes_per_launch"),
            "algorithmic_bytes_per_launch": qf["kv_bytes_per_launch"],
            "resident_instances": qf["reps_total"], "splits": qi[0].num_splits,
        }
        del qi
        torch.cuda.empty_cache()
    if not args.no_secondary:
        print("[bench] sparse FFN", file=sys.stderr, flush=True)
        result["sparse_ffn"] = sparse_ffn_bench(max(3, min(reps, 20)), args.seed)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inst0, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
