"""Benchmark of the attention hot path on one MI355X.

Workload: 72,576 video tokens (a 10 s 1344x768 clip, 72 latent frames of 1,008
tokens) x 56 heads of width 128, bf16, frame-correlated synthetic Q/K and
N(0, 1) V, seed 3.  One step is one pass of the whole path over that input:
the dense attention of all 56 heads through the head-group launcher (groups of
16: 16+16+16+8), then the 90%-sparse attention of all 56 heads through the same
launcher (per group: tile means, tile scores and top-57 selection, sparse tile
loop).  Inputs are resident in HBM before timing starts.

Effective FLOP (the count used for every TFLOP/s figure): 4 * d * (valid keys
attended) summed over heads and valid query rows; dense = 4 N^2 d H, sparse is
counted exactly from the selected tile lists (a partial tile counts its valid
keys).

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_dense_72576x16_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "video_diffusion_transformer_amd", "csrc", "attn_fwd.hip")

TOKENS, HEADS, GROUP, KEEP_FRAC, SEED = 72576, 56, 16, 0.1, 3
FRAME_TOKENS = 1008   # latent tokens per frame at 1344x768


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def sparse_flops(idx, tokens: int, d: int = 128) -> float:
    """4 d (valid keys) summed over heads and valid query rows, from int32 idx [H, T, k]."""
    import numpy as np
    T = idx.shape[1]
    valid = np.full(T, 128, dtype=np.int64)
    valid[-1] = tokens - 128 * (T - 1)
    keys = valid[idx].sum(axis=2)            # [H, T] keys seen by each query tile
    return float(4 * d * (keys * valid[None, :]).sum())


def window_flops(tokens: int, frame_tokens: int, chunk: int, nb: int, heads: int, d: int = 128,
                 prefix: int = 0) -> float:
    """QK^T + PV FLOPs over the (query, key) pairs the frame window allows;
    `prefix` non-video tokens ahead of the video see and are seen by all."""
    import numpy as np
    video = tokens - prefix
    frames = -(-video // frame_tokens)
    f = np.arange(frames)
    allowed = np.abs(f[:, None] // chunk - f[None, :] // chunk) <= nb
    allowed[:, [0, frames - 1]] = True
    allowed[[0, frames - 1], :] = True
    per_frame = np.minimum(frame_tokens, video - f * frame_tokens).astype(np.float64)
    pairs = float(per_frame @ allowed.astype(np.float64) @ per_frame)
    pairs += float(prefix) * tokens + float(video) * prefix
    return 4.0 * d * heads * pairs


def vsa_flops(idx, prefix: int, grid, tile, d: int = 128) -> float:
    """QK^T + PV FLOPs of VSA-H3 attention: non-video rows see every key; a
    video query tile sees the prefix plus the tokens of its kept tiles."""
    import numpy as np
    frames, height, width = grid
    tt, th, tw = tile
    sizes = np.array([min(tt, frames - a) * min(th, height - b) * min(tw, width - c)
                      for a in range(0, frames, tt) for b in range(0, height, th)
                      for c in range(0, width, tw)], dtype=np.float64)
    n = prefix + frames * height * width
    pairs = prefix * float(n) * idx.shape[0]
    kept = sizes[idx].sum(axis=2)                       # [H, Tv] kept video keys
    pairs += float((sizes[None, :] * (prefix + kept)).sum())
    return 4.0 * d * pairs


def cpu_baseline(q, k, v, scale, budget_s: float):
    """The fp64 oracle on head 0 of the same workload: full selection, then dense and
    sparse attention for consecutive query tiles until the time budget is spent."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    affinity = len(os.sched_getaffinity(0))
    # the oracle's parallel work is its BLAS calls; the rest is one thread
    threads = max(1, min(blas_threads, affinity))
    qw, kw, vw = (oracle.widen(t[:1]) for t in (q, k, v))
    t0 = time.perf_counter()
    idx = oracle.select_tiles(qw, kw, KEEP_FRAC)
    t_sel = time.perf_counter() - t0
    T = idx.shape[1]
    flop = 0.0
    tiles = 0
    elapsed = t_sel
    while tiles < T and elapsed < budget_s:
        rows = np.arange(tiles * 128, min(tiles * 128 + 128, TOKENS))
        t1 = time.perf_counter()
        oracle.dense(qw, kw, vw, scale, rows=rows)
        oracle.sparse(qw, kw, vw, scale, idx, rows=rows)
        elapsed += time.perf_counter() - t1
        keys = sum(min(128, TOKENS - 128 * t) for t in idx[0, tiles])
        flop += 4 * 128 * len(rows) * (TOKENS + keys)
        tiles += 1
    # the selection of one head is 1/56 of the workload's selection; charge it fully
    value = flop / elapsed / 1e12
    return {
        "value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "affinity_cores": affinity, "blas_threads": blas_threads,
        "sample": (f"fp64 numpy oracle, head 0 of {HEADS}: tile selection over all {T} tiles "
                   f"({t_sel:.1f} s), then dense and 90%-sparse attention for query tiles 0-{tiles - 1} "
                   f"({tiles * 128} rows), {elapsed:.1f} s in total; effective FLOP of those rows / time"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["dense", "sparse", "window", "vsa", "int8", "fp8", "vda",
                                       "roofline", "configs"],
                    default=None,
                    help="time only one mode (for profiler runs; value then covers that mode, "
                         "0 for window, vsa, int8, fp8, vda, configs and roofline, which are timed outside the step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter calibration runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU launch; heads would shard with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import video_diffusion_transformer_amd as fv
    from video_diffusion_transformer_amd import inputs

    fv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scale = 1.0 / math.sqrt(128)

    log("generating inputs", TOKENS, "tokens x", HEADS, "heads")
    q, k, v = inputs.make_qkv(TOKENS, HEADS, "frame", SEED)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out_dense = torch.empty_like(qd)
    out_sparse = torch.empty_like(qd)
    stream = torch.cuda.current_stream()

    idx = fv.select_tiles(qd, kd, keep_frac=KEEP_FRAC)
    torch.cuda.synchronize()
    flop_sparse = sparse_flops(idx.cpu().numpy(), TOKENS)
    flop_dense = 4.0 * TOKENS * TOKENS * 128 * HEADS
    del idx

    if args.copy_calibration:
        # one elementwise kernel that reads 1 GiB and writes 1 GiB (a device-to-device
        # copy_ may run on a DMA engine, which the shader counters do not see)
        a = torch.zeros(1 << 29, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written by one elementwise kernel")
        del a, b

    do_dense = args.only in (None, "dense")
    do_sparse = args.only in (None, "sparse")
    do_window = args.only in (None, "window")
    do_vsa = args.only in (None, "vsa")
    do_int8 = args.only in (None, "int8")
    do_fp8 = args.only in (None, "fp8")
    do_vda = args.only in (None, "vda")
    do_configs = args.only in (None, "configs")
    do_roofline = args.only in (None, "dense", "roofline")
    if not do_dense:
        flop_dense = 0.0
    if not do_sparse:
        flop_sparse = 0.0

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if do_dense:
            fv.forward_heads(qd, kd, vd, GROUP, scale=scale, mode="dense", out=out_dense)
        if ev is not None:
            ev[1].record(stream)
        if do_sparse:
            fv.forward_heads(qd, kd, vd, GROUP, scale=scale, mode="sparse", keep_frac=KEEP_FRAC,
                             out=out_sparse)
        if ev is not None:
            ev[2].record(stream)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log("timing", args.steps, "steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dense_ms = [e[0].elapsed_time(e[1]) for e in evs]
    sparse_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step = wall * 1e3 / args.steps

    # roofline of the dominant kernel, outside the step: the dense kernel alone,
    # one 16-head launch at a time on one stream (in the step the launcher
    # overlaps consecutive head groups, so a group's launch has no duration of
    # its own there)
    rl_ms = []
    if do_roofline:
        qg, kg, vg, og = qd[:GROUP], kd[:GROUP], vd[:GROUP], out_dense[:GROUP]
        rl_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for i in range(4):
            rl_ev[0].record(stream)
            fv.forward(qg, kg, vg, scale=scale, out=og)
            rl_ev[1].record(stream)
            torch.cuda.synchronize()
            if i:
                rl_ms.append(rl_ev[0].elapsed_time(rl_ev[1]))
        del qg, kg, vg, og

    # the matrix-core rate this GPU sustains right now (dependency-free MFMA
    # loop), to read the roofline figure against besides the data-sheet peak
    mfma_loop = None
    if do_roofline:
        sink = torch.empty(fv.PROBE_SINK, dtype=torch.float32, device=dev)
        fv.mfma_probe(20000, sink)
        torch.cuda.synchronize()
        iters = 400000
        p_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        p_ev[0].record(stream)
        fv.mfma_probe(iters, sink)
        p_ev[1].record(stream)
        torch.cuda.synchronize()
        pm = p_ev[0].elapsed_time(p_ev[1])
        if not bool(torch.isfinite(sink).all()):
            raise RuntimeError("MFMA probe produced non-finite sums")
        mfma_loop = {"tflops": round(fv.PROBE_FLOP_PER_ITER * iters / (pm * 1e-3) / 1e12, 2),
                     "ms": round(pm, 3),
                     "what": "bf16 v_mfma_f32_32x32x16 chains, 4 per wave, 4 waves per SIMD, no memory "
                             "traffic, run right after the roofline launches"}
        del sink

    # split of the sparse time: selection alone, outside the timed region
    sel_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    idx_buf = torch.empty((GROUP, fv.tile_count(TOKENS), fv.keep_count(TOKENS, KEEP_FRAC)),
                          dtype=torch.int32, device=dev)
    sel_ms = []
    for _ in range(3):
        sel_ev[0].record(stream)
        for h0 in range(0, HEADS, GROUP):
            h1 = min(HEADS, h0 + GROUP)
            fv.select_tiles(qd[h0:h1], kd[h0:h1], keep_frac=KEEP_FRAC, out=idx_buf[:h1 - h0])
        sel_ev[1].record(stream)
        torch.cuda.synchronize()
        sel_ms.append(sel_ev[0].elapsed_time(sel_ev[1]))

    # frame-window softmax (Video DeltaNet's softmax branch), outside the step:
    # 5-frame chunks, one neighbouring chunk on each side, first and last frame
    # as anchors; all 56 heads in one launch
    window = None
    if do_window:
        out_window = torch.empty_like(qd)
        w_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        w_ms = []
        for i in range(4):
            w_ev[0].record(stream)
            fv.forward_window(qd, kd, vd, frame_tokens=FRAME_TOKENS, chunk_frames=5, neighbours=1,
                              scale=scale, out=out_window)
            w_ev[1].record(stream)
            torch.cuda.synchronize()
            if i:
                w_ms.append(w_ev[0].elapsed_time(w_ev[1]))
        del out_window
        wm = float(np.median(w_ms))
        flop_w = window_flops(TOKENS, FRAME_TOKENS, 5, 1, HEADS)
        idx_w, cnt_w = fv.window_tiles(TOKENS, FRAME_TOKENS, 5, 1, device=dev)
        flop_w_visited = 4.0 * 128 * HEADS * 128 * 128 * float(cnt_w.sum().item())
        del idx_w, cnt_w
        window = {"ms": round(wm, 3), "flop_allowed": flop_w,
                  "tflops_effective": round(flop_w / (wm * 1e-3) / 1e12, 2),
                  "tflops_visited": round(flop_w_visited / (wm * 1e-3) / 1e12, 2),
                  "density": round(flop_w / (4.0 * TOKENS * TOKENS * 128 * HEADS), 4)}

    # dense attention with INT8 and with FP8 (E4M3) query-key scores, outside
    # the step: same inputs, same head groups
    quant = {}
    for qmode, on in (("int8", do_int8), ("fp8", do_fp8)):
        if not on:
            continue
        out_q = torch.empty_like(qd)
        i_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        i_ms = []
        for i in range(4):
            i_ev[0].record(stream)
            fv.forward_heads(qd, kd, vd, GROUP, scale=scale, mode=qmode, out=out_q)
            i_ev[1].record(stream)
            torch.cuda.synchronize()
            if i:
                i_ms.append(i_ev[0].elapsed_time(i_ev[1]))
        im = float(np.median(i_ms))
        flop_i = 4.0 * TOKENS * TOKENS * 128 * HEADS
        rec = {"ms": round(im, 3), "tflops": round(flop_i / (im * 1e-3) / 1e12, 2),
               "frac_peak_bf16": round(flop_i / (im * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        if do_dense:
            # output difference against the bf16 dense path on the same inputs
            d = (out_q.float() - out_dense.float())
            rec["rel_diff_vs_bf16_dense"] = round(float(d.norm() / out_dense.float().norm()), 5)
        quant[qmode] = rec
        del out_q
    int8 = quant.get("int8")
    fp8 = quant.get("fp8")

    # the other workloads of the path, outside the step, each on its own seeded
    # inputs: 5,040 tokens x 56 heads dense in one launch; 72,576 x 16 heads
    # dense (one 16-head group); 102,816 tokens x 56 heads (14.4 s clip, last
    # tile 32 tokens) dense and 90% sparse in 8-head groups
    configs = None
    if do_configs:
        configs = {}

        def timed(fn, reps=3):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                ev[0].record(stream)
                fn()
                ev[1].record(stream)
                torch.cuda.synchronize()
                ts.append(ev[0].elapsed_time(ev[1]))
            return float(np.median(ts))

        def entry(ms, flop):
            tf = flop / (ms * 1e-3) / 1e12
            return {"ms": round(ms, 3), "tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "flop": flop}

        for cid in (2, 3, 5):
            c = inputs.CONFIGS[cid]
            log("generating", c.name)
            cq, ck, cv = (t.to(dev) for t in inputs.make_inputs(cid))
            cout = torch.empty_like(cq)
            fd = 4.0 * c.tokens * c.tokens * 128 * c.heads
            if c.group == c.heads:
                dms = timed(lambda: fv.forward(cq, ck, cv, scale=c.scale, out=cout))
            else:
                dms = timed(lambda: fv.forward_heads(cq, ck, cv, c.group, scale=c.scale, out=cout))
            rec = {"workload": f"{c.tokens:,} tokens x {c.heads} heads, "
                               + (f"one launch" if c.group == c.heads else f"{c.group}-head groups"),
                   "dense": entry(dms, fd)}
            if "sparse" in c.modes:
                cidx = fv.select_tiles(cq, ck, keep_frac=c.keep_frac)
                torch.cuda.synchronize()
                fs = sparse_flops(cidx.cpu().numpy(), c.tokens)
                keep = int(cidx.shape[2])
                del cidx
                sms = timed(lambda: fv.forward_heads(cq, ck, cv, c.group, scale=c.scale, mode="sparse",
                                                     keep_frac=c.keep_frac, out=cout))
                rec["sparse"] = entry(sms, fs)
                rec["sparse"]["keep_tiles"] = keep
                rec["sparse"]["speedup_vs_dense"] = round(dms / sms, 3)
            configs[c.name] = rec
            del cq, ck, cv, cout
            torch.cuda.empty_cache()

    # VSA-H3 packed sequence, outside the step: a 512-token non-video prefix
    # ahead of the same 72 x 24 x 42 video grid, (4, 4, 4) tiles, 90% sparse,
    # all 56 heads in one call (new inputs: the prefix shifts the video tokens)
    vsa = None
    if do_vsa:
        del qd, kd, vd, out_dense, out_sparse
        torch.cuda.empty_cache()
        prefix, grid, tile = inputs.VSA_PREFIX, inputs.VSA_GRID_72, (4, 4, 4)
        log("generating VSA inputs", prefix, "+", grid)
        pq, pk, pv = (t.to(dev) for t in inputs.make_packed_qkv(prefix, grid, HEADS, SEED))
        pout = torch.empty_like(pq)
        v_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        v_ms = []
        for i in range(4):
            v_ev[0].record(stream)
            fv.forward_vsa(pq, pk, pv, prefix, grid, tile, KEEP_FRAC, scale=scale, out=pout)
            v_ev[1].record(stream)
            torch.cuda.synchronize()
            if i:
                v_ms.append(v_ev[0].elapsed_time(v_ev[1]))
        vidx = fv.vsa_select(pq, pk, prefix, grid, tile, KEEP_FRAC).cpu().numpy()
        # the frame window on the same packed sequence: the 512 non-video
        # tokens are dense rows and columns (text and audio keep full softmax attention)
        window_prefix = None
        if do_window:
            ft = grid[1] * grid[2]
            for i in range(4):
                v_ev[0].record(stream)
                fv.forward_window(pq, pk, pv, frame_tokens=ft, chunk_frames=5, neighbours=1, scale=scale,
                                  prefix=prefix, out=pout)
                v_ev[1].record(stream)
                torch.cuda.synchronize()
                if i == 0:
                    wp_ms = []
                else:
                    wp_ms.append(v_ev[0].elapsed_time(v_ev[1]))
            ntok = prefix + grid[0] * ft
            flop_wp = window_flops(ntok, ft, 5, 1, HEADS, prefix=prefix)
            wpm = float(np.median(wp_ms))
            window_prefix = {"ms": round(wpm, 3), "prefix": prefix, "tokens": ntok, "flop_allowed": flop_wp,
                             "tflops_effective": round(flop_wp / (wpm * 1e-3) / 1e12, 2),
                             "density": round(flop_wp / (4.0 * ntok * ntok * 128 * HEADS), 4)}
        del pq, pk, pv, pout
        vm = float(np.median(v_ms))
        flop_v = vsa_flops(vidx, prefix, grid, tile)
        ntok = prefix + grid[0] * grid[1] * grid[2]
        vsa = {"ms": round(vm, 3), "flop": flop_v, "prefix": prefix, "grid": list(grid),
               "tile": list(tile), "keep_tiles": int(vidx.shape[2]), "video_tiles": int(vidx.shape[1]),
               "tflops_effective": round(flop_v / (vm * 1e-3) / 1e12, 2),
               "density": round(flop_v / (4.0 * ntok * ntok * 128 * HEADS), 4)}

    # Video Delta Attention (the linear branch of Video DeltaNet), outside the
    # step: 72 latent frames of 1,008 tokens, 56 heads, 5-frame chunks +-1
    vda = None
    if do_vda:
        torch.cuda.empty_cache()
        frames = TOKENS // FRAME_TOKENS
        log("generating Video Delta Attention inputs", frames, "frames x", HEADS, "heads")
        vin = [t.to(dev) for t in inputs.make_vda_inputs(frames, HEADS, SEED, FRAME_TOKENS)]
        vout = torch.empty((HEADS, TOKENS, 128), dtype=torch.float32, device=dev)
        a_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        a_ms = []
        for i in range(4):
            a_ev[0].record(stream)
            fv.vda_forward(*vin, FRAME_TOKENS, 5, 1, out=vout)
            a_ev[1].record(stream)
            torch.cuda.synchronize()
            if i:
                a_ms.append(a_ev[0].elapsed_time(a_ev[1]))
        del vin, vout
        am = float(np.median(a_ms))
        # algorithmic FLOP: A_t and B_t over the interior frames' tokens (the
        # anchors are never written), the readout (one product with the summed
        # states per token), and per interior frame the inverse (2 d^3), C_t =
        # B_t M_t (2 d^3) and one state product in each scan (2 x 2 d^3)
        d2 = 128.0 * 128.0
        inner = frames - 2
        flop_a = (4.0 * inner * FRAME_TOKENS * d2 + 2.0 * TOKENS * d2) * HEADS \
            + (2.0 + 2.0) * 128.0 * d2 * inner * HEADS + 2 * 2.0 * 128.0 * d2 * inner * HEADS
        # fp32-equivalent: the products with a bf16 operand run on the bf16
        # matrix cores with the fp32 operand split into hi + lo halves, the
        # rest on the fp32 matrix cores, so no single peak applies
        vda = {"ms": round(am, 3), "flop": flop_a,
               "tflops_fp32_equivalent": round(flop_a / (am * 1e-3) / 1e12, 2),
               "frames": frames, "frame_tokens": FRAME_TOKENS}

    d_ms = float(np.median(dense_ms))
    s_ms = float(np.median(sparse_ms))
    dense_tflops = flop_dense / max(d_ms * 1e-3, 1e-12) / 1e12
    sparse_tflops = flop_sparse / max(s_ms * 1e-3, 1e-12) / 1e12
    value = (flop_dense + flop_sparse) * args.steps / wall / 1e12

    # roofline of the dominant kernel: per launch = one 16-head dense launch
    flop_launch = 4.0 * TOKENS * TOKENS * 128 * GROUP
    dense_launch_ms = float(np.median(rl_ms)) if rl_ms else float("nan")
    achieved = flop_launch / max(dense_launch_ms * 1e-3, 1e-12) / 1e12 if rl_ms else 0.0
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == kernel_source_hash():
            traffic = tr.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    loop_tf = mfma_loop["tflops"] if mfma_loop else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": "attn_fwd_kernel<0, 4, 2, 1, 64> (dense, one 16-head launch)",
                "flop_per_launch": flop_launch, "avg_launch_ms": round(dense_launch_ms, 4),
                "frac_of_mfma_loop": round(achieved / loop_tf, 4) if loop_tf else None}

    result = {
        "metric": "attn TFLOP/s + % bf16 MFMA peak, 72,576 tok x 56 heads, dense & 90% sparse",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded frame-correlated Q/K, N(0,1) V; stands in for H3 activations)",
        "config": {"workload": "video-token attention, 72,576 tokens x 56 heads x 128, "
                               "dense + 90% block-sparse (57 of 567 key tiles), head groups of 16",
                   "tokens": TOKENS, "heads": HEADS, "head_dim": 128, "group_heads": GROUP,
                   "keep_frac": KEEP_FRAC, "seed": SEED},
        "dense": {"ms": round(d_ms, 3), "tflops": round(dense_tflops, 2),
                  "frac_peak": round(dense_tflops / PEAK_BF16_TFLOPS, 4), "flop": flop_dense,
                  "frac_of_mfma_loop": round(dense_tflops / loop_tf, 4) if loop_tf else None},
        "sparse": {"ms": round(s_ms, 3), "tflops_effective": round(sparse_tflops, 2),
                   "frac_peak": round(sparse_tflops / PEAK_BF16_TFLOPS, 4), "flop": flop_sparse,
                   "selection_ms": round(float(np.median(sel_ms)), 3),
                   "speedup_vs_dense": round(d_ms / s_ms, 3) if do_dense and do_sparse else None},
        "roofline": roofline,
        "mfma_loop": mfma_loop,
    }
    if window is not None:
        if do_dense:
            window["speedup_vs_dense"] = round(d_ms / window["ms"], 3)
        result["window"] = window
        if do_vsa and window_prefix is not None:
            result["window"]["with_prefix"] = window_prefix
    if vsa is not None:
        result["vsa"] = vsa
    if vda is not None:
        result["vda"] = vda
    if configs is not None:
        result["configs"] = configs
    for qname, qrec in (("int8", int8), ("fp8", fp8)):
        if qrec is not None:
            if do_dense:
                qrec["speedup_vs_dense"] = round(d_ms / qrec["ms"], 3)
            result[qname] = qrec
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle), budget", args.cpu_budget, "s")
        result["cpu_baseline"] = cpu_baseline(q, k, v, scale, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
