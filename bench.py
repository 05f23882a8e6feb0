"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one BSA request: bsa_plan (mask features, regime lookup, physical
mapping, compaction and scans, work list) followed by bsa_forward (fused
attention kernel and, when rows are split, the combine kernel) on one batch of
seeded synthetic inputs already resident in HBM. The metric counts only the
logical blocks the mask selects: 4 * bq * bk * D FLOPs per selected block.

The headline workload is the long-video mixed-geometry configuration (the
largest one that fits one GPU). The same JSON line carries a ``configs`` list
with the forward time, effective TFLOP/s, fraction of the bf16 MFMA peak,
fraction of HBM bandwidth over the streamed K/V bytes, and merge waste of
every benchmark configuration (video-DiT, chunked prefill, the affine
patterns at both block sizes and two wider windows, long video), each timed
in this run.

Plan and forward of a request run back to back on one stream. With
``--pipeline`` the line also reports requests pipelined as a serving runtime
could run them (the plan of request i+1 built on a second stream while the
forward of request i runs, each forward waiting for its plan through an
event); every step still plans and runs its request in full.

Prints one JSON line. ``--gpus N`` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective sparse-attn TFLOP/s (selected tiles only) + % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0
# The vector-ALU roofline of the online softmax. Per score it needs at least a
# scale-and-subtract, an exponential, a row-sum add and a row-maximum compare
# (no packed fp32 arithmetic in this build). A wave64 instruction takes 4
# cycles of a 16-lane SIMD; the exponential takes 8 (measured on gfx950: half
# the FMA issue rate). 1,024 SIMDs at 2.4 GHz then finish at most
# 1024 * 2.4e9 * 64 / 20 = 7.86e12 scores/s, i.e. 4*D FLOP of selected work
# per score: 2.01 PFLOP/s at D = 64 (below the MFMA peak), 4.03 at D = 128.
VALU_CYCLES_PER_64_SCORES = 4 + 8 + 4 + 4
PEAK_SCORES_PER_S = 1024 * 2.4e9 * 64 / VALU_CYCLES_PER_64_SCORES


def peak_alu_tflops(d: int) -> float:
    return PEAK_SCORES_PER_S * 4 * d / 1e12


def workload(name: str):
    from block_sparse_attention_08_amd import workloads as W
    table = {
        "video_dit": lambda: W.video_dit(),
        "video_dit_window": lambda: W.video_dit(p_global=0.0),
        "chunked_prefill": lambda: W.chunked_prefill(),
        "affine_bs64": lambda: W.affine(bs=64),
        "affine_bs32": lambda: W.affine(bs=32),
        "affine_bs64_w4096": lambda: W.affine(bs=64, window=4096),
        "affine_bs64_w8192": lambda: W.affine(bs=64, window=8192),
        "long_video": lambda: W.long_video(),
        "decode": lambda: W.decode(q_len=1),
        "decode_q16": lambda: W.decode(q_len=16),
        "decode_hnd": lambda: W.decode(q_len=1, kv_layout="hnd"),
        "decode_q16_hnd": lambda: W.decode(q_len=16, kv_layout="hnd"),
        "tiny": lambda: W.tiny(),
    }
    return table[name]()


# Memory-bound workloads (a few queries per sequence over a long cache): their
# roofline is HBM bytes, the K and V rows of the selected blocks read once per
# (sequence, kv group) plus Q, O and LSE, per forward launch.
HBM_BOUND = {"decode", "decode_q16", "decode_kv8", "decode_hnd", "decode_q16_hnd", "decode_kv8_hnd"}
# Workloads run with K and V as OCP FP8 E4M3 (bsa_forward_kv8), quantized once
# per kv head from the bf16 workload before timing.
KV8 = {"decode_kv8": "decode", "decode_kv8_hnd": "decode_hnd"}


# Workloads whose mask is chosen on the GPU in every step (bsa_select_blocks,
# keeping this many tenths of each query block's causal candidates) from the
# step's own Q and K, before the plan and the forward.
SELECTED = {"chunked_prefill_selected": ("chunked_prefill", 1)}
# Workloads planned from affine runs (bsa_plan_acsr) instead of a mask: the
# same problem and plan as the named mask workload, no mask and no read-back.
ACSR = {"affine_acsr_bs64": "affine_bs64", "affine_acsr_bs32": "affine_bs32"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("bsa_attention.hip", "bsa_internal.h"):
        h.update(open(os.path.join(ROOT, "block_sparse_attention_08_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def profile_record(name: str):
    """The committed rocprofv3 record of a workload's attention kernel (HBM
    bytes per launch; matrix-core and VALU busy fractions), if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec


def measured_traffic(name: str, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    rec = profile_record(name)
    return rec.get("hbm_bytes_per_launch") if rec else None


def allowed_keys_per_row(w, b: int, h: int) -> np.ndarray:
    """Number of allowed keys of every query row of (b, h): the selected blocks
    (the group's union in union mode), clipped to the sequence, then causal."""
    bm = 0 if w.mask_broadcast else b
    if w.gqa_union:
        gs = w.hq // w.hkv
        sel = np.zeros(w.nkb(h), bool)
        for h2 in range((h // gs) * gs, (h // gs + 1) * gs):
            sel |= w.head_mask(bm, h2).astype(bool).any(0)
        blk = np.broadcast_to(sel, (w.nqb(h), w.nkb(h)))
    else:
        blk = w.head_mask(bm, h).astype(bool)
    keys = np.arange(w.skv)
    row_blk = np.arange(w.sq) // w.bq[h]
    out = np.zeros(w.sq, np.int64)
    for qb in range(w.nqb(h)):
        allowed = blk[qb][keys // w.bk[h]]
        rows = np.nonzero(row_blk == qb)[0]
        if not w.causal:
            out[rows] = allowed.sum()
        else:
            csum = np.cumsum(allowed)
            lim = np.clip(rows + w.causal_offset, -1, w.skv - 1)
            out[rows] = np.where(lim >= 0, csum[np.maximum(lim, 0)], 0)
    return out


def effective_flops(w) -> float:
    """4 * D * (rows x keys) summed over the effective logical blocks of every
    (batch, head): selected (the group's union in union mode) and causally
    feasible (first key <= last query + offset), with a block at the end of a
    sequence counting only the rows and keys that exist. Equal to the plan's
    whole-block count when the lengths are block multiples; for decode (one
    query in a 128-row block) it counts the one row."""
    tot = 0.0
    for bm in range(w.mask_batches):
        nb = w.batch if w.mask_broadcast else 1
        for h in range(w.hq):
            if w.gqa_union:
                gs = w.hq // w.hkv
                u = np.zeros(w.nkb(h), bool)
                for h2 in range((h // gs) * gs, (h // gs + 1) * gs):
                    u |= w.head_mask(bm, h2).astype(bool).any(0)
                blk = np.broadcast_to(u, (w.nqb(h), w.nkb(h))).copy()
            else:
                blk = w.head_mask(bm, h).astype(bool).copy()
            bq, bk = w.bq[h], w.bk[h]
            q0 = np.arange(w.nqb(h)) * bq
            k0 = np.arange(w.nkb(h)) * bk
            rq = np.minimum(bq, w.sq - q0).astype(np.float64)
            rk = np.minimum(bk, w.skv - k0).astype(np.float64)
            if w.causal:
                last_q = np.minimum(q0 + bq, w.sq) - 1
                blk &= k0[None, :] <= (last_q + w.causal_offset)[:, None]
            tot += nb * float(rq @ blk.astype(np.float64) @ rk)
    return 4.0 * w.d * tot


def streamed_bytes(w, tile: int = 128) -> float:
    """K and V bytes streamed with no reuse beyond a 128-row query tile: for
    every (batch, head) -- or (batch, kv group) in union mode, whose heads
    share one table -- and every 128-row query tile, 4 * bk * D bytes (bf16 K
    and V rows) per distinct key block that some query block overlapping the
    tile selects and that the causal bound leaves reachable; plus Q, O and
    LSE once. The no-reuse HBM traffic of the forward."""
    esz = 2 if w.dtype == "bf16" else 4
    tot = 0.0
    for bm in range(w.mask_batches):
        nb = w.batch if w.mask_broadcast else 1
        gs = w.hq // w.hkv
        for h in range(w.hq):
            if w.gqa_union and h % gs:
                continue  # the group's first head stands for the group
            if w.gqa_union:
                u = np.zeros(w.nkb(h), bool)
                for h2 in range(h, h + gs):
                    u |= w.head_mask(bm, h2).astype(bool).any(0)
                blk = np.broadcast_to(u, (w.nqb(h), w.nkb(h)))
            else:
                blk = w.head_mask(bm, h).astype(bool)
            bq, bk = w.bq[h], w.bk[h]
            nt = -(-w.sq // tile)
            if bq >= tile:
                tb = blk[np.arange(nt) * tile // bq]
            else:
                per = tile // bq
                pad = nt * per - blk.shape[0]
                tb = np.concatenate([blk, np.zeros((pad, blk.shape[1]), bool)]).reshape(nt, per, -1).any(1)
            k0 = np.arange(w.nkb(h)) * bk
            if w.causal:
                last_q = np.minimum((np.arange(nt) + 1) * tile, w.sq) - 1
                tb = tb & (k0[None, :] <= (last_q + w.causal_offset)[:, None])
            rk = np.minimum(bk, w.skv - k0).astype(np.float64)
            tot += nb * float(tb.astype(np.float64).sum(0) @ rk) * 2 * w.d * esz
    return tot + esz * 2 * w.batch * w.hq * w.sq * w.d + 4 * w.batch * w.hq * w.sq


def pre_union_flops(w) -> float:
    """4 * bq * bk * D per block a head selects itself (before the union),
    causally feasible: the selected work of a union problem before the
    query-block and group unions widen it."""
    tot = 0.0
    for bm in range(w.mask_batches):
        nb = w.batch if w.mask_broadcast else 1
        for h in range(w.hq):
            blk = w.head_mask(bm, h).astype(bool).copy()
            bq, bk = w.bq[h], w.bk[h]
            if w.causal:
                last_q = np.minimum(np.arange(w.nqb(h)) * bq + bq, w.sq) - 1
                blk &= (np.arange(w.nkb(h)) * bk)[None, :] <= (last_q + w.causal_offset)[:, None]
            tot += nb * float(blk.sum()) * bq * bk
    return 4.0 * w.d * tot


# Benchmark configurations reported in the ``configs`` list (forward only).
CONFIGS = ["video_dit", "chunked_prefill", "affine_bs32", "affine_bs64", "affine_bs64_w4096",
           "affine_bs64_w8192", "long_video"]


def forward_rates(w, eff_flops: float, fwd_ms: float, stats: dict, name: str = None) -> dict:
    """Forward rates of one workload against the three rooflines (MFMA, the
    softmax's VALU work, HBM bytes streamed with no reuse beyond a 128-row
    tile), and the bound: the unit the committed counters show busiest
    (matrix core, VALU, or HBM traffic over this time) when they were taken
    on the current kernel source, else the roofline with the longest time."""
    sb = streamed_bytes(w)
    t_mfma = eff_flops / (PEAK_BF16_TFLOPS * 1e12)
    t_alu = eff_flops / (peak_alu_tflops(w.d) * 1e12)
    t_hbm = sb / (PEAK_HBM_GBS * 1e9)
    tflops = eff_flops / (fwd_ms * 1e-3) / 1e12
    gbs = sb / (fwd_ms * 1e-3) / 1e9
    eff_area = eff_flops / (4.0 * w.d)
    out = {"forward_ms": round(fwd_ms, 4), "tflops": round(tflops, 3),
           "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
           "alu_frac": round(tflops / peak_alu_tflops(w.d), 4),
           "streamed_bytes": int(sb), "streamed_gbs": round(gbs, 1),
           "hbm_frac_streamed": round(gbs / PEAK_HBM_GBS, 4),
           "area_ratio": round(stats["executed_tiles"] * stats["tile_q"] * stats["tile_k"] / eff_area, 4)
           if eff_area else None}
    rec = profile_record(name) if name else None
    if rec and "mfma_busy" in rec:
        hbm = rec["hbm_bytes_per_launch"] / (fwd_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)
        busy = {"mfma": rec["mfma_busy"], "alu": rec["valu_busy"], "hbm": hbm}
        out["bound"] = max(busy, key=busy.get)
        out["bound_from"] = "counters"
        out["counters"] = {"mfma_busy": round(rec["mfma_busy"], 4), "valu_busy": round(rec["valu_busy"], 4),
                           "hbm_frac_measured": round(hbm, 4), "clock_ghz": round(rec["clock_ghz"], 3)}
    else:
        out["bound"] = max((t_mfma, "mfma"), (t_alu, "alu"), (t_hbm, "hbm"))[1]
        out["bound_from"] = "model"
    out["frac"] = {"mfma": out["mfma_frac"], "alu": out["alu_frac"], "hbm": out["hbm_frac_streamed"]}[out["bound"]]
    return out


def cpu_baseline(w, q, k, v, target_s: float = 20.0, kv8=None):
    """The fp64 oracle timed on this host's cores over a bounded sample of
    query rows (whole 128-row tiles, spread over heads), in TFLOP/s of
    selected work."""
    import torch
    from oracle import ref

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()

    def rows_for(ntiles, seed=0):
        g = np.random.default_rng(seed)
        out = []
        for t in range(ntiles):
            b = int(g.integers(0, w.batch))
            h = int(g.integers(0, w.hq))
            t0 = int(g.integers(0, max(1, -(-w.sq // 128)))) * 128
            for i in range(t0, min(w.sq, t0 + 128)):
                out.append((b, h, i))
        return np.array(out, np.int64)

    def work(rows):
        # 4 * D FLOPs per allowed (query, key) pair of the sampled rows.
        tot = 0
        cache = {}
        for b, h, i in rows:
            key = (int(b), int(h))
            if key not in cache:
                cache[key] = allowed_keys_per_row(w, *key)
            tot += int(cache[key][i])
        return 4.0 * w.d * tot

    def run(rows):
        if kv8 is None:
            ref.forward(w, qh, kh, vh, mode=1, rows=rows, nthreads=threads)
        else:
            ref.forward_kv8(w, qh, kh, vh, kv8[2].cpu().numpy(), kv8[3].cpu().numpy(), mode=1,
                            rows=rows, nthreads=threads)

    rows = rows_for(8)
    t = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t
    ntiles = max(8, min(20000, int(8 * target_s / max(dt, 1e-3))))
    rows = rows_for(ntiles, seed=1)
    t = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t
    flops = work(rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} query rows ({ntiles} random 128-row tiles) of the {w.name} "
                      f"workload, fp64 block-skipping oracle, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_video")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration forward table")
    ap.add_argument("--regret", action=argparse.BooleanOptionalAction, default=True,
                    help="in the configuration table, also time every candidate regime and "
                         "report the table's regret against the best")
    ap.add_argument("--lut", default=None, help="regime table (default: the packaged gfx950 table)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pipeline", action="store_true",
                    help="also time requests with the next plan overlapping the current forward")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass measurement (dense bf16 workloads only)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run three device copies of a 1 GiB tensor (1 GiB read and 1 GiB "
                         "written per launch), to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs the block-sparse attention path on one GPU; --gpus {args.gpus} "
              "is not supported (each GPU would run its own heads; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_08_amd as bsa

    torch.cuda.set_device(0)
    sel_keep = None
    if args.workload in SELECTED:
        base_name, sel_keep = SELECTED[args.workload]
    elif args.workload in KV8:
        base_name = KV8[args.workload]
    elif args.workload in ACSR:
        base_name = ACSR[args.workload]
    else:
        base_name = args.workload
    if args.calibrate_copy:
        x = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").normal_()
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": 1 << 30,
                          "bytes_written": 1 << 30, "launches": 3}), flush=True)
        return
    w = workload(base_name)
    q, k, v = w.make_qkv(device="cuda")
    kv8 = None
    if args.workload in KV8:
        kv8 = w.make_kv8(k, v)
        k, v = kv8[0], kv8[1]
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    table = torch.from_numpy(np.ascontiguousarray(w.page_table)).cuda() if w.paged else None
    lut = bsa.Lut.load(args.lut or bsa.DEFAULT_LUT)
    prob = w.problem_dict()
    if sel_keep is not None:
        prob["mask_batch_broadcast"] = 0
        mask = torch.empty(bsa.mask_size(prob), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.hq, w.sq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    plan_stream = torch.cuda.Stream()

    acsr = w.acsr if args.workload in ACSR else None

    def make_plan(s):
        if acsr is not None:
            return bsa.plan_acsr(prob, acsr, lut, stream=s)
        return bsa.plan(prob, mask, table, lut, stream=s)

    def step(ev=None, serial=True):
        if sel_keep is not None:
            bsa.select_blocks(prob, q, k, table, keep_tenths=sel_keep, out=mask,
                              stream=stream if serial else plan_stream)
        if serial:
            p = make_plan(stream)
        else:
            p = make_plan(plan_stream)
            ready = torch.cuda.Event()
            ready.record(plan_stream)
            stream.wait_event(ready)
        if ev is not None:
            ev[0].record(stream)
        if kv8 is not None:
            p.forward_kv8(q, k, v, kv8[2], kv8[3], o, lse, stream=stream)
        else:
            p.forward(q, k, v, o, lse, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        return p

    def timed(serial):
        """(ms per step, per-forward HIP-event ms) over args.steps requests."""
        events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
        plans = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            p = step(events[i], serial)
            if serial:
                # Freed in stream order: the next plan on this stream reuses
                # the memory only after this forward has run.
                p.free()
            else:
                plans.append(p)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for p in plans:
            p.free()
        return (t1 - t0) * 1e3 / args.steps, [a.elapsed_time(b) for a, b in events]

    p0 = step()
    stats = p0.stats()
    p0.free()
    eff_flops = effective_flops(w)
    for _ in range(args.warmup):
        step().free()
    torch.cuda.synchronize()

    ms_step, fwd_ms = timed(True)
    fwd_avg = float(np.mean(fwd_ms))
    ms_pipe = timed(False)[0] if args.pipeline else None

    # Plan-only timing (the planner's own cost, one feature readback included
    # for mask plans): host time from the call to its kernels' end, median of
    # 20 after 3 warm-up plans.
    plan_times = []
    for i in range(23):
        torch.cuda.synchronize()
        tp = time.perf_counter()
        p = make_plan(stream)
        torch.cuda.synchronize()
        if i >= 3:
            plan_times.append((time.perf_counter() - tp) * 1e3)
        p.free()
    plan_ms = float(np.median(plan_times))

    select = None
    if sel_keep is not None:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(10)]
        for a, b in ev:
            a.record(stream)
            bsa.select_blocks(prob, q, k, table, keep_tenths=sel_keep, out=mask, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        sel_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        esz = 2 if w.dtype == "bf16" else 4
        # Q and K read once (the heads of a group share their pooled key
        # blocks), one mask byte written per block pair.
        sel_bytes = esz * (q.numel() + w.batch * w.hkv * w.skv * w.d) + mask.numel()
        select = {"ms": round(sel_ms, 4), "keep_tenths": sel_keep, "hbm_bytes": int(sel_bytes),
                  "gbs": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
                  "frac_of_hbm_peak": round(sel_bytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    # Backward over one plan (dense bf16 workloads): bsa_backward calls timed
    # with HIP events on the stream they run on, after a forward that gives O
    # and LSE. FLOPs by the usual five-product count (S recomputed, dP, dV,
    # dK, dQ: 2.5x the forward's); the kernels execute seven products (S and
    # dP are formed once per kernel).
    backward = None
    if not args.no_backward and not w.paged and w.dtype == "bf16" and sel_keep is None and kv8 is None:
        dout = w.make_dout(device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        pb = bsa.plan(prob, mask, table, lut, stream=stream)
        pb.forward(q, k, v, o, lse, stream=stream)
        for _ in range(max(args.warmup, 1)):
            pb.backward(q, k, v, o, lse, dout, dq, dk, dv, stream=stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            pb.backward(q, k, v, o, lse, dout, dq, dk, dv, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        pb.free()
        bwd_tf = 2.5 * eff_flops / (bwd_ms * 1e-3) / 1e12
        backward = {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 3),
                    "flops_convention": "2.5 x forward (S, dP, dV, dK, dQ)",
                    "frac_of_bf16_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                    "executed_tflops": round(3.5 * eff_flops / (bwd_ms * 1e-3) / 1e12, 3),
                    "kernels": ["k_bwd_dq", "k_bwd_dkdv", "k_kv_chunks"]}
        del dout, dq, dk, dv

    value = eff_flops / (ms_step * 1e-3) / 1e12
    achieved = eff_flops / (fwd_avg * 1e-3) / 1e12
    esz = 2 if w.dtype == "bf16" else 4
    compulsory = esz * (q.numel() * 2 + k.numel() + v.numel()) + 4 * lse.numel()
    traffic = measured_traffic(args.workload, None)
    rates = forward_rates(w, eff_flops, fwd_avg, stats, args.workload)
    if rates["bound"] == "hbm":
        # Gather-bound: the no-reuse K/V stream at 8 TB/s takes longer than the
        # selected work at the MFMA peak, so the roofline is HBM bytes.
        roofline = {"bound": "hbm", "achieved": rates["streamed_gbs"], "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": rates["hbm_frac_streamed"], "traffic": traffic,
                    "kernel": "k_attn", "algorithmic_bytes": rates["streamed_bytes"],
                    "algorithmic_bytes_def": "K+V rows streamed per 128-row query tile (no reuse "
                                             "beyond the tile) + Q, O, LSE once",
                    "mfma_frac": rates["mfma_frac"], "compulsory_bytes": compulsory}
    elif rates["bound"] == "alu":
        # The softmax's VALU work per score (exponential at half the FMA
        # rate) bounds it before the matrix cores: D = 64.
        peak = peak_alu_tflops(w.d)
        roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": round(peak, 1),
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                    "kernel": "k_attn", "peak_def": "7.86e12 scores/s (20 VALU cycles per 64 scores "
                    "per SIMD at 2.4 GHz) x 4*D FLOP per score", "mfma_frac": rates["mfma_frac"],
                    "compulsory_bytes": compulsory, "hbm_frac_streamed": rates["hbm_frac_streamed"]}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic, "kernel": "k_attn", "compulsory_bytes": compulsory,
                    "hbm_frac_streamed": rates["hbm_frac_streamed"]}
    roofline["area_ratio"] = rates["area_ratio"]
    roofline["bound_from"] = rates["bound_from"]
    if "counters" in rates:
        roofline["counters"] = rates["counters"]
    if args.workload in HBM_BOUND:
        # Union tables: every head of a group selects the same blocks, so the
        # group reads effective_blocks / G blocks of K and of V once.
        G = w.hq // w.hkv
        bk = int(w.bk[0])
        kv_esz = 1 if kv8 is not None else esz
        kv_bytes = stats["effective_blocks"] // G * bk * w.d * kv_esz * 2
        alg = kv_bytes + esz * 2 * q.numel() + 4 * lse.numel()
        gbs = alg / (fwd_avg * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": "k_attn",
                    "algorithmic_bytes": int(alg)}
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_pipelined": round(ms_pipe, 4) if ms_pipe is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "q_heads": w.hq,
                   "kv_heads": w.hkv, "seqlen_q": w.sq, "seqlen_kv": w.skv, "head_dim": w.d,
                   "block_q": sorted(set(w.bq)), "block_k": sorted(set(w.bk)),
                   "density_pm": stats["density_pm"], "effective_blocks": stats["effective_blocks"],
                   "regime": {k2: stats[k2] for k2 in ("tile_q", "tile_k", "sched", "split", "pack")}},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "forward_ms": round(fwd_avg, 4),
        "forward_tflops": round(achieved, 3),
        "plan_ms": round(plan_ms, 4),
        "effective_flops": eff_flops,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if select is not None:
        line["select"] = select
    if backward is not None:
        line["backward"] = backward
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, kv8=kv8)
    if not args.no_configs:
        del q, k, v, o, lse, mask, table
        torch.cuda.empty_cache()
        line["configs"] = config_table(bsa, lut, args)
    print(json.dumps(line), flush=True)


def config_table(bsa, lut, args):
    """Forward time and rates of every benchmark configuration, measured
    here with HIP events on the launch stream; with regret, also every forced
    regime of a candidate set, and the table's regret against the best."""
    import torch
    out = []
    stream = torch.cuda.current_stream()

    def time_fwd(p, q, k, v, o, lse, reps, warm_ms=0.0):
        for _ in range(max(args.warmup, 1)):
            p.forward(q, k, v, o, lse, stream=stream)
        if warm_ms > 0:  # after an idle stretch (the host baseline), bring the clocks up first
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            while (time.perf_counter() - t0) * 1e3 < warm_ms:
                for _ in range(4):
                    p.forward(q, k, v, o, lse, stream=stream)
                torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            p.forward(q, k, v, o, lse, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    for name in CONFIGS:
        w = workload(name)
        q, k, v = w.make_qkv(device="cuda")
        mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
        table = torch.from_numpy(np.ascontiguousarray(w.page_table)).cuda() if w.paged else None
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.hq, w.sq), dtype=torch.float32, device="cuda")
        p = bsa.plan(w.problem_dict(), mask, table, lut, stream=stream)
        stats = p.stats()
        fwd_ms = time_fwd(p, q, k, v, o, lse, args.steps, warm_ms=200.0)
        p.free()
        eff = effective_flops(w)
        rec = {"workload": name, "density_pm": stats["density_pm"], "effective_flops": eff}
        rec.update(forward_rates(w, eff, fwd_ms, stats, name))
        rec["regime"] = {k2: stats[k2] for k2 in ("tile_q", "tile_k", "sched", "split", "pack")}
        if w.gqa_union:
            pre = pre_union_flops(w)
            rec["pre_union_selected_flops"] = pre
            rec["pre_union_selected_tflops"] = round(pre / (fwd_ms * 1e-3) / 1e12, 3)
        if args.regret:
            # Every candidate regime forced by a one-rule table; the table's own
            # choice is timed again beside them with the same repetitions.
            from block_sparse_attention_08_amd.lut import build_lut
            cands = build_lut.candidates(bool(w.gqa_union))
            # Regimes are compared after the planner has made them valid, so
            # candidates that end up the same plan are timed once, and the
            # table's choice is one of them.
            plans = {}
            for c in [None] + cands:
                try:
                    pc = bsa.plan(w.problem_dict(), mask, table, lut if c is None else bsa.Lut.forced(*c),
                                  stream=stream)
                except bsa.BsaError:
                    continue
                sc = pc.stats()
                # (a split that no row reaches runs as no split)
                key = (sc["tile_q"], sc["tile_k"], sc["sched"],
                       sc["split"] if sc["partial_slots"] > 0 else 0, sc["pack"])
                if c is None:
                    table_key = key
                if key in plans:
                    pc.free()
                else:
                    plans[key] = pc
            times = {}
            reps = max(5, min(20, int(200.0 / max(fwd_ms, 0.05))))  # about 0.2 s per measurement
            # Three interleaved rounds, the order rotated each round so that no
            # regime always runs first; each measurement starts after a short
            # stretch of its own forwards at full clock (a sub-millisecond
            # forward timed right after the host's planning or the previous
            # synchronisation runs up to 10% slow). The best round is kept.
            order = list(plans.items())
            for rnd in range(3):
                for key, pc in order[rnd % len(order):] + order[:rnd % len(order)]:
                    t = time_fwd(pc, q, k, v, o, lse, reps, warm_ms=30.0)
                    times[key] = min(times.get(key, t), t)
            for pc in plans.values():
                pc.free()
            best = min(times, key=times.get)
            rec["regret"] = {"table_ms": round(times[table_key], 4), "best_ms": round(times[best], 4),
                             "best_regime": dict(zip(("tile_q", "tile_k", "sched", "split", "pack"), best)),
                             "regret": round(times[table_key] / times[best] - 1.0, 4),
                             "candidates": len(times)}
        out.append(rec)
        print(f"[config] {name}: {rec['forward_ms']} ms, {rec['tflops']} TFLOP/s, "
              f"mfma {rec['mfma_frac']}, alu {rec['alu_frac']}, hbm(streamed) {rec['hbm_frac_streamed']}, "
              f"bound {rec['bound']} ({rec['bound_from']}), area {rec['area_ratio']}" + (f", regret {rec['regret']['regret']}" if args.regret else ""),
              file=sys.stderr, flush=True)
        del q, k, v, o, lse, mask, table
        torch.cuda.empty_cache()
    return out

if __name__ == "__main__":
    main()
