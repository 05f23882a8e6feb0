"""Build the regime lookup table by profiling on the local GPU.

Tessera (abstract) picks an execution plan per request through a lookup table
built from offline profiling. Table format 2: each rule also matches a range of
the query length, so decode and short chunks get their own regime. This script is
that offline step for libbsa: each mask-shape bucket has a few seeded training
workloads (other seeds, window widths, densities, shapes and block sizes than
the benchmark configurations, which stay held out); every candidate regime
(tile rows, key tile, schedule, split threshold, GQA packing) is timed on each
of them, one request = bsa_plan + bsa_forward, and the bucket's rule is the
regime with the smallest geometric mean of its time relative to the best
regime of each training workload. Rules are written in bucket order, followed
by a catch-all default.

    python -m block_sparse_attention_08_amd.lut.build_lut [--out PATH] [--steps N]
        [--only NAME,NAME --base PATH]

With --only, just the named buckets are profiled again; every other bucket
keeps its rule and comment lines from the table at --base (default: the
packaged table), in bucket order.
"""
from __future__ import annotations

import argparse
import itertools
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BIG = "1000000"
BIGIMB = "100000000"


ANYSQ = "  0 " + BIG


def buckets():
    """(name, rule key fields and ranges, training workload factories,
    candidate regimes or None for the default set). Rules carry a fifth range
    on the query length (table format 2); first match wins. The training
    workloads differ from the benchmark configurations (held out) in seed,
    shape, window, density or block size."""
    from block_sparse_attention_08_amd import workloads as W
    return [
        # Decode and short chunks: a few queries per sequence over a long paged
        # cache with GQA union tables (split-KV keeps every CU busy).
        ("decode", "* bf16 1 1  0 " + BIG + "  0 " + BIG + "  0 " + BIG + "  0 " + BIGIMB + "  1 64",
         [lambda: W.decode(seed=11), lambda: W.decode(batch=8, q_len=4, context=32768, seed=12),
          lambda: W.decode(batch=32, q_len=2, context=16384, seed=13)], decode_candidates()),
        # GQA union over a paged cache (chunked prefill).
        ("gqa-union", "* bf16 1 *  0 " + BIG + "  0 " + BIG + "  0 " + BIG + "  0 " + BIGIMB + ANYSQ,
         [lambda: W.chunked_prefill(chunk=2048, context=32768, seed=11),
          lambda: W.chunked_prefill(chunk=4096, context=49152, keep_tenths=2, seed=12),
          lambda: W.chunked_prefill(hq=16, hkv=4, chunk=8192, context=65536, seed=13)], None),
        # Large blocks (>= 128), D=128, low density: 3-D video windows.
        ("video-128", "128 bf16 0 *  128 " + BIG + "  128 " + BIG + "  0 400  0 " + BIGIMB + ANYSQ,
         [lambda: W.video_dit(seed=11), lambda: W.video_dit(heads=16, p_global=0.06, seed=12),
          lambda: W.video_dit(heads=24, grid=(16, 30, 40), window=(1, 1, 1), seed=13)], None),
        # Mixed block sizes with uneven rows (long video), D=128.
        ("mixed-128", "128 bf16 0 *  16 127  16 " + BIG + "  0 " + BIG + "  0 " + BIGIMB + ANYSQ,
         [lambda: W.long_video(heads=20, seed=11), lambda: W.long_video(heads=24, grid=(16, 48, 80), seed=12),
          lambda: W.long_video(heads=16, p_heavy=0.10, seed=13)], None),
        # 32-token blocks, D=64, low density (regular patterns; tiles merge
        # four query blocks and two key blocks).
        ("regular-32-sparse", "64 bf16 0 *  16 32  16 32  0 200  0 " + BIGIMB + ANYSQ,
         [lambda: W.affine(bs=32, window=768, s=16384), lambda: W.affine(bs=32, window=512, s=8192, batch=4),
          lambda: W.affine(bs=32, window=1536, s=32768, batch=1)], None),
        # Small blocks, D=64, low density (regular patterns).
        ("regular-64-sparse", "64 bf16 0 *  16 " + BIG + "  16 " + BIG + "  0 200  0 " + BIGIMB + ANYSQ,
         [lambda: W.affine(bs=64, window=512, s=16384), lambda: W.affine(bs=64, window=768, s=8192, batch=4),
          lambda: W.affine(bs=64, window=2048, s=32768, batch=1)], None),
        # Small blocks, D=64, dense windows.
        ("regular-64-dense", "64 bf16 0 *  16 " + BIG + "  16 " + BIG + "  201 " + BIG + "  0 " + BIGIMB + ANYSQ,
         [lambda: W.affine(bs=64, window=6144), lambda: W.affine(bs=32, window=4096, s=8192),
          lambda: W.affine(bs=64, window=12288, s=32768, batch=1)], None),
    ]


def decode_candidates():
    """64-key tiles (the cache's 64-token pages hold whole tiles), finer splits."""
    out = []
    for sched, split, pack in itertools.product(("local", "lpt"), (0, 16, 24, 32, 48, 64), (2, 1, 0)):
        out.append((128, 64, sched, split, pack))
    return out


def candidates(union):
    """Candidate regimes: union problems (union True) also try GQA packing
    (pack 1 and 2); non-union problems (False) have none; None gives both
    sets (packing is skipped for non-union workloads when timed)."""
    out = []
    for tq, tk, sched, split in itertools.product((128, 256), (64, 128), ("local", "lpt", "dealt"),
                                                  (0, 128, 256)):
        if tq == 256 and tk == 128:
            continue  # the planner turns it into 256 x 64
        for pack in ((0,) if union is False else (0, 1, 2)):
            out.append((tq, tk, sched, split, pack))
    return out


def effective_regime(bsa, w, tensors, regime):
    """The regime the planner actually runs for this workload: (Tq, Tk,
    schedule, split, pack) after validation, with split 0 when no row is
    split."""
    q, k, v, mask, table, o, lse = tensors
    p = bsa.plan(w.problem_dict(), mask, table, bsa.Lut.forced(*regime))
    st = p.stats()
    p.free()
    sched = ("local", "lpt", "dealt")[st["sched"]]
    return (st["tile_q"], st["tile_k"], sched, st["split"] if st["partial_slots"] > 0 else 0, st["pack"])


def time_regime(bsa, w, tensors, regime, steps):
    import torch
    q, k, v, mask, table, o, lse = tensors
    tq, tk, sched, split, pack = regime
    lut = bsa.Lut.forced(tq, tk, sched, split, pack)
    prob = w.problem_dict()
    p = bsa.plan(prob, mask, table, lut)
    p.forward(q, k, v, o, lse)
    torch.cuda.synchronize()
    p.free()
    torch.cuda.synchronize()
    t = time.perf_counter()
    plans = []
    for _ in range(steps):
        p = bsa.plan(prob, mask, table, lut)
        p.forward(q, k, v, o, lse)
        plans.append(p)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / steps
    for p in plans:
        p.free()
    return dt


def kept_buckets(text: str) -> dict:
    """Per bucket name, its lines in an existing table: the comment lines
    that start with "# name:" up to and including the bucket's rule line."""
    out, cur = {}, None
    for line in text.splitlines():
        if line.startswith("# ") and ":" in line and not line.startswith("#   "):
            name = line[2:].split(":")[0]
            if " " not in name:
                cur = name
                out[cur] = []
        if cur is not None:
            out[cur].append(line)
            if line.startswith("rule "):
                cur = None
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "gfx950.lut"))
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--only", default="", help="comma-separated bucket names to profile again")
    ap.add_argument("--base", default=os.path.join(HERE, "gfx950.lut"))
    args = ap.parse_args()
    only = {n for n in args.only.split(",") if n}
    kept = kept_buckets(open(args.base).read()) if only else {}
    if only and not only <= {b[0] for b in buckets()}:
        raise SystemExit(f"unknown bucket in --only: {sorted(only)}")
    import torch
    import block_sparse_attention_08_amd as bsa

    dev = torch.cuda.get_device_properties(0)
    lines = ["bsa-lut 2",
             f"# Built by block_sparse_attention_08_amd/lut/build_lut.py on {dev.name} "
             f"({dev.multi_processor_count} CUs), {args.steps} timed requests per regime.",
             "#   rule D dtype union paged bq_lo bq_hi bk_lo bk_hi dens_lo dens_hi imb_lo imb_hi "
             "sq_lo sq_hi -> Tq Tk sched split pack",
             "# Each rule is the regime with the best geometric-mean request time (bsa_plan +"
             " bsa_forward) over its bucket's training workloads; first match wins."]
    for name, key, makers, cands in buckets():
        if only and name not in only:
            lines += kept[name]
            continue
        cands = cands or candidates(None)
        rel = {c: [] for c in cands}
        descr = []
        for make in makers:
            w = make()
            q, k, v = w.make_qkv(device="cuda")
            mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
            table = torch.from_numpy(np.ascontiguousarray(w.page_table)).cuda() if w.paged else None
            o = torch.empty_like(q)
            lse = torch.empty((w.batch, w.hq, w.sq), dtype=torch.float32, device="cuda")
            tensors = (q, k, v, mask, table, o, lse)
            # Regimes that give the same plan execute alike: a split that no
            # row reaches is no split, and the planner makes every regime
            # valid for the problem. Each distinct effective regime is timed
            # once (the better of two rounds) and stands for its nominal ones.
            eff_of, timed = {}, {}
            for reg in cands:
                if reg[4] and not w.gqa_union:
                    continue
                eff_of[reg] = effective_regime(bsa, w, tensors, reg)
            for rnd in range(2):
                for e in sorted(set(eff_of.values()), key=str):
                    dt = time_regime(bsa, w, tensors, e, args.steps)
                    timed[e] = min(timed.get(e, dt), dt)
            res = {reg: timed[e] for reg, e in eff_of.items()}
            for e, dt in sorted(timed.items(), key=lambda x: x[1]):
                print(f"[lut] {name} {w.name} B={w.batch} Hq={w.hq} S={w.sq}/{w.skv}: {e} "
                      f"{dt * 1e3:.3f} ms", flush=True)
            fastest = min(res.values())
            for reg, dt in res.items():
                rel[reg].append(dt / fastest)
            descr.append(f"{w.name} B={w.batch} Hq={w.hq} S={w.sq}/{w.skv} D={w.d} "
                         f"density {1000 * int(w.mask.sum()) // max(1, w.mask.size)}pm")
            del q, k, v, o, lse, mask, table
            torch.cuda.empty_cache()
        score = {reg: float(np.exp(np.mean(np.log(r)))) for reg, r in rel.items() if len(r) == len(makers)}
        # Among regimes within 1% of the best score, take the simplest one
        # (no split, 128-row and 64-key tiles, row order, packing).
        best_score = min(score.values())
        close = [(sc, reg) for reg, sc in score.items() if sc <= best_score * 1.01]
        simplicity = lambda reg: (reg[3] != 0, reg[0] != 128, reg[1] != 64, reg[2] != "local", reg[4] == 0)
        sc, best = min(close, key=lambda x: (simplicity(x[1]), x[0]))
        tq, tk, sched, split, pack = best
        lines.append(f"# {name}: trained on " + "; ".join(descr))
        lines.append(f"#   geometric-mean time relative to each workload's best: {sc:.3f} "
                     f"(best regime overall {best_score:.3f})")
        lines.append(f"rule {key} -> {tq} {tk} {sched} {split} {pack}")
    lines.append("# Anything else: 128 x 64 tiles, row order, no split, GQA packing when possible.")
    lines.append("rule * * * * 0 " + BIG + " 0 " + BIG + " 0 " + BIG + " 0 " + BIGIMB + ANYSQ + " -> 128 64 local 0 1")
    text = "\n".join(lines) + "\n"
    bsa.Lut.parse(text)  # validate
    with open(args.out, "w") as f:
        f.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
