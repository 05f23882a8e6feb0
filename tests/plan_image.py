"""Decoder of the canonical plan image, and the element-level expansion used by
the planner tests. Test infrastructure: written from the plan format, shares
no code with either planner.

Image layout (little-endian): the 8-byte magic ``BSAPLAN1``; 40 int64 header
words; int32 bq[Hq], bk[Hq], query-block interleave[Hq], key-block
interleave[Hq]; int64
features[mask batches][Hq][4]; int32
list_off[nlists + 1]; int32 kt[nent]; int32 page[nent] (paged only); uint32
live[nent]; int32 rows[nrows][2]; int32 items[nitems][4]; int32
combine[ncomb][3].
"""
from __future__ import annotations

import dataclasses

import numpy as np

HDR = ["version", "batch", "hq", "hkv", "sq", "skv", "d", "dtype", "causal", "offset",
       "union", "paged", "page_size", "pages_per_seq", "broadcast", "tq", "tk", "sched",
       "split", "pack", "nqt", "nkt", "nlists", "nent", "nrows", "nitems", "nslots", "ncomb",
       "total_nnz", "total_blocks", "density_pm", "imb16", "min_bq", "min_bk", "nlb"]


@dataclasses.dataclass
class Plan:
    h: dict
    bq: np.ndarray
    bk: np.ndarray
    qil: np.ndarray
    kil: np.ndarray
    feat: np.ndarray
    list_off: np.ndarray
    kt: np.ndarray
    page: np.ndarray
    live: np.ndarray
    rows: np.ndarray
    items: np.ndarray
    comb: np.ndarray


def decode(img: bytes) -> Plan:
    assert img[:8] == b"BSAPLAN1", img[:8]
    pos = 8
    hdr = np.frombuffer(img, np.int64, 40, pos)
    pos += 320
    h = {k: int(hdr[i]) for i, k in enumerate(HDR)}

    def take(dtype, n):
        nonlocal pos
        a = np.frombuffer(img, dtype, n, pos)
        pos += a.nbytes
        return a

    hq = h["hq"]
    bq, bk, qil, kil = (take(np.int32, hq) for _ in range(4))
    nbm = 1 if h["broadcast"] else h["batch"]
    feat = take(np.int64, nbm * hq * 4).reshape(nbm, hq, 4)
    list_off = take(np.int32, h["nlists"] + 1)
    kt = take(np.int32, h["nent"])
    page = take(np.int32, h["nent"]) if h["paged"] else None
    live = take(np.uint32, h["nent"])
    rows = take(np.int32, 2 * h["nrows"]).reshape(-1, 2)
    items = take(np.int32, 4 * h["nitems"]).reshape(-1, 4)
    comb = take(np.int32, 3 * h["ncomb"]).reshape(-1, 3)
    assert pos == len(img), (pos, len(img))
    return Plan(h, bq, bk, qil, kil, feat, list_off, kt, page, live, rows, items, comb)


def qblock(t: int, iq: int, s: int, mq: int, nq: int) -> int:
    """Logical query block of sub-block iq of tile t under interleave s
    (written from the plan format: full groups of s*mq blocks hold s tiles
    whose blocks are s apart; consecutive blocks after the last full group)."""
    g = s * mq
    full = nq // g
    if t < full * s:
        return (t // s) * g + iq * s + t % s
    return full * g + (t - full * s) * mq + iq


def key_ranges(p: Plan, head: int, kt: int):
    """[(k0, k1, ik)]: the keys of key tile kt of a head, per key sub-block
    ik (a tile merging key blocks lists each at the position its interleave
    gives it; a tile within one key block is one range)."""
    h = p.h
    tk, skv = h["tk"], h["skv"]
    bk = int(p.bk[head])
    if bk >= tk:
        return [(kt * tk, min(skv, (kt + 1) * tk), 0)]
    mk, nk = tk // bk, -(-skv // bk)
    out = []
    for ik in range(mk):
        kb = qblock(kt, ik, int(p.kil[head]), mk, nk)
        if kb < nk:
            out.append((kb * bk, min(skv, (kb + 1) * bk), ik))
    return out


def row_geometry(p: Plan, r: int):
    """(b, list of (head, q0, q1, iq)) covered by physical row r: query rows
    [q0, q1) of head, which are query sub-block iq of the tile (None: the
    sub-block follows from the position, as in a contiguous tile).

    A packed row covers all heads of a group over Tq/G positions; the kernel's
    four 32-row waves take heads in order. A tile that merges query blocks
    lists each merged block, at the position the interleave gives it.
    """
    h = p.h
    nqt = h["nqt"]
    gs = h["hq"] // h["hkv"]
    nh = h["hkv"] if h["pack"] else h["hq"]
    qt, hh, b = r % nqt, (r // nqt) % nh, r // (nqt * nh)
    if h["pack"]:
        tr = h["tq"] // gs
        q0, q1 = qt * tr, min(h["sq"], (qt + 1) * tr)
        return b, [(hh * gs + j, q0, q1, None) for j in range(gs)]
    bq = int(p.bq[hh])
    if not h["union"] and bq < h["tq"]:
        mq, nq = h["tq"] // bq, -(-h["sq"] // bq)
        out = []
        for iq in range(mq):
            qb = qblock(qt, iq, int(p.qil[hh]), mq, nq)
            if qb < nq:
                out.append((hh, qb * bq, min(h["sq"], (qb + 1) * bq), iq))
        return b, out
    q0, q1 = qt * h["tq"], min(h["sq"], (qt + 1) * h["tq"])
    return b, [(hh, q0, q1, None)]


def expand_row(p: Plan, r: int, head: int, q0: int, q1: int, iq0=None) -> np.ndarray:
    """Element-level allowed matrix [q1-q0][skv] that the plan makes the kernel
    compute for one head of row r: live bit of the sub-block, causal, bounds.
    iq0: the query sub-block of rows [q0, q1) when given by row_geometry."""
    h = p.h
    tq, tk, skv = h["tq"], h["tk"], h["skv"]
    bq, bk = int(p.bq[head]), int(p.bk[head])
    union = h["union"]
    gs = h["hq"] // h["hkv"]
    tr = tq // gs if h["pack"] else tq
    qt = (r % h["nqt"])
    out = np.zeros((q1 - q0, skv), bool)
    e0, e1 = p.rows[r]
    aq = tq if union else min(bq, tq)
    ak = min(bk, tk)
    mk = tk // ak
    qi = np.arange(q0, q1)
    for e in range(e0, e1):
        kt, live = int(p.kt[e]), int(p.live[e])
        if union:
            iq = np.zeros_like(qi)
        elif iq0 is not None:
            iq = np.full_like(qi, iq0)
        else:
            iq = (qi - qt * tr) // aq
        for k0, k1, ik_b in key_ranges(p, head, kt):
            kj = np.arange(k0, k1)
            # sub-block within the tile: the range's own index when the tile
            # merges key blocks, else the offset within a contiguous tile
            ik = np.full_like(kj, ik_b) if bk < tk else (kj - k0) // ak
            bit = (live >> (iq[:, None] * mk + ik[None, :])) & 1
            ok = bit.astype(bool)
            if h["causal"]:
                ok &= kj[None, :] <= qi[:, None] + h["offset"]
            assert not (out[:, k0:k1] & ok).any(), "key tile listed twice"
            out[:, k0:k1] |= ok
    return out
