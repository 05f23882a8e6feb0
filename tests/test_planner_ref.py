"""Pins of the reference planner (no GPU).

The plan is pinned against the mask it was built from: expanding every entry
of every row back to elements (live bit of the sub-block, causal bound, sequence
bounds) must give exactly the element-level mask of the definition, with no key
tile listed twice. The work list must cover each row's entries exactly once.
"""
import itertools

import numpy as np
import pytest

from block_sparse_attention_08_amd import workloads as W
from tests.plan_image import decode, expand_row, qblock, row_geometry
from tests.test_oracle_pins import element_mask


def check_worklist(p):
    h = p.h
    items, rows = p.items, p.rows
    assert len(items) == h["nitems"] and (np.diff(p.list_off) >= 0).all()
    # Entries within each list ascending, kt in range.
    for l in range(h["nlists"]):
        kt = p.kt[p.list_off[l]:p.list_off[l + 1]]
        assert (np.diff(kt) > 0).all()
    assert ((p.kt >= 0) & (p.kt < h["nkt"])).all()
    assert (p.live != 0).all()
    # Items partition each row's range; split rows use consecutive slots.
    by_row = {}
    for r, e0, e1, slot in items:
        by_row.setdefault(int(r), []).append((int(e0), int(e1), int(slot)))
    assert sorted(by_row) == list(range(h["nrows"]))
    comb = {int(r): (int(s0), int(n)) for r, s0, n in p.comb}
    for r, its in by_row.items():
        its.sort()
        assert its[0][0] == rows[r][0] and its[-1][1] == rows[r][1]
        for a, b in zip(its, its[1:]):
            assert a[1] == b[0]
        if len(its) > 1:
            s0, n = comb[r]
            assert n == len(its) and [s for _, _, s in its] == list(range(s0, s0 + n))
            assert all(e1 - e0 <= h["split"] for e0, e1, _ in its)
        else:
            assert its[0][2] == -1 and r not in comb
    if h["sched"] == 1:
        ln = np.minimum(items[:, 2] - items[:, 1], 1023)
        assert (np.diff(ln) <= 0).all()
        # Stable: equal keys keep the unsorted order (row, then chunk).
        for key in np.unique(ln):
            sel = items[ln == key]
            order = sel[:, 0].astype(np.int64) * (1 << 31) + sel[:, 1]
            assert (np.diff(order) > 0).all()


def check_elements(w, p):
    for r in range(p.h["nrows"]):
        b, heads = row_geometry(p, r)
        for head, q0, q1, iq in heads:
            got = expand_row(p, r, head, q0, q1, iq)
            want = element_mask(w, b, head)[q0:q1]
            assert np.array_equal(got, want), (r, head, q0)


def test_exhaustive_4x4_masks(ref):
    """Every 4x4 logical mask, for keep / merge / subdivide on both sides."""
    allm = np.array(list(itertools.product([0, 1], repeat=16)), np.uint8)  # [65536][16]
    for bq, bk, tk in [(32, 32, 64), (64, 16, 64), (128, 128, 64), (256, 64, 128),
                       (16, 128, 128), (512, 32, 64)]:
        B = allm.shape[0]
        w = W.Workload("ex", B, 1, 1, 4 * bq, 4 * bk, 64, "bf16", [bq], [bk],
                       np.ascontiguousarray(allm.reshape(-1)))
        p = decode(ref.plan(w, force=[128, tk, 0, 0, 0]))
        h = p.h
        assert (h["tq"], h["tk"]) == (128, tk)
        aq, ak = min(bq, 128), min(bk, tk)
        mq, mk = 128 // aq, tk // ak
        naq, nak = 4 * bq // aq, 4 * bk // ak
        cov = np.zeros((B, naq, nak), np.int32)
        nqt = h["nqt"]
        ent_list = np.repeat(np.arange(h["nlists"]), np.diff(p.list_off))
        b_of = ent_list // nqt
        qt_of = ent_list % nqt
        s_of, sk_of = int(p.qil[0]), int(p.kil[0])
        for iq in range(mq):
            for ik in range(mk):
                bit = (p.live >> np.uint32(iq * mk + ik)) & 1
                sel = bit.astype(bool)
                # (tiles merge query and key sub-blocks through the head's
                # interleaves)
                a = np.array([qblock(int(t), iq, s_of, mq, naq) if bq < 128 else int(t) * mq + iq
                              for t in qt_of[sel]], np.int64)
                c = np.array([qblock(int(kt), ik, sk_of, mk, nak) if bk < tk else int(kt) * mk + ik
                              for kt in p.kt[sel]], np.int64)
                np.add.at(cov, (b_of[sel], a, c), 1)
        blk = allm.reshape(B, 4, 4)
        want = blk[:, (np.arange(naq) * aq) // bq][:, :, (np.arange(nak) * ak) // bk]
        assert cov.max() <= 1
        assert np.array_equal(cov.astype(bool), want.astype(bool)), (bq, bk, tk)
        # Row ranges equal the list of the row (non-union: one list per row).
        assert np.array_equal(p.rows[:, 0], p.list_off[:-1])
        assert np.array_equal(p.rows[:, 1], p.list_off[1:])


CASES = {
    "merge_causal": dict(batch=2, hq=3, sq=300, skv=333, bq=[16, 32, 64], bk=[16, 32, 64],
                         density=0.3, empty_rows=0.2, causal=True, causal_offset=20),
    "subdivide": dict(batch=1, hq=2, sq=700, skv=650, bq=256, bk=512, density=0.5),
    "broadcast": dict(batch=3, hq=2, sq=260, skv=200, bq=32, bk=64, density=0.4,
                      mask_broadcast=True),
    "union_causal": dict(batch=2, hq=4, hkv=1, sq=300, skv=700, bq=64, bk=32, density=0.05,
                         gqa_union=True, causal=True, causal_offset=400),
    "union_paged": dict(batch=2, hq=8, hkv=2, sq=200, skv=900, bq=128, bk=128, density=0.08,
                        gqa_union=True, causal=True, causal_offset=700, paged=True,
                        page_size=64),
    "paged_plain": dict(batch=2, hq=2, sq=100, skv=500, bq=64, bk=64, density=0.4,
                        paged=True, page_size=128),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("regime", [(128, 64, 0, 0, 1), (128, 128, 1, 3, 1), (128, 64, 1, 2, 0),
                                    (256, 64, 0, 2, 1), (256, 128, 1, 0, 0)])
def test_plan_element_coverage(ref, case, regime):
    w = W.random_problem(d=64, seed=sorted(CASES).index(case), **CASES[case])
    img = ref.plan(w, force=list(regime))
    p = decode(img)
    check_worklist(p)
    check_elements(w, p)
    if w.paged:
        lb = np.repeat(np.arange(p.h["nlists"]), np.diff(p.list_off)) // (
            w.hkv if w.gqa_union else w.hq * p.h["nqt"])
        want = w.page_table[lb, (p.kt * p.h["tk"]) // w.page_size]
        assert np.array_equal(p.page, want)
    assert ref.plan(w, force=list(regime)) == img   # deterministic


def test_pack_mode_geometry(ref):
    w = W.random_problem(batch=1, hq=8, hkv=2, sq=200, skv=600, bq=64, bk=64, density=0.1,
                         gqa_union=True, causal=True, causal_offset=400, d=64, seed=3)
    p = decode(ref.plan(w, force=[128, 64, 0, 0, 1]))
    assert p.h["pack"] == 1 and p.h["nqt"] == -(-200 // 32)
    assert p.h["nrows"] == 2 * p.h["nqt"]
    check_elements(w, p)
    # Group size 3 cannot pack into four 32-row waves: falls back to per-head rows.
    w3 = W.random_problem(batch=1, hq=6, hkv=2, sq=100, skv=300, bq=64, bk=64, density=0.1,
                          gqa_union=True, d=64, seed=4)
    assert decode(ref.plan(w3, force=[128, 64, 0, 0, 1])).h["pack"] == 0
    # Interleaved packing (pack 2) is an in-tile row order: the plan's rows,
    # lists and items are those of pack 1.
    p2 = decode(ref.plan(w, force=[128, 64, 0, 0, 2]))
    assert p2.h["pack"] == 2
    for f in ("list_off", "kt", "live", "rows", "items"):
        assert np.array_equal(getattr(p2, f), getattr(p, f)), f
    assert decode(ref.plan(w3, force=[128, 64, 0, 0, 2])).h["pack"] == 0
    with pytest.raises(ValueError):
        ref.plan(w, force=[128, 64, 0, 0, 3])


def test_regime_adjustments(ref):
    # Paged with 64-token pages forces 64-key tiles.
    w = W.random_problem(batch=1, hq=2, sq=64, skv=256, bq=64, bk=64, paged=True,
                         page_size=64, d=64, seed=5)
    assert decode(ref.plan(w, force=[128, 128, 0, 0, 0])).h["tk"] == 64
    # 16x16 blocks cannot use 128-key tiles (8 x 8 live bits > 32).
    w = W.random_problem(batch=1, hq=1, sq=64, skv=256, bq=16, bk=16, d=64, seed=6)
    assert decode(ref.plan(w, force=[128, 128, 0, 0, 0])).h["tk"] == 64
    # 256-row tiles use 64 keys; 16-row blocks cannot merge 16 ways and 4 ways at once.
    w = W.random_problem(batch=1, hq=1, sq=512, skv=256, bq=64, bk=64, d=64, seed=8)
    h = decode(ref.plan(w, force=[256, 128, 0, 0, 0])).h
    assert (h["tq"], h["tk"]) == (256, 64)
    w = W.random_problem(batch=1, hq=1, sq=512, skv=256, bq=16, bk=16, d=64, seed=9)
    h = decode(ref.plan(w, force=[256, 64, 0, 0, 0])).h
    assert (h["tq"], h["tk"]) == (128, 64)
    # fp32 always uses 128 x 64 tiles.
    w = W.random_problem(batch=1, hq=1, sq=512, skv=256, bq=64, bk=64, d=64, dtype="f32", seed=10)
    h = decode(ref.plan(w, force=[256, 128, 0, 0, 0])).h
    assert (h["tq"], h["tk"]) == (128, 64)
    # Unsupported block size.
    w = W.random_problem(batch=1, hq=1, sq=64, skv=64, bq=48, bk=64, d=64, seed=7)
    with pytest.raises(ValueError):
        ref.plan(w)


LUT = """\
bsa-lut 1
# D dtype union paged bq bq bk bk dens dens imb imb -> Tq Tk sched split pack
rule 128 bf16 0 0  128 512  128 512  0 199  0 100000 -> 128 128 lpt 40 0
rule *   *    1 *  0 1000   0 1000   0 1000 0 100000 -> 128 64 local 0 1
rule *   *    * *  0 1000   0 1000   0 1000 0 100000 -> 128 64 lpt 7 0
"""


def test_lut_rules_first_match(ref):
    w = W.random_problem(batch=1, hq=2, sq=512, skv=512, bq=128, bk=128, d=128, density=0.1,
                         seed=8)
    h = decode(ref.plan(w, lut_text=LUT)).h
    assert (h["tk"], h["sched"], h["split"], h["pack"]) == (128, 1, 40, 0)
    assert h["density_pm"] < 200
    w = W.random_problem(batch=1, hq=2, sq=512, skv=512, bq=128, bk=128, d=128, density=0.6,
                         seed=8)
    h = decode(ref.plan(w, lut_text=LUT)).h
    assert (h["tk"], h["sched"], h["split"]) == (64, 1, 7)
    h = decode(ref.plan(w)).h    # no table: built-in default
    assert (h["tq"], h["tk"], h["sched"], h["split"]) == (128, 64, 0, 0)
    for bad in ["", "bsa-lut 3\n", "bsa-lut 1\nrule 1 2 3\n",
                "bsa-lut 2\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 64 local 0 0\n",
                "bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 96 local 0 0\n",
                "bsa-lut 1\nrule * x * * 0 1 0 1 0 1 0 1 -> 128 64 local 0 0\n"]:
        with pytest.raises(ValueError):
            ref.plan(w, lut_text=bad)


LUT2 = """\
bsa-lut 2
# ... sq_lo sq_hi -> Tq Tk sched split pack
rule * * * *  0 1000  0 1000  0 1000  0 100000  1 64 -> 128 64 local 32 0
rule * * * *  0 1000  0 1000  0 1000  0 100000  0 1000000 -> 128 64 lpt 5 0
"""

LUT_DEALT = """\
bsa-lut 1
rule * * * *  0 1000  0 1000  0 1000  0 100000 -> 128 64 dealt 3 0
"""


def test_lut_dealt_schedule(ref):
    """'dealt' is schedule 2: the plan's items stay in row order (the kernel
    deals them to the XCDs in blocks); everything else equals 'local'."""
    w = W.random_problem(batch=1, hq=3, sq=700, skv=900, bq=64, bk=64, d=64, density=0.4,
                         seed=21)
    pd = decode(ref.plan(w, lut_text=LUT_DEALT))
    pl = decode(ref.plan(w, lut_text=LUT_DEALT.replace("dealt", "local")))
    assert (pd.h["sched"], pd.h["split"]) == (2, 3) and pl.h["sched"] == 0
    assert np.array_equal(pd.items, pl.items)
    assert {k: v for k, v in pd.h.items() if k != "sched"} == {k: v for k, v in pl.h.items() if k != "sched"}


def test_lut_version2_query_length_range(ref):
    """Format 2 adds a range on Sq: the first rule applies to 1..64 queries only."""
    for sq, want in ((1, (0, 32)), (64, (0, 32)), (65, (1, 5)), (300, (1, 5))):
        w = W.random_problem(batch=1, hq=2, sq=sq, skv=700, bq=64, bk=64, d=64, density=0.5,
                             seed=10)
        h = decode(ref.plan(w, lut_text=LUT2)).h
        assert (h["sched"], h["split"]) == want, (sq, h["sched"], h["split"])


def test_features_in_header(ref):
    w = W.random_problem(batch=2, hq=2, sq=300, skv=300, bq=[32, 64], bk=[64, 32], d=64,
                         density=0.25, empty_rows=0.3, seed=9)
    p = decode(ref.plan(w))
    f = ref.features(w)
    assert np.array_equal(p.feat, f)
    nnz = int(f[..., 0].sum())
    tot = sum(w.nqb(h) * w.nkb(h) for h in range(2)) * 2
    assert p.h["total_nnz"] == nnz and p.h["total_blocks"] == tot
    assert p.h["density_pm"] == 1000 * nnz // tot
    imb = max(16 * f[b, h, 1] * w.nqb(h) // f[b, h, 0] for b in range(2) for h in range(2))
    assert p.h["imb16"] == imb and (p.h["min_bq"], p.h["min_bk"]) == (32, 32)


# ---- query-block interleave ----

def interleave_choice(w, h, tq=128):
    """The interleave the plan specification gives head h, computed here from
    its definition: among s in {1, 2, 4, 8} with s * mq <= nq, the one whose
    tiles list the fewest key blocks (summed over mask batches), smallest on
    ties; 1 for union plans, unmerged heads and blocks under 32 rows."""
    bq = w.bq[h]
    if w.gqa_union or bq >= tq or bq < 32:
        return 1
    mq, nq = tq // bq, -(-w.sq // bq)
    masks = [w.head_mask(bm, h).astype(bool) for bm in range(w.mask_batches)]

    def cost(s):
        nt = -(-nq // mq)
        qbs = np.array([[qblock(t, iq, s, mq, nq) for iq in range(mq)] for t in range(nt)])
        tot = 0
        for m in masks:
            mp = np.concatenate([m, np.zeros((1, m.shape[1]), bool)])  # row nq: no block
            tot += int(mp[np.minimum(qbs, nq)].any(1).sum())
        return tot

    best, bc = 1, cost(1)
    for s in (2, 4, 8):
        if s * mq > nq:
            break
        c = cost(s)
        if c < bc:
            best, bc = s, c
    return best


def test_interleave_dilated_pattern(ref):
    """A dilated pattern (key block = query block mod 8) gathers query blocks
    of one residue into a tile: every tile lists each of its key tiles for
    all its query blocks, half as many entries as contiguous merging."""
    w = W.affine(bs=64, batch=1, heads=3, s=4096, window=256, d=64)
    p = decode(ref.plan(w, force=[128, 64, 0, 0, 0]))
    assert list(p.qil) == [interleave_choice(w, h) for h in range(3)] == [1, 8, 1]
    check_worklist(p)
    check_elements(w, p)
    nqt = p.h["nqt"]
    for r in range(nqt, 2 * nqt):  # the dilated head: 64 key blocks, 8 per residue
        e0, e1 = p.rows[r]
        assert e1 - e0 == 64 // 8
        assert (p.live[e0:e1] == 3).all()  # both query sub-blocks live in every entry


@pytest.mark.parametrize("seed", range(6))
def test_interleave_choice_random(ref, seed):
    """Heads with planted periodic rows (periods 2, 4, 8) plus noise, merged
    blocks of 32 and 64 rows, causal or not, per-batch masks: the planner's
    interleave equals the definition's, and the plan covers the mask exactly."""
    g = np.random.default_rng(seed)
    w = W.periodic(sq=2048 + 64 * int(g.integers(0, 5)), causal=bool(seed % 2),
                   causal_offset=int(g.integers(-200, 300)), seed=seed)
    p = decode(ref.plan(w, force=[128, 64, seed % 3, 0, 0]))
    assert list(p.qil) == [interleave_choice(w, h) for h in range(4)]
    assert max(p.qil) > 1
    check_worklist(p)
    check_elements(w, p)


# ---- key-block interleave ----

def key_interleave_choice(w, h, qil, tq=128, tk=64):
    """The key interleave the plan specification gives head h, from its
    definition: for 128 x 64 tiles merging two 32-key blocks, query blocks
    of 32 or 64 rows, bf16, one query head per kv head, no union, paging or
    causal bound, the s in
    {1, 2, 4, 8} with 2 s <= nk whose query tiles (interleave qil) list the
    fewest key tiles (summed over mask batches), smallest on ties; else 1."""
    bq, bk = w.bq[h], w.bk[h]
    if (w.gqa_union or w.paged or w.causal or w.dtype != "bf16" or w.hq != w.hkv or bk != 32
            or bq >= tq or bq < 32):
        return 1
    mq, nq = tq // bq, -(-w.sq // bq)
    mk, nk = tk // bk, -(-w.skv // bk)
    nt, nkt = -(-nq // mq), -(-nk // mk)
    qbs = np.array([[qblock(t, iq, qil, mq, nq) for iq in range(mq)] for t in range(nt)])
    masks = []
    for bm in range(w.mask_batches):
        m = np.zeros((nq + 1, nk + 1), bool)  # row nq and column nk: no block
        m[:nq, :nk] = w.head_mask(bm, h).astype(bool)
        masks.append(m[np.minimum(qbs, nq)].any(1))  # [tile][key block]

    def cost(s):
        kbs = np.array([[qblock(kt, ik, s, mk, nk) for ik in range(mk)] for kt in range(nkt)])
        return sum(int(sel[:, np.minimum(kbs, nk)].any(2).sum()) for sel in masks)

    best, bc = 1, cost(1)
    for s in (2, 4, 8):
        if s * mk > nk:
            break
        c = cost(s)
        if c < bc:
            best, bc = s, c
    return best


def test_key_interleave_dilated_pattern(ref):
    """A dilated pattern of 32-blocks (key block = query block mod 8): query
    tiles gather four blocks of one residue and key tiles two key blocks of
    one residue, so every listed tile is live in all eight sub-blocks, a
    quarter of the entries of contiguous merging on both sides."""
    w = W.affine(bs=32, batch=1, heads=3, s=4096, window=256, d=64)
    p = decode(ref.plan(w, force=[128, 64, 0, 0, 0]))
    assert list(p.qil) == [interleave_choice(w, h) for h in range(3)]
    assert list(p.kil) == [key_interleave_choice(w, h, int(p.qil[h])) for h in range(3)]
    assert (int(p.qil[1]), int(p.kil[1])) == (8, 8)
    check_worklist(p)
    check_elements(w, p)
    nqt = p.h["nqt"]
    for r in range(nqt, 2 * nqt):  # the dilated head: 128 key blocks, 16 per residue
        e0, e1 = p.rows[r]
        assert e1 - e0 == 128 // 8 // 2
        assert (p.live[e0:e1] == 0xFF).all()


@pytest.mark.parametrize("seed", range(6))
def test_key_interleave_choice_random(ref, seed):
    """Periodic rows over 32-key blocks (ragged key length, per-batch masks,
    merged query blocks of 32 and 64 rows), causal on odd seeds: the
    planner's key interleave equals the definition's (1 under the causal
    bound), and the plan covers the mask exactly."""
    g = np.random.default_rng(100 + seed)
    w = W.periodic(sq=2048 + 64 * int(g.integers(0, 5)), skv=1024 + 32 * int(g.integers(0, 7)),
                   bk=32, causal=bool(seed % 2), causal_offset=int(g.integers(-200, 300)), seed=seed)
    p = decode(ref.plan(w, force=[128, 64, seed % 3, 0, 0]))
    assert list(p.qil) == [interleave_choice(w, h) for h in range(4)]
    assert list(p.kil) == [key_interleave_choice(w, h, int(p.qil[h])) for h in range(4)]
    assert (max(p.kil) > 1) == (not w.causal)
    check_worklist(p)
    check_elements(w, p)
