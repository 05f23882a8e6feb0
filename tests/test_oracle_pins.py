"""Pins of the CPU oracle's forward pass against what mathematics and library
routines fix independently of it (no GPU).

Each test would fail on a plausible mistake in the oracle: a dropped or extra
key (block index, causal bound, union), a wrong head/group or page mapping, a
missing normalisation, a transposed operand, a wrong scale or log base.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_08_amd import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def f64(x):
    return x.to(torch.float64) if isinstance(x, torch.Tensor) else torch.from_numpy(x).double()


def element_mask(w, b, h):
    """Element-level allowed[i][j] from the definition (block mask, union, causal)."""
    bm = 0 if w.mask_broadcast else b
    if w.gqa_union:
        gs = w.hq // w.hkv
        g = h // gs
        u = np.zeros(w.nkb(h), bool)
        for h2 in range(g * gs, (g + 1) * gs):
            u |= w.head_mask(bm, h2).astype(bool).any(0)
        blk = np.broadcast_to(u, (w.nqb(h), w.nkb(h)))
    else:
        blk = w.head_mask(bm, h).astype(bool)
    i = np.arange(w.sq)
    j = np.arange(w.skv)
    m = blk[i[:, None] // w.bq[h], j[None, :] // w.bk[h]]
    if w.causal:
        m &= j[None, :] <= i[:, None] + w.causal_offset
    return m


def kv_rows(w, kv, b, g):
    """[skv][d] float64 K or V rows of (b, kv head g), through the page table."""
    x = f64(kv)
    if w.paged:
        j = np.arange(w.skv)
        pages = w.page_table[b][j // w.page_size]
        return x[pages, j % w.page_size, g]
    return x[b, g]


def sdpa_torch(w, q, k, v, b, h):
    """torch's float64 CPU scaled_dot_product_attention with an explicit mask."""
    g = h // (w.hq // w.hkv)
    m = torch.from_numpy(element_mask(w, b, h))
    o = torch.nn.functional.scaled_dot_product_attention(
        f64(q)[b, h][None], kv_rows(w, k, b, g)[None], kv_rows(w, v, b, g)[None],
        attn_mask=m[None])
    return o[0].numpy(), m.numpy()


def run(ref, w, q, k, v, mode=1):
    o, lse = ref.forward(w, q, k, v, mode=mode)
    return o.reshape(w.batch, w.hq, w.sq, w.d), lse.reshape(w.batch, w.hq, w.sq)


def test_p1_dense_limit_equals_textbook_and_torch(ref):
    """All-ones mask: textbook softmax(QK^T/sqrt(d))V and torch SDPA (fp64)."""
    w = W.random_problem(batch=2, hq=4, hkv=2, sq=130, skv=97, d=64, dtype="f32", bq=32,
                         bk=16, density=1.0, seed=1)
    q, k, v = w.make_qkv()
    o, lse = run(ref, w, q, k, v)
    for b in range(2):
        for h in range(4):
            g = h // 2
            Q, K, V = f64(q)[b, h].numpy(), f64(k)[b, g].numpy(), f64(v)[b, g].numpy()
            s = Q @ K.T / math.sqrt(64)
            mx = s.max(1, keepdims=True)
            p = np.exp(s - mx)
            o_tb = (p / p.sum(1, keepdims=True)) @ V
            lse_tb = np.log(p.sum(1)) + mx[:, 0]
            np.testing.assert_allclose(o[b, h], o_tb, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], lse_tb, rtol=0, atol=1e-12)
            o_t, _ = sdpa_torch(w, q, k, v, b, h)
            np.testing.assert_allclose(o[b, h], o_t, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["plain", "causal", "union", "paged"])
def test_masked_rows_match_torch_sdpa(ref, kind):
    """Arbitrary masks: torch SDPA with the element mask built from the definition."""
    kw = dict(batch=2, hq=4, hkv=2, sq=200, skv=230, d=64, dtype="f32", bq=32, bk=64,
              density=0.35, empty_rows=0.1, seed=7)
    if kind == "causal":
        kw.update(causal=True, causal_offset=25)
    if kind == "union":
        kw.update(gqa_union=True, causal=True, causal_offset=30, bq=[32, 64, 16, 32])
    if kind == "paged":
        kw.update(paged=True, page_size=16, hkv=4)
    w = W.random_problem(**kw)
    q, k, v = w.make_qkv()
    o, lse = run(ref, w, q, k, v)
    for b in range(w.batch):
        for h in range(w.hq):
            o_t, m = sdpa_torch(w, q, k, v, b, h)
            rows = m.any(1)
            np.testing.assert_allclose(o[b, h][rows], o_t[rows], rtol=0, atol=1e-12)
            assert (o[b, h][~rows] == 0).all() and np.isneginf(lse[b, h][~rows]).all()


def test_p2_probability_rows_sum_to_one(ref):
    """V = 1 everywhere: every non-empty output row is exactly the softmax row sum."""
    w = W.random_problem(batch=1, hq=2, sq=150, skv=170, d=64, dtype="f32", bq=16, bk=32,
                         density=0.4, empty_rows=0.2, causal=True, causal_offset=5, seed=3)
    q, k, _ = w.make_qkv()
    v = torch.ones_like(k)
    o, lse = run(ref, w, q, k, v)
    for h in range(2):
        rows = element_mask(w, 0, h).any(1)
        np.testing.assert_allclose(o[0, h][rows], 1.0, rtol=0, atol=1e-12)
        assert (o[0, h][~rows] == 0).all()


def test_p3_block_diagonal_equals_independent_blocks(ref):
    """Block-diagonal mask == attention run independently inside each block (torch SDPA)."""
    bs, nb, d = 32, 5, 64
    w = W.random_problem(batch=1, hq=2, sq=bs * nb, skv=bs * nb, d=d, dtype="f32", bq=bs,
                         bk=bs, density=0.0, seed=4)
    w.mask[:] = 0
    for h in range(2):
        np.fill_diagonal(w.head_mask(0, h), 1)
    q, k, v = w.make_qkv()
    o, lse = run(ref, w, q, k, v)
    for h in range(2):
        for blk in range(nb):
            sl = slice(blk * bs, (blk + 1) * bs)
            ot = torch.nn.functional.scaled_dot_product_attention(
                f64(q)[0, h, sl][None], f64(k)[0, h, sl][None], f64(v)[0, h, sl][None])[0]
            np.testing.assert_allclose(o[0, h, sl], ot.numpy(), rtol=0, atol=1e-12)


def test_p4_brute_force_long_double(ref):
    """Tiny cases: literal exp-sum formula in long double, no max subtraction."""
    for seed in range(6):
        w = W.random_problem(batch=1, hq=2, hkv=1, sq=29, skv=31, d=16, dtype="f32", bq=16,
                             bk=16, density=0.6, empty_rows=0.25, causal=seed % 2 == 1,
                             causal_offset=3, seed=100 + seed)
        q, k, v = w.make_qkv()
        o, lse = run(ref, w, q, k, v)
        Q = q.numpy().astype(np.longdouble)
        K = k.numpy().astype(np.longdouble)
        V = v.numpy().astype(np.longdouble)
        scale = np.longdouble(1) / np.sqrt(np.longdouble(16))
        for h in range(2):
            m = element_mask(w, 0, h)
            for i in range(w.sq):
                js = np.nonzero(m[i])[0]
                if len(js) == 0:
                    assert (o[0, h, i] == 0).all() and np.isneginf(lse[0, h, i])
                    continue
                e = np.array([np.exp((Q[0, h, i] * K[0, 0, j]).sum() * scale) for j in js])
                ob = (e[:, None] * V[0, 0, js]).sum(0) / e.sum()
                assert np.abs(o[0, h, i] - ob.astype(np.float64)).max() <= 1e-12
                assert abs(lse[0, h, i] - float(np.log(e.sum()))) <= 1e-12


def test_p5_closed_forms(ref):
    w = W.random_problem(batch=1, hq=2, sq=96, skv=113, d=32, dtype="f32", bq=16, bk=16,
                         density=0.3, empty_rows=0.2, causal=True, causal_offset=10, seed=5)
    q, k, v = w.make_qkv()
    # Q = 0: every allowed logit is 0, so LSE = ln(n) and O = mean of allowed V.
    o, lse = run(ref, w, torch.zeros_like(q), k, v)
    for h in range(2):
        m = element_mask(w, 0, h)
        n = m.sum(1)
        nz = n > 0
        np.testing.assert_allclose(lse[0, h][nz], np.log(n[nz]), rtol=0, atol=1e-13)
        mean = (m[nz].astype(np.float64) @ f64(v)[0, h].numpy()) / n[nz][:, None]
        np.testing.assert_allclose(o[0, h][nz], mean, rtol=0, atol=1e-13)
        assert np.isneginf(lse[0, h][~nz]).all() and (o[0, h][~nz] == 0).all()
    # V = c: O = c on every non-empty row.
    o, _ = run(ref, w, q, k, torch.full_like(v, -2.5))
    for h in range(2):
        nz = element_mask(w, 0, h).any(1)
        assert np.abs(o[0, h][nz] + 2.5).max() <= 1e-13
    # A single allowed key j: O = v_j and LSE = s_ij.
    w1 = W.random_problem(batch=1, hq=1, sq=16, skv=33, d=32, dtype="f32", bq=16, bk=16,
                          density=0.0, seed=6)
    w1.mask[:] = 0
    w1.head_mask(0, 0)[0, 2] = 1          # last block holds the single key 32
    q, k, v = w1.make_qkv()
    o, lse = run(ref, w1, q, k, v)
    s = (f64(q)[0, 0] @ f64(k)[0, 0, 32]).numpy() / math.sqrt(32)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(f64(v)[0, 0, 32].numpy(), (16, 32)),
                               rtol=0, atol=0)
    np.testing.assert_allclose(lse[0, 0], s, rtol=0, atol=1e-13)


def test_p6_paged_and_gqa_invariances(ref):
    """Shuffled page table == identity table (same pool contents), bitwise;
    GQA == MHA with each kv head repeated over its group, bitwise."""
    w = W.random_problem(batch=2, hq=4, hkv=2, sq=70, skv=150, d=64, dtype="bf16", bq=32,
                         bk=32, density=0.5, paged=True, page_size=16, causal=True,
                         causal_offset=80, seed=8)
    q, kp, vp = w.make_qkv()
    o1, l1 = run(ref, w, q, kp, vp)
    # Identity layout: rebuild the pool so page p of batch b sits at index b*pps+p.
    pps = w.pages_per_seq
    idx = torch.from_numpy(w.page_table.reshape(-1).astype(np.int64))
    w2 = W.Workload(**{**w.__dict__})
    w2.page_table = np.arange(w.batch * pps, dtype=np.int32).reshape(w.batch, pps)
    w2.num_pages = w.batch * pps
    o2, l2 = run(ref, w2, q, kp[idx], vp[idx])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # GQA vs MHA: dense K/V with repeated heads.
    wg = W.random_problem(batch=1, hq=4, hkv=2, sq=90, skv=90, d=64, bq=32, bk=32,
                          density=0.5, seed=9)
    q, k, v = wg.make_qkv()
    og, lg = run(ref, wg, q, k, v)
    wm = W.Workload(**{**wg.__dict__})
    wm.hkv = 4
    om, lm = run(ref, wm, q, k.repeat_interleave(2, 1), v.repeat_interleave(2, 1))
    assert np.array_equal(og, om) and np.array_equal(lg, lm)


@pytest.mark.parametrize("kind", ["plain", "causal_union_paged", "tiny"])
def test_p7_dense_mode_equals_block_skipping(ref, kind):
    if kind == "tiny":
        w = W.tiny()
    elif kind == "plain":
        w = W.random_problem(batch=2, hq=2, sq=100, skv=140, d=64, bq=32, bk=16,
                             density=0.3, empty_rows=0.2, mask_broadcast=True, seed=10)
    else:
        w = W.random_problem(batch=1, hq=4, hkv=2, sq=64, skv=200, d=64, bq=16, bk=32,
                             density=0.1, gqa_union=True, causal=True, causal_offset=136,
                             paged=True, page_size=32, seed=11)
    q, k, v = w.make_qkv()
    o0, l0 = run(ref, w, q, k, v, mode=0)
    o1, l1 = run(ref, w, q, k, v, mode=1)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_union_equals_expanded_mask(ref):
    """Union mode == ordinary mode on a mask whose every row is the group's OR."""
    w = W.random_problem(batch=2, hq=4, hkv=1, sq=96, skv=160, d=64, bq=[32, 16, 32, 64],
                         bk=32, density=0.08, gqa_union=True, causal=True, causal_offset=64,
                         seed=12)
    q, k, v = w.make_qkv()
    ou, lu = run(ref, w, q, k, v)
    blocks = []
    for b in range(2):
        u = np.zeros(w.nkb(0), bool)
        for h in range(4):
            u |= w.head_mask(b, h).astype(bool).any(0)
        for h in range(4):
            blocks.append(np.broadcast_to(u, (w.nqb(h), w.nkb(h))).astype(np.uint8))
    we = W.Workload(**{**w.__dict__})
    we.gqa_union = False
    we.mask = np.concatenate([x.reshape(-1) for x in blocks])
    oe, le = run(ref, we, q, k, v)
    assert np.array_equal(ou, oe) and np.array_equal(lu, le)


def test_row_sampling_matches_full_run(ref):
    w = W.random_problem(batch=2, hq=2, sq=60, skv=80, d=64, bq=16, bk=16, density=0.5, seed=13)
    q, k, v = w.make_qkv()
    o, lse = run(ref, w, q, k, v)
    rows = np.array([[1, 0, 5], [0, 1, 59], [1, 1, 0]])
    os_, ls = ref.forward(w, q, k, v, rows=rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(os_[n], o[b, h, i]) and ls[n] == lse[b, h, i]


def test_features_count_blocks(ref):
    w = W.random_problem(batch=2, hq=3, sq=100, skv=70, d=64, bq=[16, 32, 64], bk=[32, 16, 64],
                         density=0.4, empty_rows=0.3, causal=True, causal_offset=-20, seed=14)
    f = ref.features(w)
    for b in range(2):
        for h in range(3):
            m = w.head_mask(b, h).astype(bool)
            rowc = m.sum(1)
            qlast = np.minimum(w.sq, (np.arange(w.nqb(h)) + 1) * w.bq[h]) - 1
            feas = np.arange(w.nkb(h))[None, :] * w.bk[h] <= qlast[:, None] + w.causal_offset
            assert list(f[b, h]) == [m.sum(), rowc.max(), (rowc == 0).sum(), (m & feas).sum()]


def test_golden_two_key_example(ref):
    """Hand-derived fixture (tests/golden/two_keys.txt)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "two_keys.txt")
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            key, rest = line.split("=")
            vals[key.strip()] = [float(x) for x in rest.split()]
    d = 16
    w = W.random_problem(batch=1, hq=1, sq=16, skv=32, d=d, dtype="f32", bq=16, bk=16,
                         density=1.0, seed=0)
    w.head_mask(0, 0)[0, :] = 1
    q = torch.zeros(1, 1, 16, d)
    k = torch.zeros(1, 1, 32, d)
    v = torch.zeros(1, 1, 32, d)
    q[..., 0] = vals["q0"][0]
    k[0, 0, :16, 0] = vals["k_first"][0]
    k[0, 0, 16:, 0] = vals["k_second"][0]
    v[0, 0, :16, 0] = vals["v_first"][0]
    v[0, 0, 16:, 0] = vals["v_second"][0]
    o, lse = run(ref, w, q, k, v)
    np.testing.assert_allclose(o[0, 0, :, 0], vals["o0"][0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], vals["lse"][0], rtol=0, atol=1e-14)
