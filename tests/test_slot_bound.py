"""The bound on split-KV partial slots that sizes a forward call's scratch
(computed on the host from the mask features before the plan exists) holds
on the reference planner's plans: for every head, a row has at most
min(nkt, mq * largest logical row * sk) entries (union rows: nkt), and a
split row of n entries takes ceil(n / split) slots. Random problems over
merged and subdivided blocks, causal offsets, union and packed rows, forced
split regimes (CPU only; the library computes the same bound, and the GPU
tests check partial_slots <= partial_slot_bound on every plan)."""
import numpy as np
import pytest

from block_sparse_attention_08_amd import workloads as W
from tests.gpu_helpers import forced_lut_text
from tests.plan_image import decode


def cdiv(a, b):
    return -(-a // b)


def slot_bound(h, feat, bq, bk):
    split, tq, tk, nkt, nqt = h["split"], h["tq"], h["tk"], h["nkt"], h["nqt"]
    if split <= 0:
        return 0
    bound = 0
    G = h["hq"] // h["hkv"]
    for hd in range(h["hq"]):
        if h["union"] and h["pack"] and hd % G:
            continue
        maxlen = nkt
        if not h["union"]:
            maxrow = int(feat[:, hd, 1].max())
            mq = tq // bq[hd] if bq[hd] < tq else 1
            sk = bk[hd] // tk if bk[hd] > tk else 1
            maxlen = min(nkt, mq * maxrow * sk)
        if maxlen > split:
            bound += h["batch"] * nqt * cdiv(maxlen, split)
    return bound


CASES = []
g = np.random.default_rng(5)
for i in range(40):
    hq = int(g.choice([2, 4]))
    uni = bool(i % 3 == 0)
    hkv = hq // 2 if uni else hq
    bs = [int(x) for x in g.choice([16, 32, 64, 128, 256], hq)]
    bk = [bs[0]] * hq if uni else [int(x) for x in g.choice([16, 32, 64, 128, 256], hq)]
    CASES.append(dict(batch=int(g.integers(1, 3)), hq=hq, hkv=hkv, sq=int(g.integers(1, 700)),
                      skv=int(g.integers(1, 1500)), d=64, bq=bs, bk=bk,
                      density=float(g.uniform(0.05, 0.9)), causal=bool(i % 2),
                      causal_offset=int(g.integers(-100, 800)), gqa_union=uni,
                      mask_broadcast=bool(i % 5 == 1), seed=100 + i))


@pytest.mark.parametrize("i", range(len(CASES)))
def test_partial_slot_bound(ref, i):
    w = W.random_problem(**CASES[i])
    for tq, tk, split, pack in ((128, 64, 1, 0), (128, 64, 3, 1), (256, 64, 2, 2), (128, 128, 5, 0),
                                (128, 64, 16, 1)):
        try:
            img = ref.plan(w, lut_text=forced_lut_text(tq, tk, "local", split, pack))
        except ValueError:
            continue  # geometry not supported by this regime
        p = decode(img)
        assert p.h["nslots"] <= slot_bound(p.h, p.feat, p.bq, p.bk), (tq, tk, split, pack, p.h["nslots"])
