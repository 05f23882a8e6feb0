"""GPU parity of plans built from affine runs (bsa_plan_acsr).

The plan that bsa_plan_acsr builds from runs must be, byte for byte, the
reference planner's plan of the mask the oracle expands the runs to (and the
GPU mask planner's plan of that mask); the forward over it must equal the
oracle within the forward tolerances, and equal the forward over the mask
plan bit for bit (same plan, same kernels); the backward over it must equal
the backward over the mask plan bit for bit. Cases: random runs (rational
and negative slopes, strides, overlaps, four runs), ragged sizes, mixed
block sizes, causal offsets of both signs, every tile regime, and the full
affine workloads (bs 64 and 32).
"""
import numpy as np
import pytest

import block_sparse_attention_08_amd as bsa
from block_sparse_attention_08_amd import workloads as W
from tests.gpu_helpers import forced_lut_text, plan_diff, run_case, sample_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _expanded(ref, w):
    w.mask = ref.acsr_mask(w)
    return w


def _check(ref, w, lut_text=None, rows=None, label=""):
    import torch
    say(f"[case] acsr {label}: Hq={w.hq} Sq={w.sq} Skv={w.skv} D={w.d} bq={w.bq} bk={w.bk} "
        f"causal={int(w.causal)} off={w.causal_offset} runs={w.acsr}")
    text = lut_text if lut_text else open(bsa.DEFAULT_LUT).read()
    lut = bsa.Lut.parse(text)
    pa = bsa.plan_acsr(w.problem_dict(), w.acsr, lut)
    img = pa.export()
    ref_img = ref.plan(w, lut_text=text)
    assert img == ref_img, "ACSR plan differs from the reference planner: " + plan_diff(img, ref_img)
    q, k, v, mask, _ = to_device(w)
    pm = bsa.plan(w.problem_dict(), mask, None, lut)
    assert pm.export() == img
    oa, la = pa.forward(q, k, v)
    om, lm = pm.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(oa, om) and torch.equal(la, lm)
    say(f"[result] acsr {label}: plan {len(img)} bytes equal; forward equal to the mask plan's")
    pa.free()
    pm.free()
    # and the forward against the oracle (the shared helper plans from the mask)
    run_case(ref, w, lut_text=lut_text, rows=rows, label=f"acsr {label} vs oracle")


RANDOM = [
    dict(hq=3, sq=700, skv=900, bq=64, bk=64, seed=1),
    dict(hq=3, sq=333, skv=517, bq=[16, 32, 64], bk=[64, 16, 32], max_runs=4, seed=2),
    dict(hq=2, sq=1000, skv=800, bq=128, bk=32, causal=True, causal_offset=-100, seed=3),
    dict(hq=4, hkv=2, sq=600, skv=1300, bq=32, bk=128, causal=True, causal_offset=700, seed=4),
    dict(hq=2, sq=257, skv=255, d=128, bq=256, bk=64, max_runs=4, seed=5),
]


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_random_runs(ref, i):
    w = _expanded(ref, W.random_acsr(**RANDOM[i]))
    _check(ref, w, label=f"random {i}")


@pytest.mark.parametrize("tq,tk,sched,split,pack", [(128, 64, "local", 0, 0), (128, 128, "lpt", 0, 0),
                                                   (256, 64, "local", 4, 0), (256, 128, "lpt", 0, 1),
                                                   (128, 64, "local", 3, 1)])
def test_regimes(ref, tq, tk, sched, split, pack):
    w = _expanded(ref, W.random_acsr(hq=4, hkv=2, sq=900, skv=1000, bq=[32, 64, 16, 128],
                                     bk=[64, 32, 128, 16], causal=True, causal_offset=50, seed=11))
    _check(ref, w, lut_text=forced_lut_text(tq, tk, sched, split, pack),
           label=f"{tq}x{tk} {sched} split={split} pack={pack}")


@pytest.mark.parametrize("bs", [64, 32])
def test_affine_workload(ref, bs):
    """The full affine workloads (B = 2, H = 16, S = 16384, D = 64): plan bytes
    against the reference planner, forward on sampled rows."""
    w = W.affine(bs=bs)
    _check(ref, w, rows=sample_rows(w, 192, seed=bs), label=f"affine bs{bs}")


def test_backward_equals_mask_plan(ref):
    import torch
    w = _expanded(ref, W.random_acsr(hq=2, sq=500, skv=700, bq=64, bk=32, causal=True,
                                     causal_offset=100, seed=21))
    say("[case] acsr backward")
    q, k, v, mask, _ = to_device(w)
    dout = w.make_dout().cuda()
    pa = bsa.plan_acsr(w.problem_dict(), w.acsr)
    pm = bsa.plan(w.problem_dict(), mask)
    o, lse = pa.forward(q, k, v)
    ga = pa.backward(q, k, v, o, lse, dout)
    gm = pm.backward(q, k, v, o, lse, dout)
    torch.cuda.synchronize()
    for a, b in zip(ga, gm):
        assert torch.equal(a, b)
    say("[result] acsr backward equal to the mask plan's")
    pa.free()
    pm.free()


def test_rejects_union_and_paged():
    w = W.random_acsr(hq=2, sq=100, skv=100, seed=31)
    p = w.problem_dict()
    p["gqa_union"] = 1
    with pytest.raises(bsa.BsaError):
        bsa.plan_acsr(p, w.acsr)
    p = w.problem_dict()
    p["mask_batch_broadcast"] = 0
    with pytest.raises(bsa.BsaError):
        bsa.plan_acsr(p, w.acsr)
