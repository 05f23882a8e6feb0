"""bsa_forward_noalloc (static device scratch, no allocation) against
bsa_forward on the same plans, through the C ABI: two calls in a row, the
second with a smaller input, each equal to bsa_forward bit for bit and within
the oracle's tolerances; split-KV plans (partials in the static scratch) and
plans without splits; a plan whose scratch exceeds the static array is
rejected before anything is queued."""
import numpy as np
import pytest

import block_sparse_attention_08_amd as bsa
from block_sparse_attention_08_amd import workloads as W
from tests.gpu_helpers import all_rows, check_written, compare_rows, forced_lut_text, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(ref, w, lut_text, label):
    import torch
    q, k, v, mask, table = to_device(w)
    lut = bsa.Lut.parse(lut_text) if lut_text else bsa.Lut.load(bsa.DEFAULT_LUT)
    plan = bsa.plan(w.problem_dict(), mask, table, lut)
    st = plan.stats()
    o1, l1 = plan.forward(q, k, v)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((w.batch, w.hq, w.sq), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward_noalloc(q, k, v, o2, l2)
    torch.cuda.synchronize()
    check_written(o2, l2, label)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{label}: noalloc differs from bsa_forward"
    compare_rows(ref, w, (q.cpu(), k.cpu(), v.cpu()), o2, l2, all_rows(w), label)
    plan.free()
    return st


CASES = [
    ("split3", forced_lut_text(128, 64, "local", 3, 0),
     lambda s: W.random_problem(batch=2, hq=3, sq=s, skv=900, d=128, bq=64, bk=64, density=0.5,
                                empty_rows=0.05, seed=90)),
    ("tq256_split2_d64", forced_lut_text(256, 64, "lpt", 2, 1),
     lambda s: W.random_problem(batch=1, hq=4, hkv=2, sq=s, skv=700, d=64, bq=32, bk=64, density=0.4,
                                causal=True, causal_offset=200, seed=91)),
    ("packaged", None,
     lambda s: W.random_problem(batch=1, hq=2, sq=s, skv=520, d=128, bq=128, bk=128, density=0.5,
                                seed=92)),
]


@pytest.mark.parametrize("case", [c[0] for c in CASES])
def test_noalloc_matches_forward_two_calls(ref, case):
    name, lut_text, make = next(c for c in CASES if c[0] == case)
    say(f"[case] noalloc {name}")
    st1 = _both(ref, make(640), lut_text, f"noalloc/{name}/first")
    st2 = _both(ref, make(200), lut_text, f"noalloc/{name}/second (smaller)")
    if lut_text:
        assert st1["partial_slots"] > 0 and st2["partial_slots"] > 0


def test_noalloc_rejects_oversized_scratch():
    import torch
    # split at one key tile over long rows: far more partial slots than 64 MiB holds
    w = W.random_problem(batch=1, hq=8, sq=4096, skv=4096, d=128, bq=128, bk=128, density=0.9, seed=93)
    q, k, v, mask, table = to_device(w)
    plan = bsa.plan(w.problem_dict(), mask, table, bsa.Lut.parse(forced_lut_text(128, 64, "local", 1, 0)))
    st = plan.stats()
    need = 4 * st["tile_q"] * (w.d + 1) * st["partial_slot_bound"]
    assert need > 64 << 20, need
    o = torch.zeros_like(q)
    lse = torch.zeros((w.batch, w.hq, w.sq), dtype=torch.float32, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        plan.forward_noalloc(q, k, v, o, lse)
    assert e.value.status == 2 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (o == 0).all() and (lse == 0).all()  # nothing was queued
    plan.free()
