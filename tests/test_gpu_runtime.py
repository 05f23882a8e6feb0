"""GPU tests of the runtime around the kernels: repeated and concurrent
forward calls on one plan (each call takes its own set of work-queue
counters from the plan's ring of 64), plans freed right after their forward
and rebuilt on the same stream (stream-ordered plan memory), and forward
calls on a stream other than the plan's. Outputs are compared with the
oracle on every row, and across calls bit for bit (the kernels are
deterministic: which workgroup computes a row never changes its value)."""
import numpy as np
import pytest

import block_sparse_attention_08_amd as bsa
from block_sparse_attention_08_amd import workloads as W
from tests.gpu_helpers import O_MAX, O_MEAN, LSE_MAX, compare, forced_lut_text, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_all_rows(ref, w, q, k, v, o, lse, label):
    import torch
    torch.cuda.synchronize()
    rows = np.stack(np.meshgrid(np.arange(w.batch), np.arange(w.hq), np.arange(w.sq),
                                indexing="ij"), -1).reshape(-1, 3)
    o_ref, lse_ref = ref.forward(w, q.cpu(), k.cpu(), v.cpu(), mode=1, rows=rows)
    o_g = o.float().cpu().numpy().astype(np.float64).reshape(-1, w.d)
    l_g = lse.cpu().numpy().astype(np.float64).reshape(-1)
    res = compare(w, o_g, l_g, o_ref, lse_ref, rows)
    say(f"[result] {label}: max|dO|={res['max_o']:.3e} max|dLSE|={res['max_lse']:.3e}")
    assert res["empty_ok"]
    assert res["max_o"] <= O_MAX and res["mean_o"] <= O_MEAN and res["max_lse"] <= LSE_MAX, res


CASES = {
    # row order (contiguous per-XCD queues) and longest-first (strided queues)
    "local": (lambda: W.random_problem(batch=2, hq=3, sq=700, skv=650, d=128, bq=64, bk=64,
                                       density=0.4, empty_rows=0.1, seed=21),
              forced_lut_text(128, 64, "local", 0, 0)),
    "lpt_split": (lambda: W.random_problem(batch=1, hq=4, sq=900, skv=1200, d=64, bq=[32, 64, 32, 64],
                                           bk=[64, 128, 128, 64], density=0.5, causal=True,
                                           causal_offset=300, seed=22),
                  forced_lut_text(128, 64, "lpt", 3, 0)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_repeated_forward_wraps_queue_ring(ref, case):
    """70 forward calls on one plan (more than the ring's 64 counter sets):
    every call writes the same bytes, and they match the oracle."""
    import torch
    make, lut_text = CASES[case]
    w = make()
    say(f"[case] repeated forward {case}")
    q, k, v, mask, table = to_device(w)
    plan = bsa.plan(w.problem_dict(), mask, table, bsa.Lut.parse(lut_text))
    o0, l0 = plan.forward(q, k, v)
    _check_all_rows(ref, w, q, k, v, o0, l0, f"{case}/first")
    o, lse = torch.empty_like(o0), torch.empty_like(l0)
    for i in range(70):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        plan.forward(q, k, v, o, lse)
        if i % 10 == 9 or i == 69:
            torch.cuda.synchronize()
            assert torch.equal(o, o0) and torch.equal(lse, l0), f"call {i + 1} differs"
    plan.free()


def test_concurrent_forwards_two_streams(ref):
    """One plan, forward calls on two streams at once into separate outputs:
    both match the single-stream result bit for bit."""
    import torch
    w = W.video_dit(heads=3, grid=(16, 6, 12), seed=3)
    say("[case] concurrent forwards on two streams")
    q, k, v, mask, table = to_device(w)
    plan = bsa.plan(w.problem_dict(), mask, table)
    o_ref_t, l_ref_t = plan.forward(q, k, v)
    torch.cuda.synchronize()
    _check_all_rows(ref, w, q, k, v, o_ref_t, l_ref_t, "two-streams/reference")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        for s in (s1, s2):
            o, lse = torch.empty_like(o_ref_t), torch.empty_like(l_ref_t)
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                plan.forward(q, k, v, o, lse, stream=s)
            outs.append((o, lse))
    torch.cuda.synchronize()
    for i, (o, lse) in enumerate(outs):
        assert torch.equal(o, o_ref_t) and torch.equal(lse, l_ref_t), f"call {i} differs"
    plan.free()


def test_plans_freed_and_rebuilt_on_one_stream(ref):
    """Plan, forward, free, repeated with different masks on one stream without
    synchronising in between: each new plan may reuse the memory of the last
    (stream-ordered), and every result still matches the oracle."""
    import torch
    ws = [W.random_problem(batch=1, hq=2, sq=500, skv=520, d=128, bq=64, bk=64, density=dens,
                           empty_rows=0.05, seed=30 + i) for i, dens in enumerate((0.2, 0.9, 0.5, 0.05))]
    say("[case] plans freed and rebuilt")
    results = []
    for i, w in enumerate(ws):
        q, k, v, mask, table = to_device(w)
        plan = bsa.plan(w.problem_dict(), mask, table, bsa.Lut.parse(forced_lut_text(128, 64, "lpt", 0, 0)))
        o, lse = plan.forward(q, k, v)
        plan.free()  # no synchronisation: the next plan is ordered after this forward
        results.append((w, q, k, v, o, lse))
    torch.cuda.synchronize()
    for i, (w, q, k, v, o, lse) in enumerate(results):
        _check_all_rows(ref, w, q, k, v, o, lse, f"rebuilt/{i}")


def test_forward_on_another_stream(ref):
    """Plan built on one stream, forward on another that waits for it."""
    import torch
    w = W.random_problem(batch=2, hq=2, hkv=1, sq=300, skv=900, d=128, bq=128, bk=128,
                         density=0.1, gqa_union=True, causal=True, causal_offset=600, paged=True,
                         page_size=64, seed=40)
    say("[case] forward on another stream")
    q, k, v, mask, table = to_device(w)
    ps, fs = torch.cuda.Stream(), torch.cuda.Stream()
    ps.wait_stream(torch.cuda.current_stream())
    plan = bsa.plan(w.problem_dict(), mask, table, stream=ps)
    ready = torch.cuda.Event()
    ready.record(ps)
    fs.wait_event(ready)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.hq, w.sq), dtype=torch.float32, device="cuda")
    plan.forward(q, k, v, o, lse, stream=fs)
    fs.synchronize()
    _check_all_rows(ref, w, q, k, v, o, lse, "other-stream")
    plan.free()
