"""GPU parity of the FP8 K/V forward (bsa_forward_kv8) against the oracle's
ref_forward_kv8: K and V as OCP E4M3 bytes with per-kv-head scales, Q and O
bf16, every row compared within the forward's tolerances. The e4m3 values are
exact in bf16, so the arithmetic and its error budget are the bf16 path's.
Random bytes cover every non-NaN code (subnormals, the largest finite value,
both signs), so the conversion is checked against the format's definition."""
import numpy as np
import pytest

import block_sparse_attention_08_amd as bsa
from block_sparse_attention_08_amd import workloads as W
from tests.gpu_helpers import O_MAX, O_MEAN, LSE_MAX, compare, forced_lut_text, sample_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(ref, w, lut_text=None, rows=None, random_codes=False, device_gen=False, label=""):
    import torch
    say(f"[case] kv8 {label}: B={w.batch} Hq={w.hq} Hkv={w.hkv} Sq={w.sq} Skv={w.skv} D={w.d} "
        f"union={int(w.gqa_union)} paged={int(w.paged)} codes={'all' if random_codes else 'quantized'}")
    q, k, v, mask, table = to_device(w, device_gen)
    if random_codes:
        g = np.random.default_rng(11)
        k8 = torch.from_numpy(g.integers(0, 256, tuple(k.shape), dtype=np.uint8))
        v8 = torch.from_numpy(g.integers(0, 256, tuple(v.shape), dtype=np.uint8))
        for x in (k8, v8):
            x[(x & 0x7F) == 0x7F] ^= 0x01  # NaN codes become the largest finite value
        k8, v8 = k8.cuda(), v8.cuda()
        ks = torch.full((w.hkv,), 1.0 / 448.0, dtype=torch.float32, device="cuda")
        # magnitudes of order one, as the forward tolerances assume
        vs = torch.linspace(0.5, 2.0, w.hkv, dtype=torch.float32, device="cuda") / 448.0
    else:
        k8, v8, ks, vs = w.make_kv8(k, v)
    lut = bsa.Lut.parse(lut_text) if lut_text else None
    plan = bsa.plan(w.problem_dict(), mask, table, lut)
    o, lse = plan.forward_kv8(q, k8, v8, ks, vs)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.stack(np.meshgrid(np.arange(w.batch), np.arange(w.hq), np.arange(w.sq), indexing="ij"),
                        -1).reshape(-1, 3)
    rows = np.asarray(rows, np.int64)
    o_ref, l_ref = ref.forward_kv8(w, q.cpu(), k8.cpu(), v8.cpu(), ks.cpu().numpy(), vs.cpu().numpy(),
                                   rows=rows)
    ri = [torch.from_numpy(rows[:, i]).cuda() for i in range(3)]
    o_g = o[ri[0], ri[1], ri[2]].float().cpu().numpy().astype(np.float64)
    l_g = lse[ri[0], ri[1], ri[2]].cpu().numpy().astype(np.float64)
    res = compare(w, o_g, l_g, o_ref, l_ref, rows)
    say(f"[result] kv8 {label}: max|dO|={res['max_o']:.3e} mean|dO|={res['mean_o']:.3e} "
        f"max|dLSE|={res['max_lse']:.3e} rows={res['rows']}")
    assert res["empty_ok"]
    assert res["max_o"] <= O_MAX and res["mean_o"] <= O_MEAN and res["max_lse"] <= LSE_MAX, res
    plan.free()


CASES = {
    "decode_q1": lambda: W.decode(batch=3, hq=8, hkv=2, q_len=1, context=4096, seed=1),
    "decode_q1_hnd": lambda: W.decode(batch=3, hq=8, hkv=2, q_len=1, context=4096, seed=5,
                                      kv_layout="hnd"),
    "decode_q5_d64": lambda: W.decode(batch=2, hq=8, hkv=2, d=64, q_len=5, context=3072, seed=2),
    "dense_ragged_d128": lambda: W.random_problem(batch=2, hq=4, hkv=2, sq=300, skv=333, d=128, bq=64,
                                                  bk=64, density=0.4, empty_rows=0.1, causal=True,
                                                  causal_offset=33, seed=601),
    "dense_mixed_d64": lambda: W.random_problem(batch=1, hq=3, sq=257, skv=400, d=64, bq=[16, 64, 128],
                                                bk=[32, 128, 64], density=0.3, seed=602),
    "union_paged": lambda: W.random_problem(batch=2, hq=8, hkv=2, sq=200, skv=900, d=128, bq=128,
                                            bk=128, density=0.08, gqa_union=True, causal=True,
                                            causal_offset=700, paged=True, page_size=64, seed=603),
    # key-interleaved 64-key tiles (32-key blocks s apart), last block partial
    "periodic_keys_d64": lambda: W.periodic(batch=1, sq=640, skv=1000, bk=32, seed=604),
    "periodic_keys_d128": lambda: W.periodic(batch=1, sq=640, skv=1000, bk=32, d=128, seed=605),
}


@pytest.mark.parametrize("case", list(CASES))
def test_kv8_default_regime(ref, case):
    _run(ref, CASES[case](), label=case)


@pytest.mark.parametrize("case", ["decode_q1", "dense_ragged_d128", "union_paged"])
def test_kv8_all_codes(ref, case):
    _run(ref, CASES[case](), random_codes=True, label=f"{case}/all-codes")


@pytest.mark.parametrize("regime", [(128, 128, "lpt", 0, 0), (128, 64, "local", 3, 1),
                                    (256, 64, "lpt", 2, 1), (128, 64, "local", 3, 2),
                                    (256, 64, "lpt", 2, 2)], ids=str)
@pytest.mark.parametrize("case", ["dense_ragged_d128", "union_paged", "dense_mixed_d64", "decode_q1"])
def test_kv8_regimes(ref, case, regime):
    _run(ref, CASES[case](), lut_text=forced_lut_text(*regime), label=f"{case}/{regime}")


def test_kv8_full_decode(ref):
    w = W.decode(q_len=1)
    _run(ref, w, rows=sample_rows(w, 192), device_gen=True, label="decode_full")


def test_kv8_full_decode_interleaved(ref):
    w = W.decode(q_len=1)
    _run(ref, w, rows=sample_rows(w, 192), device_gen=True,
         lut_text=forced_lut_text(128, 64, "local", 32, 2), label="decode_full/ilv")


def test_kv8_rejects_fp32_and_null_scales():
    import torch
    w = W.random_problem(batch=1, hq=2, sq=64, skv=128, d=64, dtype="f32", bq=64, bk=64, seed=604)
    q, k, v, mask, _ = to_device(w)
    plan = bsa.plan(w.problem_dict(), mask, None)
    k8 = torch.zeros(k.shape, dtype=torch.uint8, device="cuda")
    s = torch.ones(w.hkv, dtype=torch.float32, device="cuda")
    with pytest.raises(bsa.BsaError):
        plan.forward_kv8(q, k8, k8, s, s)
    plan.free()
