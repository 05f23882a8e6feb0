"""GPU parity: libbsa (through its C ABI) against the CPU oracle.

Small cases compare every output row and span several tiles with ragged
tails; full-size workloads compare every row (long video: a stratified part,
see below), and every case checks that the forward wrote the whole output.
Every case also compares the GPU plan image with the reference planner's,
byte for byte.
"""
import numpy as np
import pytest

from block_sparse_attention_08_amd import workloads as W
from tests.gpu_helpers import all_rows, compare_rows, forced_lut_text, run_case, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---- small cases: all rows ----

SMALL = {
    "tiny_fp32": lambda: W.tiny(),
    "tiny_fp32_d128": lambda: W.random_problem(batch=1, hq=2, sq=256, skv=256, d=128, dtype="f32",
                                               bq=64, bk=64, density=0.5, seed=1),
    "ragged_bf16_d64": lambda: W.random_problem(batch=2, hq=3, sq=301, skv=333, d=64, bq=64, bk=32,
                                                density=0.4, empty_rows=0.15, seed=2),
    "ragged_bf16_d128": lambda: W.random_problem(batch=1, hq=2, sq=397, skv=450, d=128, bq=128,
                                                 bk=128, density=0.35, empty_rows=0.1, seed=3),
    "merge_small_blocks": lambda: W.random_problem(batch=1, hq=3, sq=300, skv=290, d=64,
                                                   bq=[16, 32, 64], bk=[16, 32, 64], density=0.3,
                                                   seed=4),
    "subdivide_big_blocks": lambda: W.random_problem(batch=1, hq=2, sq=700, skv=650, d=128,
                                                     bq=[256, 512], bk=[512, 256], density=0.5,
                                                     seed=5),
    "causal_offset": lambda: W.random_problem(batch=2, hq=2, sq=260, skv=400, d=64, bq=32, bk=64,
                                              density=0.6, causal=True, causal_offset=140, seed=6),
    "broadcast_gqa": lambda: W.random_problem(batch=3, hq=4, hkv=2, sq=200, skv=200, d=128, bq=64,
                                              bk=64, density=0.4, mask_broadcast=True, seed=7),
    "union_paged_causal": lambda: W.random_problem(batch=2, hq=8, hkv=2, sq=200, skv=900, d=128,
                                                   bq=128, bk=128, density=0.08, gqa_union=True,
                                                   causal=True, causal_offset=700, paged=True,
                                                   page_size=64, seed=8),
    "union_g2_ragged": lambda: W.random_problem(batch=1, hq=4, hkv=2, sq=150, skv=333, d=64, bq=64,
                                                bk=32, density=0.1, gqa_union=True, causal=True,
                                                causal_offset=183, seed=9),
    "paged_plain": lambda: W.random_problem(batch=2, hq=2, sq=100, skv=500, d=64, bq=64, bk=64,
                                            density=0.4, paged=True, page_size=128, seed=10),
    "all_empty": lambda: W.random_problem(batch=1, hq=2, sq=130, skv=140, d=64, bq=64, bk=64,
                                          density=0.0, seed=11),
    "tiny_video": lambda: W.video_dit(heads=2, grid=(16, 6, 12), seed=1),
    "tiny_prefill": lambda: W.chunked_prefill(hq=8, hkv=2, chunk=512, context=4096, seed=1),
    "tiny_affine32": lambda: W.affine(bs=32, batch=2, heads=3, s=1024, window=128),
    "tiny_long_video": lambda: W.long_video(heads=3, grid=(4, 16, 32), seed=1),
    # merged query blocks taken interleaved (periods 2, 4, 8), causal, ragged
    "periodic_interleave": lambda: W.periodic(sq=1000, skv=700, causal=True, causal_offset=80, seed=3),
    "dilated_bs64": lambda: W.affine(bs=64, batch=1, heads=3, s=4096, window=256),
    # 64-key tiles gathering 32-key blocks s apart (key interleave), the last
    # key block partial, D = 64 and 128
    "periodic_keys": lambda: W.periodic(sq=1000, skv=1000, bk=32, seed=7),
    "periodic_keys_d128": lambda: W.periodic(batch=1, sq=777, skv=1240, bk=32, d=128, seed=8),
    "dilated_bs32": lambda: W.affine(bs=32, batch=1, heads=3, s=4096, window=256),
    "decode_q1": lambda: W.decode(batch=3, hq=8, hkv=2, q_len=1, context=4096, seed=1),
    "decode_q5": lambda: W.decode(batch=2, hq=8, hkv=2, q_len=5, context=3072, seed=2),
    "short_chunk_q16": lambda: W.decode(batch=2, hq=4, hkv=1, d=64, q_len=16, context=2048, seed=3),
    "decode_q5_hnd": lambda: W.decode(batch=2, hq=8, hkv=2, q_len=5, context=3072, seed=4,
                                      kv_layout="hnd"),
}

REGIMES = {
    "default": None,
    "tk128_lpt": forced_lut_text(128, 128, "lpt", 0, 0),
    "split3_local": forced_lut_text(128, 64, "local", 3, 1),
    "split2_lpt_tk128": forced_lut_text(128, 128, "lpt", 2, 1),
    "tq256_local": forced_lut_text(256, 64, "local", 0, 1),
    "tq256_split3_lpt": forced_lut_text(256, 64, "lpt", 3, 1),
    # heads interleaved row by row in packed tiles
    "ilv_local": forced_lut_text(128, 64, "local", 0, 2),
    "ilv_split3": forced_lut_text(128, 64, "local", 3, 2),
    "ilv_tq256_split2_lpt": forced_lut_text(256, 64, "lpt", 2, 2),
    "ilv_tk128_split2": forced_lut_text(128, 128, "lpt", 2, 2),
    # row order dealt to the XCDs in blocks
    "dealt": forced_lut_text(128, 64, "dealt", 0, 1),
    "dealt_split3_tq256": forced_lut_text(256, 64, "dealt", 3, 0),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_small_default(ref, case):
    run_case(ref, SMALL[case](), label=case)


@pytest.mark.parametrize("regime", [r for r in REGIMES if r != "default"])
@pytest.mark.parametrize("case", ["ragged_bf16_d128", "merge_small_blocks", "causal_offset",
                                  "union_paged_causal", "union_g2_ragged", "tiny_fp32",
                                  "tiny_long_video", "periodic_interleave", "periodic_keys"])
def test_small_forced_regimes(ref, case, regime):
    run_case(ref, SMALL[case](), lut_text=REGIMES[regime], label=f"{case}/{regime}")


@pytest.mark.parametrize("regime", ["split3_local", "split2_lpt_tk128", "tq256_split3_lpt",
                                    "ilv_local", "ilv_split3", "ilv_tq256_split2_lpt",
                                    "ilv_tk128_split2", "dealt_split3_tq256"])
@pytest.mark.parametrize("case", ["decode_q1", "decode_q5", "short_chunk_q16", "decode_q5_hnd"])
def test_decode_split_regimes(ref, case, regime):
    """Split-KV on packed decode rows, where most rows of a packed tile do not
    exist: partials are written and combined for existing rows only."""
    run_case(ref, SMALL[case](), lut_text=REGIMES[regime], label=f"{case}/{regime}")


@pytest.mark.parametrize("case", ["video_dit", "chunked_prefill"])
def test_full_tq256(ref, case):
    w = W.video_dit() if case == "video_dit" else W.chunked_prefill()
    run_case(ref, w, lut_text=forced_lut_text(256, 64, "local", 0, 1), rows=sample_rows(w, 192),
             device_gen=True, label=f"{case}_full/tq256")


def test_zero_lengths(ref):
    run_case(ref, W.random_problem(batch=1, hq=2, sq=64, skv=0, d=64, bq=64, bk=64, seed=12),
             label="skv0")
    run_case(ref, W.random_problem(batch=1, hq=2, sq=0, skv=64, d=64, bq=64, bk=64, seed=13),
             rows=np.zeros((0, 3), np.int64), label="sq0")


# ---- full-size workloads ----
# Every output row is checked to be written (NaN-filled outputs, on the GPU).
# Video-DiT, chunked prefill and both affine block sizes compare every row
# with the oracle, in head ranges (one GPU run per workload, shared by its
# parts); long video compares one 128-row query tile in eight of every head
# plus the first and last row of every empty and every heavy query block.

FULL = {
    "video_dit": (lambda: W.video_dit(), 2),
    "chunked_prefill": (lambda: W.chunked_prefill(), 4),
    "affine_bs64": (lambda: W.affine(bs=64), 1),
    "affine_bs32": (lambda: W.affine(bs=32), 1),
    "long_video": (lambda: W.long_video(), 4),
}
_full_cache = {}


def _full_run(ref, name):
    """One GPU run per full-size workload, kept while its parts are compared."""
    if name not in _full_cache:
        _full_cache.clear()
        import gc
        gc.collect()
        w = FULL[name][0]()
        q, k, v, o, lse, stats = run_gpu(ref, w, device_gen=True, label=f"{name}_full")
        _full_cache[name] = (w, (q.cpu(), k.cpu(), v.cpu()), o, lse)
        del q, k, v
    return _full_cache[name]


def _long_video_rows(w, heads):
    rows = []
    nqt = -(-w.sq // 128)
    for h in heads:
        for t in range(h % 8, nqt, 8):  # one 128-row query tile in eight
            i = np.arange(t * 128, min((t + 1) * 128, w.sq))
            rows.append(np.stack([np.zeros_like(i), np.full_like(i, h), i], 1))
        cnt = w.head_mask(0, h).sum(1)
        heavy = cnt >= max(1, int(0.3 * w.head_mask(0, h).shape[1]))
        for qb in np.flatnonzero((cnt == 0) | heavy):  # empty and heavy query blocks
            lo, hi = qb * w.bq[h], min((qb + 1) * w.bq[h], w.sq) - 1
            rows.append(np.array([[0, h, lo], [0, h, hi]]))
    return np.unique(np.concatenate(rows), axis=0)


@pytest.mark.parametrize("name,part", [(n, p) for n, (_, k) in FULL.items() for p in range(k)])
def test_full_size(ref, name, part):
    w, qkv, o, lse = _full_run(ref, name)
    k = FULL[name][1]
    heads = range(part * w.hq // k, (part + 1) * w.hq // k)
    rows = _long_video_rows(w, heads) if name == "long_video" else all_rows(w, heads)
    compare_rows(ref, w, qkv, o, lse, rows, label=f"{name}_full heads {heads.start}..{heads.stop - 1}")
    if part == k - 1:
        _full_cache.clear()


@pytest.mark.parametrize("q_len", [1, 16])
def test_full_decode(ref, q_len):
    """16 sequences x 32 query heads over 8 kv heads, 65,536-token paged cache."""
    w = W.decode(q_len=q_len)
    run_case(ref, w, device_gen=True, label=f"decode_q{q_len}_full")


@pytest.mark.parametrize("q_len", [1, 16])
def test_full_decode_interleaved(ref, q_len):
    """The full decode shapes with the group's heads interleaved row by row
    (split at 32 key tiles)."""
    w = W.decode(q_len=q_len)
    run_case(ref, w, lut_text=forced_lut_text(128, 64, "local", 32, 2), device_gen=True,
             label=f"decode_q{q_len}_full/ilv")
