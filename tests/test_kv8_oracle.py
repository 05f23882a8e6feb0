"""Pins of the oracle's FP8 K/V path (no GPU): the OCP E4M3 decode against
torch's float8_e4m3fn conversion on all 256 codes and against values the
format's definition fixes, and the kv8 forward against the plain forward on
the decoded inputs."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_08_amd import workloads as W


def test_e4m3_all_codes_match_torch(ref):
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).double().numpy()
    ov = np.array([ref.e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(ov), np.isnan(tv))
    ok = ~np.isnan(tv)
    assert np.array_equal(ov[ok], tv[ok])
    assert int(np.isnan(ov).sum()) == 2  # 0x7f and 0xff only


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0x7E, 448.0), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x39, 1.125), (0xB8, -1.0), (0xFE, -448.0)])
def test_e4m3_definition_values(ref, code, value):
    assert ref.e4m3(code) == value


def test_e4m3_monotone_and_signed(ref):
    pos = [ref.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    assert math.copysign(1.0, ref.e4m3(0x80)) == -1.0 and ref.e4m3(0x80) == 0.0
    assert all(ref.e4m3(c | 0x80) == -ref.e4m3(c) for c in range(1, 0x7F))


@pytest.mark.parametrize("paged", [False, True])
def test_kv8_forward_equals_forward_on_decoded_inputs(ref, paged):
    """With power-of-two scales the decoded K, V are exact in fp32, so the
    kv8 forward must equal the plain forward on (Q, K, V) in fp32."""
    w = W.random_problem(batch=2, hq=4, hkv=2, sq=90, skv=130, d=32, bq=32, bk=64, density=0.5,
                         causal=True, causal_offset=40, paged=paged, page_size=64, seed=501)
    q, k, v = w.make_qkv()
    g = np.random.default_rng(7)
    k8 = torch.from_numpy(g.integers(0, 256, k.shape, dtype=np.uint8))
    v8 = torch.from_numpy(g.integers(0, 256, v.shape, dtype=np.uint8))
    k8[(k8 & 0x7F) == 0x7F] = 0x38  # no NaN codes
    v8[(v8 & 0x7F) == 0x7F] = 0x38
    ks = np.array([0.25, 2.0 ** -6], np.float32)
    vs = np.array([0.5, 4.0], np.float32)
    o8, l8 = ref.forward_kv8(w, q, k8, v8, ks, vs)
    head = 2 if paged else 1
    shp = [1, 1, 1, 1]
    shp[head] = -1
    dec = torch.from_numpy(np.array([ref.e4m3(c) for c in range(256)], np.float32))
    kf = dec[k8.long()] * torch.from_numpy(ks).view(shp)
    vf = dec[v8.long()] * torch.from_numpy(vs).view(shp)
    wf = W.random_problem(batch=2, hq=4, hkv=2, sq=90, skv=130, d=32, dtype="f32", bq=32, bk=64,
                          density=0.5, causal=True, causal_offset=40, paged=paged, page_size=64,
                          seed=501)
    of, lf = ref.forward(wf, q.float(), kf, vf)
    assert np.array_equal(np.isneginf(l8), np.isneginf(lf))
    fin = np.isfinite(lf)
    assert np.allclose(o8, of, rtol=1e-12, atol=1e-12) and np.allclose(l8[fin], lf[fin], rtol=1e-12, atol=1e-12)
    # V scales enter linearly: doubling them doubles O exactly.
    o2, l2 = ref.forward_kv8(w, q, k8, v8, ks, 2 * vs)
    assert np.array_equal(o2, 2 * o8) and np.array_equal(l2, l8)


def test_make_kv8_round_trip():
    w = W.random_problem(batch=1, hq=2, sq=64, skv=200, d=64, bq=64, bk=64, seed=502)
    q, k, v = w.make_qkv()
    k8, v8, ks, vs = w.make_kv8(k, v)
    assert k8.dtype == torch.uint8 and k8.shape == k.shape and ks.shape == (w.hkv,)
    dec = k8.view(torch.float8_e4m3fn).float() * ks.view(1, -1, 1, 1)
    rel = ((dec - k.float()).abs() / k.float().abs().clamp_min(1e-3)).max().item()
    assert rel < 0.07  # 3 mantissa bits: relative step 1/8, error up to 1/16 of a step away
    assert int(k8.view(torch.float8_e4m3fn).float().abs().max()) == 448
