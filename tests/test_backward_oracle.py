"""Pins of the CPU oracle's backward pass (ref_backward) against what is fixed
independently of it (no GPU):

- central finite differences of the oracle's own forward (itself pinned in
  test_oracle_pins.py): the gradient of L = sum(dO * O) with respect to every
  element of Q, K and V;
- torch's float64 autograd through a plainly written masked softmax
  attention, on larger shapes;
- exact invariants: the rows of dS sum to zero, so the dK rows of a kv head
  sum to zero; the P rows sum to one, so the dV rows sum to the dO rows of
  the non-empty query rows; a row with one allowed key has dS = 0; keys no
  row sees and rows that see no key get zero gradients;
- the sampled modes (a subset of rows, a window of keys) equal the
  corresponding slices of the full result.

A dropped term of the softmax Jacobian, a wrong sign, a missing scale, a
transposed operand, a wrong kv-head mapping or a wrong key set fails one of
them.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_08_amd import workloads as W
from tests.test_oracle_pins import element_mask

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

TINY = {
    "plain_mixed": lambda: W.random_problem(batch=1, hq=2, hkv=1, sq=19, skv=23, d=4, dtype="f32",
                                            bq=[16, 32], bk=[16, 16], density=0.6, seed=301),
    "causal_offset_empty": lambda: W.random_problem(batch=1, hq=2, sq=21, skv=18, d=4, dtype="f32",
                                                    bq=16, bk=16, density=0.7, causal=True,
                                                    causal_offset=-3, empty_rows=0.3, seed=302),
    "gqa_union": lambda: W.random_problem(batch=2, hq=4, hkv=2, sq=17, skv=20, d=4, dtype="f32",
                                          bq=16, bk=16, density=0.4, gqa_union=True, causal=True,
                                          causal_offset=2, seed=303),
    "broadcast": lambda: W.random_problem(batch=2, hq=1, sq=18, skv=33, d=4, dtype="f32", bq=16,
                                          bk=32, density=0.5, mask_broadcast=True, seed=304),
}


def _loss(ref, w, q, k, v, dout):
    o, _ = ref.forward(w, q, k, v, mode=1)
    return float(np.sum(o * dout.numpy().astype(np.float64).reshape(o.shape)))


@pytest.mark.parametrize("case", list(TINY))
def test_finite_differences(ref, case):
    w = TINY[case]()
    q, k, v = w.make_qkv()
    dout = w.make_dout()
    dq, dk, dv = ref.backward(w, q, k, v, dout)
    grads = {"q": dq.reshape(q.shape), "k": dk.reshape(k.shape), "v": dv.reshape(v.shape)}
    tensors = {"q": q, "k": k, "v": v}
    h = 1e-3
    for name, x in tensors.items():
        flat = x.numpy().reshape(-1)
        fd = np.zeros(flat.size)
        for idx in range(flat.size):
            x0 = flat[idx]
            xp, xm = np.float32(x0 + h), np.float32(x0 - h)
            flat[idx] = xp
            lp = _loss(ref, w, q, k, v, dout)
            flat[idx] = xm
            lm = _loss(ref, w, q, k, v, dout)
            flat[idx] = x0
            fd[idx] = (lp - lm) / (float(xp) - float(xm))
        g = grads[name].reshape(-1)
        err = np.abs(fd - g)
        assert np.all(err <= 2e-5 + 1e-4 * np.abs(g)), (name, float(err.max()), int(err.argmax()))
        # every tensor has gradient somewhere (the case is not vacuous)
        assert np.abs(g).max() > 1e-2, name


def _autograd(w, q, k, v, dout):
    """Gradients of sum(dout * O) by torch float64 autograd of softmax
    attention over the element-level allowed set (rows with no allowed key
    output zero)."""
    gs = w.hq // w.hkv
    Q = q.double().clone().requires_grad_(True)
    K = k.double().clone().requires_grad_(True)
    V = v.double().clone().requires_grad_(True)
    dO = dout.double()
    scale = 1.0 / np.sqrt(w.d)
    loss = 0.0
    for b in range(w.batch):
        for h in range(w.hq):
            m = torch.from_numpy(element_mask(w, b, h))
            s = scale * (Q[b, h] @ K[b, h // gs].T)
            empty = ~m.any(1, keepdim=True)
            s = torch.where(m, s, torch.full_like(s, -torch.inf))
            s = torch.where(empty, torch.zeros_like(s), s)
            p = torch.where(empty, torch.zeros_like(s), torch.softmax(s, dim=1))
            loss = loss + (dO[b, h] * (p @ V[b, h // gs])).sum()
    loss.backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("case", [
    dict(batch=2, hq=4, hkv=2, sq=70, skv=90, d=16, bq=[16, 32, 64, 16], bk=[32, 16, 16, 64],
         density=0.4, causal=True, causal_offset=20, empty_rows=0.1, seed=311),
    dict(batch=1, hq=4, hkv=1, sq=64, skv=100, d=8, bq=16, bk=32, density=0.3, gqa_union=True,
         causal=True, causal_offset=36, seed=312),
    dict(batch=2, hq=2, sq=50, skv=40, d=8, bq=32, bk=16, density=0.5, mask_broadcast=True, seed=313),
], ids=["gqa_causal_mixed", "union", "broadcast"])
def test_matches_torch_autograd(ref, case):
    w = W.random_problem(dtype="f32", **case)
    q, k, v = w.make_qkv()
    dout = w.make_dout()
    dq, dk, dv = ref.backward(w, q, k, v, dout)
    tq, tk, tv = _autograd(w, q, k, v, dout)
    for name, a, t in (("dq", dq, tq), ("dk", dk, tk), ("dv", dv, tv)):
        a = a.reshape(t.shape)
        assert np.allclose(a, t, rtol=1e-9, atol=1e-11), (name, float(np.abs(a - t).max()))


def test_invariants(ref):
    w = W.random_problem(batch=2, hq=4, hkv=2, sq=150, skv=170, d=32, bq=[16, 64, 32, 16],
                         bk=[32, 16, 64, 16], density=0.3, causal=True, causal_offset=0,
                         empty_rows=0.15, seed=321)
    q, k, v = w.make_qkv()
    dout = w.make_dout()
    dq, dk, dv = ref.backward(w, q, k, v, dout)
    dq = dq.reshape(w.batch, w.hq, w.sq, w.d)
    do = dout.double().numpy()
    gs = w.hq // w.hkv
    seen = np.zeros((w.batch, w.hkv, w.skv), bool)
    for b in range(w.batch):
        dv_expect = np.zeros((w.hkv, w.d))
        for h in range(w.hq):
            m = element_mask(w, b, h)
            seen[b, h // gs] |= m.any(0)
            rows = m.any(1)
            dv_expect[h // gs] += do[b, h][rows].sum(0)
            # rows with no key, and rows with exactly one key (P = 1, so dS = 0)
            assert np.all(dq[b, h][~rows] == 0.0)
            assert np.all(dq[b, h][m.sum(1) == 1] == 0.0)
        for g in range(w.hkv):
            tot = np.abs(dk[b, g]).sum(0)
            assert np.all(np.abs(dk[b, g].sum(0)) <= 1e-12 * tot + 1e-300)
            assert np.allclose(dv[b, g].sum(0), dv_expect[g], rtol=1e-12, atol=1e-12)
    assert np.all(dk[~seen] == 0.0) and np.all(dv[~seen] == 0.0)
    assert (~seen).any() and seen.any()
    # the case has rows with one key (causal offset 0: row 0 of a selected first block)
    assert any((element_mask(w, b, h).sum(1) == 1).any() for b in range(w.batch) for h in range(w.hq))


def test_sampled_modes_equal_full(ref):
    w = W.random_problem(batch=2, hq=2, hkv=1, sq=90, skv=120, d=16, bq=32, bk=16, density=0.5,
                         causal=True, causal_offset=30, seed=331)
    q, k, v = w.make_qkv()
    dout = w.make_dout()
    dq, dk, dv = ref.backward(w, q, k, v, dout)
    rows = np.array([[1, 1, 89], [0, 0, 0], [1, 0, 45], [0, 1, 17]], np.int64)
    dq_s, _, _ = ref.backward(w, q, k, v, dout, rows=rows, want_dkv=False)
    flat = (rows[:, 0] * w.hq + rows[:, 1]) * w.sq + rows[:, 2]
    assert np.array_equal(dq_s, dq[flat])
    _, dk_s, dv_s = ref.backward(w, q, k, v, dout, kv_range=(37, 70), want_dq=False)
    assert np.array_equal(dk_s, dk[:, :, 37:70]) and np.array_equal(dv_s, dv[:, :, 37:70])


def test_rejects_paged(ref):
    w = W.random_problem(batch=1, hq=2, sq=64, skv=128, d=16, bq=16, bk=16, paged=True, seed=341)
    q, k, v = w.make_qkv()
    with pytest.raises(ValueError):
        ref.backward(w, q, k, v, w.make_dout())
