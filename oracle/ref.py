"""ctypes front end of the CPU oracle (``libbsa_ref.so``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsa_ref.so")


def build() -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math, no FMA contraction)."""
    src = os.path.join(HERE, "bsa_ref.c")
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", "-Wall", "-Wno-unused-result", src, "-o", tmp, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class RefProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("sq", ctypes.c_int64), ("skv", ctypes.c_int64), ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("bq", ctypes.POINTER(ctypes.c_int32)), ("bk", ctypes.POINTER(ctypes.c_int32)),
        ("mask_broadcast", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("causal_offset", ctypes.c_int64), ("gqa_union", ctypes.c_int32),
        ("paged", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.ref_forward.argtypes = [P(RefProblem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.ref_forward.restype = ctypes.c_int
        L.ref_features.argtypes = [P(RefProblem), ctypes.c_void_p, ctypes.c_void_p]
        L.ref_features.restype = ctypes.c_int
        L.ref_plan.argtypes = [P(RefProblem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_char_p,
                               ctypes.c_void_p, ctypes.c_void_p, P(ctypes.c_size_t)]
        L.ref_plan.restype = ctypes.c_int
        L.ref_select.argtypes = [P(RefProblem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.ref_select.restype = ctypes.c_int
        L.ref_backward.argtypes = [P(RefProblem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int]
        L.ref_backward.restype = ctypes.c_int
        L.ref_forward_kv8.argtypes = [P(RefProblem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int]
        L.ref_forward_kv8.restype = ctypes.c_int
        L.ref_e4m3.argtypes = [ctypes.c_uint8]
        L.ref_e4m3.restype = ctypes.c_double
        _lib = L
    return _lib


class _Prob:
    """Holds a RefProblem plus the arrays it points into."""

    def __init__(self, w, scale: float = 0.0):
        self.bq = np.ascontiguousarray(w.bq, dtype=np.int32)
        self.bk = np.ascontiguousarray(w.bk, dtype=np.int32)
        self.mask = np.ascontiguousarray(w.mask, dtype=np.uint8)
        self.table = (np.ascontiguousarray(w.page_table, dtype=np.int32)
                      if w.paged else None)
        i32p = ctypes.POINTER(ctypes.c_int32)
        self.s = RefProblem(
            w.batch, w.hq, w.hkv, w.sq, w.skv, w.d, 0 if w.dtype == "bf16" else 1,
            self.bq.ctypes.data_as(i32p), self.bk.ctypes.data_as(i32p),
            int(w.mask_broadcast), int(w.causal), int(w.causal_offset), int(w.gqa_union),
            int(w.paged), int(w.page_size), int(w.pages_per_seq), int(w.num_pages), float(scale))

    def mask_ptr(self):
        return self.mask.ctypes.data if self.mask.size else None

    def table_ptr(self):
        return self.table.ctypes.data if self.table is not None else None


def _raw(x, dtype: str) -> np.ndarray:
    """Contiguous numpy view of Q/K/V storage: uint16 bf16 bits or float32."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16)
            return x.numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        assert x.dtype == np.uint16
    else:
        assert x.dtype == np.float32
    return x


def forward(w, q, k, v, mode: int = 1, rows=None, nthreads: int = 0, scale: float = 0.0):
    """Oracle forward. Returns (o[n][d] float64, lse[n] float64).

    rows: None for every (b, h, i) in order, or an int64 array of shape [n, 3].
    """
    P = _Prob(w, scale)
    qa, ka, va = _raw(q, w.dtype), _raw(k, w.dtype), _raw(v, w.dtype)
    if rows is None:
        n = w.batch * w.hq * w.sq
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        rp = rows.ctypes.data
    o = np.empty((max(n, 1), w.d), np.float64)
    lse = np.empty(max(n, 1), np.float64)
    rc = lib().ref_forward(ctypes.byref(P.s), P.mask_ptr(), P.table_ptr(), qa.ctypes.data,
                           ka.ctypes.data, va.ctypes.data, mode, rp, n, o.ctypes.data,
                           lse.ctypes.data, nthreads)
    if rc:
        raise ValueError(f"ref_forward rejected the problem ({rc})")
    return o[:n], lse[:n]


def features(w) -> np.ndarray:
    P = _Prob(w)
    nbm = 1 if w.mask_broadcast else w.batch
    out = np.zeros((nbm, w.hq, 4), np.int64)
    rc = lib().ref_features(ctypes.byref(P.s), P.mask_ptr(), out.ctypes.data)
    if rc:
        raise ValueError(f"ref_features rejected the problem ({rc})")
    return out


def plan(w, lut_text=None, force=None) -> bytes:
    """Canonical plan image from the reference planner."""
    P = _Prob(w)
    f = None
    if force is not None:
        f = np.ascontiguousarray(force, dtype=np.int32)
        assert f.size == 5
    lut = lut_text.encode() if isinstance(lut_text, str) else lut_text
    n = ctypes.c_size_t(0)
    L = lib()
    rc = L.ref_plan(ctypes.byref(P.s), P.mask_ptr(), P.table_ptr(), lut,
                    f.ctypes.data if f is not None else None, None, ctypes.byref(n))
    if rc:
        raise ValueError(f"ref_plan failed ({rc})")
    buf = np.zeros(n.value, np.uint8)
    rc = L.ref_plan(ctypes.byref(P.s), P.mask_ptr(), P.table_ptr(), lut,
                    f.ctypes.data if f is not None else None, buf.ctypes.data, ctypes.byref(n))
    if rc:
        raise ValueError(f"ref_plan failed ({rc})")
    return buf.tobytes()


def select(w, q, k, keep_tenths: int = 1, top_k: int = 0) -> np.ndarray:
    """Oracle block selection (mask producer) for the shapes of workload w
    (its own mask is ignored; mask_broadcast must be off). Returns the uint8
    mask, head-concatenated per batch, as ref_forward reads it."""
    P = _Prob(w)
    qa, ka = _raw(q, w.dtype), _raw(k, w.dtype)
    nb = sum(-(-w.sq // w.bq[h]) * -(-w.skv // w.bk[h]) for h in range(w.hq))
    out = np.zeros(max(w.batch * nb, 1), np.uint8)
    s = RefProblem.from_buffer_copy(P.s)
    s.mask_broadcast = 0
    rc = lib().ref_select(ctypes.byref(s), P.table_ptr(), qa.ctypes.data, ka.ctypes.data,
                          int(keep_tenths), int(top_k), out.ctypes.data)
    if rc:
        raise ValueError(f"ref_select rejected the problem ({rc})")
    return out[: w.batch * nb]


def backward(w, q, k, v, dout, rows=None, kv_range=None, want_dq: bool = True,
             want_dkv: bool = True, nthreads: int = 0, scale: float = 0.0):
    """Oracle backward (dense K/V). dout has Q's shape and dtype.

    Returns (dq, dk, dv) in float64: dq is [n][d] for the requested rows
    (rows as in forward; None = every (b, h, i) in order), dk and dv are
    [batch][hkv][hi - lo][d] for the key range kv_range = (lo, hi) (None = all
    keys). A part not wanted is returned as None.
    """
    P = _Prob(w, scale)
    qa, ka, va, da = (_raw(x, w.dtype) for x in (q, k, v, dout))
    if rows is None:
        n = w.batch * w.hq * w.sq
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        rp = rows.ctypes.data
    lo, hi = (0, w.skv) if kv_range is None else (max(0, kv_range[0]), min(w.skv, kv_range[1]))
    kw = max(hi - lo, 0)
    dq = np.zeros((max(n, 1), w.d), np.float64) if want_dq else None
    dk = np.zeros((w.batch, w.hkv, max(kw, 1), w.d), np.float64) if want_dkv else None
    dv = np.zeros_like(dk) if want_dkv else None
    rc = lib().ref_backward(ctypes.byref(P.s), P.mask_ptr(), qa.ctypes.data, ka.ctypes.data,
                            va.ctypes.data, da.ctypes.data, rp, n, lo, hi,
                            dq.ctypes.data if want_dq else None,
                            dk.ctypes.data if want_dkv else None,
                            dv.ctypes.data if want_dkv else None, nthreads)
    if rc:
        raise ValueError(f"ref_backward rejected the problem ({rc})")
    return (dq[:n] if want_dq else None,
            dk[:, :, :kw] if want_dkv else None,
            dv[:, :, :kw] if want_dkv else None)


def e4m3(code: int) -> float:
    """Value of one OCP FP8 E4M3 byte."""
    return lib().ref_e4m3(int(code))


def _bytes(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().contiguous().view(torch.uint8).numpy()
    except ImportError:
        pass
    return np.ascontiguousarray(x, dtype=np.uint8)


def forward_kv8(w, q, k8, v8, k_scale, v_scale, mode: int = 1, rows=None, nthreads: int = 0):
    """Oracle forward with K, V as e4m3 bytes (the workload's K/V layout) and
    fp32 per-kv-head scales; Q bf16. Returns (o[n][d], lse[n]) in float64."""
    P = _Prob(w)
    qa = _raw(q, "bf16")
    ka, va = _bytes(k8), _bytes(v8)
    ks = np.ascontiguousarray(np.asarray(k_scale, dtype=np.float32).reshape(-1))
    vs = np.ascontiguousarray(np.asarray(v_scale, dtype=np.float32).reshape(-1))
    if rows is None:
        n = w.batch * w.hq * w.sq
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        rp = rows.ctypes.data
    o = np.empty((max(n, 1), w.d), np.float64)
    lse = np.empty(max(n, 1), np.float64)
    rc = lib().ref_forward_kv8(ctypes.byref(P.s), P.mask_ptr(), P.table_ptr(), qa.ctypes.data,
                               ka.ctypes.data, va.ctypes.data, ks.ctypes.data, vs.ctypes.data, mode,
                               rp, n, o.ctypes.data, lse.ctypes.data, nthreads)
    if rc:
        raise ValueError(f"ref_forward_kv8 rejected the problem ({rc})")
    return o[:n], lse[:n]


def acsr_mask(w, heads=None) -> np.ndarray:
    """Logical mask (uint8, one mask batch, heads concatenated) that affine
    runs describe: SPLAT's affine-compressed sparse rows (abstract), read as
    follows. Run (row_num, row_den, offset, stride, count) selects, in query
    block r of a head, the key blocks floor(row_num * r / row_den) + offset
    + stride * i for 0 <= i < count, those inside [0, nkb); a row selects the
    union of its head's runs.

    heads: per head a list of run tuples (default: w.acsr)."""
    heads = w.acsr if heads is None else heads
    out = []
    for h in range(w.hq):
        nq, nk = w.nqb(h), w.nkb(h)
        m = np.zeros((nq, nk), np.uint8)
        for num, den, off, stride, count in heads[h]:
            assert den >= 1 and stride >= 1 and count >= 0
            for r in range(nq):
                first = (num * r) // den + off  # Python's // is the floor
                # only the i whose block can fall inside [0, nk)
                i_lo = max(0, -(first // stride))
                i_hi = min(count - 1, (nk - 1 - first) // stride)
                if i_lo > i_hi:
                    continue
                cols = first + stride * np.arange(i_lo, i_hi + 1, dtype=np.int64)
                cols = cols[(cols >= 0) & (cols < nk)]
                m[r, cols] = 1
        out.append(m.reshape(-1))
    return np.ascontiguousarray(np.concatenate(out) if out else np.zeros(0, np.uint8))
