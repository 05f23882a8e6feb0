"""Python binding of libbsa (block-sparse attention for MI355X).

Argument marshalling only: every step of planning and attention runs in the
library's HIP kernels. PyTorch supplies device memory and streams. The names
follow the C ABI in ``include/bsa.h``: ``lut_load``/``lut_parse``, ``plan``
(-> :class:`Plan`), ``Plan.forward``, ``Plan.export``, ``Plan.stats``.

Importing the package does not load the library; the first call does, and
raises if ``libbsa.so`` has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# BSA_LIBRARY selects another build of the library (for example a profiling build).
LIB_PATH = os.environ.get("BSA_LIBRARY") or os.path.join(PKG_DIR, "libbsa.so")
DEFAULT_LUT = os.path.join(PKG_DIR, "lut", "gfx950.lut")

BSA_OK = 0
BSA_WARN_LUT_DEFAULT = 7
STATUS_NAMES = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "shape mismatch",
                4: "out of memory", 5: "HIP error", 6: "lookup table error",
                7: "lookup table replaced by the built-in default"}
DTYPES = {"bf16": 0, "f32": 1}


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libbsa: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("seqlen_q", ctypes.c_int64),
        ("seqlen_kv", ctypes.c_int64), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("block_q", ctypes.POINTER(ctypes.c_int32)), ("block_k", ctypes.POINTER(ctypes.c_int32)),
        ("mask_batch_broadcast", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("causal_kv_offset", ctypes.c_int64), ("gqa_union", ctypes.c_int32),
        ("paged", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_s", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tile_q", "tile_k", "sched", "split", "pack",
                                              "reserved")] + \
               [(n, ctypes.c_int64) for n in ("rows", "entries", "items", "partial_slots",
                                              "combines", "logical_nnz", "logical_blocks",
                                              "density_pm", "imbalance16", "effective_blocks")] + \
               [("effective_flops", ctypes.c_double), ("tile_live_subblocks", ctypes.c_int64),
                ("executed_tiles", ctypes.c_int64), ("partial_slot_bound", ctypes.c_int64)]


class AcsrRun(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("row_num", "row_den", "offset", "stride", "count")]


ACSR_MAX_RUNS = 4


class AcsrHead(ctypes.Structure):
    _fields_ = [("num_runs", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("runs", AcsrRun * ACSR_MAX_RUNS)]


def acsr_heads(heads):
    """bsa_acsr_head array from a per-head list of runs, each run a tuple
    (row_num, row_den, offset, stride, count)."""
    arr = (AcsrHead * max(len(heads), 1))()
    for h, runs in enumerate(heads):
        runs = list(runs)
        arr[h].num_runs = len(runs)
        for j, r in enumerate(runs[:ACSR_MAX_RUNS]):
            arr[h].runs[j] = AcsrRun(*[int(x) for x in r])
    return arr


class SelectParams(ctypes.Structure):
    _fields_ = [("keep_tenths", ctypes.c_int32), ("top_k", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libbsa.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER
        L.bsa_abi_version.restype = ctypes.c_int
        L.bsa_status_str.restype = ctypes.c_char_p
        L.bsa_status_str.argtypes = [ctypes.c_int]
        L.bsa_last_error.restype = ctypes.c_char_p
        L.bsa_lut_load.argtypes = [ctypes.c_char_p, P(vp)]
        L.bsa_lut_parse.argtypes = [ctypes.c_char_p, P(vp)]
        L.bsa_lut_free.argtypes = [vp]
        L.bsa_lut_free.restype = None
        L.bsa_plan.argtypes = [P(Problem), vp, vp, vp, vp, P(vp)]
        L.bsa_forward.argtypes = [vp, P(Tensor), P(Tensor), P(Tensor), P(Tensor), vp, vp]
        if hasattr(L, "bsa_forward_noalloc"):  # (absent from builds before ABI 2)
            L.bsa_forward_noalloc.argtypes = [vp, P(Tensor), P(Tensor), P(Tensor), P(Tensor), vp, vp]
            L.bsa_forward_noalloc.restype = ctypes.c_int
        L.bsa_plan_export.argtypes = [vp, vp, P(ctypes.c_size_t)]
        L.bsa_plan_stats.argtypes = [vp, P(PlanInfo)]
        L.bsa_plan_free.argtypes = [vp]
        L.bsa_plan_free.restype = None
        L.bsa_backward.argtypes = [vp, P(Tensor), P(Tensor), P(Tensor), P(Tensor), vp, P(Tensor),
                                   P(Tensor), P(Tensor), P(Tensor), vp]
        L.bsa_forward_kv8.argtypes = [vp, P(Tensor), P(Tensor), P(Tensor), vp, vp, P(Tensor), vp, vp]
        L.bsa_select_blocks.argtypes = [P(Problem), P(SelectParams), P(Tensor), P(Tensor), vp, vp, vp]
        L.bsa_plan_acsr.argtypes = [P(Problem), P(AcsrHead), vp, vp, P(vp)]
        L.bsa_acsr_features.argtypes = [P(Problem), P(AcsrHead), P(ctypes.c_int64)]
        for f in ("bsa_lut_load", "bsa_lut_parse", "bsa_plan", "bsa_forward", "bsa_forward_kv8", "bsa_backward", "bsa_plan_export",
                  "bsa_plan_stats", "bsa_select_blocks", "bsa_plan_acsr", "bsa_acsr_features"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != BSA_OK:
        raise BsaError(status, lib().bsa_last_error().decode())


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Lut:
    """A regime lookup table (bsa_lut_t)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    @classmethod
    def load(cls, path: Optional[str] = DEFAULT_LUT) -> "Lut":
        """bsa_lut_load: path None gives the built-in table; a missing or
        malformed file also gives it, with a Python warning."""
        h = ctypes.c_void_p()
        st = lib().bsa_lut_load(path.encode() if path else None, ctypes.byref(h))
        if st == BSA_WARN_LUT_DEFAULT:
            import warnings
            warnings.warn("libbsa: " + lib().bsa_last_error().decode(), RuntimeWarning, stacklevel=2)
        else:
            _check(st)
        return cls(h.value)

    @classmethod
    def parse(cls, text: str) -> "Lut":
        h = ctypes.c_void_p()
        _check(lib().bsa_lut_parse(text.encode(), ctypes.byref(h)))
        return cls(h.value)

    @classmethod
    def forced(cls, tq=128, tk=64, sched="local", split=0, pack=1) -> "Lut":
        """A table whose single catch-all rule forces one regime."""
        return cls.parse("bsa-lut 1\nrule * * * * 0 1000000 0 1000000 0 1000000 0 100000000 -> "
                         f"{tq} {tk} {sched} {split} {pack}\n")

    @property
    def handle(self):
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value and _lib is not None:
            _lib.bsa_lut_free(self._h)
            self._h = None


def make_problem(p: dict):
    """A Problem struct from a dict (keys as in bsa_problem); returns (struct, keepalive)."""
    hq = int(p["num_q_heads"])
    bq = (ctypes.c_int32 * hq)(*[int(x) for x in p["block_q"]])
    bk = (ctypes.c_int32 * hq)(*[int(x) for x in p["block_k"]])
    dt = p.get("dtype", "bf16")
    s = Problem(int(p["batch"]), hq, int(p["num_kv_heads"]), int(p["seqlen_q"]),
                int(p["seqlen_kv"]), int(p["head_dim"]), DTYPES[dt] if isinstance(dt, str) else int(dt),
                ctypes.cast(bq, ctypes.POINTER(ctypes.c_int32)),
                ctypes.cast(bk, ctypes.POINTER(ctypes.c_int32)),
                int(p.get("mask_batch_broadcast", 0)), int(p.get("causal", 0)),
                int(p.get("causal_kv_offset", 0)), int(p.get("gqa_union", 0)),
                int(p.get("paged", 0)), int(p.get("page_size", 0)), int(p.get("pages_per_seq", 0)),
                int(p.get("num_pages", 0)), float(p.get("softmax_scale", 0.0)))
    return s, (bq, bk)


def _tensor(t, paged: bool = False) -> Tensor:
    """bsa_tensor of a 4-D torch tensor.

    Q/O and dense K/V are [batch][heads][seq][D]; a paged K/V pool is
    [pages][page_size][kv heads][D], whose token and head axes are swapped
    relative to the (stride_b, stride_h, stride_s) fields.
    """
    if t is None:
        return Tensor(None, 0, 0, 0)
    st = t.stride()
    assert t.dim() == 4 and st[-1] == 1, "expected a 4-D tensor with a contiguous last axis"
    if paged:
        return Tensor(t.data_ptr(), st[0], st[2], st[1])
    return Tensor(t.data_ptr(), st[0], st[1], st[2])


class Plan:
    """A physical tile plan (bsa_plan_t) for one problem and mask."""

    def __init__(self, problem: dict, mask, page_table=None, lut: Optional[Lut] = None,
                 stream=None, _acsr=None):
        self.problem = dict(problem)
        s, keep = make_problem(problem)
        h = ctypes.c_void_p()
        self._lut = lut
        if _acsr is not None:
            _check(lib().bsa_plan_acsr(ctypes.byref(s), acsr_heads(_acsr),
                                       lut.handle if lut is not None else None,
                                       _stream_handle(stream), ctypes.byref(h)))
        else:
            _check(lib().bsa_plan(ctypes.byref(s), mask.data_ptr() if mask is not None and mask.numel() else None,
                                  page_table.data_ptr() if page_table is not None else None,
                                  lut.handle if lut is not None else None, _stream_handle(stream),
                                  ctypes.byref(h)))
        self._h = h

    def forward(self, q, k, v, o=None, lse=None, stream=None):
        """O and LSE for Q/K/V (torch tensors on the plan's device)."""
        import torch
        p = self.problem
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((p["batch"], p["num_q_heads"], p["seqlen_q"]), dtype=torch.float32,
                              device=q.device)
        paged = bool(p.get("paged", 0))
        tq, tk, tv, to = _tensor(q), _tensor(k, paged), _tensor(v, paged), _tensor(o)
        _check(lib().bsa_forward(self._h, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                 ctypes.byref(to), lse.data_ptr() if lse.numel() else None,
                                 _stream_handle(stream)))
        return o, lse

    def forward_noalloc(self, q, k, v, o, lse, stream=None):
        """bsa_forward_noalloc: forward into caller-provided O and LSE with the
        library's static device scratch (no allocation by the library)."""
        p = self.problem
        paged = bool(p.get("paged", 0))
        tq, tk, tv, to = _tensor(q), _tensor(k, paged), _tensor(v, paged), _tensor(o)
        _check(lib().bsa_forward_noalloc(self._h, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                         ctypes.byref(to), lse.data_ptr() if lse.numel() else None,
                                         _stream_handle(stream)))
        return o, lse

    def forward_kv8(self, q, k8, v8, k_scale, v_scale, o=None, lse=None, stream=None):
        """O and LSE with K, V as e4m3 bytes (uint8 tensors of K's layout) and
        fp32 per-kv-head scales (device tensors [Hkv])."""
        import torch
        p = self.problem
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((p["batch"], p["num_q_heads"], p["seqlen_q"]), dtype=torch.float32,
                              device=q.device)
        paged = bool(p.get("paged", 0))
        tq, tk, tv, to = _tensor(q), _tensor(k8, paged), _tensor(v8, paged), _tensor(o)
        _check(lib().bsa_forward_kv8(self._h, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                     k_scale.data_ptr(), v_scale.data_ptr(), ctypes.byref(to),
                                     lse.data_ptr() if lse.numel() else None, _stream_handle(stream)))
        return o, lse

    def backward(self, q, k, v, o, lse, dout, dq=None, dk=None, dv=None, stream=None):
        """dQ, dK, dV for upstream gradient dout, given the forward's inputs
        and outputs (torch tensors on the plan's device)."""
        import torch
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        ts = [_tensor(x) for x in (q, k, v, o, dout, dq, dk, dv)]
        _check(lib().bsa_backward(self._h, *(ctypes.byref(t) for t in ts[:4]),
                                  lse.data_ptr() if lse.numel() else None, ctypes.byref(ts[4]),
                                  *(ctypes.byref(t) for t in ts[5:]), _stream_handle(stream)))
        return dq, dk, dv

    def export(self) -> bytes:
        n = ctypes.c_size_t(0)
        _check(lib().bsa_plan_export(self._h, None, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value)
        _check(lib().bsa_plan_export(self._h, buf, ctypes.byref(n)))
        return buf.raw[: n.value]

    def stats(self) -> dict:
        info = PlanInfo()
        _check(lib().bsa_plan_stats(self._h, ctypes.byref(info)))
        return {name: getattr(info, name) for name, _ in PlanInfo._fields_}

    def free(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().bsa_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def plan(problem: dict, mask, page_table=None, lut: Optional[Lut] = None, stream=None) -> Plan:
    return Plan(problem, mask, page_table, lut, stream)


def plan_acsr(problem: dict, heads, lut: Optional[Lut] = None, stream=None) -> Plan:
    """bsa_plan_acsr: a plan from affine row descriptors (per head a list of
    runs (row_num, row_den, offset, stride, count)) instead of a mask; the
    problem needs mask_batch_broadcast = 1, no union and no paging."""
    return Plan(problem, None, None, lut, stream, _acsr=heads)


def acsr_features(problem: dict, heads):
    """bsa_acsr_features: per head (selected blocks, largest row, empty rows,
    causally reachable blocks) counted on the host from the runs; no device
    is needed."""
    s, keep = make_problem(problem)
    hq = int(problem["num_q_heads"])
    out = (ctypes.c_int64 * (4 * hq))()
    _check(lib().bsa_acsr_features(ctypes.byref(s), acsr_heads(heads), out))
    return [tuple(out[4 * h:4 * h + 4]) for h in range(hq)]


def lut_load(path: Optional[str] = DEFAULT_LUT) -> Lut:
    return Lut.load(path)


def lut_parse(text: str) -> Lut:
    return Lut.parse(text)


def mask_size(problem: dict) -> int:
    """Bytes of the per-batch logical mask of a problem (bsa_plan's layout)."""
    sq, skv = int(problem["seqlen_q"]), int(problem["seqlen_kv"])
    per = sum(-(-sq // int(bq)) * -(-skv // int(bk))
              for bq, bk in zip(problem["block_q"], problem["block_k"]))
    nb = 1 if problem.get("mask_batch_broadcast", 0) else int(problem["batch"])
    return nb * per


def select_blocks(problem: dict, q, k, page_table=None, keep_tenths: int = 1, top_k: int = 0,
                  out=None, stream=None):
    """bsa_select_blocks: the logical mask (uint8 torch tensor on q's device)
    chosen from pooled query/key block scores; keep_tenths of each query
    block's causal candidates, or top_k of them when top_k > 0."""
    import torch
    s, keep = make_problem(problem)
    n = mask_size(problem)
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)[:n]
    prm = SelectParams(int(keep_tenths), int(top_k))
    paged = bool(problem.get("paged", 0))
    tq, tk = _tensor(q), _tensor(k, paged)
    _check(lib().bsa_select_blocks(ctypes.byref(s), ctypes.byref(prm), ctypes.byref(tq),
                                   ctypes.byref(tk),
                                   page_table.data_ptr() if page_table is not None else None,
                                   out.data_ptr() if n else None, _stream_handle(stream)))
    return out
