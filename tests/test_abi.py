"""The C ABI without a GPU: the library loads, exports every declared call,
and rejects bad arguments with the right status before any device work."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_08_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsa.LIB_PATH):
        from block_sparse_attention_08_amd import build
        build.build()
    return bsa.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "bsa_plan" in names and "bsa_forward" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.bsa_abi_version() == 2
    assert L.bsa_status_str(0) == b"ok" and L.bsa_status_str(6) == b"lookup table error"
    assert L.bsa_status_str(4) == b"out of memory"


BASE = dict(batch=1, num_q_heads=4, num_kv_heads=2, seqlen_q=256, seqlen_kv=256, head_dim=128,
            dtype="bf16", block_q=[64] * 4, block_k=[64] * 4)


def plan_status(L, mask=1, table=None, **kw):
    p = dict(BASE, **kw)
    s, keep = bsa.make_problem(p)
    out = ctypes.c_void_p()
    st = L.bsa_plan(ctypes.byref(s), mask, table, None, None, ctypes.byref(out))
    return st, L.bsa_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(head_dim=96), 2, "head_dim"),
    (dict(num_kv_heads=3), 1, "multiple"),
    (dict(block_q=[64, 64, 48, 64]), 2, "head 2"),
    (dict(block_k=[1024] * 4), 2, "block sizes"),
    (dict(seqlen_q=-1), 1, "negative"),
    (dict(batch=0), 1, ">= 1"),
    (dict(dtype=7), 1, "dtype"),
    (dict(causal=2), 1, "flags"),
    (dict(softmax_scale=float("nan")), 1, "softmax_scale"),
    (dict(gqa_union=1, block_k=[64, 32, 64, 64]), 1, "equal block_k"),
    (dict(paged=1, page_size=32, pages_per_seq=8, num_pages=8), 2, "page_size"),
    (dict(paged=1, page_size=64, pages_per_seq=2, num_pages=8), 1, "too short"),
    (dict(paged=1, page_size=64, pages_per_seq=4, num_pages=8), 1, "page table"),
])
def test_plan_rejects_bad_problems(L, kw, status, needle):
    st, msg = plan_status(L, **kw)
    assert st == status and needle in msg, (st, msg)


def test_plan_null_arguments(L):
    out = ctypes.c_void_p()
    assert L.bsa_plan(None, 1, None, None, None, ctypes.byref(out)) == 1
    st, msg = plan_status(L, mask=None)
    assert st == 1 and "mask" in msg
    s, keep = bsa.make_problem(BASE)
    assert L.bsa_plan(ctypes.byref(s), 1, None, None, None, None) == 1


def test_forward_and_export_null_plan(L):
    t = bsa.Tensor(None, 0, 0, 0)
    assert L.bsa_forward(None, ctypes.byref(t), ctypes.byref(t), ctypes.byref(t),
                         ctypes.byref(t), None, None) == 1
    tt = [ctypes.byref(t)] * 4
    assert L.bsa_backward(None, *tt, None, *tt, None) == 1
    assert "NULL" in L.bsa_last_error().decode()
    n = ctypes.c_size_t(0)
    assert L.bsa_plan_export(None, None, ctypes.byref(n)) == 1
    info = bsa.PlanInfo()
    assert L.bsa_plan_stats(None, ctypes.byref(info)) == 1
    L.bsa_plan_free(None)


@pytest.mark.parametrize("text,needle", [
    ("", "bsa-lut 1"), ("bsa-lut 3", "bsa-lut 1"),
    ("bsa-lut 2\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 64 local 0 0", "bad rule range"), ("bsa-lut 1\nrul", "expected 'rule'"),
    ("bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 96 local 0 0", "out of range"),
    ("bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 64 local 0 3", "out of range"),
    ("bsa-lut 1\nrule * x * * 0 1 0 1 0 1 0 1 -> 128 64 local 0 0", "bad rule key"),
    ("bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 128 64 local 0 0", "'->'"),
    ("bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 64 fifo 0 0", "bad regime"),
])
def test_lut_parse_errors(L, text, needle):
    with pytest.raises(bsa.BsaError) as e:
        bsa.Lut.parse(text)
    assert e.value.status == 6 and needle in str(e.value)


def test_lut_schedules(L):
    for sched in ("local", "lpt", "dealt"):
        assert bsa.Lut.parse(f"bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 64 {sched} 0 0").handle.value


def test_lut_files(L, tmp_path):
    lut = bsa.Lut.load(bsa.DEFAULT_LUT)
    assert lut.handle.value
    assert bsa.Lut.load(None).handle.value  # the built-in table
    # A missing or malformed file gives the built-in table with a warning
    # status (BSA_WARN_LUT_DEFAULT), not an error.
    bad = tmp_path / "bad.lut"
    bad.write_text("bsa-lut 1\nrule * * * * 0 1 0 1 0 1 0 1 -> 128 96 local 0 0\n")
    for path, needle in (("/nonexistent/table.lut", "cannot open"), (str(bad), "malformed")):
        out = ctypes.c_void_p()
        st = L.bsa_lut_load(path.encode(), ctypes.byref(out))
        msg = L.bsa_last_error().decode()
        assert st == bsa.BSA_WARN_LUT_DEFAULT and out.value, (st, msg)
        assert needle in msg and "built-in default" in msg, msg
        L.bsa_lut_free(out)
        with pytest.warns(RuntimeWarning, match="built-in default"):
            assert bsa.Lut.load(path).handle.value
    assert L.bsa_status_str(7).startswith(b"warning")


def test_log_levels(L, capfd, monkeypatch, tmp_path):
    """BSA_LOG: 0 prints nothing; 1 prints errors and warnings with their
    message; 2 also names a loaded table. Read at each call."""
    monkeypatch.setenv("BSA_LOG", "0")
    assert plan_status(L, head_dim=96)[0] == 2
    assert "[bsa]" not in capfd.readouterr().err
    monkeypatch.setenv("BSA_LOG", "1")
    st, msg = plan_status(L, head_dim=96)
    err = capfd.readouterr().err
    assert st == 2 and f"[bsa] unsupported: {msg}" in err, err
    out = ctypes.c_void_p()
    assert L.bsa_lut_load(b"/nonexistent/table.lut", ctypes.byref(out)) == bsa.BSA_WARN_LUT_DEFAULT
    L.bsa_lut_free(out)
    err = capfd.readouterr().err
    assert "[bsa] warning" in err and "cannot open" in err, err
    assert L.bsa_lut_load(bsa.DEFAULT_LUT.encode(), ctypes.byref(out)) == 0
    L.bsa_lut_free(out)
    assert "rules" not in capfd.readouterr().err
    monkeypatch.setenv("BSA_LOG", "2")
    assert L.bsa_lut_load(bsa.DEFAULT_LUT.encode(), ctypes.byref(out)) == 0
    L.bsa_lut_free(out)
    n_rules = sum(1 for line in open(bsa.DEFAULT_LUT) if line.startswith("rule "))
    assert f"[bsa] lookup table {bsa.DEFAULT_LUT}: {n_rules} rules" in capfd.readouterr().err


def test_builtin_lut_is_the_packaged_table():
    """The table compiled into the library is the packaged text, byte for
    byte (build.py regenerates the include from lut/gfx950.lut)."""
    from block_sparse_attention_08_amd import build
    inc = open(build.LUT_INC).read()
    assert inc == build.lut_include_text(open(bsa.DEFAULT_LUT).read())


def test_default_lut_accepted_by_oracle(ref):
    from block_sparse_attention_08_amd import workloads as W
    w = W.random_problem(batch=1, hq=2, sq=128, skv=128, bq=64, bk=64, d=64, seed=1)
    ref.plan(w, lut_text=open(bsa.DEFAULT_LUT).read())


def test_select_blocks_rejects_bad_arguments(L):
    """Block selection checks its arguments before queueing anything."""
    s, keep = bsa.make_problem(BASE)
    t = bsa.Tensor(16, 0, 0, 0)
    prm = bsa.SelectParams(1, 0)
    assert L.bsa_select_blocks(ctypes.byref(s), None, ctypes.byref(t), ctypes.byref(t), None, 1,
                               None) == 1
    assert L.bsa_select_blocks(ctypes.byref(s), ctypes.byref(prm), ctypes.byref(t), ctypes.byref(t),
                               None, None, None) == 1
    assert "mask" in L.bsa_last_error().decode()
    for bad in (bsa.SelectParams(0, 0), bsa.SelectParams(11, 0), bsa.SelectParams(1, -1)):
        assert L.bsa_select_blocks(ctypes.byref(s), ctypes.byref(bad), ctypes.byref(t),
                                   ctypes.byref(t), None, 1, None) == 1
        assert "keep_tenths" in L.bsa_last_error().decode()
    sb, keep2 = bsa.make_problem(dict(BASE, mask_batch_broadcast=1))
    assert L.bsa_select_blocks(ctypes.byref(sb), ctypes.byref(prm), ctypes.byref(t), ctypes.byref(t),
                               None, 1, None) == 1
    assert "one mask per batch" in L.bsa_last_error().decode()
    sp, keep3 = bsa.make_problem(dict(BASE, paged=1, page_size=64, pages_per_seq=4, num_pages=4))
    assert L.bsa_select_blocks(ctypes.byref(sp), ctypes.byref(prm), ctypes.byref(t), ctypes.byref(t),
                               None, 1, None) == 1
    assert "page table" in L.bsa_last_error().decode()


def test_mask_size_matches_layout():
    p = dict(BASE, batch=3, block_q=[32, 64, 128, 64], block_k=[64, 128, 32, 64], seqlen_q=300,
             seqlen_kv=500)
    assert bsa.mask_size(p) == 3 * (10 * 8 + 5 * 4 + 3 * 16 + 5 * 8)
