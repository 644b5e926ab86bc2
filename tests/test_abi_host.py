"""Host-side tests of libmkp (no GPU): exported symbols, argument checks,
the polymerizer against the cost-model oracle, and error paths."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mkp():
    import dynamic_shape_gemm_amd as m
    return m


def test_exports_every_declared_symbol(mkp):
    import ctypes
    header = open(os.path.join(ROOT, "include", "mkp.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = sorted(set(re.findall(r"\b(mkp_\w+)\s*\(", header)))
    assert len(declared) >= 12
    lib = ctypes.CDLL(mkp.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(mkp.EXPORTED) == declared


def test_kernel_library_listing(mkp):
    names = mkp.mkp_kernel_names()
    assert len(names) == len(set(names)) >= 8
    for n in names:
        m = re.fullmatch(r"m(\d+)n(\d+)k(\d+)(x\d+|w\d+)?(_nk)?", n)
        assert m, n
    # every tile exists for both B layouts
    kn = sorted(n for n in names if not n.endswith("_nk"))
    nk = sorted(n[:-3] for n in names if n.endswith("_nk"))
    assert kn == nk


def test_bt_entry_points_check_arguments(mkp):
    # B given as N x K needs ldb >= K; errors come back before any launch
    assert mkp.mkp_gemm_bt_raw(4, 4, 8, 1, 8, 1, 7, 1, 4, 0) == mkp.MKP_ERR_INVALID_ARG
    assert "ldb < K" in mkp.last_error()
    assert mkp.mkp_gemm_bt_raw(4, 4, 8, 0, 8, 1, 8, 1, 4, 0) == mkp.MKP_ERR_INVALID_ARG
    assert mkp.mkp_gemm_batched_bt_raw(-1, 4, 4, 8, 1, 8, 32, 1, 8, 32, 1, 4, 16, 0) == mkp.MKP_ERR_INVALID_ARG
    assert mkp.mkp_gemm_bt_raw(0, 4, 8, 0, 8, 0, 8, 0, 4, 0) == mkp.MKP_OK
    # N x K plans use N x K kernels only; K x N plans use K x N kernels
    # unless they first transpose B, and then N x K kernels only
    for bt in (False, True):
        p = mkp.mkp_plan_describe(1, 1000, 700, 300, bt=bt)
        nk = bt or p["transpose_b"]
        assert p["regions"] and all(r["kernel"].endswith("_nk") == nk for r in p["regions"])
    try:
        mkp.mkp_set_option("transpose_b", 0)
        p = mkp.mkp_plan_describe(1, 1000, 700, 300, bt=False)
        assert not p["transpose_b"] and not any(r["kernel"].endswith("_nk") for r in p["regions"])
    finally:
        mkp.mkp_set_option("transpose_b", 1)


def test_invalid_arguments_fail_before_any_launch(mkp):
    bad = [
        (-1, 4, 4, 8, 4, 4, 8, 4),   # negative M
        (4, 4, 8, 1, 7, 1, 4, 4),    # lda < K
        (4, 4, 8, 1, 8, 1, 3, 4),    # ldb < N
        (4, 4, 8, 1, 8, 1, 4, 3),    # ldc < N
        (4, 4, 8, 0, 8, 1, 4, 4),    # A NULL
        (4, 4, 8, 1, 8, 0, 4, 4),    # B NULL
    ]
    for M, N, K, A, lda, B, ldb, ldc in bad:
        rc = mkp.mkp_gemm_raw(M, N, K, A, lda, B, ldb, 1, ldc, 0)
        assert rc == mkp.MKP_ERR_INVALID_ARG, (M, N, K, lda, ldb, ldc)
        assert mkp.last_error()
    assert mkp.mkp_gemm_raw(4, 4, 8, 1, 8, 1, 4, 0, 4, 0) == mkp.MKP_ERR_INVALID_ARG  # C NULL
    assert mkp.mkp_gemm_raw(1 << 31, 4, 8, 1, 8, 1, 4, 1, 4, 0) == mkp.MKP_ERR_INVALID_ARG
    assert mkp.mkp_gemm_batched_raw(2, 4, 4, 8, 1, 8, -1, 1, 4, 32, 1, 4, 16, 0) == mkp.MKP_ERR_INVALID_ARG
    # empty products succeed without touching any pointer
    assert mkp.mkp_gemm_raw(0, 4, 8, 0, 8, 0, 4, 0, 4, 0) == mkp.MKP_OK
    assert mkp.mkp_gemm_raw(4, 0, 8, 0, 8, 0, 4, 0, 4, 0) == mkp.MKP_OK
    assert mkp.mkp_gemm_batched_raw(0, 4, 4, 8, 0, 8, 32, 0, 4, 32, 0, 4, 16, 0) == mkp.MKP_OK


def test_options_and_errors(mkp):
    with pytest.raises(mkp.MkpError):
        mkp.mkp_set_option("no_such_option", "1")
    with pytest.raises(mkp.MkpError) as e:
        mkp.mkp_set_option("force_kernel", "m1n1k1")
    assert e.value.code == mkp.MKP_ERR_UNSUPPORTED
    with pytest.raises(mkp.MkpError):
        mkp.mkp_set_option("patterns", "III")
    for key, bad in (("cost_model", "flops"), ("plan_rank", "-1"), ("nt_stores", "64"), ("nt_stores", "-1")):
        with pytest.raises(mkp.MkpError) as e:
            mkp.mkp_set_option(key, bad)
        assert e.value.code == mkp.MKP_ERR_INVALID_ARG
    # every store-policy value the option documents is accepted; 33 is the default
    for v in (0, 63, 33):
        assert mkp.mkp_set_option("nt_stores", v) == 0
    with pytest.raises(mkp.MkpError):
        mkp.mkp_load_calibration("/nonexistent/table.tbl")
    mkp.mkp_load_calibration(None)


def test_bad_tables_rejected(mkp, tmp_path):
    for text in ["device 0\n", "kernel X 16 16 16 1\n", "device 4\nkernel X 16 16 16 1\ng Y 1:1\n",
                 "frobnicate 3\n", "device 4\nkernel X 16 16 16 1\ng X 1:1\ntail X 1.0:0.5\n",
                 "device 4\nkernel X 16 16 16 1\ng X 1:1\ntail X 0.5:1.5\n",
                 "device 4\nkernel X 16 16 16 1\ng X 1:1\ntail Y 0.5:0.5\n"]:
        with pytest.raises(mkp.MkpError):
            mkp.mkp_plan_with_table(text, 1, 64, 64, 64)
    p = tmp_path / "t.tbl"
    p.write_text("device 4\nkernel notalibkernel 16 16 16 1\ng notalibkernel 1:1\n")
    with pytest.raises(mkp.MkpError):
        mkp.mkp_load_calibration(str(p))
    p.write_text("device 4\nkernel m64n64k64 32 64 64 1\ng m64n64k64 1:1\n")
    with pytest.raises(mkp.MkpError):
        mkp.mkp_load_calibration(str(p))
    mkp.mkp_load_calibration(None)


def test_buffer_too_small(mkp):
    import ctypes
    buf = ctypes.create_string_buffer(8)
    rc = mkp._lib.mkp_plan_describe(1, 100, 100, 100, 7, buf, 8)
    assert rc == mkp.MKP_ERR_BUFFER


def test_plan_describe_special_shapes(mkp):
    assert mkp.mkp_plan_describe(1, 0, 10, 10)["pattern"] == "empty"
    assert mkp.mkp_plan_describe(0, 10, 10, 10)["pattern"] == "empty"
    p = mkp.mkp_plan_describe(1, 10, 10, 0)
    assert p["pattern"] == "zero" and p["regions"] == []
    p = mkp.mkp_plan_describe(1, 4096, 4096, 4096)
    assert p["pattern"] in ("I", "II-M", "II-N") and p["regions"]


def test_force_kernel_and_split(mkp):
    try:
        mkp.mkp_set_option("force_kernel", "m64n64k64")
        mkp.mkp_set_option("force_splitk", 4)
        p = mkp.mkp_plan_describe(1, 300, 300, 4096)
        assert p["pattern"] == "I"
        assert [r["kernel"] for r in p["regions"]] == ["m64n64k64"]
        assert p["regions"][0]["s"] == 4
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


def test_shipped_table_loads(mkp):
    """The calibrated table that ships with the library fits its kernels
    (tiles and B layouts) and is the one in use."""
    mkp.mkp_load_calibration(None)
    table = mkp.mkp_stats()["table"]
    assert table.endswith("gfx950.tbl"), table
    names = set(mkp.mkp_kernel_names())
    text = open(table).read()
    listed = {line.split()[1] for line in text.splitlines() if line.startswith("kernel ")}
    assert listed == names


def test_grouped_argument_errors(mkp):
    """Bad grouped calls are refused on the host before any launch (no GPU
    needed: every check precedes the first device call)."""
    fake = 1 << 20  # never dereferenced: each call fails its checks first
    ok = dict(M=64, K=64, A=fake, lda=64, N=[64, 32], B=[fake, fake], ldb=[64, 32], C=[fake, fake], ldc=[64, 32])

    def call(bt=False, **kw):
        a = dict(ok)
        a.update(kw)
        return mkp.mkp_gemm_grouped_raw(a["M"], a["K"], a["A"], a["lda"], a["N"], a["B"], a["ldb"], a["C"],
                                        a["ldc"], 0, bt=bt)

    E = mkp.MKP_ERR_INVALID_ARG
    assert call(N=[64] * 5, B=[fake] * 5, ldb=[64] * 5, C=[fake] * 5, ldc=[64] * 5) == E   # > 4 groups
    assert call(N=[], B=[], ldb=[], C=[], ldc=[]) == E
    assert call(M=-1) == E
    assert call(N=[64, -1]) == E
    assert call(ldb=[64, 31]) == E          # ldb < N
    assert call(ldc=[63, 32]) == E          # ldc < N
    assert call(lda=63) == E                # lda < K
    assert call(A=0) == E
    assert call(B=[fake, 0]) == E
    assert call(C=[0, fake]) == E
    assert call(bt=True, ldb=[64, 63]) == E  # N x K: ldb < K
    assert "ldb" in mkp.last_error()
    # nothing to do: no launch, success
    assert call(M=0) == mkp.MKP_OK
    assert call(N=[0, 0]) == mkp.MKP_OK
    with pytest.raises(ValueError):
        mkp.mkp_gemm_grouped(64, 64, fake, 64, [64], [fake, fake], [64], [fake], [64], stream=0)


def test_grouped_plan_describe(mkp):
    p = mkp.mkp_plan_describe_grouped(4096, 768, [768, 768, 768], bt=True)
    (r,) = p["regions"]
    assert r["n"] == 3 * 768 and r["kernel"].endswith("_nk")
    p = mkp.mkp_plan_describe_grouped(100, 300, [5, 0, 700])
    assert p["regions"][0]["n"] == 705 and not p["regions"][0]["kernel"].endswith("_nk")
    assert mkp.mkp_plan_describe_grouped(0, 300, [5])["regions"] == []
    with pytest.raises(mkp.MkpError):
        mkp.mkp_plan_describe_grouped(10, 10, [1, 2, 3, 4, 5])


def test_gemm_ex_argument_errors(mkp):
    fake = 1 << 20  # never dereferenced: each call fails its checks first

    def call(**kw):
        a = dict(batch=1, M=8, N=8, K=8, A=fake, lda=8, sA=0, B=fake, ldb=8, sB=0, lay=0, C=fake, ldc=8, sC=0,
                 alpha=1.0, beta=0.0, bias=None, act=0)
        a.update(kw)
        return mkp.mkp_gemm_ex_raw(a["batch"], a["M"], a["N"], a["K"], a["A"], a["lda"], a["sA"], a["B"], a["ldb"],
                                   a["sB"], a["lay"], a["C"], a["ldc"], a["sC"], a["alpha"], a["beta"], a["bias"],
                                   a["act"], 0)

    E = mkp.MKP_ERR_INVALID_ARG
    assert call(lay=2) == E
    assert call(act=5) == E and "activation" in mkp.last_error()
    assert call(act=-1) == E
    assert call(alpha=float("nan")) == E
    assert call(beta=float("inf")) == E
    assert call(lda=7) == E
    assert call(lay=1, ldb=7) == E          # N x K needs ldb >= K
    assert call(ldc=7) == E
    assert call(M=0, act=2, beta=1.0) == mkp.MKP_OK   # empty output: nothing to do
    with pytest.raises(KeyError):
        call(act="tanh")


def test_conv2d_argument_errors(mkp):
    fake = 1 << 20  # never dereferenced: each call fails its checks first

    def call(**kw):
        a = dict(N=1, H=8, W=8, C=16, K=8, R=3, S=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, x=fake, w=fake, y=fake,
                 bias=None, act=0)
        a.update(kw)
        return mkp.mkp_conv2d_raw(a["N"], a["H"], a["W"], a["C"], a["K"], a["R"], a["S"], a["sh"], a["sw"], a["ph"],
                                  a["pw"], a["dh"], a["dw"], a["x"], a["w"], a["y"], a["bias"], a["act"], 0)

    E = mkp.MKP_ERR_INVALID_ARG
    assert call(H=0) == E
    assert call(C=0) == E
    assert call(R=0) == E
    assert call(sh=0) == E
    assert call(dw=0) == E
    assert call(ph=-1) == E
    assert call(R=11, ph=0) == E and "filter larger" in mkp.last_error()   # 11 > 8 + 0
    assert call(S=3, dw=5, pw=0) == E                                       # span 11 > 8
    assert call(act=9) == E
    assert call(x=0) == E
    assert call(N=0) == mkp.MKP_OK   # nothing to do
    assert call(K=0) == mkp.MKP_OK
    assert mkp.conv_out_size(224, 7, 2, 3, 1) == 112


def test_table_named_by_environment_must_exist(tmp_path):
    """A missing shipped table falls back to analytic estimates, but a table
    that MKP_CALIB names and that cannot be read is an error (and a warning
    on the first call), so a mistyped path is not silently replaced."""
    import os
    import subprocess
    import sys

    code = (
        "import dynamic_shape_gemm_amd as m\n"
        "try:\n"
        "    m.mkp_load_calibration(None)\n"
        "    print('loaded')\n"
        "except m.MkpError as e:\n"
        "    print('error', e.code, m.last_error())\n"
    )
    env = dict(os.environ, MKP_CALIB=str(tmp_path / "missing.tbl"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "error -1" in r.stdout and "missing.tbl" in r.stdout, r.stdout
    assert "missing.tbl" in r.stderr and "analytic" in r.stderr, r.stderr


def test_fast_marshalling_agrees_with_ctypes(mkp):
    """The CPython marshalling module forwards to the same entry points as
    ctypes: same status codes for argument errors and for empty calls."""
    assert mkp._fast is not None, "the marshalling module was not built beside the library"
    cases_gemm = [(-1, 4, 4, 1, 4, 1, 4, 1, 4, 0), (4, 4, 8, 1, 7, 1, 4, 1, 4, 0), (4, 4, 8, 0, 8, 1, 4, 1, 4, 0),
                  (0, 4, 8, 0, 8, 0, 4, 0, 4, 0), (4, 4, 8, 1, 8, 1, 4, 1, 3, 0)]
    for args in cases_gemm:
        assert mkp._fast.gemm(*args) == mkp._lib.mkp_gemm(*args), args
        assert mkp._fast.gemm_bt(*args) == mkp._lib.mkp_gemm_bt(*args), args
    cases_batched = [(0, 17, 17, 64, 1, 64, 1088, 1, 17, 1088, 1, 17, 289, 0),
                     (-2, 17, 17, 64, 1, 64, 1088, 1, 17, 1088, 1, 17, 289, 0),
                     (2, 17, 17, 64, 1, 63, 1088, 1, 17, 1088, 1, 17, 289, 0)]
    for args in cases_batched:
        assert mkp._fast.gemm_batched(*args) == mkp._lib.mkp_gemm_batched(*args), args
        assert mkp._fast.gemm_batched_bt(*args) == mkp._lib.mkp_gemm_batched_bt(*args), args
    with pytest.raises(TypeError):
        mkp._fast.gemm(1, 2, 3)
    with pytest.raises(TypeError):
        mkp._fast.gemm(1, 2, 3, "A", 4, 5, 6, 7, 8, 0)
