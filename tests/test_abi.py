"""The C ABI without a GPU: the library loads, exports every function the
header declares, the header is plain C, and host-side validation returns
the documented status codes before anything touches the device."""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import self_sparse_speculative_amd as s3r
from self_sparse_speculative_amd.s3r import PagedKVStruct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s3r.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = range(5)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(s3r_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(s3r.lib_path()):
        pytest.fail("libs3r.so is not built (run `python -m self_sparse_speculative_amd.build`)")
    return s3r.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(s3r.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", s3r.lib_path()], capture_output=True, text=True).stdout
        exported = set(re.findall(r"\bT (s3r_\w+)", out))
        assert set(names) <= exported


def test_header_is_plain_c():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc missing")
    r = subprocess.run([gcc, "-fsyntax-only", "-std=c99", "-Wall", "-Werror", "-x", "c",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings_and_version(lib):
    for st in range(5):
        assert s3r.status_string(st).startswith("S3R")
    assert lib.s3r_version() >= 100


def test_budget_matches_oracle(lib):
    rng = np.random.default_rng(0)
    for _ in range(3000):
        s_den = int(rng.integers(1, 60))
        s_num = int(rng.integers(0, s_den + 1))
        L = int(rng.integers(0, 50000))
        W = int(rng.integers(0, 200))
        assert s3r.budget(L, s_num, s_den, W) == oracle.budget(L, s_num, s_den, W)
    assert s3r.budget(-1, 1, 20, 16) == -1
    assert s3r.budget(10, 3, 2, 16) == -1
    assert s3r.budget(10, 1, 0, 16) == -1


def _kv(page=16, D=128, dtype=1, hkv=8, null=False):
    return PagedKVStruct(None if null else 0x1000, 0x1000, 0x1000, 100, 10, hkv, D, page, dtype)


def test_select_validation(lib):
    f = lib.s3r_select
    assert f(None, 100, FAKE, 2, 2, 100, 1, 20, 16, FAKE, 16, FAKE, None, None) == INVALID
    assert f(FAKE, 100, FAKE, 0, 2, 100, 1, 20, 16, FAKE, 16, FAKE, None, None) == INVALID
    assert f(FAKE, 100, FAKE, 2, 2, 100, 1, 0, 16, FAKE, 16, FAKE, None, None) == INVALID      # s_den = 0
    assert f(FAKE, 100, FAKE, 2, 2, 100, 3, 2, 16, FAKE, 16, FAKE, None, None) == INVALID      # s > 1
    assert f(FAKE, 99, FAKE, 2, 2, 100, 1, 20, 16, FAKE, 16, FAKE, None, None) == INVALID      # stride < max_ctx
    assert f(FAKE, 100, FAKE, 2, 2, 100, 1, 2, 16, FAKE, 49, FAKE, None, None) == INVALID      # cap < 50
    assert f(FAKE, 100, FAKE, 2, 2, 100, 1, 20, -1, FAKE, 16, FAKE, None, None) == INVALID     # window < 0


def test_select_grouped_validation_and_capacity(lib):
    f = lib.s3r_select_grouped
    ws = lib.s3r_select_grouped_workspace_bytes(2, 2, 100, 1, 20, 16, 16, 0)
    cap = lib.s3r_select_grouped_capacity(100, 1, 20, 16, 16)
    args = lambda unit=16, ah=0, cap_=cap, ws_b=ws, stride=100, W=16: (FAKE, stride, FAKE, 2, 2, 100, 1, 20, W, unit,
                                                                        ah, FAKE, cap_, FAKE, None, FAKE, ws_b, None)
    assert f(*args(unit=8)) == INVALID
    assert f(*args(cap_=cap - 1)) == INVALID
    assert f(*args(stride=99)) == INVALID
    assert f(*args(W=-1)) == INVALID
    assert f(*args(ws_b=ws - 1)) == WORKSPACE
    assert lib.s3r_select_grouped_workspace_bytes(2, 2, 100, 1, 20, 16, 1, 0) == 0  # plain selection
    assert lib.s3r_select_grouped_capacity(100, 1, 20, 16, 3) == -1
    # the capacity covers every context up to the bound
    for (sn, sd, W) in ((1, 20, 64), (1, 5, 1), (1, 50, 0), (1, 1, 16)):
        for M in (1, 15, 16, 17, 100, 1000, 5000):
            c16 = lib.s3r_select_grouped_capacity(M, sn, sd, W, 16)
            assert c16 >= max(oracle.grouped_count(L, sn, sd, W, 16) for L in range(1, M + 1))
            assert lib.s3r_select_grouped_capacity(M, sn, sd, W, 1) == oracle.budget(M, sn, sd, W)


def test_decode_validation(lib):
    f = lib.s3r_sparse_decode_attn
    kv = _kv()
    ws_ok = lib.s3r_sparse_decode_workspace_bytes(4, 32, 128, 100)
    args = lambda kvs, Hq=32, ws=ws_ok, scale=0.088: (FAKE, ctypes.byref(kvs), FAKE, 16, FAKE, FAKE, FAKE, None, 4,
                                                      Hq, scale, 100, FAKE, None, FAKE, ws, None)
    assert f(*args(_kv(null=True))) == INVALID
    assert f(*args(kv, Hq=30)) == INVALID                 # Hq % Hkv
    assert f(*args(kv, scale=float("nan"))) == INVALID
    assert f(*args(_kv(page=8))) == UNSUPPORTED
    assert f(*args(_kv(D=96))) == UNSUPPORTED
    assert f(*args(kv, Hq=8 * 3)) != UNSUPPORTED          # G = 3 runs on the bf16 x 128 path
    assert f(*args(_kv(dtype=0), Hq=8 * 3)) == UNSUPPORTED  # ... but not on the vector path
    assert f(*args(kv, Hq=8 * 32)) == UNSUPPORTED         # G = 32
    assert f(*args(_kv(dtype=7))) == INVALID
    assert f(*args(kv, ws=ws_ok - 1)) == WORKSPACE
    assert ws_ok == 4 * 32 * 1 * 130 * 4


def test_length_order_validation(lib):
    f = lib.s3r_length_order
    assert f(None, 4, FAKE, None) == INVALID
    assert f(FAKE, 4, None, None) == INVALID
    assert f(FAKE, 0, FAKE, None) == INVALID
    assert f(FAKE, 65536, FAKE, None) == INVALID


def test_verify_validation(lib):
    f = lib.s3r_verify_attn
    ws = lib.s3r_verify_workspace_bytes(4, 6, 32, 8, 128, 1, 160)
    assert ws > 0
    args = lambda kvs, k=6, Hq=32, msl=160, ws_b=ws, stride=160, sc=FAKE: (
        FAKE, ctypes.byref(kvs), FAKE, 4, k, Hq, 0.088, msl, FAKE, None, sc, stride, FAKE, ws_b, None)
    assert f(*args(_kv(), k=16)) == INVALID
    assert f(*args(_kv(), k=-1)) == INVALID
    assert f(*args(_kv(), msl=161)) == INVALID             # 10 pages x 16 < 161
    assert f(*args(_kv(), stride=100)) == INVALID
    assert f(*args(_kv(), msl=6)) == INVALID               # shorter than the block
    assert f(*args(_kv(), k=15, Hq=36)) == INVALID         # Hq % Hkv
    assert f(*args(_kv(hkv=4), k=15, Hq=32)) == UNSUPPORTED  # 16 * 8 = 128 rows
    assert f(*args(_kv(page=32))) == UNSUPPORTED
    assert f(*args(_kv(), ws_b=ws - 1)) == WORKSPACE
    # scores optional: stride is not checked without scores
    assert f(*args(_kv(), stride=0, sc=None, ws_b=ws - 1)) == WORKSPACE


def test_verify_deferred_validation(lib):
    fd, fs = lib.s3r_verify_attn_deferred, lib.s3r_verify_scores
    ws = lib.s3r_verify_workspace_bytes(4, 6, 32, 8, 128, 1, 160)
    dargs = lambda kvs, k=6, Hq=32, msl=160, ws_b=ws, out=FAKE: (
        FAKE, ctypes.byref(kvs), FAKE, 4, k, Hq, 0.088, msl, out, None, FAKE, ws_b, None)
    assert fd(*dargs(_kv(), out=None)) == INVALID
    assert fd(*dargs(_kv(), k=16)) == INVALID
    assert fd(*dargs(_kv(), msl=161)) == INVALID
    assert fd(*dargs(_kv(hkv=4), k=15, Hq=32)) == UNSUPPORTED
    assert fd(*dargs(_kv(), ws_b=ws - 1)) == WORKSPACE
    sargs = lambda kvs, sc=FAKE, stride=160, ws_b=ws, msl=160: (
        ctypes.byref(kvs), FAKE, 4, 6, 32, msl, sc, stride, FAKE, ws_b, None)
    assert fs(*sargs(_kv(), sc=None)) == INVALID           # scores are required here
    assert fs(*sargs(_kv(), stride=159)) == INVALID
    assert fs(*sargs(_kv(page=32))) == UNSUPPORTED
    assert fs(*sargs(_kv(), ws_b=ws - 1)) == WORKSPACE


def test_sample_validation(lib):
    f = lib.s3r_spec_sample
    ws = lib.s3r_spec_sample_workspace_bytes(4, 6, 1000)
    args = lambda k=6, V=1000, T=1.0, ws_b=ws, zd=FAKE: (FAKE, zd, FAKE, FAKE, 4, k, V, T, FAKE, FAKE, None, FAKE,
                                                        ws_b, None)
    assert f(*args(k=16)) == INVALID
    assert f(*args(V=0)) == INVALID
    assert f(*args(T=-1.0)) == INVALID
    assert f(*args(T=float("inf"))) == INVALID
    assert f(*args(zd=None)) == INVALID
    assert f(*args(ws_b=ws - 1)) == WORKSPACE
    assert f(*args(k=0, zd=None, ws_b=0)) == WORKSPACE


def test_verify_pages_and_select_pages_validation(lib):
    kv = _kv()
    ws = lib.s3r_verify_pages_workspace_bytes(4, 6, 32, 8, 128, 1, 160)
    assert 0 < ws < lib.s3r_verify_workspace_bytes(4, 6, 32, 8, 128, 1, 160)
    f = lib.s3r_verify_attn_pages
    args = lambda stride=10, ws_b=ws, pg=FAKE, kvp=kv, ms=160: (FAKE, ctypes.byref(kvp), FAKE, 4, 6, 32,
                                                              0.088, ms, FAKE, None, pg, stride, FAKE, ws_b, None)
    assert f(*args(pg=None)) == INVALID               # page scores are required
    assert f(*args(stride=9)) == INVALID              # ceil(160 / 16) = 10 pages
    assert f(*args(ws_b=ws - 1)) == WORKSPACE
    assert f(*args(kvp=_kv(page=8), ms=80, stride=5)) == UNSUPPORTED
    g = lib.s3r_select_pages
    sw = lib.s3r_select_grouped_workspace_bytes(4, 8, 160, 1, 20, 64, 16, 0)
    cap = lib.s3r_select_grouped_capacity(160, 1, 20, 64, 16)
    gargs = lambda stride=10, cap_=cap, ws_b=sw, sn=1: (FAKE, stride, FAKE, 4, 8, 160, sn, 20, 64, 0, FAKE, cap_,
                                                        FAKE, None, FAKE, ws_b, None)
    assert g(*gargs(stride=9)) == INVALID
    assert g(*gargs(cap_=cap - 1)) == INVALID
    assert g(*gargs(sn=21)) == INVALID
    assert g(*gargs(ws_b=sw - 1)) == WORKSPACE


def test_sample_noalloc_validation(lib):
    # every check before the scratch lookup: nothing here reaches a device
    f = lib.s3r_spec_sample_noalloc
    args = lambda B=4, k=6, V=1000, T=1.0, zd=FAKE, zt=FAKE: (zt, zd, FAKE, FAKE, B, k, V, T, FAKE, FAKE, None, None)
    assert f(*args(k=16)) == INVALID
    assert f(*args(V=0)) == INVALID
    assert f(*args(B=0)) == INVALID
    assert f(*args(T=float("nan"))) == INVALID
    assert f(*args(zd=None)) == INVALID
    assert f(*args(zt=None)) == INVALID
    # a batch whose workspace exceeds the library's fixed scratch is refused
    B = 1
    while lib.s3r_spec_sample_workspace_bytes(B, 15, 1000) <= s3r.SAMPLE_SCRATCH_BYTES:
        B += 256
    assert f(*args(B=B, k=15)) == WORKSPACE
    assert lib.s3r_spec_sample_workspace_bytes(5000, 15, 1000) <= s3r.SAMPLE_SCRATCH_BYTES  # the stated capacity


def test_kv_append_validation(lib):
    f = lib.s3r_kv_append
    args = lambda kvs, n=7, B=4, mp=160, pos=FAKE, kr=FAKE: (kr, FAKE, ctypes.byref(kvs), pos, B, n, mp, None)
    assert f(*args(_kv(), kr=None)) == INVALID
    assert f(*args(_kv(), pos=None)) == INVALID
    assert f(*args(_kv(null=True))) == INVALID
    assert f(*args(_kv(), n=0)) == INVALID
    assert f(*args(_kv(), B=0)) == INVALID
    assert f(*args(_kv(), mp=6)) == INVALID                # max_pos < n
    assert f(*args(_kv(), mp=161)) == INVALID              # beyond 10 pages x 16
    assert f(*args(_kv(page=32))) == UNSUPPORTED
    assert f(*args(_kv(D=96))) == UNSUPPORTED


def test_commit_validation(lib):
    f = lib.s3r_commit
    assert f(None, FAKE, 4, 6, FAKE, None, None, None, None, None) == INVALID
    assert f(FAKE, None, 4, 6, FAKE, None, None, None, None, None) == INVALID
    assert f(FAKE, FAKE, 4, 6, None, None, None, None, None, None) == INVALID
    assert f(FAKE, FAKE, 0, 6, FAKE, None, None, None, None, None) == INVALID
    assert f(FAKE, FAKE, 4, 16, FAKE, None, None, None, None, None) == INVALID


def test_workspace_queries_reject_bad_shapes(lib):
    assert lib.s3r_verify_workspace_bytes(0, 6, 32, 8, 128, 1, 100) == 0
    assert lib.s3r_verify_workspace_bytes(4, 6, 30, 8, 128, 1, 100) == 0
    assert lib.s3r_sparse_decode_workspace_bytes(4, 32, 128, 0) == 0
    assert lib.s3r_spec_sample_workspace_bytes(4, 16, 100) == 0
