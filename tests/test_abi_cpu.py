"""The C-ABI library loads, exports every declared entry point and rejects bad arguments
on the host (no GPU needed: every call here fails validation before any HIP call)."""
import ctypes
import os
import re

import pytest

import block_sparse_long_phase1_amd as sa
from block_sparse_long_phase1_amd import build as sa_build

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "star_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.LIB_PATH):
        sa_build.build()
    return sa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(star_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(lib, n), n


def test_exports_nothing_else():
    """The shared library's exported functions are exactly the header's entry points."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    if not os.path.exists(sa.LIB_PATH):
        sa_build.build()
    out = subprocess.run([nm, "-D", "--defined-only", sa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    funcs = sorted(line.split()[-1] for line in out.splitlines() if line.split()[1:2] == ["T"])
    assert funcs == declared_functions(), funcs


def test_timeline_build_exports_the_same_entry_points_plus_its_reader():
    """The profiling build (decode timestamps) is the product library plus one reader; the
    product library does not carry the reader."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    if not os.path.exists(sa_build.TIMELINE_LIB_PATH):
        sa_build.build()

    def funcs(path):
        out = subprocess.run([nm, "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
        return sorted(line.split()[-1] for line in out.splitlines() if line.split()[1:2] == ["T"])
    assert funcs(sa_build.TIMELINE_LIB_PATH) == sorted(declared_functions() + ["star_decode_timeline_read"])
    assert "star_decode_timeline_read" not in funcs(sa.LIB_PATH)


def test_status_strings(lib):
    assert lib.star_status_str(0) == b"STAR_OK"
    assert lib.star_status_str(1) == b"STAR_ERR_INVALID_ARG"
    assert lib.star_status_str(4) == b"STAR_ERR_WORKSPACE"
    assert lib.star_version().count(b".") == 2


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 128, 1, 0.1), 1),          # null q
    ((FAKE, FAKE, FAKE, FAKE, NULL, 0, 32, 32, 4, 2, 128, 1, 0.1), 1),           # L < 1
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 33, 4, 2, 128, 1, 0.1), 1),          # anchor > block
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, -1, 4, 2, 128, 1, 0.1), 1),          # anchor < 0
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 0, 0, 4, 2, 128, 1, 0.1), 1),            # block < 1
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 5, 2, 128, 1, 0.1), 1),          # hq % hkv
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 130, 1, 0.1), 2),          # d unsupported
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 128, 7, 0.1), 1),          # bad dtype
    ((ctypes.c_void_p(0x100008), FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 128, 1, 0.1), 1),  # misaligned
    ((FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 128, 1, float("inf")), 1),  # bad scale
    ((FAKE, FAKE, FAKE, FAKE, NULL, (1 << 24) + 1, 32, 32, 4, 2, 128, 1, 0.1), 2),  # > 2^31/d tokens (MFMA)
    ((FAKE, FAKE, FAKE, FAKE, NULL, (1 << 25) + 1, 32, 32, 4, 2, 64, 1, 0.1), 2),   # > 2^31/d tokens, d = 64
])
def test_phase1_validation(lib, args, expect):
    st = lib.star_phase1_encode(*args, NULL)
    assert st == expect
    assert lib.star_last_error() != b""


def test_partial_and_merge_validation(lib):
    p = lib.star_phase2_partial
    assert p(NULL, 4, FAKE, FAKE, 1024, 8, -1, 4, 2, 128, 1, 0.1, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1
    assert p(FAKE, 0, FAKE, FAKE, 1024, 8, -1, 4, 2, 128, 1, 0.1, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1
    assert p(FAKE, 4, FAKE, FAKE, 100, 8, -1, 4, 2, 128, 1, 0.1, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1  # stride < n_kv*d
    assert p(FAKE, 4, FAKE, FAKE, 1028, 8, -1, 4, 2, 128, 1, 0.1, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1  # stride*2 % 16
    big = 1 << 20
    need = lib.star_phase2_workspace_bytes(128, big, 32, 8, 128)
    assert need > 0
    assert p(FAKE, 128, FAKE, FAKE, big * 128, big, -1, 32, 8, 128, 1, 0.1, FAKE, FAKE, FAKE,
             FAKE, need - 1, NULL) == 4
    over = (1 << 24) + 1   # one token past the MFMA kernel's 32-bit offsets at d = 128
    assert p(FAKE, 4, FAKE, FAKE, over * 128, over, -1, 4, 2, 128, 1, 0.1, FAKE, FAKE, FAKE, FAKE, 1 << 30,
             NULL) == 2
    m = lib.star_softmax_merge
    assert m(FAKE, FAKE, FAKE, 0, 4, 1, 128, FAKE, 1, NULL, NULL) == 1
    assert m(FAKE, FAKE, FAKE, 2, 4, 1, 6, FAKE, 1, NULL, NULL) == 2
    assert m(NULL, FAKE, FAKE, 2, 4, 1, 128, FAKE, 1, NULL, NULL) == 1


def test_decode_validation(lib):
    d = lib.star_decode_step
    B = ctypes.c_int64 * 3
    good = B(0, 50, 100)
    args = lambda bounds, n_sh, tl, tc, ws: (FAKE, FAKE, FAKE, FAKE, FAKE, 100, bounds, n_sh, FAKE, FAKE,
                                            tl, tc, 4, 2, 128, 1, 0.1, FAKE, NULL, FAKE, ws, NULL)
    assert d(*args(B(0, 60, 50), 2, 0, 8, 1 << 30)) == 1          # not monotone
    assert d(*args(B(0, 50, 99), 2, 0, 8, 1 << 30)) == 1          # does not end at L
    assert d(*args(B(1, 50, 100), 2, 0, 8, 1 << 30)) == 1         # does not start at 0
    assert d(*args(good, 2, 8, 8, 1 << 30)) == 1                   # tail full
    assert d(*args(good, 2, -1, 8, 1 << 30)) == 1                  # negative tail
    assert d(*args(good, 0, 0, 8, 1 << 30)) == 1                   # no shards
    assert d(*args(good, 65, 0, 8, 1 << 30)) == 1                  # too many shards
    assert d(*args(good, 2, 0, 8, 16)) == 4                        # workspace too small


def test_decode_noalloc_validation(lib):
    """The no-workspace decode step checks its arguments like star_decode_step and refuses, before
    any device call, a shape whose chunk partials do not fit its static scratch."""
    d = lib.star_decode_step_noalloc
    B = ctypes.c_int64 * 3
    good = B(0, 50, 100)

    def args(bounds=good, n_sh=2, tl=0, tc=8, hq=4, hkv=2, dim=128, L=100):
        return (FAKE, FAKE, FAKE, FAKE, FAKE, L, bounds, n_sh, FAKE, FAKE, tl, tc, hq, hkv, dim, 1, 0.1, FAKE, NULL,
                NULL)
    assert d(*args(bounds=B(0, 60, 50))) == 1                      # not monotone
    assert d(*args(tl=8)) == 1                                     # tail full
    assert d(*args(n_sh=65)) == 1                                  # too many shards
    assert d(*args(hq=5)) == 1                                     # hq % hkv
    many = (ctypes.c_int64 * 65)(*[i * 64 for i in range(65)])
    assert d(*args(bounds=many, n_sh=64, L=4096, hq=1024, hkv=64)) == 4   # partials beyond the scratch
    assert b"static scratch" in lib.star_last_error()
    assert d(*args(hq=2048, hkv=2048)) == 4                        # more kv heads than counters
    need = lib.star_decode_workspace_bytes(4096, 8, 64, 1024, 64, 128)
    assert need > 8 << 20


def test_kv_fp8_validation(lib):
    sc, qz = lib.star_kv_fp8_scales, lib.star_kv_quantize_fp8
    assert sc(NULL, 100, 8, 128, 1, FAKE, NULL) == 1                     # null x
    assert sc(FAKE, -1, 8, 128, 1, FAKE, NULL) == 1                      # negative tokens
    assert sc(FAKE, 100, 0, 128, 1, FAKE, NULL) == 1                     # no heads
    assert sc(FAKE, 100, 70000, 128, 1, FAKE, NULL) == 1                 # too many heads for the grid
    assert sc(FAKE, 100, 8, 100, 1, FAKE, NULL) == 2                     # d % 8
    assert sc(FAKE, 100, 8, 128, 7, FAKE, NULL) == 1                     # bad dtype
    assert sc(FAKE, 100, 8, 128, 1, NULL, NULL) == 1                     # null scale
    assert sc(ctypes.c_void_p(0x100008), 100, 8, 128, 1, FAKE, NULL) == 1  # misaligned x
    assert qz(FAKE, 100, 8, 128, 1, FAKE, NULL, NULL) == 1               # null out
    assert qz(FAKE, 100, 8, 128, 1, NULL, FAKE, NULL) == 1               # null scale
    assert qz(FAKE, 100, 8, 128, 1, FAKE, ctypes.c_void_p(0x100008), NULL) == 1  # misaligned out


def test_decode_kv8_validation(lib):
    d = lib.star_decode_step_kv8
    B = ctypes.c_int64 * 3
    good = B(0, 50, 100)

    def args(bounds=good, ks=FAKE, hq=4, hkv=2, dim=128, dt=1, tl=0, tc=8, ws=1 << 30):
        return (FAKE, FAKE, FAKE, FAKE, FAKE, ks, FAKE, 100, bounds, 2, FAKE, FAKE, tl, tc, hq, hkv, dim, dt, 0.1,
                FAKE, NULL, FAKE, ws, NULL)
    assert d(*args(ks=NULL)) == 1                          # null scale
    assert d(*args(bounds=B(0, 60, 50))) == 1              # not monotone
    assert d(*args(tl=8)) == 1                             # tail full
    assert d(*args(dt=0)) == 2                             # fp32: no E4M3 path
    assert d(*args(dim=96)) == 2                           # head dim 96
    assert d(*args(hq=6, hkv=2)) == 2                      # G = 3
    assert d(*args(ws=16)) == 4                            # workspace too small


def test_partial_kv8_validation(lib):
    p = lib.star_phase2_partial_kv8

    def args(q=FAKE, ks=FAKE, k8=FAKE, stride=1024 * 128, n_kv=1024, hq=4, hkv=2, dim=128, dt=1, rows=8, ws=1 << 30):
        return (q, rows, k8, FAKE, ks, FAKE, stride, n_kv, -1, hq, hkv, dim, dt, 0.1, FAKE, FAKE, FAKE, FAKE, ws, NULL)
    assert p(*args(q=NULL)) == 1                           # null q
    assert p(*args(ks=NULL)) == 1                          # null scale
    assert p(*args(k8=NULL)) == 1                          # null codes with tokens
    assert p(*args(k8=ctypes.c_void_p(0x100008))) == 1     # misaligned codes
    assert p(*args(stride=1024 * 128 + 8)) == 1            # stride not a multiple of 16 bytes
    assert p(*args(stride=100)) == 1                       # stride < n_kv * d
    assert p(*args(rows=0)) == 1                           # no rows
    assert p(*args(dt=0)) == 2                             # fp32: no E4M3 path
    assert p(*args(dim=96)) == 2                           # head dim 96
    assert p(*args(hq=6, hkv=2)) == 2                      # G = 3
    assert p(*args(n_kv=(1 << 24) + 1, stride=((1 << 24) + 1) * 128)) == 2   # past the 32-bit offsets
    assert p(*args(n_kv=1 << 20, stride=(1 << 20) * 128, ws=16)) == 4         # split partition, short workspace


def test_query_kv8_validation(lib):
    q = lib.star_phase2_query_kv8
    B = ctypes.c_int64 * 3
    good = B(0, 50, 100)

    def args(bounds=good, ks=FAKE, k8=FAKE, hq=4, hkv=2, dim=128, dt=1, rows=8, tl=8, tc=8, ws=1 << 30):
        return (FAKE, rows, k8, FAKE, ks, FAKE, 100, bounds, 2, FAKE, FAKE, tl, tc, hq, hkv, dim, dt, 0.1,
                FAKE, NULL, FAKE, ws, NULL)
    assert q(*args(ks=NULL)) == 1                          # null scale
    assert q(*args(k8=NULL)) == 1                          # null codes
    assert q(*args(k8=ctypes.c_void_p(0x100008))) == 1     # misaligned codes
    assert q(*args(bounds=B(0, 60, 50))) == 1              # not monotone
    assert q(*args(tl=7)) == 1                             # fewer cached tokens than rows
    assert q(*args(dt=0)) == 2                             # fp32: no E4M3 path
    assert q(*args(dim=96)) == 2                           # head dim 96
    assert q(*args(hq=6, hkv=2)) == 2                      # G = 3
    assert q(*args(ws=16)) == 4                            # workspace too small


def test_query_validation(lib):
    q = lib.star_phase2_query
    B = ctypes.c_int64 * 3
    good = B(0, 50, 100)
    args = lambda rows, bounds, n_sh, tl, tc, ws: (FAKE, rows, FAKE, FAKE, 100, bounds, n_sh, FAKE, FAKE, tl, tc,
                                                  4, 2, 128, 1, 0.1, FAKE, NULL, FAKE, ws, NULL)
    assert q(*args(8, B(0, 60, 50), 2, 8, 8, 1 << 30)) == 1          # not monotone
    assert q(*args(8, B(0, 50, 99), 2, 8, 8, 1 << 30)) == 1          # does not end at L
    assert q(*args(0, good, 2, 8, 8, 1 << 30)) == 1                  # no rows
    assert q(*args(8, good, 2, 7, 8, 1 << 30)) == 1                  # fewer cached tokens than rows
    assert q(*args(8, good, 2, 9, 8, 1 << 30)) == 1                  # tail_len > tail_cap
    assert q(*args(8, good, 65, 8, 8, 1 << 30)) == 1                 # too many shards
    assert q(*args(8, good, 2, 8, (1 << 24) + 1, 1 << 30)) == 2      # cache past the 32-bit offsets
    assert q(*args(8, good, 2, 8, 8, 16)) == 4                       # workspace too small
    a = list(args(8, good, 2, 8, 8, 1 << 30))
    a[0] = NULL
    assert q(*a) == 1                                                # null q


def test_workspace_queries(lib):
    assert lib.star_phase2_query_workspace_bytes(128, 4, 32, 8, 128) > 0
    assert lib.star_phase2_query_workspace_bytes(128, 0, 32, 8, 128) == 0
    assert lib.star_phase2_query_workspace_bytes(16, 2, 1, 1, 96) == 0  # vector path needs none
    assert lib.star_phase2_query_workspace_bytes(16, 2, 1, 1, 64) > 0   # head dim 64: MFMA path
    assert lib.star_decode_workspace_bytes(32768, 160, 4, 32, 8, 128) > 0
    assert lib.star_decode_workspace_bytes(0, 160, 4, 32, 8, 128) == 0
    assert lib.star_phase2_workspace_bytes(128, 0, 32, 8, 128) == 0
    assert lib.star_phase2_workspace_bytes(16, 2048, 1, 1, 96) == 0  # vector path needs none


def test_binding_names_match_abi():
    for n in declared_functions():
        if n in ("star_status_str", "star_last_error", "star_version"):
            continue
        assert hasattr(sa, n), n


def test_missing_library_raises(tmp_path):
    """Without the native library the binding raises; it has no other implementation."""
    with pytest.raises(RuntimeError, match="not found"):
        sa.load_library(str(tmp_path / "libstarattn.so"))


def test_host_tensors_are_rejected(lib):
    """No CPU fallback: host tensors are refused before any native call."""
    import torch
    q = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        sa.star_phase1_encode(q, k, k.clone(), 8, 8)
    with pytest.raises(ValueError, match="device tensor"):
        sa.star_phase2_query(q, k, k.clone(), [0, 8], k.clone(), k.clone(), 8)
    with pytest.raises(ValueError, match="device tensor"):
        sa.star_phase2_partial(q, k, k.clone(), 8 * 128, 8)


def test_partition_views_are_checked_before_any_call(lib):
    """The partial bindings take the kv head stride from the views (or check the one given
    against both) and refuse views that are short or run past their storage."""
    import torch
    q = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 64, 128, dtype=torch.bfloat16)
    v = torch.zeros(2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must equal"):
        sa.star_phase2_partial(q, k, v, 65 * 128, 64)                       # stride not the views'
    with pytest.raises(ValueError, match="must equal"):
        sa.star_phase2_partial(q, k, torch.zeros(2, 80, 128, dtype=torch.bfloat16)[:, :64], None, 64)  # v's stride
    with pytest.raises(ValueError, match="elements apart"):
        sa.star_phase2_partial(q, k, v[:, ::2], None, 32)                  # v tokens not d apart
    with pytest.raises(ValueError, match="v view holds"):
        sa.star_phase2_partial(q, k, v[:, :16], None, 32)                  # v shorter than n_kv
    with pytest.raises(ValueError, match="k view holds"):
        sa.star_phase2_partial(q, k[:, 40:], v[:, 40:], None, 32)          # 24 tokens left, 32 asked
    k8 = torch.zeros(2, 64, 128, dtype=torch.uint8)
    with pytest.raises(ValueError, match="must equal"):
        sa.star_phase2_partial_kv8(q, k8, k8.clone(), torch.ones(2), torch.ones(2), 100, 64)
    with pytest.raises(ValueError, match="device tensor"):                 # valid views reach the device check
        sa.star_phase2_partial(q, k, v, None, 64)


def test_negative_scale_is_rejected(lib):
    """A negative scale would flip which score is a row's largest; every entry point refuses it."""
    st = lib.star_phase1_encode(FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 128, 1, ctypes.c_float(-0.1), NULL)
    assert st == 1 and b"scale" in lib.star_last_error()
    p = lib.star_phase2_partial
    assert p(FAKE, 4, FAKE, FAKE, 1024, 8, -1, 4, 2, 128, 1, ctypes.c_float(-1.0), FAKE, FAKE, FAKE, NULL, 0,
             NULL) == 1
    B = ctypes.c_int64 * 3
    good = B(0, 50, 100)
    d = lib.star_decode_step
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 100, good, 2, FAKE, FAKE, 0, 8, 4, 2, 128, 1, ctypes.c_float(-0.5),
             FAKE, NULL, FAKE, 1 << 30, NULL) == 1
    q = lib.star_phase2_query
    assert q(FAKE, 8, FAKE, FAKE, 100, good, 2, FAKE, FAKE, 8, 8, 4, 2, 128, 1, ctypes.c_float(-0.5), FAKE, NULL,
             FAKE, 1 << 30, NULL) == 1
    assert lib.star_phase1_encode(FAKE, FAKE, FAKE, FAKE, NULL, 64, 32, 32, 4, 2, 128, 1, ctypes.c_float(0.0),
                                  NULL) != 1 or b"scale" not in lib.star_last_error()
