"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments before making any HIP call (so these
tests need no GPU; nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "online_softmax.h")


@pytest.fixture(scope="module")
def L():
    import online_normalizer_amd as ons
    return ons.lib()


@pytest.fixture(scope="module")
def ons():
    import online_normalizer_amd
    return online_normalizer_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:os|safe|naive)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["os_softmax_forward", "os_softmax_topk", "safe_softmax_forward", "os_softmax_stats",
              "naive_softmax_forward", "os_topk_select", "os_softmax_forward_split_noalloc",
              "os_softmax_forward_lse", "os_softmax_forward_split", "os_softmax_forward_workspace_bytes",
              "os_forward_split_plan", "os_device_copy_rows", "os_softmax_topk_ex", "os_last_error", "os_softmax_forward_tuned", "os_forward_plan", "os_device_copy", "os_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} not exported"


def test_exported_symbols_are_c_linkage():
    from online_normalizer_amd import LIB_PATH
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms


def test_version(ons):
    assert ons.os_version() == 200


EINVAL, EUNSUP = -1, -2
F32, BF16 = 0, 1
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced (validation fails first)


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, 4, 4, F32), EINVAL),        # null input
    ((FAKE, None, 4, 4, F32), EINVAL),        # null output
    ((FAKE, FAKE, -1, 4, F32), EINVAL),       # negative rows
    ((FAKE, FAKE, 4, -1, F32), EINVAL),       # negative cols
    ((FAKE, FAKE, 4, 4, 7), EINVAL),          # unknown dtype
    ((FAKE, FAKE, 4, (1 << 28) + 1, F32), EINVAL),  # cols beyond OS_MAX_COLS
    ((FAKE, FAKE, 1 << 62, 1 << 20, F32), EINVAL),  # rows*cols overflow
    ((FAKE + 2, FAKE, 4, 4, F32), EINVAL),    # fp32 pointer not 4-byte aligned
    ((FAKE + 1, FAKE, 4, 4, BF16), EINVAL),   # bf16 pointer not 2-byte aligned
    ((None, None, 0, 4, F32), 0),             # empty: no-op
    ((None, None, 4, 0, BF16), 0),            # empty rows: no-op
])
def test_forward_and_safe_validation(L, ons, args, code):
    for fn in (L.os_softmax_forward, L.safe_softmax_forward, L.naive_softmax_forward):
        rc = fn(*args, None)
        assert rc == code, (fn.__name__, ons.os_last_error())
        if code != 0:
            assert ons.os_last_error()
        else:
            assert ons.os_last_error() == ""


def test_tuned_validation(L, ons):
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 1024, F32, 48, 4, 0, None)
    assert rc == EUNSUP and "lanes_per_row=48" in ons.os_last_error()
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 1024, BF16, 1024, 16, 0, None)
    assert rc == EUNSUP  # that shape exists for fp32 only
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 1025, F32, 64, 4, 0, None)
    assert rc == EINVAL and "cannot hold" in ons.os_last_error()
    # rows that are not 16-byte aligned span up to one more 16-byte block
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 1023, F32, 64, 4, 0, None)
    assert rc == EINVAL and "16-byte block" in ons.os_last_error()
    rc = L.os_softmax_forward_tuned(FAKE + 4, FAKE + 4, 4, 1024, F32, 64, 4, 0, None)
    assert rc == EINVAL and "16-byte block" in ons.os_last_error()
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 2042, BF16, 64, 4, 0, None)
    assert rc == EINVAL and "16-byte block" in ons.os_last_error()
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 64, F32, 64, 4, -1, None)
    assert rc == EINVAL
    rc = L.os_softmax_forward_tuned(FAKE, FAKE, 4, 64, F32, -4, 4, 0, None)
    assert rc == EINVAL


def test_stats_validation(L):
    assert L.os_softmax_stats(FAKE, None, FAKE, 4, 4, F32, None) == EINVAL
    assert L.os_softmax_stats(FAKE, FAKE + 1, FAKE, 4, 4, F32, None) == EINVAL
    assert L.os_softmax_stats(None, FAKE, FAKE, 4, 4, F32, None) == EINVAL
    assert L.os_softmax_stats(None, None, None, 0, 4, F32, None) == 0


def test_lse_validation(L):
    f = L.os_softmax_forward_lse
    assert f(FAKE, FAKE, None, 4, 4, F32, None) == EINVAL          # no lse
    assert f(FAKE, FAKE, FAKE + 2, 4, 4, F32, None) == EINVAL      # misaligned lse
    assert f(None, FAKE, FAKE, 4, 4, F32, None) == EINVAL          # no input
    assert f(FAKE, FAKE + 2, FAKE, 4, 4, F32, None) == EINVAL      # misaligned output
    assert f(FAKE, None, FAKE, 4, 4, 7, None) == EINVAL            # unknown dtype
    assert f(FAKE, None, FAKE, -1, 4, F32, None) == EINVAL         # negative rows
    assert f(None, None, None, 0, 4, F32, None) == 0               # no rows: nothing to do


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, 4, 100, 0), EINVAL),     # K < 1
    ((FAKE, FAKE, FAKE, 4, 100, 33), EINVAL),    # K > KMAX
    ((FAKE, FAKE, FAKE, 4, 5, 6), EINVAL),       # K > cols
    ((None, FAKE, FAKE, 4, 100, 8), EINVAL),
    ((FAKE, None, FAKE, 4, 100, 8), EINVAL),
    ((FAKE, FAKE, None, 4, 100, 8), EINVAL),
    ((FAKE + 2, FAKE, FAKE, 4, 100, 8), EINVAL),
    ((FAKE, FAKE, FAKE, -3, 100, 8), EINVAL),
    ((FAKE, FAKE, FAKE, 4, (1 << 28) + 1, 8), EINVAL),  # cols beyond OS_MAX_COLS
    ((None, None, None, 0, 100, 8), 0),
])
def test_topk_validation(L, args, code):
    assert L.os_softmax_topk(*args, None) == code
    x, p, i, rows, cols, K = args
    assert L.os_topk_select(x, F32, p, i, rows, cols, K, None) == code


def test_topk_select_validation(L):
    f = L.os_topk_select
    assert f(FAKE, 7, FAKE, FAKE, 4, 100, 8, None) == EINVAL        # unknown dtype
    assert f(FAKE + 1, BF16, FAKE, FAKE, 4, 100, 8, None) == EINVAL  # bf16 input not 2-byte aligned
    assert f(FAKE, BF16, FAKE + 2, FAKE, 4, 100, 8, None) == EINVAL  # misaligned values
    assert f(None, BF16, None, None, 0, 100, 8, None) == 0           # no rows


def test_topk_split_validation(L, ons):
    assert ons.os_softmax_topk_workspace_bytes(10, 8, 1) == 0
    need = ons.os_softmax_topk_workspace_bytes(10, 8, 4)
    assert need >= 10 * 4 * 8 + 10 * 4 * 8 * 8
    with pytest.raises(ons.OnlineSoftmaxError):
        ons.os_softmax_topk_workspace_bytes(10, 8, 17)
    with pytest.raises(ons.OnlineSoftmaxError):
        ons.os_softmax_topk_workspace_bytes(1 << 58, 32, 16)                # size would overflow
    f = L.os_softmax_topk_split
    assert f(FAKE, FAKE, FAKE, 10, 1000, 8, 0, FAKE, need, None) == EINVAL      # splits < 1
    assert f(FAKE, FAKE, FAKE, 10, 1000, 8, 17, FAKE, need, None) == EINVAL     # splits > 16
    assert f(FAKE, FAKE, FAKE, 10, 1000, 8, 4, None, need, None) == EINVAL      # no workspace
    assert f(FAKE, FAKE, FAKE, 10, 1000, 8, 4, FAKE, need - 1, None) == EINVAL  # short workspace
    assert f(FAKE, FAKE, FAKE, 10, 1000, 8, 4, FAKE + 16, need, None) == EINVAL  # misaligned workspace
    assert f(FAKE, FAKE, FAKE, 10, 1000, 9, 4, FAKE, need, None) == EINVAL      # K changed: short
    assert f(None, None, None, 0, 1000, 8, 4, None, 0, None) == 0               # empty
    assert ons.os_topk_plan(256, 128256, 8) == 1
    assert ons.os_topk_plan(16, 128256, 8) == 8
    assert ons.os_topk_plan(64, 128256, 8) == 4
    assert ons.os_topk_plan(4096, 128256, 8) == 1
    assert ons.os_topk_plan(16, 1000, 8) == 1
    assert ons.os_topk_plan(64, 32000, 8) == 1
    assert ons.os_topk_plan(16, 1 << 20, 8) == 8
    assert ons.os_topk_plan(128, 65536, 8) == 1    # measured faster unsplit
    assert ons.os_topk_plan(64, 65536, 8) == 1
    assert ons.os_topk_plan(128, 128256, 8) == 1


def test_forward_split_validation(L, ons):
    assert ons.os_softmax_forward_workspace_bytes(10, 1) == 0
    need = ons.os_softmax_forward_workspace_bytes(10, 4)
    assert need == 10 * 4 * 8
    with pytest.raises(ons.OnlineSoftmaxError):
        ons.os_softmax_forward_workspace_bytes(10, 257)
    with pytest.raises(ons.OnlineSoftmaxError):
        ons.os_softmax_forward_workspace_bytes(-1, 2)
    with pytest.raises(ons.OnlineSoftmaxError):
        ons.os_softmax_forward_workspace_bytes(1 << 58, 256)                # size would overflow
    assert L.os_softmax_forward_split(FAKE, FAKE, 1 << 58, 1, F32, 256, FAKE, 1 << 62, None) == EINVAL
    f = L.os_softmax_forward_split
    assert f(FAKE, FAKE, 10, 1000, F32, 0, FAKE, need, None) == EINVAL       # splits < 1
    assert f(FAKE, FAKE, 10, 1000, F32, 257, FAKE, need, None) == EINVAL     # splits > 256
    assert f(FAKE, FAKE, 10, 1000, F32, 4, None, need, None) == EINVAL       # no workspace
    assert f(FAKE, FAKE, 10, 1000, F32, 4, FAKE, need - 1, None) == EINVAL   # short workspace
    assert f(FAKE, FAKE, 10, 1000, F32, 4, FAKE + 4, need, None) == EINVAL   # misaligned workspace
    assert f(FAKE, None, 10, 1000, F32, 4, FAKE, need, None) == EINVAL       # no output
    assert f(FAKE, FAKE, 10, 1000, 5, 4, FAKE, need, None) == EINVAL         # unknown dtype
    assert f(None, None, 0, 1000, F32, 4, None, 0, None) == 0                # empty
    assert ons.os_forward_split_plan(4096, 32000) == 1
    assert ons.os_forward_split_plan(16, 32000) == 1      # register-resident rows are never split
    assert ons.os_forward_split_plan(64, 1000) == 1
    assert ons.os_forward_split_plan(0, 1000) == 1
    assert ons.os_forward_split_plan(16, 1 << 20) == 16   # <= 256 workgroups
    assert ons.os_forward_split_plan(1, 1 << 24) == 256
    assert ons.os_forward_split_plan(1, 1 << 20) == 256   # slices of 1024 vectors
    assert ons.os_forward_split_plan(16, 128256) == 16
    assert ons.os_forward_split_plan(64, 128256) == 4
    assert ons.os_forward_split_plan(256, 128256) == 1


def test_forward_split_noalloc_validation(L, ons):
    """Argument checks of the no-allocation split forward, all before any HIP
    call: the static scratch holds OS_STATIC_SCRATCH_BYTES / 8 slice states."""
    f = L.os_softmax_forward_split_noalloc
    cap = ons.OS_STATIC_SCRATCH_BYTES // 8
    assert ons.OS_STATIC_SCRATCH_BYTES == 1 << 20
    assert f(FAKE, FAKE, cap // 256 + 1, 1 << 20, F32, 256, None) == EINVAL   # beyond the scratch
    assert "static scratch" in ons.os_last_error()
    assert f(FAKE, FAKE, cap // 2 + 1, 1 << 20, F32, 2, None) == EINVAL  # beyond the scratch at 2 splits
    assert f(FAKE, FAKE, 1 << 58, 1, F32, 256, None) == EINVAL
    assert f(FAKE, FAKE, 10, 1000, F32, 0, None) == EINVAL       # splits < 1
    assert f(FAKE, FAKE, 10, 1000, F32, 257, None) == EINVAL     # splits > 256
    assert f(FAKE, None, 10, 1000, F32, 4, None) == EINVAL       # no output
    assert f(None, FAKE, 10, 1000, F32, 4, None) == EINVAL       # no input
    assert f(FAKE, FAKE, 10, 1000, 5, 4, None) == EINVAL         # unknown dtype
    assert f(FAKE + 2, FAKE, 10, 1000, F32, 4, None) == EINVAL   # misaligned input
    assert f(None, None, 0, 1000, F32, 4, None) == 0             # empty
    assert f(None, None, 10, 0, F32, 4, None) == 0               # empty rows


def test_bench_exp_validation(L):
    f = L.os_bench_exp
    assert f(FAKE, 4, 10, 2, None) == EINVAL          # chains 1 or 8
    assert f(FAKE, 0, 10, 8, None) == EINVAL          # no workgroups
    assert f(FAKE, (1 << 20) + 1, 10, 8, None) == EINVAL
    assert f(FAKE, 4, 0, 8, None) == EINVAL           # no rounds
    assert f(None, 4, 10, 8, None) == EINVAL
    assert f(FAKE + 2, 4, 10, 8, None) == EINVAL      # misaligned


def test_read_validation(L):
    f = L.os_device_read
    assert f(FAKE, 20, FAKE, 8192, None) == EINVAL          # not a multiple of 16
    assert f(FAKE + 4, 32, FAKE, 8192, None) == EINVAL      # misaligned source
    assert f(None, 32, FAKE, 8192, None) == EINVAL
    assert f(FAKE, 32, None, 8192, None) == EINVAL
    assert f(FAKE, 1 << 30, FAKE, 8191, None) == EINVAL     # sink too small (2048 workgroups x 4)
    assert f(FAKE, 8192, FAKE, 7, None) == EINVAL           # 2 tiles need 8 floats
    assert f(None, 0, None, 0, None) == 0                   # nothing to read


def test_copy_validation(L):
    assert L.os_device_copy(FAKE, FAKE + 4096, 20, None) == EINVAL      # not a multiple of 16
    assert L.os_device_copy(FAKE + 4, FAKE + 4096, 32, None) == EINVAL  # misaligned
    assert L.os_device_copy(FAKE, FAKE + 16, 64, None) == EINVAL        # overlap
    assert L.os_device_copy(None, None, 0, None) == 0


def test_topk_ex_validation(L, ons):
    f = L.os_softmax_topk_ex
    need = ons.os_softmax_topk_workspace_bytes(10, 8, 4)
    assert f(FAKE, 5, FAKE, FAKE, 10, 1000, 8, 1, None, 0, None) == EINVAL          # unknown dtype
    assert f(FAKE + 1, BF16, FAKE, FAKE, 10, 1000, 8, 1, None, 0, None) == EINVAL   # odd bf16 address
    assert f(FAKE + 2, F32, FAKE, FAKE, 10, 1000, 8, 1, None, 0, None) == EINVAL    # fp32 needs 4 bytes
    assert f(FAKE, BF16, FAKE, FAKE, 10, 1000, 0, 1, None, 0, None) == EINVAL       # K < 1
    assert f(FAKE, BF16, FAKE, FAKE, 10, 4, 8, 1, None, 0, None) == EINVAL          # K > cols
    assert f(FAKE, BF16, FAKE, FAKE, 10, 1000, 8, 4, None, need, None) == EINVAL    # no workspace
    assert f(FAKE, BF16, FAKE, FAKE, 10, 1000, 8, 17, FAKE, need, None) == EINVAL   # splits > 16
    assert f(None, BF16, None, None, 0, 1000, 8, 1, None, 0, None) == 0             # empty


def test_copy_rows_validation(L):
    f = L.os_device_copy_rows
    assert f(FAKE, FAKE + (1 << 20), 4, 20, None) == EINVAL          # row_bytes not a multiple of 16
    assert f(FAKE, FAKE + (1 << 20), 4, 131088, None) == EINVAL      # row longer than 128 KiB
    assert f(None, FAKE, 4, 64, None) == EINVAL                      # NULL
    assert f(FAKE + 8, FAKE + (1 << 20), 4, 64, None) == EINVAL      # misaligned
    assert f(FAKE, FAKE + 64, 4, 64, None) == EINVAL                 # overlap
    assert f(FAKE, FAKE, -1, 64, None) == EINVAL
    assert f(None, None, 0, 64, None) == 0                           # nothing to copy


def test_forward_plan(ons):
    import torch
    assert ons.os_forward_plan(1) == (4, 1)
    assert ons.os_forward_plan(128) == (32, 1)
    assert ons.os_forward_plan(1024) == (128, 2)
    assert ons.os_forward_plan(2048, torch.bfloat16) == (128, 2)
    assert ons.os_forward_plan(4096) == (512, 2)
    assert ons.os_forward_plan(4097) == (256, 5)   # not 16-byte aligned, 1025 slots: 256 lanes of 5 vectors
    assert ons.os_forward_plan(4100) == (512, 4)
    assert ons.os_forward_plan(2052) == (256, 4)
    # every automatic shape holds its row, and a row that is not 16-byte
    # aligned (row bytes not a multiple of 16) gets room for one more block,
    # unless a multi-row shape (<= 64 lanes per row) reads it through LDS,
    # where its length alone counts
    for cols in range(1, 70000, 97):
        for dt, vec in ((torch.float32, 4), (torch.bfloat16, 8)):
            lanes, vecs = ons.os_forward_plan(cols, dt)
            extra = 0 if cols % vec == 0 else vec - 1
            assert lanes == 0 or lanes * vecs * vec >= cols + extra or (lanes <= 64 and lanes * vecs * vec >= cols)
    assert ons.os_forward_plan(127) == (8, 4)    # 33 blocks, but read through LDS: 32 slots of its own
    assert ons.os_forward_plan(129) == (16, 4)    # 33 blocks, through LDS
    assert ons.os_forward_plan(124) == (32, 1)
    assert ons.os_forward_plan(127, torch.bfloat16) == (8, 2)    # 16 slots of its own, 17 spanned
    assert ons.os_forward_plan(15) == (4, 1)     # 4 slots of its own, 5 spanned
    assert ons.os_forward_plan(4095, torch.bfloat16) == (128, 8)   # 513 spanned: no large shape through LDS
    assert ons.os_forward_plan(1001, torch.bfloat16) == (64, 2)   # the same shape either way: direct loads
    assert ons.os_forward_plan(1023) == (64, 8)    # 257 blocks; the aligned plan's 128 x 2 is one-row
    assert ons.os_forward_plan(17) == (4, 2)       # short unaligned fp32 rows: small shapes, read through LDS
    assert ons.os_forward_plan(33) == (4, 4)
    assert ons.os_forward_plan(61) == (8, 2)
    assert ons.os_forward_plan(65) == (8, 4)
    assert ons.os_forward_plan(65, torch.bfloat16) == (4, 4)   # 9 blocks, direct loads
    # one-row shapes keep 8 blocks spare for unaligned rows: 16381 fp32
    # columns span 4096 blocks, exactly what 1024 x 4 holds
    assert ons.os_forward_plan(16349) == (1024, 4)   # 4088 blocks
    assert ons.os_forward_plan(16381) == (1024, 5)
    assert ons.os_forward_plan(16384) == (1024, 6)  # aligned fp32 rows past 4088 slots too
    assert ons.os_forward_plan(16384, torch.bfloat16) == (512, 5)
    assert ons.os_forward_plan(32000) == (1024, 8)
    assert ons.os_forward_plan(32768) == (1024, 8)
    assert ons.os_forward_plan(32769) == (0, 0)    # the hybrid: registers and LDS
    assert ons.os_forward_plan(65536) == (0, 0)
    assert ons.os_forward_plan(65537) == (0, 0)
    assert ons.os_forward_plan(65536, torch.bfloat16) == (1024, 8)
    assert ons.os_forward_plan(65537, torch.bfloat16) == (0, 0)
    with pytest.raises(ons.OnlineSoftmaxError):
        ons.os_forward_plan(-5)


def test_binding_rejects_host_tensors(ons):
    import torch
    with pytest.raises(ValueError):
        ons.os_softmax_forward(torch.zeros(4, 4))


def test_single_hip_runtime(ons):
    assert len(ons._hip_runtimes_mapped()) <= 1


def test_error_message_is_thread_local(L, ons):
    import threading
    assert L.os_softmax_forward(None, FAKE, 4, 4, F32, None) == EINVAL
    seen = []
    t = threading.Thread(target=lambda: seen.append(ons.os_last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert "NULL" in ons.os_last_error()


def test_build_scripts_load_without_the_package():
    """__graft_entry__.build() must work on a fresh checkout, before any library
    exists: its build scripts load by path, without importing the packages
    whose __init__ needs the library."""
    import subprocess
    import sys
    code = (
        "import os, sys, __graft_entry__ as g\n"
        "h = g._script(os.path.join(g.ROOT, 'online_normalizer_amd', 'build.py'), '_h')\n"
        "o = g._script(os.path.join(g.ROOT, 'oracle', 'build.py'), '_o')\n"
        "assert callable(h.build) and callable(o.build)\n"
        "assert 'online_normalizer_amd' not in sys.modules and 'oracle' not in sys.modules\n"
        "print('ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr
