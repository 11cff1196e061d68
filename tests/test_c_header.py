"""The C ABI from C: include/online_softmax.h compiles as C99 (and C++17) with
every warning as an error, and a C program linked against the library calls
the entry points that need no GPU: the version, the plans and workspace sizes,
the empty-problem no-ops, and argument errors with their messages.  No kernel
is launched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "online_normalizer_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "online_softmax.h"

#define CHECK(c) do { if (!(c)) { printf("failed: %s (line %d): %s\n", #c, __LINE__, os_last_error()); return 1; } } while (0)

int main(void) {
    int lanes = 0, vecs = 0;
    float buf[4];
    CHECK(os_version() > 0);
    /* plans and sizes */
    CHECK(os_forward_plan(32000, OS_F32, &lanes, &vecs) == OS_OK && lanes > 0 && vecs > 0);
    CHECK(os_forward_split_plan(1, 1 << 24, OS_F32) == 256);
    CHECK(os_topk_plan(16, 128256, 8) > 1 && os_topk_plan(256, 128256, 8) == 1);
    CHECK(os_softmax_topk_workspace_bytes(16, 8, 4) > 0 && os_softmax_topk_workspace_bytes(16, 8, 1) == 0);
    CHECK(os_softmax_forward_workspace_bytes(16, 8) > 0);
    CHECK(os_softmax_topk_workspace_bytes(16, OS_TOPK_KMAX + 1, 1) == OS_EINVAL);
    /* empty problems are no-ops, even with NULL pointers */
    CHECK(os_softmax_forward(NULL, NULL, 0, 4, OS_F32, NULL) == OS_OK);
    CHECK(safe_softmax_forward(NULL, NULL, 4, 0, OS_BF16, NULL) == OS_OK);
    CHECK(os_attention_forward(NULL, NULL, NULL, NULL, NULL, 0, 16, 16, 128, 0.1f, 0, NULL) == OS_OK);
    /* argument errors, found before any HIP call, with a message */
    CHECK(os_softmax_forward(NULL, buf, 4, 4, OS_F32, NULL) == OS_EINVAL && strlen(os_last_error()) > 0);
    CHECK(os_softmax_forward(buf, buf, 4, 4, 7, NULL) == OS_EINVAL);
    CHECK(os_softmax_forward(buf, buf, 4, OS_MAX_COLS + 1, OS_F32, NULL) == OS_EINVAL);
    CHECK(os_softmax_topk(buf, buf, (int32_t *)buf, 1, 4, 0, NULL) == OS_EINVAL);
    CHECK(os_softmax_forward_split_noalloc(buf, buf, 1 << 20, 64, OS_F32, 16, NULL) == OS_EINVAL);
    CHECK(os_attention_forward(buf, buf, buf, buf, NULL, 1, 4, 4, 64, 0.1f, 0, NULL) == OS_EINVAL);
    CHECK(os_attention_forward(buf, buf, buf, buf, NULL, 1, 4, 5, 128, 0.1f, 1, NULL) == OS_EINVAL);
    printf("ok\n");
    return 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


def test_header_compiles_as_c_and_cxx(tmp_path):
    cc, cxx = _compiler("gcc"), _compiler("g++")
    src = tmp_path / "inc.c"
    src.write_text('#include "online_softmax.h"\nint probe(void) { return OS_OK; }\n')
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INCLUDE, "-c", str(src), "-o",
                    str(tmp_path / "c.o")], check=True)
    srcx = tmp_path / "inc.cpp"
    srcx.write_text('#include "online_softmax.h"\nint probe() { return OS_OK; }\n')
    subprocess.run([cxx, "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INCLUDE, "-c", str(srcx),
                    "-o", str(tmp_path / "cxx.o")], check=True)


def test_c_program_calls_the_library(tmp_path):
    cc = _compiler("gcc")
    if not os.path.exists(os.path.join(LIBDIR, "libonline_softmax.so")):
        pytest.skip("library not built")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE, str(src), "-L", LIBDIR,
                    "-lonline_softmax", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
