"""The public header compiles as C and as C++, and a C program links
against libvattn.so and runs its host-only paths (no GPU touched): status
strings, empty shapes and synchronous argument errors."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(ROOT, "non_causal_flash_amd")
HIP_LIB_DIR = "/opt/rocm/lib"

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "vattn.h"

int main(void) {
    float *q = 0, *k = 0, *v = 0, *out = 0;
    float table[8];
    float factors[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    int fails = 0;
    /* every code has a static description */
    for (int s = VATTN_OK; s <= VATTN_ERR_ROPE; ++s)
        if (vattn_status_string(s) == 0 || strlen(vattn_status_string(s)) == 0) ++fails;
    /* empty shapes are no-ops, whatever the pointers */
    if (vattn_forward(q, k, v, out, 0, 64, 64, 0) != VATTN_OK) ++fails;
    if (vattn_forward_precision(q, k, v, out, 4, 0, 64, VATTN_PRECISION_SPLIT, 0) != VATTN_OK)
        ++fails;
    if (vattn_forward_strided(q, k, v, out, 0, 10, 40, 400, 40, VATTN_PRECISION_AUTO, 0)
        != VATTN_OK) ++fails;
    if (vattn_forward_f16(q, k, v, out, 0, 10, 40, 400, 40, VATTN_PRECISION_FAST, 0)
        != VATTN_OK) ++fails;
    if (vattn_forward_rope(q, k, v, out, 0, 10, 64, 640, 64, 64, table,
                           VATTN_PRECISION_AUTO, 0) != VATTN_OK) ++fails;
    if (vattn_forward_rope_f16(q, k, v, out, 0, 10, 64, 640, 64, 64, table,
                               VATTN_PRECISION_AUTO, 0) != VATTN_OK) ++fails;
    if (vattn_rope_table(table, 0, 8, 10000.0f, factors, 0, 0) != VATTN_OK) ++fails;
    /* argument errors, reported before any launch */
    if (vattn_forward(q, k, v, out, 4, 64, 64, 0) != VATTN_ERR_NULL) ++fails;
    if (vattn_forward(q, k, v, out, 4, 64, 65, 0) != VATTN_ERR_HEAD_DIM) ++fails;
    if (vattn_forward(q, k, v, out, -1, 64, 64, 0) != VATTN_ERR_SIZE) ++fails;
    if (vattn_forward_precision(q, k, v, out, 4, 64, 64, 9, 0) != VATTN_ERR_ARG) ++fails;
    if (vattn_rope_table(table, 4, 7, 10000.0f, 0, 0, 0) != VATTN_ERR_ROPE) ++fails;
    printf("fails %d last_hip_error %d\n", fails, vattn_last_hip_error());
    return fails != 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip("%s not available" % name)
    return path


def test_header_compiles_as_c99_and_cxx17(tmp_path):
    src = tmp_path / "use.c"
    src.write_text(PROGRAM)
    for cc, std in ((_compiler("gcc"), "-std=c99"), (_compiler("g++"), "-std=c++17")):
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror",
                            "-x", "c" if std == "-std=c99" else "c++", "-I", INCLUDE,
                            "-c", str(src), "-o", str(tmp_path / "use.o")],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr


def test_c_program_links_and_runs_host_paths(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libvattn.so")):
        pytest.skip("libvattn.so not built")
    src = tmp_path / "use.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use"
    r = subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-I", INCLUDE, str(src),
                        "-L", LIB_DIR, "-lvattn", "-Wl,-rpath," + LIB_DIR,
                        "-Wl,-rpath," + HIP_LIB_DIR, "-o", str(exe)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "fails 0" in run.stdout
