"""The header is plain C: a C11 program that includes only include/gdr.h,
built with gcc -std=c11 -pedantic -Wall -Wextra -Werror and linked against
libgdr.so, calls the library the way a C caller would.  Only calls that need
no GPU run here: the version and status strings, the workspace query, and
entry points that fail validation before any HIP call."""
import os
import shutil
import subprocess

import pytest

import gated_deltanet_chunked_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "gdr.h"
#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("failed: %s\n", #c); ++fails; } } while (0)

int main(void) {
  CHECK(strncmp(gdr_version(), "libgdr", 6) == 0);
  CHECK(strcmp(gdr_status_string(GDR_OK), gdr_status_string(GDR_ERR_INVALID_ARGUMENT)) != 0);
  size_t ws = gdr_chunk_fwd_workspace_size(4096, 1, 16, 32, 128, GDR_BF16);
  CHECK(ws > 0);
  CHECK(gdr_chunk_fwd_workspace_size(4096, 1, 16, 32, 64, GDR_BF16) == 0);
  /* no inputs at all: refused before any launch */
  gdr_status s = gdr_chunk_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 4096, 16, 32, 128,
                               GDR_BF16, 0.08838834764831845f, GDR_FLAG_QK_L2NORM, NULL, NULL,
                               NULL, 0, NULL);
  CHECK(s == GDR_ERR_INVALID_ARGUMENT);
  s = gdr_recurrent_step(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 256, 16, 32, 128, GDR_BF16,
                         0.08838834764831845f, GDR_FLAG_QK_L2NORM, NULL, NULL);
  CHECK(s == GDR_ERR_INVALID_ARGUMENT);
  printf("%s\n", fails ? "FAIL" : "OK");
  return fails != 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    libdir = os.path.dirname(gdr.load()._name)
    src = tmp_path / "caller.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "caller"
    cmd = ["gcc", "-std=c11", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-lgdr", "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
