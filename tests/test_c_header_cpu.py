"""The boundary as a C program sees it: include/gdn.h compiles as strict C99
and as C++, and a C program linked against libgdn.so gets the documented
sizes and status codes from the host-side calls (every call below is either
pure host computation or fails validation, so no GPU is needed)."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest

from gated_deltanet_linear_04_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

PROGRAM = r"""
#include "gdn.h"
#include <stdio.h>
#include <string.h>

#define CHECK(cond, code) do { if (!(cond)) { printf("fail %d\n", code); return code; } } while (0)

int main(void) {
  gdn_desc d;
  gdn_layer_desc ld;
  size_t ws, lws;
  float probe_out[256];
  CHECK(gdn_desc_init(&d, 1, 2048, 16, 32, 128, 128, GDN_BF16) == GDN_OK, 1);
  CHECK(d.hq == 16 && d.hk == 16 && d.hv == 32 && d.dk == 128 && d.dv == 128, 2);
  ws = gdn_prefill_workspace_size(&d);
  CHECK(ws > 0 && ws % 256 == 0, 3);
  CHECK(gdn_prefill_workspace_size(NULL) == 0, 4);
  /* invalid calls return a status and launch nothing */
  CHECK(gdn_prefill(NULL, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == GDN_ERR_INVALID, 5);
  CHECK(strlen(gdn_last_error()) > 0, 6);
  CHECK(gdn_prefill(&d, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == GDN_ERR_INVALID, 7);
  CHECK(gdn_decode(NULL, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 0) == GDN_ERR_INVALID, 8);
  d.dk = 64;
  CHECK(gdn_prefill_workspace_size(&d) == 0, 9);
  CHECK(gdn_layer_desc_init(&ld, 1, 2048, 2560, 16, 32, 4) == GDN_OK, 10);
  lws = gdn_layer_workspace_size(&ld);
  CHECK(lws > ws, 11);
  CHECK(gdn_layer_prefill(&ld, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == GDN_ERR_INVALID, 12);
  CHECK(gdn_gemm_bf16(16, 16, 33, 0, 33, 0, 33, 0, 16, 0) != GDN_OK, 13);
  CHECK(gdn_conv_silu_bf16(4, 12, 4, 0, 12, 0, 0, 0, 1, 0, 0, 0) != GDN_OK, 14);
  CHECK(gdn_mfma_probe(0, 1, probe_out, 0) == GDN_ERR_INVALID, 15);
  CHECK(strcmp(gdn_status_string(GDN_ERR_WORKSPACE), gdn_status_string(GDN_OK)) != 0, 16);
  CHECK(gdn_version() >= 100, 17);
  CHECK(d.short_tokens == 8, 18);
  printf("ok %zu %zu %zu\n", ws, lws, sizeof(gdn_desc));
  return 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip("%s not available" % name)
    return path


@pytest.fixture(scope="module")
def libdir():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return os.path.dirname(B.LIB_PATH)


def test_header_compiles_as_strict_c99_and_cxx(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "gdn.h"\nint main(void) { return (int)sizeof(gdn_desc) > 0 ? 0 : 1; }\n')
    subprocess.run([_compiler("gcc"), "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-fsyntax-only", "-I", INCLUDE, str(src)], check=True)
    srcxx = tmp_path / "h.cc"
    srcxx.write_text('#include "gdn.h"\nint main() { gdn_desc d{}; return d.num_seqs; }\n')
    subprocess.run([_compiler("g++"), "-std=c++17", "-Wall", "-Wextra", "-Werror",
                    "-fsyntax-only", "-I", INCLUDE, str(srcxx)], check=True)


def test_c_program_against_the_library(tmp_path, libdir):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-Werror", "-I", INCLUDE, str(src),
                    "-o", str(exe), "-L", libdir, "-lgdn", "-Wl,-rpath," + libdir], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("ok ")
    ws, lws, dsz = (int(x) for x in r.stdout.split()[1:4])
    # the binding's mirror of the descriptor has the C layout's size
    assert dsz == ctypes.sizeof(B.GdnDesc)
    assert ws == B.workspace_size(B.make_desc(1, 2048, 16, 32, B.GDN_BF16))
    assert lws == B.layer_workspace_size(B.make_layer_desc(1, 2048, 2560, 16, 32, 4))
