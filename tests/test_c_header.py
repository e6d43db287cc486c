"""include/sa.h is a plain C header: a C99 program compiled with gcc
(-Wall -Werror -pedantic) against it and linked with libsa.so builds graphs,
exports rows and gets every validation status back on a host without a GPU
(no compute call reaches the device)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_causal_attention_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "sa.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAIL line %d\n", __LINE__); return 1; } } while (0)

int main(void) {
  sa_graph* g = NULL;
  const int64_t offs[4] = {8, 2, 8, 100};
  int64_t T = 0, W = 0, E = 0, dil[SA_MAX_DILATED];
  int32_t nd = 0, kind = -1;
  int64_t rp[6], cols[64];
  size_t bytes = 1;
  char buf[128];
  sa_attn_desc d;

  CHECK(sa_build_graph(16, 3, offs, 4, &g) == SA_OK);
  CHECK(sa_graph_info(g, &T, &W, &nd, dil, &E) == SA_OK);
  CHECK(T == 16 && W == 3 && nd == 1 && dil[0] == 8);
  CHECK(E == 3 * 4 / 2 + 3 * 13 + 8);  /* W'(W'+1)/2 + W'(T-W') + (T - 8) */
  CHECK(sa_graph_kind(g, &kind) == SA_OK && kind == SA_GRAPH_DISTANCE);
  CHECK(sa_graph_device_bytes(g, &bytes) == SA_OK && bytes == 0);
  /* rows 8..12: row 8 lists 0, 6, 7, 8 */
  CHECK(sa_graph_rows(g, 8, 13, rp, cols, 64) == SA_OK);
  CHECK(rp[0] == 0 && rp[1] == 4 && cols[0] == 0 && cols[1] == 6 && cols[3] == 8);
  CHECK(sa_graph_rows(g, 8, 13, rp, cols, 3) == SA_ERR_INVALID_ARG && rp[5] == 20);

  memset(&d, 0, sizeof d);
  d.B = 1; d.H = 2; d.T = 16; d.D = 48; d.dtype = SA_BF16; d.grad_dtype = SA_F32;
  CHECK(sa_describe_plan(g, &d, 0, buf, sizeof buf) == SA_ERR_UNSUPPORTED);  /* D = 48 */
  d.D = 64; d.T = 17;
  CHECK(sa_describe_plan(g, &d, 0, buf, sizeof buf) == SA_ERR_SHAPE_MISMATCH);
  d.T = 16;
  CHECK(sa_describe_plan(g, &d, 0, buf, sizeof buf) == SA_OK && strncmp(buf, "gather", 6) == 0);
  CHECK(sa_fwd(g, &d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == SA_ERR_INVALID_ARG);
  CHECK(sa_bwd_workspace_size(g, &d, &bytes) == SA_OK && bytes > 0);
  sa_graph_free(g);

  {  /* explicit lists: 3 rows, reverse lists formed by the library */
    const int64_t lrp[4] = {0, 1, 3, 5}, lcols[5] = {0, 0, 1, 0, 2};
    int64_t rrp[4], rcols[5];
    CHECK(sa_build_graph_csr(3, lrp, lcols, &g) == SA_OK);
    CHECK(sa_graph_kind(g, &kind) == SA_OK && kind == SA_GRAPH_CSR);
    CHECK(sa_graph_rows_reverse(g, 0, 3, rrp, rcols, 5) == SA_OK);
    CHECK(rrp[1] == 3 && rcols[0] == 0 && rcols[1] == 1 && rcols[2] == 2 && rcols[3] == 1 && rcols[4] == 2);
    CHECK(sa_graph_device_bytes(g, &bytes) == SA_OK && bytes == 2 * (256 + 256));
    CHECK(sa_graph_upload(g, NULL, bytes, NULL) == SA_ERR_INVALID_ARG);
    sa_graph_free(g);
  }
  CHECK(strcmp(sa_status_str(SA_OK), "ok") == 0);
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_against_the_header(tmp_path):
    lib = os.path.join(LIBDIR, "libsa.so")
    if not os.path.exists(lib):
        pytest.skip("libsa.so is not built")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", LIBDIR, "-lsa", "-Wl,-rpath," + LIBDIR], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
