"""The public headers are plain C: a C11 program that includes them, links
against liblongflow.so and calls the entry points that need no GPU (sizing,
status strings, argument checks) compiles with gcc -std=c11 -pedantic and runs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "decode_kv_cache_02_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "longflow.h"
#include "longflow_probe.h"

int main(void) {
  lf_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.num_layers = 32; cfg.batch = 64; cfg.num_q_heads = 32; cfg.num_kv_heads = 8;
  cfg.head_dim = 128; cfg.budget = 3277; cfg.dtype = LF_DTYPE_BF16; cfg.mode = LF_MODE_EVICT;
  size_t bytes = 0;
  if (lf_cache_bytes(&cfg, &bytes) != LF_OK) return 1;
  /* K and V of 32 layers x 512 pairs x 3328 slots x 128 x 2 bytes, plus sidecars */
  if (bytes < (size_t)32 * 512 * 3328 * 128 * 2 * 2) return 2;
  cfg.order = LF_ORDER_DEFERRED; cfg.scope = LF_SCOPE_SEQUENCE; cfg.norm = LF_NORM_L2;
  size_t bytes2 = 0;
  if (lf_cache_bytes(&cfg, &bytes2) != LF_OK || bytes2 <= bytes) return 3;
  cfg.head_dim = 96;
  if (lf_cache_bytes(&cfg, &bytes) != LF_ERR_UNSUPPORTED) return 4;
  if (strcmp(lf_status_str(LF_ERR_CAPACITY), "LF_ERR_CAPACITY") != 0) return 5;
  if (lf_decode_step(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL) != LF_ERR_INVALID_ARG) return 6;
  if (lf_probe_stream_read(NULL, 16, 1, NULL, NULL) != LF_ERR_INVALID_ARG) return 7;
  if (lf_decode_step_noalloc(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL) != LF_ERR_INVALID_ARG) return 8;
  if (lf_probe_hbm_attributes(NULL, NULL) != LF_ERR_INVALID_ARG) return 9;
  if (lf_probe_stream_read_timing(NULL, 16, 1, NULL, NULL, NULL) != LF_ERR_INVALID_ARG) return 10;
  if (lf_probe_decode_timing(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL) != LF_ERR_INVALID_ARG) return 11;
  lf_cache_destroy(NULL);
  printf("ok %zu\n", bytes2);
  return 0;
}
"""


def test_headers_compile_as_c_and_link(tmp_path):
    lib = os.path.join(LIB_DIR, "liblongflow.so")
    if not os.path.exists(lib):
        pytest.skip("liblongflow.so not built")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", LIB_DIR, "-llongflow", f"-Wl,-rpath,{LIB_DIR}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.startswith("ok ")
