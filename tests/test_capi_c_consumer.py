"""The boundary as a C program sees it (no GPU needed): include/bgt.h compiles
as C99, a C program links libbgt.so, and calls that validate before any HIP
call return the documented status codes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "bit_gemm_token_amd")

SRC = r"""
#include <stdio.h>
#include <string.h>
#include "bgt.h"

int main(void) {
  int fails = 0;
  int a = 0;
  void* fake = (void*)0x10000;
  if (bgt_abi_version() < 105) { puts("abi"); ++fails; }
  if (bgt_w4a8_gemm_is(NULL, fake, fake, fake, 1024, 16, 64, 256, fake, NULL, NULL) != BGT_ERR_NULL) { puts("null"); ++fails; }
  if (bgt_w4a8_gemm_is(fake, fake, fake, fake, 1000, 16, 64, 256, fake, NULL, NULL) != BGT_ERR_ALPHA) { puts("alpha"); ++fails; }
  if (bgt_w8a8_gemm_is(fake, fake, fake, fake, 3, 1024, 16, 64, 256, fake, BGT_F32, NULL, NULL) != BGT_ERR_MODE) { puts("width"); ++fails; }
  if (bgt_pack_weights_int8(fake, 200, 32, 128, 0, fake, fake, fake, &a, NULL) != BGT_ERR_SHAPE) { puts("shape"); ++fails; }
  if (bgt_w4a8_moe_gemm_is(fake, fake, 16, fake, fake, 0, 32, fake, fake, 4, 1024, 64, 256, fake, BGT_F32, NULL, NULL) != BGT_ERR_SHAPE) { puts("experts"); ++fails; }
  if (strcmp(bgt_status_string(BGT_OK), "ok") != 0) { puts("status"); ++fails; }
  if (strcmp(bgt_w4a8_kernel_name(1, 22016, 4096, 0), "k_w4a8_decode<IS>") != 0) { puts("name"); ++fails; }
  printf("%d failures\n", fails);
  return fails;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_links_and_validates(tmp_path):
    lib = os.path.join(LIBDIR, "libbgt.so")
    if not os.path.exists(lib):
        pytest.skip("libbgt.so not built")
    src = tmp_path / "consumer.c"
    src.write_text(SRC)
    exe = tmp_path / "consumer"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-L", LIBDIR, "-lbgt", "-Wl,-rpath," + LIBDIR, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
