"""The boundary from plain C (no Python, no ctypes): a C99 program that includes
include/psa.h and links libpsa.so compiles warning-free and gets the documented status
codes and error messages from argument validation, which runs before any HIP call (so no
GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "vision_transformer_attention_psapackqkv_amd")

C_SRC = r'''
#include <stdio.h>
#include <string.h>
#include "psa.h"

int main(void) {
  if (psa_abi_version() != PSA_ABI_VERSION) { printf("version %d\n", psa_abi_version()); return 1; }
  static char buf[256] __attribute__((aligned(16)));
  psa_status s = psa_pack_qkv(NULL, buf, 1, 1, 16, 8, 8, PSA_BF16, NULL);
  if (s != PSA_ERR_NULL || !strstr(psa_last_error(), "psa_pack_qkv")) { printf("null: %d %s\n", s, psa_last_error()); return 2; }
  s = fa2_fwd(buf, buf + 64, buf + 128, buf + 192, NULL, 1, 1, 1, 24, 0.5f, PSA_BF16, NULL, 0, NULL);
  if (s != PSA_ERR_UNSUPPORTED || !strstr(psa_last_error(), "head_dim")) { printf("dim: %d %s\n", s, psa_last_error()); return 3; }
  s = psa_merge_attn(buf, buf + 8, 1, 1, 16, 1, 1, PSA_F32, NULL);
  if (s != PSA_ERR_ALIGN) { printf("align: %d %s\n", s, psa_last_error()); return 4; }
  s = psa_extract_v(buf, buf + 16, 1, 1, 16, 1, 1, (psa_dtype)7, NULL);
  if (s != PSA_ERR_UNSUPPORTED) { printf("dtype: %d %s\n", s, psa_last_error()); return 5; }
  printf("ok\n");
  return 0;
}
'''


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(PKG, "libpsa.so")
    if not os.path.exists(lib):
        pytest.skip("libpsa.so not built")
    src = tmp_path / "consumer.c"
    src.write_text(C_SRC)
    exe = tmp_path / "consumer"
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                         str(src), "-L", PKG, "-lpsa", f"-Wl,-rpath,{PKG}", "-o", str(exe)],
                        capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
