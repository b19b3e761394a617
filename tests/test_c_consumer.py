"""The boundary is a C ABI: a C99 program compiles against include/batq.h and
include/batq_probe.h with gcc (-Wall -Wextra -Werror), links libbatq.so, and
calls the host helpers and the argument checks that return before any HIP call.
CPU only; no device work is launched."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

PKG = os.path.join(ROOT, "w4a4_bit_gemm_amd")

PROGRAM = r"""
#include "batq.h"
#include "batq_probe.h"
#include <math.h>
#include <stdio.h>
#include <string.h>

#define CHECK(c) do { if (!(c)) { printf("failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
  CHECK(batq_abi_version() == BATQ_ABI_VERSION);
  CHECK(strcmp(batq_status_str(BATQ_OK), "unknown status") != 0);

  /* clip ratios: sigmoid in double, rounded once to float */
  const float logits[4] = {0.0f, 3.0f, -2.5f, 10.0f};
  float r[4];
  CHECK(batq_clip_ratios(logits, r, 4) == BATQ_OK);
  for (int i = 0; i < 4; ++i) CHECK(r[i] == (float)(1.0 / (1.0 + exp(-(double)logits[i]))));
  CHECK(batq_clip_ratios(NULL, r, 4) == BATQ_ERR_NULL);
  CHECK(batq_clip_ratios(logits, r, -1) == BATQ_ERR_SHAPE);

  /* inverse-transposed factors: (2 I)^-T = I / 2, (4 I)^-T = I / 4, exact */
  float A[64] = {0}, B[2 * 16] = {0}, Ai[64], Bi[2 * 16];
  for (int i = 0; i < 8; ++i) A[9 * i] = 2.0f;
  for (int k = 0; k < 2; ++k)
    for (int i = 0; i < 4; ++i) B[16 * k + 5 * i] = 4.0f;
  CHECK(batq_gpk_invert(8, 4, 2, A, B, Ai, Bi) == BATQ_OK);
  for (int i = 0; i < 64; ++i) CHECK(Ai[i] == (i % 9 == 0 ? 0.5f : 0.0f));
  for (int i = 0; i < 32; ++i) CHECK(Bi[i] == ((i % 16) % 5 == 0 ? 0.25f : 0.0f));
  float Z[64] = {0};
  CHECK(batq_gpk_invert(8, 4, 2, Z, B, Ai, Bi) == BATQ_ERR_SINGULAR);
  CHECK(batq_gpk_invert(8, 8, 2, A, B, Ai, Bi) == BATQ_ERR_SHAPE);

  /* size queries */
  CHECK(batq_weight_packed_bytes(4096, 4096) == (4096 / 32) * (4096 / 256) * (4 * 64 * 16 + 64 * 4));
  CHECK(batq_packed_gemm_kernel(16384, 4096, 4096, 0) == 1);
  CHECK(batq_packed_gemm_kernel(2048, 4096, 12288, 0) == 0);
  CHECK(batq_decode_workspace_bytes(16, 4096, 4096) > 0);

  /* argument checks return before any HIP call; an empty batch is a no-op */
  void* fake = (void*)(uintptr_t)0x10000;
  CHECK(batq_act_transform_quant(NULL, 64, 256, 256, 8, 4, (const float*)fake, (const float*)fake, NULL, NULL,
                                 (uint8_t*)fake, (uint8_t*)fake, 0) == BATQ_ERR_NULL);
  CHECK(batq_act_transform_quant(fake, 64, 250, 256, 8, 4, (const float*)fake, (const float*)fake, NULL, NULL,
                                 (uint8_t*)fake, (uint8_t*)fake, 0) == BATQ_ERR_SHAPE);
  CHECK(batq_act_transform_quant(fake, 64, 256, 256, 8, 4, (const float*)fake, (const float*)fake,
                                 (const float*)fake, NULL, (uint8_t*)fake, (uint8_t*)fake, 0) == BATQ_ERR_NULL);
  CHECK(batq_act_transform_quant(fake, 0, 256, 256, 8, 4, (const float*)fake, (const float*)fake, NULL, NULL,
                                 (uint8_t*)fake, (uint8_t*)fake, 0) == BATQ_OK);
  CHECK(batq_mxfp4_gemm(NULL, fake, fake, fake, 16, 16, 64, fake, BATQ_OUT_BF16, 0) == BATQ_ERR_NULL);
  CHECK(batq_probe_stream_granule() > 0);
  printf("ok\n");
  return 0;
}
"""


def test_c_program_compiles_links_and_calls_the_abi(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = os.path.join(PKG, "libbatq.so")
    assert os.path.exists(lib), "libbatq.so is not built"
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
           "-L", PKG, "-lbatq", f"-Wl,-rpath,{PKG}", "-lm", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
