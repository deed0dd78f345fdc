"""The C ABI from C itself (no GPU needed): a C99 program that includes
include/wide.h, links libwide.so and calls the host-only paths (status strings,
workspace queries, argument checks that return before anything is enqueued)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "sparse_wide_mask_amd")

PROG = r"""
#include <stdio.h>
#include <string.h>
#include "wide.h"

int main(void) {
  wide_layer_cfg cfg = {4096, 14336, 112, {32, 8, 128, 500000.0f}, 1e-5f};
  size_t ws = wide_layer_masked_workspace(8192, &cfg, WIDE_PREFILL, 0);
  size_t bad = wide_layer_masked_workspace(8192, &cfg, 7, 0);
  int st = wide_ffn_masked(NULL, NULL, NULL, NULL, NULL, 8, 256, 1024, 16, WIDE_PREFILL, NULL,
                           NULL, 0, 0, NULL);
  int noop = wide_ffn_masked(NULL, NULL, NULL, NULL, NULL, 0, 256, 1024, 16, WIDE_PREFILL, NULL,
                             NULL, 0, 0, NULL);
  int f32 = wide_ffn_masked_f32(NULL, NULL, NULL, NULL, NULL, 8, 256, 1000, 16, NULL, NULL, 0, 0,
                                NULL);
  printf("%zu %zu %d %d %d %s\n", ws, bad, st, noop, f32, wide_status_string(WIDE_EWORKSPACE));
  return 0;
}
"""


def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(LIB_DIR, "libwide.so")
    if not os.path.exists(lib):
        pytest.skip("libwide.so not built")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_wide.c"
    exe = tmp_path / "use_wide"
    src.write_text(PROG)
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), lib, f"-Wl,-rpath,{LIB_DIR}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    ws, bad, st, noop, f32 = (int(x) for x in out[:5])
    assert ws > 8192 * 4096 * 2          # at least the normalised activations
    assert bad == 0                      # invalid mode: no workspace size
    assert st == 1 and f32 == 1          # WIDE_EINVAL: NULL pointers / d_ff % n != 0
    assert noop == 0                     # T == 0 is a no-op
    assert " ".join(out[5:]) == "workspace too small"
