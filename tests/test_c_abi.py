"""include/qsa.h is plain C: a C99 program that includes it compiles with gcc, links against
libqsa.so and calls the host-side entry points (status strings, workspace sizes, argument
checks that fail before any device call), without Python or torch in the way."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_decode_qsa_amd")

PROGRAM = r"""
#include <stdio.h>
#include "qsa.h"

int main(void) {
  /* every status code has a string */
  for (int s = 0; s <= 6; ++s) printf("%d %s\n", s, qsa_status_string((qsa_status_t)s));
  /* workspace sizes are host arithmetic */
  size_t ws = qsa_decode_workspace_size(4, 32, 4, 65536, 512, 4);
  size_t wm = qsa_decode_multi_workspace_size(4, 1, 32, 4, 65536, 512, 4);
  printf("ws %zu %zu\n", ws, wm);
  /* checks that fail on the host return their code and launch nothing */
  int8_t* fake = (int8_t*)0x1000;
  qsa_status_t st = qsa_index_score(fake, fake, (const int32_t*)fake, (const int32_t*)fake, 2, 4, 64, 32, 16, 256,
                                    (int32_t*)fake, NULL, NULL);
  printf("page_size_32 %d\n", (int)st);
  st = qsa_decode_noalloc(fake, fake, fake, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 4096, 32, 4,
                          128, 4, 64, 64, 4096, 65536, 512, 4, 0.088f, (int32_t*)fake, (int32_t*)fake,
                          (int32_t*)fake, (float*)fake, (float*)fake, (float*)fake, NULL, NULL);
  printf("noalloc_too_big %d\n", (int)st);
  printf("version %d\n", qsa_version());
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_header_is_c99_and_library_links_from_c(tmp_path):
    lib = os.path.join(PKG, "libqsa.so")
    if not os.path.exists(lib):
        pytest.skip("libqsa.so not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", PKG, "-lqsa", f"-Wl,-rpath,{PKG}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert out["0"] == "ok" and "unknown" not in " ".join(out[str(s)] for s in range(7))
    ws, wm = map(int, out["ws"].split())
    assert ws == wm > 0
    assert out["page_size_32"] == "3"            # QSA_ERR_UNSUPPORTED
    assert out["noalloc_too_big"] == "6"         # QSA_ERR_SCRATCH
    assert int(out["version"]) >= 200
