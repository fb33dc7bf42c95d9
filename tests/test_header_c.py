"""The C ABI from C: include/hc_mi355x.h compiles on its own as C99 and as C++11 (strict
warnings, no HIP headers needed), and a plain C program links against the built library and
gets the documented answers from its size queries, status strings and argument checks (no
call reaches a kernel, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

from hyper_connection_residual_hc_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc_mi355x.h")

C_PROGRAM = r"""
#include <stdio.h>
#include "hc_mi355x.h"

int main(void) {
  int fake = 0;
  printf("%d\n", hc_abi_version());
  printf("%s %s\n", hc_status_string(HC_OK), hc_status_string(HC_ERR_SHAPE));
  printf("%zu %zu\n", hc_fn_packed_bytes(5120), hc_pre_stats_workspace_bytes(4096, 5120));
  /* M = 0 is a no-op; NULL inputs with M > 0 and a width the post does not take are errors */
  printf("%d\n", hc_post(NULL, 0, NULL, 0, NULL, NULL, 0, 5120, NULL, 0, NULL));
  printf("%d\n", hc_post(NULL, 5120, NULL, 4 * 5120, NULL, NULL, 5, 5120, NULL, 4 * 5120, NULL));
  printf("%d\n", hc_post((const uint16_t*)&fake, 640, (const uint16_t*)&fake, 2560,
                         (const float*)&fake, (const float*)&fake, 5, 640, (uint16_t*)&fake, 2560,
                         NULL));
  return 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not available")
    return path


@pytest.mark.parametrize("lang,std,cc", [("c", "c99", "gcc"), ("c++", "c++11", "g++")])
def test_header_compiles_alone(lang, std, cc):
    r = subprocess.run([_compiler(cc), "-fsyntax-only", "-x", lang, f"-std={std}", "-Wall",
                        "-Wextra", "-Werror", "-pedantic", HEADER], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_links_and_calls_the_abi(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        from hyper_connection_residual_hc_amd import build
        build.build()
    gcc = _compiler("gcc")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_lib.LIB_PATH)
    libname = os.path.basename(_lib.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", libdir, f"-l:{libname}",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    lines = run.stdout.split("\n")
    assert lines[0] == "100"
    assert lines[1] == "HC_OK HC_ERR_SHAPE"
    assert lines[2] == f"{4 * 5120 * 5 * 16 * 2} {16 * 4096 * 25 * 4}"
    assert lines[3:6] == ["0", "1", "2"]
