"""The boundary is a C ABI: a C99 program built with -pedantic -Werror includes
include/jattn.h, links libjattn.so and drives the host-only calls (plan
creation with a zero-length sample, summary, export, a refused descriptor and
its error text).  CPU only."""
import os
import shutil
import subprocess

import pytest

from jagged_variable_length_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = r"""
#include <stdio.h>
#include <string.h>
#include "jattn.h"

int main(void) {
  const int64_t qo[4] = {0, 5, 12, 12}, ko[4] = {0, 7, 9, 30};
  jattn_desc d;
  jattn_plan* p = NULL;
  jattn_plan_summary s;
  int64_t n = 0;
  int rc;
  memset(&d, 0, sizeof d);
  d.B = 3;
  d.H = 2;
  d.D = 64;
  d.act = JATTN_SOFTMAX;
  d.mask = JATTN_MASK_NONE;
  d.has_bias = 1;
  d.want_dbias = 1;
  d.in_dtype = d.out_dtype = d.grad_dtype = JATTN_BF16;
  d.dbias_dtype = JATTN_F32;
  d.order = JATTN_ZIGZAG;
  rc = jattn_plan_create(&d, qo, ko, &p);
  if (rc != JATTN_OK) {
    printf("create %d %s\n", rc, jattn_last_error());
    return 1;
  }
  if (jattn_plan_info(p, &s) != JATTN_OK) return 2;
  if (jattn_plan_export(p, JATTN_PLAN_FWD * 2, NULL, 0, &n) != JATTN_OK) return 3;
  printf("%lld %lld %lld %.1f %lld\n", (long long)s.Tq, (long long)s.Tk, (long long)s.bias_elems, s.flops_fwd,
         (long long)n);
  jattn_plan_destroy(p);
  d.D = 48;
  rc = jattn_plan_create(&d, qo, ko, &p);
  printf("%d %s\n", rc, jattn_strerror(rc));
  return rc == JATTN_E_SHAPE ? 0 : 4;
}
"""


def test_c_program_uses_the_abi(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    assert os.path.exists(B.LIB_PATH), "build the library first"
    src = tmp_path / "consumer.c"
    exe = tmp_path / "consumer"
    src.write_text(SRC)
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-l:libjattn.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    first, second = out.stdout.strip().splitlines()
    tq, tk, nb, flops, n = first.split()
    pairs = 5 * 7 + 7 * 2 + 0 * 21  # the third sample has no queries
    assert (int(tq), int(tk), int(nb)) == (12, 30, 2 * pairs)
    assert float(flops) == 4.0 * 2 * 64 * pairs
    assert int(n) > 0 and int(n) % 4 == 0  # (b, h, tile, cost) quadruples
    assert second.startswith(f"{B.JATTN_E_SHAPE} ")
