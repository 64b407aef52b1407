"""The boundary as a C caller sees it: include/pa.h compiled as C99 with
-pedantic (no warnings), a program linked against libpa.so, and calls that
need no GPU (a partition-size plan for a stated device, workspace sizing,
argument validation that fails before any HIP call, status names)."""

import shutil
import subprocess
from pathlib import Path

import pytest

from paged_kv_cache_size_amd import binding as B

ROOT = Path(__file__).resolve().parents[1]

CLIENT = r"""
#include <stdio.h>
#include "pa.h"

int main(void) {
  int32_t ps = pa_decode_plan_partition_size(256, 32, 8, 128, 4096, 16, PA_BF16, NULL, 256, 2);
  size_t ws = pa_decode_workspace_bytes(256, 32, 128, 4096, 16);
  /* a null output pointer: refused before anything is enqueued */
  int rc = pa_decode_step(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 4, 8, 2, 128, 16, 8, 64, 128,
                          0.088f, PA_BF16, NULL, 0, 16, PA_KV_SPLIT, NULL);
  printf("%d %zu %d %s\n", (int)ps, ws, rc, pa_status_string(rc));
  return 0;
}
"""


def test_c_client_compiles_links_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = Path(B.LIB_PATH)
    if not lib.exists():
        pytest.skip("libpa.so not built")
    src = tmp_path / "client.c"
    src.write_text(CLIENT)
    exe = tmp_path / "client"
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", str(ROOT / "include"),
                          str(src), "-L", str(lib.parent), "-lpa", f"-Wl,-rpath,{lib.parent}", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    ps, ws, rc, name = run.stdout.split(maxsplit=3)
    assert int(ps) == B.lib().pa_decode_plan_partition_size(256, 32, 8, 128, 4096, 16, B.PA_BF16, None, 256, 2)
    assert int(ps) > 0 and int(ws) > 0
    assert int(rc) == B.PA_ERR_INVALID_ARG and name.startswith("PA_ERR_INVALID_ARG")
