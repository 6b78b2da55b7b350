"""The C ABI from plain C: include/wsvd.h compiles as C11 with gcc, a C
program links against libwsvd.so, and the pure-host entry points and a
rejected call behave as documented.  CPU only: nothing reaches a kernel."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rank_kv_cache_flash_amd")
LIB = os.path.join(PKG, "libwsvd.so")
ROCM_INC = "/opt/rocm/include"

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "wsvd.h"

int main(void) {
    /* pure-host helpers */
    if (strstr(wsvd_version(), "gfx950") == NULL) return 1;
    if (strlen(wsvd_status_string(WSVD_ERR_WORKSPACE)) == 0) return 2;
    if (wsvd_decode_num_splits(1, 32, 1088, 0) < 1) return 3;
    if (wsvd_decode_workspace_bytes(1, 32, 128, 1088, 0) == 0) return 4;
    if (wsvd_factorize_svd_workspace_bytes(4096, 32, 128) == 0) return 5;
    /* a call that host validation rejects before any HIP call */
    int st = wsvd_decode_attn(0, 32, 128, 32, 1088, NULL, NULL, WSVD_BF16, NULL, NULL, WSVD_BF16, NULL, NULL,
                              NULL, NULL, WSVD_BF16, 0.0f, 0, NULL, 0, NULL, WSVD_BF16, NULL);
    if (st != WSVD_ERR_SHAPE) return 6;
    st = wsvd_combine_splits(1, 1, 128, 1, NULL, NULL, NULL, WSVD_F32, NULL);
    if (st != WSVD_ERR_NULL) return 7;
    printf("ok %s\n", wsvd_version());
    return 0;
}
"""


@pytest.fixture(scope="module")
def built(tmp_path_factory):
    if not os.path.exists(LIB):
        pytest.fail("libwsvd.so is not built (python -m rank_kv_cache_flash_amd.build)")
    if shutil.which("gcc") is None or not os.path.isdir(ROCM_INC):
        pytest.skip("gcc or the ROCm headers are not available")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "main.c"
    src.write_text(C_SRC)
    exe = d / "main"
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{ROCM_INC}",
           str(src), f"-L{PKG}", "-lwsvd", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return exe


def test_header_compiles_as_c_and_links(built):
    r = subprocess.run([str(built)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("ok wsvd")
