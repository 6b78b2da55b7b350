"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled with host-only ASan + UBSan (the host side is the
C ABI's checks, the split rule, the workspace layout and the launchers'
sizing) into a test copy of libwsvd.so; a C driver built with the same
sanitizers calls every pure-host helper over ordinary, edge and extreme
sizes, and every entry point with arguments that host validation rejects.
Any sanitizer report fails the run.  CPU only: no call reaches a kernel.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rank_kv_cache_flash_amd")
CLANG = "/opt/rocm/llvm/bin/clang"

C_SRC = r"""
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "wsvd.h"

#define P ((void*)(uintptr_t)0x7f0000000000ull)  /* aligned, never dereferenced */
#define CHECK(cond, code) do { if (!(cond)) { printf("fail %d\n", code); return code; } } while (0)

static const int sizes[] = {-1, 0, 1, 2, 3, 7, 16, 32, 48, 64, 128, 255, 1024, 4096, 65536, 1 << 20, INT_MAX};
#define NS ((int)(sizeof(sizes) / sizeof(sizes[0])))

int main(void) {
    volatile size_t sink = 0;
    /* pure-host helpers over every combination of edge sizes */
    for (int i = 0; i < NS; ++i)
        for (int j = 0; j < NS; ++j)
            for (int k = 0; k < NS; ++k) {
                const int a = sizes[i], b = sizes[j], c = sizes[k];
                sink += (size_t)wsvd_decode_num_splits(a, b, c, 0);
                sink += (size_t)wsvd_decode_num_splits(a, b, c, 3);
                sink += wsvd_decode_workspace_bytes(a, b, 128, c, 0);
                sink += wsvd_decode_workspace_bytes(a, b, 64, c, 7);
                sink += wsvd_decode_lse_offset(a, b, 128, c, 0);
                sink += wsvd_decode_opart_offset(a, b, 128, c, 5);
                sink += wsvd_decode_counter_bytes(a, b);
                sink += wsvd_append_workspace_bytes(a, 4096, b, 48);
                sink += wsvd_append_workspace_bytes(64, a, b, 16);
                sink += wsvd_append_counter_bytes(a, b, 64);
                sink += wsvd_shared_decode_workspace_bytes(a, b, 1024, c, 0);
                sink += wsvd_factorize_svd_workspace_bytes(a, b, 128);
            }
    for (int st = -9; st <= 1; ++st) CHECK(wsvd_status_string(st) != NULL, 1);
    CHECK(strstr(wsvd_version(), "gfx950") != NULL, 2);

    /* decode: one rejected call per host check */
    #define DEC(nb, nh, H, r, Lc, L, q, qdt, CK, CV, Cdt, sK, sV, BK, BV, Bdt, S, ws, wsb, out, odt) \
        wsvd_decode_attn(nb, nh, H, r, Lc, L, q, qdt, CK, CV, Cdt, sK, sV, BK, BV, Bdt, 0.f, S, ws, wsb, out, odt, NULL)
    CHECK(DEC(0, 4, 64, 16, 256, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_SHAPE, 10);
    CHECK(DEC(1, 4, 64, 128, 256, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_SHAPE, 11);
    CHECK(DEC(INT_MAX, INT_MAX, 64, 16, INT_MAX, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_SHAPE, 12);
    CHECK(DEC(1, 4, 64, 16, 256, NULL, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_NULL, 13);
    CHECK(DEC(1, 4, 64, 16, 256, P, P, WSVD_I8, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_DTYPE, 14);
    CHECK(DEC(1, 4, 64, 16, 256, P, P, WSVD_F32, P, P, WSVD_I8, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_NULL, 15);
    CHECK(DEC(1, 4, 96, 16, 256, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_UNSUPPORTED, 16);
    CHECK(DEC(1, 4, 64, 16, 256, P, (char*)P + 4, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_ALIGN, 17);
    CHECK(DEC(1, 4, 64, 16, 256, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_WORKSPACE, 18);
    CHECK(DEC(1, 4, 64, 16, 256, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 257, P, 1 << 30, P, WSVD_F32) == WSVD_ERR_SHAPE, 19);
    CHECK(DEC(1, 4, 64, 16, 1 << 30, P, P, WSVD_F32, P, P, WSVD_F32, NULL, NULL, P, P, WSVD_F32, 0, P, 16, P, WSVD_F32) == WSVD_ERR_SHAPE, 20);
    CHECK(wsvd_decode_attn_noalloc(1, 32, 128, 32, 1088, P, P, WSVD_BF16, P, P, WSVD_BF16, NULL, NULL, P, P, WSVD_BF16,
                                   0.f, 0, NULL, WSVD_BF16, NULL) == WSVD_ERR_NULL, 21);
    CHECK(wsvd_decode_attn_noalloc(65537, 1, 128, 32, 16, P, P, WSVD_BF16, P, P, WSVD_BF16, NULL, NULL, P, P, WSVD_BF16,
                                   0.f, 0, P, WSVD_BF16, NULL) == WSVD_ERR_WORKSPACE, 22);
    CHECK(wsvd_decode_attn_rope(1, 4, 128, 48, 256, P, P, WSVD_BF16, P, P, WSVD_BF16, P, P, WSVD_BF16, P, P, 0.f, 0,
                                P, 1 << 20, P, WSVD_BF16, NULL) == WSVD_ERR_UNSUPPORTED, 23);
    CHECK(wsvd_dense_decode_attn(1, 4, 128, 256, P, P, WSVD_BF16, P, P, WSVD_F32, 0.f, 0, P, 1 << 20, P, WSVD_BF16,
                                 NULL) == WSVD_ERR_DTYPE, 24);
    CHECK(wsvd_combine_splits(1, 1, 128, 0, P, P, P, WSVD_F32, NULL) == WSVD_ERR_SHAPE, 25);
    CHECK(wsvd_combine_splits(1, 1, 100, 2, P, P, P, WSVD_F32, NULL) == WSVD_ERR_UNSUPPORTED, 26);
    CHECK(wsvd_append_latent(64, 4096, 32, 48, 8192, P, WSVD_BF16, P, P, WSVD_BF16, P, P, P, WSVD_I8, P, P, P,
                             1 << 30, NULL) == WSVD_ERR_UNSUPPORTED, 27);
    CHECK(wsvd_append_latent(64, 4000, 32, 32, 8192, P, WSVD_BF16, P, P, WSVD_BF16, P, P, P, WSVD_BF16, NULL, NULL, P,
                             1 << 30, NULL) == WSVD_ERR_UNSUPPORTED, 28);
    CHECK(wsvd_append_latent(64, 4096, 32, 48, 8192, P, WSVD_BF16, P, P, WSVD_BF16, P, P, P, WSVD_BF16, NULL, NULL,
                             NULL, 0, NULL) == WSVD_ERR_WORKSPACE, 29);
    CHECK(wsvd_append_latent_w8a8(64, 4096, 32, 48, 8192, P, P, P, P, P, P, P, P, P, WSVD_BF16, NULL, NULL, P, 16,
                                  NULL) == WSVD_ERR_WORKSPACE, 30);
    CHECK(wsvd_w8a8_quantize_activations(4, 3000, P, WSVD_BF16, P, P, NULL) == WSVD_ERR_UNSUPPORTED, 31);
    CHECK(wsvd_w8a8_prepare_factor(4096, 16, P, WSVD_I8, P, P, NULL) == WSVD_ERR_DTYPE, 32);
    CHECK(wsvd_rope_tables(0, 128, 10000.f, P, P, NULL) == WSVD_ERR_SHAPE, 33);
    CHECK(wsvd_factorize_svd(4096, 32, 128, 200, P, P, P, P, NULL, P, 1 << 30, NULL) == WSVD_ERR_SHAPE, 34);
    CHECK(wsvd_weighted_update_A(4096, 32, 128, 40, P, P, P, P, NULL) == WSVD_ERR_UNSUPPORTED, 35);
    CHECK(wsvd_weighted_update_B(4096, 32, 100, 32, P, P, P, P, NULL) == WSVD_ERR_UNSUPPORTED, 36);
    CHECK(wsvd_shared_decode_attn(1, 32, 128, 1000, 1088, P, P, P, P, P, P, 0.f, 0, P, 1 << 30, P, WSVD_BF16,
                                  NULL) == WSVD_ERR_UNSUPPORTED, 37);
    printf("ok %zu\n", (size_t)sink);
    return 0;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    from rank_kv_cache_flash_amd import build as B
    if not os.path.exists(CLANG) or shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC):
        pytest.skip("ROCm clang / hipcc not available")
    from concurrent.futures import ThreadPoolExecutor
    d = tmp_path_factory.mktemp("san")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = [str(d / src.replace(".hip", ".o")) for src in B.SOURCES]
    cmds = [[B.HIPCC, *B.FLAGS, *B.SOURCE_FLAGS.get(src, []), *san, "-c", os.path.join(B.CSRC, src), "-o", o]
            for src, o in zip(B.SOURCES, objs)]
    with ThreadPoolExecutor(min(8, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    lib = str(d / "libwsvd.so")
    _run([B.HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", lib, *objs])
    src = d / "main.c"
    src.write_text(C_SRC)
    exe = str(d / "main")
    _run([CLANG, "-std=c11", "-Wall", "-Werror", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include", str(src), f"-L{d}", "-lwsvd",
          f"-Wl,-rpath,{d}", "-o", exe])
    return exe


def test_abi_host_code_is_clean_under_asan_and_ubsan(sanitized):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert r.stdout.strip().splitlines()[-1].startswith("ok")
