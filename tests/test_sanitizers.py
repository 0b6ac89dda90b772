"""Sanitizer runs on the CPU: the oracle (oracle.c) and the host half of the
C ABI (argument checks, split planning, workspace layout, status strings of
csrc/smla.hip), each built into a small driver with AddressSanitizer and
UndefinedBehaviorSanitizer and run to completion; any report fails the test.
The drivers are written here; they call only functions the two libraries
export.  No GPU is used (the C ABI calls end in their host checks or in
SMLA_ERR_NO_DEVICE)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
SMLA_HIP = os.path.join(ROOT, "sparse_mla_decode_02_amd", "csrc", "smla.hip")
SMLA_PAGED_HIP = os.path.join(ROOT, "sparse_mla_decode_02_amd", "csrc", "smla_paged.hip")
SMLA_FOURWAVE_HIP = os.path.join(ROOT, "sparse_mla_decode_02_amd", "csrc", "smla_fourwave.hip")
INCLUDE = os.path.join(ROOT, "include")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")

ORACLE_DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
int oracle_decode_fmt(const uint16_t*, const uint8_t*, int64_t, const int32_t*, int64_t, const int32_t*,
                      int, int, int, double, double*, double*, int, int);
int oracle_decode_paged(const uint16_t*, const uint8_t*, int64_t, int32_t, const int32_t*, int64_t,
                        const int32_t*, int64_t, const int32_t*, int, int, int, double, double*, double*,
                        int, int);
int oracle_decode_padded512(const uint16_t*, const uint8_t*, int64_t, const int32_t*, int64_t,
                            const int32_t*, int, int, int, double, double*, double*);
double oracle_e4m3fn_value(uint8_t);
double oracle_ue8m0_value(uint8_t);
static uint32_t st = 12345u;
static uint32_t nxt(void) { st = st * 1664525u + 1013904223u; return st >> 8; }
int main(void) {
    enum { B = 3, H = 16, K = 40, S = 97 };
    for (int c = 0; c < 256; c++) (void)oracle_e4m3fn_value((uint8_t)c);
    for (int c = 0; c < 256; c++) (void)oracle_ue8m0_value((uint8_t)c);
    for (int fmt = 0; fmt < 2; fmt++) {
        const int R = fmt ? 584 : 640;
        uint16_t* q = malloc(sizeof(uint16_t) * B * H * 512);
        uint8_t* kv = malloc((size_t)B * S * R);
        int32_t* idx = malloc(sizeof(int32_t) * B * K);
        int32_t seqlens[B] = {S, 50, 0};
        double* out = malloc(sizeof(double) * B * H * 512);
        double* out2 = malloc(sizeof(double) * B * H * 512);
        double lse[B * H], lse2[B * H];
        for (int i = 0; i < B * H * 512; i++) q[i] = (uint16_t)(0x3C00 + (nxt() & 0x3FF)) ^ (uint16_t)((nxt() & 1) << 15);
        for (size_t i = 0; i < (size_t)B * S * R; i++) kv[i] = (uint8_t)(nxt() & 0x7E);
        for (int b = 0; b < B; b++)
            for (int t = 0; t < S; t++) {
                uint8_t* row = kv + ((size_t)b * S + t) * R;
                if (fmt == 0) { for (int g = 0; g < 8; g++) { float s = 0.01f * (1 + g); memcpy(row + 448 + 4 * g, &s, 4); } }
                else { for (int g = 0; g < 8; g++) row[448 + g] = (uint8_t)(120 + g); }
            }
        for (int i = 0; i < B * K; i++) idx[i] = (int32_t)(nxt() % (S + 20)) - 10;   /* some < 0, some >= seqlen */
        int used = oracle_decode_fmt(q, kv, S, idx, K, seqlens, B, H, K, 0.0441941738, out, lse, 2, fmt);
        if (used < 1) return 1;
        for (int i = 0; i < B * H * 512; i++) if (!isfinite(out[i])) return 2;
        if (fmt == 0) {
            oracle_decode_padded512(q, kv, S, idx, K, seqlens, B, H, K, 0.0441941738, out2, lse2);
            if (memcmp(out, out2, sizeof(double) * B * H * 512) != 0) return 3;
        }
        /* the same rows through a pool of pages of 8 rows, pages in reverse order */
        const int P = 8, NP = (S + P - 1) / P;
        uint8_t* pool = malloc((size_t)B * NP * P * R);
        int32_t* bt = malloc(sizeof(int32_t) * B * NP);
        memset(pool, 0xFF, (size_t)B * NP * P * R);
        for (int b = 0; b < B; b++)
            for (int p = 0; p < NP; p++) {
                const int page = B * NP - 1 - (b * NP + p);
                bt[b * NP + p] = page;
                for (int r = 0; r < P && p * P + r < S; r++)
                    memcpy(pool + ((size_t)page * P + r) * R, kv + ((size_t)b * S + p * P + r) * R, R);
            }
        oracle_decode_paged(q, pool, (int64_t)B * NP, P, bt, NP, idx, K, seqlens, B, H, K, 0.0441941738, out2,
                            lse2, 2, fmt);
        if (memcmp(out, out2, sizeof(double) * B * H * 512) != 0) return 4;
        free(pool); free(bt); free(q); free(kv); free(idx); free(out); free(out2);
    }
    puts("oracle sanitizer run: ok");
    return 0;
}
"""

ABI_DRIVER = r"""
#include <stdio.h>
#include <string.h>
#include "smla.h"
int main(void) {
    int bad = 0;
    for (int s = 0; s <= 9; s++) if (!smla_status_str((smla_status)s)[0]) bad = 1;
    const int Bs[] = {0, 1, 3, 32, 64, 96}, Hs[] = {16, 48, 64, 256}, Ks[] = {0, 1, 45, 512, 2048, 1 << 20};
    for (int bi = 0; bi < 6; bi++) for (int hi = 0; hi < 4; hi++) for (int ki = 0; ki < 6; ki++)
        for (int ns = 0; ns <= 9; ns += 3) for (int fmt = 0; fmt < 2; fmt++) {
            smla_shape s = {Bs[bi], Hs[hi], Ks[ki], ns, 131072, fmt};
            const int n = smla_num_splits(&s);
            const int c = smla_split_size(&s);
            const size_t w = smla_workspace_bytes(&s);
            if (n < 1 || c < 32 || (n == 1) != (w == 0 && n == 1)) bad = 2;
            char fake[64];
            smla_status st = sparse_mla_decode(fake, fake, (const int*)fake, (const int*)fake, 0.05f, fake,
                                               (float*)fake, &s, NULL, 0, NULL);
            if (st == SMLA_OK && s.batch > 0) bad = 3;
            st = sparse_mla_decode_noalloc(fake, fake, (const int*)fake, (const int*)fake, 0.05f, fake,
                                           (float*)fake, &s, NULL);
            if (st == SMLA_OK && s.batch > 0) bad = 4;
        }
    smla_shape bads[] = {{1, 15, 64, 0, 128, 0}, {-1, 16, 64, 0, 128, 0}, {1, 16, -1, 0, 128, 0},
                         {1, 16, (1 << 20) + 1, 0, 128, 0}, {1, 16, 64, 0, 0, 0}, {1, 16, 64, 0, 128, 2},
                         {1, 16, 64, 0, (int64_t)1 << 40, 0}};
    for (unsigned i = 0; i < sizeof(bads) / sizeof(bads[0]); i++)
        if (smla_num_splits(&bads[i]) != -1 || smla_workspace_bytes(&bads[i]) != 0) bad = 5;
    smla_paged pg = {48, 8, 100};
    smla_shape ok = {2, 16, 64, 1, 1, 0};
    char fake[64];
    if (sparse_mla_decode_paged(fake, fake, (const int*)fake, (const int*)fake, (const int*)fake, 0.05f, fake,
                                (float*)fake, &ok, &pg, NULL, 0, NULL) != SMLA_ERR_SHAPE) bad = 6;
    if (sparse_mla_combine(NULL, NULL, 1, 16, 2, NULL, NULL, NULL) != SMLA_ERR_NULL) bad = 7;
    printf("C ABI host sanitizer run: %s (%d)\n", bad ? "FAILED" : "ok", bad);
    return bad;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    drv = tmp_path / "oracle_driver.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_asan"
    rc, log = _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", ORACLE_C, str(drv), "-o", str(exe), "-lm"])
    assert rc == 0, log
    rc, log = _run([str(exe)], env=ENV)
    assert rc == 0 and "oracle sanitizer run: ok" in log and "runtime error" not in log, log


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_c_abi_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    drv = tmp_path / "abi_driver.cpp"
    drv.write_text(ABI_DRIVER)
    exe = tmp_path / "abi_asan"
    # sanitizers for the host code only (each -fsanitize= behind -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (SMLA_HIP, SMLA_FOURWAVE_HIP, SMLA_PAGED_HIP):
        objs.append(tmp_path / (os.path.basename(src) + ".o"))
        rc, log = _run([_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c", src, "-o", str(objs[-1])])
        assert rc == 0, log
    obj_drv = tmp_path / "drv.o"
    rc, log = _run([_hipcc(), "-O1", "-g", "-std=c++17", "-I", INCLUDE, *san, "-x", "c++", "-c", str(drv),
                    "-o", str(obj_drv)])
    assert rc == 0, log
    rc, log = _run([_hipcc(), "--offload-arch=gfx950", *san, *map(str, objs), str(obj_drv), "-o", str(exe)])
    assert rc == 0, log
    rc, log = _run([str(exe)], env=ENV)
    assert rc == 0 and "C ABI host sanitizer run: ok" in log and "runtime error" not in log, log
