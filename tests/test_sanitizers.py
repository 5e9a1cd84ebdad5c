"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The oracle (oracle/ref_attn.c) is rebuilt with -fsanitize=address,undefined
   and every oracle pin runs against that build in a child Python process
   with libasan preloaded: any out-of-bounds access, use after free or
   undefined operation (signed overflow, bad shift, misaligned load) in the
   oracle aborts the child.
2. The C ABI's argument validation (exact_io_aware_59_amd/csrc/fa_api.hip,
   host code only) is compiled as plain C++ with the same sanitizers and
   linked against stub launchers that record the call instead of enqueueing
   a kernel; a driver then calls every entry point with valid, invalid,
   aliasing and overflowing arguments on fake addresses.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _gcc_lib(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _gcc_lib("libasan.so")
    if asan is None or shutil.which("gcc") is None:
        pytest.skip("gcc's libasan is not available")
    so = str(tmp_path / "libref_attn_asan.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", *SAN,
                    os.path.join(ROOT, "oracle", "ref_attn.c"), "-o", so, "-lm"], check=True)
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import oracle
        from tests import oracle_pins as P
        orc = oracle.Oracle({so!r})
        for pin in P.ALL_PINS:
            pin(orc)
            print("ok", pin.__name__, flush=True)
        """)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=900)
    assert r.returncode == 0, f"oracle pins under ASan/UBSan failed:\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    n_ok = r.stdout.count("\nok ") + r.stdout.startswith("ok ")
    from tests import oracle_pins as P
    assert n_ok == len(P.ALL_PINS), r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-3000:]


STUB = r"""
#include <hip/hip_runtime.h>
#include "fa_kernels.h"
int g_launches = 0;
namespace fa {
static hipError_t rec() { g_launches++; return hipSuccess; }
hipError_t launch_fwd_bf16(const FwdArgs&) { return rec(); }
hipError_t launch_bwd_bf16(const BwdArgs&) { return rec(); }
hipError_t launch_bwd_prep_bf16(const BwdArgs&) { return rec(); }
hipError_t launch_bwd_main_bf16(const BwdArgs&) { return rec(); }
hipError_t launch_bwd_dq_bf16(const BwdArgs&) { return rec(); }
hipError_t launch_bwd_dq_first_bf16(const BwdArgs&) { return rec(); }
hipError_t launch_fwd_f32(const FwdArgs&) { return rec(); }
hipError_t launch_bwd_f32(const BwdArgs&) { return rec(); }
hipError_t launch_decode_bf16(const DecArgs&) { return rec(); }
hipError_t launch_fp8_quantize(const F8QuantArgs&) { return rec(); }
hipError_t launch_fwd_fp8(const F8FwdArgs&) { return rec(); }
}
// the static scratch of fa_bwd_noalloc: its "device address" is the host stand-in here
hipError_t hipGetDevice(int* dev) { *dev = 0; return hipSuccess; }
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) { *ptr = const_cast<void*>(symbol); return hipSuccess; }
"""

DRIVER = r"""
#include <stdio.h>
#include <stdint.h>
#include <math.h>
#include "fa.h"
extern int g_launches;
#define P(i) ((void*)(uintptr_t)(((uint64_t)(i) + 1) << 40))
static int fails = 0;
#define EXPECT(call, want) do { int got_ = (call); if (got_ != (want)) { \
    printf("FAIL line %d: got %d want %d\n", __LINE__, got_, want); fails++; } } while (0)
int main(void) {
    const int big = 2147483647;
    /* valid calls reach the (stub) launcher */
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), 2, 16, 4096, 128, 0.088f, 1, NULL, NULL), FA_OK);
    EXPECT(fa_fwd_f32((float*)P(1), (float*)P(2), (float*)P(3), (float*)P(4), (float*)P(5), 1, 1, 128, 64,
                      0.125f, 0, (const uint8_t*)P(6), NULL), FA_OK);
    size_t ws = fa_bwd_workspace_size(2, 16, 4096, 128);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), 2, 16, 4096, 128, 0.088f, 1,
                  NULL, P(10), ws, NULL), FA_OK);
    EXPECT(fa_bwd_prep(P(4), P(5), (float*)P(6), 2, 16, 4096, 128, P(10), ws, NULL), FA_OK);
    EXPECT(fa_bwd_main(P(1), P(2), P(3), P(5), P(8), P(9), 2, 16, 4096, 128, 0.088f, 1, NULL, P(10), ws, NULL),
           FA_OK);
    EXPECT(fa_bwd_dq(P(1), P(2), P(3), P(5), P(7), 2, 16, 4096, 128, 0.088f, 1, NULL, P(10), ws, NULL), FA_OK);
    EXPECT(fa_bwd_dq_first(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), 2, 16, 4096, 128, 0.088f, 1, NULL,
                           P(10), ws, NULL), FA_OK);
    EXPECT(fa_bwd_dq_first(P(1), P(2), P(3), NULL, P(5), (float*)P(6), P(7), 2, 16, 4096, 128, 0.088f, 1, NULL,
                           P(10), ws, NULL), FA_ERR_INVALID_ARG);
    fa_variant var = {100, -1, (const float*)P(11)};
    EXPECT(fa_fwd_ex(P(1), P(2), P(3), P(4), (float*)P(5), 2, 16, 4096, 128, 0.088f, 1, NULL, &var, NULL), FA_OK);
    size_t dws = fa_decode_workspace_size(16, 32, 8, 1, 128, 256, 32);
    EXPECT(fa_decode_paged(P(1), P(2), P(3), (const int32_t*)P(4), (const int32_t*)P(5), P(6), (float*)P(7),
                           16, 32, 8, 1, 128, 600, 256, 32, 0.088f, 1, dws ? P(8) : NULL, dws, NULL), FA_OK);
    EXPECT(fa_fp8_quantize(P(1), (uint8_t*)P(2), (int8_t*)P(3), 2, 16, 4096, 128, (const float*)P(4), 1, NULL),
           FA_OK);
    EXPECT(fa_fwd_fp8((const uint8_t*)P(1), (const int8_t*)P(2), (const uint8_t*)P(3), (const int8_t*)P(4),
                      (const uint8_t*)P(5), (const int8_t*)P(6), P(7), (float*)P(8), 2, 16, 4096, 128, 0.088f, 1,
                      NULL), FA_OK);
    EXPECT(fa_bwd_noalloc(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), 2, 16, 4096, 128, 0.088f,
                          1, NULL, NULL, NULL), FA_OK);
    int launched = g_launches;
    EXPECT(fa_bwd_noalloc(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), big, big, big, 128, 0.1f,
                          1, NULL, NULL, NULL), FA_ERR_SCRATCH);
    EXPECT(fa_bwd_noalloc(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), 1, 1, FA_NOALLOC_MAX_ROWS + 1,
                          64, 0.1f, 1, NULL, NULL, NULL), FA_ERR_SCRATCH);
    EXPECT(fa_bwd_noalloc(NULL, P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), 2, 16, 4096, 128, 0.1f,
                          1, NULL, NULL, NULL), FA_ERR_INVALID_ARG);
    /* invalid calls never reach a launcher; overflowing sizes must not overflow inside the checks */
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), big, big, big, big, 0.1f, 0, NULL, NULL),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), -1, 1, 1, 64, 0.1f, 0, NULL, NULL), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), 1, 1, 1 << 30, 64, 0.1f, 0, NULL, NULL),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), 1, 1, 128, 64, NAN, 0, NULL, NULL), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(P(1), P(1), P(3), P(1), (float*)P(5), 1, 1, 128, 64, 0.1f, 0, NULL, NULL), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), 1, 1, 128, 72, 0.1f, 0, NULL, NULL), FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), 1, 1, 128, 272, 0.1f, 0, NULL, NULL), FA_ERR_UNSUPPORTED);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), 1, 1, 128, 144, 0.1f, 0,
                  NULL, P(10), ws, NULL), FA_ERR_UNSUPPORTED);
    EXPECT((int)fa_bwd_workspace_size(big, big, big, 128), 0);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(8), P(9), 2, 16, 4096, 128, 0.088f, 1,
                  NULL, P(10), ws - 1, NULL), FA_ERR_WORKSPACE);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), (float*)P(6), P(7), P(7), P(9), 2, 16, 4096, 128, 0.088f, 1,
                  NULL, P(10), ws, NULL), FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_workspace_size(big, big, 1, big, 128, big, big) == 0 ? 1 : 0, 1);
    EXPECT(fa_decode_paged(P(1), P(2), P(3), (const int32_t*)P(4), (const int32_t*)P(5), P(6), (float*)P(7),
                           big, big, 1, big, 128, big, big, big, 0.1f, 1, NULL, 0, NULL), FA_ERR_INVALID_ARG);
    EXPECT(fa_fp8_quantize(P(1), (uint8_t*)P(1), (int8_t*)P(3), 1, 1, 64, 64, NULL, 0, NULL), FA_ERR_INVALID_ARG);
    fa_variant bad = {1, 1, (const float*)((char*)P(11) + 2)};
    EXPECT(fa_fwd_ex(P(1), P(2), P(3), P(4), (float*)P(5), 1, 1, 128, 64, 0.1f, 0, NULL, &bad, NULL),
           FA_ERR_INVALID_ARG);
    if (g_launches != launched) { printf("FAIL: an invalid call launched\n"); fails++; }
    printf("%s: %d failures, %d launches\n", fails ? "FAILED" : "OK", fails, g_launches);
    return fails != 0;
}
"""


def test_abi_validation_under_asan_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("g++ or the HIP headers are not available")
    (tmp_path / "stub.cpp").write_text(STUB)
    (tmp_path / "driver.c").write_text(DRIVER)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "exact_io_aware_59_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
           # HIP_SYMBOL as amd_hip_runtime.h defines it (host-only, the symbol is its host stand-in)
           "-DHIP_SYMBOL(X)=X"]
    exe = str(tmp_path / "abi_check")
    objs = []
    for src, lang in ((os.path.join(ROOT, "exact_io_aware_59_amd", "csrc", "fa_api.hip"), "c++"),
                      (str(tmp_path / "stub.cpp"), "c++"), (str(tmp_path / "driver.c"), "c")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        std = "-std=c++17" if lang == "c++" else "-std=c11"
        r = subprocess.run([cxx if lang == "c++" else "gcc", "-x", lang, std, "-O1", *SAN, *inc, "-c", src,
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    subprocess.run([cxx, *SAN, *objs, "-o", exe, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1"))
    assert r.returncode == 0 and "OK:" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
