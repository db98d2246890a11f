"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

crisp_api.cpp (argument validation, size queries, workspace carving) is
compiled with both sanitizers on its host side only, linked with the library's
other objects into a small driver program, and the driver runs every entry
point's validation paths and every size query, including the largest accepted
shapes (where a 32-bit or signed size product would overflow) and shapes just
past each limit.  Any sanitizer report aborts the driver, so the test passes
only if the host code does nothing undefined on these paths and every call
returns its documented status.  No HIP call is made: every call fails
validation first, or is a pure size query.
"""
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_patsearch_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJS = ["route.o", "select.o", "attn.o", "flex.o", "probe.o"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

DRIVER = textwrap.dedent(r"""
    #include <cstdio>
    #include <cstdint>
    #include <cstring>
    #include "crisp.h"

    static int fails = 0;
    #define EXPECT(call, want) do { int got_ = (call); if (got_ != (want)) { \
        std::printf("FAIL line %d: %s = %d, want %d\n", __LINE__, #call, got_, (want)); ++fails; } } while (0)

    static crisp_cfg cfg() {
      crisp_cfg c; c.block = 128; c.last_q = 128; c.w_sink = 128; c.w_local = 128; c.k_min_tokens = 1024;
      c.tau = 0.2f; c.alpha = 1.0f; c.gamma = 0.95f; return c;
    }
    static crisp_shape shp(int b, int n, int hq, int hk, int d) { crisp_shape s; s.batch = b; s.n = n; s.h_q = hq;
      s.h_kv = hk; s.d = d; return s; }

    int main() {
      crisp_cfg c = cfg();
      size_t bytes = 0;
      int64_t blocks = 0;
      int32_t use = -1;
      // size queries over the accepted range, up to the largest shapes
      const crisp_shape ok[] = {shp(1, 384, 1, 1, 64), shp(1, 1 << 20, 8, 1, 128), shp(1, 1 << 20, 16, 4, 128),
                                shp(2, 1 << 19, 16, 8, 128), shp(4095, 512, 16, 16, 64), shp(65535, 384, 1, 1, 64),
                                shp(0, 4096, 2, 2, 64), shp(3, 131072, 40, 8, 128)};
      for (const crisp_shape& s : ok) {
        for (int call = 0; call <= 5; ++call) {
          bytes = 0;
          EXPECT(crisp_workspace_bytes(&s, &c, call, &bytes), CRISP_OK);
        }
        EXPECT(crisp_max_blocks(&s, &blocks), CRISP_OK);
        EXPECT(crisp_use_dense(&s, &use), CRISP_OK);
      }
      // just past each limit
      const crisp_shape bad[] = {shp(1, (1 << 20) + 128, 8, 1, 128), shp(1, 256, 1, 1, 64), shp(1, 4096 + 64, 1, 1, 64),
                                 shp(65536, 384, 1, 1, 64), shp(1, 1 << 20, 2048, 1, 128), shp(-1, 4096, 1, 1, 64),
                                 shp(1, 4096, 3, 2, 64), shp(1, 4096, 2, 0, 64), shp(1, 4096, 2, 2, 96),
                                 shp(1, -128, 1, 1, 64), shp(2147483647, 4096, 2147483647, 1, 64)};
      for (const crisp_shape& s : bad) {
        EXPECT(crisp_workspace_bytes(&s, &c, 0, &bytes), CRISP_ERR_SHAPE);
        EXPECT(crisp_max_blocks(&s, &blocks), CRISP_ERR_SHAPE);
      }
      const crisp_shape s = shp(1, 4096, 2, 2, 64);
      EXPECT(crisp_workspace_bytes(&s, &c, 6, &bytes), CRISP_ERR_PARAM);
      EXPECT(crisp_workspace_bytes(&s, &c, -1, &bytes), CRISP_ERR_PARAM);
      EXPECT(crisp_workspace_bytes(nullptr, &c, 0, &bytes), CRISP_ERR_NULL);
      EXPECT(crisp_workspace_bytes(&s, nullptr, 0, &bytes), CRISP_ERR_NULL);
      EXPECT(crisp_workspace_bytes(&s, &c, 0, nullptr), CRISP_ERR_NULL);
      // settings
      crisp_cfg b1 = c; b1.gamma = 0.f; EXPECT(crisp_workspace_bytes(&s, &b1, 0, &bytes), CRISP_ERR_PARAM);
      crisp_cfg b2 = c; b2.alpha = -1.f; EXPECT(crisp_workspace_bytes(&s, &b2, 0, &bytes), CRISP_ERR_PARAM);
      crisp_cfg b3 = c; b3.block = 64; EXPECT(crisp_workspace_bytes(&s, &b3, 0, &bytes), CRISP_ERR_UNSUPPORTED);
      crisp_cfg b4 = c; b4.k_min_tokens = 100; EXPECT(crisp_workspace_bytes(&s, &b4, 0, &bytes), CRISP_ERR_PARAM);
      // every entry point with a required pointer missing or a bad shape fails before any HIP call
      char* fake = reinterpret_cast<char*>(0x10000);
      float* f = reinterpret_cast<float*>(fake);
      int8_t* i8 = reinterpret_cast<int8_t*>(fake);
      int64_t* i64 = reinterpret_cast<int64_t*>(fake);
      int32_t* i32 = reinterpret_cast<int32_t*>(fake);
      uint8_t* u8 = reinterpret_cast<uint8_t*>(fake);
      const crisp_shape big = shp(1, (1 << 20) + 128, 8, 1, 128);
      EXPECT(crisp_route(&s, &c, nullptr, fake, f, i8, f, f, fake, 1 << 30, nullptr), CRISP_ERR_NULL);
      EXPECT(crisp_route(&big, &c, fake, fake, f, i8, f, f, fake, 1 << 30, nullptr), CRISP_ERR_SHAPE);
      EXPECT(crisp_route(&s, &c, fake, fake, f, i8, f, f, fake, 0, nullptr), CRISP_ERR_WORKSPACE);
      EXPECT(crisp_route_noalloc(&s, &c, nullptr, fake, f, i8, f, f, nullptr), CRISP_ERR_NULL);
      EXPECT(crisp_route_noalloc(&big, &c, fake, fake, f, i8, f, f, nullptr), CRISP_ERR_SHAPE);
      const crisp_shape huge = shp(1, 1 << 20, 32, 8, 128);
      EXPECT(crisp_route_noalloc(&huge, &c, fake, fake, f, i8, f, f, nullptr), CRISP_ERR_SCRATCH);
      EXPECT(crisp_select(&s, &c, fake, fake, nullptr, f, f, i64, i32, 1 << 20, u8, fake, 1 << 30, nullptr),
             CRISP_ERR_NULL);
      EXPECT(crisp_select(&s, &c, fake, fake, i8, f, f, i64, i32, 1, u8, fake, 1 << 30, nullptr), CRISP_ERR_CAPACITY);
      EXPECT(crisp_select(&s, &c, fake, fake, i8, f, f, i64, i32, 1 << 20, u8, fake, 0, nullptr), CRISP_ERR_WORKSPACE);
      EXPECT(crisp_select_variant(&s, &c, 8, fake, fake, i8, f, f, i64, i32, 1 << 20, u8, fake, 1 << 30, nullptr),
             CRISP_ERR_PARAM);
      EXPECT(crisp_sparse_attn(&s, &c, fake, fake, nullptr, i64, i32, 1, fake, 0, fake, 1 << 30, nullptr),
             CRISP_ERR_NULL);
      EXPECT(crisp_sparse_attn(&s, &c, fake, fake, fake, i64, i32, 1, fake, 2, fake, 1 << 30, nullptr),
             CRISP_ERR_PARAM);
      EXPECT(crisp_sparse_attn(&s, &c, fake + 2, fake, fake, i64, i32, 1, fake, 0, fake, 1 << 30, nullptr),
             CRISP_ERR_ALIGN);
      EXPECT(dense_attn(&big, fake, fake, fake, fake, 0, fake, 1 << 30, nullptr), CRISP_ERR_SHAPE);
      EXPECT(dense_attn(&s, fake, fake, fake, fake, 0, fake, 0, nullptr), CRISP_ERR_WORKSPACE);
      EXPECT(flex_route(&s, &c, -1.f, fake, fake, f, f, i8, fake, 1 << 30, nullptr), CRISP_ERR_PARAM);
      EXPECT(crisp_use_dense(nullptr, &use), CRISP_ERR_NULL);
      EXPECT(crisp_mfma_probe(nullptr, f, 1, nullptr, nullptr), CRISP_ERR_NULL);
      // status strings for every code and for codes that are not statuses
      for (int code = -12; code <= 3; ++code) {
        const char* m = crisp_status_string(code);
        if (!m || !std::strlen(m)) { std::printf("FAIL: empty status string for %d\n", code); ++fails; }
      }
      const char* e = crisp_last_error();
      if (!e) { std::printf("FAIL: crisp_last_error returned NULL\n"); ++fails; }
      std::printf(fails ? "FAILED %d\n" : "ok\n", fails);
      return fails ? 1 : 0;
    }
    """)


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in OBJS):
        from long_context_sparse_patsearch_amd.build import build
        build(verbose=False)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-w",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    api = tmp_path / "crisp_api_san.o"
    drv_src = tmp_path / "driver.cpp"
    drv_src.write_text(DRIVER)
    exe = tmp_path / "abi_driver"
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    r = subprocess.run([HIPCC, *flags, *SAN, *inc, "-c", os.path.join(CSRC, "crisp_api.cpp"), "-o", str(api)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([HIPCC, *flags, *SAN, *inc, "-c", str(drv_src), "-o", str(tmp_path / "driver.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    objs = [str(api), str(tmp_path / "driver.o")] + [os.path.join(BUILD, o) for o in OBJS]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", str(exe), *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and out.strip().endswith("ok"), out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
