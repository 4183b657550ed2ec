"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only; the GPU is not used).

- The oracle's C codec (oracle/mx_codec.c), built with gcc's sanitizers and driven by a small C
  program over edge values (signed zeros, the saturation boundary, subnormal ties, infinities,
  very large and very small magnitudes) and random blocks, checked against values the OCP E4M3
  and MX definitions fix.
- The C ABI's host paths: moe_api.hip built with host-side sanitizers (the device code is
  unchanged), linked with the library's other objects and a C++ driver that calls every size query
  over valid, unsupported and overflowing shapes and every entry point with null or misaligned
  pointers, which must be refused before any HIP call.

Any sanitizer report aborts the program, which fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routing_expert_grouped_amd", "csrc")
BUILD = os.path.join(ROOT, "routing_expert_grouped_amd", "_build")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

CODEC_DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
void oracle_e4m3_encode(const double* y, uint8_t* out, size_t n);
void oracle_mx_quantize_rows(const double* v, size_t nrows, size_t ncols, uint8_t* codes,
                             uint8_t* scales);
void oracle_mx_roundtrip_axis(const double* v, double* out, size_t outer, size_t L, size_t inner,
                              double* amax);
static int fails = 0;
static void expect(int ok, const char* what) { if (!ok) { printf("FAIL %s\n", what); ++fails; } }
int main(void) {
  /* E4M3: 448 is the largest finite code (0x7E), anything above saturates there, ties go to the
     even mantissa, subnormals are n * 2^-9, the sign of zero is kept */
  const double y[] = {0.0, -0.0, 448.0, 464.0, 1e300, INFINITY, -INFINITY, ldexp(1, -10),
                      ldexp(3, -10), ldexp(1, -9), 1.0, 1.0625, 1.1875, -2.5, ldexp(1, -1074),
                      240.0, 232.0};
  const uint8_t want[] = {0x00, 0x80, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00,
                          0x02, 0x01, 0x38, 0x38, 0x3A, 0xC2, 0x00,
                          0x77, 0x76};
  const size_t n = sizeof(y) / sizeof(y[0]);
  uint8_t got[sizeof(y) / sizeof(y[0])];
  oracle_e4m3_encode(y, got, n);
  for (size_t i = 0; i < n; ++i) {
    if (got[i] != want[i]) printf("  e4m3(%g) = 0x%02X, want 0x%02X\n", y[i], got[i], want[i]);
    expect(got[i] == want[i], "e4m3 edge value");
  }
  /* MX rows: a zero block (scale 2^-127), a block with amax 2^127 (scale 2^119), a block of tiny
     values whose exponent clamps at -127, and random blocks */
  enum { R = 5, C = 96 };
  double* v = malloc(sizeof(double) * R * C);
  uint8_t* codes = malloc(R * C);
  uint8_t* scales = malloc(R * C / 32);
  srand(7);
  for (int i = 0; i < R * C; ++i) v[i] = ((double)rand() / RAND_MAX - 0.5) * 8.0;
  for (int q = 0; q < 32; ++q) { v[q] = 0.0; v[C + q] = ldexp(q % 2 ? 1 : -1, 127 - q % 5);
                                 v[2 * C + q] = ldexp(1, -140 - q % 3); }
  oracle_mx_quantize_rows(v, R, C, codes, scales);
  expect(scales[0] == 0, "zero block scale");
  for (int q = 0; q < 32; ++q) expect((codes[q] & 0x7F) == 0, "zero block codes");
  expect(scales[C / 32] == 127 + 119, "2^127 block scale");
  expect(scales[2 * C / 32] == 0, "clamped tiny block scale");
  for (int i = 0; i < R * C; ++i) expect((codes[i] & 0x7F) <= 0x7E, "no NaN code");
  /* the round trip along a middle axis, [outer][L][inner] with inner > 1 */
  enum { O = 3, L = 64, I = 5 };
  double* a = malloc(sizeof(double) * O * L * I);
  double* b = malloc(sizeof(double) * O * L * I);
  double amax[I];
  for (int i = 0; i < O * L * I; ++i) a[i] = ((double)rand() / RAND_MAX - 0.5) * 1e3;
  oracle_mx_roundtrip_axis(a, b, O, L, I, amax);
  /* every element within a quarter of its block's largest magnitude (saturation of a block
     maximum between 448 and 512 scaled units is the largest error the definition allows) */
  for (int o = 0; o < O; ++o)
    for (int blk = 0; blk < L / 32; ++blk)
      for (int i = 0; i < I; ++i) {
        double m = 0.0;
        for (int q = 0; q < 32; ++q) m = fmax(m, fabs(a[(o * L + 32 * blk + q) * I + i]));
        for (int q = 0; q < 32; ++q) {
          const int at = (o * L + 32 * blk + q) * I + i;
          expect(fabs(b[at] - a[at]) <= m / 4, "round trip error");
        }
      }
  free(v); free(codes); free(scales); free(a); free(b);
  printf("%s\n", fails ? "FAILED" : "OK");
  return fails != 0;
}
"""

ABI_DRIVER = r"""
#include <cstdint>
#include <cstdio>
#include <vector>
#include "moe.h"
static int bad = 0;
static void refused(int line, int st, int want) {
  if (st != want) { std::printf("line %d returned %d, want %d\n", line, st, want); ++bad; }
}
int main() {
  if (moe_abi_version() < 1) ++bad;
  for (int c = -3; c <= 9; ++c)
    if (!moe_status_string(c)) ++bad;
  const std::vector<moe_shape> shapes = {
      {64, 256, 128, 8, 2, 8, 0},                 // the tiny layer
      {2048, 7168, 3072, 384, 6, 6, 0},           // DeepSeek-V4-Pro-shaped share
      {4096, 4096, 1024, 512, 10, 512, 0},        // Qwen-shaped layer
      {2048, 7168, 2048, 384, 8, 6, 2048},        // Kimi-shaped share with a shared expert
      {8192, 6144, 2048, 256, 8, 256, 0},         // GLM-5.2-shaped layer
      {1, 256, 256, 1, 1, 1, 0},                  // one token, one expert
      {0, 256, 256, 8, 2, 8, 0},                  // no tokens
      {64, 100, 128, 8, 2, 8, 0},                 // h not tiled
      {64, 256, 128, 8, 17, 8, 0},                // k above 16
      {64, 256, 128, 2000, 2, 2000, 0},           // too many experts
      {-5, -256, -128, -8, -2, -8, -1},           // negative sizes
      {1 << 30, 1 << 14, 1 << 14, 1024, 16, 1024, 0},                           // T k overflows
      {2147483647, 2147483392, 2147483392, 1024, 16, 1024, 2147483392}};        // every product
  unsigned long long acc = 0;
  for (const moe_shape& s : shapes)
    for (moe_dtype dt : {MOE_BF16, MOE_MXFP8}) {
      acc += moe_prepared_weight_bytes(&s, dt) + moe_route_workspace_bytes(&s) +
             moe_permute_workspace_bytes(&s) + moe_expert_ffn_workspace_bytes(&s, dt) +
             moe_forward_workspace_bytes(&s, dt) + moe_saved_bytes(&s, dt) +
             moe_forward_persistent_workspace_bytes(&s, dt) +
             moe_prepared_bwd_weight_bytes(&s, dt) + moe_backward_workspace_bytes(&s, dt);
      for (size_t r : {(size_t)0, (size_t)1000, (size_t)1 << 20, (size_t)1 << 30, (size_t)1 << 40})
        acc += (unsigned long long)moe_forward_ring_tokens(&s, dt, r);
    }
  // null and misaligned required pointers are refused before any HIP call
  const moe_shape s = shapes[0];
  const moe_shape sb = {64, 256, 256, 8, 2, 8, 0};  // a shape the backward covers
  void* mis = reinterpret_cast<void*>(uintptr_t(0x1000) + 4);
  const int E = MOE_EINVAL;
  refused(__LINE__, moe_check_e4m3(nullptr, nullptr), E);
  refused(__LINE__, moe_prepare_weights(&s, MOE_BF16, nullptr, nullptr, nullptr, nullptr,
                                        nullptr), E);
  refused(__LINE__, moe_route(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr), E);
  refused(__LINE__, moe_forward(&s, MOE_BF16, (const uint16_t*)mis, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), E);
  refused(__LINE__, moe_forward(nullptr, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), E);
  refused(__LINE__, moe_forward_ring(&s, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr), E);
  refused(__LINE__, moe_backward(&sb, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, 1, nullptr, nullptr), E);
  refused(__LINE__, moe_backward(&s, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, 1, nullptr, nullptr), MOE_EUNSUPPORTED);
  std::printf("%s %llu\n", bad ? "FAILED" : "OK", acc);
  return bad != 0;
}
"""


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert res.returncode == 0, (" ".join(cmd[:3]), res.stdout[-2000:], res.stderr[-3000:])
    return res


def test_oracle_codec_under_asan_ubsan():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        drv = os.path.join(d, "drv.c")
        exe = os.path.join(d, "drv")
        with open(drv, "w") as f:
            f.write(CODEC_DRIVER)
        _run([gcc, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-fsanitize=float-cast-overflow",
              os.path.join(ROOT, "oracle", "mx_codec.c"), drv, "-lm", "-o", exe])
        out = _run([exe], env=ENV)
    assert out.stdout.strip().endswith("OK"), out.stdout
    assert "runtime error" not in out.stderr


def test_abi_host_paths_under_asan_ubsan():
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    others = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD)
                    if f.endswith(".o") and f != "moe_api.o") if os.path.isdir(BUILD) else []
    if not others:
        pytest.fail("no library objects: build with `python -m routing_expert_grouped_amd.build`")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    with tempfile.TemporaryDirectory() as d:
        api = os.path.join(d, "moe_api.o")
        drv_src = os.path.join(d, "drv.cpp")
        drv = os.path.join(d, "drv.o")
        exe = os.path.join(d, "drv")
        with open(drv_src, "w") as f:
            f.write(ABI_DRIVER)
        _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
              "-c", os.path.join(CSRC, "moe_api.hip"), "-o", api])
        _run([hipcc, "--cuda-host-only", "-O1", "-g", "-std=c++17", *san,
              "-I", os.path.join(ROOT, "include"), "-c", drv_src, "-o", drv])
        _run([hipcc, "--offload-arch=gfx950", *san[:4], api, drv, *others, "-o", exe])
        out = _run([exe], env=ENV)
    assert out.stdout.startswith("OK"), out.stdout
    assert "runtime error" not in out.stderr
