// Host-side exhaustive check of the HIP library's codec arithmetic (aq_device.hpp) against the
// CPU oracle (liboracle.so, loaded with dlopen).  Test code: it runs on the CPU only and launches
// nothing on a GPU.  Prints one line per check and exits non-zero on the first mismatch.
#include <dlfcn.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "aq_device.hpp"

typedef float (*f_ff)(float, float);
typedef float (*f_f)(float);

static int fail(const char *what, float a, float b, float got, float want) {
  printf("FAIL %s: in (%.9g, %.9g) got %.9g want %.9g\n", what, a, b, got, want);
  return 1;
}

int main(int argc, char **argv) {
  if (argc < 2) { printf("usage: codec_check liboracle.so\n"); return 2; }
  void *h = dlopen(argv[1], RTLD_NOW);
  if (!h) { printf("dlopen: %s\n", dlerror()); return 2; }
  f_f o_e4m3 = (f_f)dlsym(h, "oracle_e4m3");
  f_f o_e2m1 = (f_f)dlsym(h, "oracle_e2m1");
  f_ff o_scale = (f_ff)dlsym(h, "oracle_block_scale");
  f_ff o_val = (f_ff)dlsym(h, "oracle_fq_value");
  if (!o_e4m3 || !o_e2m1 || !o_scale || !o_val) { printf("missing oracle symbol\n"); return 2; }
  int bad = 0;

  // 1. div6 equals the IEEE quotient for every fp32 a >= 2^-120 (below, the quotient and the
  //    Markstein residual lose bits to underflow), and the block scale E4M3(a/6) is right for
  //    every non-negative finite fp32 (the small ones all give the scale 0).
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 16)
  for (int64_t u = 0; u < 0x7F800000LL; ++u) {
    float a = aq::u2f((uint32_t)u);
    float w = a / 6.0f;
    if (u >= 0x03800000LL && aq::div6(a) != w) bad += (bad == 0) ? fail("div6", a, 6, aq::div6(a), w) : 1;
    if (aq::round_e4m3(aq::div6(a)) != aq::round_e4m3(w))
      bad += (bad == 0) ? fail("e4m3(div6) subnormal", a, 6, aq::div6(a), w) : 1;
  }
  printf("div6: %s\n", bad ? "MISMATCH" : "ok");
  if (bad) return 1;

  // 2. Markstein quotient x / S for the 8 significands of E4M3 scales, x over 11 binades
  //    (quotients from 2^-5 to 2^7); the computation is invariant under power-of-two scaling.
  for (int m = 0; m < 8; ++m) {
    float S = 1.0f + m / 8.0f, inv = 1.0f / S;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 16)
    for (int64_t u = aq::f2u(0.0625f); u < (int64_t)aq::f2u(128.0f); ++u) {
      float x = aq::u2f((uint32_t)u);
      float w = x / S;
      if (aq::div_e4m3(x, S, inv) != w) bad += (bad == 0) ? fail("div_e4m3", x, S, aq::div_e4m3(x, S, inv), w) : 1;
    }
  }
  printf("div_e4m3: %s\n", bad ? "MISMATCH" : "ok");
  if (bad) return 1;

  // 3. E4M3 rounding for every fp32 in [0, 2^10) against the oracle's nearest-value search,
  //    sampled densely (every 7th bit pattern) plus every value within 4 ulps of an E4M3
  //    value or midpoint.
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 14)
  for (int64_t u = 0; u < (int64_t)aq::f2u(1024.0f); u += 7) {
    float v = aq::u2f((uint32_t)u);
    float w = o_e4m3(v);
    if (aq::round_e4m3(v) != w) bad += (bad == 0) ? fail("round_e4m3", v, 0, aq::round_e4m3(v), w) : 1;
  }
  for (int code = 0; code < 127; ++code) {
    int e = code >> 3, mm = code & 7;
    float lo = e ? ldexpf(1.0f + mm / 8.0f, e - 7) : ldexpf((float)mm, -9);
    float hi = (code == 126) ? 480.0f : ((code + 1) >> 3 ? ldexpf(1.0f + ((code + 1) & 7) / 8.0f, ((code + 1) >> 3) - 7)
                                                          : ldexpf((float)(code + 1), -9));
    float pts[2] = {lo, (lo + hi) * 0.5f};
    for (float p : pts)
      for (int d = -4; d <= 4; ++d) {
        int64_t uu = (int64_t)aq::f2u(p) + d;
        if (uu < 0) continue;
        float v = aq::u2f((uint32_t)uu);
        if (aq::round_e4m3(v) != o_e4m3(v)) bad += (bad == 0) ? fail("round_e4m3", v, 0, aq::round_e4m3(v), o_e4m3(v)) : 1;
      }
  }
  printf("round_e4m3: %s\n", bad ? "MISMATCH" : "ok");
  if (bad) return 1;

  // 4. E2M1 rounding for every fp32 in [0, 16).
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 16)
  for (int64_t u = 0; u < (int64_t)aq::f2u(16.0f); ++u) {
    float r = aq::u2f((uint32_t)u);
    float w = o_e2m1(r);
    if (aq::round_e2m1(r) != w) bad += (bad == 0) ? fail("round_e2m1", r, 0, aq::round_e2m1(r), w) : 1;
  }
  printf("round_e2m1: %s\n", bad ? "MISMATCH" : "ok");
  if (bad) return 1;

  // 4b. The Newton step recovers fp32(1/S) from any start within 2 ulps, for every positive
  //     E4M3 value S (the device seeds it with the hardware reciprocal).
  for (int code = 1; code < 127; ++code) {
    int e = code >> 3, mm = code & 7;
    float S = e ? ldexpf(1.0f + mm / 8.0f, e - 7) : ldexpf((float)mm, -9);
    float want = 1.0f / S;
    for (int d = -2; d <= 2; ++d) {
      float y0 = aq::u2f(aq::f2u(want) + d);
      if (aq::newton_recip(S, y0) != want) bad += (bad == 0) ? fail("newton_recip", S, y0, aq::newton_recip(S, y0), want) : 1;
    }
  }
  printf("newton_recip: %s\n", bad ? "MISMATCH" : "ok");
  if (bad) return 1;

  // 5. Unit-scale fake quantization end to end: every bf16 amax and every bf16 x with
  //    |x| <= amax, against the oracle's block scale and element rule.
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 64)
  for (int ia = 0; ia < 0x7F80; ++ia) {
    float amax = aq::u2f((uint32_t)ia << 16);
    float S = aq::block_scale_unit(amax);
    float Sw = o_scale(amax, 1.0f);
    if (S != Sw) { bad += (bad == 0) ? fail("block_scale_unit", amax, 0, S, Sw) : 1; continue; }
    float inv = S == 0.0f ? 0.0f : 1.0f / S;
    for (int ix = 0; ix <= ia; ++ix)
      for (int sgn = 0; sgn < 2; ++sgn) {
        float x = aq::u2f(((uint32_t)ix << 16) | (sgn ? 0x80000000u : 0));
        float got = aq::fq_unit(x, S, inv), want = o_val(x, Sw);
        if (aq::f2u(got) != aq::f2u(want)) bad += (bad == 0) ? fail("fq_unit", amax, x, got, want) : 1;
      }
  }
  printf("fq_unit (all bf16 amax, x): %s\n", bad ? "MISMATCH" : "ok");
  return bad ? 1 : 0;
}
