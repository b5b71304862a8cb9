// fn_device.hpp -- device-side building blocks of the per-sample random
// decisions: Philox4x32-10, correctly rounded fp32 exp / sqrt / division in
// integer arithmetic, one erase attempt, and the wave-cooperative draw of a
// sample's flip bit and erase rectangle.
//
// The draw follows the page "(11) FusedNormalization"
// (tech-renaissance.cn/blog/?p=487): section 5 (flip first, rectangle
// second), section 10 (uniform(a, b) = a + r (b - a) from a Philox word),
// section 12 (gate, up to ten attempts of area fraction then log aspect
// ratio, sides rounded, accepted strictly inside the image, then row and
// column of the corner).
//
// Reproducibility: everything that decides a rectangle is either integer
// arithmetic or a correctly rounded fp32 operation, so the decisions are
// bit-identical to any other correct implementation of the same reading.
// This file must be compiled with -ffp-contract=off: the sampler's fp32
// expressions are separately rounded operations, never fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fn {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies whose high
// halves are xored into the other counter words and the key, the key bumped
// by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
struct Block4 {
  uint32_t w[4];
};

__device__ __forceinline__ Block4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32->64 multiply (v_mad_u64_u32) gives both halves
    const uint64_t pa = (uint64_t)kMulA * c0, pb = (uint64_t)kMulB * c2;
    const uint32_t hi_a = (uint32_t)(pa >> 32), lo_a = (uint32_t)pa;
    const uint32_t hi_b = (uint32_t)(pb >> 32), lo_b = (uint32_t)pb;
    const uint32_t n0 = hi_b ^ c1 ^ k0, n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
    k0 += kWeyl0;
    k1 += kWeyl1;
  }
  return Block4{{c0, c1, c2, c3}};
}

// Block `block` of sample n's stream under `seed`: counter (block, n), key seed.
__device__ __forceinline__ Block4 stream_block(uint64_t seed, uint64_t n, uint64_t block) {
  return philox4x32_10((uint32_t)block, (uint32_t)(block >> 32), (uint32_t)n, (uint32_t)(n >> 32),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

// 24-bit uniform in [0, 1): exact.
__device__ __forceinline__ float word_to_unit(uint32_t w) {
  return (float)(w >> 8) * 0x1p-24f;
}

// Inclusive randint(lo, hi) from one word, multiply-shift: lo plus the high
// word of w * (hi - lo + 1).  Requires 0 <= hi - lo < 2^32 - 1.
__device__ __forceinline__ int32_t word_randint(int32_t lo, int32_t hi, uint32_t w) {
  const uint32_t span = (uint32_t)(hi - lo) + 1u;
  return lo + (int32_t)__umulhi(w, span);
}

// ---------------------------------------------------------------------------
// Correctly rounded fp32 exp for |L| <= 80, integer fixed point.
//   L is converted exactly to Q96.  With step = ln 2 / 32 (to 96 fraction
//   bits), k = floor(L / step) and r = L - k step in [0, step); then
//   e^L = 2^(k >> 5) * 2^((k & 31)/32) * e^r.  e^r comes from its Taylor
//   series to the 1/8! term by Horner's rule in Q62 with r in Q64; the table
//   entry 2^(j/32) is the exactly rounded Q62 value; the product is rounded
//   to 24 bits (nearest even).
//   Error before the final rounding: the Horner truncations and coefficient
//   roundings stay below 1.6 units of 2^-62 (each step's error is damped by
//   r < 0.022), the series tail below 2^-68, truncating r to Q64 2^-64, the
//   table entry half a unit and the product's truncation one unit: relative
//   error < 2^-59.8.  The rounding is therefore correct whenever e^L is not
//   within 2^-59.8 (relative) of a midpoint between two floats.
// ---------------------------------------------------------------------------
#include "exp2_table.inc"

// Taylor coefficients, built at compile time: round(2^62 / j!) for the exact
// path and 1/j! rounded to double for the fast path.
struct InvFactorials {
  uint64_t q62[20];
  double dbl[20];
  constexpr InvFactorials() : q62{}, dbl{} {
    uint64_t f = 1;
    for (int j = 0; j < 20; ++j) {
      if (j > 1) f *= (uint64_t)j;
      q62[j] = ((1ull << 62) + f / 2) / f;
      dbl[j] = 1.0 / (double)f;  // j! is exact in double for j <= 18; 1/j! rounded once
    }
  }
};
constexpr InvFactorials kInvFact{};

__device__ __forceinline__ float cr_expf_exact(float L) {
  const float mag = __builtin_fabsf(L);
  if (!(mag <= 80.0f)) return L > 0.0f ? __builtin_inff() : (L < 0.0f ? 0.0f : L);  // outside the domain
  // |L| < 2^-30: e^L rounds to 1 (the nearest midpoints are 1 + 2^-24 and 1 - 2^-25).
  if (!(mag >= 0x1p-30f)) return 1.0f;

  const uint32_t bits = __float_as_uint(L);
  const int biased = (int)((bits >> 23) & 0xFFu);
  const uint32_t mant = (bits & 0x7FFFFFu) | 0x800000u;
  // L = mant * 2^(biased - 150); in Q96 that is mant << (biased - 54), biased in [97, 133].
  __int128 lq = (__int128)mant << (biased - 54);
  if (bits >> 31) lq = -lq;

  const __int128 step = ((__int128)kLn2Over32Q96Hi << 64) | (__int128)kLn2Over32Q96Lo;
  int k = (int)__builtin_floorf(L * 46.1662413f);  // estimate of floor(L / step), fixed up below
  __int128 r = lq - (__int128)k * step;
#pragma unroll
  for (int fix = 0; fix < 2; ++fix) {
    if (r < 0) {
      r += step;
      --k;
    } else if (r >= step) {
      r -= step;
      ++k;
    }
  }
  const uint64_t r64 = (uint64_t)(r >> 32);  // r in Q64, r < ln 2 / 32

  uint64_t p = kInvFact.q62[8];
#pragma unroll
  for (int j = 7; j >= 0; --j) p = kInvFact.q62[j] + __umul64hi(p, r64);
  // m = 2^((k & 31)/32) * e^r in Q62, in [2^62, 2^64)
  const uint64_t t = kExp2Q62[k & 31];
  const uint64_t m = (__umul64hi(t, p) << 2) | ((t * p) >> 62);
  int e = k >> 5;  // floor(k / 32)
  int shift = 39;
  if (m >> 63) {
    shift = 40;
    ++e;
  }
  uint64_t m24 = m >> shift;
  const uint64_t rest = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rest > half || (rest == half && (m24 & 1))) ++m24;
  if (m24 == (1ull << 24)) {
    m24 >>= 1;
    ++e;
  }
  return __uint_as_float(((uint32_t)(e + 127) << 23) | ((uint32_t)m24 & 0x7FFFFFu));
}

// ---------------------------------------------------------------------------
// Correctly rounded fp32 exp, fast path first (the usual scheme for correct
// rounding: a cheap approximation with a proven error bound, and the exact
// evaluation only when that bound cannot decide the rounding).  The fast
// path touches no memory (a table lookup would cost a memory latency at the
// start of every work-group).
//   In double: k = round(L / ln 2), r = L - k ln 2 by a Cody-Waite pair
//   (k*hi is exact for |k| < 2^11 and so is L - k*hi; the low term adds at
//   most 2^-56 relative), |r| <= 0.35, e^r by its degree-14 Taylor polynomial
//   (tail below 2^-57), scaled by 2^k.  Relative error below 3 units of
//   2^-53 < 2^-50.
//   The result y rounds to f; if no fp32 rounding midpoint lies within
//   y * 2^-50 of y, the true value rounds to f as well.  Otherwise (about
//   one argument in 2^25) the exact fixed-point evaluation above decides.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float cr_expf(float L) {
  const float mag = __builtin_fabsf(L);
  if (!(mag <= 80.0f) || !(mag >= 0x1p-30f)) return cr_expf_exact(L);
  const double x = (double)L;
  const double kd = __builtin_rint(x * 1.4426950408889634);  // 1 / ln 2
  double r = __builtin_fma(-kd, kLn2Hi, x);
  r = __builtin_fma(-kd, kLn2Lo, r);
  double p = kInvFact.dbl[14];
#pragma unroll
  for (int j = 13; j >= 0; --j) p = __builtin_fma(p, r, kInvFact.dbl[j]);
  const double y = __builtin_ldexp(p, (int)kd);
  const float f = (float)y;  // nearest even
  const uint32_t fb = __float_as_uint(f);
  const double ulp = __builtin_ldexp(1.0, (int)((fb >> 23) & 0xFFu) - 150);
  double mid;
  if (y >= (double)f)
    mid = (double)f + 0.5 * ulp;
  else
    mid = (double)f - ((fb & 0x7FFFFFu) == 0 ? 0.25 : 0.5) * ulp;  // spacing halves below a power of 2
  const double dist = __builtin_fabs(y - mid);
  if (dist > y * 0x1p-50) return f;
  return cr_expf_exact(L);
}

// Correctly rounded fp32 square root and division: the compiler's IEEE
// sequences for sqrtf and '/' (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt and without fast-math flags).
__device__ __forceinline__ float cr_sqrtf(float x) { return __builtin_sqrtf(x); }
__device__ __forceinline__ float cr_divf(float a, float b) { return a / b; }

// Round half away from zero of a non-negative float, as an integer; values
// at or beyond 2^31 come back as INT32_MAX (never accepted as a side; below
// 2^31 the result is at most 2^31 - 127).
__device__ __forceinline__ int32_t round_half_away(float s) {
  if (!(s < 0x1p31f)) return INT32_MAX;
  const float whole = __builtin_truncf(s);
  const float frac = s - whole;  // exact: whole >= s/2 or whole == 0
  return (int32_t)whole + (frac >= 0.5f ? 1 : 0);
}

// ---------------------------------------------------------------------------
// The sampler's arguments, prepared once on the host.
// ---------------------------------------------------------------------------
struct DrawArgs {
  uint64_t seed;
  uint64_t first_sample;     // sample n of a call draws from stream first_sample + n
  int32_t H, W;
  float flip_p, erase_p;
  float scale_min, scale_max;
  float log_rmin, log_rmax;  // RN32(ln ratio_min), RN32(ln ratio_max)
  float img_area;            // fl(H) * fl(W), exact for H*W <= 2^24
};

struct Attempt {
  int32_t eh, ew;
  bool fits;
};

// One erase attempt from its area word and log-ratio word (page section 12):
// t = smin + u (smax - smin); area = t * img_area; L = lmin + u' (lmax - lmin);
// ar = exp(L); sides round(sqrt(area * ar)), round(sqrt(area / ar)).
__device__ __forceinline__ Attempt erase_attempt(const DrawArgs& a, uint32_t w_scale,
                                                 uint32_t w_ratio) {
  const float scale_span = a.scale_max - a.scale_min;
  const float fraction = a.scale_min + word_to_unit(w_scale) * scale_span;
  const float area = fraction * a.img_area;
  const float log_span = a.log_rmax - a.log_rmin;
  const float log_aspect = a.log_rmin + word_to_unit(w_ratio) * log_span;
  const float aspect = cr_expf(log_aspect);
  const int32_t eh = round_half_away(cr_sqrtf(area * aspect));
  const int32_t ew = round_half_away(cr_sqrtf(cr_divf(area, aspect)));
  return Attempt{eh, ew, eh > 0 && ew > 0 && eh < a.H && ew < a.W};
}

struct SampleParams {
  int32_t flip, erase, i, j, eh, ew, attempt, words_used;
};

// Word `idx` (0..7) of the two consecutive blocks lo, hi.
__device__ __forceinline__ uint32_t pick_word(const Block4& lo, const Block4& hi, int idx) {
  uint32_t v = hi.w[3];
  v = idx == 0 ? lo.w[0] : v;
  v = idx == 1 ? lo.w[1] : v;
  v = idx == 2 ? lo.w[2] : v;
  v = idx == 3 ? lo.w[3] : v;
  v = idx == 4 ? hi.w[0] : v;
  v = idx == 5 ? hi.w[1] : v;
  v = idx == 6 ? hi.w[2] : v;
  return v;
}

// Lane i of a 16-lane row reads `x` from lane i + 2 of the same row (a DPP
// row shift; lanes 14 and 15 keep their own value).
__device__ __forceinline__ uint32_t from_lane_plus2(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x102 /* row_shl:2 */, 0xF, 0xF,
                                               false);
}

// ---------------------------------------------------------------------------
// The decisions of one sample, computed by a group of 16 lanes (lanes
// 16g .. 16g+15 of a wavefront draw for the sample their caller passes --
// stream a.first_sample + n; a
// wavefront serves four samples at once).  Every lane of the wavefront must
// make the call together; the group's first lane (16g) gets the result, the
// other lanes' results are unspecified.
//
// The stream is consumed in a fixed order, so the words of attempt a sit at
// a known offset: flip word (if any), gate word, then two words per attempt,
// then two for the corner.  Lane a < 10 of a group evaluates attempt a and
// the corner it would draw, all ten in parallel; the first lane whose
// rectangle fits is the accepted attempt -- the same result as trying the
// attempts one after another.  Attempt a reads words k .. k+3, k = f + 2a
// (f = 1 + [flip drawn]), which lie in blocks k/4 and k/4 + 1: lane a
// computes block k/4 itself and takes block k/4 + 1 from lane a + 2, which
// computed exactly that block.  The flip and gate words are words 0 and 1,
// in the first lane's own block 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ SampleParams draw_sample_params16(const DrawArgs& a, uint64_t n) {
  const int lane = (int)(threadIdx.x & 63u);
  const int gl = lane & 15;
  const int has_flip = a.flip_p > 0.0f ? 1 : 0;
  const int has_gate = a.erase_p > 0.0f ? 1 : 0;
  const int first_attempt_word = has_flip + 1;  // after the flip word and the gate word
  const int k = first_attempt_word + 2 * gl;

  const Block4 own = stream_block(a.seed, a.first_sample + n, (uint64_t)(k >> 2));
  const uint32_t w0 = own.w[0];  // in the first lane: words 0 and 1 of the stream
  const uint32_t w_gate = has_flip ? own.w[1] : own.w[0];

  Attempt t{0, 0, false};
  int32_t ci = 0, cj = 0;
  if (has_gate) {  // the same for every lane: no attempt is drawn when erasing is off
    Block4 hi;
#pragma unroll
    for (int c = 0; c < 4; ++c) hi.w[c] = from_lane_plus2(own.w[c]);
    const int o = k & 3;
    const uint32_t w_scale = pick_word(own, hi, o);
    const uint32_t w_ratio = pick_word(own, hi, o + 1);
    const uint32_t w_row = pick_word(own, hi, o + 2);
    const uint32_t w_col = pick_word(own, hi, o + 3);
    t = erase_attempt(a, w_scale, w_ratio);
    ci = t.fits ? word_randint(0, a.H - t.eh, w_row) : 0;
    cj = t.fits ? word_randint(0, a.W - t.ew, w_col) : 0;
  }

  // first fitting attempt of each group, its values read into every lane of
  // that group (the lane numbers are wavefront-uniform)
  const uint64_t fits_all = __ballot(t.fits && gl < 10);
  const int grp = lane >> 4;
  uint32_t fits = 0;
  int32_t win_eh = 0, win_ew = 0, win_i = 0, win_j = 0, a_star = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t fg = (uint32_t)(fits_all >> (16 * g)) & 0x3FFu;
    const int ag = fg ? __builtin_ctz(fg) : 0;
    const int src = 16 * g + ag;
    const int32_t eh_g = __builtin_amdgcn_readlane(t.eh, src);
    const int32_t ew_g = __builtin_amdgcn_readlane(t.ew, src);
    const int32_t i_g = __builtin_amdgcn_readlane(ci, src);
    const int32_t j_g = __builtin_amdgcn_readlane(cj, src);
    if (grp == g) {
      fits = fg;
      a_star = ag;
      win_eh = eh_g;
      win_ew = ew_g;
      win_i = i_g;
      win_j = j_g;
    }
  }

  SampleParams p{};
  p.flip = has_flip ? (word_to_unit(w0) < a.flip_p ? 1 : 0) : 0;
  p.attempt = -1;
  p.words_used = has_flip + has_gate;
  const bool tried = has_gate && word_to_unit(w_gate) < a.erase_p;
  if (tried && fits) {
    p.erase = 1;
    p.attempt = a_star;
    p.eh = win_eh;
    p.ew = win_ew;
    p.i = win_i;
    p.j = win_j;
    p.words_used += 2 * (a_star + 1) + 2;
  } else if (tried) {
    p.words_used += 20;
  }
  return p;
}

}  // namespace fn
