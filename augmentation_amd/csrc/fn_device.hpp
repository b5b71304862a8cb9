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
    const uint32_t hi_a = __umulhi(kMulA, c0), lo_a = kMulA * c0;
    const uint32_t hi_b = __umulhi(kMulB, c2), lo_b = kMulB * c2;
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

// Inclusive randint(lo, hi) from one word, multiply-shift.
__device__ __forceinline__ int32_t word_randint(int32_t lo, int32_t hi, uint32_t w) {
  const uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
  return lo + (int32_t)(((uint64_t)w * span) >> 32);
}

// ---------------------------------------------------------------------------
// Correctly rounded fp32 exp for |L| <= 80, integer fixed point.
//   L is converted exactly to Q96; k = floor(L / ln 2) and r = L - k ln 2 in
//   [0, ln 2) use ln 2 to 96 fraction bits; e^r comes from its Taylor series
//   to the 1/19! term by Horner's rule in Q62 with r in Q64; the result is
//   rounded to 24 bits (nearest even) and scaled by 2^k.
//   Error of e^r before rounding: below 5 units of 2^-62 from the Horner
//   truncations and coefficient roundings (each step's error is damped by
//   r < 0.7), 2^-71 from the series tail, 2^-64 from truncating r: relative
//   error < 2^-59.5.  The rounding is therefore correct whenever e^L is not
//   within 2^-59.5 (relative) of a midpoint between two floats.
// ---------------------------------------------------------------------------
constexpr uint64_t factorial(int j) { return j <= 1 ? 1ull : (uint64_t)j * factorial(j - 1); }
// round(2^62 / j!)
constexpr uint64_t inv_factorial_q62(int j) {
  return ((1ull << 62) + factorial(j) / 2) / factorial(j);
}

__device__ __forceinline__ float cr_expf(float L) {
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

  const __int128 kLn2Q96 = ((__int128)0xB17217F7ull << 64) | (__int128)0xD1CF79ABC9E3B398ull;
  int k = (int)__builtin_floorf(L * 1.44269504f);  // estimate, fixed up below
  __int128 r = lq - (__int128)k * kLn2Q96;
#pragma unroll
  for (int fix = 0; fix < 2; ++fix) {
    if (r < 0) {
      r += kLn2Q96;
      --k;
    } else if (r >= kLn2Q96) {
      r -= kLn2Q96;
      ++k;
    }
  }
  const uint64_t r64 = (uint64_t)(r >> 32);  // r in Q64, r < ln 2

  uint64_t p = inv_factorial_q62(19);
#pragma unroll
  for (int j = 18; j >= 0; --j) p = inv_factorial_q62(j) + __umul64hi(p, r64);
  // p = e^r in Q62, in [2^62, 2^63): keep 24 bits, round to nearest even.
  uint64_t m24 = p >> 39;
  const uint64_t rest = p & ((1ull << 39) - 1);
  const uint64_t half = 1ull << 38;
  if (rest > half || (rest == half && (m24 & 1))) ++m24;
  if (m24 == (1ull << 24)) {
    m24 >>= 1;
    ++k;
  }
  return __uint_as_float(((uint32_t)(k + 127) << 23) | ((uint32_t)m24 & 0x7FFFFFu));
}

// ---------------------------------------------------------------------------
// Correctly rounded fp32 sqrt of a positive normal float, integer arithmetic:
// the mantissa is scaled to M in [2^48, 2^50) with an even exponent, q =
// floor(sqrt(M)) has exactly 25 bits; the 25th bit is the rounding bit (an
// exact tie is impossible for a square root).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t isqrt_u50(uint64_t M) {
  uint64_t q = (uint64_t)__builtin_sqrt((double)M);  // estimate; M < 2^53 converts exactly
#pragma unroll
  for (int fix = 0; fix < 3; ++fix) {
    if (q * q > M) --q;
  }
#pragma unroll
  for (int fix = 0; fix < 3; ++fix) {
    if ((q + 1) * (q + 1) <= M) ++q;
  }
  return q;
}

__device__ __forceinline__ float cr_sqrtf(float x) {
  const uint32_t bits = __float_as_uint(x);
  const int e = (int)(bits >> 23) - 150;  // x = m * 2^e
  const uint64_t m = (bits & 0x7FFFFFu) | 0x800000u;
  uint64_t M;
  int f;  // sqrt(x) = sqrt(M) * 2^f
  if (e & 1) {
    M = m << 25;
    f = (e - 25) / 2;
  } else {
    M = m << 26;
    f = (e - 26) / 2;
  }
  const uint64_t q = isqrt_u50(M);  // [2^24, 2^25)
  uint32_t mant = (uint32_t)(q >> 1);
  int exp2 = f + 1;                 // value = mant * 2^exp2
  if (q & 1) ++mant;
  if (mant == (1u << 24)) {
    mant >>= 1;
    ++exp2;
  }
  return __uint_as_float(((uint32_t)(exp2 + 23 + 127) << 23) | (mant & 0x7FFFFFu));
}

// ---------------------------------------------------------------------------
// Correctly rounded fp32 a / b for positive normal a, b with a normal
// quotient, integer long division of the mantissas (an exact tie is
// impossible for a quotient of two floats).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float cr_divf(float a, float b) {
  const uint32_t ab = __float_as_uint(a), bb = __float_as_uint(b);
  const int ea = (int)(ab >> 23), eb = (int)(bb >> 23);
  const uint64_t ma = (ab & 0x7FFFFFu) | 0x800000u, mb = (bb & 0x7FFFFFu) | 0x800000u;
  const uint64_t num = ma << 26;
  const uint64_t Q = num / mb;
  const bool inexact = (num - Q * mb) != 0;
  uint32_t mant;
  bool round_bit, sticky;
  int biased;
  if (Q >= (1ull << 26)) {  // 27 bits
    mant = (uint32_t)(Q >> 3);
    round_bit = (Q >> 2) & 1;
    sticky = (Q & 3) != 0 || inexact;
    biased = ea - eb + 127;
  } else {  // 26 bits
    mant = (uint32_t)(Q >> 2);
    round_bit = (Q >> 1) & 1;
    sticky = (Q & 1) != 0 || inexact;
    biased = ea - eb + 126;
  }
  if (round_bit && (sticky || (mant & 1))) ++mant;
  if (mant == (1u << 24)) {
    mant >>= 1;
    ++biased;
  }
  return __uint_as_float(((uint32_t)biased << 23) | (mant & 0x7FFFFFu));
}

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

// ---------------------------------------------------------------------------
// The decisions of sample n, computed by one whole wavefront (all 64 lanes
// must call it together; every lane gets the result).
//
// The stream is consumed in a fixed order, so the words of attempt a sit at
// a known offset: flip word (if any), gate word, then two words per attempt,
// then two for the corner.  Lane a < 10 evaluates attempt a and the corner
// it would draw, all ten in parallel; the first lane whose rectangle fits is
// the accepted attempt -- the same result as trying them one after another.
// ---------------------------------------------------------------------------
__device__ __forceinline__ SampleParams draw_sample_params(const DrawArgs& a, uint64_t n) {
  const int lane = (int)(threadIdx.x & 63u);
  const int has_flip = a.flip_p > 0.0f ? 1 : 0;
  const int has_gate = a.erase_p > 0.0f ? 1 : 0;
  const int first_attempt_word = has_flip + 1;  // the flip word, then the gate word

  const int att = lane < 10 ? lane : 9;
  const int kbase = first_attempt_word + 2 * att;  // area, ratio, row, column words
  const int blk = kbase >> 2;
  const Block4 lo = stream_block(a.seed, n, (uint64_t)blk);
  const Block4 hi = stream_block(a.seed, n, (uint64_t)blk + 1);
  const int o = kbase & 3;
  const uint32_t w_scale = pick_word(lo, hi, o);
  const uint32_t w_ratio = pick_word(lo, hi, o + 1);
  const uint32_t w_row = pick_word(lo, hi, o + 2);
  const uint32_t w_col = pick_word(lo, hi, o + 3);

  const Attempt t = erase_attempt(a, w_scale, w_ratio);
  const int32_t ci = t.fits ? word_randint(0, a.H - t.eh, w_row) : 0;
  const int32_t cj = t.fits ? word_randint(0, a.W - t.ew, w_col) : 0;

  // The flip and gate words are words 0 and 1 of block 0, which lane 0 holds
  // (its first attempt word is word 1 or 2).
  const uint32_t w0 = __shfl(lo.w[0], 0);
  const uint32_t w1 = __shfl(lo.w[1], 0);
  const uint32_t w_flip = w0;
  const uint32_t w_gate = has_flip ? w1 : w0;

  SampleParams p{};
  p.flip = has_flip ? (word_to_unit(w_flip) < a.flip_p ? 1 : 0) : 0;
  p.attempt = -1;
  p.words_used = has_flip + has_gate;
  const bool tried = has_gate && word_to_unit(w_gate) < a.erase_p;
  const uint64_t fits = __ballot(t.fits && lane < 10);
  if (tried) {
    if (fits != 0) {
      const int win = __builtin_ctzll(fits);
      p.erase = 1;
      p.attempt = win;
      p.eh = __shfl(t.eh, win);
      p.ew = __shfl(t.ew, win);
      p.i = __shfl(ci, win);
      p.j = __shfl(cj, win);
      p.words_used += 2 * (win + 1) + 2;
    } else {
      p.words_used += 20;
    }
  }
  return p;
}

}  // namespace fn
