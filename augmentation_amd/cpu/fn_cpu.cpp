// fn_cpu.cpp -- FusedNormalization on the host CPU with SSE4.1 and F16C, the
// way page "(11) FusedNormalization" runs it: one image at a time per
// worker thread, the flip decision first, each row mirrored (pixel order,
// channels kept) and normalized as x * mul - sub in fp32 vectors (section
// 7), converted to fp16 with round to nearest even by F16C (section 6),
// optionally padded to 4 channels (section 8), and the RandomErasing
// rectangle drawn after the flip and zeroed over the output once the pass
// is done (sections 5 and 12).  Decisions follow the same readings as the
// GPU library, so both produce the same flip bits and rectangles.
//
// This is a host comparison path for measurements and tests: the GPU
// library never calls it, and it never calls the GPU library.
#include <immintrin.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <system_error>
#include <thread>
#include <vector>

#include "fn_cpu.h"

#define FNC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// the last error message of this thread (a fixed buffer: recording an error
// never allocates)
thread_local char g_error[256];

int fail(int code, const char* msg) {
  snprintf(g_error, sizeof(g_error), "%s", msg);
  return code;
}

// ---------------------------------------------------------------------------
// Decisions (page section 10: every random number a pure function of seed
// and offset; section 12: the rectangle sampler).
// ---------------------------------------------------------------------------

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).
void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t pa = (uint64_t)0xD2511F53u * c[0];
    const uint64_t pb = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(pb >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(pa >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)pb;
    c[3] = (uint32_t)pa;
    c[0] = n0;
    c[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Sequential reader of sample n's word stream: word k is output k % 4 of
// the block with counter (k / 4, n) under key seed.
struct Stream {
  uint64_t seed, n, block = 0;
  uint32_t buf[4];
  int used = 4;
  uint32_t next() {
    if (used == 4) {
      buf[0] = (uint32_t)block;
      buf[1] = (uint32_t)(block >> 32);
      buf[2] = (uint32_t)n;
      buf[3] = (uint32_t)(n >> 32);
      philox(buf, (uint32_t)seed, (uint32_t)(seed >> 32));
      ++block;
      used = 0;
    }
    return buf[used++];
  }
};

float unit(uint32_t w) { return (float)(w >> 8) * 0x1p-24f; }

int32_t randint_incl(int32_t lo, int32_t hi, uint32_t w) {
  return lo + (int32_t)(((uint64_t)w * (uint64_t)((int64_t)hi - lo + 1)) >> 32);
}

// exp rounded once to fp32 from x87 extended precision.
float exp_f32(float L) { return (float)expl((long double)L); }

// Nearest integer, halves away from zero, of a non-negative float; values
// at or beyond 2^31 become INT32_MAX (never a valid side).
int32_t round_away(float s) {
  if (!(s < 0x1p31f)) return INT32_MAX;
  const float whole = truncf(s);
  return (int32_t)whole + (s - whole >= 0.5f ? 1 : 0);
}

struct Draw {
  float scale_min, scale_max, log_rmin, log_rmax, img_area;
  float flip_p, erase_p;
  int32_t H, W;
};

void draw_sample(const Draw& d, uint64_t seed, uint64_t n, fn_cpu_sample_params* p) {
  Stream s{seed, n, 0, {0, 0, 0, 0}, 4};
  memset(p, 0, sizeof(*p));
  p->attempt = -1;
  int32_t words = 0;
  if (d.flip_p > 0.0f) {
    p->flip = unit(s.next()) < d.flip_p;
    ++words;
  }
  if (d.erase_p > 0.0f) {
    ++words;
    if (unit(s.next()) < d.erase_p) {
      for (int a = 0; a < 10; ++a) {
        // every float operation rounded on its own, as written on the page
        const float span = d.scale_max - d.scale_min;
        const float part = unit(s.next()) * span;
        const float fraction = d.scale_min + part;
        const float area = fraction * d.img_area;
        const float lspan = d.log_rmax - d.log_rmin;
        const float lpart = unit(s.next()) * lspan;
        const float ratio = exp_f32(d.log_rmin + lpart);
        words += 2;
        const float hh = area * ratio;
        const float ww = area / ratio;
        const int32_t eh = round_away(sqrtf(hh));
        const int32_t ew = round_away(sqrtf(ww));
        if (eh > 0 && ew > 0 && eh < d.H && ew < d.W) {
          p->i = randint_incl(0, d.H - eh, s.next());
          p->j = randint_incl(0, d.W - ew, s.next());
          words += 2;
          p->eh = eh;
          p->ew = ew;
          p->erase = 1;
          p->attempt = a;
          break;
        }
      }
    }
  }
  p->words_used = words;
}

// ---------------------------------------------------------------------------
// Pixels.
// ---------------------------------------------------------------------------

uint16_t half_rne(float v) {  // F16C, round to nearest even
  return (uint16_t)_mm_extract_epi16(_mm_cvtps_ph(_mm_set_ss(v), _MM_FROUND_TO_NEAREST_INT), 0);
}

struct Consts {
  int C, oc;       // channels in, channels out (4 when padded)
  int out;         // FN_CPU_OUT_*
  bool page_form;  // x * mul - sub in fp32 stores the accurate result for every byte
  float mul[4], sub[4];
  double mul_d[4], sub_d[4];
  // the fp32 constants of 4 consecutive output elements starting at element
  // 4 q (channel (4 q + l) mod oc of lane l); pad lanes multiply by 0
  __m128 mulv[4], subv[4];
};

// The accurate value of byte x in channel c: evaluated in double and rounded
// once to fp32.
float accurate(const Consts& k, int x, int c) {
  return (float)((double)x * k.mul_d[c] - k.sub_d[c]);
}

float page_value(const Consts& k, int x, int c) {
  const float prod = (float)x * k.mul[c];
  return prod - k.sub[c];
}

// Normalized elements [0, count) of one output row from its bytes in output
// order (`src`, C or, padded, 4 bytes per pixel), into `dst`.
void normalize_row(const Consts& k, const uint8_t* src, int64_t count, void* dst) {
  float* d32 = static_cast<float*>(dst);
  uint16_t* d16 = static_cast<uint16_t*>(dst);
  int64_t e = 0;
  if (k.page_form) {
    const int period = k.oc == 3 ? 3 : 1;  // 4-element groups before the channel pattern repeats
    for (int q = 0; e + 16 <= count; e += 16) {
      const __m128i bytes = _mm_loadu_si128(reinterpret_cast<const __m128i*>(src + e));
      __m128 v[4];
      for (int g = 0; g < 4; ++g) {
        const __m128i w = g == 0 ? _mm_cvtepu8_epi32(bytes)
                        : g == 1 ? _mm_cvtepu8_epi32(_mm_srli_si128(bytes, 4))
                        : g == 2 ? _mm_cvtepu8_epi32(_mm_srli_si128(bytes, 8))
                                 : _mm_cvtepu8_epi32(_mm_srli_si128(bytes, 12));
        const int p = (q + g) % period;
        v[g] = _mm_sub_ps(_mm_mul_ps(_mm_cvtepi32_ps(w), k.mulv[p]), k.subv[p]);
      }
      q = (q + 4) % period;
      if (k.out == FN_CPU_OUT_FP32) {
        for (int g = 0; g < 4; ++g) _mm_storeu_ps(d32 + e + 4 * g, v[g]);
      } else {
        for (int g = 0; g < 4; g += 2) {
          const __m128i lo = _mm_cvtps_ph(v[g], _MM_FROUND_TO_NEAREST_INT);
          const __m128i hi = _mm_cvtps_ph(v[g + 1], _MM_FROUND_TO_NEAREST_INT);
          _mm_storeu_si128(reinterpret_cast<__m128i*>(d16 + e + 4 * g), _mm_unpacklo_epi64(lo, hi));
        }
      }
    }
  }
  for (; e < count; ++e) {  // the tail, and every element when the page form is not exact
    const int c = (int)(e % k.oc);
    float y;
    if (c >= k.C)
      y = 0.0f;
    else
      y = k.page_form ? page_value(k, src[e], c) : accurate(k, src[e], c);
    if (k.out == FN_CPU_OUT_FP32)
      d32[e] = y;
    else
      d16[e] = half_rne(y);
  }
}

// Bytes of one output row in output order (mirrored pixels when flipped,
// channels kept; each pixel padded to oc bytes with zeros) from its source
// row, P pixels per byte shuffle: P*C source bytes b0 .. b0+P*C-1 become P*oc
// output bytes.  A 16-byte load starts at b0 when that stays inside the row,
// else it ends at the block's last byte; the masks below index the loaded
// vector from either start.  Pixels no load can reach from inside the row
// are copied one at a time.
struct Gather {
  int C, oc, P;
  __m128i mask[2][2];  // [flip][load ends at the block's end]
  Gather(int C_, int oc_) : C(C_), oc(oc_), P(oc_ == 3 ? 4 : 16 / oc_) {
    for (int f = 0; f < 2; ++f)
      for (int e = 0; e < 2; ++e) {
        alignas(16) int8_t m[16];
        const int shift = e ? 16 - P * C : 0;  // vector index of byte b0
        for (int t = 0; t < 16; ++t) {
          const int p = t / oc, c = t % oc;
          m[t] = (p < P && c < C) ? (int8_t)(shift + (f ? P - 1 - p : p) * C + c) : (int8_t)0x80;
        }
        mask[f][e] = _mm_load_si128(reinterpret_cast<const __m128i*>(m));
      }
  }
  void row(const uint8_t* src, int32_t W, bool flip, uint8_t* dst) const {
    const int64_t row_bytes = (int64_t)W * C;
    int32_t w = 0;
    for (; w + P <= W; w += P) {
      const int64_t b0 = (int64_t)(flip ? W - w - P : w) * C;
      int e;
      int64_t at;
      if (b0 + 16 <= row_bytes) {
        e = 0;
        at = b0;
      } else if (b0 + P * C - 16 >= 0) {
        e = 1;
        at = b0 + P * C - 16;
      } else {
        break;
      }
      const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i*>(src + at));
      _mm_storeu_si128(reinterpret_cast<__m128i*>(dst + (int64_t)w * oc),
                       _mm_shuffle_epi8(v, mask[flip][e]));
    }
    for (; w < W; ++w) {
      const uint8_t* px = src + (int64_t)(flip ? W - 1 - w : w) * C;
      for (int c = 0; c < oc; ++c) dst[(int64_t)w * oc + c] = c < C ? px[c] : 0;
    }
  }
};

struct Job {
  const uint8_t* in;
  void* out;
  int64_t n_begin, n_end;
  int32_t H, W;
  uint64_t seed;
  int64_t first_sample_id;
  const Draw* draw;
  const Consts* k;
  const Gather* gather;
  fn_cpu_sample_params* params;  // may be null
  uint8_t* rowbuf;               // one output row in output order, plus 32 bytes
};

void run_job(const Job& j) {
  const Consts& k = *j.k;
  const int C = k.C, oc = k.oc;
  const int64_t in_row = (int64_t)j.W * C, out_row = (int64_t)j.W * oc;
  const int esz = k.out == FN_CPU_OUT_FP32 ? 4 : 2;
  for (int64_t n = j.n_begin; n < j.n_end; ++n) {
    fn_cpu_sample_params P;
    draw_sample(*j.draw, j.seed, (uint64_t)(j.first_sample_id + n), &P);
    if (j.params) j.params[n] = P;
    const uint8_t* img = j.in + n * (int64_t)j.H * in_row;
    uint8_t* outb = static_cast<uint8_t*>(j.out) + n * (int64_t)j.H * out_row * esz;
    for (int32_t h = 0; h < j.H; ++h) {
      const uint8_t* row = img + (int64_t)h * in_row;
      const uint8_t* src = row;
      if (P.flip || oc != C) {  // bytes in output order: mirrored pixels and/or padding
        j.gather->row(row, j.W, P.flip != 0, j.rowbuf);
        src = j.rowbuf;
      }
      normalize_row(k, src, out_row, outb + (int64_t)h * out_row * esz);
    }
    if (P.erase) {  // the rectangle, zeroed over the finished output (+0)
      for (int32_t h = P.i; h < P.i + P.eh; ++h)
        memset(outb + ((int64_t)h * out_row + (int64_t)P.j * oc) * esz, 0,
               (size_t)P.ew * oc * esz);
    }
  }
}

}  // namespace

FNC_EXPORT const char* fn_cpu_last_error(void) { return g_error; }

FNC_EXPORT int fn_cpu_fused_normalize(const uint8_t* in, int64_t N, int32_t H, int32_t W,
                                      int32_t C, const float* mean, const float* std, float flip_p,
                                      float erase_p, float scale_min, float scale_max,
                                      float ratio_min, float ratio_max, uint64_t seed,
                                      int64_t first_sample_id, int32_t out_dtype, void* out,
                                      fn_cpu_sample_params* params, int32_t threads) {
  g_error[0] = '\0';
  if (H <= 0 || W <= 0 || C < 1 || C > 4 || N < 0) return fail(FN_CPU_EINVAL, "bad shape");
  if ((int64_t)H * W > ((int64_t)1 << 24)) return fail(FN_CPU_EINVAL, "H*W exceeds 2^24");
  if (!(flip_p >= 0.0f && flip_p <= 1.0f) || !(erase_p >= 0.0f && erase_p <= 1.0f))
    return fail(FN_CPU_EINVAL, "probabilities must be in [0, 1]");
  if (!(scale_min >= 0x1p-30f && scale_min <= scale_max && scale_max <= 1.0f) ||
      !(ratio_min >= 0x1p-30f && ratio_min <= ratio_max && ratio_max <= 0x1p30f))
    return fail(FN_CPU_EINVAL, "scale or ratio range out of its domain");
  if (out_dtype != FN_CPU_OUT_FP32 && out_dtype != FN_CPU_OUT_FP16 &&
      out_dtype != FN_CPU_OUT_FP16_PAD4)
    return fail(FN_CPU_EINVAL, "unknown out_dtype");
  if (first_sample_id < 0) return fail(FN_CPU_EINVAL, "first_sample_id must be >= 0");
  if (N > INT64_MAX / 16 / ((int64_t)H * W)) return fail(FN_CPU_EINVAL, "N*H*W*16 overflows int64");
  if (N == 0) return 0;
  if (!in || !out || !mean || !std) return fail(FN_CPU_EINVAL, "NULL pointer");
  for (int c = 0; c < C; ++c)
    if (!isfinite(mean[c]) || !(std[c] > 0.0f) || !isfinite(std[c]))
      return fail(FN_CPU_EINVAL, "mean must be finite and std positive and finite");

  Consts k{};
  k.C = C;
  k.oc = out_dtype == FN_CPU_OUT_FP16_PAD4 ? 4 : C;
  k.out = out_dtype;
  for (int c = 0; c < C; ++c) {
    k.mul_d[c] = 1.0 / (255.0 * (double)std[c]);
    k.sub_d[c] = (double)mean[c] / (double)std[c];
    k.mul[c] = (float)k.mul_d[c];
    k.sub[c] = (float)k.sub_d[c];
  }
  // the page's fp32 form where, for every byte of every channel, it stores
  // the same bits as the accurate value; the double evaluation elsewhere
  k.page_form = true;
  for (int c = 0; c < C && k.page_form; ++c)
    for (int x = 0; x < 256 && k.page_form; ++x) {
      const float a = accurate(k, x, c), p = page_value(k, x, c);
      k.page_form = out_dtype == FN_CPU_OUT_FP32 ? fabsf(a - p) <= 1e-6f
                                                  : half_rne(a) == half_rne(p);
    }
  for (int q = 0; q < 4; ++q) {
    float m[4], s[4];
    for (int l = 0; l < 4; ++l) {
      const int c = (4 * q + l) % k.oc;
      m[l] = c < C ? k.mul[c] : 0.0f;
      s[l] = c < C ? k.sub[c] : 0.0f;
    }
    k.mulv[q] = _mm_loadu_ps(m);
    k.subv[q] = _mm_loadu_ps(s);
  }
  Draw d{scale_min, scale_max, (float)logl((long double)ratio_min),
         (float)logl((long double)ratio_max), (float)H * (float)W, flip_p, erase_p, H, W};

  const Gather gather(C, k.oc);
  const int T = (int)std::max<int64_t>(1, std::min<int64_t>(threads, N));
  // everything that can fail is obtained before any output is written
  std::vector<Job> jobs;
  std::vector<std::vector<uint8_t>> rowbufs;
  std::vector<std::thread> pool;
  try {
    jobs.resize(T);
    rowbufs.resize(T);
    for (auto& b : rowbufs) b.resize((size_t)(W * (int64_t)k.oc) + 32);
    pool.reserve(T);
  } catch (const std::bad_alloc&) {
    return fail(FN_CPU_ENOMEM, "out of host memory");
  }
  for (int t = 0; t < T; ++t)
    jobs[t] = Job{in, out, (int64_t)((__int128)N * t / T), (int64_t)((__int128)N * (t + 1) / T),
                  H, W, seed, first_sample_id, &d, &k, &gather, params, rowbufs[t].data()};
  int started = 0;
  if (T > 1) {
    for (; started < T; ++started) {
      try {
        pool.emplace_back(run_job, std::cref(jobs[started]));
      } catch (const std::system_error&) {
        break;  // no more threads: the calling thread does the rest
      }
    }
  }
  for (int t = started; t < T; ++t) run_job(jobs[t]);
  for (auto& th : pool) th.join();
  return 0;
}
