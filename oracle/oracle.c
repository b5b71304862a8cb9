/*
 * oracle.c -- plain, slow CPU reference for FusedNormalization.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; the two meet only at the seeded synthetic inputs.
 *
 * What it computes (page "(11) FusedNormalization", tech-renaissance.cn/blog/?p=487):
 *   - section 5 (what is fused): per output pixel, read the source pixel at
 *     the mirrored column when the image is flipped, apply ToTensor (x/255)
 *     then Normalize ((v - mean)/std), write; RandomErasing then zeroes a
 *     rectangle of the output.
 *   - section 5 (execute()): the flip decision is drawn first, the erase
 *     rectangle second, both before the pixel pass.
 *   - section 10 (reproducible randomness): every random number is a pure
 *     function of (seed, offset) through a Philox counter-based generator.
 *   - section 12 (RandomErasing): gate, up to ten attempts of
 *     (area fraction, log aspect ratio), rounding of the side lengths,
 *     acceptance test, then the top-left corner (row first, column second).
 *
 * Precision.  The parameter sampler follows the page's fp32 arithmetic one
 * rounded operation at a time (this file must be built with
 * -ffp-contract=off, on a target whose float evaluation method is 0).  The
 * pixel value is evaluated in double and rounded once to fp32, which is the
 * correctly rounded value of the exact expression.
 *
 * Readings of points the pages leave open (each one is listed with its
 * reason in the design notes):
 *   - Generator stream: word k of sample n is lane k%4 of
 *     Philox4x32-10(counter = {k/4 lo, k/4 hi, n lo, n hi}, key = {seed lo, seed hi}).
 *   - 32-bit word to float: top 24 bits times 2^-24, exact, in [0, 1).
 *   - A feature with probability <= 0 draws no word; flip iff u < flip_p;
 *     erase is attempted iff u < erase_p.
 *   - exp is correctly rounded to fp32 (long double expl, then one rounding);
 *     sqrt and division are IEEE fp32; round() is half away from zero.
 *   - randint(lo, hi) is inclusive of both ends and uses one word:
 *     lo + floor(w * (hi - lo + 1) / 2^32).
 *   - The rectangle is in output (post-flip) coordinates and covers all C
 *     channels; erased elements are +0.0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FLT_EVAL_METHOD__) && __FLT_EVAL_METHOD__ != 0
#error "the oracle needs float expressions evaluated in float"
#endif

typedef struct {
    int32_t flip;       /* 1: the output is the mirrored image            */
    int32_t erase;      /* 1: the rectangle below is zeroed               */
    int32_t i, j;       /* top-left corner (row, column) of the rectangle */
    int32_t eh, ew;     /* rectangle height and width in pixels           */
    int32_t attempt;    /* accepted attempt 0..9, or -1                   */
    int32_t words_used; /* generator words consumed by this sample        */
} or_sample_params;

/* ------------------------------------------------------------------------ */
/* Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As   */
/* Easy as 1, 2, 3", SC'11, section 4 (the Philox S-P network).  One round   */
/* multiplies counter words 0 and 2 by two fixed odd constants; the high     */
/* halves are xored with the other counter words and the key, and the words */
/* are permuted.  The key is bumped by two Weyl constants between rounds.   */
/* ------------------------------------------------------------------------ */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t prod_a = (uint64_t)0xD2511F53u * (uint64_t)x0;
        uint64_t prod_b = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
        uint32_t y0 = (uint32_t)(prod_b >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)prod_b;
        uint32_t y2 = (uint32_t)(prod_a >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)prod_a;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Word k of sample n's stream (reading of page section 10's (seed, offset)). */
uint32_t or_word(uint64_t seed, uint64_t n, uint64_t k)
{
    uint64_t block = k / 4;
    uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), (uint32_t)n, (uint32_t)(n >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    return out[k % 4];
}

/* Uniform float in [0, 1) from one word: top 24 bits, exact. */
float or_u01(uint32_t w)
{
    return (float)(w >> 8) * 0x1p-24f;
}

/* Inclusive randint from one word. */
int32_t or_randint(int32_t lo, int32_t hi, uint32_t w)
{
    uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    return lo + (int32_t)(((uint64_t)w * span) >> 32);
}

/* RN32(ln r): the log-ratio bounds the erase sampler draws between. */
float or_log_ratio(float r)
{
    return (float)logl((long double)r);
}

/* RN32(e^L): correctly rounded exp (long double, then one rounding). */
float or_expf(float L)
{
    return (float)expl((long double)L);
}

/* One erase attempt from its two words (page section 12): area fraction,
 * log aspect ratio, exp, side lengths rounded half away from zero.
 * Writes the rounded sides; returns 1 if the rectangle fits strictly
 * inside the H x W image, 0 otherwise.  Sides that do not fit an int32 are
 * reported as -1 (they are rejected anyway). */
int or_erase_dims(uint32_t w_scale, uint32_t w_ratio, int32_t H, int32_t W,
                  float scale_min, float scale_max, float log_rmin, float log_rmax,
                  int32_t* eh_out, int32_t* ew_out)
{
    const float img_area = (float)H * (float)W;

    float scale_span = scale_max - scale_min;
    float scale_draw = or_u01(w_scale) * scale_span;
    float target_fraction = scale_min + scale_draw;
    float erase_area = target_fraction * img_area;

    float log_span = log_rmax - log_rmin;
    float log_draw = or_u01(w_ratio) * log_span;
    float log_aspect = log_rmin + log_draw;
    float aspect = or_expf(log_aspect);

    float side_h = sqrtf(erase_area * aspect);
    float side_w = sqrtf(erase_area / aspect);
    float eh_f = roundf(side_h);
    float ew_f = roundf(side_w);

    *eh_out = (eh_f < 2147483647.0f) ? (int32_t)eh_f : -1;
    *ew_out = (ew_f < 2147483647.0f) ? (int32_t)ew_f : -1;
    return eh_f > 0.0f && ew_f > 0.0f && eh_f < (float)H && ew_f < (float)W;
}

/* Parameters of one sample from an explicit word stream (the draw order of
 * execute() and generate_erase_rect() on page sections 5 and 12).
 * Returns 0, or -1 if the stream is shorter than the draws need. */
int or_params_from_words(const uint32_t* words, int64_t nwords, int32_t H, int32_t W,
                         float flip_p, float erase_p, float scale_min, float scale_max,
                         float log_rmin, float log_rmax, or_sample_params* p)
{
    int64_t k = 0;
    memset(p, 0, sizeof(*p));
    p->attempt = -1;

    if (flip_p > 0.0f) {
        if (k >= nwords) return -1;
        p->flip = or_u01(words[k++]) < flip_p;
    }
    if (erase_p > 0.0f) {
        if (k >= nwords) return -1;
        if (or_u01(words[k++]) < erase_p) {
            for (int32_t a = 0; a < 10; ++a) {
                if (k + 2 > nwords) return -1;
                int32_t eh, ew;
                int ok = or_erase_dims(words[k], words[k + 1], H, W, scale_min, scale_max,
                                       log_rmin, log_rmax, &eh, &ew);
                k += 2;
                if (ok) {
                    if (k + 2 > nwords) return -1;
                    p->i = or_randint(0, H - eh, words[k++]);
                    p->j = or_randint(0, W - ew, words[k++]);
                    p->eh = eh;
                    p->ew = ew;
                    p->erase = 1;
                    p->attempt = a;
                    break;
                }
            }
        }
    }
    p->words_used = (int32_t)k;
    return 0;
}

/* The longest stream one sample can need: flip, gate, 10 attempts, i, j. */
#define OR_MAX_WORDS 24

/* Parameters of samples first_n .. first_n+count-1. */
void or_params(uint64_t seed, int64_t first_n, int64_t count, int32_t H, int32_t W,
               float flip_p, float erase_p, float scale_min, float scale_max,
               float ratio_min, float ratio_max, or_sample_params* out)
{
    const float log_rmin = or_log_ratio(ratio_min);
    const float log_rmax = or_log_ratio(ratio_max);
    for (int64_t s = 0; s < count; ++s) {
        uint32_t words[OR_MAX_WORDS];
        for (int k = 0; k < OR_MAX_WORDS; ++k)
            words[k] = or_word(seed, (uint64_t)(first_n + s), (uint64_t)k);
        or_params_from_words(words, OR_MAX_WORDS, H, W, flip_p, erase_p, scale_min, scale_max,
                             log_rmin, log_rmax, &out[s]);
    }
}

/* The output of one image given its parameters: the plain definition,
 *   out[h,w,c] = +0                                    inside the rectangle,
 *              = RN32((x/255 - mean_c) / std_c)        otherwise,
 * with x the input byte at (h, W-1-w, c) when flipped and (h, w, c) if not
 * (page section 5: flip before ToTensor/Normalize; page section 12: erase
 * after normalize, to zero, over all channels). */
static void apply_one(const uint8_t* img, int32_t H, int32_t W, int32_t C,
                      const float* mean, const float* std, const or_sample_params* p, float* out)
{
    for (int32_t h = 0; h < H; ++h) {
        for (int32_t w = 0; w < W; ++w) {
            int in_rect = p->erase && h >= p->i && h < p->i + p->eh && w >= p->j && w < p->j + p->ew;
            int32_t src_w = p->flip ? (W - 1 - w) : w;
            for (int32_t c = 0; c < C; ++c) {
                size_t o = ((size_t)h * (size_t)W + (size_t)w) * (size_t)C + (size_t)c;
                if (in_rect) {
                    out[o] = 0.0f;
                } else {
                    uint8_t x = img[((size_t)h * (size_t)W + (size_t)src_w) * (size_t)C + (size_t)c];
                    double v = (double)x / 255.0;
                    out[o] = (float)((v - (double)mean[c]) / (double)std[c]);
                }
            }
        }
    }
}

void or_apply(const uint8_t* in, int64_t N, int32_t H, int32_t W, int32_t C,
              const float* mean, const float* std, const or_sample_params* params, float* out)
{
    const size_t img = (size_t)H * (size_t)W * (size_t)C;
    for (int64_t n = 0; n < N; ++n)
        apply_one(in + (size_t)n * img, H, W, C, mean, std, &params[n], out + (size_t)n * img);
}

/* ---- the whole operation over a batch, split by image over threads ---- */

typedef struct {
    const uint8_t* in; /* image first_n */
    float* out;        /* image first_n */
    int64_t first_n, n_begin, n_end;
    int32_t H, W, C;
    const float *mean, *std;
    float flip_p, erase_p, scale_min, scale_max, ratio_min, ratio_max;
    uint64_t seed;
} or_job;

static void* run_job(void* arg)
{
    const or_job* j = (const or_job*)arg;
    const size_t img = (size_t)j->H * (size_t)j->W * (size_t)j->C;
    for (int64_t n = j->n_begin; n < j->n_end; ++n) {
        or_sample_params p;
        or_params(j->seed, n, 1, j->H, j->W, j->flip_p, j->erase_p, j->scale_min, j->scale_max,
                  j->ratio_min, j->ratio_max, &p);
        size_t at = (size_t)(n - j->first_n) * img;
        apply_one(j->in + at, j->H, j->W, j->C, j->mean, j->std, &p, j->out + at);
    }
    return NULL;
}

/* Images first_n .. first_n+count-1 of the batch starting at `in`
 * (in and out point at image first_n); threads <= 1 runs inline.
 * Returns the number of threads used. */
int or_fused_normalize(const uint8_t* in, int64_t first_n, int64_t count, int32_t H, int32_t W,
                       int32_t C, const float* mean, const float* std, float flip_p, float erase_p,
                       float scale_min, float scale_max, float ratio_min, float ratio_max,
                       uint64_t seed, float* out, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > count) threads = (int)(count > 0 ? count : 1);
    or_job* jobs = (or_job*)calloc((size_t)threads, sizeof(or_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
    for (int t = 0; t < threads; ++t) {
        or_job* j = &jobs[t];
        j->first_n = first_n;
        j->n_begin = first_n + count * t / threads;
        j->n_end = first_n + count * (t + 1) / threads;
        j->in = in;
        j->out = out;
        j->H = H; j->W = W; j->C = C;
        j->mean = mean; j->std = std;
        j->flip_p = flip_p; j->erase_p = erase_p;
        j->scale_min = scale_min; j->scale_max = scale_max;
        j->ratio_min = ratio_min; j->ratio_max = ratio_max;
        j->seed = seed;
    }
    if (threads == 1) {
        run_job(&jobs[0]);
    } else {
        for (int t = 0; t < threads; ++t) pthread_create(&tids[t], NULL, run_job, &jobs[t]);
        for (int t = 0; t < threads; ++t) pthread_join(tids[t], NULL);
    }
    free(jobs);
    free(tids);
    return threads;
}

/* ---- array forms of two helpers, for exhaustive tests (plain loops) ---- */

void or_expf_array(const float* L, int64_t count, float* out)
{
    for (int64_t s = 0; s < count; ++s) out[s] = or_expf(L[s]);
}

/* eh/ew of one attempt per (w_scale[s], w_ratio[s]) pair; accepted[s] = 0/1. */
void or_erase_dims_array(const uint32_t* w_scale, const uint32_t* w_ratio, int64_t count,
                         int32_t H, int32_t W, float scale_min, float scale_max,
                         float ratio_min, float ratio_max,
                         int32_t* eh_out, int32_t* ew_out, uint8_t* accepted)
{
    const float log_rmin = or_log_ratio(ratio_min);
    const float log_rmax = or_log_ratio(ratio_max);
    for (int64_t s = 0; s < count; ++s)
        accepted[s] = (uint8_t)or_erase_dims(w_scale[s], w_ratio[s], H, W, scale_min, scale_max,
                                             log_rmin, log_rmax, &eh_out[s], &ew_out[s]);
}
