/*
 * fn_cpu.h -- FusedNormalization on the host CPU (SSE4.1 + F16C): the C ABI of
 * libfn_cpu.so.
 *
 * The page "(11) FusedNormalization" (tech-renaissance.cn/blog/?p=487) runs
 * the fused step on CPU worker threads, one image per call of execute()
 * (section 5): the flip decision first, then each row mirrored by pixel (the
 * channel order kept) and normalized as x * mul - sub with 4-wide fp32 SIMD
 * (section 7), stored as fp32 or converted to fp16 by F16C with round to
 * nearest even (section 6), optionally in the 4-channel padded layout
 * (section 8); the RandomErasing rectangle (section 12) is zeroed over the
 * finished output.  This library is that method on the host: a comparison
 * path for measurements and tests.  The GPU library (fn.h) never calls it.
 *
 * Decisions use the same readings as fn.h's fn_params (Philox4x32-10 word k
 * of sample n = output k%4 of counter (k/4, n) under key seed; one fp32
 * rounding per operation; exp, sqrt and division rounded once; sides rounded
 * half away from zero; inclusive corner draws), so for the same arguments
 * both libraries take the same flip bits and rectangles.
 *
 * Values: x * mul - sub with mul = RN32(1/(255 std)), sub = RN32(mean/std),
 * each product and difference rounded to fp32 (the page's arithmetic) where,
 * over all 256 byte values of every channel, that stores the same fp16 bits
 * as the value evaluated in double and rounded once (fp16 output), or lies
 * within 1e-6 of it (fp32 output); otherwise every element is evaluated in
 * double and rounded once.
 */
#ifndef FN_CPU_H
#define FN_CPU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FN_CPU_EINVAL (-1)
#define FN_CPU_ENOMEM (-2)  /* host memory for the per-thread row buffers */

#define FN_CPU_OUT_FP32 0       /* 4-byte floats                                 */
#define FN_CPU_OUT_FP16 1       /* 2-byte halves, C channels per pixel           */
#define FN_CPU_OUT_FP16_PAD4 2  /* 2-byte halves, 4 channels per pixel, pads +0 */

/* One sample's decisions; the same fields and layout as fn_sample_params. */
typedef struct {
    int32_t flip, erase, i, j, eh, ew, attempt, words_used;
} fn_cpu_sample_params;

/*
 * fn_cpu_fused_normalize -- the operation on a batch in host memory.
 *
 *   in         N*H*W*C bytes, NHWC, contiguous (host memory).
 *   N, H, W, C images, height, width, channels (1 <= C <= 4, H*W <= 2^24).
 *   mean, std  C floats each (std > 0, all finite).
 *   flip_p, erase_p, scale_min/max, ratio_min/max, seed
 *              as fn_fused_normalize (fn.h).
 *   first_sample_id  sample n draws from stream first_sample_id + n.
 *   out_dtype  FN_CPU_OUT_FP32, FN_CPU_OUT_FP16 or FN_CPU_OUT_FP16_PAD4.
 *   out        N*H*W*OC elements (OC = 4 when padded, else C), host memory.
 *   params     NULL, or N records that receive each sample's decisions.
 *   threads    worker threads (images are split evenly); < 1 means 1.
 *
 * Synchronous; returns 0, or FN_CPU_EINVAL or FN_CPU_ENOMEM (message from
 * fn_cpu_last_error() on the calling thread) with nothing written.  When the
 * system refuses a worker thread, the calling thread processes that
 * thread's images itself.
 */
int fn_cpu_fused_normalize(const uint8_t* in, int64_t N, int32_t H, int32_t W, int32_t C,
                           const float* mean, const float* std, float flip_p, float erase_p,
                           float scale_min, float scale_max, float ratio_min, float ratio_max,
                           uint64_t seed, int64_t first_sample_id, int32_t out_dtype, void* out,
                           fn_cpu_sample_params* params, int32_t threads);

/* The message of the last nonzero return on the calling thread ("" if none). */
const char* fn_cpu_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FN_CPU_H */
