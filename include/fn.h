/*
 * fn.h -- FusedNormalization on AMD Instinct MI355X (gfx950): the C ABI of libfn.so.
 *
 * One memory pass turns a batch of uint8 NHWC images into per-channel
 * normalized (x/255 - mean)/std tensors in fp32 or fp16, with a per-sample
 * random horizontal flip and a per-sample RandomErasing rectangle applied in
 * the same pass.  The operation is the FusedNormalization step of the page
 * "(11) FusedNormalization: fusing the last steps of data augmentation into one
 * memory pass" (tech-renaissance.cn/blog/?p=487):
 *   - section 5: ToTensor (x/255), RandomHorizontalFlip, Normalize
 *     ((v - mean)/std) and RandomErasing fused into one execute() call; the
 *     flip is drawn first, then the rectangle;
 *   - section 6: fp32 output or fp16 output (round to nearest even);
 *   - section 10: every random number is a pure function of (seed, offset)
 *     through the Philox counter-based generator;
 *   - section 12: the rectangle sampler (gate, up to 10 attempts of area
 *     fraction and log aspect ratio, rounding, acceptance, corner).
 * The page runs this per image on CPU threads; here one call processes a
 * whole batch on one GPU.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device memory (hipMalloc or a PyTorch CUDA
 *     tensor); pointers without the suffix are host memory.  All memory is
 *     owned by the caller; the library keeps no pointer after returning and
 *     allocates nothing.
 *   - `stream` is a hipStream_t cast to void* (NULL = the null stream).  Work
 *     is enqueued asynchronously on it; the call does not synchronize.  The
 *     caller keeps the buffers alive until the stream has finished the work.
 *   - Return value: FN_OK (0) on success, or a negative FN_E* code.  On an
 *     error nothing is enqueued and no output byte is written; the message is
 *     available from fn_last_error() on the calling thread.
 *   - All entry points are thread-safe and reentrant (no global state beyond
 *     the thread-local error message).
 */
#ifndef FN_H
#define FN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FN_OK 0
#define FN_EINVAL (-1)    /* an argument is out of its documented domain           */
#define FN_EOVERFLOW (-2) /* a size does not fit the index arithmetic              */
#define FN_EHIP (-3)      /* the HIP runtime reported an error (message kept)      */

/* Output element type. */
#define FN_OUT_FP32 0 /* 4-byte IEEE binary32                                       */
#define FN_OUT_FP16 1 /* 2-byte IEEE binary16, rounded to nearest even (page sec. 6) */
#define FN_OUT_FP16_PAD4 2 /* binary16 with 4 channels per pixel: channels c < C as
                              FN_OUT_FP16, channels C..3 are +0 -- the page's
                              mixed-precision layout (page sec. 8) */

/* One sample's random decisions (32 bytes, all int32):
 *   flip        1 if the image is mirrored left-right, else 0;
 *   erase       1 if the rectangle below is zeroed, else 0;
 *   i, j        row and column of the rectangle's top-left corner, in output
 *               (post-flip) coordinates; 0 when erase is 0;
 *   eh, ew      rectangle height and width in pixels (0 < eh < H, 0 < ew < W
 *               when erase is 1; 0 when erase is 0);
 *   attempt     index 0..9 of the accepted attempt, or -1 when none was;
 *   words_used  generator words the sample consumed (see fn_params). */
typedef struct {
    int32_t flip, erase, i, j, eh, ew, attempt, words_used;
} fn_sample_params;

/*
 * fn_fused_normalize -- the whole operation on a batch (page sec. 5, 6, 10, 12).
 *
 *   in_u8_dev   N*H*W*C bytes, image n at byte offset n*H*W*C, row-major
 *               (h, w, c) inside an image (NHWC, contiguous).  Any alignment.
 *   N           images (N = 0: validate the arguments, enqueue nothing).
 *   H, W, C     image height, width, channels; 1 <= C <= 4; H*W <= 2^24.
 *   mean, std   host arrays of C floats; std[c] > 0, all finite.
 *   flip_p      probability in [0, 1] of mirroring an image (page sec. 5
 *               uses 0.5); 0 draws no flip word.
 *   erase_p     probability in [0, 1] of trying to erase (page sec. 12); 0
 *               draws no gate word.
 *   scale_min/max  area-fraction range, 2^-30 <= scale_min <= scale_max <= 1
 *               (page sec. 4 defaults 0.02, 0.33).
 *   ratio_min/max  aspect-ratio range, 2^-30 <= ratio_min <= ratio_max <= 2^30
 *               (page sec. 4 defaults 0.3, 3.3).
 *   seed        64-bit generator key; sample n draws from the stream keyed by
 *               (seed, n), so the result does not depend on the launch shape.
 *   out_dtype   FN_OUT_FP32, FN_OUT_FP16 or FN_OUT_FP16_PAD4.
 *   out_dev     N*H*W*OC elements of out_dtype in NHWC order, OC = C (no
 *               padding) or 4 for FN_OUT_FP16_PAD4, aligned to the element
 *               size (4 or 2 bytes); must not overlap the input.
 *               Speed only: a 16-byte aligned out_dev whose rows are whole
 *               16-byte vectors (W*OC*element size a multiple of 16) takes
 *               the fastest kernel; other outputs take a flat layout at
 *               about two thirds of its rate; input rows that leave room
 *               for only one tile per compute unit in LDS (about 80 KB on
 *               MI355X) take slower paths.  Results are the same bits.
 *
 * Result, per sample n with P = fn_params(seed, ...)[n]:
 *   out[n,h,w,c] = +0                                 if P.erase and
 *                                                     P.i <= h < P.i+P.eh and P.j <= w < P.j+P.ew
 *                = (x/255 - mean_c)/std_c             otherwise,
 *   x = in[n, h, P.flip ? W-1-w : w, c].  The pixel order is mirrored, the
 *   channel order inside a pixel is kept (page sec. 7).  The value is
 *   computed as page sec. 7 writes it, x*mul_c - sub_c, with mul_c =
 *   1/(255 std_c) and sub_c = mean_c/std_c each carried as a pair of fp32
 *   numbers (their double values split into high and low parts):
 *   fma(x, mul_hi, -sub_hi) + fma(x, mul_lo, -sub_lo).  fp32 output is within
 *   2e-6 of the correctly rounded value for |value| < 8 and within about one
 *   fp32 ulp of it relative to the value; fp16 output is that fp32 value
 *   rounded to nearest even, within one fp16 ulp of the correctly rounded
 *   fp32 value.  With FN_OUT_FP16_PAD4, out[n,h,w,c] for c < C is the fp16
 *   value above and out[n,h,w,c] = +0 for C <= c < 4.
 *
 * Errors: FN_EINVAL for a null pointer (N > 0), a device pointer that is not
 * device memory or whose buffer is shorter than the sizes above, a misaligned
 * out_dev, any scalar outside its domain, an unknown out_dtype, or
 * overlapping in/out;
 * FN_EOVERFLOW for N*H*W*C*4 beyond int64 or H*W > 2^24; FN_EHIP if the
 * launch fails.
 */
int fn_fused_normalize(const uint8_t* in_u8_dev, int64_t N, int32_t H, int32_t W, int32_t C,
                       const float* mean, const float* std, float flip_p, float erase_p,
                       float scale_min, float scale_max, float ratio_min, float ratio_max,
                       uint64_t seed, int32_t out_dtype, void* out_dev, void* stream);

/*
 * fn_params -- the per-sample random decisions alone (page sec. 5 execute(),
 * sec. 10 uniform()/randint(), sec. 12 generate_erase_rect()).
 *
 * Writes params_dev[n] for n in [0, N): exactly the decisions
 * fn_fused_normalize takes with the same (seed, H, W, probabilities, ranges).
 * Arguments as for fn_fused_normalize; params_dev holds N fn_sample_params.
 *
 * Generator: word k of sample n is output k%4 of Philox4x32-10 (Salmon et al.,
 * SC'11) with counter (k/4 low, k/4 high, n low, n high) and key (seed low,
 * seed high).  A word becomes u = (word >> 8) * 2^-24.  Words are consumed in
 * order: the flip word (if flip_p > 0; flip iff u < flip_p), the gate word (if
 * erase_p > 0; try iff u < erase_p), then per attempt an area-fraction word
 * and a log-ratio word, and after an accepted attempt a row word and a column
 * word (randint(lo, hi) = lo + floor(word * (hi-lo+1) / 2^32), inclusive).
 * The attempt arithmetic is fp32 with one rounding per operation; exp, sqrt
 * and division are correctly rounded; sides are rounded half away from zero.
 *
 * Errors: as fn_fused_normalize (params_dev must be device memory of at
 * least N*32 bytes).
 */
int fn_params(uint64_t seed, int64_t N, int32_t H, int32_t W, float flip_p, float erase_p,
              float scale_min, float scale_max, float ratio_min, float ratio_max,
              fn_sample_params* params_dev, void* stream);

/*
 * fn_fused_normalize_ex -- fn_fused_normalize on a strided source, with the
 * sample numbering offset.
 *
 *   in_u8_dev        the first byte read: channel 0 of pixel (0, 0) of image 0.
 *   in_row_stride    bytes from one source row to the next, >= W*C.
 *   in_image_stride  bytes from one source image to the next, >= 0 (images
 *                    may overlap; 0 reads the same image N times).
 *                    Row h of image n starts at
 *                    in_u8_dev + n*in_image_stride + h*in_row_stride and
 *                    holds W*C bytes.  With W*C and H*W*C this is
 *                    fn_fused_normalize's layout.  The page's per-image
 *                    entry point takes such a row stride (page sec. 5,
 *                    execute(input_ptr, width, height, input_stride, ...)),
 *                    and the crop that precedes the fused step in the
 *                    operator chain (page sec. 4) is then a pointer offset:
 *                    pass the window's top-left pixel and the full image's
 *                    strides.
 *   first_sample_id  >= 0; sample n of this call draws from stream
 *                    (seed, first_sample_id + n) (page sec. 10: decisions
 *                    are a function of seed and offset only).  Splitting a
 *                    batch into slices [a, b) called with first_sample_id =
 *                    a reproduces the whole batch's result bit for bit, on
 *                    one device or several.
 *   all other arguments as fn_fused_normalize; the output is compact.
 *
 * Errors: as fn_fused_normalize, plus FN_EINVAL for in_row_stride < W*C,
 * in_image_stride < 0 or first_sample_id < 0, and FN_EOVERFLOW when the
 * input span (N-1)*in_image_stride + (H-1)*in_row_stride + W*C exceeds
 * 2^62.  The whole span must lie in one device allocation.
 */
int fn_fused_normalize_ex(const uint8_t* in_u8_dev, int64_t in_row_stride,
                          int64_t in_image_stride, int64_t N, int32_t H, int32_t W, int32_t C,
                          const float* mean, const float* std, float flip_p, float erase_p,
                          float scale_min, float scale_max, float ratio_min, float ratio_max,
                          uint64_t seed, int64_t first_sample_id, int32_t out_dtype,
                          void* out_dev, void* stream);

/* fn_params_ex -- fn_params for samples first_sample_id .. first_sample_id +
 * N - 1: params_dev[n] is sample first_sample_id + n's record, the decisions
 * fn_fused_normalize_ex takes with the same first_sample_id.  Errors as
 * fn_params, plus FN_EINVAL for first_sample_id < 0. */
int fn_params_ex(uint64_t seed, int64_t first_sample_id, int64_t N, int32_t H, int32_t W,
                 float flip_p, float erase_p, float scale_min, float scale_max, float ratio_min,
                 float ratio_max, fn_sample_params* params_dev, void* stream);

/* The message of the last nonzero return on the calling thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* fn_last_error(void);

/* ------------------------------------------------------------------------ */
/* Test and measurement hooks.  Not part of the operation; exposed so tests  */
/* can check the building blocks exhaustively and the benchmark can measure  */
/* the operation's traffic alone.  Same conventions as above.                */
/* ------------------------------------------------------------------------ */

/* One erase attempt (page sec. 12) per index s in [0, count): from the area
 * word w_scale_dev[s] and the log-ratio word w_ratio_dev[s], writes the rounded
 * sides eh_dev[s], ew_dev[s] (-1 if beyond int32) and accepted_dev[s] (1 if
 * 0 < eh < H and 0 < ew < W).  Same domains as fn_params. */
int fn_test_erase_dims(const uint32_t* w_scale_dev, const uint32_t* w_ratio_dev, int64_t count,
                       int32_t H, int32_t W, float scale_min, float scale_max, float ratio_min,
                       float ratio_max, int32_t* eh_dev, int32_t* ew_dev, uint8_t* accepted_dev,
                       void* stream);

/* The correctly rounded fp32 operations the sampler uses, per index s:
 *   op 0: out[s] = RN32(exp(a[s]))   for |a[s]| <= 80;
 *   op 1: out[s] = RN32(sqrt(a[s]))  for positive normal a[s];
 *   op 2: out[s] = RN32(a[s] / b[s]) for positive normal a[s], b[s] whose
 *         quotient is a normal float.
 * Outside those domains the output is unspecified (but written, and the
 * kernel still ends normally).  b_dev may be NULL for ops 0 and 1. */
int fn_test_cr_ops(int32_t op, const float* a_dev, const float* b_dev, int64_t count,
                   float* out_dev, void* stream);

/* The operation's traffic without its arithmetic, as the practical bandwidth
 * roof of the fused kernels: reads in_bytes from src_dev and writes every
 * byte zero-extended to `widen` bytes, in_bytes * widen bytes in all, as
 * 16-byte streaming stores.
 *   widen 2 (the fp16 operation's 1:2 read:write mix): the output is the
 *     input widened to 16 bits, in order.
 *   widen 4 (the fp32 one's 1:4 mix): per block of 256 input vectors of 16
 *     bytes starting at vector b (m = min(256, in_bytes/16 - b) vectors in
 *     the block), dword k of vector v, widened to four 32-bit values, is
 *     output vector 4b + k*m + (v - b).
 * in_bytes a multiple of 16; both pointers 16-byte aligned; no overlap.
 * Errors as above (FN_EINVAL for any other widen). */
int fn_test_stream(const void* src_dev, void* dst_dev, int64_t in_bytes, int32_t widen,
                   void* stream);

/* Measurement hook of the instrumented build libfn_timeline.so (the same
 * sources compiled with FN_TIMELINE=1): every later fused call whose tiles
 * kernel runs records, for each tile t < tiles, four 64-bit stamps of the
 * GPU's 100 MHz real-time clock at stamps_dev + 4 t: its work-group's start,
 * the end of staging (tile loaded and decisions drawn), its stores issued
 * (first wavefront) and its stores acknowledged (all wavefronts).  The
 * tile order is the kernel's own (tile t covers the t-th range of rows).
 * stamps_dev is a caller-owned device buffer of tiles * 32 bytes that must
 * outlive those calls; tiles = 0 stops recording.  Not thread-safe: one
 * setting per process.  The product library libfn.so returns FN_EINVAL. */
int fn_test_timeline(void* stamps_dev, int64_t tiles);

#ifdef __cplusplus
}
#endif

#endif /* FN_H */
