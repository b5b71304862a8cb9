// fn_api.hip -- the C ABI of libfn.so: argument validation, the host-side
// constants of the operation, and kernel launches.  Declarations, argument
// meaning, layouts and error behaviour are documented in include/fn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fn.h"
#include "fn_kernels.hpp"

#define FN_EXPORT extern "C" __attribute__((visibility("default")))


namespace {

// the last error message of this thread: a fixed buffer, so that recording
// an error never allocates (and nothing can throw across the C ABI)
thread_local char g_last_error[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return FN_OK;
}

bool in_unit(float p) { return p >= 0.0f && p <= 1.0f; }  // false for NaN

// The calling thread's current device.
int current_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(FN_EHIP, "hipGetDevice failed");
  }
  return FN_OK;
}

// The buffer [p, p + bytes) must be device memory of the current device,
// inside one allocation.  *dev caches the current device across the checks
// of one call (-1: not queried yet).  Failed queries leave no sticky HIP
// error behind.
int check_device_range(const void* p, size_t bytes, const char* name, int* dev) {
  if (p == nullptr) return fail(FN_EINVAL, "%s is NULL", name);
  if (*dev < 0) {
    const int rc = current_device(dev);
    if (rc) return rc;
  }
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FN_EINVAL, "%s is not device memory (%s)", name, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice)
    return fail(FN_EINVAL, "%s is not device memory (memory type %d)", name, (int)attr.type);
  if (attr.device != *dev)
    return fail(FN_EINVAL, "%s lives on device %d, the current device is %d", name, attr.device,
                *dev);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FN_EINVAL, "%s: cannot determine its allocation (%s)", name, hipGetErrorString(e));
  }
  const uintptr_t lo = (uintptr_t)base, hi = lo + size, b = (uintptr_t)p;
  if (b < lo || bytes > hi - b)
    return fail(FN_EINVAL, "%s: %zu bytes needed, %zu available in its allocation", name, bytes,
                (size_t)(hi - b));
  return FN_OK;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Sampler arguments shared by fn_params, fn_fused_normalize and the hooks.
int make_draw_args(uint64_t seed, int32_t H, int32_t W, float flip_p, float erase_p,
                   float scale_min, float scale_max, float ratio_min, float ratio_max,
                   fn::DrawArgs* a) {
  if (H <= 0 || W <= 0) return fail(FN_EINVAL, "H and W must be positive (got %d, %d)", H, W);
  if ((int64_t)H * (int64_t)W > (int64_t)1 << 24)
    return fail(FN_EOVERFLOW, "H*W = %lld exceeds 2^24", (long long)H * W);
  if (!in_unit(flip_p)) return fail(FN_EINVAL, "flip_p must be in [0, 1]");
  if (!in_unit(erase_p)) return fail(FN_EINVAL, "erase_p must be in [0, 1]");
  if (!(scale_min >= 0x1p-30f && scale_min <= scale_max && scale_max <= 1.0f))
    return fail(FN_EINVAL, "need 2^-30 <= scale_min <= scale_max <= 1");
  if (!(ratio_min >= 0x1p-30f && ratio_min <= ratio_max && ratio_max <= 0x1p30f))
    return fail(FN_EINVAL, "need 2^-30 <= ratio_min <= ratio_max <= 2^30");
  a->seed = seed;
  a->first_sample = 0;
  a->H = H;
  a->W = W;
  a->flip_p = flip_p;
  a->erase_p = erase_p;
  a->scale_min = scale_min;
  a->scale_max = scale_max;
  // RN32(ln r): the extended-precision log is far more accurate than the
  // half-ulp margin of any fp32 rounding it could get wrong.
  a->log_rmin = (float)logl((long double)ratio_min);
  a->log_rmax = (float)logl((long double)ratio_max);
  a->img_area = (float)H * (float)W;
  return FN_OK;
}

unsigned blocks_for(int64_t items, int64_t per_block) {
  return (unsigned)((items + per_block - 1) / per_block);
}

// Compute units of device `dev`, queried once per device.
int device_cu_count(int dev, int* cus) {
  static std::atomic<int> cache[64];
  if (dev >= 0 && dev < 64 && cache[dev].load(std::memory_order_relaxed) > 0) {
    *cus = cache[dev].load(std::memory_order_relaxed);
    return FN_OK;
  }
  int v = 0;
  const hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || v <= 0) {
    (void)hipGetLastError();
    return fail(FN_EHIP, "cannot query the compute unit count: %s", hipGetErrorString(e));
  }
  if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  *cus = v;
  return FN_OK;
}

// LDS bytes per compute unit of device `dev`, cached per device; 0 if the
// runtime does not report it.
size_t device_lds_per_cu(int dev) {
  static std::atomic<long> cache[64];
  if (dev >= 0 && dev < 64) {
    const long c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c > 0 ? (size_t)c : 0;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
      hipSuccess) {
    (void)hipGetLastError();
    v = 0;
  }
  if (dev >= 0 && dev < 64) cache[dev].store(v > 0 ? (long)v : -1, std::memory_order_relaxed);
  return v > 0 ? (size_t)v : 0;
}

// LDS bytes one work-group may use on device `dev`, cached per device; 0 if
// the runtime does not report it.
size_t device_lds_per_block(int dev) {
  static std::atomic<long> cache[64];
  if (dev >= 0 && dev < 64) {
    const long c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c > 0 ? (size_t)c : 0;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
    (void)hipGetLastError();
    v = 0;
  }
  if (dev >= 0 && dev < 64) cache[dev].store(v > 0 ? (long)v : -1, std::memory_order_relaxed);
  return v > 0 ? (size_t)v : 0;
}

// Largest staging buffer of a tiles-kernel work-group on device `dev`: what
// one work-group may hold (all: true), or what lets two share a compute unit
// (all: false), after the decision records and a margin.  Rows up to the
// second take the tiles kernels outright (measured: they beat the pixel-group
// kernel there); wider rows up to the first take them when the pixel-group
// kernel does not apply (one resident work-group per compute unit still beats
// the element-wise kernel).
int64_t tile_buffer_limit(int dev, bool all) {
  const int64_t fixed = (int64_t)sizeof(fn::SampleParams) * fn::kMaxImagesPerBlock + 64;
  // 64 KB per work-group and per compute unit where the runtime reports
  // nothing (every CDNA device has at least that)
  const int64_t block = device_lds_per_block(dev) > 0 ? (int64_t)device_lds_per_block(dev) : 65536;
  const int64_t cu = device_lds_per_cu(dev) > 0 ? (int64_t)device_lds_per_cu(dev) : 65536;
  const int64_t lim = all ? block : std::min(block, cu / 2);
  return std::max<int64_t>(lim - fixed, 0);
}

// Dynamic LDS of one tiles-kernel work-group: its staging buffer, padded so
// that at most kWgsPerCu work-groups fit on a compute unit (fewer resident
// work-groups queue less at the memory and finish sooner; measured).  Only
// buffers below that share are padded, and never beyond 64 KB.
size_t tiles_lds_bytes(int dev, int32_t buffer_bytes) {
  size_t lds = (size_t)buffer_bytes;
  const size_t per_cu = device_lds_per_cu(dev);
  if (fn::kWgsPerCu > 0 && per_cu > 0) {
    const size_t cap = per_cu / fn::kWgsPerCu;   // kWgsPerCu fit ...
    const size_t over = per_cu / (fn::kWgsPerCu + 1) + 1;  // ... one more does not
    const size_t want = cap - 1024;  // room for the static decision records
    if (want >= over && want <= 65536) lds = std::max(lds, want);
  }
  return lds;
}

fn::FastDiv make_fast_div(uint32_t d) {
  fn::FastDiv f;
  f.d = d;
  f.m = d > 1 ? (uint32_t)((((uint64_t)1) << 32) / d + 1) : 0u;
  return f;
}

// Pixels per lane group for the grouped kernel, or 0 if it does not apply:
// W must be a multiple of the group, the input aligned to the group's load
// vector (16, 8 or 4 bytes), and the output 16-byte aligned with a group
// size that is a multiple of 4 bytes.  Prefers the widest group.
int pick_group_pixels(int32_t W, int32_t C, int out_bytes, uintptr_t in, uintptr_t out) {
  if (out % 16 != 0) return 0;
  const int choices[3] = {16, 8, 4};
  for (int px : choices) {
    if (px > fn::kGroupPxMax) continue;
    if (W % px != 0) continue;
    const int nb = px * C;
    const int align = nb % 16 == 0 ? 16 : (nb % 8 == 0 ? 8 : 4);
    if (nb % 4 != 0 || in % (uintptr_t)align != 0) continue;
    if ((nb * out_bytes) % 4 != 0) continue;
    return px;
  }
  return 0;
}

template <int C, int PX>
void launch_grouped_c(const fn::FusedArgs& a, int out_dtype, unsigned grid, hipStream_t st) {
  if (out_dtype == FN_OUT_FP32)
    fn::fused_grouped_kernel<C, PX, float><<<grid, fn::kBlock, 0, st>>>(a);
  else
    fn::fused_grouped_kernel<C, PX, _Float16><<<grid, fn::kBlock, 0, st>>>(a);
}

template <int PX>
void launch_grouped_px(const fn::FusedArgs& a, int C, int out_dtype, unsigned grid,
                       hipStream_t st) {
  switch (C) {
    case 1: launch_grouped_c<1, PX>(a, out_dtype, grid, st); break;
    case 2: launch_grouped_c<2, PX>(a, out_dtype, grid, st); break;
    case 3: launch_grouped_c<3, PX>(a, out_dtype, grid, st); break;
    default: launch_grouped_c<4, PX>(a, out_dtype, grid, st); break;
  }
}

template <int C, bool kComp>
void launch_tiles_c(const fn::FusedArgs& a, int out_dtype, bool nt, unsigned grid, size_t lds,
                    hipStream_t st) {
  if (out_dtype == FN_OUT_FP32)
    fn::fused_tiles_kernel<C, float, false, kComp>
        <<<grid, fn::tiles_threads<float>(), lds, st>>>(a);
  else if (out_dtype == FN_OUT_FP16_PAD4 && nt)
    fn::fused_tiles_kernel<C, _Float16, true, kComp, fn::kStoreNt>
        <<<grid, fn::tiles_threads<_Float16>(), lds, st>>>(a);
  else if (out_dtype == FN_OUT_FP16_PAD4)
    fn::fused_tiles_kernel<C, _Float16, true, kComp>
        <<<grid, fn::tiles_threads<_Float16>(), lds, st>>>(a);
  else if (nt)
    fn::fused_tiles_kernel<C, _Float16, false, kComp, fn::kStoreNt>
        <<<grid, fn::tiles_threads<_Float16>(), lds, st>>>(a);
  else
    fn::fused_tiles_kernel<C, _Float16, false, kComp>
        <<<grid, fn::tiles_threads<_Float16>(), lds, st>>>(a);
}

template <bool kComp>
void launch_tiles_k(const fn::FusedArgs& a, int C, int out_dtype, bool nt, unsigned grid,
                    size_t lds, hipStream_t st) {
  switch (C) {
    case 1: launch_tiles_c<1, kComp>(a, out_dtype, nt, grid, lds, st); break;
    case 2: launch_tiles_c<2, kComp>(a, out_dtype, nt, grid, lds, st); break;
    case 3: launch_tiles_c<3, kComp>(a, out_dtype, nt, grid, lds, st); break;
    default: launch_tiles_c<4, kComp>(a, out_dtype, nt, grid, lds, st); break;
  }
}

// nt: the non-temporal-store instance for long fp16 launches (packed or padded)
void launch_tiles(const fn::FusedArgs& a, int C, int out_dtype, bool comp, bool nt, unsigned grid,
                  size_t lds, hipStream_t st) {
  if (comp)
    launch_tiles_k<true>(a, C, out_dtype, nt, grid, lds, st);
  else
    launch_tiles_k<false>(a, C, out_dtype, nt, grid, lds, st);
}

template <int C, bool kComp>
void launch_flat_c(const fn::FusedArgs& a, int out_dtype, unsigned grid, size_t lds,
                   hipStream_t st) {
  if (out_dtype == FN_OUT_FP32)
    fn::fused_flat_kernel<C, float, false, kComp><<<grid, fn::tiles_threads<float>(), lds, st>>>(a);
  else if (out_dtype == FN_OUT_FP16_PAD4)
    fn::fused_flat_kernel<C, _Float16, true, kComp>
        <<<grid, fn::tiles_threads<_Float16>(), lds, st>>>(a);
  else
    fn::fused_flat_kernel<C, _Float16, false, kComp>
        <<<grid, fn::tiles_threads<_Float16>(), lds, st>>>(a);
}

template <bool kComp>
void launch_flat_k(const fn::FusedArgs& a, int C, int out_dtype, unsigned grid, size_t lds,
                   hipStream_t st) {
  switch (C) {
    case 1: launch_flat_c<1, kComp>(a, out_dtype, grid, lds, st); break;
    case 2: launch_flat_c<2, kComp>(a, out_dtype, grid, lds, st); break;
    case 3: launch_flat_c<3, kComp>(a, out_dtype, grid, lds, st); break;
    default: launch_flat_c<4, kComp>(a, out_dtype, grid, lds, st); break;
  }
}

void launch_flat(const fn::FusedArgs& a, int C, int out_dtype, bool comp, unsigned grid,
                 size_t lds, hipStream_t st) {
  if (comp)
    launch_flat_k<true>(a, C, out_dtype, grid, lds, st);
  else
    launch_flat_k<false>(a, C, out_dtype, grid, lds, st);
}

// Bits of the binary16 value nearest to v (ties to even), as the GPU's
// float-to-half conversion gives them.
uint16_t half_bits_rne(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);   // NaN
  if (mag >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // at or beyond 65520: infinity
  if (mag >= 0x38800000u) {                                   // normal: 2^-14 and up
    const uint32_t m = mag - 0x38000000u;                     // exponent rebiased 127 -> 15
    return (uint16_t)(sign | ((m + 0x0FFFu + ((m >> 13) & 1u)) >> 13));
  }
  // subnormal or zero: units of 2^-24, scaling by 2^24 is exact
  const float units = std::nearbyint(std::fabs(v) * 0x1p24f);  // default rounding: ties to even
  return (uint16_t)(sign | (uint32_t)units);
}

uint32_t float_bits(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  return u;
}

// True if one fma per element, fma(x, mul, nsub), stores exactly what the
// two-fma form fma(x, mul, nsub) + fma(x, mul_lo, nsub_lo) stores, for every
// byte value x of every channel: the fp32 bits, or the binary16 bits of
// their rounding.  The inputs are bytes, so this covers every element the
// kernel can meet.
bool single_fma_exact_uncached(const fn::FusedArgs& a, int C, int out_dtype) {
  for (int c = 0; c < C; ++c) {
    for (int x = 0; x < 256; ++x) {
      const float xf = (float)x;
      const float one = std::fma(xf, a.mul[c], a.nsub[c]);
      const float two = one + std::fma(xf, a.mul_lo[c], a.nsub_lo[c]);
      if (out_dtype == FN_OUT_FP32) {
        if (float_bits(one) != float_bits(two)) return false;
      } else if (half_bits_rne(one) != half_bits_rne(two)) {
        return false;
      }
    }
  }
  return true;
}

// single_fma_exact_uncached, remembered per thread for the last constants
// (a training loop calls with the same mean and std every time).
bool single_fma_exact(const fn::FusedArgs& a, int C, int out_dtype) {
  struct Last {
    bool valid = false, result = false;
    int C = 0, out_dtype = 0;
    float mul[4], mul_lo[4], nsub[4], nsub_lo[4];
  };
  thread_local Last last;
  const bool same = last.valid && last.C == C && last.out_dtype == out_dtype &&
                    std::memcmp(last.mul, a.mul, sizeof(last.mul)) == 0 &&
                    std::memcmp(last.mul_lo, a.mul_lo, sizeof(last.mul_lo)) == 0 &&
                    std::memcmp(last.nsub, a.nsub, sizeof(last.nsub)) == 0 &&
                    std::memcmp(last.nsub_lo, a.nsub_lo, sizeof(last.nsub_lo)) == 0;
  if (!same) {
    last.result = single_fma_exact_uncached(a, C, out_dtype);
    last.C = C;
    last.out_dtype = out_dtype;
    std::memcpy(last.mul, a.mul, sizeof(last.mul));
    std::memcpy(last.mul_lo, a.mul_lo, sizeof(last.mul_lo));
    std::memcpy(last.nsub, a.nsub, sizeof(last.nsub));
    std::memcpy(last.nsub_lo, a.nsub_lo, sizeof(last.nsub_lo));
    last.valid = true;
  }
  return last.result;
}

// Tile plan of the tiles kernel: the largest tile of at most kTileBytesTarget
// input bytes (whole rows, or whole images when one fits), shrunk -- down to
// kMinTileBytes -- so that the batch gives every compute unit at least 8
// tiles.  row_slot > 0: strided rows, staged row_slot LDS bytes apart.
// Sets the tile fields of `a`.
int plan_tiles(fn::FusedArgs* a, int64_t N, int32_t H, int64_t row, int64_t elems, int cus,
               int64_t row_slot, int64_t lds_limit) {
  // LDS bytes one row occupies: the row itself, or its slot of whole
  // granules when strided (never fewer than 32 bytes, however narrow the row)
  const int64_t row_lds = row_slot > 0 ? row_slot : row;
  int64_t target = fn::kTileBytesTarget;
  const int64_t want = (int64_t)cus * 8;
  if (elems / want < target) target = std::max<int64_t>(elems / want, fn::kMinTileBytes);
  if (target < row_lds) target = row_lds;
  const int64_t image_lds = (int64_t)H * row_lds;
  int64_t tile_bytes;
  if (image_lds <= target) {
    const int64_t g = std::min<int64_t>(target / image_lds, fn::kMaxImagesPerBlock);
    a->images_per_tile = (int32_t)g;
    a->rows_per_tile = H;
    a->tiles_per_image = 1;
    a->total_tiles = (N + g - 1) / g;
    tile_bytes = g * H * row;
  } else {
    const int64_t r = std::max<int64_t>(1, std::min<int64_t>(H, target / row_lds));
    a->images_per_tile = 1;
    a->rows_per_tile = (int32_t)r;
    a->tiles_per_image = (int32_t)((H + r - 1) / r);
    a->total_tiles = N * a->tiles_per_image;
    tile_bytes = r * row;
  }
  // contiguous: the tile's bytes plus the partial granules at both ends;
  // strided: one 16-byte-granule slot per row, and 16 bytes of slack for the
  // aligned dword reads that run up to 10 bytes past the last row's end (the
  // contiguous layout's 32 extra bytes cover them too)
  const int64_t tile_rows = a->images_per_tile == 1 ? a->rows_per_tile : a->images_per_tile * H;
  const int64_t lds = row_slot > 0 ? tile_rows * row_slot + 16 : (tile_bytes + 32 + 15) / 16 * 16;
  if (lds > lds_limit) return fail(FN_EOVERFLOW, "tile exceeds the LDS budget");
  if (a->total_tiles > 0x7FFFFFFF) return fail(FN_EOVERFLOW, "grid size limit exceeded");
  a->lds_buffer_bytes = (int32_t)lds;
  return FN_OK;
}

void launch_grouped(const fn::FusedArgs& a, int C, int px, int out_dtype, unsigned grid,
                    hipStream_t st) {
  if (px == 16)
    launch_grouped_px<16>(a, C, out_dtype, grid, st);
  else if (px == 8)
    launch_grouped_px<8>(a, C, out_dtype, grid, st);
  else
    launch_grouped_px<4>(a, C, out_dtype, grid, st);
}

}  // namespace

FN_EXPORT const char* fn_last_error(void) { return g_last_error; }

FN_EXPORT int fn_params_ex(uint64_t seed, int64_t first_sample_id, int64_t N, int32_t H,
                           int32_t W, float flip_p, float erase_p, float scale_min,
                           float scale_max, float ratio_min, float ratio_max,
                           fn_sample_params* params_dev, void* stream) {
  static_assert(sizeof(fn_sample_params) == sizeof(fn::SampleParams), "layout");
  fn::DrawArgs a;
  int rc = make_draw_args(seed, H, W, flip_p, erase_p, scale_min, scale_max, ratio_min, ratio_max,
                          &a);
  if (rc) return rc;
  if (first_sample_id < 0) return fail(FN_EINVAL, "first_sample_id must be >= 0");
  a.first_sample = (uint64_t)first_sample_id;
  if (N < 0) return fail(FN_EINVAL, "N must be >= 0");
  if (N > ((int64_t)1 << 36)) return fail(FN_EOVERFLOW, "N too large");
  if (N == 0) return ok();
  int dev = -1;
  rc = check_device_range(params_dev, (size_t)N * sizeof(fn_sample_params), "params_dev", &dev);
  if (rc) return rc;
  const int64_t samples_per_block = fn::kBlock / 16;
  fn::params_kernel<<<blocks_for(N, samples_per_block), fn::kBlock, 0, (hipStream_t)stream>>>(
      a, N, reinterpret_cast<fn::SampleParams*>(params_dev));
  return launch_status("params_kernel launch");
}

FN_EXPORT int fn_params(uint64_t seed, int64_t N, int32_t H, int32_t W, float flip_p,
                        float erase_p, float scale_min, float scale_max, float ratio_min,
                        float ratio_max, fn_sample_params* params_dev, void* stream) {
  return fn_params_ex(seed, 0, N, H, W, flip_p, erase_p, scale_min, scale_max, ratio_min,
                      ratio_max, params_dev, stream);
}

namespace {

#if FN_TIMELINE
// where the tiles kernel of later launches records its stamps (instrumented
// builds only; set by fn_test_timeline)
uint64_t* g_timeline = nullptr;
int64_t g_timeline_tiles = 0;
#endif

// Both fused entry points.  strides == nullptr: the compact layout; else
// {row stride, image stride} of the source in bytes.
int fused_normalize_impl(const uint8_t* in_u8_dev, const int64_t* strides, int64_t N, int32_t H,
                         int32_t W, int32_t C, const float* mean, const float* std, float flip_p,
                         float erase_p, float scale_min, float scale_max, float ratio_min,
                         float ratio_max, uint64_t seed, int64_t first_sample_id,
                         int32_t out_dtype, void* out_dev, void* stream) {
  fn::FusedArgs a{};
  int rc = make_draw_args(seed, H, W, flip_p, erase_p, scale_min, scale_max, ratio_min, ratio_max,
                          &a.draw);
  if (rc) return rc;
#if FN_TIMELINE
  a.timeline = g_timeline;
  a.timeline_tiles = g_timeline_tiles;
#endif
  if (C < 1 || C > 4) return fail(FN_EINVAL, "C must be in 1..4 (got %d)", C);
  if (N < 0) return fail(FN_EINVAL, "N must be >= 0");
  if (first_sample_id < 0) return fail(FN_EINVAL, "first_sample_id must be >= 0");
  a.draw.first_sample = (uint64_t)first_sample_id;
  if (out_dtype != FN_OUT_FP32 && out_dtype != FN_OUT_FP16 && out_dtype != FN_OUT_FP16_PAD4)
    return fail(FN_EINVAL, "unknown out_dtype %d", out_dtype);
  if (mean == nullptr || std == nullptr) return fail(FN_EINVAL, "mean and std must not be NULL");
  for (int c = 0; c < C; ++c) {
    if (!std::isfinite(mean[c])) return fail(FN_EINVAL, "mean[%d] is not finite", c);
    if (!(std[c] > 0.0f) || !std::isfinite(std[c]))
      return fail(FN_EINVAL, "std[%d] must be positive and finite", c);
  }
  const int64_t img = (int64_t)H * W * C;
  if (N > INT64_MAX / 16 / ((int64_t)H * W)) return fail(FN_EOVERFLOW, "N*H*W*4*4 overflows int64");
  const int64_t elems = N * img;
  const int64_t row = (int64_t)W * C;
  int64_t row_stride = row, image_stride = img;
  if (strides != nullptr) {
    row_stride = strides[0];
    image_stride = strides[1];
    if (row_stride < row) return fail(FN_EINVAL, "in_row_stride must be >= W*C");
    if (image_stride < 0) return fail(FN_EINVAL, "in_image_stride must be >= 0");
  }
  // input bytes from the first one read to the last: (N-1) image strides,
  // (H-1) row strides and one row
  int64_t span = 0;
  if (N > 0) {
    const __int128 s128 = (__int128)(N - 1) * image_stride + (__int128)(H - 1) * row_stride + row;
    if (s128 > (__int128)INT64_MAX / 2) return fail(FN_EOVERFLOW, "input span overflows int64");
    span = (int64_t)s128;
  }
  const bool strided = row_stride != row || image_stride != img;
  const int out_bytes = out_dtype == FN_OUT_FP32 ? 4 : 2;
  const int oc = out_dtype == FN_OUT_FP16_PAD4 ? 4 : C;  // output channels per pixel
  const int64_t out_elems = N * H * (int64_t)W * oc;

  // generic kernel tiles: about 8 KiB of input, whole rows
  int64_t rows = (8192 + row - 1) / row;
  if (rows > H) rows = H;
  a.rows_per_tile = (int32_t)rows;
  a.tiles_per_image = (int32_t)((H + rows - 1) / rows);
  if (N > (int64_t)0x7FFFFFFF / a.tiles_per_image)
    return fail(FN_EOVERFLOW, "N*tiles exceeds the grid size limit");
  if (N == 0) return ok();

  if ((uintptr_t)out_dev % (uintptr_t)out_bytes != 0)
    return fail(FN_EINVAL, "out_dev must be aligned to its element size (%d bytes)", out_bytes);
  int dev = -1;
  rc = check_device_range(in_u8_dev, (size_t)span, "in_u8_dev", &dev);
  if (rc) return rc;
  rc = check_device_range(out_dev, (size_t)out_elems * out_bytes, "out_dev", &dev);
  if (rc) return rc;
  const uintptr_t i0 = (uintptr_t)in_u8_dev, i1 = i0 + (uintptr_t)span;
  const uintptr_t o0 = (uintptr_t)out_dev, o1 = o0 + (uintptr_t)out_elems * out_bytes;
  if (i0 < o1 && o0 < i1) return fail(FN_EINVAL, "input and output overlap");

  a.in = in_u8_dev;
  a.out = out_dev;
  a.N = N;
  a.H = H;
  a.W = W;
  a.C = C;
  a.oc = oc;
  // 1/(255 std_c) and -mean_c/std_c, each rounded once to double and split
  // into an fp32 pair hi + lo (the difference is exact in double)
  for (int c = 0; c < 4; ++c) {
    a.mul[c] = a.mul_lo[c] = a.nsub[c] = a.nsub_lo[c] = 0.0f;
    if (c < C) {
      const double m = 1.0 / (255.0 * (double)std[c]);
      const double n = -((double)mean[c] / (double)std[c]);
      a.mul[c] = (float)m;
      a.mul_lo[c] = (float)(m - (double)a.mul[c]);
      a.nsub[c] = (float)n;
      a.nsub_lo[c] = (float)(n - (double)a.nsub[c]);
    }
  }

  hipStream_t st = (hipStream_t)stream;
  a.total_bytes = span;
  a.in_row_stride = row_stride;
  a.in_image_stride = image_stride;
  a.strided = strided ? 1 : 0;
  const int64_t row_out = (int64_t)W * oc;
  // strided rows: one slot of whole 16-byte granules per row
  const int64_t row_slot = strided ? (15 + row + 15) / 16 * 16 : 0;
  // the staging buffer of a one-row tile (plan_tiles' sizes)
  const int64_t one_row = strided ? row_slot + 16 : (row + 32 + 15) / 16 * 16;
  const int px = out_dtype == FN_OUT_FP16_PAD4 || strided
                     ? 0
                     : pick_group_pixels(W, C, out_bytes, (uintptr_t)in_u8_dev, (uintptr_t)out_dev);
  const int64_t lds_all = tile_buffer_limit(dev, true);
  if (one_row <= tile_buffer_limit(dev, false) || (px == 0 && one_row <= lds_all)) {
    int cus = 0;
    rc = device_cu_count(dev, &cus);
    if (rc) return rc;
    rc = plan_tiles(&a, N, H, row, elems, cus, row_slot, lds_all);
    if (rc) return rc;
    a.row_slot = (int32_t)row_slot;
    a.div_gps = make_fast_div((uint32_t)std::max<int64_t>(row_slot / 16, 1));
    a.div_row = make_fast_div((uint32_t)row);
    a.div_row_out = make_fast_div((uint32_t)row_out);
    a.div_h = make_fast_div((uint32_t)H);
    a.div_tpi = make_fast_div((uint32_t)a.tiles_per_image);
    {
      const int32_t chunk = out_dtype == FN_OUT_FP32 ? 4 : 8;  // outputs per 16-byte store
      const int32_t threads = out_dtype == FN_OUT_FP32 ? fn::tiles_threads<float>()
                                                       : fn::tiles_threads<_Float16>();
      // chunks per row: 0 for rows shorter than one vector, which only the
      // flat kernel takes
      const int32_t cpr = (int32_t)(row_out / chunk);
      a.div_cpr = make_fast_div((uint32_t)std::max<int32_t>(cpr, 1));
      a.rows_per_pass = cpr >= 1 && cpr <= threads ? threads / cpr : 0;
    }
    const bool comp = !single_fma_exact(a, C, out_dtype);
    const size_t lds = tiles_lds_bytes(dev, a.lds_buffer_bytes);
    // the tiles kernel's lanes need whole 16-byte vectors per row from a
    // 16-byte aligned output; any other element-aligned output takes the
    // flat layout
    if ((uintptr_t)out_dev % 16 == 0 && row_out % (16 / out_bytes) == 0) {
      // algorithmic bytes of the launch: input read once, output written once
      const int64_t moved = elems + out_elems * out_bytes;
      const bool nt = out_dtype != FN_OUT_FP32 && fn::kTilesNtMinBytes > 0 &&
                      moved >= fn::kTilesNtMinBytes;
      launch_tiles(a, C, out_dtype, comp, nt, (unsigned)a.total_tiles, lds, st);
      return launch_status("fused_tiles_kernel launch");
    }
    {
      // padded layout: the row-start vectors' values beside the tile, when
      // they fit in what one work-group may use (the flat kernel reads
      // edge_offset only for that layout)
      const int64_t tile_rows = a.images_per_tile == 1 ? a.rows_per_tile
                                                       : (int64_t)a.images_per_tile * H;
      const int64_t off = ((int64_t)a.lds_buffer_bytes + 15) / 16 * 16;
      const int64_t edge_bytes = (tile_rows + 1) * (16 / out_bytes) * (int64_t)sizeof(float);
      size_t flat_lds = lds;
      if (out_dtype == FN_OUT_FP16_PAD4 && off + edge_bytes <= lds_all) {
        a.edge_offset = (int32_t)off;
        flat_lds = tiles_lds_bytes(dev, (int32_t)(off + edge_bytes));
      }
      launch_flat(a, C, out_dtype, comp, (unsigned)a.total_tiles, flat_lds, st);
    }
    return launch_status("fused_flat_kernel launch");
  }
  if (px > 0) {
    a.groups_per_row = (uint32_t)(W / px);
    a.groups_per_image = (uint32_t)((int64_t)H * W / px);
    a.total_groups = N * (int64_t)a.groups_per_image;
    a.div_gpi = make_fast_div(a.groups_per_image);
    a.div_gpr = make_fast_div(a.groups_per_row);
    // groups per lane: as many as allowed while one work-group touches at
    // most kMaxImagesPerBlock images
    int iter = fn::kMaxIter;
    while (iter > 1 && (int64_t)fn::kBlock * iter > (int64_t)(fn::kMaxImagesPerBlock - 1) *
                                                         a.groups_per_image)
      --iter;
    if ((int64_t)fn::kBlock * iter <= (int64_t)(fn::kMaxImagesPerBlock - 1) * a.groups_per_image) {
      a.iter = iter;
      const int64_t per_block = (int64_t)fn::kBlock * iter;
      const int64_t grid = (a.total_groups + per_block - 1) / per_block;
      if (grid > 0x7FFFFFFF) return fail(FN_EOVERFLOW, "grid size limit exceeded");
      launch_grouped(a, C, px, out_dtype, (unsigned)grid, st);
      return launch_status("fused_grouped_kernel launch");
    }
  }
  const unsigned grid = (unsigned)(N * a.tiles_per_image);
  if (out_dtype == FN_OUT_FP32)
    fn::fused_generic_kernel<float><<<grid, fn::kBlock, 0, st>>>(a);
  else
    fn::fused_generic_kernel<_Float16><<<grid, fn::kBlock, 0, st>>>(a);
  return launch_status("fused_generic_kernel launch");
}

}  // namespace

FN_EXPORT int fn_fused_normalize(const uint8_t* in_u8_dev, int64_t N, int32_t H, int32_t W,
                                 int32_t C, const float* mean, const float* std, float flip_p,
                                 float erase_p, float scale_min, float scale_max, float ratio_min,
                                 float ratio_max, uint64_t seed, int32_t out_dtype, void* out_dev,
                                 void* stream) {
  return fused_normalize_impl(in_u8_dev, nullptr, N, H, W, C, mean, std, flip_p, erase_p,
                              scale_min, scale_max, ratio_min, ratio_max, seed, 0, out_dtype,
                              out_dev, stream);
}

FN_EXPORT int fn_fused_normalize_ex(const uint8_t* in_u8_dev, int64_t in_row_stride,
                                    int64_t in_image_stride, int64_t N, int32_t H, int32_t W,
                                    int32_t C, const float* mean, const float* std, float flip_p,
                                    float erase_p, float scale_min, float scale_max,
                                    float ratio_min, float ratio_max, uint64_t seed,
                                    int64_t first_sample_id, int32_t out_dtype, void* out_dev,
                                    void* stream) {
  const int64_t strides[2] = {in_row_stride, in_image_stride};
  return fused_normalize_impl(in_u8_dev, strides, N, H, W, C, mean, std, flip_p, erase_p,
                              scale_min, scale_max, ratio_min, ratio_max, seed, first_sample_id,
                              out_dtype, out_dev, stream);
}

FN_EXPORT int fn_test_erase_dims(const uint32_t* w_scale_dev, const uint32_t* w_ratio_dev,
                                 int64_t count, int32_t H, int32_t W, float scale_min,
                                 float scale_max, float ratio_min, float ratio_max,
                                 int32_t* eh_dev, int32_t* ew_dev, uint8_t* accepted_dev,
                                 void* stream) {
  fn::DrawArgs a;
  int rc = make_draw_args(0, H, W, 0.0f, 1.0f, scale_min, scale_max, ratio_min, ratio_max, &a);
  if (rc) return rc;
  if (count < 0) return fail(FN_EINVAL, "count must be >= 0");
  if (count > ((int64_t)1 << 36)) return fail(FN_EOVERFLOW, "count too large");
  if (count == 0) return ok();
  int dev = -1;
  if ((rc = check_device_range(w_scale_dev, count * 4, "w_scale_dev", &dev)) ||
      (rc = check_device_range(w_ratio_dev, count * 4, "w_ratio_dev", &dev)) ||
      (rc = check_device_range(eh_dev, count * 4, "eh_dev", &dev)) ||
      (rc = check_device_range(ew_dev, count * 4, "ew_dev", &dev)) ||
      (rc = check_device_range(accepted_dev, count, "accepted_dev", &dev)))
    return rc;
  fn::erase_dims_kernel<<<blocks_for(count, fn::kBlock), fn::kBlock, 0, (hipStream_t)stream>>>(
      a, w_scale_dev, w_ratio_dev, count, eh_dev, ew_dev, accepted_dev);
  return launch_status("erase_dims_kernel launch");
}

FN_EXPORT int fn_test_cr_ops(int32_t op, const float* a_dev, const float* b_dev, int64_t count,
                             float* out_dev, void* stream) {
  if (op < 0 || op > 2) return fail(FN_EINVAL, "op must be 0 (exp), 1 (sqrt) or 2 (div)");
  if (count < 0) return fail(FN_EINVAL, "count must be >= 0");
  if (count > ((int64_t)1 << 36)) return fail(FN_EOVERFLOW, "count too large");
  if (count == 0) return ok();
  int rc;
  int dev = -1;
  if ((rc = check_device_range(a_dev, count * 4, "a_dev", &dev)) ||
      (rc = check_device_range(out_dev, count * 4, "out_dev", &dev)))
    return rc;
  if (op == 2 && (rc = check_device_range(b_dev, count * 4, "b_dev", &dev))) return rc;
  fn::cr_ops_kernel<<<blocks_for(count, fn::kBlock), fn::kBlock, 0, (hipStream_t)stream>>>(
      op, a_dev, op == 2 ? b_dev : a_dev, count, out_dev);
  return launch_status("cr_ops_kernel launch");
}

FN_EXPORT int fn_test_timeline(void* stamps_dev, int64_t tiles) {
#if FN_TIMELINE
  if (tiles < 0) return fail(FN_EINVAL, "tiles must be >= 0");
  if (tiles > ((int64_t)1 << 31)) return fail(FN_EOVERFLOW, "tiles too large");
  if (tiles > 0) {
    if (stamps_dev == nullptr) return fail(FN_EINVAL, "stamps_dev must not be NULL");
    int dev = -1;
    const int rc = check_device_range(stamps_dev, (size_t)tiles * 4 * sizeof(uint64_t),
                                      "stamps_dev", &dev);
    if (rc) return rc;
  }
  g_timeline = tiles > 0 ? reinterpret_cast<uint64_t*>(stamps_dev) : nullptr;
  g_timeline_tiles = tiles;
  return ok();
#else
  (void)stamps_dev;
  (void)tiles;
  return fail(FN_EINVAL, "this library records no timeline (libfn_timeline.so does)");
#endif
}

FN_EXPORT int fn_test_stream(const void* src_dev, void* dst_dev, int64_t in_bytes, int32_t widen,
                             void* stream) {
  if (widen != 2 && widen != 4) return fail(FN_EINVAL, "widen must be 2 or 4");
  if (in_bytes < 0 || in_bytes % 16 != 0) return fail(FN_EINVAL, "in_bytes must be a multiple of 16");
  if ((((uintptr_t)src_dev | (uintptr_t)dst_dev) & 15u) != 0)
    return fail(FN_EINVAL, "src_dev and dst_dev must be 16-byte aligned");
  if (in_bytes > ((int64_t)1 << 40)) return fail(FN_EOVERFLOW, "in_bytes too large");
  if (in_bytes == 0) return ok();
  int rc;
  int dev = -1;
  if ((rc = check_device_range(src_dev, (size_t)in_bytes, "src_dev", &dev)) ||
      (rc = check_device_range(dst_dev, (size_t)(in_bytes * widen), "dst_dev", &dev)))
    return rc;
  const uintptr_t s0 = (uintptr_t)src_dev, d0 = (uintptr_t)dst_dev;
  if (s0 < d0 + (uintptr_t)(in_bytes * widen) && d0 < s0 + (uintptr_t)in_bytes)
    return fail(FN_EINVAL, "source and destination overlap");
  const int64_t lanes = in_bytes / (widen == 2 ? 8 : 16);
  const unsigned grid = blocks_for(lanes, fn::kBlock);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(src_dev);
  fn::u32x4* dst = reinterpret_cast<fn::u32x4*>(dst_dev);
  if (widen == 2)
    fn::stream_kernel<2><<<grid, fn::kBlock, 0, (hipStream_t)stream>>>(src, dst, lanes);
  else
    fn::stream_kernel<4><<<grid, fn::kBlock, 0, (hipStream_t)stream>>>(src, dst, lanes);
  return launch_status("stream_kernel launch");
}
