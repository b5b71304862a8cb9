// fn_kernels.hpp -- the GPU kernels of libfn.so (gfx950, wave64).
//
//   params_kernel        one wavefront per sample: the sample's decisions.
//   fused_kernel         the one-pass operation (page "(11)
//                        FusedNormalization", section 5): per work-group a
//                        tile of whole rows of one image; wave 0 draws the
//                        image's decisions, then every element is read from
//                        the mirrored or original column, normalized with one
//                        fma, zeroed inside the rectangle, and stored as fp32
//                        or round-to-nearest-even fp16.
//   erase_dims_kernel,
//   cr_ops_kernel,
//   copy_kernel          test and measurement hooks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fn_device.hpp"

namespace fn {

constexpr int kBlock = 256;  // four wave64 wavefronts

struct FusedArgs {
  const uint8_t* in;
  void* out;
  int64_t N;
  int32_t H, W, C;
  int32_t rows_per_tile, tiles_per_image;
  float mul[4];  // RN32(1 / (255 std_c))
  float sub[4];  // RN32(mean_c / std_c)
  DrawArgs draw;
};

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) params_kernel(DrawArgs a, int64_t N,
                                                        SampleParams* __restrict__ out) {
  const int64_t n = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  if (n >= N) return;  // whole wavefronts leave together
  const SampleParams p = draw_sample_params(a, (uint64_t)n);
  if ((threadIdx.x & 63u) == 0) out[n] = p;
}

// ---------------------------------------------------------------------------
template <typename OutT>
__device__ __forceinline__ OutT to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ _Float16 to_out<_Float16>(float v) {
  return (_Float16)v;  // v_cvt_f16_f32: round to nearest even
}

template <typename OutT>
__global__ void __launch_bounds__(kBlock) fused_kernel(FusedArgs a) {
  __shared__ SampleParams s_params;
  const int64_t n = blockIdx.x / a.tiles_per_image;
  const int tile = (int)(blockIdx.x % a.tiles_per_image);
  if (threadIdx.x < 64) {
    const SampleParams p = draw_sample_params(a.draw, (uint64_t)n);
    if (threadIdx.x == 0) s_params = p;
  }
  __syncthreads();
  const SampleParams p = s_params;

  const int32_t W = a.W, C = a.C;
  const int64_t row_elems = (int64_t)W * C;
  const int32_t h0 = tile * a.rows_per_tile;
  const int32_t h1 = min(a.H, h0 + a.rows_per_tile);
  const int64_t img_base = n * (int64_t)a.H * row_elems;
  const int64_t begin = img_base + (int64_t)h0 * row_elems;
  const int64_t count = (int64_t)(h1 - h0) * row_elems;
  OutT* __restrict__ out = reinterpret_cast<OutT*>(a.out);

  for (int64_t idx = threadIdx.x; idx < count; idx += kBlock) {
    const int32_t h = h0 + (int32_t)(idx / row_elems);
    const int32_t rem = (int32_t)(idx % row_elems);
    const int32_t w = rem / C;
    const int32_t c = rem - w * C;
    const bool erased = p.erase && h >= p.i && h < p.i + p.eh && w >= p.j && w < p.j + p.ew;
    float v = 0.0f;
    if (!erased) {
      const int32_t src_w = p.flip ? (W - 1 - w) : w;
      const uint8_t x = a.in[img_base + (int64_t)h * row_elems + (int64_t)src_w * C + c];
      v = __builtin_fmaf((float)x, a.mul[c], -a.sub[c]);
    }
    out[begin + idx] = to_out<OutT>(v);
  }
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) erase_dims_kernel(DrawArgs a,
                                                            const uint32_t* __restrict__ w_scale,
                                                            const uint32_t* __restrict__ w_ratio,
                                                            int64_t count, int32_t* __restrict__ eh,
                                                            int32_t* __restrict__ ew,
                                                            uint8_t* __restrict__ accepted) {
  const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (s >= count) return;
  const Attempt t = erase_attempt(a, w_scale[s], w_ratio[s]);
  eh[s] = t.eh == INT32_MAX ? -1 : t.eh;
  ew[s] = t.ew == INT32_MAX ? -1 : t.ew;
  accepted[s] = t.fits ? 1 : 0;
}

__global__ void __launch_bounds__(kBlock) cr_ops_kernel(int32_t op, const float* __restrict__ x,
                                                        const float* __restrict__ y, int64_t count,
                                                        float* __restrict__ out) {
  const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (s >= count) return;
  float r;
  if (op == 0) {
    r = cr_expf(x[s]);
  } else if (op == 1) {
    r = cr_sqrtf(x[s]);
  } else {
    r = cr_divf(x[s], y[s]);
  }
  out[s] = r;
}

__global__ void __launch_bounds__(kBlock) copy_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst, int64_t vecs) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t v = (int64_t)blockIdx.x * kBlock + threadIdx.x; v < vecs; v += stride)
    dst[v] = src[v];
}

}  // namespace fn
