// fn_kernels.hpp -- the GPU kernels of libfn.so (gfx950, wave64).
//
//   params_kernel          four samples per wavefront: each sample's decisions.
//   fused_tiles_kernel     the one-pass operation (page "(11)
//                          FusedNormalization", section 5), used whenever a
//                          row holds whole 16-byte output vectors and the
//                          output is 16-byte aligned: one tile of whole rows
//                          (or whole images) per work-group, staged in LDS by
//                          global-to-LDS DMA while the tile's decisions are
//                          drawn; each lane then writes 16-byte vectors of a
//                          row, reading flipped sources from LDS.
//   fused_flat_kernel      the same staging for the other outputs whose rows
//                          fit a tile: rows that end inside a 16-byte vector,
//                          or an output aligned only to its element size;
//                          lanes take the buffer's aligned 16-byte vectors,
//                          and the few that hold a row start are done element
//                          by element in a second pass.
//   fused_grouped_kernel   rows whose one-row tile would leave room for only
//                          one work-group per compute unit (or not fit at
//                          all), when the width is a multiple of a pixel
//                          group PX and the output is 16-byte aligned: each
//                          lane owns groups of PX consecutive pixels of one
//                          row; a flipped group reads the mirrored group of
//                          the same row and reverses the pixel order in
//                          registers, keeping the channel order; a group
//                          wholly inside the erase rectangle reads nothing.
//   fused_generic_kernel   any other row too wide for a tile, one element at
//                          a time.
//   Values are (x/255 - mean)/std from fp32 constant pairs (see
//   normalize()), stored as fp32 or round-to-nearest-even fp16.
//   erase_dims_kernel,
//   cr_ops_kernel,
//   stream_kernel          test and measurement hooks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fn_device.hpp"

namespace fn {

// Build-time tuning of the grouped kernel:
//   FN_GROUP_PX_MAX  widest pixel group tried (16, 8 or 4)
//   FN_GROUP_ITER    pixel groups per lane (1..4)
// and of the tiles kernel's lane-contiguous stores:
//   FN_NT_STORE      policy of its 16-byte stores: 0 default, 1
//                    non-temporal, 2 streaming system-scope (sc0 sc1 nt)
//   FN_NT_MIN_BYTES  fp16 launches moving at least this many bytes store
//                    non-temporal instead (0: never)
#ifndef FN_GROUP_PX_MAX
#define FN_GROUP_PX_MAX 16
#endif
#ifndef FN_GROUP_ITER
#define FN_GROUP_ITER 4
#endif
#ifndef FN_NT_STORE
#define FN_NT_STORE 2
#endif
#ifndef FN_NT_MIN_BYTES
#define FN_NT_MIN_BYTES 335544320
#endif

// Tiles kernel (defaults chosen by measurement):
//   FN_TILE_BYTES      most input bytes of one tile
//   FN_MIN_TILE_BYTES  smallest tile the plan shrinks to for small batches
//   FN_WGS_PER_CU      most work-groups resident on a compute unit (0: no
//                      cap); enforced through the LDS size each requests
//   FN_XCD_RUN         consecutive tiles one XCD takes in turn (1: tile =
//                      work-group index)
#ifndef FN_TILE_BYTES
#define FN_TILE_BYTES 8192
#endif
#ifndef FN_MIN_TILE_BYTES
#define FN_MIN_TILE_BYTES 2048
#endif
#ifndef FN_WGS_PER_CU
#define FN_WGS_PER_CU 6
#endif
#ifndef FN_XCD_RUN
#define FN_XCD_RUN 16
#endif
// FN_TIMELINE 1: the instrumented build (libfn_timeline.so), whose tiles
// kernel records four real-time-clock stamps per tile (fn_test_timeline);
// the product library is built with 0.
#ifndef FN_TIMELINE
#define FN_TIMELINE 0
#endif


constexpr int kBlock = 256;             // four wave64 wavefronts
constexpr int kTileBytesTarget = FN_TILE_BYTES;
constexpr int kMinTileBytes = FN_MIN_TILE_BYTES;
constexpr int kWgsPerCu = FN_WGS_PER_CU;
constexpr uint32_t kXcdRun = FN_XCD_RUN;
constexpr int kMaxImagesPerBlock = 16;  // images whose decisions one work-group draws
constexpr int kMaxIter = FN_GROUP_ITER;  // pixel groups per lane in the grouped kernel
constexpr int kGroupPxMax = FN_GROUP_PX_MAX;

// Division of 32-bit x by a fixed d >= 1 through a multiply-high and one
// correction (valid for x + d < 2^32): m = floor(2^32 / d) + 1 overestimates
// 1/d by less than 1/2^32, so mulhi(x, m) is x/d or x/d + 1.
struct FastDiv {
  uint32_t d, m;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t x, FastDiv f) {
  if (f.d == 1) return x;
  uint32_t q = __umulhi(x, f.m);
  if (q * f.d > x) --q;
  return q;
}

struct FusedArgs {
  const uint8_t* in;
  void* out;
  int64_t N;
  int32_t H, W, C;
  int32_t oc;                 // output channels per pixel: C, or 4 when padded
  // generic kernel: tiles of whole rows
  int32_t rows_per_tile, tiles_per_image;
  // grouped kernel
  int64_t total_groups;       // N * H * W / PX
  uint32_t groups_per_image;  // H * W / PX
  uint32_t groups_per_row;    // W / PX
  FastDiv div_gpi, div_gpr;
  int32_t iter;               // groups per lane, 1..kMaxIter
  // tiles kernel: a tile is rows_per_tile rows of one image, or
  // images_per_tile whole images
  int32_t images_per_tile;
  int64_t total_tiles;
  int32_t lds_buffer_bytes;   // the LDS staging buffer of one tile
  int64_t total_bytes;        // input bytes from the first to the last one read
  // input rows: row h of image n starts at in + n * in_image_stride +
  // h * in_row_stride; strided == 0 when that is the compact layout
  int64_t in_row_stride, in_image_stride;
  int32_t strided;
  int32_t row_slot;           // strided tiles: LDS bytes per row (16 * granules)
  FastDiv div_gps;            // by row_slot / 16
  FastDiv div_row;            // by W * C
  FastDiv div_row_out;        // by W * oc
  FastDiv div_h;              // by H
  FastDiv div_tpi;            // by tiles_per_image
  // tiles kernel lanes: output chunks per row (W * oc / E) and rows per pass
  // (work-group size / chunks per row, when at least 1)
  FastDiv div_cpr;
  int32_t rows_per_pass;
  // flat kernel: LDS byte offset of the row-start vectors' values (E floats
  // per row start of the tile); 0: the second pass stores them itself
  int32_t edge_offset;
  // 1 / (255 std_c) = mul + mul_lo and -mean_c / std_c = nsub + nsub_lo,
  // each the double value split into an fp32 pair (see normalize())
  float mul[4], mul_lo[4];
  float nsub[4], nsub_lo[4];
  DrawArgs draw;
#if FN_TIMELINE
  uint64_t* timeline;      // 4 stamps per tile, tiles < timeline_tiles
  int64_t timeline_tiles;  // 0: no recording
#endif
};

// (x/255 - mean)/std of one byte x from the constant pairs m = mh + ml
// (1/(255 std)) and n = nh + nl (-mean/std).  The first fma holds the part
// where x*m and n cancel exactly inside one rounding; the second adds the
// low parts.  The result is within about one fp32 ulp of the exact value
// relative to the result itself, also where the value is near zero (one fma
// on rounded constants errs there by up to ~1e-7 absolute, several fp16
// ulps of a tiny result).
// kComp false: the first fma alone.  The host takes that form only after
// checking, for every byte value of every channel, that it yields exactly
// the stored output of the two-fma form (see single_fma_exact in
// fn_api.hip), so both forms write the same bits.
template <bool kComp = true>
__device__ __forceinline__ float normalize(float x, float mh, float ml, float nh, float nl) {
  if constexpr (kComp) return __builtin_fmaf(x, mh, nh) + __builtin_fmaf(x, ml, nl);
  return __builtin_fmaf(x, mh, nh);
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) params_kernel(DrawArgs a, int64_t N,
                                                        SampleParams* __restrict__ out) {
  const int64_t first = (int64_t)blockIdx.x * (kBlock / 16);
  if (first + (int64_t)(threadIdx.x >> 6) * 4 >= N) return;  // whole wavefronts leave together
  const int64_t n = first + (threadIdx.x >> 4);
  const SampleParams p = draw_sample_params16(a, (uint64_t)n);
  if ((threadIdx.x & 15u) == 0 && n < N) out[n] = p;
}

// ---------------------------------------------------------------------------
// Draws the decisions of images n_first .. n_first + count - 1 (count <= 16)
// into s_params, 16 lanes per image; wavefronts with nothing to draw skip.
__device__ __forceinline__ void draw_block_params(const DrawArgs& a, int64_t n_first, int count,
                                                  SampleParams* s_params) {
  const int wave = (int)(threadIdx.x >> 6);
  if (wave * 4 < count) {
    const int slot = (int)(threadIdx.x >> 4);
    const SampleParams p = draw_sample_params16(a, (uint64_t)(n_first + slot));
    if ((threadIdx.x & 15u) == 0 && slot < count) s_params[slot] = p;
  }
  __syncthreads();
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int NB>
__device__ __forceinline__ void load_group(const uint8_t* __restrict__ p, uint32_t (&w)[NB / 4]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int v = 0; v < NB / 16; ++v) {
      const uint4 q = reinterpret_cast<const uint4*>(p)[v];
      w[4 * v] = q.x;
      w[4 * v + 1] = q.y;
      w[4 * v + 2] = q.z;
      w[4 * v + 3] = q.w;
    }
  } else if constexpr (NB % 8 == 0) {
#pragma unroll
    for (int v = 0; v < NB / 8; ++v) {
      const uint2 q = reinterpret_cast<const uint2*>(p)[v];
      w[2 * v] = q.x;
      w[2 * v + 1] = q.y;
    }
  } else {
#pragma unroll
    for (int v = 0; v < NB / 4; ++v) w[v] = reinterpret_cast<const uint32_t*>(p)[v];
  }
}

// One 16-byte store with the system-scope streaming policy (sc0 sc1 nt),
// which no compiler builtin expresses.  The compiler does not know that the
// asm is a store, so it does not keep the data VGPRs of a store wider than
// 8 bytes unwritten for the two wait states this chip needs before a VALU
// instruction may overwrite them; the s_nop after the store provides them
// (without it a value computed right after the store can reach memory in
// place of the stored one).
__device__ __forceinline__ void stream_store16(u32x4* p, u32x4 q) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 1" ::"v"(p), "v"(q) : "memory");
}

// Cache policy of a 16-byte output store.  kStoreSys (sc0 sc1 nt) writes
// through to memory at system scope: fastest where every 128-byte line is
// written whole by one store instruction (the tiles kernel) and the launch
// is short.  kStoreNt leaves lines in L2 until evicted: a line written in
// parts by different instructions leaves as one write (the flat kernel's
// lines at row starts), and long fp16 launches stream faster
// (kTilesNtMinBytes).  kStorePlain: lane-strided patterns, where
// non-temporal stores measured 3x slower.
enum StorePolicy : int { kStorePlain = 0, kStoreNt = 1, kStoreSys = 2 };
constexpr int kTilesStore = FN_NT_STORE;
// fp16 launches (packed or 4-channel) of at least this many algorithmic
// bytes store with kStoreNt; 0: never.  Measured on 224x224x3 batches:
// packed 2.5% faster at 2,048 images, 1-1.7% at 1,024, 1% slower at 512 and
// 256; 4-channel 2% faster at 2,048 and 0.6-1.7% at 1,024; fp32 output 1-2%
// slower at every size, so it keeps kTilesStore.
constexpr int64_t kTilesNtMinBytes = FN_NT_MIN_BYTES;

// Stores NE output values as 16-, 8- or 4-byte vectors; 16-byte vectors
// with the cache policy kPolicy.
template <typename OutT, int NE, int kPolicy = kStorePlain>
__device__ __forceinline__ void store_group(OutT* __restrict__ dst, const float (&v)[NE]) {
  constexpr int kBytes = NE * (int)sizeof(OutT);
  constexpr int kWords = kBytes / 4;
  uint32_t u[kWords];
  if constexpr (sizeof(OutT) == 4) {
#pragma unroll
    for (int e = 0; e < NE; ++e) u[e] = __float_as_uint(v[e]);
  } else {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < NE; e += 2) {
      const half2_t h = {to_out<_Float16>(v[e]), to_out<_Float16>(v[e + 1])};
      u[e / 2] = __builtin_bit_cast(uint32_t, h);
    }
  }
  if constexpr (kBytes % 16 == 0) {
#pragma unroll
    for (int s = 0; s < kWords / 4; ++s) {
      const u32x4 q = {u[4 * s], u[4 * s + 1], u[4 * s + 2], u[4 * s + 3]};
      u32x4* p = reinterpret_cast<u32x4*>(dst) + s;
      if constexpr (kPolicy == kStoreNt) {
        __builtin_nontemporal_store(q, p);
      } else if constexpr (kPolicy == kStoreSys) {
        stream_store16(p, q);
      } else {
        *p = q;
      }
    }
  } else if constexpr (kBytes % 8 == 0) {
#pragma unroll
    for (int s = 0; s < kWords / 2; ++s)
      reinterpret_cast<uint2*>(dst)[s] = make_uint2(u[2 * s], u[2 * s + 1]);
  } else {
#pragma unroll
    for (int s = 0; s < kWords; ++s) reinterpret_cast<uint32_t*>(dst)[s] = u[s];
  }
}

// One group's outputs from its (possibly mirrored) source bytes: pixel p of
// the output takes pixel PX-1-p of the source when flipped, channels in
// order; pixels whose bit is set in `erased` are +0.
template <int C, int PX, bool kFlip, bool kMasked>
__device__ __forceinline__ void group_values(const uint32_t (&w)[PX * C / 4], uint32_t erased,
                                             const FusedArgs& a, float (&v)[PX * C]) {
  constexpr int NW = PX * C / 4;
#pragma unroll
  for (int p = 0; p < PX; ++p) {
    const int sp = kFlip ? (PX - 1 - p) : p;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float x;
      switch (((sp * C + c) & 3)) {  // resolved at compile time
        case 0: x = (float)(w[(sp * C + c) >> 2] & 0xFFu); break;
        case 1: x = (float)((w[(sp * C + c) >> 2] >> 8) & 0xFFu); break;
        case 2: x = (float)((w[(sp * C + c) >> 2] >> 16) & 0xFFu); break;
        default: x = (float)(w[(sp * C + c) >> 2] >> 24); break;
      }
      float y = normalize(x, a.mul[c], a.mul_lo[c], a.nsub[c], a.nsub_lo[c]);
      if (kMasked) y = ((erased >> p) & 1u) ? 0.0f : y;
      v[p * C + c] = y;
    }
  }
  (void)NW;
}

template <int C, int PX, typename OutT>
__global__ void __launch_bounds__(kBlock) fused_grouped_kernel(FusedArgs a) {
  constexpr int NB = PX * C;  // input bytes (= output elements) per group
  constexpr uint32_t kAll = (PX >= 32) ? 0xFFFFFFFFu : ((1u << PX) - 1u);
  __shared__ SampleParams s_params[kMaxImagesPerBlock];

  const int64_t per_block = (int64_t)kBlock * a.iter;
  const int64_t g_begin = (int64_t)blockIdx.x * per_block;
  const int64_t g_end = min(g_begin + per_block, a.total_groups);
  const int64_t n_first = g_begin / a.groups_per_image;
  const int n_count = (int)((g_end - 1) / a.groups_per_image - n_first + 1);
  draw_block_params(a.draw, n_first, n_count, s_params);

  const uint32_t local0 = (uint32_t)(g_begin - n_first * (int64_t)a.groups_per_image);
  uint32_t words[kMaxIter][NB / 4];
  uint32_t erased[kMaxIter];
  int32_t flip[kMaxIter];
#pragma unroll
  for (int k = 0; k < kMaxIter; ++k) {
    erased[k] = kAll;
    flip[k] = 0;
    const int64_t g = g_begin + threadIdx.x + (int64_t)k * kBlock;
    if (k < a.iter && g < g_end) {
      const uint32_t local = local0 + threadIdx.x + (uint32_t)k * kBlock;
      const uint32_t img = fast_div(local, a.div_gpi);
      const uint32_t rem = local - img * a.groups_per_image;
      const uint32_t h = fast_div(rem, a.div_gpr);
      const uint32_t wg = rem - h * a.groups_per_row;  // group index within the row
      const SampleParams& P = s_params[img];
      uint32_t m = 0;
      if (P.erase && (int32_t)h >= P.i && (int32_t)h < P.i + P.eh) {
        const int32_t px0 = (int32_t)wg * PX;
        const int32_t lo = max(P.j - px0, 0), hi = min(P.j + P.ew - px0, PX);
        if (lo < hi) m = (kAll >> (PX - (hi - lo))) << lo;
      }
      erased[k] = m;
      flip[k] = P.flip;
      if (m != kAll) {
        const int64_t src = P.flip ? g + (int64_t)a.groups_per_row - 1 - 2 * (int64_t)wg : g;
        load_group<NB>(a.in + src * NB, words[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxIter; ++k) {
    const int64_t g = g_begin + threadIdx.x + (int64_t)k * kBlock;
    if (k < a.iter && g < g_end) {
      float v[NB];
      if (erased[k] == kAll) {
#pragma unroll
        for (int e = 0; e < NB; ++e) v[e] = 0.0f;
      } else if (erased[k] == 0) {
        if (flip[k])
          group_values<C, PX, true, false>(words[k], 0, a, v);
        else
          group_values<C, PX, false, false>(words[k], 0, a, v);
      } else {
        if (flip[k])
          group_values<C, PX, true, true>(words[k], erased[k], a, v);
        else
          group_values<C, PX, false, true>(words[k], erased[k], a, v);
      }
      store_group<OutT, NB>(reinterpret_cast<OutT*>(a.out) + g * NB, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Tiles of the tiles kernel: a tile is a run of whole rows -- rows_per_tile
// rows of one image (images_per_tile == 1), or images_per_tile whole images.
struct Tile {
  int64_t n_first;  // first image
  int32_t h0;       // first row in that image
  int32_t rows;     // rows in the tile (across images when several)
  int32_t images;   // images the tile touches
  int64_t pixel;    // index of the tile's first pixel, (n_first * H + h0) * W
  int64_t start;    // offset of the tile's first byte in the compact layout
  int32_t len;      // bytes of the tile in the compact layout (rows * W * C)
};

// The tile work-group b takes.  The dispatcher deals work-groups round-robin
// over the chip's 8 XCDs (b to XCD b mod 8), each with its own L2; with
// tile = b, neighbouring tiles, which share the 128-byte lines at their
// common edge, would always run on different XCDs.  Within each block of
// 8 * kXcdRun work-groups, work-group o takes tile (o mod 8) * kXcdRun +
// o / 8: every XCD works through runs of kXcdRun consecutive tiles, and the
// tiles in flight stay one contiguous front of the batch.  The grid's last
// partial block keeps tile = b.  Measured (runs of 16 against 1): up to 2%
// faster, nowhere slower; runs of 32-128 are slower, and eighths of the
// batch per XCD (eight separate fronts) 6-12% slower.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t grid) {
  constexpr uint32_t kBlockTiles = 8u * kXcdRun;
  if (kXcdRun <= 1u || b >= grid / kBlockTiles * kBlockTiles) return b;
  const uint32_t base = b / kBlockTiles * kBlockTiles, o = b - base;
  return base + (o % 8u) * kXcdRun + o / 8u;
}

__device__ __forceinline__ Tile tile_at(const FusedArgs& a, uint32_t t) {
  Tile T;
  const int32_t row = a.W * a.C;
  if (a.images_per_tile == 1) {
    const uint32_t n = fast_div(t, a.div_tpi);
    T.n_first = n;
    T.h0 = (int32_t)(t - n * (uint32_t)a.tiles_per_image) * a.rows_per_tile;
    T.rows = min(a.rows_per_tile, a.H - T.h0);
    T.images = 1;
  } else {
    T.n_first = (int64_t)t * a.images_per_tile;
    T.h0 = 0;
    T.images = (int32_t)min((int64_t)a.images_per_tile, a.N - T.n_first);
    T.rows = T.images * a.H;
  }
  T.pixel = (T.n_first * a.H + T.h0) * (int64_t)a.W;
  T.start = T.pixel * a.C;
  T.len = T.rows * row;
  return T;
}

// Image index (into s_params, relative to n_base) and image row of tile row r.
__device__ __forceinline__ void tile_row_image(const FusedArgs& a, const Tile& T, int64_t n_base,
                                               int32_t r, uint32_t* slot, int32_t* h) {
  if (a.images_per_tile == 1) {
    *slot = (uint32_t)(T.n_first - n_base);
    *h = T.h0 + r;
  } else {
    const uint32_t img = fast_div((uint32_t)r, a.div_h);
    *slot = (uint32_t)(T.n_first - n_base) + img;
    *h = r - (int32_t)img * a.H;
  }
}

// How a lane reads its source bytes from LDS (see ChunkSetup::values).
constexpr int kSrcAny = -1, kSrcFlip = 0, kSrcAligned = 1, kSrcBytes = 2;

// ---------------------------------------------------------------------------
// What one lane needs to turn the E elements of a row starting at element
// x0 into outputs, independent of the row: the channel of each element and
// its constants, and the byte offsets (from the row start) of its mirrored
// sources.  Element x = w*C + c takes byte (W-1-w)*C + c when flipped; with
// x0 = w0*C + c0 and rc_k = (c0 + k) mod C that byte is
// (W-1-w0)*C - c0 - k + 2 rc_k.
template <int C, int E, bool kComp>
struct ChunkSetup {
  int32_t x0;
  float mul[C], mul_lo[C], nsub[C], nsub_lo[C];  // rotated: element k uses index k % C
  int32_t mirror[E];      // mirrored source byte of element k, from the row start

  __device__ __forceinline__ ChunkSetup(const FusedArgs& a, int32_t first) : x0(first) {
    const int32_t w0 = x0 / C;
    const int32_t c0 = x0 - w0 * C;
    int32_t rc[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      int32_t cj = c0 + j;
      cj = cj >= C ? cj - C : cj;
      rc[j] = cj;
      float m = a.mul[0], ml = a.mul_lo[0], s = a.nsub[0], sl = a.nsub_lo[0];
#pragma unroll
      for (int cc = 1; cc < C; ++cc) {
        m = cj == cc ? a.mul[cc] : m;
        ml = cj == cc ? a.mul_lo[cc] : ml;
        s = cj == cc ? a.nsub[cc] : s;
        sl = cj == cc ? a.nsub_lo[cc] : sl;
      }
      mul[j] = m;
      mul_lo[j] = ml;
      nsub[j] = s;
      nsub_lo[j] = sl;
    }
    const int32_t base = (a.W - 1 - w0) * C - c0;
#pragma unroll
    for (int k = 0; k < E; ++k) mirror[k] = base - k + 2 * rc[k % C];
  }

  // Outputs of this lane's E elements of one row (LDS row start `row_lds`,
  // image row h, the image's decisions P).  kSrc says how the source bytes
  // are read: kSrcFlip mirrored bytes (P.flip set), kSrcAligned E/4 dwords
  // (row_lds + x0 4-byte aligned), kSrcBytes E/4 + 1 aligned dwords shifted
  // into place (any alignment; reads up to 3 bytes past the row, which the
  // staging buffer's slack covers); kSrcAny decides per call.
  template <int kSrc = kSrcAny>
  __device__ __forceinline__ void values(const uint8_t* s_tile, int32_t row_lds,
                                         const SampleParams& P, int32_t h, float (&v)[E]) const {
    float x[E];
    const int32_t src = row_lds + x0;
    const int mode = kSrc != kSrcAny ? kSrc : (P.flip ? kSrcFlip : ((src & 3) == 0 ? kSrcAligned
                                                                                  : kSrcBytes));
    if (mode == kSrcFlip) {
#pragma unroll
      for (int k = 0; k < E; ++k) x[k] = (float)s_tile[row_lds + mirror[k]];
    } else if (mode == kSrcAligned) {
      uint32_t wv[E / 4];
#pragma unroll
      for (int q = 0; q < E / 4; ++q) wv[q] = reinterpret_cast<const uint32_t*>(s_tile + src)[q];
#pragma unroll
      for (int k = 0; k < E; ++k) x[k] = (float)((wv[k >> 2] >> (8 * (k & 3))) & 0xFFu);
    } else {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(s_tile + (src & ~3));
      const uint32_t sh = (uint32_t)src & 3u;
      uint32_t wa[E / 4 + 1];
#pragma unroll
      for (int q = 0; q <= E / 4; ++q) wa[q] = w[q];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        // byte k of the window: v_alignbyte_b32 takes 4 bytes of hi:lo at a byte shift
        const uint32_t d = __builtin_amdgcn_alignbyte(wa[(k >> 2) + 1], wa[k >> 2], sh);
        x[k] = (float)((d >> (8 * (k & 3))) & 0xFFu);
      }
    }
#pragma unroll
    for (int k = 0; k < E; ++k)
      v[k] = normalize<kComp>(x[k], mul[k % C], mul_lo[k % C], nsub[k % C], nsub_lo[k % C]);
    if (P.erase && h >= P.i && h < P.i + P.eh) {
      const int32_t lo = P.j * C - x0, hi = (P.j + P.ew) * C - x0;
#pragma unroll
      for (int k = 0; k < E; ++k) v[k] = (k >= lo && k < hi) ? 0.0f : v[k];
    }
  }
};

// The padded fp16 layout (page sec. 8): every pixel has 4 output channels,
// channels c < C normalized, channels C..3 +0.  A lane's 8 outputs are two
// whole pixels w0, w0 + 1 (x0 = 4 w0); pixel w takes source pixel W-1-w when
// flipped, channels in order; an erased pixel is +0 in every channel.
template <int C, bool kComp>
struct Pad4Chunk {
  int32_t x0;
  int32_t w0;
  int32_t direct, mirror;  // source byte of pixel w0, from the row start, unflipped / flipped
  float mul[C], mul_lo[C], nsub[C], nsub_lo[C];

  __device__ __forceinline__ Pad4Chunk(const FusedArgs& a, int32_t first) : x0(first) {
    w0 = first >> 2;
    direct = w0 * C;
    mirror = (a.W - 1 - w0) * C;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      mul[c] = a.mul[c];
      mul_lo[c] = a.mul_lo[c];
      nsub[c] = a.nsub[c];
      nsub_lo[c] = a.nsub_lo[c];
    }
  }

  template <int kSrc = kSrcAny>
  __device__ __forceinline__ void values(const uint8_t* s_tile, int32_t row_lds,
                                         const SampleParams& P, int32_t h, float (&v)[8]) const {
    const bool flip = kSrc != kSrcAny ? kSrc == kSrcFlip : P.flip != 0;
    // the two source pixels are 2C contiguous bytes: w0, w0 + 1 unflipped,
    // W-2-w0, W-1-w0 (output pixels 1, 0) flipped; read as three aligned
    // dwords shifted into place
    const int32_t b = row_lds + (flip ? mirror - C : direct);
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(s_tile + (b & ~3));
    const uint32_t sh = (uint32_t)b & 3u;
    const uint32_t w0w = wp[0], w1w = wp[1], w2w = wp[2];
    const uint32_t d[2] = {__builtin_amdgcn_alignbyte(w1w, w0w, sh),
                           __builtin_amdgcn_alignbyte(w2w, w1w, sh)};
    bool er[2] = {false, false};
    if (P.erase && h >= P.i && h < P.i + P.eh) {
      er[0] = w0 >= P.j && w0 < P.j + P.ew;
      er[1] = w0 + 1 >= P.j && w0 + 1 < P.j + P.ew;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int sp = flip ? 1 - p : p;  // source pixel of output pixel p
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < C) {
          const int j = sp * C + c;  // byte of the window
          const float x = (float)((d[j >> 2] >> (8 * (j & 3))) & 0xFFu);
          v[4 * p + c] = er[p] ? 0.0f : normalize<kComp>(x, mul[c], mul_lo[c], nsub[c], nsub_lo[c]);
        } else {
          v[4 * p + c] = 0.0f;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Wavefronts first .. first + count - 1 of the work-group move tile T's input
// bytes into `buf` (byte b of the tile at buf[head + b], head = the tile
// start's offset within its 16-byte granule): batch k of 64 granules goes to
// wavefront first + (k mod count) as one global-to-LDS DMA load.  Granules
// that straddle the ends of the input buffer are read byte by byte.  `index`
// = this wavefront's number minus `first`; both are wavefront-uniform.
__device__ __forceinline__ void load_tile_waves(const FusedArgs& a, const Tile& T, uint8_t* buf,
                                                int32_t index, int32_t count) {
  const int lane = (int)(threadIdx.x & 63u);
  const uintptr_t in_lo = (uintptr_t)a.in, in_hi = in_lo + (uintptr_t)a.total_bytes;
  const uintptr_t t_lo = in_lo + (uintptr_t)T.start;
  const uintptr_t gbase = t_lo & ~(uintptr_t)15;
  const int32_t head = (int32_t)(t_lo - gbase);
  const int32_t ngran = (head + T.len + 15) >> 4;
  const bool interior = gbase >= in_lo && gbase + 16 * (uintptr_t)ngran <= in_hi;
  if (interior) {
    // every granule lies inside the buffer (all tiles but the edges of an
    // unaligned batch): a wavefront-uniform base plus the lane's 16 bytes
    const uint8_t* src = reinterpret_cast<const uint8_t*>(gbase) + 16 * lane;
    for (int32_t batch = 64 * index; batch < ngran; batch += 64 * count) {
      if (batch + lane < ngran)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + 16 * batch),
                                         (__attribute__((address_space(3))) void*)(buf + 16 * batch),
                                         16, 0, 0);
    }
    return;
  }
  for (int32_t batch = 64 * index; batch < ngran; batch += 64 * count) {
    const int32_t g = batch + lane;
    const uintptr_t A = gbase + 16 * (uintptr_t)g;
    if (g < ngran && A >= in_lo && A + 16 <= in_hi) {
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(A),
                                       (__attribute__((address_space(3))) void*)(buf + 16 * batch),
                                       16, 0, 0);
    } else if (g < ngran) {
      for (int b = 0; b < 16; ++b) {
        const uintptr_t addr = A + (uintptr_t)b;
        if (addr >= in_lo && addr < in_hi) buf[16 * g + b] = *reinterpret_cast<const uint8_t*>(addr);
      }
    }
  }
}

// First input byte of row r of tile T in a strided source.  A tile of one
// image is a base plus r row strides.
__device__ __forceinline__ uintptr_t tile_row_src(const FusedArgs& a, const Tile& T, int32_t r) {
  if (a.images_per_tile == 1)
    return (uintptr_t)a.in + (uintptr_t)(T.n_first * a.in_image_stride +
                                         (int64_t)(T.h0 + r) * a.in_row_stride);
  uint32_t slot;
  int32_t h;
  tile_row_image(a, T, T.n_first, r, &slot, &h);
  return (uintptr_t)a.in + (uintptr_t)(((int64_t)T.n_first + slot) * a.in_image_stride +
                                       (int64_t)h * a.in_row_stride);
}

// The strided counterpart of load_tile_waves: row r of the tile is staged at
// buf + r * row_slot, its first byte at offset head_r = (its address & 15).
// Granule q of the tile is granule q mod gps of row q / gps (gps = row_slot
// / 16) and lands at buf + 16 q, so a batch of 64 granules is still one DMA
// per wavefront; granules past the end of a row are not read.
__device__ __forceinline__ void load_tile_rows_waves(const FusedArgs& a, const Tile& T,
                                                     uint8_t* buf, int32_t index,
                                                     int32_t count) {
  const int lane = (int)(threadIdx.x & 63u);
  const uintptr_t in_lo = (uintptr_t)a.in, in_hi = in_lo + (uintptr_t)a.total_bytes;
  const int32_t row = a.W * a.C;
  const int32_t gps = a.row_slot >> 4;
  const int32_t ngran = T.rows * gps;
  for (int32_t batch = 64 * index; batch < ngran; batch += 64 * count) {
    const int32_t q = batch + lane;
    const int32_t r = (int32_t)fast_div((uint32_t)q, a.div_gps);
    const int32_t g = q - r * gps;
    const uintptr_t src = tile_row_src(a, T, min(r, T.rows - 1));
    const int32_t head = (int32_t)(src & 15u);
    const uintptr_t A = (src & ~(uintptr_t)15) + 16 * (uintptr_t)g;
    const bool needed = q < ngran && 16 * g < head + row;
    if (needed && A >= in_lo && A + 16 <= in_hi) {
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(A),
                                       (__attribute__((address_space(3))) void*)(buf + 16 * batch),
                                       16, 0, 0);
    } else if (needed) {
      for (int b = 0; b < 16; ++b) {
        const uintptr_t addr = A + (uintptr_t)b;
        if (addr >= in_lo && addr < in_hi) buf[16 * q + b] = *reinterpret_cast<const uint8_t*>(addr);
      }
    }
  }
}

// Work-group size of the tiles kernel: 256 lanes for 8-element (fp16) chunks,
// 512 for 4-element (fp32) chunks, so that a pass covers whole rows of
// typical widths with few idle lanes.
#ifndef FN_TILE_THREADS_F16
#define FN_TILE_THREADS_F16 256
#endif
template <typename OutT>
constexpr int tiles_threads() {
  return sizeof(OutT) == 2 ? FN_TILE_THREADS_F16 : 512;
}

// Stages tile T in LDS and its images' decisions in s_params, for the tiles
// kernels: every wavefront issues its share of the tile's global-to-LDS DMA
// loads first; then the first ceil(images / 4) wavefronts draw the decisions
// of the tile's images (a 16-lane group per image) while the loads are in
// flight.  Ends with a barrier, after which the whole tile is in LDS.
template <int kWaves>
__device__ __forceinline__ void stage_tile(const FusedArgs& a, const Tile& T, uint8_t* s_lds,
                                           SampleParams* s_params) {
  const int n_count = T.images;
  const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
  const int32_t draw_waves = min(kWaves, (n_count + 3) >> 2);
  if (a.strided)
    load_tile_rows_waves(a, T, s_lds, wave, kWaves);
  else
    load_tile_waves(a, T, s_lds, wave, kWaves);
  if (wave < draw_waves) {
    const int slot = (int)(threadIdx.x >> 4);
    const SampleParams p = draw_sample_params16(a.draw, (uint64_t)(T.n_first + slot));
    if ((threadIdx.x & 15u) == 0 && slot < n_count) s_params[slot] = p;
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's DMA loads have landed
  __syncthreads();
}

// LDS offset of the first byte of row r of a staged tile (head = the offset
// of a compact tile's first byte, row = W * C).
__device__ __forceinline__ int32_t staged_row(const FusedArgs& a, const Tile& T, int32_t head,
                                              int32_t row, int32_t r) {
  if (a.strided) return r * a.row_slot + (int32_t)(tile_row_src(a, T, r) & 15u);
  return head + r * row;
}

#if FN_TIMELINE
// Instrumented builds: the stamps of tile t, from the 100 MHz real-time
// clock: work-group start, staged (after the staging barrier), stores
// issued (wavefront 0) and stores acknowledged (every wavefront, after
// waiting for its stores).  The wait and barrier at the end are the only
// work the instrumentation adds.
__device__ __forceinline__ void timeline_record(const FusedArgs& a, uint32_t t, uint64_t start,
                                                uint64_t staged) {
  const uint64_t issued = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint64_t acked = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0 && a.timeline != nullptr && (int64_t)t < a.timeline_tiles) {
    uint64_t* d = a.timeline + 4 * (size_t)t;
    d[0] = start;
    d[1] = staged;
    d[2] = issued;
    d[3] = acked;
  }
}
#endif

// The fused pass, one tile per work-group (grid = total_tiles): the tile is
// staged (stage_tile), then every lane makes E = 16/sizeof(OutT) consecutive
// output elements of a row at a time (two whole 4-channel pixels when kPad4)
// and stores them as one 16-byte vector, lane-contiguous across the
// wavefront.  A tile of one image reads its decisions into scalar registers
// and picks the way its source bytes are read (mirrored, aligned dwords or
// bytes) once.  Many small independent work-groups per compute unit hide the
// memory latency.
// Requires W*OC a multiple of E (OC = 4 when kPad4, else C) and a 16-byte
// aligned output; the input may be compact or strided (a.strided).  kStore:
// the cache policy of the stores.
template <int C, typename OutT, bool kPad4, bool kComp, int kStore = kTilesStore>
__global__ void __launch_bounds__(tiles_threads<OutT>()) fused_tiles_kernel(FusedArgs a) {
  constexpr int kThreads = tiles_threads<OutT>();
  constexpr int kWaves = kThreads / 64;
  constexpr int E = 16 / (int)sizeof(OutT);
  constexpr int OC = kPad4 ? 4 : C;  // output channels per pixel
  static_assert(!kPad4 || E == 8, "the padded layout is fp16: two pixels per 16-byte vector");
  using Setup = typename std::conditional<kPad4, Pad4Chunk<C, kComp>, ChunkSetup<C, E, kComp>>::type;
  extern __shared__ __align__(16) uint8_t s_lds[];
  __shared__ SampleParams s_params[kMaxImagesPerBlock];

#if FN_TIMELINE
  const uint64_t tl_start = __builtin_amdgcn_s_memrealtime();
#endif
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const Tile T = tile_at(a, tile);
  stage_tile<kWaves>(a, T, s_lds, s_params);
#if FN_TIMELINE
  const uint64_t tl_staged = __builtin_amdgcn_s_memrealtime();
#endif

  const int32_t head = (int32_t)(((uintptr_t)a.in + (uintptr_t)T.start) & 15u);
  const int32_t row = a.W * C;        // input bytes of a row
  auto row_lds = [&](int32_t r) -> int32_t { return staged_row(a, T, head, row, r); };
  const int32_t row_out = a.W * OC;   // output elements of a row
  const int32_t cpr = row_out / E;    // chunks per row
  const int ct = (int)threadIdx.x;
  OutT* __restrict__ out = reinterpret_cast<OutT*>(a.out) + T.pixel * OC;
  // A tile of one image reads its decision record into registers once;
  // tiles of several images look up each row's record.
  const bool single = a.images_per_tile == 1;
  const SampleParams P0 = s_params[0];
  if (cpr <= kThreads) {
    const int32_t rpi = a.rows_per_pass;  // kThreads / cpr
    const int32_t slot_row = (int32_t)fast_div((uint32_t)ct, a.div_cpr);
    if (slot_row < rpi) {
      const Setup cs(a, (ct - slot_row * cpr) * E);
      if (single) {
        // The tile's decisions are the same in every lane: keep them in
        // scalar registers, and pick the way source bytes are read once per
        // tile (a scalar branch) instead of per row and lane.
        SampleParams P;
        P.flip = __builtin_amdgcn_readfirstlane(P0.flip);
        P.erase = __builtin_amdgcn_readfirstlane(P0.erase);
        P.i = __builtin_amdgcn_readfirstlane(P0.i);
        P.j = __builtin_amdgcn_readfirstlane(P0.j);
        P.eh = __builtin_amdgcn_readfirstlane(P0.eh);
        P.ew = __builtin_amdgcn_readfirstlane(P0.ew);
        auto rows = [&](auto mode) {
          constexpr int kSrc = decltype(mode)::value;
          if (a.strided) {
            for (int32_t r = slot_row; r < T.rows; r += rpi) {
              float v[E];
              cs.template values<kSrc>(s_lds, row_lds(r), P, T.h0 + r, v);
              store_group<OutT, E, kStore>(out + (int64_t)r * row_out + cs.x0, v);
            }
          } else {
            // compact rows: LDS start and output advance by fixed steps
            int32_t lds = head + slot_row * row;
            OutT* dst = out + (int64_t)slot_row * row_out + cs.x0;
            for (int32_t r = slot_row; r < T.rows; r += rpi) {
              float v[E];
              cs.template values<kSrc>(s_lds, lds, P, T.h0 + r, v);
              store_group<OutT, E, kStore>(dst, v);
              lds += rpi * row;
              dst += (int64_t)rpi * row_out;
            }
          }
        };
        // compact rows start at head + r * row: all 4-byte aligned when both are
        const bool aligned = !a.strided && ((head | row) & 3) == 0;
        if (P.flip)
          rows(std::integral_constant<int, kSrcFlip>());
        else if (a.strided)  // each strided row has its own alignment
          rows(std::integral_constant<int, kSrcAny>());
        else if (aligned)
          rows(std::integral_constant<int, kSrcAligned>());
        else
          rows(std::integral_constant<int, kSrcBytes>());
      } else {
        for (int32_t r = slot_row; r < T.rows; r += rpi) {
          uint32_t slot;
          int32_t h;
          tile_row_image(a, T, T.n_first, r, &slot, &h);
          const SampleParams P = s_params[slot];
          float v[E];
          cs.values(s_lds, row_lds(r), P, h, v);
          store_group<OutT, E, kStore>(out + (int64_t)r * row_out + cs.x0, v);
        }
      }
    }
  } else if (single) {
    // Rows wider than one pass of the lanes: lane ct takes the chunk columns
    // ct, ct + kThreads, ... and each column down all rows of the tile, so
    // one lane setup serves the whole column; the decisions sit in scalar
    // registers and the source read form is picked once, as above.
    SampleParams P;
    P.flip = __builtin_amdgcn_readfirstlane(P0.flip);
    P.erase = __builtin_amdgcn_readfirstlane(P0.erase);
    P.i = __builtin_amdgcn_readfirstlane(P0.i);
    P.j = __builtin_amdgcn_readfirstlane(P0.j);
    P.eh = __builtin_amdgcn_readfirstlane(P0.eh);
    P.ew = __builtin_amdgcn_readfirstlane(P0.ew);
    auto columns = [&](auto mode) {
      constexpr int kSrc = decltype(mode)::value;
      for (int32_t c = ct; c < cpr; c += kThreads) {
        const Setup cs(a, c * E);
        for (int32_t r = 0; r < T.rows; ++r) {
          float v[E];
          cs.template values<kSrc>(s_lds, row_lds(r), P, T.h0 + r, v);
          store_group<OutT, E, kStore>(out + (int64_t)r * row_out + cs.x0, v);
        }
      }
    };
    const bool aligned = !a.strided && ((head | row) & 3) == 0;
    if (P.flip)
      columns(std::integral_constant<int, kSrcFlip>());
    else if (a.strided)
      columns(std::integral_constant<int, kSrcAny>());
    else if (aligned)
      columns(std::integral_constant<int, kSrcAligned>());
    else
      columns(std::integral_constant<int, kSrcBytes>());
  } else {
    const int32_t nchunks = T.rows * cpr;
    for (int32_t q = ct; q < nchunks; q += kThreads) {
      const int32_t off = q * E;
      const uint32_t r = fast_div((uint32_t)off, a.div_row_out);
      const int32_t x0 = off - (int32_t)r * row_out;
      uint32_t slot;
      int32_t h;
      tile_row_image(a, T, T.n_first, (int32_t)r, &slot, &h);
      const SampleParams P = s_params[slot];
      const Setup cq(a, x0);
      float v[E];
      cq.values(s_lds, row_lds((int32_t)r), P, h, v);
      store_group<OutT, E, kStore>(out + off, v);
    }
  }
#if FN_TIMELINE
  timeline_record(a, tile, tl_start, tl_staged);
#endif
}

// Normalized value of input byte x in channel c (a lane-varying c < C).
template <int C, bool kComp>
__device__ __forceinline__ float normalize_channel(const FusedArgs& a, float x, int32_t c) {
  float m = a.mul[0], ml = a.mul_lo[0], n = a.nsub[0], nl = a.nsub_lo[0];
#pragma unroll
  for (int cc = 1; cc < C; ++cc) {
    m = c == cc ? a.mul[cc] : m;
    ml = c == cc ? a.mul_lo[cc] : ml;
    n = c == cc ? a.nsub[cc] : n;
    nl = c == cc ? a.nsub_lo[cc] : nl;
  }
  return normalize<kComp>(x, m, ml, n, nl);
}

// Output l of a staged tile (l relative to the tile's first output).
template <int C, int OC, bool kComp>
__device__ __forceinline__ float flat_element(const FusedArgs& a, const Tile& T,
                                              const uint8_t* s_lds, const SampleParams* s_params,
                                              int32_t head, int32_t l) {
  const int32_t row = a.W * C;
  const int32_t row_out = a.W * OC;
  const int32_t r = (int32_t)fast_div((uint32_t)l, a.div_row_out);
  const int32_t x = l - r * row_out;
  const int32_t w = x / OC;
  const int32_t c = x - w * OC;
  uint32_t slot;
  int32_t h;
  tile_row_image(a, T, T.n_first, r, &slot, &h);
  const SampleParams P = s_params[slot];
  const bool erased = P.erase && h >= P.i && h < P.i + P.eh && w >= P.j && w < P.j + P.ew;
  if (c >= C || erased) return 0.0f;
  const int32_t sw = P.flip ? a.W - 1 - w : w;
  const float xb = (float)s_lds[staged_row(a, T, head, row, r) + sw * C + c];
  return normalize_channel<C, kComp>(a, xb, c);
}

// Outputs l0 .. l0 + E - 1 of a staged tile, one at a time; those outside
// the tile (count outputs) are left 0.
template <int C, int OC, int E, bool kComp>
__device__ __forceinline__ void flat_elements(const FusedArgs& a, const Tile& T,
                                              const uint8_t* s_lds, const SampleParams* s_params,
                                              int32_t head, int32_t l0, int32_t count,
                                              float (&v)[E]) {
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int32_t l = l0 + k;
    v[k] = l >= 0 && l < count ? flat_element<C, OC, kComp>(a, T, s_lds, s_params, head, l) : 0.0f;
  }
}

// The fused pass for outputs that the lane layout of fused_tiles_kernel does
// not fit: rows of W*OC outputs that are not a whole number of 16-byte
// vectors, or an output aligned only to its element size.  The tile is
// staged as there.  Its outputs are the count contiguous elements from f0 on,
// covered by the 16-byte-aligned vectors of the output buffer.  A vector
// inside one row (and, when kPad4, starting at a pixel) is one chunk,
// evaluated as in fused_tiles_kernel with its own lane setup; the lanes take
// those first, one vector each in turn.  The other vectors hold a row start
// (or the tile's end) at an element other than their first: a second pass
// walks the tile's row starts and gives each element of such a vector a lane
// of its own, so that the few of them neither hold up whole wavefronts of the
// first pass nor leave a few lanes working alone.  Only the tile's own
// elements are stored: the tile next to it stores the rest of a vector they
// share, so no byte is written twice.  All stores are non-temporal
// (kStoreNt): the lines that the two passes (or two tiles) write in parts
// then merge in L2 instead of reaching memory as partial writes.  For the
// padded layout the second pass runs first and leaves the values of the
// row-start vectors inside the tile in LDS (a.edge_offset), and the first
// pass stores them with their neighbours.
template <int C, typename OutT, bool kPad4, bool kComp>
__global__ void __launch_bounds__(tiles_threads<OutT>()) fused_flat_kernel(FusedArgs a) {
  constexpr int kThreads = tiles_threads<OutT>();
  constexpr int kWaves = kThreads / 64;
  constexpr int E = 16 / (int)sizeof(OutT);
  constexpr int OC = kPad4 ? 4 : C;
  using Setup = typename std::conditional<kPad4, Pad4Chunk<C, kComp>, ChunkSetup<C, E, kComp>>::type;
  extern __shared__ __align__(16) uint8_t s_lds[];
  __shared__ SampleParams s_params[kMaxImagesPerBlock];

  const Tile T = tile_at(a, xcd_tile(blockIdx.x, gridDim.x));
  stage_tile<kWaves>(a, T, s_lds, s_params);

  const int32_t head = (int32_t)(((uintptr_t)a.in + (uintptr_t)T.start) & 15u);
  const int32_t row = a.W * C;
  const int32_t row_out = a.W * OC;
  const int32_t count = T.rows * row_out;  // outputs of the tile
  // element e of the output lies at out + e * sizeof(OutT); vector k of the
  // buffer holds elements k*E - mu .. k*E - mu + E - 1
  const int32_t mu = (int32_t)(((uintptr_t)a.out & 15u) / sizeof(OutT));
  const int64_t f0 = T.pixel * OC;                    // the tile's first output
  const int64_t k0 = (f0 + mu) / E;                   // first vector it overlaps
  const int32_t nvec = (int32_t)((f0 + count + mu + E - 1) / E - k0);
  // padded outputs off a pixel boundary: no vector starts at a pixel
  const bool all_elements = kPad4 && (mu & 3) != 0;
  OutT* __restrict__ out = reinterpret_cast<OutT*>(a.out);
  // the padded layout hands its row-start vectors to the first pass
  // through LDS (second_pass below); the other layouts measured faster
  // storing them in the second pass
  float* edge = nullptr;
  if constexpr (kPad4) {
    if (a.edge_offset > 0 && !all_elements) edge = reinterpret_cast<float*>(s_lds + a.edge_offset);
  }

  // a tile of one image reads its decisions into scalar registers once
  // (measured: 2% faster on padded 299-wide rows, level elsewhere)
  const bool single = a.images_per_tile == 1;
  SampleParams Pu;
  {
    const SampleParams P0 = s_params[0];
    Pu.flip = __builtin_amdgcn_readfirstlane(P0.flip);
    Pu.erase = __builtin_amdgcn_readfirstlane(P0.erase);
    Pu.i = __builtin_amdgcn_readfirstlane(P0.i);
    Pu.j = __builtin_amdgcn_readfirstlane(P0.j);
    Pu.eh = __builtin_amdgcn_readfirstlane(P0.eh);
    Pu.ew = __builtin_amdgcn_readfirstlane(P0.ew);
  }
  auto first_pass = [&](auto single_c) {
    constexpr bool kSingle = decltype(single_c)::value;
    for (int32_t q = (int32_t)threadIdx.x; q < nvec; q += kThreads) {
      const int64_t e0 = (k0 + q) * E - mu;
      const int32_t l0 = (int32_t)(e0 - f0);
      float v[E];
      if (all_elements) {
        flat_elements<C, OC, E, kComp>(a, T, s_lds, s_params, head, l0, count, v);
        if (l0 >= 0 && l0 + E <= count) {
          store_group<OutT, E, kStoreNt>(out + e0, v);
        } else {
#pragma unroll
          for (int k = 0; k < E; ++k)
            if (l0 + k >= 0 && l0 + k < count)
              __builtin_nontemporal_store(to_out<OutT>(v[k]), out + e0 + k);
        }
        continue;
      }
      if (l0 < 0 || l0 + E > count) continue;  // an end of the tile: second pass
      const int32_t r = (int32_t)fast_div((uint32_t)l0, a.div_row_out);
      const int32_t x0 = l0 - r * row_out;
      if (x0 + E > row_out) {
        // holds the next row's start: the second pass has left its values
        // in LDS (or stores it itself when they do not fit there)
        if (edge == nullptr) continue;
#pragma unroll
        for (int k = 0; k < E; ++k) v[k] = edge[(r + 1) * E + k];
        store_group<OutT, E, kStoreNt>(out + e0, v);
        continue;
      }
      int32_t h;
      SampleParams P;
      if constexpr (kSingle) {
        h = T.h0 + r;
        P = Pu;
      } else {
        uint32_t slot;
        tile_row_image(a, T, T.n_first, r, &slot, &h);
        P = s_params[slot];
      }
      const Setup cs(a, x0);
      // one read form per image: shifted dwords serve every alignment, so the
      // lanes of a wavefront that spans two rows of different alignment do
      // not split
      if (P.flip)
        cs.template values<kSrcFlip>(s_lds, staged_row(a, T, head, row, r), P, h, v);
      else
        cs.template values<kSrcBytes>(s_lds, staged_row(a, T, head, row, r), P, h, v);
      store_group<OutT, E, kStoreNt>(out + e0, v);
    }
  };
  // second pass: the vector holding the start of row b (b = T.rows: the
  // tile's end) when that is not its first element, one element per lane
  // (E lanes per vector); a vector holding several row starts is done at
  // the first of them.  A vector inside the tile goes to LDS (edge) when
  // there is room, for the first pass to store it with its neighbours: a
  // line written by one store instruction leaves L2 whole, one written in
  // two parts a microsecond apart often leaves in two.
  auto second_pass = [&]() {
    const int32_t n2 = (T.rows + 1) * E;
    for (int32_t t = (int32_t)threadIdx.x; t < n2; t += kThreads) {
      const int32_t b = t / E;
      const int32_t k = t - b * E;
      const int64_t e = f0 + (int64_t)b * row_out + mu;  // shifted element index
      if (e % E == 0) continue;
      const int64_t kv = e / E;
      if (b > 0) {
        const int64_t ep = e - row_out;
        if (ep % E != 0 && ep / E == kv) continue;
      }
      const int64_t e0 = kv * E - mu;
      const int32_t lv = (int32_t)(e0 - f0);
      const int32_t l = lv + k;
      if (l < 0 || l >= count) continue;
      const float y = flat_element<C, OC, kComp>(a, T, s_lds, s_params, head, l);
      if (edge != nullptr && lv >= 0 && lv + E <= count)
        edge[b * E + k] = y;
      else
        __builtin_nontemporal_store(to_out<OutT>(y), out + e0 + k);
    }
  };
  if (all_elements) {
    if (single)
      first_pass(std::true_type());
    else
      first_pass(std::false_type());
    return;
  }
  if (edge != nullptr) {
    second_pass();
    __syncthreads();
  }
  if (single)
    first_pass(std::true_type());
  else
    first_pass(std::false_type());
  if (edge == nullptr) second_pass();
}

// ---------------------------------------------------------------------------
template <typename OutT>
__global__ void __launch_bounds__(kBlock) fused_generic_kernel(FusedArgs a) {
  __shared__ SampleParams s_params[kMaxImagesPerBlock];
  const int64_t n = blockIdx.x / a.tiles_per_image;
  const int tile = (int)(blockIdx.x % a.tiles_per_image);
  draw_block_params(a.draw, n, 1, s_params);
  const SampleParams p = s_params[0];

  const int32_t W = a.W, C = a.C, OC = a.oc;
  const int64_t row_out = (int64_t)W * OC;   // output elements of a row
  const int32_t h0 = tile * a.rows_per_tile;
  const int32_t h1 = min(a.H, h0 + a.rows_per_tile);
  const int64_t img_base = n * a.in_image_stride;
  const int64_t begin = (n * (int64_t)a.H + h0) * row_out;
  const int64_t count = (int64_t)(h1 - h0) * row_out;
  OutT* __restrict__ out = reinterpret_cast<OutT*>(a.out);

  for (int64_t idx = threadIdx.x; idx < count; idx += kBlock) {
    const int32_t h = h0 + (int32_t)(idx / row_out);
    const int32_t rem = (int32_t)(idx % row_out);
    const int32_t w = rem / OC;
    const int32_t c = rem - w * OC;
    const bool erased = p.erase && h >= p.i && h < p.i + p.eh && w >= p.j && w < p.j + p.ew;
    float v = 0.0f;
    if (!erased && c < C) {
      const int32_t src_w = p.flip ? (W - 1 - w) : w;
      const uint8_t x = a.in[img_base + (int64_t)h * a.in_row_stride + (int64_t)src_w * C + c];
      v = normalize((float)x, a.mul[c], a.mul_lo[c], a.nsub[c], a.nsub_lo[c]);
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

// The operation's traffic without its arithmetic, in the shape that moved
// each mix fastest on the hardware, so that its rate is the practical roof
// for the fused kernels.  Every store is a 16-byte streaming store and every
// store instruction is lane-contiguous (lane-strided stores run several
// times slower).
//   K = 2 (the fp16 operation's 1:2 read:write mix): lane i reads input bytes
//     8i .. 8i+7 and writes them zero-extended to 16 bits as output vector i:
//     the output is the input widened in order.
//   K = 4 (the fp32 operation's 1:4 mix): lane i reads input vector i (16
//     bytes) and writes its dword k (4 bytes, each zero-extended to 32 bits)
//     as output vector 4 b + k m + (i - b), where the lane's block of m lanes
//     starts at lane b.
// `lanes` = input bytes / 8 (K = 2) or / 16 (K = 4).
template <int K>
__global__ void __launch_bounds__(kBlock) stream_kernel(const uint8_t* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t lanes) {
  const int64_t b0 = (int64_t)blockIdx.x * kBlock;
  const int64_t i = b0 + threadIdx.x;
  if (i >= lanes) return;
  if constexpr (K == 2) {
    const uint2 w = reinterpret_cast<const uint2*>(src)[i];
    // v_perm_b32 byte selectors: 0..3 pick bytes of the second operand, 12 gives 0
    const u32x4 q{__builtin_amdgcn_perm(0u, w.x, 0x0C010C00u), __builtin_amdgcn_perm(0u, w.x, 0x0C030C02u),
                  __builtin_amdgcn_perm(0u, w.y, 0x0C010C00u), __builtin_amdgcn_perm(0u, w.y, 0x0C030C02u)};
    stream_store16(dst + i, q);
  } else {
    const int64_t m = min((int64_t)kBlock, lanes - b0);  // lanes of this block
    const u32x4 w = reinterpret_cast<const u32x4*>(src)[i];
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 q{d[k] & 0xFFu, (d[k] >> 8) & 0xFFu, (d[k] >> 16) & 0xFFu, d[k] >> 24};
      stream_store16(dst + 4 * b0 + k * m + threadIdx.x, q);
    }
  }
}

}  // namespace fn
