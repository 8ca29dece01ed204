// Prompt GEMM Y[M,N] = X[M,K] W[N,K]^T with R4 weights rebuilt on the fly
// and multiplied on gfx950 bf16 MFMA, and its bf16-weight twin.
//
// "Binade" package page (pypi.org/project/binade), "Results": prompt
// processing runs the 12B model's matmuls with a fused GEMM; "Limitations":
// on long prompts the fused GEMM is weighed against rebuilding BF16 weights;
// "NVIDIA GPUs": a GEMM's order is a chain of matrix-core steps along K, with
// split-K partitions that follow a fixed rule.
//
// Order (every kernel here, independent of M, tiling and launch shape): K is
// cut into S = min(8, ceil(K / 1024)) slices of whole 32-column blocks (slice
// s holds blocks [s*nb/S, (s+1)*nb/S) of the nb = K/32 blocks). In a slice,
// an output's fp32 accumulator starts at +0.0 and takes the slice's blocks in
// increasing order, one v_mfma_f32_16x16x32_bf16 step per block (lane group
// g of the step carries columns 8g..8g+7 of the block). The output is
// (((p0 + p1) + p2) + ...) + p(S-1) over the slices' accumulators. The R4 kernels
// rebuild exactly the bf16 weights the twins read, so both issue identical
// MFMA sequences and their outputs agree bit for bit.
//
// Small M (<= 128): one wave per 16 weight rows, 1-8 tiles of 16 X rows; the
// weights are rebuilt straight into MFMA operands in registers, the next
// blocks are loaded while the current ones multiply, and the S slices of a
// tile are S waves of one block, added in slice order through LDS. Blocks
// that share weight rows are placed on the same XCD (blocks are dealt to the
// 8 XCDs round robin), so their weight reads meet in that XCD's L2.
// Large M: 128x128 tiles, 4 waves of 64x64 (4x4 MFMA tiles); per block the
// X and rebuilt W tiles go through double-buffered LDS; slices run in order
// with a running total.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint8_t* w;          // R4 sm plane or bf16 weights (twin)
  const uint8_t* nib;
  const uint32_t* esc_pre;
  const uint32_t* esc;
  const uint16_t* x;
  void* y;
  int64_t m, n, ldx, ldy;
  int32_t k;
  int32_t y_bf16;
  uint32_t n_esc;
  uint32_t lut0, lut1, lut2, lut3;   // rotated exponents of ranks 0..15
  int32_t slices;                    // S
  int32_t mtiles;                    // small kernel: tiles of 16*MT X rows
  int64_t tiles;                     // small kernel: weight-row tiles * mtiles
};

constexpr int kXcds = 8;

// Block range [lo, hi) of slice s.
__device__ __forceinline__ void slice_blocks(int32_t k, int32_t S, int32_t s, int32_t& lo,
                                             int32_t& hi) {
  const int32_t nb = k >> 5;
  lo = (s * nb) / S;
  hi = ((s + 1) * nb) / S;
}

__device__ __forceinline__ bool has_escape(uint32_t P) {
  return (P & (P >> 1) & (P >> 2) & (P >> 3) & 0x11111111u) != 0u;
}

// Rare: put the side-list exponents of row n, columns c0 .. c0+7 into the
// rotated exponent words E[0] (columns c0..c0+3) and E[1] (c0+4..c0+7).
__device__ __forceinline__ void patch8(const GemmArgs& a, int64_t n, int32_t c0,
                                                 uint32_t& E0, uint32_t& E1) {
  const int32_t C = (a.k + kChunk - 1) / kChunk;
  const int32_t j = c0 / kChunk;
  const int64_t chunk = n * C + j;
  uint32_t hi = a.esc_pre[chunk + 1];
  uint32_t lo = a.esc_pre[chunk];
  hi = hi < a.n_esc ? hi : a.n_esc;
  lo = lo < hi ? lo : hi;
  const uint32_t pos0 = static_cast<uint32_t>(c0 - j * kChunk);
  while (lo < hi) {   // first entry at or after pos0 (a chunk's entries are sorted)
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if ((a.esc[mid] & 0xFFFFu) < pos0)
      lo = mid + 1;
    else
      hi = mid;
  }
  const uint32_t end = a.esc_pre[chunk + 1] < a.n_esc ? a.esc_pre[chunk + 1] : a.n_esc;
  for (uint32_t e = lo; e < end; ++e) {
    const uint32_t ent = a.esc[e];
    const uint32_t d = (ent & 0xFFFFu) - pos0;
    if (d >= 8u) break;
    const uint32_t sh = (d & 3u) * 8u;
    const uint32_t ex = rot_exponent((ent >> 16) & 0xFFu) << sh;
    if (d < 4u)
      E0 = (E0 & ~(0xFFu << sh)) | ex;
    else
      E1 = (E1 & ~(0xFFu << sh)) | ex;
  }
}

// 8 bf16 weights (columns c0 .. c0+7 of row n) from their sm bytes and
// nibble word, as 4 dwords of bf16 pairs.
__device__ __forceinline__ uint4 rebuild8(const GemmArgs& a, const Lut& L, uint2 sm, uint32_t P,
                                          int64_t n, int32_t c0) {
  uint32_t E0 = lookup4(P, L);
  uint32_t E1 = lookup4(P >> 4, L);
  if (has_escape(P)) patch8(a, n, c0, E0, E1);
  uint32_t H0, L0, H1, L1;
  split4_rot(sm.x, E0, H0, L0);
  split4_rot(sm.y, E1, H1, L1);
  return make_uint4(weight_pair_bf16<0>(H0, L0), weight_pair_bf16<2>(H0, L0),
                    weight_pair_bf16<0>(H1, L1), weight_pair_bf16<2>(H1, L1));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void store_out(const GemmArgs& a, int64_t m, int64_t n, float v) {
  if (m < a.m && n < a.n) {
    if (a.y_bf16)
      static_cast<uint16_t*>(a.y)[m * a.ldy + n] = to_bf16_rne(v);
    else
      static_cast<float*>(a.y)[m * a.ldy + n] = v;
  }
}

// ---------------------------------------------------------------- small M
// Raw loads of one 32-column block for one lane: the weight row's 8 columns
// (R4: sm + nibbles; twin: bf16) and MT X rows' 8 columns.
template <bool kR4, int MT>
struct SmallRaw {
  uint2 sm;
  uint32_t nib;
  uint4 w;
  uint4 x[MT];
};

// Rows past N (or M) are read from the last row instead: an MFMA output
// depends only on its own A row and B column, and those outputs are never
// stored, so every load is unconditional.
template <bool kR4, int MT>
__device__ __forceinline__ void small_load(const GemmArgs& a, const uint8_t* wrow,
                                           const uint8_t* nrow, const uint16_t* const (&xrow)[MT],
                                           int32_t c, SmallRaw<kR4, MT>& r) {
  if (kR4) {
    r.sm = *reinterpret_cast<const uint2*>(wrow + c);
    r.nib = *reinterpret_cast<const uint32_t*>(nrow + (c >> 1));
  } else {
    r.w = *reinterpret_cast<const uint4*>(wrow + 2 * c);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) r.x[t] = *reinterpret_cast<const uint4*>(xrow[t] + c);
}

// Block (x = tile of 16 weight rows and 16*MT X rows, as dealt to XCDs),
// one wave per slice. kDepth blocks are in flight per wave.
template <bool kR4, int MT>
__global__ __launch_bounds__(512) void gemm_small_kernel(GemmArgs a) {
  constexpr int kDepth = MT == 1 ? 8 : (MT == 2 ? 4 : 2);
  constexpr int kMaxSlices = 8;
  __shared__ floatx4 part[kMaxSlices][64];
  const int lane = threadIdx.x & 63;
  const int s = uniform(static_cast<int>(threadIdx.x >> 6));   // slice
  // XCD-aware tile: the blocks on one XCD take consecutive tiles, so the X
  // tiles of one weight-row tile share that XCD's L2
  const int64_t per = (a.tiles + kXcds - 1) / kXcds;
  const int64_t tile = static_cast<int64_t>(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= a.tiles) return;
  const int64_t nt = tile / a.mtiles;
  const int64_t mt = tile - nt * a.mtiles;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n = min(nt * 16 + r, a.n - 1);
  const uint8_t* wrow = kR4 ? a.w + n * a.k : a.w + 2 * n * a.k;
  const uint8_t* nrow = a.nib + n * (a.k >> 1);
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = a.x + min((mt * MT + t) * 16 + r, a.m - 1) * a.ldx;
  const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};
  int32_t b0, b1;
  slice_blocks(a.k, a.slices, s, b0, b1);

  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  SmallRaw<kR4, MT> q[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (b0 + d < b1) small_load<kR4, MT>(a, wrow, nrow, xrow, (b0 + d) * 32 + 8 * g, q[d]);
  int32_t b = b0;
  // steady state: every refill is in range, no branches inside
  for (; b + 2 * kDepth <= b1; b += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int32_t c = (b + d) * 32 + 8 * g;
      bf16x8 B;
      if (kR4)
        B = as_bf16x8(rebuild8(a, L, q[d].sm, q[d].nib, n, c));
      else
        B = as_bf16x8(q[d].w);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(q[d].x[t]), B, acc[t], 0, 0, 0);
      small_load<kR4, MT>(a, wrow, nrow, xrow, c + 32 * kDepth, q[d]);
    }
  }
  // the last < 2 * kDepth blocks
#pragma unroll
  for (int d = 0; d < 2 * kDepth; ++d) {
    if (b + d >= b1) break;
    const int dd = d % kDepth;
    const int32_t c = (b + d) * 32 + 8 * g;
    bf16x8 B;
    if (kR4)
      B = as_bf16x8(rebuild8(a, L, q[dd].sm, q[dd].nib, n, c));
    else
      B = as_bf16x8(q[dd].w);
#pragma unroll
    for (int t = 0; t < MT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(q[dd].x[t]), B, acc[t], 0, 0, 0);
    if (d < kDepth && b + d + kDepth < b1)
      small_load<kR4, MT>(a, wrow, nrow, xrow, c + 32 * kDepth, q[dd]);
  }

  // slices in order: ((p0 + p1) + p2) + ..., one X tile at a time
  if (a.slices > 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t > 0) __syncthreads();   // wave 0 has read the previous tile
      if (s > 0) part[s][lane] = acc[t];
      __syncthreads();
      if (s == 0)
        for (int j = 1; j < a.slices; ++j) acc[t] += part[j][lane];
    }
    if (s != 0) return;
  }
  // D layout: lane holds column r, rows 4g .. 4g+3 of each 16x16 tile
  const int64_t on = nt * 16 + r;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) store_out(a, (mt * MT + t) * 16 + 4 * g + i, on, acc[t][i]);
}

// ---------------------------------------------------------------- large M
constexpr int kBM = 128, kBN = 128;
constexpr int kLdsStride = 32 + 8;   // bf16 elements per LDS row (80 bytes)

// One thread's share of a 32-column block: 16 columns of one X row and of
// one weight row (raw).
template <bool kR4>
struct LargeRaw {
  uint4 x0, x1;
  uint4 sm;          // R4: 16 sm bytes
  uint2 nib;         // R4: 16 nibbles
  uint4 w0, w1;      // twin: 16 bf16
};

template <bool kR4>
__device__ __forceinline__ void large_load(const GemmArgs& a, int32_t blk, int sc, int64_t xm,
                                           bool xm_ok, int64_t wnr, bool wn_ok,
                                           LargeRaw<kR4>& q) {
  const int32_t c = blk * 32 + sc;
  if (xm_ok) {
    const uint4* px = reinterpret_cast<const uint4*>(a.x + xm * a.ldx + c);
    q.x0 = px[0];
    q.x1 = px[1];
  } else {
    q.x0 = q.x1 = make_uint4(0, 0, 0, 0);
  }
  if (kR4) {
    q.sm = wn_ok ? *reinterpret_cast<const uint4*>(a.w + wnr * a.k + c) : make_uint4(0, 0, 0, 0);
    q.nib = wn_ok ? *reinterpret_cast<const uint2*>(a.nib + wnr * (a.k >> 1) + (c >> 1))
                  : make_uint2(0, 0);
  } else if (wn_ok) {
    const uint4* pw =
        reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.w) + wnr * a.k + c);
    q.w0 = pw[0];
    q.w1 = pw[1];
  } else {
    q.w0 = q.w1 = make_uint4(0, 0, 0, 0);
  }
}

template <bool kR4>
__device__ __forceinline__ void large_stage(const GemmArgs& a, const Lut& L,
                                            uint16_t (*xs)[kLdsStride],
                                            uint16_t (*ws)[kLdsStride], int sr, int sc,
                                            int32_t blk, int64_t wnr, const LargeRaw<kR4>& q) {
  *reinterpret_cast<uint4*>(&xs[sr][sc]) = q.x0;
  *reinterpret_cast<uint4*>(&xs[sr][sc + 8]) = q.x1;
  uint4 w0, w1;
  if (kR4) {
    const int32_t c = blk * 32 + sc;
    w0 = rebuild8(a, L, make_uint2(q.sm.x, q.sm.y), q.nib.x, wnr, c);
    w1 = rebuild8(a, L, make_uint2(q.sm.z, q.sm.w), q.nib.y, wnr, c + 8);
  } else {
    w0 = q.w0;
    w1 = q.w1;
  }
  *reinterpret_cast<uint4*>(&ws[sr][sc]) = w0;
  *reinterpret_cast<uint4*>(&ws[sr][sc + 8]) = w1;
}

template <bool kR4>
__global__ __launch_bounds__(256, 2) void gemm_large_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kBM][kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kBN][kLdsStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // XCD-aware tile order: consecutive tiles (same weight columns) per XCD
  const int64_t tiles_n = (a.n + kBN - 1) / kBN, tiles_m = (a.m + kBM - 1) / kBM;
  const int64_t tiles = tiles_n * tiles_m;
  const int64_t per = (tiles + kXcds - 1) / kXcds;
  const int64_t tile = static_cast<int64_t>(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= tiles) return;
  const int64_t n0 = (tile / tiles_m) * kBN;
  const int64_t m0 = (tile % tiles_m) * kBM;
  const int wm = (wave >> 1) * 64;
  const int wn = (wave & 1) * 64;
  const int sr = tid >> 1;           // staging row 0..127
  const int sc = (tid & 1) * 16;     // staging column 0 or 16
  const int64_t xm = m0 + sr, wnr = n0 + sr;
  const bool xm_ok = xm < a.m, wn_ok = wnr < a.n;
  const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};
  const int r = lane & 15, g = lane >> 4;

  floatx4 acc[4][4], tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[i][j] = acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t nb = a.k >> 5;
  LargeRaw<kR4> q;
  large_load<kR4>(a, 0, sc, xm, xm_ok, wnr, wn_ok, q);
  large_stage<kR4>(a, L, xs[0], ws[0], sr, sc, 0, wnr, q);
  __syncthreads();
  int32_t s = 0, s_hi;
  {
    int32_t lo;
    slice_blocks(a.k, a.slices, 0, lo, s_hi);
  }
  for (int32_t blk = 0; blk < nb; ++blk) {
    const int buf = blk & 1;
    if (blk + 1 < nb) large_load<kR4>(a, blk + 1, sc, xm, xm_ok, wnr, wn_ok, q);
    bf16x8 A[4], Bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      A[i] = *reinterpret_cast<const bf16x8*>(&xs[buf][wm + 16 * i + r][8 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      Bv[j] = *reinterpret_cast<const bf16x8*>(&ws[buf][wn + 16 * j + r][8 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], Bv[j], acc[i][j], 0, 0, 0);
    if (blk + 1 == s_hi) {
      // end of slice s: add its accumulators to the total in slice order
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tot[i][j] = s == 0 ? acc[i][j] : tot[i][j] + acc[i][j];
          acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      ++s;
      if (s < a.slices) {
        int32_t lo;
        slice_blocks(a.k, a.slices, s, lo, s_hi);
      }
    }
    if (blk + 1 < nb) large_stage<kR4>(a, L, xs[buf ^ 1], ws[buf ^ 1], sr, sc, blk + 1, wnr, q);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t on = n0 + wn + 16 * j + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(a, m0 + wm + 16 * i + 4 * g + e, on, tot[i][j][e]);
    }
}

int32_t check_xy(const uint16_t* x, int64_t m, int64_t ldx, void* y,
                 int64_t ldy, int64_t n, int64_t k, int32_t y_dtype) {
  if (m < 0 || n < 0 || k <= 0) return BINADE_EINVAL;
  if (k % 32 != 0 || k > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (m == 0 || n == 0) return BINADE_OK;
  if (x == nullptr || y == nullptr) return BINADE_EINVAL;
  if (ldx < k || ldy < n) return BINADE_EINVAL;
  if (!aligned16(x) || ldx % 8 != 0) return BINADE_EUNSUPPORTED;
  if (m > (1ll << 31) || n > (1ll << 31)) return BINADE_EUNSUPPORTED;
  return BINADE_OK;
}

int32_t slices_for(int64_t k) {
  const int64_t s = (k + 1023) / 1024;
  const int64_t nb = k / 32;
  int64_t S = s < 8 ? s : 8;
  if (S > nb) S = nb;
  return static_cast<int32_t>(S < 1 ? 1 : S);
}

constexpr int64_t kSmallMaxM = 128;

template <bool kR4, int MT>
int32_t launch_small(GemmArgs a, hipStream_t stream) {
  a.mtiles = static_cast<int32_t>((a.m + 16 * MT - 1) / (16 * MT));
  a.tiles = ((a.n + 15) / 16) * a.mtiles;
  const int64_t per = (a.tiles + kXcds - 1) / kXcds;
  const int64_t blocks = per * kXcds;
  if (blocks > 0x7FFFFFFFll) return BINADE_EUNSUPPORTED;
  hipLaunchKernelGGL((gemm_small_kernel<kR4, MT>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * a.slices), 0, stream, a);
  return launch_status();
}

int32_t launch(GemmArgs a, bool r4, hipStream_t stream) {
  a.slices = slices_for(a.k);
  if (a.m <= kSmallMaxM) {
    if (r4) {
      if (a.m <= 16) return launch_small<true, 1>(a, stream);
      if (a.m <= 32) return launch_small<true, 2>(a, stream);
      if (a.m <= 64) return launch_small<true, 4>(a, stream);
      return launch_small<true, 8>(a, stream);
    }
    if (a.m <= 16) return launch_small<false, 1>(a, stream);
    if (a.m <= 32) return launch_small<false, 2>(a, stream);
    if (a.m <= 64) return launch_small<false, 4>(a, stream);
    return launch_small<false, 8>(a, stream);
  }
  const int64_t tiles = ((a.n + kBN - 1) / kBN) * ((a.m + kBM - 1) / kBM);
  const int64_t blocks = ((tiles + kXcds - 1) / kXcds) * kXcds;
  if (blocks > 0x7FFFFFFFll) return BINADE_EUNSUPPORTED;
  if (r4)
    hipLaunchKernelGGL(gemm_large_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(gemm_large_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, a);
  return launch_status();
}

uint32_t pack4(const uint8_t* l) {
  return uint32_t(l[0]) | (uint32_t(l[1]) << 8) | (uint32_t(l[2]) << 16) |
         (uint32_t(l[3]) << 24);
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int32_t binade_r4_gemm(const binade_r4* w, const uint16_t* x,
                                  int64_t m, int64_t ldx, void* y, int64_t ldy,
                                  int32_t y_dtype, void* stream) {
  if (w == nullptr || w->rows < 0 || w->cols <= 0) return BINADE_EINVAL;
  int32_t s = check_xy(x, m, ldx, y, ldy, w->rows, w->cols, y_dtype);
  if (s != BINADE_OK || m == 0 || w->rows == 0) return s;
  if (w->sm == nullptr || w->nib == nullptr || w->esc_pre == nullptr ||
      (w->n_esc > 0 && w->esc == nullptr))
    return BINADE_EINVAL;
  if (!aligned16(w->sm) || !aligned16(w->nib)) return BINADE_EUNSUPPORTED;
  if (w->n_esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  GemmArgs a{};
  a.w = w->sm;
  a.nib = w->nib;
  a.esc_pre = w->esc_pre;
  a.esc = w->esc;
  a.n_esc = static_cast<uint32_t>(w->n_esc);
  a.lut0 = rot_exponents4(pack4(w->lut));
  a.lut1 = rot_exponents4(pack4(w->lut + 4));
  a.lut2 = rot_exponents4(pack4(w->lut + 8));
  a.lut3 = rot_exponents4(pack4(w->lut + 12));
  a.x = x;
  a.y = y;
  a.m = m;
  a.n = w->rows;
  a.k = static_cast<int32_t>(w->cols);
  a.ldx = ldx;
  a.ldy = ldy;
  a.y_bf16 = y_dtype == BINADE_BF16;
  return launch(a, true, static_cast<hipStream_t>(stream));
}

extern "C" int32_t binade_bf16_gemm(const uint16_t* w, int64_t rows,
                                    int64_t cols, const uint16_t* x, int64_t m,
                                    int64_t ldx, void* y, int64_t ldy,
                                    int32_t y_dtype, void* stream) {
  if (rows < 0 || cols <= 0) return BINADE_EINVAL;
  int32_t s = check_xy(x, m, ldx, y, ldy, rows, cols, y_dtype);
  if (s != BINADE_OK || m == 0 || rows == 0) return s;
  if (w == nullptr) return BINADE_EINVAL;
  if (!aligned16(w)) return BINADE_EUNSUPPORTED;
  GemmArgs a{};
  a.w = reinterpret_cast<const uint8_t*>(w);
  a.x = x;
  a.y = y;
  a.m = m;
  a.n = rows;
  a.k = static_cast<int32_t>(cols);
  a.ldx = ldx;
  a.ldy = ldy;
  a.y_bf16 = y_dtype == BINADE_BF16;
  return launch(a, false, static_cast<hipStream_t>(stream));
}
