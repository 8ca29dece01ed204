// Batch-1 matrix-vector product on R4 weights, its bf16-weight twin, and the
// R4 -> bf16 unpack.
//
// "Binade" package page (pypi.org/project/binade), "Results": the batch-1
// matvec on R4 moves its bytes as efficiently as the BF16 one does, so a
// token is faster by the ratio of bytes; "How it works": R4 holds each rank as a 4-bit
// code, the few large ranks going to a side list, and the matvec adds its
// products in one fixed order so its outputs equal the BF16 computation's
// bit for bit.
//
// Order (shared with the twin, independent of the launch shape): K is cut
// into lane tiles of 32 columns; tile j belongs to slot j mod 64; slot l's
// two fp32 sums (even / odd columns) start at +0.0 and take its tiles in
// increasing j with one fma per column; then slot values a0 + a1 are reduced
// by p[l] += p[l+s] for s = 32..1. One wave of 64 lanes is exactly one slot
// per lane, so a wave pass over 2048 columns is one row-chunk.
//
// Mapping on gfx950: a wave owns R rows and walks their chunks; lane l reads
// its tile's 32 sign/mantissa bytes (two 16-byte loads) and 16 nibble bytes
// (one 16-byte load) per row, rebuilds the 32 fp32 weights in registers with
// v_perm_b32 lookups into the 16-byte table, and shares one x tile (four
// 16-byte loads, converted once) across the R rows. Escapes are patched from
// the chunk's side list by a uniform scalar loop before the weights are
// assembled. The slot tree is five xor shuffles after the last chunk.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

struct GemvArgs {
  const uint8_t* sm;       // R4 sign/mantissa plane (or bf16 weights, twin)
  const uint8_t* nib;
  const uint32_t* esc_pre;
  const uint32_t* esc;
  const uint16_t* x;
  void* y;
  int64_t rows;
  int32_t cols;
  int32_t y_bf16;
  uint32_t n_esc;
  uint32_t lut0, lut1, lut2, lut3;
};

__device__ __forceinline__ void store_y(const GemvArgs& a, int64_t row,
                                        float v) {
  if (a.y_bf16)
    static_cast<uint16_t*>(a.y)[row] = to_bf16_rne(v);
  else
    static_cast<float*>(a.y)[row] = v;
}

// Raw loads of one lane tile of R rows plus its x tile.
template <int R>
struct TileLoads {
  uint4 s0[R], s1[R], nb[R];
  uint4 xq[4];
};

template <int R>
__device__ __forceinline__ void load_tiles(TileLoads<R>& b, const GemvArgs& a,
                                           const int64_t (&row)[R], int t) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint4* ps = reinterpret_cast<const uint4*>(a.sm + row[r] * a.cols + 32 * t);
    b.s0[r] = ps[0];
    b.s1[r] = ps[1];
    b.nb[r] = *reinterpret_cast<const uint4*>(a.nib + row[r] * (a.cols >> 1) + 16 * t);
  }
  const uint4* px = reinterpret_cast<const uint4*>(a.x + 32 * t);
#pragma unroll
  for (int v = 0; v < 4; ++v) b.xq[v] = px[v];
}

// Rebuild and multiply one lane tile of R rows (tile t of row-chunk j).
template <int R>
__device__ __forceinline__ void fma_tiles(const TileLoads<R>& b, const GemvArgs& a,
                                          const Lut& Lr, const int64_t (&row)[R],
                                          int C, int j, int lane, float (&acc0)[R],
                                          float (&acc1)[R]) {
  float xf[32];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t w[4] = {b.xq[v].x, b.xq[v].y, b.xq[v].z, b.xq[v].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xf[8 * v + 2 * e] = bf16_lo(w[e]);
      xf[8 * v + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint32_t E[8];
    tile_exponents<true>(b.nb[r], Lr, a.esc_pre, a.esc, a.n_esc, row[r] * C + j, lane, E);
    const uint32_t S[8] = {b.s0[r].x, b.s0[r].y, b.s0[r].z, b.s0[r].w,
                           b.s1[r].x, b.s1[r].y, b.s1[r].z, b.s1[r].w};
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t H, Lo;
      split4_rot(S[d], E[d], H, Lo);
      fma_group(H, Lo, xf + 4 * d, acc0[r], acc1[r]);
    }
  }
}

// One wave owns rows row0 .. row0+R-1 (rows past the end are computed on a
// clamped row index and not stored). Full row-chunks run with every lane
// active and the next chunk's loads in flight; a ragged last chunk (K not a
// multiple of 2048) runs on its first K/32 mod 64 lanes.
template <int R, bool kPrefetch>
__device__ __forceinline__ void r4_gemv_rows(const GemvArgs& a, int64_t row0, int lane) {
  const int J = a.cols >> 5;
  const int Cf = J >> 6;          // full chunks
  const int tail = J & 63;        // lanes in the ragged chunk
  const int C = Cf + (tail ? 1 : 0);
  const Lut Lr{a.lut0, a.lut1, a.lut2, a.lut3};   // rotated table
  int64_t row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) row[r] = row0 + r < a.rows ? row0 + r : a.rows - 1;

  float acc0[R], acc1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc0[r] = acc1[r] = 0.0f;

  if (kPrefetch) {
    if (Cf > 0) {
      TileLoads<R> A, B;
      load_tiles(A, a, row, lane);
      int j = 0;
      for (; j + 2 <= Cf; j += 2) {
        load_tiles(B, a, row, (j + 1) * 64 + lane);
        fma_tiles(A, a, Lr, row, C, j, lane, acc0, acc1);
        if (j + 2 < Cf) load_tiles(A, a, row, (j + 2) * 64 + lane);
        fma_tiles(B, a, Lr, row, C, j + 1, lane, acc0, acc1);
      }
      if (j < Cf) fma_tiles(A, a, Lr, row, C, j, lane, acc0, acc1);
    }
  } else {
    for (int j = 0; j < Cf; ++j) {
      TileLoads<R> A;
      load_tiles(A, a, row, j * 64 + lane);
      fma_tiles(A, a, Lr, row, C, j, lane, acc0, acc1);
    }
  }
  if (tail && lane < tail) {
    TileLoads<R> A;
    load_tiles(A, a, row, Cf * 64 + lane);
    fma_tiles(A, a, Lr, row, C, Cf, lane, acc0, acc1);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float p = slot_tree(acc0[r] + acc1[r]);
    if (lane == 0 && row0 + r < a.rows) store_y(a, row0 + r, p);
  }
}

// One wave owns rows row0 .. row0+R-1 (rows past the end are computed on a
// clamped row index and not stored). Full row-chunks run with every lane
// active; a ragged last chunk (K not a multiple of 2048) runs on its first
// K/32 mod 64 lanes.
template <int R, bool kPrefetch>
__global__ __launch_bounds__(256) void r4_gemv_kernel(GemvArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 =
      uniform64((static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) +
                 (threadIdx.x >> 6)) * R);
  if (row0 >= a.rows) return;
  r4_gemv_rows<R, kPrefetch>(a, row0, lane);
}

template <int R>
__device__ __forceinline__ void bf16_gemv_rows(const GemvArgs& a, int64_t row0, int lane);

// Several independent products in one launch: items 0..count-1 own the
// consecutive block ranges [first_block[i], first_block[i+1]).
constexpr int kMaxBatch = 16;
struct GemvBatch {
  GemvArgs item[kMaxBatch];
  uint32_t first_block[kMaxBatch + 1];
  int32_t count;
};

template <int R, bool kR4>
__global__ __launch_bounds__(256) void gemv_batch_kernel(GemvBatch b) {
  const int lane = threadIdx.x & 63;
  const uint32_t blk = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int t = 1; t < kMaxBatch; ++t)
    if (t < b.count && blk >= b.first_block[t]) i = t;
  // the item is read through the argument segment's address (an index into
  // a by-value argument array would be copied to scratch memory)
  const GemvArgs* items = (const GemvArgs*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() +
                                            offsetof(GemvBatch, item));
  const GemvArgs a = items[uniform(i)];
  const int64_t row0 = uniform64((static_cast<int64_t>(blk - b.first_block[i]) * (blockDim.x >> 6) +
                                  (threadIdx.x >> 6)) * R);
  if (row0 >= a.rows) return;
  if (kR4)
    r4_gemv_rows<R, false>(a, row0, lane);
  else
    bf16_gemv_rows<R>(a, row0, lane);
}

template <int R>
__device__ __forceinline__ void bf16_gemv_rows(const GemvArgs& a, int64_t row0, int lane) {
  const int J = a.cols >> 5;
  const int C = (J + 63) >> 6;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.sm);

  float acc0[R], acc1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc0[r] = acc1[r] = 0.0f;

  for (int j = 0; j < C; ++j) {
    const int t = j * 64 + lane;
    if (t >= J) continue;  // only in the last chunk
    uint4 wv[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r;
      const uint4* p = reinterpret_cast<const uint4*>(W + row * a.cols + 32 * t);
      if (row < a.rows) {
#pragma unroll
        for (int v = 0; v < 4; ++v) wv[r][v] = p[v];
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) wv[r][v] = make_uint4(0, 0, 0, 0);
      }
    }
    float xf[32];
    load_x_tile(a.x, t, xf);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t w[4] = {wv[r][v].x, wv[r][v].y, wv[r][v].z, wv[r][v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc0[r] = __builtin_fmaf(bf16_lo(w[e]), xf[8 * v + 2 * e], acc0[r]);
          acc1[r] = __builtin_fmaf(bf16_hi(w[e]), xf[8 * v + 2 * e + 1], acc1[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    const float p = slot_tree(acc0[r] + acc1[r]);
    if (lane == 0 && row < a.rows) store_y(a, row, p);
  }
}

template <int R>
__global__ __launch_bounds__(256) void bf16_gemv_kernel(GemvArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 =
      uniform64((static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) +
                 (threadIdx.x >> 6)) * R);
  if (row0 >= a.rows) return;
  bf16_gemv_rows<R>(a, row0, lane);
}

// ---------------------------------------------------------------- 2..8 rows
// The decode step of a few sequences at once: Y[b, :] = W x_b for b < m
// (m <= 8), each output in exactly the batch-1 order above, so row b of Y is
// bit-identical to the batch-1 product of x_b. Per lane tile a wave loads and
// rebuilds its weights once and runs them through the MB rows' two fma
// chains (x rows past m repeat row m-1 and are not stored). Rows of x and y
// are ldx and ldy elements apart.
struct GemvRowsArgs {
  GemvArgs g;              // weights, table, rows, cols, y_bf16 (g.x, g.y: row 0)
  int64_t ldx, ldy;
  int32_t m;
};

// The x rows are staged in LDS: a block of kRowsWaves waves (R weight rows
// each) copies each row-chunk's 2048 columns of the MB x rows into LDS once,
// and every wave reads its lanes' 32 columns from there, so the vector
// memory path carries the weights and one copy of x per block instead of one
// per wave (8 rows at 15360 x 3840: 73 -> 50 us).
constexpr int kRowsWaves = 8;

template <int MB, bool kR4, int R>
__global__ __launch_bounds__(64 * kRowsWaves) void gemv_rows_lds_kernel(GemvRowsArgs ra) {
  __shared__ __align__(16) uint32_t xs[MB][kChunk / 2];   // bf16 pairs
  const GemvArgs& a = ra.g;
  const int lane = threadIdx.x & 63;
  // R weight rows per wave: each converted x value feeds R rows' chains
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kRowsWaves +
                        uniform(static_cast<uint32_t>(threadIdx.x >> 6))) * R;
  int64_t rr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) rr[i] = row0 + i < a.rows ? row0 + i : a.rows - 1;
  const int J = a.cols >> 5;
  const int C = (J + 63) >> 6;
  const Lut Lr{a.lut0, a.lut1, a.lut2, a.lut3};
  float acc0[R][MB], acc1[R][MB];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc0[i][b] = acc1[i][b] = 0.0f;

  for (int j = 0; j < C; ++j) {
    const int t = j * 64 + lane;
    const bool active = t < J;
    // this wave's weight loads first
    uint4 s0[R], s1[R], nb[R], q[R][4];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      s0[i] = s1[i] = nb[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) q[i][v] = s0[i];
      if (active) {
        if (kR4) {
          const uint4* ps = reinterpret_cast<const uint4*>(a.sm + rr[i] * a.cols + 32 * t);
          s0[i] = ps[0];
          s1[i] = ps[1];
          nb[i] = *reinterpret_cast<const uint4*>(a.nib + rr[i] * (a.cols >> 1) + 16 * t);
        } else {
          const uint4* pw = reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(a.sm) + rr[i] * a.cols + 32 * t);
#pragma unroll
          for (int v = 0; v < 4; ++v) q[i][v] = pw[v];
        }
      }
    }
    // the chunk's x columns of the MB rows (16 bytes per thread per pass)
    __syncthreads();   // the previous chunk's x is no longer read
    const int cols_here = min(kChunk, a.cols - j * kChunk);
    for (int i = threadIdx.x; i < MB * (kChunk / 8); i += 64 * kRowsWaves) {
      const int b = i / (kChunk / 8), piece = i % (kChunk / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (8 * piece < cols_here) {
        const int bb = b < ra.m ? b : ra.m - 1;
        v = *reinterpret_cast<const uint4*>(a.x + bb * ra.ldx + j * kChunk + 8 * piece);
      }
      reinterpret_cast<uint4*>(xs[b])[piece] = v;
    }
    __syncthreads();
    if (!active) continue;
    float w[R][32];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (kR4) {
        uint32_t E[8];
        tile_exponents<true>(nb[i], Lr, a.esc_pre, a.esc, a.n_esc, rr[i] * C + j, lane, E);
        const uint32_t S[8] = {s0[i].x, s0[i].y, s0[i].z, s0[i].w,
                               s1[i].x, s1[i].y, s1[i].z, s1[i].w};
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          uint32_t H, Lo;
          split4_rot(S[d], E[d], H, Lo);
          w[i][4 * d] = weight_f32<0>(H, Lo);
          w[i][4 * d + 1] = weight_f32<1>(H, Lo);
          w[i][4 * d + 2] = weight_f32<2>(H, Lo);
          w[i][4 * d + 3] = weight_f32<3>(H, Lo);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t d4[4] = {q[i][v].x, q[i][v].y, q[i][v].z, q[i][v].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[i][8 * v + 2 * e] = bf16_lo(d4[e]);
            w[i][8 * v + 2 * e + 1] = bf16_hi(d4[e]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const uint4* px = reinterpret_cast<const uint4*>(xs[b]) + 4 * lane;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 xq = px[v];
        const uint32_t d4[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_lo(d4[e]), x1 = bf16_hi(d4[e]);
#pragma unroll
          for (int i = 0; i < R; ++i) {
            acc0[i][b] = __builtin_fmaf(w[i][8 * v + 2 * e], x0, acc0[i][b]);
            acc1[i][b] = __builtin_fmaf(w[i][8 * v + 2 * e + 1], x1, acc1[i][b]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const float p = slot_tree(acc0[i][b] + acc1[i][b]);
      if (lane == 0 && row0 + i < a.rows && b < ra.m) {
        const int64_t o = b * ra.ldy + row0 + i;
        if (a.y_bf16)
          static_cast<uint16_t*>(a.y)[o] = to_bf16_rne(p);
        else
          static_cast<float*>(a.y)[o] = p;
      }
    }
}

int32_t launch_gemv_rows(const GemvRowsArgs& ra, bool r4, hipStream_t stream) {
  // two weight rows per wave halve the x conversions (8 rows of x); only
  // where the blocks still fill the chip (measured: 15360 rows 50 -> 42 us,
  // 3840 rows slower)
  const int R = (ra.m > 4 && ra.g.rows >= 8192) ? 2 : 1;
  const dim3 sgrid(static_cast<uint32_t>((ra.g.rows + kRowsWaves * R - 1) / (kRowsWaves * R)));
  const dim3 sblock(64 * kRowsWaves);
#define BINADE_ROWS_LAUNCH(MB)                                                              \
  if (R == 2) {                                                                             \
    if (r4) hipLaunchKernelGGL((gemv_rows_lds_kernel<MB, true, 2>), sgrid, sblock, 0, stream, ra);   \
    else hipLaunchKernelGGL((gemv_rows_lds_kernel<MB, false, 2>), sgrid, sblock, 0, stream, ra);     \
  } else {                                                                                  \
    if (r4) hipLaunchKernelGGL((gemv_rows_lds_kernel<MB, true, 1>), sgrid, sblock, 0, stream, ra);   \
    else hipLaunchKernelGGL((gemv_rows_lds_kernel<MB, false, 1>), sgrid, sblock, 0, stream, ra);     \
  }
  if (ra.m <= 2) {
    BINADE_ROWS_LAUNCH(2)
  } else if (ra.m <= 4) {
    BINADE_ROWS_LAUNCH(4)
  } else {
    BINADE_ROWS_LAUNCH(8)
  }
#undef BINADE_ROWS_LAUNCH
  return launch_status();
}

// One wave per row-chunk; lane l rebuilds its tile's 32 bf16 patterns.
__global__ __launch_bounds__(256) void r4_unpack_kernel(GemvArgs a,
                                                        uint16_t* out) {
  const int lane = threadIdx.x & 63;
  const int J = a.cols >> 5;
  const int C = (J + 63) >> 6;
  const int64_t c = uniform64(static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) +
                              (threadIdx.x >> 6));
  if (c >= a.rows * C) return;
  const int64_t row = c / C;
  const int j = static_cast<int>(c - row * C);
  const int t = j * 64 + lane;
  const bool active = t < J;
  const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};
  uint4 s0 = make_uint4(0, 0, 0, 0), s1 = s0, nb = s0;
  if (active) {
    const uint4* ps = reinterpret_cast<const uint4*>(a.sm + row * a.cols + 32 * t);
    s0 = ps[0];
    s1 = ps[1];
    nb = *reinterpret_cast<const uint4*>(a.nib + row * (a.cols >> 1) + 16 * t);
  }
  uint32_t E[8];
  tile_exponents(nb, L, a.esc_pre, a.esc, a.n_esc, c, lane, E);
  if (!active) return;
  const uint32_t S[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint32_t o[16];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t H, Lo;
    split4(S[d], E[d], H, Lo);
    o[2 * d] = weight_pair_bf16<0>(H, Lo);
    o[2 * d + 1] = weight_pair_bf16<2>(H, Lo);
  }
  uint4* po = reinterpret_cast<uint4*>(out + row * a.cols + 32 * t);
#pragma unroll
  for (int v = 0; v < 4; ++v)
    po[v] = make_uint4(o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]);
}

uint32_t pack_lut(const uint8_t* l, int q) {
  return uint32_t(l[4 * q]) | (uint32_t(l[4 * q + 1]) << 8) |
         (uint32_t(l[4 * q + 2]) << 16) | (uint32_t(l[4 * q + 3]) << 24);
}

int32_t check_r4(const binade_r4* w) {
  if (w == nullptr || w->rows < 0 || w->cols <= 0) return BINADE_EINVAL;
  if (w->cols % 32 != 0) return BINADE_EUNSUPPORTED;
  if (w->cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (w->rows == 0) return BINADE_OK;
  if (w->sm == nullptr || w->nib == nullptr || w->esc_pre == nullptr ||
      (w->n_esc > 0 && w->esc == nullptr))
    return BINADE_EINVAL;
  if (!aligned16(w->sm) || !aligned16(w->nib)) return BINADE_EUNSUPPORTED;
  if (w->n_esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  return BINADE_OK;
}

GemvArgs args_from_r4(const binade_r4* w, bool rotated) {
  GemvArgs a{};
  a.sm = w->sm;
  a.nib = w->nib;
  a.esc_pre = w->esc_pre;
  a.esc = w->esc;
  a.rows = w->rows;
  a.cols = static_cast<int32_t>(w->cols);
  a.n_esc = static_cast<uint32_t>(w->n_esc);
  a.lut0 = pack_lut(w->lut, 0);
  a.lut1 = pack_lut(w->lut, 1);
  a.lut2 = pack_lut(w->lut, 2);
  a.lut3 = pack_lut(w->lut, 3);
  if (rotated) {
    a.lut0 = dev::rot_exponents4(a.lut0);
    a.lut1 = dev::rot_exponents4(a.lut1);
    a.lut2 = dev::rot_exponents4(a.lut2);
    a.lut3 = dev::rot_exponents4(a.lut3);
  }
  return a;
}

// Launch shape: rows per wave R and whether a wave prefetches its next
// chunk. Neither changes the arithmetic. BINADE_GEMV_ROWS_PER_WAVE (1, 2, 4)
// and BINADE_GEMV_PREFETCH (0, 1), read once at the first launch, override
// the defaults.
struct GemvShape {
  int rows_per_wave;
  bool prefetch;
};

GemvShape read_gemv_shape() {
  GemvShape s{1, false};   // one row per wave measured fastest at every shape
  if (const char* env = getenv("BINADE_GEMV_ROWS_PER_WAVE")) {
    const int r = atoi(env);
    if (r == 1 || r == 2 || r == 4) s.rows_per_wave = r;
  }
  if (const char* env = getenv("BINADE_GEMV_PREFETCH")) s.prefetch = atoi(env) != 0;
  return s;
}

GemvShape gemv_shape(int64_t rows) {
  (void)rows;
  static const GemvShape shape = read_gemv_shape();
  return shape;
}

int32_t launch_gemv(const GemvArgs& a, bool r4, hipStream_t stream) {
  const GemvShape sh = gemv_shape(a.rows);
  const int R = sh.rows_per_wave;
  const int64_t waves = (a.rows + R - 1) / R;
  const dim3 grid(static_cast<uint32_t>((waves + 3) / 4));
  const dim3 block(256);
  if (r4) {
    if (sh.prefetch) {
      if (R == 4) hipLaunchKernelGGL((r4_gemv_kernel<4, true>), grid, block, 0, stream, a);
      else if (R == 2) hipLaunchKernelGGL((r4_gemv_kernel<2, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((r4_gemv_kernel<1, true>), grid, block, 0, stream, a);
    } else {
      if (R == 4) hipLaunchKernelGGL((r4_gemv_kernel<4, false>), grid, block, 0, stream, a);
      else if (R == 2) hipLaunchKernelGGL((r4_gemv_kernel<2, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((r4_gemv_kernel<1, false>), grid, block, 0, stream, a);
    }
  } else {
    if (R == 4) hipLaunchKernelGGL(bf16_gemv_kernel<4>, grid, block, 0, stream, a);
    else if (R == 2) hipLaunchKernelGGL(bf16_gemv_kernel<2>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(bf16_gemv_kernel<1>, grid, block, 0, stream, a);
  }
  return launch_status();
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int32_t binade_r4_gemv(const binade_r4* w, const uint16_t* x,
                                  void* y, int32_t y_dtype, void* stream) {
  int32_t s = check_r4(w);
  if (s != BINADE_OK) return s;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (w->rows == 0) return BINADE_OK;
  if (x == nullptr || y == nullptr) return BINADE_EINVAL;
  if (!aligned16(x)) return BINADE_EUNSUPPORTED;
  GemvArgs a = args_from_r4(w, true);
  a.x = x;
  a.y = y;
  a.y_bf16 = y_dtype == BINADE_BF16;
  return launch_gemv(a, true, static_cast<hipStream_t>(stream));
}

namespace binade {
namespace {

// Launches `items` in groups of kMaxBatch (one launch per group).
int32_t launch_gemv_batch(const GemvArgs* items, int32_t count, bool r4, hipStream_t stream) {
  const int R = gemv_shape(0).rows_per_wave == 1 ? 1 : 2;
  for (int32_t base = 0; base < count; base += kMaxBatch) {
    GemvBatch b{};
    uint64_t blocks = 0;
    int n = 0;
    for (int32_t i = base; i < count && n < kMaxBatch; ++i) {
      b.item[n] = items[i];
      b.first_block[n] = static_cast<uint32_t>(blocks);
      const int64_t waves = (items[i].rows + R - 1) / R;
      blocks += static_cast<uint64_t>((waves + 3) / 4);
      ++n;
    }
    if (blocks == 0) continue;
    if (blocks > 0x7FFFFFFFull) return BINADE_EUNSUPPORTED;
    b.first_block[n] = static_cast<uint32_t>(blocks);
    b.count = n;
    const dim3 grid(static_cast<uint32_t>(blocks));
    if (r4) {
      if (R == 2) hipLaunchKernelGGL((gemv_batch_kernel<2, true>), grid, dim3(256), 0, stream, b);
      else hipLaunchKernelGGL((gemv_batch_kernel<1, true>), grid, dim3(256), 0, stream, b);
    } else {
      if (R == 2) hipLaunchKernelGGL((gemv_batch_kernel<2, false>), grid, dim3(256), 0, stream, b);
      else hipLaunchKernelGGL((gemv_batch_kernel<1, false>), grid, dim3(256), 0, stream, b);
    }
    const int32_t s = launch_status();
    if (s != BINADE_OK) return s;
  }
  return BINADE_OK;
}

}  // namespace
}  // namespace binade

extern "C" int32_t binade_r4_gemv_batch(const binade_r4* ws,
                                        const uint16_t* const* xs,
                                        void* const* ys, int32_t count,
                                        int32_t y_dtype, void* stream) {
  if (count < 0 || (count > 0 && (ws == nullptr || xs == nullptr || ys == nullptr)))
    return BINADE_EINVAL;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  GemvArgs items[kMaxBatch];
  for (int32_t base = 0; base < count; base += kMaxBatch) {
    int n = 0;
    for (int32_t i = base; i < count && i < base + kMaxBatch; ++i) {
      const int32_t s = check_r4(&ws[i]);
      if (s != BINADE_OK) return s;
      if (ws[i].rows == 0) continue;
      if (xs[i] == nullptr || ys[i] == nullptr) return BINADE_EINVAL;
      if (!aligned16(xs[i])) return BINADE_EUNSUPPORTED;
      GemvArgs a = args_from_r4(&ws[i], true);
      a.x = xs[i];
      a.y = ys[i];
      a.y_bf16 = y_dtype == BINADE_BF16;
      items[n++] = a;
    }
    const int32_t s = launch_gemv_batch(items, n, true, static_cast<hipStream_t>(stream));
    if (s != BINADE_OK) return s;
  }
  return BINADE_OK;
}

extern "C" int32_t binade_bf16_gemv_batch(const uint16_t* const* ws, const int64_t* rows,
                                          const int64_t* cols, const uint16_t* const* xs,
                                          void* const* ys, int32_t count, int32_t y_dtype,
                                          void* stream) {
  if (count < 0 || (count > 0 && (ws == nullptr || rows == nullptr || cols == nullptr ||
                                  xs == nullptr || ys == nullptr)))
    return BINADE_EINVAL;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  GemvArgs items[kMaxBatch];
  for (int32_t base = 0; base < count; base += kMaxBatch) {
    int n = 0;
    for (int32_t i = base; i < count && i < base + kMaxBatch; ++i) {
      if (rows[i] < 0 || cols[i] <= 0) return BINADE_EINVAL;
      if (cols[i] % 32 != 0 || cols[i] > (1 << 30)) return BINADE_EUNSUPPORTED;
      if (rows[i] == 0) continue;
      if (ws[i] == nullptr || xs[i] == nullptr || ys[i] == nullptr) return BINADE_EINVAL;
      if (!aligned16(ws[i]) || !aligned16(xs[i])) return BINADE_EUNSUPPORTED;
      GemvArgs a{};
      a.sm = reinterpret_cast<const uint8_t*>(ws[i]);
      a.rows = rows[i];
      a.cols = static_cast<int32_t>(cols[i]);
      a.x = xs[i];
      a.y = ys[i];
      a.y_bf16 = y_dtype == BINADE_BF16;
      items[n++] = a;
    }
    const int32_t s = launch_gemv_batch(items, n, false, static_cast<hipStream_t>(stream));
    if (s != BINADE_OK) return s;
  }
  return BINADE_OK;
}

extern "C" int32_t binade_bf16_gemv(const uint16_t* w, int64_t rows,
                                    int64_t cols, const uint16_t* x, void* y,
                                    int32_t y_dtype, void* stream) {
  if (rows < 0 || cols <= 0) return BINADE_EINVAL;
  if (cols % 32 != 0 || cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (rows == 0) return BINADE_OK;
  if (w == nullptr || x == nullptr || y == nullptr) return BINADE_EINVAL;
  if (!aligned16(w) || !aligned16(x)) return BINADE_EUNSUPPORTED;
  GemvArgs a{};
  a.sm = reinterpret_cast<const uint8_t*>(w);
  a.rows = rows;
  a.cols = static_cast<int32_t>(cols);
  a.x = x;
  a.y = y;
  a.y_bf16 = y_dtype == BINADE_BF16;
  return launch_gemv(a, false, static_cast<hipStream_t>(stream));
}

extern "C" int32_t binade_unpack(const binade_r4* w, uint16_t* out,
                                 void* stream) {
  int32_t s = check_r4(w);
  if (s != BINADE_OK) return s;
  if (w->rows == 0) return BINADE_OK;
  if (out == nullptr) return BINADE_EINVAL;
  if (!aligned16(out)) return BINADE_EUNSUPPORTED;
  GemvArgs a = args_from_r4(w, false);
  const int64_t chunks = w->rows * ((w->cols / 32 + 63) / 64);
  const dim3 grid(static_cast<uint32_t>((chunks + 3) / 4));
  hipLaunchKernelGGL(r4_unpack_kernel, grid, dim3(256), 0,
                     static_cast<hipStream_t>(stream), a, out);
  return launch_status();
}

extern "C" int32_t binade_r4_gemv_rows(const binade_r4* w, const uint16_t* x, int64_t ldx,
                                       int32_t m, void* y, int64_t ldy, int32_t y_dtype,
                                       void* stream) {
  int32_t s = check_r4(w);
  if (s != BINADE_OK) return s;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (m < 1 || m > 8 || ldx < w->cols || ldy < w->rows) return BINADE_EINVAL;
  if (w->rows == 0) return BINADE_OK;
  if (x == nullptr || y == nullptr) return BINADE_EINVAL;
  if (!aligned16(x) || ldx % 8 != 0) return BINADE_EUNSUPPORTED;
  GemvRowsArgs ra{};
  ra.g = args_from_r4(w, true);
  ra.g.x = x;
  ra.g.y = y;
  ra.g.y_bf16 = y_dtype == BINADE_BF16;
  ra.ldx = ldx;
  ra.ldy = ldy;
  ra.m = m;
  return launch_gemv_rows(ra, true, static_cast<hipStream_t>(stream));
}

extern "C" int32_t binade_bf16_gemv_rows(const uint16_t* w, int64_t rows, int64_t cols,
                                         const uint16_t* x, int64_t ldx, int32_t m, void* y,
                                         int64_t ldy, int32_t y_dtype, void* stream) {
  if (rows < 0 || cols <= 0) return BINADE_EINVAL;
  if (cols % 32 != 0 || cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (m < 1 || m > 8 || ldx < cols || ldy < rows) return BINADE_EINVAL;
  if (rows == 0) return BINADE_OK;
  if (w == nullptr || x == nullptr || y == nullptr) return BINADE_EINVAL;
  if (!aligned16(w) || !aligned16(x) || ldx % 8 != 0) return BINADE_EUNSUPPORTED;
  GemvRowsArgs ra{};
  ra.g.sm = reinterpret_cast<const uint8_t*>(w);
  ra.g.rows = rows;
  ra.g.cols = static_cast<int32_t>(cols);
  ra.g.x = x;
  ra.g.y = y;
  ra.g.y_bf16 = y_dtype == BINADE_BF16;
  ra.ldx = ldx;
  ra.ldy = ldy;
  ra.m = m;
  return launch_gemv_rows(ra, false, static_cast<hipStream_t>(stream));
}
