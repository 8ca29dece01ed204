// Prompt GEMM Y[M,N] = X[M,K] W[N,K]^T with R4 weights rebuilt on the fly
// and multiplied on gfx950 bf16 MFMA, and its bf16-weight twin.
//
// "Binade" package page (pypi.org/project/binade), "Results": prompt
// processing runs the 12B model's matmuls with a fused GEMM; "Limitations":
// on long prompts the fused GEMM is weighed against rebuilding BF16 weights;
// "NVIDIA GPUs": a GEMM's order is a chain of matrix-core steps along K, with
// split-K partitions that follow a fixed rule.
//
// Order (every kernel here, independent of M, tiling and launch shape):
// K is cut into nsb = K / 128 super-blocks of 128 columns, then (K % 128)/32
// tail blocks of 32. Super-block u is four v_mfma_f32_16x16x32_bf16 steps;
// in step j, lane group g (lanes 16g .. 16g+15) carries columns
// 128u + 32g + 8j .. +7, so a lane's operands for the four steps are 32
// contiguous columns of its row. A tail block is one step whose lane group
// g carries columns 8g .. 8g+7 of the block. The super-blocks are split into
// S = min(8, ceil(K / 1024)) slices (slice s: [s*nsb/S, (s+1)*nsb/S); the
// last slice also takes the tail blocks). Per output and slice one fp32
// accumulator starts at +0.0 and takes the slice's steps in order; the
// output is (((p0 + p1) + p2) + ...) in slice order. The R4 kernels rebuild
// exactly the bf16 weights the twins read, so both issue identical MFMA
// sequences and their outputs agree bit for bit.
//
// Small M without a workspace (<= 16): one wave per 16 weight rows and 16 X
// rows; each lane loads its 32 columns of a super-block with 16-byte loads,
// the weights are rebuilt straight into MFMA operands in registers, the
// next super-block is
// loaded while the current one multiplies, and the S slices of a tile are S
// waves of one block, added in slice order through LDS. Blocks that share
// weight rows are placed on the same XCD (blocks are dealt to the 8 XCDs
// round robin), so their weight reads meet in that XCD's L2.
// M up to 32 (streamed): one block per (slice, group of 8 weight-row
// tiles) holds its slice's X columns in LDS; waves stream their tiles'
// weights two super-blocks ahead; slice partials go to the workspace and a
// second kernel adds them in slice order.
// M up to 128: tiles of 128 X rows by 128 weight rows, 8 waves; per
// super-block the X rows and the rebuilt weights go through LDS (rows
// padded to 272 bytes) while the next super-block is loaded into
// registers. Larger M: tiles of 256 X rows, X copied by DMA straight into
// two alternating LDS buffers one super-block ahead, weights through
// registers into one buffer; both tiles swizzled instead of padded. A
// block runs all slices of its tile with a running total, or, when the
// tiles alone cannot fill the chip and the caller gave a workspace, one
// slice, whose fp32 partials a second kernel adds in slice order.
#include <hip/hip_runtime.h>

#include <mutex>

#include "binade.h"
#include "device_common.h"

// Fixed device scratch of binade_r4_gemm_noalloc: the split slices' partial
// sums (32 MiB). Every device the library runs on holds its own copy until
// the process ends. In host code `scratch` names a host-side stand-in, never
// the device memory: host code uses only the per-device address that
// scratch_address() looks up.
static __device__ __align__(256) uint8_t scratch[32ll << 20];

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
  float* part;                       // split large kernel: [S][M][N] partials
};

constexpr int kXcds = 8;

constexpr int kSB = 128;   // columns per super-block

// Super-block range [lo, hi) of slice s; the last slice also owns the tail
// blocks (K % 128) / 32.
__device__ __forceinline__ void slice_superblocks(int32_t k, int32_t S, int32_t s, int32_t& lo,
                                                  int32_t& hi) {
  const int32_t nsb = k / kSB;
  lo = (s * nsb) / S;
  hi = ((s + 1) * nsb) / S;
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

// The side-list entries of one weight row over a column range [col0, col1)
// that touches at most two row-chunks, at most four per chunk, read once
// before the range is walked, so that an escape is patched from registers.
// Entry: (rotated exponent << 16) | column - col0; 0xFFFF: none. `over`: the range
// touches a third chunk or a chunk has more than four entries (then the
// search of patch8 is used).
struct EscTab {
  uint32_t ent[8];
  uint32_t over;
};

__device__ __forceinline__ void esc_tab_build(const GemmArgs& a, int64_t n, int32_t col0,
                                              int32_t col1, EscTab& t) {
  const int64_t C = (a.k + kChunk - 1) / kChunk;
  const int32_t j0 = col0 / kChunk, jl = (col1 - 1) / kChunk;
  uint32_t over = jl > j0 + 1 ? 1u : 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int32_t j = j0 + h;
    uint32_t eb = 0, ee = 0;
    if (j <= jl) {
      ee = a.esc_pre[n * C + j + 1];
      eb = a.esc_pre[n * C + j];
      ee = ee < a.n_esc ? ee : a.n_esc;
      eb = eb < ee ? eb : ee;
    }
    if (ee - eb > 4u) over = 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = 0xFFFFu;
      if (eb + i < ee) {
        const uint32_t ent = a.esc[eb + i];
        const int32_t col = j * kChunk + static_cast<int32_t>(ent & 0xFFFFu);
        if (col >= col0 && col < col1)
          v = (rot_exponent((ent >> 16) & 0xFFu) << 16) | static_cast<uint32_t>(col - col0);
      }
      t.ent[4 * h + i] = v;
    }
  }
  t.over = over;
}

// Patch the exponents of columns c .. c+7 (c = col0 + c_rel) from the table.
__device__ __forceinline__ void esc_tab_patch(const EscTab& t, int32_t c_rel, uint32_t& E0,
                                              uint32_t& E1) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t d = (t.ent[i] & 0xFFFFu) - static_cast<uint32_t>(c_rel);
    if (d < 8u) {
      const uint32_t sh = (d & 3u) * 8u;
      const uint32_t ex = (t.ent[i] >> 16) << sh;
      if (d < 4u)
        E0 = (E0 & ~(0xFFu << sh)) | ex;
      else
        E1 = (E1 & ~(0xFFu << sh)) | ex;
    }
  }
}

// rebuild8 with the escapes of the row taken from its table.
__device__ __forceinline__ uint4 rebuild8_tab(const GemmArgs& a, const Lut& L, uint2 sm,
                                              uint32_t P, int64_t n, int32_t c0,
                                              const EscTab& t, int32_t c_rel) {
  uint32_t E0 = lookup4(P, L);
  uint32_t E1 = lookup4(P >> 4, L);
  if (has_escape(P)) {
    if (t.over)
      patch8(a, n, c0, E0, E1);
    else
      esc_tab_patch(t, c_rel, E0, E1);
  }
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
// One lane's loads for one super-block: 32 columns of its weight row (R4:
// 32 sm bytes + 16 nibble bytes; twin: 32 bf16) and of MT X rows.
template <bool kR4, int MT>
struct SmallRaw {
  uint4 s0, s1, nb;   // R4
  uint4 w[4];         // twin
  uint4 x[MT][4];
};

// Rows past N (or M) are read from the last row instead: an MFMA output
// depends only on its own A row and B column, and those outputs are never
// stored, so every load is unconditional. c = first of the lane's columns.
template <bool kR4, int MT>
__device__ __forceinline__ void small_load(const uint8_t* wrow, const uint8_t* nrow,
                                           const uint16_t* const (&xrow)[MT], int32_t c,
                                           SmallRaw<kR4, MT>& r) {
  if (kR4) {
    const uint4* ps = reinterpret_cast<const uint4*>(wrow + c);
    r.s0 = ps[0];
    r.s1 = ps[1];
    r.nb = *reinterpret_cast<const uint4*>(nrow + (c >> 1));
  } else {
    const uint4* pw = reinterpret_cast<const uint4*>(wrow + 2 * c);
#pragma unroll
    for (int v = 0; v < 4; ++v) r.w[v] = pw[v];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const uint4* px = reinterpret_cast<const uint4*>(xrow[t] + c);
#pragma unroll
    for (int v = 0; v < 4; ++v) r.x[t][v] = px[v];
  }
}

// The four MFMA steps of one super-block (columns c .. c+31 of this lane).
template <bool kR4, int MT>
__device__ __forceinline__ void small_steps(const GemmArgs& a, const Lut& L, int64_t n,
                                            int32_t c, const SmallRaw<kR4, MT>& q,
                                            floatx4 (&acc)[MT]) {
  const uint32_t S[8] = {q.s0.x, q.s0.y, q.s0.z, q.s0.w, q.s1.x, q.s1.y, q.s1.z, q.s1.w};
  const uint32_t P[4] = {q.nb.x, q.nb.y, q.nb.z, q.nb.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x8 B;
    if (kR4)
      B = as_bf16x8(rebuild8(a, L, make_uint2(S[2 * j], S[2 * j + 1]), P[j], n, c + 8 * j));
    else
      B = as_bf16x8(q.w[j]);
#pragma unroll
    for (int t = 0; t < MT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(q.x[t][j]), B, acc[t], 0, 0, 0);
  }
}

// Block (x = tile of 16 weight rows and 16*MT X rows, as dealt to XCDs),
// one wave per slice; the next super-block's loads are in flight while the
// current one multiplies.
template <bool kR4, int MT>
__global__ __launch_bounds__(512) void gemm_small_kernel(GemmArgs a) {
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
  int32_t u0, u1;
  slice_superblocks(a.k, a.slices, s, u0, u1);

  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  SmallRaw<kR4, MT> q0, q1;
  if (u0 < u1) small_load<kR4, MT>(wrow, nrow, xrow, u0 * kSB + 32 * g, q0);
  int32_t u = u0;
  for (; u + 2 <= u1; u += 2) {
    small_load<kR4, MT>(wrow, nrow, xrow, (u + 1) * kSB + 32 * g, q1);
    small_steps<kR4, MT>(a, L, n, u * kSB + 32 * g, q0, acc);
    if (u + 2 < u1) small_load<kR4, MT>(wrow, nrow, xrow, (u + 2) * kSB + 32 * g, q0);
    small_steps<kR4, MT>(a, L, n, (u + 1) * kSB + 32 * g, q1, acc);
  }
  if (u < u1) small_steps<kR4, MT>(a, L, n, u * kSB + 32 * g, q0, acc);

  if (s == a.slices - 1) {
    // tail blocks: one plain 32-column step each
    const int32_t tail0 = (a.k / kSB) * kSB;
    for (int32_t c0 = tail0; c0 < a.k; c0 += 32) {
      const int32_t c = c0 + 8 * g;
      bf16x8 B;
      if (kR4)
        B = as_bf16x8(rebuild8(a, L, *reinterpret_cast<const uint2*>(wrow + c),
                               *reinterpret_cast<const uint32_t*>(nrow + (c >> 1)), n, c));
      else
        B = as_bf16x8(*reinterpret_cast<const uint4*>(wrow + 2 * c));
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(xrow[t] + c)), B, acc[t], 0, 0, 0);
    }
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

// ---------------------------------------------------------------- small M, streamed
// One block per (slice, group of 8 weight-row tiles): the block copies its
// slice's X columns (16*MT rows) into LDS once, then each wave streams one
// or more 16-row tiles over the slice's super-blocks, kRing super-blocks of
// weight loads in flight (the ring runs on across tiles), X operands read
// from LDS. A tile's slice partial goes to the workspace (or to Y when there
// is one slice); gemm_combine_kernel adds the slices in order.
constexpr int kStreamWaves = 8;
#ifndef BINADE_GEMM_STREAM_RING
#define BINADE_GEMM_STREAM_RING 2
#endif
constexpr int kRing = BINADE_GEMM_STREAM_RING;

template <bool kR4>
struct StreamRaw;
template <>
struct StreamRaw<true> {
  uint4 s0, s1, nb;
};
template <>
struct StreamRaw<false> {
  uint4 w[4];
};

// Weight loads of one super-block for lane (r, g): 32 columns from column
// offset c of the row (R4: sm and nibble rows; twin: bf16 row in `srow`).
template <bool kR4>
__device__ __forceinline__ void stream_load(const uint8_t* srow, const uint8_t* nrow, int32_t c,
                                            StreamRaw<kR4>& q) {
  if constexpr (kR4) {
    const uint4* ps = reinterpret_cast<const uint4*>(srow + c);
    q.s0 = ps[0];
    q.s1 = ps[1];
    q.nb = *reinterpret_cast<const uint4*>(nrow + (c >> 1));
  } else {
    const uint4* pw = reinterpret_cast<const uint4*>(srow + 2 * c);
#pragma unroll
    for (int v = 0; v < 4; ++v) q.w[v] = pw[v];
  }
}

// Escape tables of a tile's weight rows in LDS (the tiled kernel): per row
// the 8 entries and the `over` word of an EscTab built over a column range
// of at most two row-chunks (kEscRange columns from a chunk pair's start).
constexpr int kEscWords = 9;
constexpr int kEscRange = 2 * kChunk;

__device__ __forceinline__ void esc_tab_store(const EscTab& t, uint32_t* row) {
#pragma unroll
  for (int i = 0; i < 8; ++i) row[i] = t.ent[i];
  row[8] = t.over;
}

// Escapes among the 8 ranks of nibble word P (columns c0 .. c0+7 of row n):
// patch E0 (c0 .. c0+3) and E1 (c0+4 .. c0+7) from the row's LDS table
// (c_rel: c0 relative to the table's first column).
__device__ __forceinline__ void esc_patch_lds(const GemmArgs& a, int64_t n, int32_t c0,
                                              uint32_t P, const uint32_t* trow, int32_t c_rel,
                                              uint32_t& E0, uint32_t& E1) {
  if (has_escape(P)) {
    if (trow[8]) {
      patch8(a, n, c0, E0, E1);
    } else {
      EscTab t;
#pragma unroll
      for (int i = 0; i < 8; ++i) t.ent[i] = trow[i];
      t.over = 0;
      esc_tab_patch(t, c_rel, E0, E1);
    }
  }
}

// Nonzero when any of the 32 nibbles of q is 15 (an escape): a nibble of
// ~P is zero exactly where P's is 15, and (v - 0x11..) & ~v & 0x88.. flags a
// word holding a zero nibble.
__device__ __forceinline__ uint32_t any_escape32(uint4 nb) {
  const uint32_t P[4] = {nb.x, nb.y, nb.z, nb.w};
  uint32_t f = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) f |= (0xEEEEEEEEu - P[j]) & P[j] & 0x88888888u;
  return f;
}

// Escapes among the 8 ranks of nibble word P (columns c .. c+7 of row n):
// patch their exponents in E0 (c .. c+3) and E1 (c+4 .. c+7).
__device__ __forceinline__ void esc_patch_word(const GemmArgs& a, const EscTab& t, int64_t n,
                                               int32_t c, int32_t c_rel, uint32_t P,
                                               uint32_t& E0, uint32_t& E1) {
  if (has_escape(P)) {
    if (t.over)
      patch8(a, n, c, E0, E1);
    else
      esc_tab_patch(t, c_rel, E0, E1);
  }
}

// The four weights of sm word S with exponents E as two bf16 pairs.
__device__ __forceinline__ uint2 bf16_pairs4(uint32_t S, uint32_t E) {
  uint32_t H, Lo;
  split4_rot(S, E, H, Lo);
  return make_uint2(weight_pair_bf16<0>(H, Lo), weight_pair_bf16<2>(H, Lo));
}

// The 32 weights of one super-block for lane (r, g) (columns c .. c+31 of
// row n; c_rel: c relative to the table's first column), as the four MFMA
// operands of steps 0..3. Values, not references: the words stay in VGPRs.
__device__ __forceinline__ void rebuild32(const GemmArgs& a, const Lut& L, uint4 s0, uint4 s1,
                                          uint4 nb, int64_t n, int32_t c, const EscTab& t,
                                          int32_t c_rel, bf16x8 (&B)[4]) {
  uint32_t E0 = lookup4(nb.x, L), E1 = lookup4(nb.x >> 4, L);
  uint32_t E2 = lookup4(nb.y, L), E3 = lookup4(nb.y >> 4, L);
  uint32_t E4 = lookup4(nb.z, L), E5 = lookup4(nb.z >> 4, L);
  uint32_t E6 = lookup4(nb.w, L), E7 = lookup4(nb.w >> 4, L);
  if (any_escape32(nb)) {
    esc_patch_word(a, t, n, c, c_rel, nb.x, E0, E1);
    esc_patch_word(a, t, n, c + 8, c_rel + 8, nb.y, E2, E3);
    esc_patch_word(a, t, n, c + 16, c_rel + 16, nb.z, E4, E5);
    esc_patch_word(a, t, n, c + 24, c_rel + 24, nb.w, E6, E7);
  }
  uint2 p0 = bf16_pairs4(s0.x, E0), p1 = bf16_pairs4(s0.y, E1);
  B[0] = as_bf16x8(make_uint4(p0.x, p0.y, p1.x, p1.y));
  p0 = bf16_pairs4(s0.z, E2), p1 = bf16_pairs4(s0.w, E3);
  B[1] = as_bf16x8(make_uint4(p0.x, p0.y, p1.x, p1.y));
  p0 = bf16_pairs4(s1.x, E4), p1 = bf16_pairs4(s1.y, E5);
  B[2] = as_bf16x8(make_uint4(p0.x, p0.y, p1.x, p1.y));
  p0 = bf16_pairs4(s1.z, E6), p1 = bf16_pairs4(s1.w, E7);
  B[3] = as_bf16x8(make_uint4(p0.x, p0.y, p1.x, p1.y));
}

// X operand of m-tile t for lane (r, g), LDS column col (bf16 elements).
template <int MT>
__device__ __forceinline__ bf16x8 stream_x(const uint16_t* xs, int32_t xstride, int t, int r,
                                           int32_t col) {
  return *reinterpret_cast<const bf16x8*>(xs + (t * 16 + r) * xstride + col);
}

template <bool kR4, int MT>
__global__ __launch_bounds__(64 * kStreamWaves) void gemm_stream_kernel(GemmArgs a,
                                                                        int32_t xstride,
                                                                        int32_t groups) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(static_cast<int>(tid >> 6));
  const int32_t S = a.slices;
  const int32_t s = static_cast<int32_t>(blockIdx.x % S);
  const int32_t gi = static_cast<int32_t>(blockIdx.x / S);
  int32_t lo, hi;
  slice_superblocks(a.k, S, s, lo, hi);
  const int32_t nsb = a.k / kSB;
  const int32_t c_lo = lo * kSB;
  const int32_t tails = s == S - 1 ? (a.k - nsb * kSB) / 32 : 0;
  const int32_t cols = (hi - lo) * kSB + 32 * tails;

  const int64_t ntiles = (a.n + 15) / 16;
  const int64_t t0 = (ntiles * gi) / groups, t1 = (ntiles * (gi + 1)) / groups;
  const int32_t len = hi - lo;
  // this wave's tiles: t0 + wave, t0 + wave + 8, ...
  const int64_t my = t1 > t0 + wave ? (t1 - t0 - wave + kStreamWaves - 1) / kStreamWaves : 0;
  const int64_t items = my * len;
  const int r = lane & 15, g = lane >> 4;
  int64_t cs_tile = t0 + wave;
  const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};

  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // load side and consume side walk the same (tile, u) sequence; a row
  // past N reads row N-1 (its outputs are never stored)
  const int64_t rstep = static_cast<int64_t>(kStreamWaves) * 16;
  const int64_t sm_row = kR4 ? a.k : 2 * static_cast<int64_t>(a.k);
  int64_t ld_row = t0 * 16 + wave * 16 + r, cs_n = min(ld_row, a.n - 1);
  const uint8_t* ld_s = a.w + min(ld_row, a.n - 1) * sm_row;
  const uint8_t* ld_nb = a.nib + min(ld_row, a.n - 1) * (a.k >> 1);
  int32_t ld_u = lo, cs_u = lo;
  StreamRaw<kR4> ring[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) {
    if (k < items) {
      stream_load<kR4>(ld_s, ld_nb, ld_u * kSB + 32 * g, ring[k]);
      if (++ld_u == hi) {
        ld_u = lo;
        ld_row += rstep;
        ld_s = a.w + min(ld_row, a.n - 1) * sm_row;
        ld_nb = a.nib + min(ld_row, a.n - 1) * (a.k >> 1);
      }
    }
  }
  // the escapes of this lane's row over the slice's columns
  EscTab tab;
  if (kR4 && items > 0) esc_tab_build(a, cs_n, c_lo, c_lo + cols, tab);
  // (the first weight loads are in flight while the block copies X)
  // the slice's X columns, rows past M repeated from row M-1 (never stored)
  {
    const int32_t segs = cols / 8;
    for (int32_t i = tid; i < 16 * MT * segs; i += 64 * kStreamWaves) {
      const int32_t row = i / segs, seg = i - row * segs;
      const int64_t xm = min(static_cast<int64_t>(row), a.m - 1);
      *reinterpret_cast<uint4*>(xs + row * xstride + 8 * seg) =
          *reinterpret_cast<const uint4*>(a.x + xm * a.ldx + c_lo + 8 * seg);
    }
  }
  __syncthreads();

  for (int64_t i = 0; i < items; i += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      if (i + k < items) {
        const int64_t n = cs_n;
        const int32_t c = cs_u * kSB + 32 * g;
        const int32_t xc = (cs_u - lo) * kSB + 32 * g;
        const StreamRaw<kR4> q = ring[k];
        if (i + k + kRing < items) {
          stream_load<kR4>(ld_s, ld_nb, ld_u * kSB + 32 * g, ring[k]);
          if (++ld_u == hi) {
            ld_u = lo;
            ld_row += rstep;
            ld_s = a.w + min(ld_row, a.n - 1) * sm_row;
            ld_nb = a.nib + min(ld_row, a.n - 1) * (a.k >> 1);
          }
        }
        bf16x8 B[4];
        if constexpr (kR4) {
          rebuild32(a, L, q.s0, q.s1, q.nb, n, c, tab, xc, B);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) B[j] = as_bf16x8(q.w[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                stream_x<MT>(xs, xstride, t, r, xc + 8 * j), B[j], acc[t], 0, 0, 0);
        if (++cs_u == hi) {
          // tail blocks (last slice only), then the tile's partial
          for (int32_t b = 0; b < tails; ++b) {
            const int32_t c0 = nsb * kSB + 32 * b + 8 * g;
            bf16x8 B;
            if constexpr (kR4)
              B = as_bf16x8(rebuild8_tab(
                  a, L, *reinterpret_cast<const uint2*>(a.w + n * a.k + c0),
                  *reinterpret_cast<const uint32_t*>(a.nib + n * (a.k >> 1) + (c0 >> 1)), n, c0,
                  tab, c0 - c_lo));
            else
              B = as_bf16x8(*reinterpret_cast<const uint4*>(a.w + 2 * (n * a.k + c0)));
#pragma unroll
            for (int t = 0; t < MT; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  stream_x<MT>(xs, xstride, t, r, len * kSB + 32 * b + 8 * g), B, acc[t], 0, 0,
                  0);
          }
          const int64_t on = cs_tile * 16 + r;   // (tile of the consume side)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t om = t * 16 + 4 * g + e;
              if (S == 1)
                store_out(a, om, on, acc[t][e]);
              else if (om < a.m && on < a.n)
                a.part[(static_cast<int64_t>(s) * a.m + om) * a.n + on] = acc[t][e];
            }
            acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
          }
          cs_u = lo;
          cs_tile += kStreamWaves;
          cs_n = min(cs_tile * 16 + r, a.n - 1);
          if (kR4 && i + k + 1 < items) esc_tab_build(a, cs_n, c_lo, c_lo + cols, tab);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- large M
// Tiles of BM X rows by 128 weight rows; waves of 64 X rows x 16*NJ weight
// rows: (BM/64) x (128/(16*NJ)) waves. Each rebuilt weight feeds BM X rows.
// Unsplit, a block runs every slice of its tile in order with a running
// total. Split, a block runs one slice and writes its accumulators to the
// workspace; gemm_combine_kernel then adds the slices in order (the same
// fp32 adds as the running total).
constexpr int kBN = 128;
// bf16 elements per LDS row: 128 + 8, so that rows start 4 banks apart and
// both the 16-byte stores of staging and the 16-byte MFMA operand reads of
// 8 consecutive rows fall in distinct banks
constexpr int kLdsStride = kSB + 8;

template <int BM, int NJ>
constexpr int large_threads() {
  return (BM / 64) * (kBN / (16 * NJ)) * 64;
}

// One thread's loads for one super-block, T threads. X: BM*16/T rows
// (v*T/16 + tid/16) x 16 bytes (segment tid%16); twin weights: 128*16/T
// such rows; R4: 128*8/T rows (v*T/8 + tid/8) x 16 sm bytes (segment tid%8)
// and their 8 nibble bytes.
template <bool kR4, int BM, int T>
struct LargeRaw;
template <int BM, int T>
struct LargeRaw<true, BM, T> {
  uint4 x[BM * 16 / T];
  uint4 sm[kBN * 8 / T];
  uint2 nb[kBN * 8 / T];
};
template <int BM, int T>
struct LargeRaw<false, BM, T> {
  uint4 x[BM * 16 / T];
  uint4 w[kBN * 16 / T];
};

// Rows past M or N load zeros (their outputs are never stored; the zero is
// assigned first and the load made conditional, since a conditional
// expression over two uint4 lvalues would select an address). Each load
// address is a block-uniform base plus a 32-bit per-lane byte offset, so the
// loop keeps one offset register per operand instead of a pointer per row.
template <bool kR4, int BM, int T>
__device__ __forceinline__ void large_load(const GemmArgs& a, int32_t c0, int tid, int64_t m0,
                                           int64_t n0, uint32_t xo, uint32_t wo, uint32_t no,
                                           LargeRaw<kR4, BM, T>& q) {
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  constexpr int XR = T / 16;
#pragma unroll
  for (int v = 0; v < BM / XR; ++v) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x + (m0 + v * XR) * a.ldx + c0);
    q.x[v] = z4;
    if (m0 + v * XR + (tid >> 4) < a.m) q.x[v] = *reinterpret_cast<const uint4*>(base + xo);
  }
  if constexpr (kR4) {
    constexpr int RR = T / 8;
#pragma unroll
    for (int v = 0; v < kBN / RR; ++v) {
      const bool ok = n0 + v * RR + (tid >> 3) < a.n;
      const uint8_t* bs = a.w + (n0 + v * RR) * a.k + c0;
      const uint8_t* bn = a.nib + (n0 + v * RR) * (a.k >> 1) + (c0 >> 1);
      q.sm[v] = z4;
      q.nb[v] = make_uint2(0, 0);
      if (ok) {
        q.sm[v] = *reinterpret_cast<const uint4*>(bs + wo);
        q.nb[v] = *reinterpret_cast<const uint2*>(bn + no);
      }
    }
  } else {
    constexpr int WR = T / 16;
#pragma unroll
    for (int v = 0; v < kBN / WR; ++v) {
      const uint8_t* base = a.w + ((n0 + v * WR) * a.k + c0) * 2;
      q.w[v] = z4;
      if (n0 + v * WR + (tid >> 4) < a.n) q.w[v] = *reinterpret_cast<const uint4*>(base + wo);
    }
  }
}

template <bool kR4, int BM, int T>
__device__ __forceinline__ void large_stage(const GemmArgs& a, const Lut& L, int32_t c0, int tid,
                                            int64_t n0, uint16_t (*xs)[kLdsStride],
                                            uint16_t (*ws)[kLdsStride],
                                            const LargeRaw<kR4, BM, T>& q,
                                            const uint32_t (*etab)[kEscWords], int32_t tcol0) {
  constexpr int XR = T / 16;
#pragma unroll
  for (int v = 0; v < BM / XR; ++v)
    *reinterpret_cast<uint4*>(&xs[v * XR + (tid >> 4)][8 * (tid & 15)]) = q.x[v];
  if constexpr (kR4) {
    constexpr int RR = T / 8, RP = kBN / RR;
    const int cc = 16 * (tid & 7);
    // exponents of every row first, one test for an escape among all of
    // this thread's nibbles, then the (rare) patches from the row tables
    uint32_t E[RP][4];
    uint32_t esc = 0;
#pragma unroll
    for (int v = 0; v < RP; ++v) {
      E[v][0] = lookup4(q.nb[v].x, L);
      E[v][1] = lookup4(q.nb[v].x >> 4, L);
      E[v][2] = lookup4(q.nb[v].y, L);
      E[v][3] = lookup4(q.nb[v].y >> 4, L);
      esc |= (0xEEEEEEEEu - q.nb[v].x) & q.nb[v].x & 0x88888888u;
      esc |= (0xEEEEEEEEu - q.nb[v].y) & q.nb[v].y & 0x88888888u;
    }
    if (esc) {
#pragma unroll
      for (int v = 0; v < RP; ++v) {
        const int row = v * RR + (tid >> 3);
        // rows past N hold zeros, which have no escapes
        esc_patch_lds(a, n0 + row, c0 + cc, q.nb[v].x, etab[row], c0 + cc - tcol0, E[v][0],
                      E[v][1]);
        esc_patch_lds(a, n0 + row, c0 + cc + 8, q.nb[v].y, etab[row], c0 + cc + 8 - tcol0,
                      E[v][2], E[v][3]);
      }
    }
#pragma unroll
    for (int v = 0; v < RP; ++v) {
      const int row = v * RR + (tid >> 3);
      const uint2 p0 = bf16_pairs4(q.sm[v].x, E[v][0]), p1 = bf16_pairs4(q.sm[v].y, E[v][1]);
      const uint2 p2 = bf16_pairs4(q.sm[v].z, E[v][2]), p3 = bf16_pairs4(q.sm[v].w, E[v][3]);
      *reinterpret_cast<uint4*>(&ws[row][cc]) = make_uint4(p0.x, p0.y, p1.x, p1.y);
      *reinterpret_cast<uint4*>(&ws[row][cc + 8]) = make_uint4(p2.x, p2.y, p3.x, p3.y);
    }
  } else {
    constexpr int WR = T / 16;
#pragma unroll
    for (int v = 0; v < kBN / WR; ++v)
      *reinterpret_cast<uint4*>(&ws[v * WR + (tid >> 4)][8 * (tid & 15)]) = q.w[v];
  }
}

// Staging of one 32-column tail block (plain lane-group mapping); needs at
// least 2*BM and 2*128 threads.
template <bool kR4, int BM>
__device__ __forceinline__ void large_stage_tail(const GemmArgs& a, const Lut& L, int32_t c0,
                                                 int tid, int64_t m0, int64_t n0,
                                                 uint16_t (*xs)[kLdsStride],
                                                 uint16_t (*ws)[kLdsStride]) {
  if (tid < 2 * BM) {
    const int row = tid >> 1, cc = 16 * (tid & 1);
    const int64_t xm = min(m0 + row, a.m - 1);   // rows past M: never stored
    const uint4* px = reinterpret_cast<const uint4*>(a.x + xm * a.ldx + c0 + cc);
    *reinterpret_cast<uint4*>(&xs[row][cc]) = px[0];
    *reinterpret_cast<uint4*>(&xs[row][cc + 8]) = px[1];
  }
  if (tid < 2 * kBN) {
    const int row = tid >> 1, cc = 16 * (tid & 1);
    const int64_t wn = min(n0 + row, a.n - 1);   // rows past N: never stored
    uint4 lo, hi;
    if constexpr (kR4) {
      const uint4 sm = *reinterpret_cast<const uint4*>(a.w + wn * a.k + c0 + cc);
      const uint2 nb = *reinterpret_cast<const uint2*>(a.nib + wn * (a.k >> 1) + ((c0 + cc) >> 1));
      lo = rebuild8(a, L, make_uint2(sm.x, sm.y), nb.x, wn, c0 + cc);
      hi = rebuild8(a, L, make_uint2(sm.z, sm.w), nb.y, wn, c0 + cc + 8);
    } else {
      const uint4* pw = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.w) +
                                                       wn * a.k + c0 + cc);
      lo = pw[0];
      hi = pw[1];
    }
    *reinterpret_cast<uint4*>(&ws[row][cc]) = lo;
    *reinterpret_cast<uint4*>(&ws[row][cc + 8]) = hi;
  }
}

// One MFMA step over the staged operands: A rows from xs, B rows from ws,
// 8 columns starting at column `col` of the staged block.
template <int NJ>
__device__ __forceinline__ void large_step(const uint16_t (*xs)[kLdsStride],
                                           const uint16_t (*ws)[kLdsStride], int wm, int wn,
                                           int r, int col, floatx4 (&acc)[4][NJ]) {
  bf16x8 A[4], Bv[NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    A[i] = *reinterpret_cast<const bf16x8*>(&xs[wm + 16 * i + r][col]);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    Bv[j] = *reinterpret_cast<const bf16x8*>(&ws[wn + 16 * j + r][col]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], Bv[j], acc[i][j], 0, 0, 0);
}

template <int NJ>
__device__ __forceinline__ void fold(int32_t s, floatx4 (&acc)[4][NJ], floatx4 (&tot)[4][NJ]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      tot[i][j] = s == 0 ? acc[i][j] : tot[i][j] + acc[i][j];
      acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

// Waves per SIMD the launch bounds ask the register allocator for.
template <int BM, int NJ, bool kSplit>
constexpr int large_min_waves() {
  return large_threads<BM, NJ>() == 512 && NJ == 2 && kSplit ? 4 : 2;
}

// kSplit: blockIdx -> (tile, slice), one slice per block, fp32 partials to
// a.part[slice][m][n]; otherwise blockIdx -> tile, all slices in order.
template <bool kR4, int BM, int NJ, bool kSplit>
__global__ __launch_bounds__((large_threads<BM, NJ>()), (large_min_waves<BM, NJ, kSplit>()))
void gemm_large_kernel(GemmArgs a) {
  constexpr int T = large_threads<BM, NJ>();
  constexpr int NW = kBN / (16 * NJ);   // waves along N
  static_assert(T >= 2 * BM && T >= 2 * kBN, "tail staging needs 2 threads per row");
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM][kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t ws[kBN][kLdsStride];
  __shared__ uint32_t etab[kR4 ? kBN : 1][kEscWords];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // XCD-aware order: consecutive items (same weight rows) per XCD
  const int64_t tiles_n = (a.n + kBN - 1) / kBN, tiles_m = (a.m + BM - 1) / BM;
  const int32_t S = a.slices;
  const int64_t items = tiles_n * tiles_m * (kSplit ? S : 1);
  const int64_t per = (items + kXcds - 1) / kXcds;
  const int64_t item = static_cast<int64_t>(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (item >= items) return;
  const int64_t tile = kSplit ? item / S : item;
  const int32_t s_only = kSplit ? static_cast<int32_t>(item - tile * S) : 0;
  const int64_t n0 = (tile / tiles_m) * kBN;
  const int64_t m0 = (tile % tiles_m) * BM;
  const int wm = (wave / NW) * 64;
  const int wn = (wave % NW) * (16 * NJ);
  const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};
  const int r = lane & 15, g = lane >> 4;

  floatx4 acc[4][NJ], tot[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) tot[i][j] = acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t nsb = a.k / kSB;
  int32_t s = s_only, u_lo, s_hi;
  slice_superblocks(a.k, S, s, u_lo, s_hi);
  const int32_t u_end = kSplit ? s_hi : nsb;
  const bool with_tail = !kSplit || s_only == S - 1;
  // per-lane byte offsets (the launch bounds K and ldx so these fit)
  const uint32_t xo = static_cast<uint32_t>(((tid >> 4) * a.ldx + 8 * (tid & 15)) * 2);
  const uint32_t wo = kR4 ? static_cast<uint32_t>((tid >> 3) * a.k + 16 * (tid & 7))
                          : static_cast<uint32_t>(((tid >> 4) * a.k + 8 * (tid & 15)) * 2);
  const uint32_t no = static_cast<uint32_t>((tid >> 3) * (a.k >> 1) + 8 * (tid & 7));
  if (u_lo < u_end) {
    LargeRaw<kR4, BM, T> q;
    large_load<kR4, BM, T>(a, u_lo * kSB, tid, m0, n0, xo, wo, no, q);
    int32_t tcol0 = 0;   // first column of the escape tables
    const int32_t u_first = u_lo;
    for (int32_t u = u_lo; u < u_end; ++u) {
      __syncthreads();   // every wave is done reading the previous super-block
      if (kR4 && (u == u_first || (u * kSB) % kEscRange == 0)) {
        // tables of the tile's rows from here to the end of this chunk pair
        tcol0 = u * kSB;
        const int32_t tcol1 = min(a.k, (tcol0 / kEscRange + 1) * kEscRange);
        if (tid < kBN) {
          EscTab t;
          if (n0 + tid < a.n) {
            esc_tab_build(a, n0 + tid, tcol0, tcol1, t);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) t.ent[i] = 0xFFFFu;
            t.over = 0;
          }
          esc_tab_store(t, etab[tid]);
        }
        __syncthreads();
      }
      large_stage<kR4, BM, T>(a, L, u * kSB, tid, n0, xs, ws, q, etab, tcol0);
      __syncthreads();
      // the next super-block (the last one again on the last pass: always in
      // bounds, and the load stays unconditional)
      large_load<kR4, BM, T>(a, min(u + 1, u_end - 1) * kSB, tid, m0, n0, xo, wo, no, q);
#pragma unroll
      for (int j = 0; j < 4; ++j) large_step<NJ>(xs, ws, wm, wn, r, 32 * g + 8 * j, acc);
      if (!kSplit && u + 1 == s_hi && s + 1 < S) {
        fold<NJ>(s, acc, tot);   // end of slice s (the last slice ends after the tail)
        ++s;
        slice_superblocks(a.k, S, s, u_lo, s_hi);
      }
    }
  }
  if (with_tail) {
    for (int32_t c0 = nsb * kSB; c0 < a.k; c0 += 32) {
      __syncthreads();
      large_stage_tail<kR4, BM>(a, L, c0, tid, m0, n0, xs, ws);
      __syncthreads();
      large_step<NJ>(xs, ws, wm, wn, r, 8 * g, acc);
    }
  }

  if (kSplit && S > 1) {
    float* part = a.part + static_cast<int64_t>(s_only) * a.m * a.n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t on = n0 + wn + 16 * j + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t om = m0 + wm + 16 * i + 4 * g + e;
          if (om < a.m && on < a.n) part[om * a.n + on] = acc[i][j][e];
        }
      }
    return;
  }
  if (!kSplit) fold<NJ>(s, acc, tot);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t on = n0 + wn + 16 * j + r;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        store_out(a, m0 + wm + 16 * i + 4 * g + e, on, kSplit ? acc[i][j][e] : tot[i][j][e]);
    }
}

// ---------------------------------------------------------------- large M, X by DMA
// Tiles of 256 X rows by 128 weight rows, 8 waves of 64 x 64 (4 along M, 2
// along N). Per super-block the X tile goes from global memory straight
// into LDS (16 bytes per lane, no registers) one super-block ahead, into two
// alternating buffers; the weights go through registers (rebuilt for R4,
// escapes patched from per-row tables held in registers) into one buffer.
// Both LDS tiles are unpadded rows of 16 pieces of 8 columns, piece p of
// row R stored at slot p ^ (R & 7): the DMA writes whole rows in order, and
// the 8 rows an MFMA operand read touches hit 8 different bank groups.
constexpr int kDmaBM = 256;
constexpr int kDmaThreads = 512;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from src to LDS dst + 16 * lane (dst wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
// The compiler does not see the DMA's LDS writes: wait for every vector
// memory load of this wave, with fences so LDS accesses stay on their side.
__device__ __forceinline__ void dma_wait() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Block barrier for LDS hand-offs only: this wave's LDS operations are
// complete, then s_barrier. (__syncthreads also waits for every outstanding
// global load, which would drain the loads issued ahead for the next
// super-block.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Element offset of piece p of row R in a swizzled tile.
__device__ __forceinline__ int swz(int R, int p) {
  return R * kSB + 8 * (p ^ (R & 7));
}

// One MFMA step over swizzled tiles: lane (r, g) reads piece pc (= 4g + j
// for step j of a super-block, g for a tail block) of its rows.
__device__ __forceinline__ void dma_step(const uint16_t* xt, const uint16_t* wt, int wm, int wn,
                                         int r, int pc, floatx4 (&acc)[4][4]) {
  bf16x8 A[4], Bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    A[i] = *reinterpret_cast<const bf16x8*>(xt + swz(wm + 16 * i + r, pc));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    Bv[j] = *reinterpret_cast<const bf16x8*>(wt + swz(wn + 16 * j + r, pc));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], Bv[j], acc[i][j], 0, 0, 0);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// dma_step with the operand reads issued from inline asm: the compiler
// would otherwise wait for every outstanding DMA before any LDS read (it
// cannot tell the buffers apart), stalling on the next super-block's X.
// The reads complete inside the asm (lgkmcnt(0)). xa / wa: LDS byte
// addresses of this lane's piece in rows wm + r and wn + r; the other rows
// are 16 rows (4096 bytes) apart, at the same slot.
__device__ __forceinline__ void dma_step_asm(uint32_t xa, uint32_t wa, floatx4 (&acc)[4][4]) {
  bf16x8 A0, A1, A2, A3, B0, B1, B2, B3;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:4096\n\t"
      "ds_read_b128 %2, %8 offset:8192\n\t"
      "ds_read_b128 %3, %8 offset:12288\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:4096\n\t"
      "ds_read_b128 %6, %9 offset:8192\n\t"
      "ds_read_b128 %7, %9 offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(A0), "=&v"(A1), "=&v"(A2), "=&v"(A3), "=&v"(B0), "=&v"(B1), "=&v"(B2), "=&v"(B3)
      : "v"(xa), "v"(wa)
      : "memory");
  const bf16x8 A[4] = {A0, A1, A2, A3}, Bv[4] = {B0, B1, B2, B3};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], Bv[j], acc[i][j], 0, 0, 0);
}

template <bool kR4>
struct DmaRaw;
template <>
struct DmaRaw<true> {   // rows v*64 + tid/8, 16 sm bytes + 8 nibble bytes each
  uint4 sm[2];
  uint2 nb[2];
};
template <>
struct DmaRaw<false> {  // rows v*32 + tid/16, 16 bytes each
  uint4 w[4];
};

template <bool kR4>
__device__ __forceinline__ void dma_wload(const GemmArgs& a, int32_t c0, int tid, int64_t n0,
                                          uint32_t wo, uint32_t no, DmaRaw<kR4>& q) {
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  if constexpr (kR4) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const uint8_t* bs = a.w + (n0 + v * 64) * a.k + c0;
      const uint8_t* bn = a.nib + (n0 + v * 64) * (a.k >> 1) + (c0 >> 1);
      q.sm[v] = z4;
      q.nb[v] = make_uint2(0, 0);
      if (n0 + v * 64 + (tid >> 3) < a.n) {
        q.sm[v] = *reinterpret_cast<const uint4*>(bs + wo);
        q.nb[v] = *reinterpret_cast<const uint2*>(bn + no);
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint8_t* base = a.w + ((n0 + v * 32) * a.k + c0) * 2;
      q.w[v] = z4;
      if (n0 + v * 32 + (tid >> 4) < a.n) q.w[v] = *reinterpret_cast<const uint4*>(base + wo);
    }
  }
}

// One super-block of weights as this thread's 4 bf16 operand pieces
// (rebuilt for R4: rows v*64 + tid/8, pieces 2q, 2q+1 of each; twin: rows
// v*32 + tid/16, piece tid % 16).
template <bool kR4>
__device__ __forceinline__ void dma_wbuild(const GemmArgs& a, const Lut& L, int32_t c0, int tid,
                                           int64_t n0, const DmaRaw<kR4>& q,
                                           const EscTab (&tab)[2], int32_t tcol0,
                                           uint4 (&wv)[4]) {
  if constexpr (kR4) {
    const int cc = 16 * (tid & 7);
    uint32_t E[2][4];
    uint32_t esc = 0;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      E[v][0] = lookup4(q.nb[v].x, L);
      E[v][1] = lookup4(q.nb[v].x >> 4, L);
      E[v][2] = lookup4(q.nb[v].y, L);
      E[v][3] = lookup4(q.nb[v].y >> 4, L);
      esc |= (0xEEEEEEEEu - q.nb[v].x) & q.nb[v].x & 0x88888888u;
      esc |= (0xEEEEEEEEu - q.nb[v].y) & q.nb[v].y & 0x88888888u;
    }
    if (esc) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int64_t n = n0 + v * 64 + (tid >> 3);
        esc_patch_word(a, tab[v], n, c0 + cc, c0 + cc - tcol0, q.nb[v].x, E[v][0], E[v][1]);
        esc_patch_word(a, tab[v], n, c0 + cc + 8, c0 + cc + 8 - tcol0, q.nb[v].y, E[v][2],
                       E[v][3]);
      }
    }
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const uint2 p0 = bf16_pairs4(q.sm[v].x, E[v][0]), p1 = bf16_pairs4(q.sm[v].y, E[v][1]);
      const uint2 p2 = bf16_pairs4(q.sm[v].z, E[v][2]), p3 = bf16_pairs4(q.sm[v].w, E[v][3]);
      wv[2 * v] = make_uint4(p0.x, p0.y, p1.x, p1.y);
      wv[2 * v + 1] = make_uint4(p2.x, p2.y, p3.x, p3.y);
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) wv[v] = q.w[v];
  }
}

template <bool kR4>
__device__ __forceinline__ void dma_wstore(int tid, uint16_t* wt, const uint4 (&wv)[4]) {
  if constexpr (kR4) {
    const int qq = tid & 7;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int row = v * 64 + (tid >> 3);
      *reinterpret_cast<uint4*>(wt + swz(row, 2 * qq)) = wv[2 * v];
      *reinterpret_cast<uint4*>(wt + swz(row, 2 * qq + 1)) = wv[2 * v + 1];
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      *reinterpret_cast<uint4*>(wt + swz(v * 32 + (tid >> 4), tid & 15)) = wv[v];
  }
}

template <bool kR4, bool kSplit>
__global__ __launch_bounds__(kDmaThreads, 2) void gemm_dma_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][kDmaBM * kSB];
  __shared__ __attribute__((aligned(16))) uint16_t wt[kBN * kSB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(static_cast<int>(tid >> 6));
  const int64_t tiles_n = (a.n + kBN - 1) / kBN, tiles_m = (a.m + kDmaBM - 1) / kDmaBM;
  const int32_t S = a.slices;
  const int64_t items = tiles_n * tiles_m * (kSplit ? S : 1);
  const int64_t per = (items + kXcds - 1) / kXcds;
  const int64_t item = static_cast<int64_t>(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (item >= items) return;
  const int64_t tile = kSplit ? item / S : item;
  const int32_t s_only = kSplit ? static_cast<int32_t>(item - tile * S) : 0;
  const int64_t n0 = (tile / tiles_m) * kBN;
  const int64_t m0 = (tile % tiles_m) * kDmaBM;
  const int wm = (wave >> 1) * 64;
  const int wn = (wave & 1) * 64;
  uint32_t l0 = a.lut0, l1 = a.lut1, l2 = a.lut2, l3 = a.lut3;
  asm volatile("" : "+v"(l0), "+v"(l1), "+v"(l2), "+v"(l3));
  const Lut L{l0, l1, l2, l3};
  const int r = lane & 15, g = lane >> 4;

  floatx4 acc[4][4], tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[i][j] = acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t nsb = a.k / kSB;
  int32_t s = s_only, u_lo, s_hi;
  slice_superblocks(a.k, S, s, u_lo, s_hi);
  const int32_t u_first = u_lo;
  const int32_t u_end = kSplit ? s_hi : nsb;
  const bool with_tail = !kSplit || s_only == S - 1;

  // X: this wave's 8 DMA pieces per super-block, rows (8 wave + q) * 4 +
  // lane / 16 of the tile (rows past M read row M-1: never stored), each
  // lane loading the piece that belongs at its slot
  const uint8_t* xtile = reinterpret_cast<const uint8_t*>(a.x + m0 * a.ldx);
  const int32_t xrows = static_cast<int32_t>(min(static_cast<int64_t>(kDmaBM), a.m - m0));
  const int32_t ldx2 = static_cast<int32_t>(a.ldx) * 2;
  // byte offset of DMA piece qd of this lane from the super-block's start
  auto xoff = [&](int qd) -> uint32_t {
    const int R = (8 * wave + qd) * 4 + (lane >> 4);
    const int pc = (lane & 15) ^ (R & 7);
    return static_cast<uint32_t>(min(R, xrows - 1) * ldx2 + 16 * pc);
  };
  const uint32_t wo = kR4 ? static_cast<uint32_t>((tid >> 3) * a.k + 16 * (tid & 7))
                          : static_cast<uint32_t>(((tid >> 4) * a.k + 8 * (tid & 15)) * 2);
  const uint32_t no = static_cast<uint32_t>((tid >> 3) * (a.k >> 1) + 8 * (tid & 7));

  EscTab tab[2];
  int32_t tcol0 = u_lo * kSB;
  auto build_tabs = [&](int32_t c0) {
    tcol0 = c0;
    const int32_t c1 = min(a.k, (c0 / kEscRange + 1) * kEscRange);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int64_t n = n0 + v * 64 + (tid >> 3);
      if (n < a.n) {
        esc_tab_build(a, n, c0, c1, tab[v]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) tab[v].ent[i] = 0xFFFFu;
        tab[v].over = 0;
      }
    }
  };

  if (u_lo < u_end) {
    DmaRaw<kR4> q;
    uint4 wv[4];
    dma_wload<kR4>(a, u_lo * kSB, tid, n0, wo, no, q);
#pragma unroll
    for (int qd = 0; qd < 8; ++qd)
      dma16(xtile + u_lo * kSB * 2 + xoff(qd), &xt[0][(8 * wave + qd) * 4 * kSB]);
    if (kR4) build_tabs(u_lo * kSB);
    for (int32_t u = u_lo; u < u_end; ++u) {
      const int b = (u - u_first) & 1;
      if (kR4 && u != u_first && (u * kSB) % kEscRange == 0) build_tabs(u * kSB);
      dma_wait();
      lds_barrier();   // compute of u-1 done everywhere; X(u) in LDS
      if constexpr (kR4) {
        // this super-block's weights, loaded during the previous products
        dma_wbuild<kR4>(a, L, u * kSB, tid, n0, q, tab, tcol0, wv);
        dma_wstore<kR4>(tid, wt, wv);
      } else {
        dma_wstore<kR4>(tid, wt, q.w);
      }
      if (u + 1 < u_end) {
        dma_wload<kR4>(a, (u + 1) * kSB, tid, n0, wo, no, q);
#pragma unroll
        for (int qd = 0; qd < 8; ++qd)
          dma16(xtile + (u + 1) * kSB * 2 + xoff(qd), &xt[b ^ 1][(8 * wave + qd) * 4 * kSB]);
      }
      lds_barrier();   // W(u) in LDS; the loads for u + 1 stay in flight
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma_step_asm(lds_addr(xt[b] + swz(wm + r, 4 * g + j)),
                     lds_addr(wt + swz(wn + r, 4 * g + j)), acc);
      if (!kSplit && u + 1 == s_hi && s + 1 < S) {
        fold<4>(s, acc, tot);
        ++s;
        slice_superblocks(a.k, S, s, u_lo, s_hi);
      }
    }
  }
  if (with_tail) {
    // 32-column tail blocks: plain stores into the same swizzled tiles
    for (int32_t c0 = nsb * kSB; c0 < a.k; c0 += 32) {
      __syncthreads();
      {
        const int row = tid >> 1, p0 = 2 * (tid & 1);
        const int64_t xm = min(m0 + row, a.m - 1);
        const uint4* px = reinterpret_cast<const uint4*>(a.x + xm * a.ldx + c0 + 8 * p0);
        *reinterpret_cast<uint4*>(&xt[0][swz(row, p0)]) = px[0];
        *reinterpret_cast<uint4*>(&xt[0][swz(row, p0 + 1)]) = px[1];
      }
      {
        const int row = tid >> 2, pc = tid & 3;
        const int64_t wn_ = min(n0 + row, a.n - 1);
        const int32_t c = c0 + 8 * pc;
        uint4 v;
        if constexpr (kR4)
          v = rebuild8(a, L, *reinterpret_cast<const uint2*>(a.w + wn_ * a.k + c),
                       *reinterpret_cast<const uint32_t*>(a.nib + wn_ * (a.k >> 1) + (c >> 1)),
                       wn_, c);
        else
          v = *reinterpret_cast<const uint4*>(a.w + 2 * (wn_ * a.k + c));
        *reinterpret_cast<uint4*>(&wt[swz(row, pc)]) = v;
      }
      __syncthreads();
      dma_step(xt[0], wt, wm, wn, r, g, acc);
    }
  }

  if (kSplit && S > 1) {
    float* part = a.part + static_cast<int64_t>(s_only) * a.m * a.n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t on = n0 + wn + 16 * j + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t om = m0 + wm + 16 * i + 4 * g + e;
          if (om < a.m && on < a.n) part[om * a.n + on] = acc[i][j][e];
        }
      }
    return;
  }
  if (!kSplit) fold<4>(s, acc, tot);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t on = n0 + wn + 16 * j + r;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        store_out(a, m0 + wm + 16 * i + 4 * g + e, on, kSplit ? acc[i][j][e] : tot[i][j][e]);
    }
}

// ---------------------------------------------------------------- R4, M <= 128, split
// One block of 4 waves per (group of 64*NT weight rows, slice). Each wave
// streams NT tiles of 16 R4 weight rows through registers in the MFMA
// operand layout of the streamed kernel (lane (r, g): row r of a tile,
// columns 32g .. 32g+31 of a super-block), rebuilt one step at a time while
// the previous step's products run on the matrix cores. The X rows (16*MT
// of them; rows past M repeat row M-1, never stored) go global -> LDS by
// DMA one super-block ahead into two swizzled buffers. LDS carries X only,
// and each X operand read feeds NT products: a super-block costs 4 KiB of
// LDS reads per m-tile per wave, against twice that per weight row in the
// tiled kernel, which also stages the rebuilt weights. The bf16 twin keeps
// the tiled kernel, the faster of the two for plain weights (the same bits
// either way: the order depends on K only).
constexpr int kWregWaves = 4;

// The MT X operands of one step (m-tiles 16 rows = 4096 bytes apart from
// LDS byte address xa), read in one batch that completes inside the asm
// (see dma_step_asm).
template <int MT>
__device__ __forceinline__ void x_read_asm(uint32_t xa, bf16x8 (&A)[MT]) {
  static_assert(MT == 2 || MT == 4 || MT == 8, "m-tiles per block");
  if constexpr (MT == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(A[0]), "=&v"(A[1])
        : "v"(xa)
        : "memory");
  } else if constexpr (MT == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:4096\n\t"
        "ds_read_b128 %2, %4 offset:8192\n\t"
        "ds_read_b128 %3, %4 offset:12288\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(A[0]), "=&v"(A[1]), "=&v"(A[2]), "=&v"(A[3])
        : "v"(xa)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:4096\n\t"
        "ds_read_b128 %2, %8 offset:8192\n\t"
        "ds_read_b128 %3, %8 offset:12288\n\t"
        "ds_read_b128 %4, %8 offset:16384\n\t"
        "ds_read_b128 %5, %8 offset:20480\n\t"
        "ds_read_b128 %6, %8 offset:24576\n\t"
        "ds_read_b128 %7, %8 offset:28672\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(A[0]), "=&v"(A[1]), "=&v"(A[2]), "=&v"(A[3]), "=&v"(A[4]), "=&v"(A[5]),
          "=&v"(A[6]), "=&v"(A[7])
        : "v"(xa)
        : "memory");
  }
}

template <int NT, int MT>
__global__ __launch_bounds__(64 * kWregWaves, 2) void gemm_wreg_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][16 * MT * kSB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(static_cast<int>(tid >> 6));
  constexpr int kRows = 16 * NT * kWregWaves;   // weight rows per block
  const int32_t S = a.slices;
  const int64_t items = ((a.n + kRows - 1) / kRows) * S;
  const int64_t per = (items + kXcds - 1) / kXcds;
  const int64_t item = static_cast<int64_t>(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (item >= items) return;
  const int64_t grp = item / S;
  const int32_t s = static_cast<int32_t>(item - grp * S);
  int32_t u_lo, u_hi;
  slice_superblocks(a.k, S, s, u_lo, u_hi);
  const int32_t nsb = a.k / kSB;
  const int32_t tails = s == S - 1 ? (a.k - nsb * kSB) / 32 : 0;
  uint32_t l0 = a.lut0, l1 = a.lut1, l2 = a.lut2, l3 = a.lut3;
  asm volatile("" : "+v"(l0), "+v"(l1), "+v"(l2), "+v"(l3));
  const Lut L{l0, l1, l2, l3};
  const int r = lane & 15, g = lane >> 4;

  // this lane's weight rows (rows past N read row N-1; never stored)
  int64_t wrow[NT];
  const uint8_t* ps[NT];
  const uint8_t* pn[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    wrow[nt] = min(grp * kRows + (wave * NT + nt) * 16 + r, a.n - 1);
    ps[nt] = a.w + wrow[nt] * a.k;
    pn[nt] = a.nib + wrow[nt] * (a.k >> 1);
  }
  // X: this wave's kDma DMA pieces per super-block, rows (kDma wave + qd) * 4
  // + lane / 16, each lane loading the piece that belongs at its slot
  constexpr int kDma = 4 * MT / kWregWaves;
  static_assert(kDma >= 1 && kDma * kWregWaves == 4 * MT, "X pieces per wave");
  const int32_t xrows = static_cast<int32_t>(min(static_cast<int64_t>(16 * MT), a.m));
  const int32_t ldx2 = static_cast<int32_t>(a.ldx) * 2;
  const uint8_t* xsrc = reinterpret_cast<const uint8_t*>(a.x);
  auto x_dma = [&](int32_t u, int b) {
    const uint8_t* src = xsrc + static_cast<int64_t>(u) * (kSB * 2);
#pragma unroll
    for (int qd = 0; qd < kDma; ++qd) {
      const int R = (kDma * wave + qd) * 4 + (lane >> 4);
      const int pc = (lane & 15) ^ (R & 7);
      dma16(src + (min(R, xrows - 1) * ldx2 + 16 * pc), &xt[b][(kDma * wave + qd) * 4 * kSB]);
    }
  };
  // two sets of weight words, used in turn (the loop is unrolled by two so
  // that no register copy ties the sets together)
  StreamRaw<true> qa[NT], qb[NT];
  auto w_load = [&](int32_t u, StreamRaw<true>(&q)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) stream_load<true>(ps[nt], pn[nt], u * kSB + 32 * g, q[nt]);
  };
  EscTab tab[NT];
  int32_t tcol0 = u_lo * kSB;
  auto build_tabs = [&](int32_t c0) {
    tcol0 = c0;
    const int32_t c1 = min(a.k, (c0 / kEscRange + 1) * kEscRange);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) esc_tab_build(a, wrow[nt], c0, c1, tab[nt]);
  };
  // the weights of step j (columns c + 8j .. c + 8j + 7) of each tile
  auto operands = [&](const StreamRaw<true>(&q)[NT], int32_t c, int j, bf16x8(&Bj)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t S[8] = {q[nt].s0.x, q[nt].s0.y, q[nt].s0.z, q[nt].s0.w,
                             q[nt].s1.x, q[nt].s1.y, q[nt].s1.z, q[nt].s1.w};
      const uint32_t P[4] = {q[nt].nb.x, q[nt].nb.y, q[nt].nb.z, q[nt].nb.w};
      Bj[nt] = as_bf16x8(rebuild8_tab(a, L, make_uint2(S[2 * j], S[2 * j + 1]), P[j], wrow[nt],
                                      c + 8 * j, tab[nt], c + 8 * j - tcol0));
    }
  };

  floatx4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // Super-block u from weight words qc; the next one's loads go to qn. The
  // weights of step j + 1 are rebuilt while the products of step j run.
  auto superblock = [&](int32_t u, const StreamRaw<true>(&qc)[NT], StreamRaw<true>(&qn)[NT]) {
    const int b = (u - u_lo) & 1;
    if (u != u_lo && (u * kSB) % kEscRange == 0) build_tabs(u * kSB);
    dma_wait();      // this wave's X(u) pieces and W(u) words have landed
    lds_barrier();   // every wave's X(u); every wave is done reading X(u-1)
    const int32_t c = u * kSB + 32 * g;
    bf16x8 B0[NT], B1[NT], B2[NT], B3[NT];
    operands(qc, c, 0, B0);
    if (u + 1 < u_hi) {   // the next super-block, in flight during the products
      x_dma(u + 1, b ^ 1);
      w_load(u + 1, qn);
    }
    auto products = [&](int j, const bf16x8(&Bj)[NT]) {
      bf16x8 A[MT];
      x_read_asm<MT>(lds_addr(xt[b] + swz(r, 4 * g + j)), A);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], Bj[nt], acc[t][nt], 0, 0, 0);
    };
    products(0, B0);
    operands(qc, c, 1, B1);
    products(1, B1);
    operands(qc, c, 2, B2);
    products(2, B2);
    operands(qc, c, 3, B3);
    products(3, B3);
  };

  if (u_lo < u_hi) {
    x_dma(u_lo, 0);
    w_load(u_lo, qa);
    build_tabs(u_lo * kSB);
    int32_t u = u_lo;
    for (; u + 1 < u_hi; u += 2) {
      superblock(u, qa, qb);
      superblock(u + 1, qb, qa);
    }
    if (u < u_hi) superblock(u, qa, qb);
  }
  // 32-column tail blocks (last slice): operands straight from memory
  for (int32_t tb = 0; tb < tails; ++tb) {
    const int32_t c0 = nsb * kSB + 32 * tb + 8 * g;
    bf16x8 Bt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      Bt[nt] = as_bf16x8(rebuild8(a, L, *reinterpret_cast<const uint2*>(ps[nt] + c0),
                                  *reinterpret_cast<const uint32_t*>(pn[nt] + (c0 >> 1)),
                                  wrow[nt], c0));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t xm = min(static_cast<int64_t>(16 * t + r), a.m - 1);
      const bf16x8 A = as_bf16x8(*reinterpret_cast<const uint4*>(a.x + xm * a.ldx + c0));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bt[nt], acc[t][nt], 0, 0, 0);
    }
  }

  float* part = a.part + static_cast<int64_t>(s) * a.m * a.n;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t on = grp * kRows + (wave * NT + nt) * 16 + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t om = 16 * t + 4 * g + e;
        if (om < a.m && on < a.n) part[om * a.n + on] = acc[t][nt][e];
      }
    }
}

// y[m][n] = ((p0 + p1) + p2) + ... over the S (<= 8) slice partials, in
// slice order. Block (x, y): row y, columns 1024x .. 1024x+1023, four per
// thread; every slice's load is issued before the adds.
__global__ __launch_bounds__(256) void gemm_combine_kernel(GemmArgs a) {
  constexpr int kMaxSlices = 8;
  const int64_t m = blockIdx.y;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (n0 >= a.n) return;
  const int64_t mn = a.m * a.n;
  const float* p = a.part + m * a.n + n0;
  float v[4];
  if ((a.n & 3) == 0) {
    float4 q[kMaxSlices];
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s)
      if (s < a.slices) q[s] = *reinterpret_cast<const float4*>(p + s * mn);
    v[0] = q[0].x; v[1] = q[0].y; v[2] = q[0].z; v[3] = q[0].w;
#pragma unroll
    for (int s = 1; s < kMaxSlices; ++s)
      if (s < a.slices) {
        v[0] = v[0] + q[s].x; v[1] = v[1] + q[s].y; v[2] = v[2] + q[s].z; v[3] = v[3] + q[s].w;
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = n0 + i < a.n ? p[i] : 0.0f;
    for (int32_t s = 1; s < a.slices; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n0 + i < a.n) v[i] = v[i] + p[s * mn + i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) store_out(a, m, n0 + i, v[i]);
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
  const int64_t nsb = k / kSB;
  int64_t S = s < 8 ? s : 8;
  if (S > nsb) S = nsb;
  return static_cast<int32_t>(S < 1 ? 1 : S);
}

// M up to this runs the small kernel (16*MT X rows per wave, no LDS).
#ifndef BINADE_GEMM_SMALL_MAX_M
#define BINADE_GEMM_SMALL_MAX_M 16
#endif
// The tiled kernel splits the slices over blocks when it has fewer tiles
// than this and M is at most kSplitMaxM (the partials cost 8*S*M*N bytes of
// traffic).
#ifndef BINADE_GEMM_SPLIT_BELOW
#define BINADE_GEMM_SPLIT_BELOW 512
#endif
constexpr int64_t kSmallMaxM = BINADE_GEMM_SMALL_MAX_M;
constexpr int64_t kSplitBelow = BINADE_GEMM_SPLIT_BELOW;
constexpr int64_t kSplitMaxM = 512;

// Tiles for M above 128: 256 X rows (8 waves, one block per CU) or 128
// (4 waves, two blocks per CU).
#ifndef BINADE_GEMM_LARGE_BM
#define BINADE_GEMM_LARGE_BM 256
#endif

// M up to this runs the streamed kernel when the slices' partials have a
// workspace (or K has one slice) and the X slice fits in LDS.
#ifndef BINADE_GEMM_STREAM_MAX_M
#define BINADE_GEMM_STREAM_MAX_M 32
#endif
// weight-row tiles per wave in the streamed kernel
#ifndef BINADE_GEMM_STREAM_TPW
#define BINADE_GEMM_STREAM_TPW 1
#endif
constexpr int64_t kStreamMaxM = BINADE_GEMM_STREAM_MAX_M;
constexpr int64_t kStreamLdsMax = 160 * 1024;

// LDS row stride (bf16 elements) of the streamed kernel's X slice: the
// widest slice plus 8, so that rows start 4 banks apart.
int32_t stream_xstride(int64_t k, int32_t S) {
  const int64_t nsb = k / kSB;
  int64_t w = 0;
  for (int32_t s = 0; s < S; ++s) {
    int64_t c = (((s + 1) * nsb) / S - (s * nsb) / S) * kSB;
    if (s == S - 1) c += k - nsb * kSB;
    w = c > w ? c : w;
  }
  return static_cast<int32_t>(w + 8);
}

struct Plan {
  int smt = 0;       // streamed kernel: X tiles of 16 (0: not streamed)
  int32_t groups = 0;
  int64_t lds = 0;
  int mt = 0;        // small kernel: X tiles of 16 per wave (0: tiled kernel)
  int bm = 0;        // tiled kernel: X rows per tile
  int nj = 0;        // tiled kernel: 16-row MFMA tiles per wave along N
  bool split = false;
  int wreg = 0;      // split with M <= 128: weight-row tiles per wave of the
                     // register-W kernel (0: the tiled kernel)
  int64_t blocks = 0;
  int64_t part_bytes = 0;   // workspace the split needs
};

// The register-W kernel for split shapes with M <= 128 (0: the tiled kernel).
#ifndef BINADE_GEMM_WREG
#define BINADE_GEMM_WREG 1
#endif
constexpr int64_t kWregTwoTilesFrom = 384;

int64_t wreg_blocks(int64_t n, int nt, int32_t S) {
  const int64_t rows = 16 * kWregWaves * nt;   // weight rows per block
  const int64_t items = ((n + rows - 1) / rows) * S;
  return ((items + kXcds - 1) / kXcds) * kXcds;
}

int64_t large_blocks(int64_t m, int64_t n, int bm, int64_t per_tile) {
  const int64_t items = ((n + kBN - 1) / kBN) * ((m + bm - 1) / bm) * per_tile;
  return ((items + kXcds - 1) / kXcds) * kXcds;
}

Plan plan_for(int64_t m, int64_t n, int64_t k, bool r4) {
  Plan p;
  const int32_t S = slices_for(k);
  if (m <= kStreamMaxM && k >= kSB) {
    const int smt = m <= 16 ? 1 : 2;
    const int64_t lds = static_cast<int64_t>(16 * smt) * stream_xstride(k, S) * 2;
    if (lds <= kStreamLdsMax) {
      const int64_t ntiles = (n + 15) / 16;
      const int64_t per = static_cast<int64_t>(kStreamWaves) * BINADE_GEMM_STREAM_TPW;
      p.smt = smt;
      p.lds = lds;
      p.groups = static_cast<int32_t>((ntiles + per - 1) / per);
      p.blocks = static_cast<int64_t>(p.groups) * S;
      p.part_bytes = S > 1 ? static_cast<int64_t>(S) * m * n * 4 : 0;
      return p;
    }
  }
  if (m <= kSmallMaxM) {
    p.mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    const int64_t mtiles = (m + 16 * p.mt - 1) / (16 * p.mt);
    const int64_t tiles = ((n + 15) / 16) * mtiles;
    p.blocks = ((tiles + kXcds - 1) / kXcds) * kXcds;
    return p;
  }
  if (m <= 128) {
    p.bm = 128;
    p.nj = 2;
  } else {
    p.bm = BINADE_GEMM_LARGE_BM;
    p.nj = 4;
  }
  const int64_t tiles = ((n + kBN - 1) / kBN) * ((m + p.bm - 1) / p.bm);
  p.split = S > 1 && tiles < kSplitBelow && m <= kSplitMaxM;
  p.blocks = large_blocks(m, n, p.bm, p.split ? S : 1);
  p.part_bytes = p.split ? static_cast<int64_t>(S) * m * n * 4 : 0;
  if (r4 && p.split && p.bm == 128 && BINADE_GEMM_WREG) {
    // two weight-row tiles per wave when that still gives 1.5 blocks per CU
    p.wreg = ((n + 127) / 128) * S >= kWregTwoTilesFrom ? 2 : 1;
    p.blocks = wreg_blocks(n, p.wreg, S);
  }
  return p;
}

template <bool kR4, int MT>
void launch_small(GemmArgs a, int64_t blocks, hipStream_t stream) {
  a.mtiles = static_cast<int32_t>((a.m + 16 * MT - 1) / (16 * MT));
  a.tiles = ((a.n + 15) / 16) * a.mtiles;
  hipLaunchKernelGGL((gemm_small_kernel<kR4, MT>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * a.slices), 0, stream, a);
}

template <bool kR4, int MT>
void launch_stream(const GemmArgs& a, const Plan& p, hipStream_t stream) {
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_stream_kernel<kR4, MT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(kStreamLdsMax));
  });
  hipLaunchKernelGGL((gemm_stream_kernel<kR4, MT>), dim3(static_cast<uint32_t>(p.blocks)),
                     dim3(64 * kStreamWaves), static_cast<uint32_t>(p.lds), stream, a,
                     static_cast<int32_t>(p.lds / (32 * MT)), p.groups);
}

template <bool kR4, int BM, int NJ>
void launch_large(const GemmArgs& a, bool split, int64_t blocks, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(blocks)), block(large_threads<BM, NJ>());
  if (split)
    hipLaunchKernelGGL((gemm_large_kernel<kR4, BM, NJ, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_large_kernel<kR4, BM, NJ, false>), grid, block, 0, stream, a);
}

// M above 128 runs the DMA-fed tiled kernel (256-row tiles) when its 32-bit
// per-lane X offsets fit (255 rows of ldx elements).
#ifndef BINADE_GEMM_DMA
#define BINADE_GEMM_DMA 1
#endif

template <int NT>
void launch_wreg(const GemmArgs& a, int64_t blocks, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(blocks)), block(64 * kWregWaves);
  if (a.m <= 32)
    hipLaunchKernelGGL((gemm_wreg_kernel<NT, 2>), grid, block, 0, stream, a);
  else if (a.m <= 64)
    hipLaunchKernelGGL((gemm_wreg_kernel<NT, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_wreg_kernel<NT, 8>), grid, block, 0, stream, a);
}

template <bool kR4>
void launch_large_cfg(const GemmArgs& a, const Plan& p, hipStream_t stream) {
  if constexpr (kR4) {
    if (p.wreg != 0) {
      p.wreg == 2 ? launch_wreg<2>(a, p.blocks, stream) : launch_wreg<1>(a, p.blocks, stream);
      return;
    }
  }
  if (p.nj == 2) {
    launch_large<kR4, 128, 2>(a, p.split, p.blocks, stream);
  } else if (BINADE_GEMM_DMA && BINADE_GEMM_LARGE_BM == kDmaBM && a.ldx < (1 << 23)) {
    const dim3 grid(static_cast<uint32_t>(p.blocks)), block(kDmaThreads);
    if (p.split)
      hipLaunchKernelGGL((gemm_dma_kernel<kR4, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_dma_kernel<kR4, false>), grid, block, 0, stream, a);
  } else {
    launch_large<kR4, BINADE_GEMM_LARGE_BM, 4>(a, p.split, p.blocks, stream);
  }
}

int32_t launch(GemmArgs a, bool r4, void* workspace, int64_t workspace_bytes,
               hipStream_t stream) {
  a.slices = slices_for(a.k);
  Plan p = plan_for(a.m, a.n, a.k, r4);
  if (p.blocks > 0x7FFFFFFFll) return BINADE_EUNSUPPORTED;
  if (p.smt != 0) {
    if (p.part_bytes == 0 ||
        (workspace != nullptr && workspace_bytes >= p.part_bytes && aligned16(workspace))) {
      a.part = p.part_bytes ? static_cast<float*>(workspace) : nullptr;
      if (p.smt == 1) r4 ? launch_stream<true, 1>(a, p, stream) : launch_stream<false, 1>(a, p, stream);
      else r4 ? launch_stream<true, 2>(a, p, stream) : launch_stream<false, 2>(a, p, stream);
      if (p.part_bytes) {
        const dim3 cg(static_cast<uint32_t>((a.n + 1023) / 1024), static_cast<uint32_t>(a.m));
        hipLaunchKernelGGL(gemm_combine_kernel, cg, dim3(256), 0, stream, a);
      }
      return launch_status();
    }
    // no room for the partials: the kernels below give the same bits
    p = Plan{};
    p.mt = a.m <= 16 ? 1 : 0;
    if (p.mt) {
      const int64_t tiles = (a.n + 15) / 16;
      p.blocks = ((tiles + kXcds - 1) / kXcds) * kXcds;
    } else {
      p.bm = 128;
      p.nj = 2;
      p.split = false;
      p.blocks = large_blocks(a.m, a.n, p.bm, 1);
    }
  }
  if (p.mt == 1) r4 ? launch_small<true, 1>(a, p.blocks, stream)
                    : launch_small<false, 1>(a, p.blocks, stream);
  else if (p.mt == 2) r4 ? launch_small<true, 2>(a, p.blocks, stream)
                         : launch_small<false, 2>(a, p.blocks, stream);
  else if (p.mt == 4) r4 ? launch_small<true, 4>(a, p.blocks, stream)
                         : launch_small<false, 4>(a, p.blocks, stream);
  if (p.mt != 0) return launch_status();
  // per-lane offsets in the tiled kernel are 32-bit: 64 rows of K bytes or
  // 32 rows of 2*ldx bytes must stay below 2^32
  if (a.k > (1 << 25) || a.ldx > (1 << 25)) return BINADE_EUNSUPPORTED;
  if (p.split && (workspace == nullptr || workspace_bytes < p.part_bytes ||
                  !aligned16(workspace))) {
    // no room for the partials: run every slice in one block (same bits)
    p.split = false;
    p.wreg = 0;
    p.blocks = large_blocks(a.m, a.n, p.bm, 1);
  }
  if (p.wreg != 0 && a.ldx >= (1 << 23)) {   // its DMA offsets are 32-bit
    p.wreg = 0;
    p.blocks = large_blocks(a.m, a.n, p.bm, a.slices);
  }
  a.part = p.split ? static_cast<float*>(workspace) : nullptr;
  r4 ? launch_large_cfg<true>(a, p, stream) : launch_large_cfg<false>(a, p, stream);
  if (p.split) {
    const dim3 cg(static_cast<uint32_t>((a.n + 1023) / 1024), static_cast<uint32_t>(a.m));
    hipLaunchKernelGGL(gemm_combine_kernel, cg, dim3(256), 0, stream, a);
  }
  return launch_status();
}

uint32_t pack4(const uint8_t* l) {
  return uint32_t(l[0]) | (uint32_t(l[1]) << 8) | (uint32_t(l[2]) << 16) |
         (uint32_t(l[3]) << 24);
}

constexpr int64_t kScratchBytes = sizeof(scratch);
constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up once per device with
// that device current. nullptr (and *status set) when HIP reports an error.
void* scratch_address(int32_t* status) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_hip_error(static_cast<int32_t>(e));
    *status = BINADE_EHIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = BINADE_EUNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_last_hip_error(static_cast<int32_t>(e));
      *status = BINADE_EHIP;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

// Argument checks and kernel arguments of the R4 GEMM. *nothing is set when
// the product is empty (M = 0 or N = 0).
int32_t r4_gemm_args(const binade_r4* w, const uint16_t* x, int64_t m,
                     int64_t ldx, void* y, int64_t ldy, int32_t y_dtype,
                     GemmArgs* a, bool* nothing) {
  *nothing = false;
  if (w == nullptr || w->rows < 0 || w->cols <= 0) return BINADE_EINVAL;
  int32_t s = check_xy(x, m, ldx, y, ldy, w->rows, w->cols, y_dtype);
  if (s != BINADE_OK) return s;
  if (m == 0 || w->rows == 0) {
    *nothing = true;
    return BINADE_OK;
  }
  if (w->sm == nullptr || w->nib == nullptr || w->esc_pre == nullptr ||
      (w->n_esc > 0 && w->esc == nullptr))
    return BINADE_EINVAL;
  if (!aligned16(w->sm) || !aligned16(w->nib)) return BINADE_EUNSUPPORTED;
  if (w->n_esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  *a = GemmArgs{};
  a->w = w->sm;
  a->nib = w->nib;
  a->esc_pre = w->esc_pre;
  a->esc = w->esc;
  a->n_esc = static_cast<uint32_t>(w->n_esc);
  a->lut0 = rot_exponents4(pack4(w->lut));
  a->lut1 = rot_exponents4(pack4(w->lut + 4));
  a->lut2 = rot_exponents4(pack4(w->lut + 8));
  a->lut3 = rot_exponents4(pack4(w->lut + 12));
  a->x = x;
  a->y = y;
  a->m = m;
  a->n = w->rows;
  a->k = static_cast<int32_t>(w->cols);
  a->ldx = ldx;
  a->ldy = ldy;
  a->y_bf16 = y_dtype == BINADE_BF16;
  return BINADE_OK;
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int64_t binade_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 32 != 0 || k > (1 << 30)) return 0;
  return plan_for(m, n, k, true).part_bytes;   // the same for the twin
}

extern "C" int32_t binade_r4_gemm(const binade_r4* w, const uint16_t* x,
                                  int64_t m, int64_t ldx, void* y, int64_t ldy,
                                  int32_t y_dtype, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  GemmArgs a{};
  bool nothing = false;
  int32_t s = r4_gemm_args(w, x, m, ldx, y, ldy, y_dtype, &a, &nothing);
  if (s != BINADE_OK || nothing) return s;
  return launch(a, true, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" int64_t binade_gemm_scratch_bytes(void) { return kScratchBytes; }

extern "C" int32_t binade_r4_gemm_noalloc(const binade_r4* w, const uint16_t* x,
                                          int64_t m, int64_t ldx, void* y,
                                          int64_t ldy, int32_t y_dtype,
                                          void* stream) {
  GemmArgs a{};
  bool nothing = false;
  int32_t s = r4_gemm_args(w, x, m, ldx, y, ldy, y_dtype, &a, &nothing);
  if (s != BINADE_OK || nothing) return s;
  const int64_t need = plan_for(a.m, a.n, a.k, true).part_bytes;
  if (need > kScratchBytes) return BINADE_ENOSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address(&s);
    if (ws == nullptr) return s;
  }
  return launch(a, true, ws, need, static_cast<hipStream_t>(stream));
}

extern "C" int32_t binade_bf16_gemm(const uint16_t* w, int64_t rows,
                                    int64_t cols, const uint16_t* x, int64_t m,
                                    int64_t ldx, void* y, int64_t ldy,
                                    int32_t y_dtype, void* workspace,
                                    int64_t workspace_bytes, void* stream) {
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
  return launch(a, false, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}
