// Prompt GEMM Y[M,N] = X[M,K] W[N,K]^T with R4 weights decoded into LDS and
// multiplied on gfx950 bf16 MFMA, and its bf16-weight twin.
//
// "Binade" package page (pypi.org/project/binade), "Results": prompt
// processing runs the 12B model's matmuls with a fused GEMM; "Limitations":
// on long prompts the fused GEMM is weighed against rebuilding BF16 weights;
// "NVIDIA GPUs": a GEMM's order is a chain of matrix-core steps along K.
//
// Order (shared by both kernels, independent of tiling): every output has one
// fp32 accumulator starting at +0.0; K is taken in blocks of 32 in increasing
// order, and each block is one v_mfma_f32_16x16x32_bf16 step on it. There is
// no split-K. The R4 kernel rebuilds exactly the bf16 weights the twin reads,
// so both issue identical MFMA sequences.
//
// Tiling: a 256-thread block owns a 64x64 output tile; each wave a 32x32
// quarter (2x2 MFMA tiles). Per K block the block stages X[64,32] and the
// rebuilt W[64,32] in LDS (row stride padded to 80 bytes), then every lane
// reads its 8 consecutive K values of one row as a 16-byte LDS load for the
// A (X) and B (W) operands.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64, kBN = 64, kBK = 32;
constexpr int kLdsStride = kBK + 8;  // in bf16 elements

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
  uint32_t lut0, lut1, lut2, lut3;
};

// First side-list index in [lo, hi) whose in-chunk position is >= pos
// (entries of one chunk are sorted by position).
__device__ __forceinline__ uint32_t esc_lower_bound(const uint32_t* esc,
                                                    uint32_t lo, uint32_t hi,
                                                    uint32_t pos) {
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if ((esc[mid] & 0xFFFFu) < pos)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Rebuild 8 weights of row n, columns c0 .. c0+7 (c0 % 8 == 0), as 4 dwords
// of bf16 pairs.
__device__ __forceinline__ uint4 r4_rebuild8(const GemmArgs& a, int64_t n,
                                             int32_t c0) {
  const uint2 s = *reinterpret_cast<const uint2*>(a.w + n * a.k + c0);
  const uint32_t P = *reinterpret_cast<const uint32_t*>(a.nib + n * (a.k >> 1) + (c0 >> 1));
  const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};
  uint32_t E0 = lookup4(P, L);
  uint32_t E1 = lookup4(P >> 4, L);
  const int32_t C = (a.k + kChunk - 1) / kChunk;
  const int32_t j = c0 / kChunk;
  const int64_t chunk = n * C + j;
  uint32_t hi = a.esc_pre[chunk + 1];
  uint32_t lo = a.esc_pre[chunk];
  hi = hi < a.n_esc ? hi : a.n_esc;
  lo = lo < hi ? lo : hi;
  if (lo < hi) {
    const uint32_t pos0 = static_cast<uint32_t>(c0 - j * kChunk);
    for (uint32_t e = esc_lower_bound(a.esc, lo, hi, pos0); e < hi; ++e) {
      const uint32_t ent = a.esc[e];
      const uint32_t d = (ent & 0xFFFFu) - pos0;
      if (d >= 8u) break;
      const uint32_t sh = (d & 3u) * 8u;
      const uint32_t ex = ((ent >> 16) & 0xFFu) << sh;
      if (d < 4u)
        E0 = (E0 & ~(0xFFu << sh)) | ex;
      else
        E1 = (E1 & ~(0xFFu << sh)) | ex;
    }
  }
  uint32_t H0, L0, H1, L1;
  split4(s.x, E0, H0, L0);
  split4(s.y, E1, H1, L1);
  return make_uint4(weight_pair_bf16<0>(H0, L0), weight_pair_bf16<2>(H0, L0),
                    weight_pair_bf16<0>(H1, L1), weight_pair_bf16<2>(H1, L1));
}

template <bool kR4>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kBM][kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t ws[kBN][kLdsStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
  const int wm = (wave >> 1) * 32;
  const int wn = (wave & 1) * 32;
  const int sr = tid >> 2;          // staging row 0..63
  const int sq = (tid & 3) * 8;     // staging column 0, 8, 16, 24

  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) acc[i][jn] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int KB = a.k / kBK;
  for (int kb = 0; kb < KB; ++kb) {
    const int32_t c0 = kb * kBK + sq;
    {
      const int64_t m = m0 + sr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < a.m) v = *reinterpret_cast<const uint4*>(a.x + m * a.ldx + c0);
      *reinterpret_cast<uint4*>(&xs[sr][sq]) = v;
    }
    {
      const int64_t n = n0 + sr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < a.n) {
        if (kR4)
          v = r4_rebuild8(a, n, c0);
        else
          v = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(a.w) + n * a.k + c0);
      }
      *reinterpret_cast<uint4*>(&ws[sr][sq]) = v;
    }
    __syncthreads();
    bf16x8 A[2], Bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      A[i] = *reinterpret_cast<const bf16x8*>(&xs[wm + 16 * i + (lane & 15)][8 * (lane >> 4)]);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
      Bv[jn] = *reinterpret_cast<const bf16x8*>(&ws[wn + 16 * jn + (lane & 15)][8 * (lane >> 4)]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], Bv[jn], acc[i][jn], 0, 0, 0);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int64_t n = n0 + wn + 16 * jn + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
        if (m < a.m && n < a.n) {
          const float v = acc[i][jn][r];
          if (a.y_bf16)
            static_cast<uint16_t*>(a.y)[m * a.ldy + n] = to_bf16_rne(v);
          else
            static_cast<float*>(a.y)[m * a.ldy + n] = v;
        }
      }
    }
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
  if (m > 65535ll * kBM || n > 0x7FFFFFFFll) return BINADE_EUNSUPPORTED;
  return BINADE_OK;
}

int32_t launch(const GemmArgs& a, bool r4, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((a.n + kBN - 1) / kBN),
                  static_cast<uint32_t>((a.m + kBM - 1) / kBM));
  if (r4)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(256), 0, stream, a);
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
  a.lut0 = pack4(w->lut);
  a.lut1 = pack4(w->lut + 4);
  a.lut2 = pack4(w->lut + 8);
  a.lut3 = pack4(w->lut + 12);
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
