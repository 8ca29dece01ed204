// MoE expert-gather GEMV on R4 experts and its bf16-expert twin.
//
// "Binade" package page (pypi.org/project/binade), "How it works": the MoE
// expert gather adds its products in the matvec's order; "Limitations": the
// fused kernels cover every expert product. Each (token, slot) pair p has an
// expert idx[p]; its output row is that expert's matvec of the pair's input,
// with exactly the binade_r4_gemv order.
//
// Mapping: block (g, e) covers rows 4g..4g+3 of expert e, one wave per row.
// A wave first finds, with one ballot per 64 pairs, every pair that chose
// expert e (an expert nobody chose costs one idx read and exits), then walks
// the row's chunks once per group of up to 4 such pairs: the 32 weights of
// its lane tile are rebuilt in registers once and multiplied against each
// pair's x tile. So an expert chosen by several pairs is read from HBM once.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

constexpr int kPairsPerPass = 4;

struct MoeArgs {
  const uint8_t* w;        // R4 sm plane, or bf16 experts (twin)
  const uint8_t* nib;
  const uint32_t* esc_pre;
  const uint32_t* esc;
  const uint16_t* x;
  const int32_t* idx;
  void* y;
  uint32_t* status;
  int64_t n_rows;          // rows per expert
  int32_t cols;
  int32_t n_experts;
  int32_t n_pairs;
  int32_t top_k;
  int32_t x_per_slot;
  int32_t y_bf16;
  uint32_t n_esc;
  uint32_t lut0, lut1, lut2, lut3;
};

template <bool kR4>
__device__ __forceinline__ void tile_weights(const MoeArgs& a, int64_t grow,
                                             int64_t chunk, int t, bool active,
                                             int lane, float (&w)[32]) {
  if (kR4) {
    uint4 s0 = make_uint4(0, 0, 0, 0), s1 = s0, nb = s0;
    if (active) {
      const uint4* ps = reinterpret_cast<const uint4*>(a.w + grow * a.cols + 32 * t);
      s0 = ps[0];
      s1 = ps[1];
      nb = *reinterpret_cast<const uint4*>(a.nib + grow * (a.cols >> 1) + 16 * t);
    }
    const Lut L{a.lut0, a.lut1, a.lut2, a.lut3};
    uint32_t E[8];
    tile_exponents(nb, L, a.esc_pre, a.esc, a.n_esc, chunk, lane, E);
    const uint32_t S[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t H, Lo;
      split4(S[d], E[d], H, Lo);
      w[4 * d] = weight_f32<0>(H, Lo);
      w[4 * d + 1] = weight_f32<1>(H, Lo);
      w[4 * d + 2] = weight_f32<2>(H, Lo);
      w[4 * d + 3] = weight_f32<3>(H, Lo);
    }
  } else {
    if (active) {
      const uint4* p = reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint16_t*>(a.w) + grow * a.cols + 32 * t);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 d = p[v];
        const uint32_t q[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[8 * v + 2 * e] = bf16_lo(q[e]);
          w[8 * v + 2 * e + 1] = bf16_hi(q[e]);
        }
      }
    }
  }
}

__device__ __forceinline__ void store_out(const MoeArgs& a, int64_t i, float v) {
  if (a.y_bf16)
    static_cast<uint16_t*>(a.y)[i] = to_bf16_rne(v);
  else
    static_cast<float*>(a.y)[i] = v;
}

template <bool kR4>
__global__ __launch_bounds__(256) void moe_gemv_kernel(MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const int32_t e = static_cast<int32_t>(blockIdx.y);
  const int64_t row = uniform64(static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  if (row >= a.n_rows) return;
  const int J = a.cols >> 5;
  const int C = (J + 63) >> 6;
  const int64_t grow = static_cast<int64_t>(e) * a.n_rows + row;

  for (int32_t base = 0; base < a.n_pairs; base += 64) {
    const int32_t p = base + lane;
    const int32_t v = p < a.n_pairs ? a.idx[p] : 0;
    uint64_t mine = __ballot(p < a.n_pairs && v == e);
    const uint64_t badm = __ballot(p < a.n_pairs && (v < 0 || v >= a.n_experts));
    if (badm != 0 && e == 0) {
      // out-of-range indices: flag once per row and zero those output rows
      if (lane == 0 && row == 0 && a.status != nullptr)
        atomicOr(a.status, static_cast<uint32_t>(BINADE_DEV_BAD_INDEX));
      if (((badm >> lane) & 1u) != 0) store_out(a, static_cast<int64_t>(p) * a.n_rows + row, 0.0f);
    }
    while (mine != 0) {
      // next group of up to 4 pairs, in increasing pair order
      int32_t pp[kPairsPerPass];
      int np = 0;
#pragma unroll
      for (int g = 0; g < kPairsPerPass; ++g) {
        pp[g] = -1;
        if (mine != 0) {
          const int b = __builtin_ctzll(mine);
          mine &= mine - 1;
          pp[g] = base + b;
          ++np;
        }
      }
      float a0[kPairsPerPass], a1[kPairsPerPass];
#pragma unroll
      for (int g = 0; g < kPairsPerPass; ++g) a0[g] = a1[g] = 0.0f;
      for (int j = 0; j < C; ++j) {
        const int t = j * 64 + lane;
        const bool active = t < J;
        float w[32];
        tile_weights<kR4>(a, grow, grow * C + j, t, active, lane, w);
        if (!active) continue;
#pragma unroll
        for (int g = 0; g < kPairsPerPass; ++g) {
          if (g >= np) break;
          const int64_t xrow = a.x_per_slot ? pp[g] : pp[g] / a.top_k;
          float xf[32];
          load_x_tile(a.x + xrow * a.cols, t, xf);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            a0[g] = __builtin_fmaf(w[2 * i], xf[2 * i], a0[g]);
            a1[g] = __builtin_fmaf(w[2 * i + 1], xf[2 * i + 1], a1[g]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < kPairsPerPass; ++g) {
        if (g >= np) break;
        const float r = slot_tree(a0[g] + a1[g]);
        if (lane == 0) store_out(a, static_cast<int64_t>(pp[g]) * a.n_rows + row, r);
      }
    }
  }
}

int32_t launch(const MoeArgs& a, bool r4, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((a.n_rows + 3) / 4),
                  static_cast<uint32_t>(a.n_experts));
  if (r4)
    hipLaunchKernelGGL(moe_gemv_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(moe_gemv_kernel<false>, grid, dim3(256), 0, stream, a);
  return launch_status();
}

int32_t check_common(int32_t n_experts, int64_t rows, int64_t cols,
                     const uint16_t* x, const int32_t* idx, int64_t n_tokens,
                     int32_t top_k, void* y, int32_t y_dtype) {
  if (n_experts <= 0 || rows < 0 || cols <= 0 || n_tokens < 0 || top_k <= 0)
    return BINADE_EINVAL;
  if (rows % n_experts != 0) return BINADE_EINVAL;
  if (cols % 32 != 0 || cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (y_dtype != BINADE_F32 && y_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (n_experts > 65535 || n_tokens * top_k > (1ll << 30)) return BINADE_EUNSUPPORTED;
  if (rows == 0 || n_tokens == 0) return BINADE_OK;
  if (x == nullptr || idx == nullptr || y == nullptr) return BINADE_EINVAL;
  if (!aligned16(x)) return BINADE_EUNSUPPORTED;
  return BINADE_OK;
}

uint32_t pack4(const uint8_t* l) {
  return uint32_t(l[0]) | (uint32_t(l[1]) << 8) | (uint32_t(l[2]) << 16) |
         (uint32_t(l[3]) << 24);
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int32_t binade_r4_moe_gemv(const binade_r4* w, int32_t n_experts,
                                      const uint16_t* x, int32_t x_per_slot,
                                      const int32_t* idx, int64_t n_tokens,
                                      int32_t top_k, void* y, int32_t y_dtype,
                                      uint32_t* dev_status, void* stream) {
  if (w == nullptr) return BINADE_EINVAL;
  int32_t s = check_common(n_experts, w->rows, w->cols, x, idx, n_tokens, top_k,
                           y, y_dtype);
  if (s != BINADE_OK || w->rows == 0 || n_tokens == 0) return s;
  if (w->sm == nullptr || w->nib == nullptr || w->esc_pre == nullptr ||
      (w->n_esc > 0 && w->esc == nullptr))
    return BINADE_EINVAL;
  if (!aligned16(w->sm) || !aligned16(w->nib)) return BINADE_EUNSUPPORTED;
  if (w->n_esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  MoeArgs a{};
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
  a.idx = idx;
  a.y = y;
  a.status = dev_status;
  a.n_rows = w->rows / n_experts;
  a.cols = static_cast<int32_t>(w->cols);
  a.n_experts = n_experts;
  a.n_pairs = static_cast<int32_t>(n_tokens * top_k);
  a.top_k = top_k;
  a.x_per_slot = x_per_slot != 0;
  a.y_bf16 = y_dtype == BINADE_BF16;
  return launch(a, true, static_cast<hipStream_t>(stream));
}

extern "C" int32_t binade_bf16_moe_gemv(const uint16_t* w, int32_t n_experts,
                                        int64_t rows_per_expert, int64_t cols,
                                        const uint16_t* x, int32_t x_per_slot,
                                        const int32_t* idx, int64_t n_tokens,
                                        int32_t top_k, void* y, int32_t y_dtype,
                                        uint32_t* dev_status, void* stream) {
  if (rows_per_expert < 0 || n_experts <= 0) return BINADE_EINVAL;
  int32_t s = check_common(n_experts, rows_per_expert * n_experts, cols, x, idx,
                           n_tokens, top_k, y, y_dtype);
  if (s != BINADE_OK || rows_per_expert == 0 || n_tokens == 0) return s;
  if (w == nullptr) return BINADE_EINVAL;
  if (!aligned16(w)) return BINADE_EUNSUPPORTED;
  MoeArgs a{};
  a.w = reinterpret_cast<const uint8_t*>(w);
  a.x = x;
  a.idx = idx;
  a.y = y;
  a.status = dev_status;
  a.n_rows = rows_per_expert;
  a.cols = static_cast<int32_t>(cols);
  a.n_experts = n_experts;
  a.n_pairs = static_cast<int32_t>(n_tokens * top_k);
  a.top_k = top_k;
  a.x_per_slot = x_per_slot != 0;
  a.y_bf16 = y_dtype == BINADE_BF16;
  return launch(a, false, static_cast<hipStream_t>(stream));
}
