// MoE epilogue: the gate.up activation between a MoE layer's expert
// products, and the top-k weighted combine after the down product.
//
// "Binade" package page (pypi.org/project/binade), "How it works" and
// "Limitations": a MoE layer's expert products (gate and up per chosen
// expert, then down) run as gathered matvecs; their outputs meet in an
// activation and, per token, in a sum over the chosen experts weighted by
// the router. Both steps are elementwise and HBM-bound; each thread owns
// outputs whose arithmetic is stated in binade.h:
//  - silu_mul: h = silu(g) * u with silu(g) = g / (1 + exp(-g)), in fp64 from
//    the fp32 inputs, rounded once to fp32 (then to bf16);
//  - combine: out[t, j] = fma chain over the token's top_k slots in slot
//    order from +0.0, in fp32 (then bf16).
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

__global__ __launch_bounds__(256) void silu_mul_kernel(const float* gate, const float* up,
                                                       int64_t n, void* h, int32_t h_bf16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const double g = gate[i];
    const double s = g / (1.0 + exp(-g));
    const float v = static_cast<float>(s * static_cast<double>(up[i]));
    if (h_bf16)
      static_cast<uint16_t*>(h)[i] = to_bf16_rne(v);
    else
      static_cast<float*>(h)[i] = v;
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const float* y, const float* weights,
                                                      int64_t n_tokens, int32_t top_k, int64_t n,
                                                      void* out, int32_t out_bf16) {
  const int64_t total = n_tokens * n;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    const int64_t t = i / n, j = i - t * n;
    const float* wt = weights + t * top_k;
    const float* yt = y + t * top_k * n + j;
    float acc = 0.0f;
    for (int32_t s = 0; s < top_k; ++s) acc = __builtin_fmaf(wt[s], yt[s * n], acc);
    if (out_bf16)
      static_cast<uint16_t*>(out)[i] = to_bf16_rne(acc);
    else
      static_cast<float*>(out)[i] = acc;
  }
}

uint32_t elementwise_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<uint32_t>(b < 8192 ? b : 8192);
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int32_t binade_moe_silu_mul(const float* gate, const float* up, int64_t n, void* h,
                                       int32_t h_dtype, void* stream) {
  if (n < 0 || (h_dtype != BINADE_F32 && h_dtype != BINADE_BF16)) return BINADE_EINVAL;
  if (n == 0) return BINADE_OK;
  if (gate == nullptr || up == nullptr || h == nullptr) return BINADE_EINVAL;
  hipLaunchKernelGGL(silu_mul_kernel, dim3(elementwise_blocks(n)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), gate, up, n, h,
                     static_cast<int32_t>(h_dtype == BINADE_BF16));
  return launch_status();
}

extern "C" int32_t binade_moe_combine(const float* y, const float* weights, int64_t n_tokens,
                                      int32_t top_k, int64_t n, void* out, int32_t out_dtype,
                                      void* stream) {
  if (n_tokens < 0 || n < 0 || top_k < 1 || top_k > 64) return BINADE_EINVAL;
  if (out_dtype != BINADE_F32 && out_dtype != BINADE_BF16) return BINADE_EINVAL;
  if (n_tokens == 0 || n == 0) return BINADE_OK;
  if (y == nullptr || weights == nullptr || out == nullptr) return BINADE_EINVAL;
  hipLaunchKernelGGL(combine_kernel, dim3(elementwise_blocks(n_tokens * n)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), y, weights, n_tokens, top_k, n, out,
                     static_cast<int32_t>(out_dtype == BINADE_BF16));
  return launch_status();
}
