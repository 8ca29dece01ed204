// Format 2 (Rice-coded ranks) -> R4 runtime layout, on the GPU at load.
//
// "Binade" package page (pypi.org/project/binade), intro and "How it works":
// the file stores ranks in Rice codes (~10.75 bits per weight); at load a
// GPU kernel turns them into R4, every rank in 4 bits with rare escapes.
// "Lossless BF16 weight compression" page, "Best measured configuration":
// a decoder with per-block lengths found by a warp prefix sum and its output
// staged on chip is what made the Huffman exponent decoder fast; the same
// two ideas are used here, with the lengths found from the bits themselves.
//
// One wave decodes one row-chunk (<= 2048 weights). Phase 1: the lanes
// popcount the chunk's unary words (every weight's code ends in exactly one
// 1 bit), a wave prefix sum turns the counts into weight indices, and the
// lane holding the terminator of weight 32m-1 records where lane tile m
// starts. Phase 2: lane l decodes its 32 weights serially from that bit,
// adds the k remainder bits, clamps ranks to 4 bits and writes its 16 nibble
// bytes with one 16-byte store (so the chunk's output is one contiguous,
// coalesced 1 KiB). Escapes (rank >= 15) wait in LDS until a second prefix
// sum gives their place in the side list.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

constexpr int kWavesPerBlock = 4;

struct RiceArgs {
  const uint32_t* unary;
  const uint32_t* rem;
  const uint64_t* anchor;
  const uint32_t* esc_pre;
  uint8_t* nib;
  uint32_t* esc;
  uint32_t* status;
  uint64_t unary_words;
  uint64_t rem_words;
  uint64_t n_esc;
  int64_t rows;
  int64_t n_chunks;
  int32_t cols;
  uint32_t k;
  uint32_t n;
  uint32_t table[64];  // exp_of_rank, 4 bytes per word
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Bit position of the n-th (0-based) set bit of v; v has more than n set.
__device__ __forceinline__ uint32_t select_bit(uint32_t v, uint32_t n) {
  uint32_t pos = 0;
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
    const uint32_t c = __popc(v & ((1u << w) - 1u));
    if (n >= c) {
      n -= c;
      v >>= w;
      pos += w;
    }
  }
  return pos;
}

__device__ __forceinline__ uint32_t load_word(const uint32_t* p, uint64_t i,
                                              uint64_t cap) {
  return i < cap ? p[i] : 0u;
}

__device__ __forceinline__ void flag(uint32_t* status, uint32_t bits,
                                     int lane) {
  if (status != nullptr && lane == 0) atomicOr(status, bits);
}

__global__ __launch_bounds__(256) void rice_to_r4_kernel(RiceArgs a) {
  __shared__ uint64_t tile_start[kWavesPerBlock][64];
  __shared__ uint32_t esc_tmp[kWavesPerBlock][32][64];
  __shared__ uint32_t expo_w[64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < 64) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 64; ++q)
      if (static_cast<int>(threadIdx.x) == q) v = a.table[q];
    expo_w[threadIdx.x] = v;
  }
  __syncthreads();
  const uint8_t* expo = reinterpret_cast<const uint8_t*>(expo_w);

  const int64_t c = uniform64(static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave);
  if (c >= a.n_chunks) return;
  const int64_t C = (a.cols + kChunk - 1) / kChunk;
  const int64_t row = c / C;
  const int32_t j = static_cast<int32_t>(c - row * C);
  const int32_t Lc = min(kChunk, a.cols - j * kChunk);
  const int32_t T = Lc >> 5;
  const uint64_t A = a.anchor[c];
  const uint64_t B = a.anchor[c + 1];
  const uint64_t fb = static_cast<uint64_t>(row) * a.cols + static_cast<uint64_t>(j) * kChunk;

  if (B < A + static_cast<uint64_t>(Lc) || B - A > 256ull * Lc ||
      B > a.unary_words * 32ull) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }

  // ---- phase 1: where does each lane tile start?
  const uint64_t wA = A >> 5;
  const uint64_t nw = ((B - 1) >> 5) - wA + 1;
  if (lane == 0) tile_start[wave][0] = A;
  uint32_t carry = 0;
  bool last_bit_set = false;
  for (uint64_t base = 0; base < nw; base += 64) {
    const uint64_t wi = base + lane;
    uint32_t word = 0;
    if (wi < nw) {
      word = load_word(a.unary, wA + wi, a.unary_words);
      if (wi == 0) word &= 0xFFFFFFFFu << (A & 31u);
      if (wi == nw - 1) {
        const uint32_t top = static_cast<uint32_t>((B - 1) & 31u);
        word &= 0xFFFFFFFFu >> (31u - top);
        last_bit_set = (word >> top) & 1u;
      }
    }
    const uint32_t pc = __popc(word);
    const uint32_t incl = wave_inclusive_sum(pc, lane);
    const uint32_t s_first = carry + incl - pc;
    const uint32_t s = s_first | 31u;  // next weight index ending a lane tile
    if (pc > 0 && s < s_first + pc) {
      const uint32_t m = (s + 1) >> 5;
      if (static_cast<int32_t>(m) < T)
        tile_start[wave][m] = (wA + wi) * 32ull + select_bit(word, s - s_first) + 1;
    }
    carry += __shfl(incl, 63, 64);
  }
  const bool ends_in_one = __any(last_bit_set);
  if (carry != static_cast<uint32_t>(Lc) || !ends_in_one) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  wave_sync();

  // ---- phase 2: lane l decodes weights 32l .. 32l+31 of the chunk
  uint32_t out[4] = {0, 0, 0, 0};
  uint32_t n_esc_lane = 0;
  bool bad = false;
  if (lane < T) {
    const uint64_t pos = tile_start[wave][lane];
    uint64_t wnext = (pos >> 5) + 2;
    const uint32_t off = static_cast<uint32_t>(pos & 31u);
    uint64_t buf = (static_cast<uint64_t>(load_word(a.unary, wnext - 1, a.unary_words)) << 32 |
                    load_word(a.unary, wnext - 2, a.unary_words)) >> off;
    uint32_t have = 64u - off;

    const uint32_t k = a.k;
    const uint32_t kmask = (1u << k) - 1u;
    uint64_t rbuf = 0;
    uint32_t rhave = 0;
    uint64_t rnext = 0;
    if (k > 0) {
      rnext = ((fb + 32ull * lane) * k) >> 5;  // word aligned: 32 | (fb + 32 l)
      rbuf = static_cast<uint64_t>(load_word(a.rem, rnext + 1, a.rem_words)) << 32 |
             load_word(a.rem, rnext, a.rem_words);
      rnext += 2;
      rhave = 64;
    }

#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t q = 0;
      while (buf == 0) {  // the code runs past the valid bits
        q += have;
        if (q > 255u) break;
        buf = static_cast<uint64_t>(load_word(a.unary, wnext + 1, a.unary_words)) << 32 |
              load_word(a.unary, wnext, a.unary_words);
        wnext += 2;
        have = 64;
      }
      if (q > 255u) {
        bad = true;
        break;
      }
      const uint32_t t = static_cast<uint32_t>(__builtin_ctzll(buf));
      q += t;
      const uint32_t sh = t + 1;
      buf = sh >= 64 ? 0ull : (buf >> sh);
      have -= sh;
      if (have < 32) {
        buf |= static_cast<uint64_t>(load_word(a.unary, wnext, a.unary_words)) << have;
        ++wnext;
        have += 32;
      }
      uint32_t remv = 0;
      if (k > 0) {
        remv = static_cast<uint32_t>(rbuf) & kmask;
        rbuf >>= k;
        rhave -= k;
        if (rhave < 32) {
          rbuf |= static_cast<uint64_t>(load_word(a.rem, rnext, a.rem_words)) << rhave;
          ++rnext;
          rhave += 32;
        }
      }
      const uint32_t r = (q << k) | remv;
      if (r >= a.n) {
        bad = true;
        break;
      }
      const uint32_t v = r < 15u ? r : 15u;
      out[i >> 3] |= v << (8 * ((i & 7) & 3) + 4 * ((i & 7) >> 2));
      if (r >= 15u) {
        esc_tmp[wave][n_esc_lane][lane] =
            (static_cast<uint32_t>(expo[r]) << 16) | static_cast<uint32_t>(32 * lane + i);
        ++n_esc_lane;
      }
    }
  }
  if (__any(bad)) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }

  // ---- escapes: place in the side list after a prefix sum over lanes
  const uint32_t incl = wave_inclusive_sum(n_esc_lane, lane);
  const uint32_t total = __shfl(incl, 63, 64);
  const uint32_t e0 = a.esc_pre[c];
  const uint32_t e1 = a.esc_pre[c + 1];
  if (e1 < e0 || e1 - e0 != total || e1 > a.n_esc) {
    flag(a.status, BINADE_DEV_CORRUPT_ESC, lane);
  } else {
    const uint32_t base = e0 + incl - n_esc_lane;
    for (uint32_t i = 0; i < n_esc_lane; ++i) a.esc[base + i] = esc_tmp[wave][i][lane];
  }
  if (lane < T) {
    uint4* dst = reinterpret_cast<uint4*>(a.nib + static_cast<uint64_t>(row) * (a.cols >> 1) +
                                          static_cast<uint64_t>(j) * (kChunk / 2) + 16u * lane);
    *dst = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int32_t binade_rice_to_r4(const binade_rice* in, binade_r4* out,
                                     uint32_t* dev_status, void* stream) {
  if (in == nullptr || out == nullptr || in->rows <= 0 || in->cols <= 0 ||
      in->n == 0 || in->n > 256 || in->k > 7)
    return BINADE_EINVAL;
  if (in->cols % 32 != 0 || in->cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (in->sm == nullptr || in->unary == nullptr || in->anchor == nullptr ||
      in->esc_pre == nullptr || (in->k > 0 && in->rem == nullptr) ||
      out->nib == nullptr || (in->n_esc > 0 && out->esc == nullptr))
    return BINADE_EINVAL;
  if (!aligned16(in->sm) || !aligned16(out->nib) ||
      (reinterpret_cast<uintptr_t>(in->unary) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(in->rem) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(in->anchor) & 7u) != 0)
    return BINADE_EUNSUPPORTED;
  if (in->n_esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  const int64_t C = (in->cols + BINADE_CHUNK - 1) / BINADE_CHUNK;
  const int64_t n_chunks = in->rows * C;

  out->rows = in->rows;
  out->cols = in->cols;
  out->sm = in->sm;
  out->esc_pre = in->esc_pre;
  out->n_esc = in->n_esc;
  for (int r = 0; r < 16; ++r)
    out->lut[r] = (r < 15 && static_cast<uint32_t>(r) < in->n) ? in->exp_of_rank[r] : 0;

  RiceArgs a{};
  a.unary = in->unary;
  a.rem = in->rem;
  a.anchor = in->anchor;
  a.esc_pre = in->esc_pre;
  a.nib = out->nib;
  a.esc = out->esc;
  a.status = dev_status;
  a.unary_words = in->unary_words;
  a.rem_words = in->k > 0 ? in->rem_words : 0;
  a.n_esc = in->n_esc;
  a.rows = in->rows;
  a.n_chunks = n_chunks;
  a.cols = static_cast<int32_t>(in->cols);
  a.k = in->k;
  a.n = in->n;
  for (int q = 0; q < 64; ++q)
    a.table[q] = uint32_t(in->exp_of_rank[4 * q]) | (uint32_t(in->exp_of_rank[4 * q + 1]) << 8) |
                 (uint32_t(in->exp_of_rank[4 * q + 2]) << 16) |
                 (uint32_t(in->exp_of_rank[4 * q + 3]) << 24);
  const dim3 grid(static_cast<uint32_t>((n_chunks + kWavesPerBlock - 1) / kWavesPerBlock));
  hipLaunchKernelGGL(rice_to_r4_kernel, grid, dim3(64 * kWavesPerBlock), 0,
                     static_cast<hipStream_t>(stream), a);
  return launch_status();
}
