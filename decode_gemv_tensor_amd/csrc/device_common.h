// Device helpers shared by the libbinade kernels (gfx950, wave64).
//
// Weight rebuild: "Binade" package page (pypi.org/project/binade), intro and
// "How it works": a weight is its sign+mantissa byte plus the exponent that
// its 4-bit rank selects in the tensor's table (rank 15 = escape, whose
// exponent comes from the side list).
#ifndef BINADE_DEVICE_COMMON_H
#define BINADE_DEVICE_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "binade.h"

namespace binade {
namespace dev {

constexpr int kWave = 64;
constexpr int kTile = 32;                 // weights per lane tile
constexpr int kChunk = kWave * kTile;     // one wave pass = one row-chunk
static_assert(kChunk == BINADE_CHUNK, "row-chunk must be one wave pass");

// The 16-entry rank -> exponent table as four dwords (bytes 0-3, 4-7, 8-11,
// 12-15), kept in VGPRs so v_perm_b32 can index it.
struct Lut {
  uint32_t t0, t1, t2, t3;
};

__device__ __forceinline__ uint32_t vperm(uint32_t hi, uint32_t lo,
                                          uint32_t sel) {
  // v_perm_b32: byte i of the result = byte sel[i] of the 8-byte value
  // {hi, lo} (0-3 from lo, 4-7 from hi), 12 -> 0x00.
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four ranks, one per byte (values 0..15 in the low nibble; high nibble
// ignored), -> their four exponent bytes.
__device__ __forceinline__ uint32_t lookup4(uint32_t ranks, const Lut& L) {
  const uint32_t sel = ranks & 0x07070707u;
  const uint32_t lo = vperm(L.t1, L.t0, sel);
  const uint32_t hi = vperm(L.t3, L.t2, sel);
  // 0xFF in bytes whose rank is below 8: selector 4 picks byte 0 of the
  // all-ones word, selector 12 gives zero
  const uint32_t m = vperm(0xFFFFFFFFu, 0u, (ranks & 0x08080808u) | 0x04040404u);
  return (lo & m) | (hi & ~m);
}

// Split four (sm, exponent) byte pairs into the high and low bytes of their
// bf16 patterns: high = sign | e >> 1, low = (e & 1) << 7 | mantissa.
__device__ __forceinline__ void split4(uint32_t S, uint32_t E, uint32_t& H,
                                       uint32_t& Lo) {
  H = (S & 0x80808080u) | ((E >> 1) & 0x7F7F7F7Fu);
  Lo = (S & 0x7F7F7F7Fu) | ((E << 7) & 0x80808080u);
}

// The exponent byte rotated right by one: (e >> 1) | (e & 1) << 7. With the
// table held in this form, both bf16 bytes of four weights are one bit-field
// insert each (split4_rot).
__host__ __device__ __forceinline__ uint32_t rot_exponent(uint32_t e) {
  return ((e >> 1) & 0x7Fu) | ((e & 1u) << 7);
}
__host__ __device__ __forceinline__ uint32_t rot_exponents4(uint32_t e4) {
  return ((e4 >> 1) & 0x7F7F7F7Fu) | ((e4 << 7) & 0x80808080u);
}

__device__ __forceinline__ void split4_rot(uint32_t S, uint32_t Er, uint32_t& H,
                                           uint32_t& Lo) {
  H = (S & 0x80808080u) | (Er & 0x7F7F7F7Fu);
  Lo = (Er & 0x80808080u) | (S & 0x7F7F7F7Fu);
}

// fp32 value of weight b (0..3) of a split group: bf16 bits in the top half.
template <int b>
__device__ __forceinline__ float weight_f32(uint32_t H, uint32_t Lo) {
  constexpr uint32_t sel = ((4u + b) << 24) | (uint32_t(b) << 16) | 0x0C0Cu;
  return __uint_as_float(vperm(H, Lo, sel));
}

// bf16 patterns of weights b and b+1 of a split group, packed in one dword.
template <int b>
__device__ __forceinline__ uint32_t weight_pair_bf16(uint32_t H, uint32_t Lo) {
  constexpr uint32_t sel = ((5u + b) << 24) | ((1u + b) << 16) |
                           ((4u + b) << 8) | uint32_t(b);
  return vperm(H, Lo, sel);
}

// fma 4 weights of one split group into the two running sums of a lane
// tile, columns 4d .. 4d+3 (4d is even: even columns go to a0, odd to a1).
__device__ __forceinline__ void fma_group(uint32_t H, uint32_t Lo,
                                          const float* xg, float& a0,
                                          float& a1) {
  a0 = __builtin_fmaf(weight_f32<0>(H, Lo), xg[0], a0);
  a1 = __builtin_fmaf(weight_f32<1>(H, Lo), xg[1], a1);
  a0 = __builtin_fmaf(weight_f32<2>(H, Lo), xg[2], a0);
  a1 = __builtin_fmaf(weight_f32<3>(H, Lo), xg[3], a1);
}

__device__ __forceinline__ float bf16_lo(uint32_t d) {
  return __uint_as_float(d << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t d) {
  return __uint_as_float(d & 0xFFFF0000u);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
    return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Escape patch: replace exponent byte `idx & 3` of dword `idx >> 2` of E[8].
// idx is wave-uniform; a switch keeps every E[q] in its own register (an
// indexed form would put E in scratch memory).
__device__ __forceinline__ void patch_exponent(uint32_t (&E)[8], uint32_t idx,
                                               uint32_t expo) {
  const uint32_t sh = (idx & 3u) * 8u;
  const uint32_t m = 0xFFu << sh;
  const uint32_t v = expo << sh;
  switch (idx >> 2) {
    case 0: E[0] = (E[0] & ~m) | v; break;
    case 1: E[1] = (E[1] & ~m) | v; break;
    case 2: E[2] = (E[2] & ~m) | v; break;
    case 3: E[3] = (E[3] & ~m) | v; break;
    case 4: E[4] = (E[4] & ~m) | v; break;
    case 5: E[5] = (E[5] & ~m) | v; break;
    case 6: E[6] = (E[6] & ~m) | v; break;
    default: E[7] = (E[7] & ~m) | v; break;
  }
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}


// 32 x values of lane tile t as fp32 (four 16-byte loads).
__device__ __forceinline__ void load_x_tile(const uint16_t* x, int t,
                                            float (&xf)[32]) {
  const uint4* p = reinterpret_cast<const uint4*>(x + 32 * t);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint4 d = p[v];
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xf[8 * v + 2 * e] = bf16_lo(w[e]);
      xf[8 * v + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
}

// The slot tree: p[l] = p[l] + p[l + s] for l < s, s = 32 .. 1; lane 0 ends
// with the row's value (lanes >= s hold values no lane reads).
__device__ __forceinline__ float slot_tree(float p) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_xor(p, s, 64);
  return p;
}

// The 8 exponent dwords of one lane tile: table lookups of its 16 nibble
// bytes, then the escapes of the row-chunk (uniform loop over the chunk's
// side-list entries; the lane owning an entry's position patches it). With
// kRot the table L is rotated (rot_exponents4) and so are the patches.
template <bool kRot = false>
__device__ __forceinline__ void tile_exponents(uint4 nb, const Lut& L,
                                               const uint32_t* esc_pre,
                                               const uint32_t* esc,
                                               uint32_t n_esc, int64_t chunk,
                                               int lane, uint32_t (&E)[8]) {
  const uint32_t P[4] = {nb.x, nb.y, nb.z, nb.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    E[2 * q] = lookup4(P[q], L);
    E[2 * q + 1] = lookup4(P[q] >> 4, L);
  }
  uint32_t e_end = uniform(esc_pre[chunk + 1]);
  uint32_t e_beg = uniform(esc_pre[chunk]);
  e_end = e_end < n_esc ? e_end : n_esc;
  e_beg = e_beg < e_end ? e_beg : e_end;
  for (uint32_t e = e_beg; e < e_end; ++e) {
    const uint32_t ent = uniform(esc[e]);
    const uint32_t off = ent & 0xFFFFu;
    const uint32_t ex = (ent >> 16) & 0xFFu;
    if (static_cast<uint32_t>(lane) == (off >> 5))
      patch_exponent(E, off & 31u, kRot ? rot_exponent(ex) : ex);
  }
}

}  // namespace dev

// Host-side bookkeeping shared by the entry points.
void set_last_hip_error(int32_t e);
int32_t launch_status();  // BINADE_OK or BINADE_EHIP after a launch

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

}  // namespace binade

#endif
