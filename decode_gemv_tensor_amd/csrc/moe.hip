// MoE expert-gather GEMV on R4 experts and its bf16-expert twin.
//
// "Binade" package page (pypi.org/project/binade), "How it works": the MoE
// expert gather adds its products in the matvec's order; "Limitations": the
// fused kernels cover every expert product. Each (token, slot) pair p has an
// expert idx[p]; its output row is that expert's matvec of the pair's input,
// with exactly the binade_r4_gemv order.
//
// Mapping: a row of J lane tiles (32 columns each) with J > 32 takes a
// whole wave (lane l: tiles l, l + 64, ...); shorter rows are packed
// 64 / 2^ceil(log2 J) to a wave, one lane group per row, lane i of a group
// holding tile i. The blocks are persistent: each finds the set of chosen
// experts once (a bit per expert from idx, in LDS, with per-word counts),
// so experts nobody chose cost nothing; waves then take jobs (u-th chosen
// expert, row group of 2 row sets for whole-wave rows or 4 for packed rows)
// in turn. A job finds with one ballot per 64 pairs the pairs that chose its
// expert, loads its rows' escape metadata once (escape prefixes and
// side-list entries, a lane each), and walks each row set once per pair:
// lane tiles rebuilt through an LDS table of exponent pairs (one lookup per
// nibble byte), escapes patched from registers. A second pair of the same
// expert re-reads the rows the wave has just read, from cache. Rows of
// 64 < J <= 96 tiles (two chunks, the second on at most 32 lanes) are taken
// two at a time, their second chunks in one pass on the wave's two halves.
//
// A packed row's slots 32, 16, ... down to its group width hold no tile, so
// the matvec's tree adds +0.0 to each of the group's slots at those levels;
// one "+ 0.0f" does the same, and the rest of the tree runs inside the group.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

// Row sets per wave (MoeArgs::sets): the expert choice and the escape
// metadata are found once for all of them. Measured best: 2 for whole-wave
// rows, 4 for packed rows.
#ifndef BINADE_MOE_SETS_WHOLE
#define BINADE_MOE_SETS_WHOLE 2
#endif
#ifndef BINADE_MOE_SETS_PACKED
#define BINADE_MOE_SETS_PACKED 4
#endif
constexpr int kSetsWholeRows = BINADE_MOE_SETS_WHOLE, kSetsPackedRows = BINADE_MOE_SETS_PACKED;

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
  uint32_t lut0, lut1, lut2, lut3;   // rotated exponents of ranks 0..15
  int32_t width_log2;      // lanes per row: 6 (a whole wave) or less (packed)
  int32_t sets;            // row sets per wave
  int64_t groups;          // row groups (of sets row sets) per expert
};

__device__ __forceinline__ void store_out(const MoeArgs& a, int64_t i, float v) {
  if (a.y_bf16)
    static_cast<uint16_t*>(a.y)[i] = to_bf16_rne(v);
  else
    static_cast<float*>(a.y)[i] = v;
}

// Exponent table of pairs in LDS: entry b, for a byte b of an R4 nibble
// word (rank of weight i in its low nibble, of weight i + 4 in its high
// nibble), holds the two rotated exponents, low byte first. One lookup per
// byte replaces two 16-entry v_perm lookups (this kernel is bound by its
// instruction issue).
__device__ __forceinline__ void build_pair_table(const MoeArgs& a, uint16_t* pt) {
  const uint32_t b = threadIdx.x;   // 256 threads, one entry each
  const uint32_t t[4] = {a.lut0, a.lut1, a.lut2, a.lut3};
  const uint32_t lo = (t[(b & 15) >> 2] >> (8 * (b & 3))) & 0xFFu;
  const uint32_t hi = (t[b >> 6] >> (8 * ((b >> 4) & 3))) & 0xFFu;
  pt[b] = static_cast<uint16_t>(lo | (hi << 8));
}

// The exponents of the 8 weights of nibble word P: lo for weights 0..3,
// hi for 4..7 (bytes in weight order).
__device__ __forceinline__ void pair_lookup8(uint32_t P, const uint16_t* pt, uint32_t& lo,
                                             uint32_t& hi) {
  const uint32_t A = pt[P & 0xFFu] | (static_cast<uint32_t>(pt[(P >> 8) & 0xFFu]) << 16);
  const uint32_t B = pt[(P >> 16) & 0xFFu] | (static_cast<uint32_t>(pt[P >> 24]) << 16);
  lo = __builtin_amdgcn_perm(B, A, 0x06040200u);   // A = e0 e4 e1 e5, B = e2 e6 e3 e7
  hi = __builtin_amdgcn_perm(B, A, 0x07050301u);
}

// Exponent dwords of one lane tile of a packed wave: table lookups, then
// every packed row's escapes (uniform loop per row; the lane holding the
// entry's tile patches it).
__device__ __forceinline__ void moe_tile_exponents(const MoeArgs& a, uint4 nb, const uint16_t* pt,
                                                   int64_t grow0, int64_t n_valid, int G,
                                                   int wl, int C, int j, int lane,
                                                   uint32_t (&E)[8]) {
  const uint32_t P[4] = {nb.x, nb.y, nb.z, nb.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    pair_lookup8(P[q], pt, E[2 * q], E[2 * q + 1]);
  }
  const int gi = lane >> wl;
  for (int r = 0; r < G; ++r) {
    if (r >= n_valid) break;
    const int64_t chunk = (grow0 + r) * C + j;
    uint32_t e_end = uniform(a.esc_pre[chunk + 1]);
    uint32_t e_beg = uniform(a.esc_pre[chunk]);
    e_end = e_end < a.n_esc ? e_end : a.n_esc;
    e_beg = e_beg < e_end ? e_beg : e_end;
    for (uint32_t e = e_beg; e < e_end; ++e) {
      const uint32_t ent = uniform(a.esc[e]);
      const uint32_t off = ent & 0xFFFFu;
      // off is the column within the 2048-column chunk: tile off >> 5 of it
      const uint32_t tile = off >> 5;
      const uint32_t my_tile = G > 1 ? static_cast<uint32_t>(lane & ((1 << wl) - 1))
                                     : static_cast<uint32_t>(lane);
      if (gi == r && my_tile == tile)
        patch_exponent(E, off & 31u, rot_exponent((ent >> 16) & 0xFFu));
    }
  }
}

constexpr int kMaxExpertWords = 2048;   // experts <= 65536
constexpr int kMaxPairsLds = 2048;      // idx values kept in LDS

// Block setup, once per block: the set of experts some pair chose (a bit per
// expert) and, per 32-expert word, the count of chosen experts before it;
// *n_chosen = their number, *any_bad = whether an index is out of range.
// Every thread of the block takes part.
__device__ __forceinline__ void chosen_set(const MoeArgs& a, uint32_t* present, uint32_t* before,
                                           int32_t* idx_s, uint32_t* n_chosen,
                                           uint32_t* any_bad) {
  const int nw = (a.n_experts + 31) >> 5;
  for (int i = threadIdx.x; i < nw; i += blockDim.x) present[i] = 0u;
  if (threadIdx.x == 0) *any_bad = 0u;
  __syncthreads();
  for (int32_t p = threadIdx.x; p < a.n_pairs; p += blockDim.x) {
    const int32_t v = a.idx[p];
    if (p < kMaxPairsLds) idx_s[p] = v;
    if (v >= 0 && v < a.n_experts)
      atomicOr(&present[v >> 5], 1u << (v & 31));
    else
      *any_bad = 1u;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // wave 0: exclusive prefix count of set bits over the words
    uint32_t acc = 0;
    for (int base = 0; base < nw; base += 64) {
      const int i = base + static_cast<int>(threadIdx.x);
      const uint32_t c = i < nw ? __popc(present[i]) : 0u;
      uint32_t incl = c;
      for (int sh = 1; sh < 64; sh <<= 1) {
        const uint32_t o = __shfl_up(incl, sh, 64);
        if (static_cast<int>(threadIdx.x) >= sh) incl += o;
      }
      if (i < nw) before[i] = acc + incl - c;
      acc += __shfl(incl, 63, 64);
    }
    if (threadIdx.x == 0) *n_chosen = acc;
  }
  __syncthreads();
}

// The u-th chosen expert (increasing index), u < n_chosen: the last word
// whose count before it is <= u, then the matching set bit in it.
__device__ __forceinline__ int32_t chosen_expert(const MoeArgs& a, const uint32_t* present,
                                                 const uint32_t* before, uint32_t u) {
  const int nw = (a.n_experts + 31) >> 5;
  int lo = 0, hi = nw - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (before[mid] <= u)
      lo = mid;
    else
      hi = mid - 1;
  }
  uint32_t w = present[lo];
  for (uint32_t k = u - before[lo]; k > 0; --k) w &= w - 1u;
  return (lo << 5) + __builtin_ctz(w);
}

// The same patches from registers: lane c holds the escape prefix of the
// wave's c-th chunk (chunks of its rows in order, pre_lane), lane i holds
// side-list entry e0 + i (ent_lane). Chunk c = (row r, chunk j) of the rows'
// flat chunk range; only chunks j of this pass are walked.
__device__ __forceinline__ void moe_patch_regs(uint32_t pre_lane, uint32_t ent_lane, uint32_t e0,
                                               int cbase, int n_valid, int C, int j, int wl,
                                               int G, int lane, uint32_t (&E)[8]) {
  const int gi = lane >> wl;
  const uint32_t my_tile = G > 1 ? static_cast<uint32_t>(lane & ((1 << wl) - 1))
                                 : static_cast<uint32_t>(lane);
  for (int r = 0; r < n_valid; ++r) {
    const int c = cbase + r * C + j;
    const uint32_t lo = __builtin_amdgcn_readlane(pre_lane, c);
    const uint32_t hi = __builtin_amdgcn_readlane(pre_lane, c + 1);
    for (uint32_t q = lo; q < hi; ++q) {
      const uint32_t ent = __builtin_amdgcn_readlane(ent_lane, static_cast<int>(q - e0));
      const uint32_t off = ent & 0xFFFFu;
      if (gi == r && my_tile == (off >> 5))
        patch_exponent(E, off & 31u, rot_exponent((ent >> 16) & 0xFFu));
    }
  }
}

// Raw loads of one lane tile: R4 sm + nibbles, or the twin's bf16 words.
template <bool kR4>
struct MoeRaw {
  uint4 s0, s1, nb;   // R4
  uint4 q[4];         // twin
};

template <bool kR4>
__device__ __forceinline__ void moe_load(const MoeArgs& a, int64_t grow, int t, bool active,
                                         MoeRaw<kR4>& r) {
  const uint4 z = make_uint4(0, 0, 0, 0);
  if (kR4) {
    r.s0 = r.s1 = r.nb = z;
    if (active) {
      const uint4* ps = reinterpret_cast<const uint4*>(a.w + grow * a.cols + 32 * t);
      r.s0 = ps[0];
      r.s1 = ps[1];
      r.nb = *reinterpret_cast<const uint4*>(a.nib + grow * (a.cols >> 1) + 16 * t);
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) r.q[v] = z;
    if (active) {
      const uint4* pw = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.w) +
                                                       grow * a.cols + 32 * t);
#pragma unroll
      for (int v = 0; v < 4; ++v) r.q[v] = pw[v];
    }
  }
}

// One lane tile's 32 weights as fp32 (escapes patched for R4).
template <bool kR4>
__device__ __forceinline__ void moe_weights(const MoeArgs& a, const MoeRaw<kR4>& r, const uint16_t* pt,
                                            bool regs, uint32_t pre_lane, uint32_t ent_lane,
                                            uint32_t e0, int cbase, int64_t grow0,
                                            int64_t n_valid, int G, int wl, int C, int j,
                                            int lane, float (&w)[32]) {
  if (kR4) {
    uint32_t E[8];
    if (regs) {
      const uint32_t P[4] = {r.nb.x, r.nb.y, r.nb.z, r.nb.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pair_lookup8(P[q], pt, E[2 * q], E[2 * q + 1]);
      }
      moe_patch_regs(pre_lane, ent_lane, e0, cbase, static_cast<int>(n_valid), C, j, wl, G, lane,
                     E);
    } else {
      moe_tile_exponents(a, r.nb, pt, grow0, n_valid, G, wl, C, j, lane, E);
    }
    const uint32_t S[8] = {r.s0.x, r.s0.y, r.s0.z, r.s0.w, r.s1.x, r.s1.y, r.s1.z, r.s1.w};
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t H, Lo;
      split4_rot(S[d], E[d], H, Lo);
      w[4 * d] = weight_f32<0>(H, Lo);
      w[4 * d + 1] = weight_f32<1>(H, Lo);
      w[4 * d + 2] = weight_f32<2>(H, Lo);
      w[4 * d + 3] = weight_f32<3>(H, Lo);
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t q[4] = {r.q[v].x, r.q[v].y, r.q[v].z, r.q[v].w};
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        w[8 * v + 2 * k2] = bf16_lo(q[k2]);
        w[8 * v + 2 * k2 + 1] = bf16_hi(q[k2]);
      }
    }
  }
}

// A wave's rows: a.sets row sets of expert e, set s = rows
// row0 + s*G .. +G-1 (G = 1: a whole-wave row). The expert, the pairs that
// chose it and the rows' escape metadata are found once for all the sets;
// tiles are loaded per chunk inside each pass over a pair, which keeps the
// register count (and so the waves per SIMD) where this latency-bound
// kernel wants it.
template <bool kR4, bool kMerge>
__device__ __forceinline__ void moe_rows(const MoeArgs& a, const uint16_t* pt, int32_t e, int64_t row0,
                                         int G, int gi, int ti, int wl, int J, int C, int lane,
                                         const int32_t* idx_s) {
  const int64_t left = a.n_rows - row0;
  const int64_t n_rows_w = left < G * a.sets ? left : G * a.sets;   // >= 1
  const int64_t grow_w = static_cast<int64_t>(e < 0 ? 0 : e) * a.n_rows + row0;

  // the wave's escape prefixes and side-list entries, in registers when
  // they fit a lane each (the usual case)
  const int F = static_cast<int>(n_rows_w) * C;   // chunks of the wave's rows
  uint32_t pre_lane = 0, ent_lane = 0, e0 = 0;
  bool regs = false;
  if (kR4 && e >= 0 && F + 1 <= 64) {
    const uint32_t pv = lane <= F ? a.esc_pre[grow_w * C + lane] : 0u;
    pre_lane = pv < a.n_esc ? pv : a.n_esc;
    e0 = __builtin_amdgcn_readlane(pre_lane, 0);
    const uint32_t e1 = __builtin_amdgcn_readlane(pre_lane, F);
    if (e1 >= e0 && e1 - e0 <= 64u) {
      regs = true;
      ent_lane = static_cast<uint32_t>(lane) < e1 - e0 ? a.esc[e0 + lane] : 0u;
      // prefixes must not decrease, or the register walk would misread
      const uint32_t prev = __shfl_up(pre_lane, 1, 64);
      if (__any(lane >= 1 && lane <= F && pre_lane < prev)) regs = false;
    }
  }

  const bool merged =
      kMerge && G == 1 && C == 2 && a.sets == 2 && J > 64 && J <= 96 && row0 + 1 < a.n_rows;
  for (int32_t base = 0; base < a.n_pairs; base += 64) {
    const int32_t p = base + lane;
    const int32_t v = p < a.n_pairs ? (p < kMaxPairsLds ? idx_s[p] : a.idx[p]) : 0;
    const uint64_t mine_all = __ballot(p < a.n_pairs && v == e);
    if (mine_all == 0) continue;
    if (merged) {
      // Two whole-wave rows of 64 < J <= 96 tiles: row A's and row B's first
      // chunks in two passes, then both second chunks in one pass (row A on
      // lanes 0..31, row B on lanes 32..63, its slot sums moved there and
      // back unchanged). Each slot's chain and the slot tree are those of
      // the passes below.
      const int64_t growA = grow_w, growB = grow_w + 1;
      uint64_t mine = mine_all;
      while (mine != 0) {
        const int b = __builtin_ctzll(mine);
        mine &= mine - 1;
        const int32_t pp = base + b;
        const int64_t xrow = a.x_per_slot ? pp : pp / a.top_k;
        const uint16_t* xr = a.x + xrow * a.cols;
        float a0A = 0.0f, a1A = 0.0f, a0B = 0.0f, a1B = 0.0f;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
          MoeRaw<kR4> rj;
          moe_load<kR4>(a, h ? growB : growA, lane, true, rj);
          float w[32];
          moe_weights<kR4>(a, rj, pt, regs, pre_lane, ent_lane, e0, 2 * h, h ? growB : growA, 1,
                           1, 6, 2, 0, lane, w);
          float xf[32];
          load_x_tile(xr, lane, xf);
          float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s0 = __builtin_fmaf(w[2 * i], xf[2 * i], s0);
            s1 = __builtin_fmaf(w[2 * i + 1], xf[2 * i + 1], s1);
          }
          if (h) {
            a0B = s0;
            a1B = s1;
          } else {
            a0A = s0;
            a1A = s1;
          }
        }
        const int half = lane >> 5;
        const int t1 = 64 + (lane & 31);
        const bool act = t1 < J;
        const float m0 = __shfl(a0B, (lane - 32) & 63, 64);
        const float m1 = __shfl(a1B, (lane - 32) & 63, 64);
        float c0 = half ? m0 : a0A, c1 = half ? m1 : a1A;
        {
          MoeRaw<kR4> rj;
          moe_load<kR4>(a, half ? growB : growA, t1, act, rj);
          float w[32];
          moe_weights<kR4>(a, rj, pt, regs, pre_lane, ent_lane, e0, 0, growA, 2, 2, 5, 2, 1, lane,
                           w);
          if (act) {
            float xf[32];
            load_x_tile(xr, t1, xf);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              c0 = __builtin_fmaf(w[2 * i], xf[2 * i], c0);
              c1 = __builtin_fmaf(w[2 * i + 1], xf[2 * i + 1], c1);
            }
          }
        }
        const float sum = c0 + c1;
        const float bsum = __shfl(sum, (lane + 32) & 63, 64);
        float rA = half ? a0A + a1A : sum;
        float rB = half ? a0B + a1B : bsum;
        rA = slot_tree(rA);
        rB = slot_tree(rB);
        if (lane == 0) {
          store_out(a, static_cast<int64_t>(pp) * a.n_rows + row0, rA);
          store_out(a, static_cast<int64_t>(pp) * a.n_rows + row0 + 1, rB);
        }
      }
      continue;
    }
    for (int set = 0; set < a.sets; ++set) {
      const int64_t set0 = row0 + static_cast<int64_t>(set) * G;
      if (set0 >= a.n_rows) break;
      const int64_t n_valid = a.n_rows - set0 < G ? a.n_rows - set0 : G;
      const bool row_ok = gi < n_valid;
      const int64_t row = set0 + (row_ok ? gi : 0);
      const int64_t grow0 = grow_w + (set0 - row0);
      const int64_t grow = grow0 + (row - set0);
      const int cbase = set * G * C;   // this set's first chunk in the wave's metadata
      uint64_t mine = mine_all;
      while (mine != 0) {
        const int b = __builtin_ctzll(mine);
        mine &= mine - 1;
        const int32_t pp = base + b;
        float a0 = 0.0f, a1 = 0.0f;
        for (int j = 0; j < C; ++j) {
          const int t = G > 1 ? ti : j * 64 + lane;
          const bool active = t < J;
          MoeRaw<kR4> rj;
          moe_load<kR4>(a, grow, t, active, rj);
          float w[32];
          moe_weights<kR4>(a, rj, pt, regs, pre_lane, ent_lane, e0, cbase, grow0, n_valid, G, wl,
                           C, j, lane, w);
          if (!active) continue;
          const int64_t xrow = a.x_per_slot ? pp : pp / a.top_k;
          float xf[32];
          load_x_tile(a.x + xrow * a.cols, t, xf);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            a0 = __builtin_fmaf(w[2 * i], xf[2 * i], a0);
            a1 = __builtin_fmaf(w[2 * i + 1], xf[2 * i + 1], a1);
          }
        }
        float r = a0 + a1;
        if (G == 1) {
          r = slot_tree(r);
        } else {
          r = r + 0.0f;   // the tree levels whose partner slots hold no tile
          for (int sh = (1 << wl) >> 1; sh >= 1; sh >>= 1) r = r + __shfl_xor(r, sh, 64);
        }
        if (ti == 0 && row_ok) store_out(a, static_cast<int64_t>(pp) * a.n_rows + row, r);
      }
    }
  }
}

// Persistent blocks: the chosen set is found once per block; wave w then
// takes the jobs w, w + W, ... (W waves in the grid), job = (u-th chosen
// expert, row group) with a.groups row groups per expert.
// kMerge: rows of 64 < J <= 96 lane tiles run the merged second pass (the
// instantiation holds more registers, so other row widths use the other).
template <bool kR4, bool kMerge>
__global__ __launch_bounds__(256) void moe_gemv_kernel(MoeArgs a) {
  __shared__ uint32_t present[kMaxExpertWords];
  __shared__ uint32_t before[kMaxExpertWords];
  __shared__ int32_t idx_s[kMaxPairsLds];
  __shared__ uint32_t n_chosen, any_bad;
  __shared__ uint16_t pt[256];
  if (kR4) build_pair_table(a, pt);   // visible after chosen_set's barriers
  chosen_set(a, present, before, idx_s, &n_chosen, &any_bad);
  const int lane = threadIdx.x & 63;
  const int wl = a.width_log2;
  const int G = 64 >> wl;                       // rows per row set
  const int gi = lane >> wl;                    // this lane's row in the set
  const int ti = lane & ((1 << wl) - 1);        // this lane's tile (packed)
  const int J = a.cols >> 5;
  const int C = (J + 63) >> 6;
  const uint32_t U = uniform(n_chosen);
  const uint64_t jobs = static_cast<uint64_t>(U) * a.groups;
  const uint64_t W = static_cast<uint64_t>(gridDim.x) * (blockDim.x >> 6);
  for (uint64_t job = uniform64(static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) +
                                (threadIdx.x >> 6));
       job < jobs; job += W) {
    const uint32_t u = static_cast<uint32_t>(job / a.groups);
    const int32_t e = uniform(chosen_expert(a, present, before, u));
    const int64_t row0 = static_cast<int64_t>(job - static_cast<uint64_t>(u) * a.groups) * G *
                         a.sets;
    moe_rows<kR4, kMerge>(a, pt, e, row0, G, gi, ti, wl, J, C, lane, idx_s);
  }
  if (uniform(any_bad) != 0u) {
    // out-of-range indices: flag once, and zero those pairs' rows (rows
    // dealt to the blocks in equal ranges)
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.status != nullptr)
      atomicOr(a.status, static_cast<uint32_t>(BINADE_DEV_BAD_INDEX));
    const int64_t per = (a.n_rows + gridDim.x - 1) / gridDim.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t r1 = r0 + per < a.n_rows ? r0 + per : a.n_rows;
    for (int32_t p = 0; p < a.n_pairs; ++p) {
      const int32_t v = p < kMaxPairsLds ? idx_s[p] : a.idx[p];
      if (v >= 0 && v < a.n_experts) continue;
      for (int64_t r = r0 + threadIdx.x; r < r1; r += blockDim.x)
        store_out(a, static_cast<int64_t>(p) * a.n_rows + r, 0.0f);
    }
  }
}

// Blocks of the persistent MoE kernel that fit on the current device at once
// (queried once per device and kind).
int32_t resident_blocks(bool r4, bool merge, int64_t& blocks) {
  static int64_t cached[2][2][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return launch_status();
  if (dev < 64 && cached[r4][merge][dev] > 0) {
    blocks = cached[r4][merge][dev];
    return BINADE_OK;
  }
  int per_cu = 0, cus = 0;
  const void* k = r4 ? (merge ? reinterpret_cast<const void*>(&moe_gemv_kernel<true, true>)
                              : reinterpret_cast<const void*>(&moe_gemv_kernel<true, false>))
                     : (merge ? reinterpret_cast<const void*>(&moe_gemv_kernel<false, true>)
                              : reinterpret_cast<const void*>(&moe_gemv_kernel<false, false>));
  const hipError_t q = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, 0);
  if (q != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return launch_status();
  blocks = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  if (dev < 64) cached[r4][merge][dev] = blocks;
  return BINADE_OK;
}

int32_t launch(MoeArgs a, bool r4, hipStream_t stream) {
  const int J = a.cols >> 5;
  int wl = 0;
  while ((1 << wl) < J && wl < 6) ++wl;
  a.width_log2 = J > 32 ? 6 : wl;
  a.sets = a.width_log2 == 6 ? kSetsWholeRows : kSetsPackedRows;
  const int64_t rows_per_group = static_cast<int64_t>(64 >> a.width_log2) * a.sets;
  a.groups = (a.n_rows + rows_per_group - 1) / rows_per_group;
  // at most min(experts, pairs) experts are chosen
  const int64_t chosen_max = a.n_experts < a.n_pairs ? a.n_experts : a.n_pairs;
  const int64_t waves = chosen_max * a.groups;
  // rows of 64 < J <= 96 tiles: the instantiation with the merged second pass
  const bool merge = J > 64 && J <= 96;
  int64_t resident = 0;
  const int32_t st = resident_blocks(r4, merge, resident);
  if (st != BINADE_OK) return st;
  const int64_t need = (waves + 3) / 4;
  const dim3 grid(static_cast<uint32_t>(need < resident ? (need > 0 ? need : 1) : resident));
  if (r4) {
    if (merge) hipLaunchKernelGGL((moe_gemv_kernel<true, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((moe_gemv_kernel<true, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (merge) hipLaunchKernelGGL((moe_gemv_kernel<false, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((moe_gemv_kernel<false, false>), grid, dim3(256), 0, stream, a);
  }
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
  a.lut0 = rot_exponents4(pack4(w->lut));
  a.lut1 = rot_exponents4(pack4(w->lut + 4));
  a.lut2 = rot_exponents4(pack4(w->lut + 8));
  a.lut3 = rot_exponents4(pack4(w->lut + 12));
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
