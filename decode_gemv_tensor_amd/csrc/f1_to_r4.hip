// Format 1 (a fixed code width per 128-weight tile, with escapes) -> R4, on
// the GPU at load.
//
// "Binade" package page (pypi.org/project/binade), "How it works": the
// second file format keeps one code width per 128-weight tile and escapes
// the ranks that do not fit; at load a GPU kernel turns either file format
// into R4 (4-bit ranks, the few ranks >= 15 in a side list). The byte
// layout is the one binade.h states for binade_f1.
//
// One wave per job of at most 2048 weights: one row-chunk when rows are
// longer than a chunk, else G = 2048 / cols whole rows. Lane l owns the
// job's weights 32l .. 32l+31, which lie in one tile (tiles are 128 columns
// of a row and 32 divides cols). Every tile holds a whole number of 32-bit
// words (w * len bits, 32 | len), so a valid job starts on a word and lane
// l's codes are exactly w_l whole words.
//  0. The job's index entries are scalar loads. The code words, escape
//     bytes and each lane's tile width come in through buffer loads whose
//     range is the job's own span: out-of-range reads give zero and touch
//     no memory, so no load needs a branch. Code words and escape bytes go
//     to LDS.
//  1. A wave prefix sum of the lanes' widths gives each lane's first word.
//  2. The lane turns its words into R4 nibbles with shifts and masks fixed
//     for its width (1 to 4; any width and table size on a checked path),
//     and marks its escape codes (all w bits set) in a 32-bit mask in
//     weight order.
//  3. A prefix sum of the escape counts places each lane in the escape
//     bytes; the lane walks its escapes, adds min(rank, 15) - min(code, 15)
//     to the nibble in LDS, and marks ranks >= 15 for the R4 side list,
//     whose entries a third prefix sum places.
//  4. One 16-byte store per lane: the job's nibbles are one coalesced block.
// The job's anchors and prefixes are checked against what the codes imply;
// a mismatch sets the device status word and the job writes nothing.
#include <hip/hip_runtime.h>

#include <cstddef>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

constexpr int kF1Tile = 128;
constexpr int kF1Waves = 4;
constexpr int kCodeWords = 512 + 4;   // a job's codes (2048 weights x 8 bits) and a look-ahead word
constexpr int kEscStage = 256;        // escape bytes staged per job (more are read from memory)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct F1Args {
  const uint8_t* width;
  const uint32_t* codes;
  const uint8_t* esc_rank;
  const uint64_t* anchor;
  const uint32_t* f1_pre;
  const uint32_t* esc_pre;
  uint8_t* nib;
  uint32_t* esc;
  uint32_t* status;
  uint64_t code_bits;
  uint64_t code_words;
  uint64_t n_f1esc;
  uint64_t n_esc;
  int64_t rows;
  int64_t jobs;
  int32_t cols;
  uint32_t n;
  uint32_t tiles_per_row;    // T = ceil(cols / 128)
  uint32_t chunks_per_row;   // C = ceil(cols / 2048)
  uint32_t job_rows;         // G = 2048 / cols when C == 1
  uint32_t col_recip;        // ceil(2^32 / cols) when C == 1: o / cols = mulhi(o, col_recip) for o < 2048
  uint32_t chunk_recip;      // floor(2^32 / C) + 1 when C > 1: j / C is mulhi(j, chunk_recip) or one less
  uint8_t exp_of_rank[256];
};

// A buffer resource over bytes [base, base + bytes): loads beyond it return
// zero and access nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ uint32_t load_u8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ void f1_flag(uint32_t* status, uint32_t bits, int lane) {
  if (status != nullptr && lane == 0) atomicOr(status, bits);
}

__device__ __forceinline__ uint32_t f1_scan(uint32_t v) {   // inclusive, 64 lanes
  constexpr int kRowShr = 0x110, kBcast15 = 0x142, kBcast31 = 0x143;
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 8, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0u, v, kBcast31, 0xC, 0xF, false);
  return v;
}

// LDS writes of the wave visible to its own later reads.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint32_t f1_lane63(uint32_t v) {
  return __builtin_amdgcn_readlane(v, 63);
}

// Bit shift of weight i's nibble in a lane's 16 output bytes (R4 order:
// groups of 8 weights per word, weight i in byte i % 4, high nibble for the
// group's last four).
__host__ __device__ constexpr uint32_t nib_shift(uint32_t i) {
  return 8u * (i & 3u) + (i & 4u);
}

// Flags at bit 8k + 4h + S of an R4 word (the nibble of weight 4h + k of its
// eight) -> 8 bits in weight order.
template <int S>
__device__ __forceinline__ uint32_t weight_order(uint32_t e) {
  uint32_t t = (e | (e >> 7)) & (0x00330033u << S);
  t = t | (t >> 14);
  return (t >> S) & 0xFFu;
}

// 4 codes of `bits` bits at stride `bits` (low bits of u) -> bytes 0..3.
__device__ __forceinline__ uint32_t spread1(uint32_t u) {   // u < 16
  return __umul24(u, 0x00204081u) & 0x01010101u;
}
__device__ __forceinline__ uint32_t spread2(uint32_t u) {   // u < 256
  uint32_t t = (u | (u << 12)) & 0x000F000Fu;
  return (t | (t << 6)) & 0x03030303u;
}
__device__ __forceinline__ uint32_t spread3(uint32_t u) {   // u < 4096
  uint32_t t = (u | (u << 10)) & 0x003F003Fu;
  return (t | (t << 5)) & 0x07070707u;
}

// Decoders for a lane's 32 codes of width W from W words g (code i at bit
// W*i), for a table whose every rank below the escape code exists: nibbles
// in R4 order into out, escape codes as bits of esc in weight order.
__device__ __forceinline__ void decode_w1(const uint32_t* g, uint32_t (&out)[4], uint32_t& esc) {
  const uint32_t x = g[0];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t b = (x >> (8 * d)) & 0xFFu;
    out[d] = spread1(b & 0xFu) | (spread1(b >> 4) << 4);
  }
  esc = x;   // code 1 is the escape
}

__device__ __forceinline__ void decode_w2(const uint32_t* g, uint32_t (&out)[4], uint32_t& esc) {
  const uint32_t g0 = g[0], g1 = g[1];
  esc = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = ((d < 2 ? g0 : g1) >> (16 * (d & 1))) & 0xFFFFu;
    const uint32_t o = spread2(x & 0xFFu) | (spread2(x >> 8) << 4);
    out[d] = o;
    esc |= weight_order<2>((o + 0x11111111u) & 0x44444444u) << (8 * d);   // nibble 3
  }
}

__device__ __forceinline__ void decode_w3(const uint32_t* g, uint32_t (&out)[4], uint32_t& esc) {
  const uint32_t g0 = g[0], g1 = g[1], g2 = g[2];
  const uint32_t x[4] = {g0, __builtin_amdgcn_alignbit(g1, g0, 24), __builtin_amdgcn_alignbit(g2, g1, 16),
                         g2 >> 8};
  esc = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t o = spread3(x[d] & 0xFFFu) | (spread3(__builtin_amdgcn_ubfe(x[d], 12, 12)) << 4);
    out[d] = o;
    esc |= weight_order<3>((o + 0x11111111u) & 0x88888888u) << (8 * d);   // nibble 7
  }
}

__device__ __forceinline__ void decode_w4(const uint32_t* g, uint32_t (&out)[4], uint32_t& esc) {
  esc = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = g[d];   // nibble k = weight k
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
    out[d] = vperm(hi, lo, 0x05010400u) | (vperm(hi, lo, 0x07030602u) << 4);
    uint32_t t = (((x & 0x77777777u) + 0x11111111u) & x & 0x88888888u) >> 3;   // nibble 15
    t = (t | (t >> 3)) & 0x03030303u;
    t = (t | (t >> 6)) & 0x000F000Fu;
    esc |= ((t | (t >> 12)) & 0xFFu) << (8 * d);
  }
}

// Code i (width w) of a lane whose codes start at word g[0].
__device__ __forceinline__ uint32_t code_at(const uint32_t* g, uint32_t w, uint32_t i) {
  const uint32_t b = i * w;
  return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(g[(b >> 5) + 1], g[b >> 5], b & 31u), 0u, w);
}

// Any width 1..8 and any table, every code checked: nibbles min(code, 15);
// escape codes as bits of esc, direct codes >= 15 as bits of big; a direct
// code outside the table sets bad.
__device__ __forceinline__ void decode_checked(const uint32_t* g, uint32_t w, uint32_t n,
                                               uint32_t (&out)[4], uint32_t& esc, uint32_t& big,
                                               bool& bad) {
  const uint32_t esc_code = (1u << w) - 1u;
  esc = 0;
  big = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t o = 0;
#pragma unroll 1
    for (uint32_t k = 0; k < 8; ++k) {
      const uint32_t i = 8u * d + k;
      const uint32_t code = code_at(g, w, i);
      const bool is_esc = code == esc_code;
      o |= min(code, 15u) << nib_shift(k);
      esc |= (is_esc ? 1u : 0u) << i;
      big |= (code >= 15u && !is_esc ? 1u : 0u) << i;
      bad = bad || (code >= n && !is_esc);
    }
    out[d] = o;
  }
}

// One job's geometry, index entries and loads (issued, not yet waited for).
struct F1Job {
  uint64_t c0, fb, A, Bend;
  uint32_t cnt, len, f0, f1end, e0, e1end, nw, n_escj;
  bool bad, bad_esc, live, row_start;
  __amdgpu_buffer_rsrc_t re;
  u32x4 v0, v1;
  uint32_t ev, w, row_local, col;
  uint64_t row_anchor;
  uint32_t row_f1, row_esc;
};

__device__ __forceinline__ void f1_load(const F1Args& a, uint32_t j, uint32_t lane, F1Job& J) {
  const uint32_t T = a.tiles_per_row, C = a.chunks_per_row;
  const uint32_t cols = static_cast<uint32_t>(a.cols);
  // ---- the job: chunks [c0, c0 + cnt), weights [fb, fb + len), tiles from t0
  uint64_t t0;
  uint32_t ntiles;
  if (C > 1) {
    uint32_t row = __umulhi(j, a.chunk_recip);
    if (row * C > j) --row;
    const uint32_t q = j - row * C;
    J.c0 = j;
    J.cnt = 1;
    J.fb = static_cast<uint64_t>(row) * cols + q * kChunk;
    J.len = min(static_cast<uint32_t>(kChunk), cols - q * kChunk);
    t0 = static_cast<uint64_t>(row) * T + q * (kChunk / kF1Tile);
    ntiles = (J.len + kF1Tile - 1) / kF1Tile;
  } else {
    const uint64_t row0 = static_cast<uint64_t>(j) * a.job_rows;
    J.cnt = static_cast<uint32_t>(min(static_cast<uint64_t>(a.job_rows), static_cast<uint64_t>(a.rows) - row0));
    J.c0 = row0;
    J.fb = row0 * cols;
    J.len = J.cnt * cols;
    t0 = row0 * T;
    ntiles = J.cnt * T;
  }
  J.A = a.anchor[J.c0];
  J.Bend = a.anchor[J.c0 + J.cnt];
  J.f0 = a.f1_pre[J.c0];
  J.f1end = a.f1_pre[J.c0 + J.cnt];
  J.e0 = a.esc_pre[J.c0];
  J.e1end = a.esc_pre[J.c0 + J.cnt];
  const bool first = j == 0, last = j + 1 == static_cast<uint64_t>(a.jobs);
  // codes start on a word, at most 8 bits per weight, inside the buffer;
  // escapes inside the list; the first job starts at zero, the last ends at
  // the totals
  J.bad = (J.A & 31u) != 0 || J.Bend < J.A || J.Bend - J.A > 8ull * J.len || J.Bend > a.code_bits ||
          (a.code_bits + 31) / 32 > a.code_words || J.f1end < J.f0 || J.f1end > a.n_f1esc ||
          (first && (J.A != 0 || J.f0 != 0)) ||
          (last && (J.Bend != a.code_bits || J.f1end != a.n_f1esc));
  J.bad_esc = J.e1end < J.e0 || J.e1end > a.n_esc || (first && J.e0 != 0) ||
              (last && J.e1end != a.n_esc);

  // ---- 0. loads
  J.nw = J.bad ? 0u : static_cast<uint32_t>((J.Bend - J.A) >> 5);   // <= 512
  const __amdgpu_buffer_rsrc_t rc = span(a.codes + (J.A >> 5), 4u * J.nw);
  J.v0 = __builtin_amdgcn_raw_buffer_load_b128(rc, 16u * lane, 0, 0);
  J.v1 = u32x4{0u, 0u, 0u, 0u};
  if (J.nw > 256u) J.v1 = __builtin_amdgcn_raw_buffer_load_b128(rc, 1024u + 16u * lane, 0, 0);
  J.n_escj = J.bad ? 0u : J.f1end - J.f0;
  J.re = span(a.esc_rank + J.f0, J.n_escj);
  J.ev = load_u8(J.re, 4u * lane) | (load_u8(J.re, 4u * lane + 1u) << 8) |
         (load_u8(J.re, 4u * lane + 2u) << 16) | (load_u8(J.re, 4u * lane + 3u) << 24);
  const uint32_t o = 32u * lane;   // the lane's first weight in the job
  J.live = o < J.len;
  J.row_local = 0;
  J.col = o;
  uint32_t tile = lane >> 2;
  if (C == 1) {
    J.row_local = __umulhi(o, a.col_recip);
    J.col = o - J.row_local * cols;
    tile = J.row_local * T + (J.col >> 7);
  }
  J.w = load_u8(span(a.width + t0, J.bad ? 0u : ntiles), tile);
  if (!J.live) J.w = 0;
  // rows that start inside the job (short rows): their index entries
  J.row_anchor = 0;
  J.row_f1 = 0;
  J.row_esc = 0;
  J.row_start = C == 1 && J.live && lane > 0 && J.col == 0;
  if (C == 1) {
    const uint64_t r = J.c0 + min(J.row_local, J.cnt - 1u);
    J.row_anchor = a.anchor[r];
    J.row_f1 = a.f1_pre[r];
    J.row_esc = a.esc_pre[r];
  }
}

// Decode a loaded job and write its nibbles and side-list entries.
__device__ __forceinline__ void f1_finish(const F1Args& a, const uint8_t* exp_of_rank, F1Job& J,
                                          uint32_t lane, uint32_t* words, uint32_t* esc_words,
                                          uint32_t* nib_words) {
  const uint32_t C = a.chunks_per_row, n = a.n;
  const uint8_t* escs = reinterpret_cast<const uint8_t*>(esc_words);
  wave_sync_lds();   // the previous job of this wave is done with the LDS
  *reinterpret_cast<u32x4*>(words + 4u * lane) = J.v0;
  if (J.nw > 256u) *reinterpret_cast<u32x4*>(words + 256u + 4u * lane) = J.v1;
  esc_words[lane] = J.ev;

  // ---- 1. the lane's first word
  const uint32_t w = J.w;
  const uint32_t w_incl = f1_scan(w);
  const uint32_t lw = w_incl - w;
  bool bad = J.bad || w > 8u || (static_cast<uint64_t>(f1_lane63(w_incl)) << 5) != J.Bend - J.A;
  if (J.row_start) bad = bad || J.row_anchor != J.A + (static_cast<uint64_t>(lw) << 5);
  if (__any(bad)) {
    f1_flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  wave_sync_lds();

  // ---- 2. the lane's 32 codes
  const uint32_t* g = words + lw;
  uint32_t out[4] = {0u, 0u, 0u, 0u};
  uint32_t esc = 0, big = 0;
  if (w == 3u && n >= 7u)
    decode_w3(g, out, esc);
  else if (w == 2u && n >= 3u)
    decode_w2(g, out, esc);
  else if (w == 1u)
    decode_w1(g, out, esc);
  else if (w == 4u && n >= 15u)
    decode_w4(g, out, esc);
  else if (w != 0u)
    decode_checked(g, w, n, out, esc, big, bad);
  uint32_t* nb = nib_words + 4u * lane;
  *reinterpret_cast<u32x4*>(nb) = u32x4{out[0], out[1], out[2], out[3]};

  // ---- 3. escapes: place in the escape bytes, patch the nibbles
  const uint32_t ne = __popc(esc);
  const uint32_t e_incl = f1_scan(ne);
  const uint32_t e_before = e_incl - ne;
  bad = bad || f1_lane63(e_incl) != J.n_escj;
  if (J.row_start) bad = bad || J.row_f1 != J.f0 + e_before;
  if (__any(bad)) {
    f1_flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  const uint32_t esc_code = (1u << w) - 1u, esc_nib = min(esc_code, 15u);
  const bool staged = J.n_escj <= static_cast<uint32_t>(kEscStage);
  uint32_t side = big;   // weights whose rank is >= 15, in weight order
  {
    uint32_t m = esc, k = e_before;
    while (m) {
      const uint32_t i = __builtin_ctz(m);
      m &= m - 1u;
      const uint32_t rank = staged ? static_cast<uint32_t>(escs[k]) : load_u8(J.re, k);
      ++k;
      bad = bad || rank < esc_code || rank >= n;
      side |= (rank >= 15u ? 1u : 0u) << i;
      atomicAdd(nb + (i >> 3), (min(rank, 15u) - esc_nib) << nib_shift(i));
    }
  }
  if (__any(bad)) {
    f1_flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }

  // ---- R4 side list: ranks >= 15, in weight order
  const uint32_t nr = __popc(side);
  const uint32_t r_incl = f1_scan(nr);
  const uint32_t r_before = r_incl - nr;
  bool bad_esc = J.bad_esc || J.e1end - J.e0 != f1_lane63(r_incl);
  if (J.row_start) bad_esc = bad_esc || J.row_esc != J.e0 + r_before;
  if (__any(bad_esc)) {
    f1_flag(a.status, BINADE_DEV_CORRUPT_ESC, lane);
  } else if (J.e1end != J.e0) {
    uint32_t m = side, k = J.e0 + r_before;
    const uint32_t col_base = C > 1 ? 32u * lane : J.col;
    while (m) {
      const uint32_t i = __builtin_ctz(m);
      m &= m - 1u;
      uint32_t rank;
      if ((esc >> i) & 1u) {
        const uint32_t e = e_before + __popc(esc & ((1u << i) - 1u));
        rank = staged ? static_cast<uint32_t>(escs[e]) : load_u8(J.re, e);
      } else {
        rank = code_at(g, w, i);
      }
      a.esc[k++] = (static_cast<uint32_t>(exp_of_rank[rank & 0xFFu]) << 16) | (col_base + i);
    }
  }

  // ---- 4. the lane's 16 nibble bytes
  if (J.live)
    *reinterpret_cast<u32x4*>(a.nib + (J.fb >> 1) + 16u * lane) = *reinterpret_cast<const u32x4*>(nb);
}

// kJobs consecutive jobs per wave, every job's loads issued before the first
// is decoded. One job per wave is what runs: two and four measured 3% and
// 35-40% slower (the loads of later jobs gained nothing, the registers they
// hold cost waves).
template <int kJobs>
__global__ __launch_bounds__(64 * kF1Waves) void f1_to_r4_kernel(F1Args args) {
  __shared__ __align__(16) uint32_t code_lds[kF1Waves][kCodeWords];
  __shared__ __align__(16) uint32_t esc_lds[kF1Waves][kEscStage / 4];
  __shared__ __align__(16) uint32_t nib_lds[kF1Waves][64 * 4];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const F1Args& a = *(const F1Args*)kp;
  const uint8_t* exp_of_rank = (const uint8_t*)kp + offsetof(F1Args, exp_of_rank);
  const uint32_t j0 = (blockIdx.x * kF1Waves + wave) * kJobs;
  F1Job J[kJobs];
#pragma unroll
  for (int i = 0; i < kJobs; ++i)
    if (j0 + i < static_cast<uint64_t>(a.jobs)) f1_load(a, j0 + i, lane, J[i]);
#pragma unroll
  for (int i = 0; i < kJobs; ++i)
    if (j0 + i < static_cast<uint64_t>(a.jobs))
      f1_finish(a, exp_of_rank, J[i], lane, code_lds[wave], esc_lds[wave], nib_lds[wave]);
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int32_t binade_f1_to_r4(const binade_f1* in, binade_r4* out,
                                   uint32_t* dev_status, void* stream) {
  if (in == nullptr || out == nullptr || in->rows <= 0 || in->cols <= 0 || in->n == 0 ||
      in->n > 256)
    return BINADE_EINVAL;
  if (in->cols % 32 != 0 || in->cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  if (in->sm == nullptr || in->width == nullptr || in->codes == nullptr ||
      in->anchor == nullptr || in->f1_pre == nullptr || in->esc_pre == nullptr ||
      (in->n_f1esc > 0 && in->esc_rank == nullptr) || out->nib == nullptr ||
      (in->n_esc > 0 && out->esc == nullptr) || in->code_words == 0)
    return BINADE_EINVAL;
  if (!aligned16(in->sm) || !aligned16(out->nib) ||
      (reinterpret_cast<uintptr_t>(in->codes) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(in->anchor) & 7u) != 0)
    return BINADE_EUNSUPPORTED;
  if (in->n_esc > 0xFFFFFFFFull || in->n_f1esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  const int64_t C = (in->cols + BINADE_CHUNK - 1) / BINADE_CHUNK;
  if (in->rows * C >= (1ll << 31)) return BINADE_EUNSUPPORTED;

  out->rows = in->rows;
  out->cols = in->cols;
  out->sm = in->sm;
  out->esc_pre = in->esc_pre;
  out->n_esc = in->n_esc;
  for (int r = 0; r < 16; ++r)
    out->lut[r] = (r < 15 && static_cast<uint32_t>(r) < in->n) ? in->exp_of_rank[r] : 0;

  F1Args a{};
  a.width = in->width;
  a.codes = in->codes;
  a.esc_rank = in->esc_rank;
  a.anchor = in->anchor;
  a.f1_pre = in->f1_pre;
  a.esc_pre = in->esc_pre;
  a.nib = out->nib;
  a.esc = out->esc;
  a.status = dev_status;
  a.code_bits = in->code_bits;
  a.code_words = in->code_words;
  a.n_f1esc = in->n_f1esc;
  a.n_esc = in->n_esc;
  a.rows = in->rows;
  a.cols = static_cast<int32_t>(in->cols);
  a.n = in->n;
  a.tiles_per_row = static_cast<uint32_t>((in->cols + kF1Tile - 1) / kF1Tile);
  a.chunks_per_row = static_cast<uint32_t>(C);
  if (C > 1) {
    a.jobs = in->rows * C;
    a.chunk_recip = static_cast<uint32_t>((1ull << 32) / static_cast<uint64_t>(C) + 1);
  } else {
    const int64_t G = BINADE_CHUNK / in->cols;
    a.job_rows = static_cast<uint32_t>(G);
    a.col_recip = static_cast<uint32_t>(((1ull << 32) + in->cols - 1) / in->cols);
    a.jobs = (in->rows + G - 1) / G;
  }
  for (int r = 0; r < 256; ++r) a.exp_of_rank[r] = in->exp_of_rank[r];
  const int64_t blocks = (a.jobs + kF1Waves - 1) / kF1Waves;
  if (blocks > 0x7FFFFFFFll) return BINADE_EUNSUPPORTED;
  hipLaunchKernelGGL(f1_to_r4_kernel<1>, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kF1Waves),
                     0, static_cast<hipStream_t>(stream), a);
  return launch_status();
}
