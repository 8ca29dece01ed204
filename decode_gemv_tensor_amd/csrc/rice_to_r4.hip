// Format 2 (Rice-coded ranks) -> R4 runtime layout, on the GPU at load.
//
// "Binade" package page (pypi.org/project/binade), intro and "How it works":
// the file stores ranks in Rice codes (~10.75 bits per weight); at load a
// GPU kernel rewrites them as R4: a 4-bit code per rank, with the few
// large ranks sent to a side list.
// "Lossless BF16 weight compression" page, "Best measured configuration":
// a decoder with per-block lengths found by a warp prefix sum and its output
// staged on chip is what made the Huffman exponent decoder fast; the same
// two ideas are used here, with the lengths found from the bits themselves.
//
// One wave decodes a job of at most 4096 weights: two row-chunks of one row
// when rows are longer than a chunk, else 2 * (2048 / cols) whole rows. A
// job is made of one or two runs (one row-chunk, or 2048 / cols rows).
//
// Byte-table path (Rice k = 1, tables of at least 15 exponents, jobs whose
// unary bits fit 8128 bits and whose chunk starts are at least 128 weights
// apart; the tensors of LLM layers), one job at a time:
//  Each lane takes a contiguous range of unary bytes (up to 16). One LDS
//  table entry per byte value gives, for the codes that end in that byte,
//  their q << k packed as nibbles, the first code's zeros inside the byte,
//  and the zeros left over after the last code; the zeros carried in from
//  earlier bytes only touch the first code. A lane's first weight index
//  comes from a wave prefix sum of its byte range's one bits, its carried
//  zeros from a wave prefix maximum of the last one-bit positions. The
//  nibbles go, in weight order, into a 2 KiB LDS buffer by OR; each lane
//  then reads two 32-weight tiles back, puts them in R4 nibble order, adds
//  the remainder bits (an LDS table spreads 8 of them to their nibbles) and
//  writes 16 bytes per tile. A code whose rank may reach 15 takes a rare
//  branch that computes the rank exactly and records the escape in LDS.
//  The job's bounds, escape prefixes and inner chunk starts are loaded
//  first, then its words.
//
// General path (every other job), run by run:
//  Phase 1: the lanes load the chunk's unary words (each weight's code ends
//   in exactly one 1 bit) into LDS and popcount them; a wave prefix sum turns
//   the counts into weight indices, and the lane holding the terminator of
//   weight 32m-1 records where lane tile m starts.
//  Phase 2: lane l decodes its 32 weights from LDS, 8 per read: a 32-bit
//   window at the group's start bit (two LDS words, one funnel shift) holds
//   the 8 codes, each ending at the window's lowest remaining 1 bit; rank =
//   q << k | remainder bits (prefetched from global memory during phase 1).
//   The loop has no branches: a lane's single escape is found from the
//   largest (rank, index) it saw; only a lane with a code longer than its
//   window, two escapes or a rank outside the table decodes again exactly.
//  Each lane writes its 16 nibble bytes with one 16-byte store, so a chunk's
//  output is one contiguous, coalesced 1 KiB. Escapes (rank >= 15) wait in
//  LDS (8 per lane) until a prefix sum gives their place in the side list; a
//  lane with more escapes writes them in a second, exact pass.
#include <hip/hip_runtime.h>

#include <cstring>

#include "binade.h"
#include "device_common.h"


namespace binade {
namespace {

using namespace dev;

constexpr int kWavesPerBlock = 4;
// waves per SIMD the register budget must allow (launch bound)
#ifndef BINADE_DECODE_MIN_WAVES
#define BINADE_DECODE_MIN_WAVES 1
#endif
#ifndef BINADE_DECODE_GROUP
#define BINADE_DECODE_GROUP 4
#endif
constexpr int kWalkGroup = BINADE_DECODE_GROUP;   // byte-table entries a lane loads ahead
constexpr int kStageWords = 384;     // unary words staged per run (6 bits/weight)
constexpr int kEscSlots = 7;         // escapes kept per lane in LDS
constexpr int kByteSlots = 2;        // escapes kept per lane (byte-table path)
constexpr int kJobWeights = 2 * kChunk;            // weights per job, at most
constexpr uint32_t kByteMaxBits = 8192 - 64;       // unary bits per job (byte-table path)
// LDS per wave (words). General path: staged unary words, 64 words of lane
// tile starts, then the escape slots. Byte-table path: the job's unary
// words (plus look-ahead), its remainder words, the nibble buffer and the
// escape slots.
constexpr int kGeneralWords = (kStageWords + 4) + 64;
// Byte-table path: the stage area holds the job's unary words until every
// lane has its bits; then its first 128 words hold the escape counters and
// the next 128 the escape slots.
constexpr int kByteStage = 256 + 4;
constexpr int kByteCtrOff = 0;                      // 2 x 64 escape counters
constexpr int kByteSlotOff = 128;                   // kByteSlots x 64 escape slots
constexpr int kByteRem = kByteStage;                // 128 remainder words
constexpr int kByteNib = kByteRem + 128;            // 4096 nibbles + 4 words
constexpr int kWaveWords = kByteNib + kJobWeights / 8 + 4;
// 8 blocks of 4 waves per CU: LDS (160 KiB) holds them
static_assert(8 * (kWavesPerBlock * kWaveWords * 4 + 256 * 20) <= 160 * 1024, "LDS per block");
static_assert(256 + 4 <= kByteStage && kByteSlotOff + kByteSlots * 64 <= kByteStage,
              "byte path stage area");
static_assert(kGeneralWords + kEscSlots * 64 <= kWaveWords, "general path LDS");
static_assert(kByteNib % 4 == 0 && kWaveWords % 4 == 0, "16-byte aligned LDS regions");

// Per byte value b of the unary plane and Rice k (0 or 1): the codes that end
// in b (each ends in a one bit; bit 0 is the earliest). Entry words:
//  [0] (q << k) of the 2nd, 3rd, ... code in nibbles 1, 2, ... (nibble 0 is
//      left 0: the first code also has zeros carried in from earlier bytes)
//  [1] the first code's zeros inside b, << k; kNoCode if b has no one bit
//  [2] 4 * (codes ending in b): nibble bits the byte adds
//  [3] zeros after b's last one bit, << k: the carry out (INT32_MAX if b == 0,
//      so that min(carry in + (8 << k), [3]) is the carry out either way)
// spread[r]: the 8 remainder bits r of weights 8g .. 8g+7 placed at the low
// bit of each weight's nibble in R4 order (weight i -> byte i % 4, high
// nibble for i >= 4).
constexpr int32_t kNoCode = -(1 << 30);
// Both tables for k = 1 (the byte-table path's k), built at compile time and
// copied into each block's LDS at its start.
struct ByteTables {
  uint32_t lut[256][4];
  uint32_t spread[256];
};

__host__ __device__ constexpr ByteTables make_byte_tables() {
  constexpr uint32_t k = 1;
  ByteTables t{};
  for (uint32_t b = 0; b < 256; ++b) {
    uint32_t nib = 0, m = 0, first = 0, prev = 0;
    for (uint32_t i = 0; i < 8; ++i) {
      if (((b >> i) & 1u) == 0u) continue;
      if (m == 0)
        first = i;
      else
        nib |= ((i - prev - 1u) << k) << (4u * m);
      prev = i;
      ++m;
    }
    t.lut[b][0] = nib;
    t.lut[b][1] = m ? first << k : static_cast<uint32_t>(kNoCode);
    t.lut[b][2] = 4u * m;
    t.lut[b][3] = m ? (7u - prev) << k : 0x7FFFFFFFu;
    uint32_t v = 0;
    for (uint32_t i = 0; i < 8; ++i) v |= ((b >> i) & 1u) << (8u * (i & 3u) + 4u * (i >> 2));
    t.spread[b] = v;
  }
  return t;
}

__device__ const ByteTables kByteTables = make_byte_tables();

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
  // jobs (one per wave): two row-chunks of one row when C = ceil(cols /
  // 2048) > 1, else 2G whole rows (G = 2048 / cols); a job is the runs
  // (one row-chunk, or G rows) sub_rows row-chunks apiece
  uint32_t chunks_per_row;  // C
  uint32_t pairs_per_row;   // P = ceil(C / 2) when C > 1
  uint32_t p_recip;         // ceil(2^32 / P) when P > 1: j / P = mulhi(j, p_recip), or one less
  uint32_t job_rows;        // 2G when C == 1
  uint32_t sub_rows;        // row-chunks per run: 1 (C > 1) or G
  int32_t sub_len;          // weights per full run: 2048 or G * cols
  uint32_t unit;            // distance between row-chunk starts in a job: 2048 or cols
  uint32_t unit_recip;      // ceil(2^32 / unit): i / unit = mulhi(i, unit_recip) for i <= 4096
  int64_t jobs;
  // the exponents of ranks 15 .. n-1 (only escapes look them up) sit in
  // the launch's argument pool; esc_tbl: byte offset of rank 15's, from the
  // start of the launch's arguments
  uint32_t esc_tbl;
};

// v mod chunk_mod, chunk_mod being the row-chunk width (2048) or, for rows
// shorter than a chunk, the row length: a mask in the first case.
__device__ __forceinline__ uint32_t mod_chunk(uint32_t v, uint32_t chunk_mod) {
  return chunk_mod == static_cast<uint32_t>(kChunk) ? (v & (kChunk - 1u)) : v % chunk_mod;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then row 15 / lane 31 broadcasts carry the
// row totals across rows.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  constexpr int kRowShr = 0x110, kBcast15 = 0x142, kBcast31 = 0x143;
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 8, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0u, v, kBcast31, 0xC, 0xF, false);
  return v;
}

// Inclusive prefix maximum over the 64 lanes (same DPP pattern as the sum).
__device__ __forceinline__ int32_t wave_inclusive_max(int32_t v) {
  constexpr int kRowShr = 0x110, kBcast15 = 0x142, kBcast31 = 0x143;
  constexpr int kLow = -0x7FFFFFFF - 1;
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, kRowShr + 1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, kRowShr + 2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, kRowShr + 4, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, kRowShr + 8, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, kBcast15, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(kLow, v, kBcast31, 0xC, 0xF, false));
  return v;
}

// The value of lane l - 1 (lane 0 gets first).
__device__ __forceinline__ int32_t wave_shift_up(int32_t v, int32_t first) {
  constexpr int kWaveShr1 = 0x138;
  return __builtin_amdgcn_update_dpp(first, v, kWaveShr1, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return __builtin_amdgcn_readlane(v, 63);
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

// Reads unary bits from a word source (LDS or global) through a 64-bit
// buffer whose bit 0 is the next unread bit.
template <bool kLds>
struct BitReader {
  const uint32_t* src;   // LDS words (relative) or global words (absolute)
  uint64_t cap;          // words readable (global) / staged (LDS)
  uint64_t buf;
  uint32_t have;         // valid bits in buf
  uint64_t next;         // index of the next word to append
  uint32_t nxt;          // prefetched word `next`
  uint64_t pos;          // bit position of buf's bit 0

  __device__ __forceinline__ uint32_t word(uint64_t i) const {
    return i < cap ? src[i] : 0u;
  }
  __device__ __forceinline__ void init(uint64_t bitpos) {
    const uint64_t w = bitpos >> 5;
    const uint32_t off = static_cast<uint32_t>(bitpos & 31u);
    buf = ((static_cast<uint64_t>(word(w + 1)) << 32) | word(w)) >> off;
    have = 64u - off;
    next = w + 2;
    nxt = word(next);
    pos = bitpos;
  }
  // keep at least 33 valid bits
  __device__ __forceinline__ void top_up() {
    if (have < 33u) {
      buf |= static_cast<uint64_t>(nxt) << have;
      have += 32u;
      ++next;
      nxt = word(next);
    }
  }
  // exact: zeros before the next 1 bit (the 1 is consumed); > 255 = corrupt
  __device__ __forceinline__ uint32_t unary() {
    uint32_t q = 0;
    for (;;) {
      top_up();
      const uint32_t lo = static_cast<uint32_t>(buf);
      if (lo != 0u) {
        const uint32_t t = __builtin_ctz(lo);
        buf >>= (t + 1u);
        have -= t + 1u;
        pos += t + 1u;
        return q + t;
      }
      q += 32u;
      buf >>= 32;
      have -= 32u;
      pos += 32u;
      if (q > 255u) return q;
    }
  }
};

// Exact serial decode of one lane tile (32 weights): fills out[4] with
// nibbles, and writes escapes either to the LDS slots (emit == false; the
// count may exceed the slots) or to the side list at esc_at (emit == true).
// An escape's position is (run_off + i) mod chunk_mod. Returns false on a
// corrupt code.
template <bool kLds>
__device__ bool decode_tile_exact(BitReader<kLds>& br, const RiceArgs& a,
                                  const uint8_t* a_table, uint64_t rem_bit, uint32_t run_off,
                                  uint32_t chunk_mod, uint32_t (&out)[4],
                                  uint32_t& n_esc_lane, uint32_t* slots,
                                  bool emit, uint32_t* esc_at) {
  const uint32_t k = a.k;
  out[0] = out[1] = out[2] = out[3] = 0;
  n_esc_lane = 0;
  for (int i = 0; i < 32; ++i) {
    const uint32_t q = br.unary();
    if (q > 255u) return false;
    uint32_t remv = 0;
    if (k > 0) {
      const uint64_t b = rem_bit + static_cast<uint64_t>(i) * k;
      const uint64_t w = b >> 5;
      const uint32_t off = static_cast<uint32_t>(b & 31u);
      const uint64_t two = (static_cast<uint64_t>(load_word(a.rem, w + 1, a.rem_words)) << 32) |
                           load_word(a.rem, w, a.rem_words);
      remv = static_cast<uint32_t>(two >> off) & ((1u << k) - 1u);
    }
    const uint32_t r = (q << k) | remv;
    if (r >= a.n) return false;
    const uint32_t sh = 8u * ((i & 7) & 3) + 4u * ((i & 7) >> 2);
    out[i >> 3] |= (r < 15u ? r : 15u) << sh;
    if (r >= 15u) {
      const uint32_t ent = (static_cast<uint32_t>(a_table[r & 0xFFu]) << 16) | mod_chunk(run_off + i, chunk_mod);
      if (emit)
        esc_at[n_esc_lane] = ent;
      else if (n_esc_lane < kEscSlots)
        slots[n_esc_lane * 64] = ent;
      ++n_esc_lane;
    }
  }
  return true;
}

// A wave's job: consecutive row-chunks [c0, c0 + cnt), weights
// [fb, fb + len) (len <= 4096), made of up to two runs.
struct Job {
  int64_t c0;
  int64_t cnt;
  int64_t fb;
  int32_t len;
};

// A run of row-chunks: one row-chunk when rows are longer than a chunk,
// else G = 2048 / cols whole rows.
struct Run {
  int64_t c0;      // first row-chunk
  int64_t cnt;     // row-chunks in the run
  int64_t fb;      // flat index of the first weight
  int32_t len;     // weights in the run (multiple of 32, <= 2048)
};

// The job j (wave-uniform) of a tensor; all arithmetic on scalars.
__device__ __forceinline__ void job_of(const RiceArgs& a, int64_t j, Job& job) {
  if (a.chunks_per_row == 1u) {
    const int64_t G2 = a.job_rows;
    job.c0 = j * G2;
    job.cnt = min(G2, a.n_chunks - job.c0);
    job.fb = job.c0 * a.cols;
    job.len = static_cast<int32_t>(job.cnt) * a.cols;
  } else {
    const uint32_t C = a.chunks_per_row, P = a.pairs_per_row;
    const uint32_t j32 = static_cast<uint32_t>(j);   // < 2^31
    uint32_t row = j32;
    if (P > 1u) {
      row = __umulhi(j32, a.p_recip);
      if (row * P > j32) --row;
    }
    const uint32_t jp = j32 - row * P;
    job.c0 = static_cast<int64_t>(row) * C + 2u * jp;
    job.cnt = min(2u, C - 2u * jp);
    job.fb = static_cast<int64_t>(row) * a.cols + static_cast<int64_t>(jp) * kJobWeights;
    job.len = min(kJobWeights, a.cols - static_cast<int32_t>(jp) * kJobWeights);
  }
}

// Run i (0 or 1) of a job; false if the job has no such run.
__device__ __forceinline__ bool run_of(const RiceArgs& a, const Job& job, int i, Run& run) {
  const int64_t g = a.sub_rows;
  run.c0 = job.c0 + i * g;
  run.cnt = min(g, job.cnt - i * g);
  run.fb = job.fb + static_cast<int64_t>(i) * a.sub_len;
  run.len = min(a.sub_len, job.len - i * a.sub_len);
  return run.cnt > 0;
}

// What a wave loads first: the run's bounds, its first two unary words per
// lane and the lane's remainder words.
struct Prefetch {
  uint64_t A, B;
  uint32_t w0, w1;
  uint32_t rw0, rw1;
};

__device__ __forceinline__ void prefetch_bounds(const RiceArgs& a, const Run& run,
                                                Prefetch& pf) {
  pf.A = a.anchor[run.c0];
  pf.B = a.anchor[run.c0 + run.cnt];
}

__device__ __forceinline__ void prefetch_words(const RiceArgs& a, const Run& run,
                                               int lane, Prefetch& pf) {
  // uniform bases and a 32-bit lane offset; words past the plane read as 0
  // (only the run's own words: up to the word holding its last bit)
  const uint64_t wA = pf.A >> 5;
  const uint64_t left = a.unary_words > wA ? a.unary_words - wA : 0ull;
  const uint64_t need = pf.B > pf.A ? ((pf.B - 1) >> 5) - wA + 1 : 0ull;
  const uint64_t lim = need < left ? need : left;
  const uint32_t avail = lim > 0x7FFFFFFFull ? 0x7FFFFFFFu : static_cast<uint32_t>(lim);
  const uint32_t* ub = a.unary + wA;
  const uint32_t wi = 2u * static_cast<uint32_t>(lane);
  pf.w0 = wi < avail ? ub[wi] : 0u;
  pf.w1 = wi + 1u < avail ? ub[wi + 1u] : 0u;
  pf.rw0 = pf.rw1 = 0;
  if (a.k == 1 || a.k == 2) {
    // remainder bits of lane tile l start at bit (fb + 32 l) * k, a word
    // boundary since fb is a multiple of 32
    const uint64_t r0 = (static_cast<uint64_t>(run.fb) * a.k) >> 5;
    const uint64_t rleft = a.rem_words > r0 ? a.rem_words - r0 : 0ull;
    const uint64_t rneed = static_cast<uint64_t>(run.len >> 5) * a.k;   // the run's tiles
    const uint64_t rlim = rneed < rleft ? rneed : rleft;
    const uint32_t ravail = rlim > 0x7FFFFFFFull ? 0x7FFFFFFFu : static_cast<uint32_t>(rlim);
    const uint32_t* rb = a.rem + r0;
    const uint32_t ri = static_cast<uint32_t>(lane) * a.k;
    pf.rw0 = ri < ravail ? rb[ri] : 0u;
    if (a.k == 2) pf.rw1 = ri + 1u < ravail ? rb[ri + 1u] : 0u;
  }
}

// Decode one run (phases 1 and 2, escapes, nibble store).
__device__ __forceinline__ void decode_run(const RiceArgs& a, const uint8_t* table,
                                           const Run& run, const Prefetch& pf, int lane,
                                           uint32_t* stage, uint32_t* tstart,
                                           uint32_t* slots) {
  const int64_t c = run.c0, cnt = run.cnt;
  const int32_t Lc = run.len;
  const int32_t T = Lc >> 5;
  const uint64_t A = pf.A, B = pf.B;
  const uint64_t fb = static_cast<uint64_t>(run.fb);
  const uint32_t k = a.k;
  if (B < A + static_cast<uint64_t>(Lc) || B - A > 256ull * Lc ||
      B > a.unary_words * 32ull) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  const uint64_t rem_bit = (fb + 32ull * lane) * k;

  // ---- phase 1: stage the unary words, find where each lane tile starts
  const uint64_t wA = A >> 5;
  const uint64_t nw = ((B - 1) >> 5) - wA + 1;
  const bool staged = nw <= static_cast<uint64_t>(kStageWords);
  if (lane == 0) tstart[0] = static_cast<uint32_t>(A & 31u);
  uint32_t carry = 0;
  bool last_bit_set = false;
  for (uint64_t base = 0; base < nw; base += 128) {
    const uint64_t wi = base + 2u * lane;     // this lane's two words
    uint32_t w0 = 0, w1 = 0;
    if (base == 0) {
      w0 = wi < nw ? pf.w0 : 0u;
      w1 = wi + 1 < nw ? pf.w1 : 0u;
    } else {
      if (wi < nw) w0 = load_word(a.unary, wA + wi, a.unary_words);
      if (wi + 1 < nw) w1 = load_word(a.unary, wA + wi + 1, a.unary_words);
    }
    if (staged) {
      if (wi < nw) stage[wi] = w0;
      if (wi + 1 < nw) stage[wi + 1] = w1;
    }
    if (wi == 0) w0 &= 0xFFFFFFFFu << (A & 31u);
    const uint32_t top = static_cast<uint32_t>((B - 1) & 31u);
    if (wi == nw - 1) {
      w0 &= 0xFFFFFFFFu >> (31u - top);
      last_bit_set = (w0 >> top) & 1u;
    } else if (wi + 1 == nw - 1) {
      w1 &= 0xFFFFFFFFu >> (31u - top);
      last_bit_set = (w1 >> top) & 1u;
    }
    const uint32_t pc0 = __popc(w0);
    const uint32_t pc = pc0 + __popc(w1);
    const uint32_t incl = wave_inclusive_sum(pc);
    const uint32_t s_first = carry + incl - pc;
    // weight indices 32m-1 ending in these 64 bits (at most two)
    for (uint32_t s = s_first | 31u; s < s_first + pc; s += 32u) {
      const uint32_t m = (s + 1) >> 5;
      const uint32_t n = s - s_first;
      const uint32_t bit = n < pc0 ? select_bit(w0, n) : 32u + select_bit(w1, n - pc0);
      if (static_cast<int32_t>(m) < T) tstart[m] = static_cast<uint32_t>(wi * 32ull + bit + 1);
    }
    carry += lane63(incl);
  }
  if (staged && lane < 4) stage[nw + lane] = 0;  // reader look-ahead
  const bool ends_in_one = __any(last_bit_set);
  if (carry != static_cast<uint32_t>(Lc) || !ends_in_one) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  wave_sync();
  // Rows that start inside the run (short rows): lane m checks the row
  // starting at its tile (rows starting inside a tile, when cols % 32 == 0
  // but the tile holds two rows, do not occur: 32 | cols).
  int64_t my_chunk = -1;
  if (cnt > 1 && lane > 0 && lane < T && (32 * lane) % a.cols == 0)
    my_chunk = c + (32 * lane) / a.cols;
  if (cnt > 1) {
    const bool off = my_chunk >= 0 &&
                     static_cast<uint64_t>(tstart[lane]) + wA * 32ull != a.anchor[my_chunk];
    if (__any(off)) {
      flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
      return;
    }
  }

  // ---- phase 2: lane l decodes weights 32l .. 32l+31 of the run
  uint32_t out[4] = {0, 0, 0, 0};
  uint32_t n_esc_lane = 0;
  bool bad = false;
  const uint32_t run_off = 32u * lane;
  const uint32_t chunk_mod = a.cols < kChunk ? static_cast<uint32_t>(a.cols) : kChunk;
  const uint32_t start = lane < T ? tstart[lane] : 0u;
  if (lane < T) {
    if (staged && k <= 2) {
      // Fast path, branch-free: 8 weights per LDS read. A 32-bit window at
      // the group's start bit holds the group's 8 codes unless one is long
      // (then the window holds fewer than 8 one bits); code j ends at the
      // window's j-th lowest 1 bit, found and then cleared. Every rank is
      // exact; nibbles take min(rank, 15).
      uint32_t p = start;
      uint32_t fewest = 32;
      uint32_t rmax = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w = p >> 5;
        uint32_t cur = __builtin_amdgcn_alignbit(stage[w + 1], stage[w], p & 31u);
        fewest = min(fewest, static_cast<uint32_t>(__popc(cur)));
        const uint32_t rwd = (k == 2 && d >= 2) ? pf.rw1 : pf.rw0;
        uint32_t prev = 0xFFFFFFFFu;
        uint32_t o = 0;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint32_t t = static_cast<uint32_t>(__builtin_ctz(cur | 0x80000000u));
          const uint32_t q = t + ~prev;                 // t - prev - 1
          prev = t;
          cur &= cur - 1u;
          const uint32_t remv = __builtin_amdgcn_ubfe(rwd, ((8 * d + jj) * k) & 31u, k);
          const uint32_t r = (q << k) | remv;
          rmax = max(rmax, r);
          o |= min(r, 15u) << (8u * (jj & 3) + 4u * (jj >> 2));
        }
        p += prev + 1u;
        out[d] = o;
      }
      bool exact = fewest < 8u || rmax >= a.n;
      if (!exact && rmax >= 15u) {
        // one escape: the tile's only nibble 15, and its rank is the largest
        int found = -1;
        uint32_t n15 = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t v = out[d];
          const uint32_t ones = v & (v >> 1) & (v >> 2) & (v >> 3) & 0x11111111u;
          n15 += __popc(ones);
          if (ones != 0u && found < 0) {
            const uint32_t bp = __builtin_ctz(ones);          // 0, 4, 8, ... 28
            found = 8 * d + static_cast<int>((bp >> 3) + 4 * ((bp >> 2) & 1u));
          }
        }
        if (n15 == 1u) {
          slots[0] = (static_cast<uint32_t>(table[rmax & 0xFFu]) << 16) | mod_chunk(run_off + found, chunk_mod);
          n_esc_lane = 1;
        } else {
          exact = true;
        }
      }
      if (exact) {
        BitReader<true> lr{stage, nw + 4, 0, 0, 0, 0, 0};
        lr.init(start);
        bad = !decode_tile_exact(lr, a, table, rem_bit, run_off, chunk_mod, out, n_esc_lane, slots,
                                 false, nullptr);
      }
    } else {
      if (staged) {
        BitReader<true> lr{stage, nw + 4, 0, 0, 0, 0, 0};
        lr.init(start);
        bad = !decode_tile_exact(lr, a, table, rem_bit, run_off, chunk_mod, out, n_esc_lane, slots,
                                 false, nullptr);
      } else {
        BitReader<false> gr{a.unary, a.unary_words, 0, 0, 0, 0, 0};
        gr.init(wA * 32ull + start);
        bad = !decode_tile_exact(gr, a, table, rem_bit, run_off, chunk_mod, out, n_esc_lane, slots,
                                 false, nullptr);
      }
    }
  }
  if (__any(bad)) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }

  // ---- escapes: place in the side list after a prefix sum over lanes
  const uint32_t e0 = a.esc_pre[c];
  const uint32_t e1 = a.esc_pre[c + cnt];
  uint32_t before, total;
  if (__ballot(n_esc_lane > 1u) == 0) {
    const uint64_t has = __ballot(n_esc_lane != 0u);
    before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(has >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(has), 0u));
    total = __popcll(has);
  } else {
    const uint32_t incl = wave_inclusive_sum(n_esc_lane);
    before = incl - n_esc_lane;
    total = lane63(incl);
  }
  const bool esc_off = my_chunk >= 0 && a.esc_pre[my_chunk] != e0 + before;
  if (e1 < e0 || e1 - e0 != total || e1 > a.n_esc || __any(esc_off)) {
    flag(a.status, BINADE_DEV_CORRUPT_ESC, lane);
  } else if (n_esc_lane > 0) {
    uint32_t* dst = a.esc + (e0 + before);
    if (n_esc_lane <= static_cast<uint32_t>(kEscSlots)) {
      for (uint32_t i = 0; i < n_esc_lane; ++i) dst[i] = slots[i * 64];
    } else {
      // more escapes than slots: decode the tile again, writing them out
      uint32_t o2[4], cnt2 = 0;
      if (staged) {
        BitReader<true> lr{stage, nw + 4, 0, 0, 0, 0, 0};
        lr.init(start);
        decode_tile_exact(lr, a, table, rem_bit, run_off, chunk_mod, o2, cnt2, slots, true, dst);
      } else {
        BitReader<false> gr{a.unary, a.unary_words, 0, 0, 0, 0, 0};
        gr.init(wA * 32ull + start);
        decode_tile_exact(gr, a, table, rem_bit, run_off, chunk_mod, o2, cnt2, slots, true, dst);
      }
    }
  }
  if (lane < T) {
    uint4* dst = reinterpret_cast<uint4*>(a.nib + (fb >> 1) + 16u * lane);
    *dst = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// LDS words by byte address (the 32-bit offset in the workgroup's LDS).
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ __forceinline__ uint32_t lds_address(const uint32_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u32*)p));
}
__device__ __forceinline__ void lds_or(uint32_t addr, uint32_t v) {
  __hip_atomic_fetch_or((lds_u32*)addr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_and(uint32_t addr, uint32_t v) {
  __hip_atomic_fetch_and((lds_u32*)addr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Nibbles of 8 weights in weight order (weight i at bits 4i) -> R4 order
// (weight i in byte i % 4, high nibble for i >= 4).
__device__ __forceinline__ uint32_t to_r4_order(uint32_t n) {
  // low nibbles: weights 0..3 from bytes of n and n >> 4; high nibbles:
  // weights 4..7 from bytes of n << 4 and n
  const uint32_t lo = __builtin_amdgcn_perm(n >> 4, n, 0x05010400u);
  const uint32_t hi = __builtin_amdgcn_perm(n << 4, n, 0x03070206u);
  return (lo & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);
}

// LDS atomics on a lane's own words (no other lane touches them).
__device__ __forceinline__ uint32_t lds_add_rtn(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add((lds_u32*)lds_address(p), v, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Escape bookkeeping of a lane in LDS, so that the rare branch of the walk
// changes no register the common path carries: ctr[0] counts the lane's
// escapes (bit 31: a rank outside the table), ctr[64] those before the
// weight limit; slots[64 i] holds escape i (index << 8 | rank), i < 3.
constexpr uint32_t kBadRank = 0x80000000u;

// One lane's walk over kSteps bytes of unary bits (byte j is byte j % 4 of
// x[j / 4], bit 0 first; bits past the lane's range are zero). c: zeros
// carried in, << K. sb: 4 * index of the lane's first weight in the job.
// kEmit == false: ORs the nibbles (q << K, 15 at most; remainders come
// later) into the nibble buffer at LDS byte address nb and records escapes
// in ctr / slots. kEmit == true: writes the escapes to dst (n_esc counts
// them).
template <uint32_t K, int kSteps, bool kEmit>
__device__ __forceinline__ void byte_walk(const uint32_t (&x)[4], int32_t c, uint32_t sb,
                                          const uint4* lut, const uint32_t* remw, uint32_t n,
                                          uint32_t nb, uint32_t* ctr, uint32_t* slots,
                                          uint32_t limit, const uint8_t* table,
                                          uint32_t chunk_mod, uint32_t* dst, uint32_t& n_esc) {
  constexpr int32_t kThr = K ? 14 : 15;   // smallest q << K whose rank can be >= 15
  constexpr int kGroup = kSteps < kWalkGroup ? kSteps : kWalkGroup;   // table entries loaded ahead
#pragma unroll
  for (int j0 = 0; j0 < kSteps; j0 += kGroup) {
    uint4 e[kGroup];
#pragma unroll
    for (int jj = 0; jj < kGroup; ++jj) {
      const int j = j0 + jj;
      if (j < kSteps) e[jj] = lut[__builtin_amdgcn_ubfe(x[j >> 2], 8 * (j & 3), 8)];
    }
#pragma unroll
    for (int jj = 0; jj < kGroup; ++jj) {
      if (j0 + jj >= kSteps) break;
      const int32_t t = static_cast<int32_t>(e[jj].y) + c;     // first code's q << K
      if (t >= kThr) {
        // rare: the first code may be an escape
        const uint32_t idx = sb >> 2;
        const uint32_t rank =
            static_cast<uint32_t>(t) | (K ? ((remw[idx >> 5] >> (idx & 31u)) & 1u) : 0u);
        if (rank >= 15u) {
          if (kEmit) {
            if (rank < n)
              dst[n_esc++] = (static_cast<uint32_t>(table[rank]) << 16) | mod_chunk(idx, chunk_mod);
          } else {
            const uint32_t pos = lds_add_rtn(ctr, rank < n ? 1u : kBadRank) & ~kBadRank;
            if (pos < static_cast<uint32_t>(kByteSlots)) slots[pos * 64] = (idx << 8) | rank;
            if (idx < limit) lds_add_rtn(ctr + 64, 1u);
          }
        }
      }
      if (!kEmit) {
        const uint32_t v = e[jj].x | static_cast<uint32_t>(min(max(t, 0), 15));
        // v << (sb % 32) over the word holding nibble sb / 4 and the next
        const uint64_t w = static_cast<uint64_t>(v) << (sb & 31u);
        // nb + 4 * (sb / 32), as two instructions
        uint32_t addr;
        asm("v_bfe_u32 %0, %1, 5, 27\n\tv_lshl_add_u32 %0, %0, 2, %2"
            : "=&v"(addr)
            : "v"(sb), "v"(nb));
        lds_or(addr, static_cast<uint32_t>(w));
        lds_or(addr + 4u, static_cast<uint32_t>(w >> 32));
      }
      // zeros carried to the next byte: those after its last code, or all 8
      c = min(c + static_cast<int32_t>(8u << K), static_cast<int32_t>(e[jj].w));
      sb += e[jj].z;
    }
  }
}

// Bit position (0..127) of the n-th (0-based) set bit of x[0..3]; x has more
// than n set bits.
__device__ __forceinline__ uint32_t select_bit4(const uint32_t (&x)[4], uint32_t n) {
  uint32_t base = 0;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const uint32_t pcq = __popc(x[q]);
    if (n < pcq) return base + select_bit(x[q], n);
    n -= pcq;
    base += 32u;
  }
  return base + select_bit(x[3], n);
}

// One job's loads: its bit bounds (uniform) and escape prefixes, four unary
// words and two remainder words per lane.
struct JobLoads {
  uint64_t A, B;      // anchors of the first and one-past-last row-chunk
  uint32_t e0, e1;    // escape prefixes of the same
  uint64_t ia;        // anchor of row-chunk c0 + 1 + lane (lane < cnt - 1)
  uint32_t ie;        // escape prefix of the same
  uint4 w;            // unary words A/32 + 4*lane .. +3 (0 past the job)
  uint32_t rw0, rw1;  // remainder words of tiles lane and lane + 64 (k = 1)
};

// The job's bounds, and for a job of several row-chunks the anchors and
// escape prefixes of its inner chunk starts (lane i: chunk c0 + 1 + i), all
// requested before any other work.
__device__ __forceinline__ void job_bounds(const RiceArgs& a, const Job& job, int lane,
                                           JobLoads& L) {
  L.A = a.anchor[job.c0];
  L.B = a.anchor[job.c0 + job.cnt];
  L.e0 = a.esc_pre[job.c0];
  L.e1 = a.esc_pre[job.c0 + job.cnt];
  L.ia = 0;
  L.ie = 0;
  if (job.cnt > 1) {
    const int64_t inner = job.c0 + 1 + min(static_cast<int64_t>(lane), job.cnt - 2);
    L.ia = a.anchor[inner];
    L.ie = a.esc_pre[inner];
  }
  L.A = uniform64(static_cast<int64_t>(L.A));
  L.B = uniform64(static_cast<int64_t>(L.B));
}

// The job's words (B > A): uniform bases and 32-bit lane offsets; only the
// job's own words are read.
__device__ __forceinline__ void job_words(const RiceArgs& a, const Job& job, int lane,
                                          JobLoads& L) {
  const uint64_t wA = L.A >> 5;
  const uint64_t left = a.unary_words > wA ? a.unary_words - wA : 0ull;
  const uint64_t need = ((L.B - 1) >> 5) - wA + 1;
  const uint32_t avail = static_cast<uint32_t>(need < left ? need : left);   // <= 255
  const uint32_t* ub = a.unary + wA;
  const uint32_t wi = 4u * static_cast<uint32_t>(lane);
  if (wi + 3u < avail) {
    L.w = make_uint4(ub[wi], ub[wi + 1u], ub[wi + 2u], ub[wi + 3u]);
  } else {
    L.w.x = wi < avail ? ub[wi] : 0u;
    L.w.y = wi + 1u < avail ? ub[wi + 1u] : 0u;
    L.w.z = wi + 2u < avail ? ub[wi + 2u] : 0u;
    L.w.w = 0u;
  }
  // remainder bits (k = 1) of the job's tile t: word fb / 32 + t
  const uint64_t r0 = static_cast<uint64_t>(job.fb) >> 5;
  const uint64_t rleft = a.rem_words > r0 ? a.rem_words - r0 : 0ull;
  const uint64_t rneed = static_cast<uint64_t>(job.len >> 5);
  const uint32_t ravail = static_cast<uint32_t>(rneed < rleft ? rneed : rleft);   // <= 128
  const uint32_t* rb = a.rem + r0;
  L.rw0 = static_cast<uint32_t>(lane) < ravail ? rb[lane] : 0u;
  L.rw1 = static_cast<uint32_t>(lane) + 64u < ravail ? rb[lane + 64] : 0u;
}

// Decode one job on the byte-table path, Rice k = K. Lane l takes the job's
// unary bits [spl*8*l, spl*8*(l+1)) (spl bytes, 1..16, counted from the
// job's first bit).
template <uint32_t K>
__device__ __forceinline__ void decode_job_bytes(const RiceArgs& a, const uint8_t* table,
                                                 const Job& job, const JobLoads& f, int lane,
                                                 uint32_t* lds, const uint4* lut,
                                                 const uint32_t* spread) {
  uint32_t* stage = lds;
  uint32_t* remw = lds + kByteRem;
  uint32_t* nibw = lds + kByteNib;
  uint32_t* slots = lds + kByteSlotOff + lane;
  uint32_t* ctr = lds + kByteCtrOff + lane;
  const int64_t cnt = job.cnt;
  const int32_t Lc = job.len;
  const int32_t T = Lc >> 5;
  const uint64_t A = f.A, B = f.B;
  if (B < A + static_cast<uint64_t>(Lc) || B > a.unary_words * 32ull) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  const uint64_t wA = A >> 5;
  const uint32_t uA = static_cast<uint32_t>(A & 31u);
  const uint32_t nbits = static_cast<uint32_t>(B - A);            // <= kByteMaxBits
  const uint32_t Brel = uA + nbits;                                // end, from word wA
  const uint32_t nw = (Brel + 31u) >> 5;                           // <= 255
  const uint32_t spl = (((nbits + 7u) >> 3) + 63u) >> 6;           // 1..16

  // ---- stage the job's unary words (words past the job are already zero;
  // the bits past its end in its last word are cleared; the bits before its
  // first bit are never read), zeros up to word 259, and its remainder
  // words; clear the nibble buffer
  {
    reinterpret_cast<uint4*>(stage)[lane] = f.w;
    if (lane < 4) stage[256 + lane] = 0u;
    if (lane == 0)
      lds_and(lds_address(stage + (nw - 1u)), 0xFFFFFFFFu >> (31u - ((Brel - 1u) & 31u)));
    remw[lane] = f.rw0;
    remw[64 + lane] = f.rw1;
    reinterpret_cast<uint4*>(nibw)[lane] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(nibw)[64 + lane] = make_uint4(0u, 0u, 0u, 0u);
    if (lane == 0) reinterpret_cast<uint4*>(nibw)[128] = make_uint4(0u, 0u, 0u, 0u);
  }
  wave_sync();

  // ---- the lane's bits
  const uint32_t bit0 = uA + 8u * spl * static_cast<uint32_t>(lane);
  const uint32_t wi = bit0 >> 5, off = bit0 & 31u;
  uint32_t x[4];
  {
    uint32_t sw[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) sw[q] = stage[wi + q];
    const uint32_t bits = 8u * spl;   // 8 .. 128
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t xq = __builtin_amdgcn_alignbit(sw[q + 1], sw[q], off);
      const uint32_t lo = 32u * q;
      const uint32_t keep =
          bits <= lo ? 0u : (bits - lo >= 32u ? 0xFFFFFFFFu : (1u << (bits - lo)) - 1u);
      x[q] = xq & keep;
    }
  }
  const uint32_t last_word = stage[(Brel - 1u) >> 5];
  // the unary words are read: the escape counters take over their area (a
  // wave's LDS operations complete in order)
  ctr[0] = 0u;
  ctr[64] = 0u;
  const uint32_t pc = __popc(x[0]) + __popc(x[1]) + __popc(x[2]) + __popc(x[3]);
  const uint32_t incl = wave_inclusive_sum(pc);
  const uint32_t s_first = incl - pc;
  if (lane63(incl) != static_cast<uint32_t>(Lc) ||
      ((last_word >> ((Brel - 1u) & 31u)) & 1u) == 0u) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  // zeros carried into the lane: from its first bit back to the last one bit
  // of an earlier lane (every lane's bits start after the job's first bit)
  const int32_t top = x[3]   ? 127 - __clz(x[3])
                      : x[2] ? 95 - __clz(x[2])
                      : x[1] ? 63 - __clz(x[1])
                             : 31 - __clz(x[0]);
  const int32_t last = pc ? static_cast<int32_t>(bit0) + top : static_cast<int32_t>(uA) - 1;
  const int32_t prev = wave_shift_up(wave_inclusive_max(last), static_cast<int32_t>(uA) - 1);
  const int32_t c_in = (static_cast<int32_t>(bit0) - prev - 1) << K;
  const uint32_t sb0 = 4u * s_first;

  // a row-chunk that starts inside the job: the lane holding the one bit
  // that ends the chunk's previous weight checks the chunk's anchor and
  // escape prefix (a lane holds at most 128 codes and chunk starts are at
  // least 128 weights apart, so at most one per lane)
  uint32_t limit = 0;
  if (cnt > 1) {
    const uint32_t r = __umulhi(s_first, a.unit_recip) + 1u;   // first start > s_first
    const uint32_t start = r * a.unit;
    if (pc > 0u && start <= s_first + pc && start < static_cast<uint32_t>(Lc)) limit = start;
  }

  const uint32_t chunk_mod = a.cols < kChunk ? static_cast<uint32_t>(a.cols) : kChunk;
  const uint32_t nb = lds_address(nibw);
  uint32_t unused = 0;
  if (spl <= 4u)
    byte_walk<K, 4, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table, chunk_mod,
                           nullptr, unused);
  else if (spl <= 8u)
    byte_walk<K, 8, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table, chunk_mod,
                           nullptr, unused);
  else if (spl <= 10u)
    byte_walk<K, 10, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table,
                            chunk_mod, nullptr, unused);
  else if (spl <= 11u)   // 3072-weight jobs at k = 1 (≈ 650 bytes)
    byte_walk<K, 11, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table,
                            chunk_mod, nullptr, unused);
  else if (spl <= 12u)
    byte_walk<K, 12, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table,
                            chunk_mod, nullptr, unused);
  else if (spl <= 14u)
    byte_walk<K, 14, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table,
                            chunk_mod, nullptr, unused);
  else
    byte_walk<K, 16, false>(x, c_in, sb0, lut, remw, a.n, nb, ctr, slots, limit, table,
                            chunk_mod, nullptr, unused);
  const uint32_t cw = ctr[0];
  const bool ok = (cw & kBadRank) == 0u;
  const uint32_t n_esc_lane = cw & ~kBadRank;
  const uint32_t n_before = ctr[64];
  // the inner chunk start's anchor and escape prefix, from the lane that
  // loaded them (chunk c0 + r: lane r - 1)
  const int inner = limit != 0u ? static_cast<int>(__umulhi(limit, a.unit_recip)) - 1 : 0;
  const uint32_t ia_lo = __shfl(static_cast<uint32_t>(f.ia), inner);
  const uint32_t ia_hi = __shfl(static_cast<uint32_t>(f.ia >> 32), inner);
  const uint32_t ie = __shfl(f.ie, inner);
  bool off_anchor = false;
  if (limit != 0u) {
    const uint32_t pos = select_bit4(x, limit - 1u - s_first);   // that weight's one bit
    off_anchor = (static_cast<uint64_t>(ia_hi) << 32 | ia_lo) != wA * 32ull + bit0 + pos + 1u;
  }
  if (__any(!ok || off_anchor)) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM, lane);
    return;
  }
  wave_sync();

  // ---- R4 nibbles: read back 32 weights per tile, R4 order, remainder bits
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = lane + 64 * h;
    if (t < T) {
      const uint4 nn = reinterpret_cast<const uint4*>(nibw)[t];
      uint4 o;
      o.x = to_r4_order(nn.x);
      o.y = to_r4_order(nn.y);
      o.z = to_r4_order(nn.z);
      o.w = to_r4_order(nn.w);
      if (K) {
        const uint32_t rw = h ? f.rw1 : f.rw0;
        o.x |= spread[rw & 0xFFu];
        o.y |= spread[(rw >> 8) & 0xFFu];
        o.z |= spread[(rw >> 16) & 0xFFu];
        o.w |= spread[rw >> 24];
      }
      *reinterpret_cast<uint4*>(a.nib + (static_cast<uint64_t>(job.fb) >> 1) + 16u * t) = o;
    }
  }

  // ---- escapes: place in the side list after a prefix sum over lanes
  const uint32_t e0 = f.e0;
  const uint32_t e1 = f.e1;
  uint32_t before, total;
  if (__ballot(n_esc_lane > 1u) == 0) {
    const uint64_t has = __ballot(n_esc_lane != 0u);
    before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(has >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(has), 0u));
    total = __popcll(has);
  } else {
    const uint32_t esc_incl = wave_inclusive_sum(n_esc_lane);
    before = esc_incl - n_esc_lane;
    total = lane63(esc_incl);
  }
  const bool esc_off = limit != 0u && ie != e0 + before + n_before;
  if (e1 < e0 || e1 - e0 != total || e1 > a.n_esc || __any(esc_off)) {
    flag(a.status, BINADE_DEV_CORRUPT_ESC, lane);
  } else if (n_esc_lane > 0) {
    uint32_t* dst = a.esc + (e0 + before);
    if (n_esc_lane <= static_cast<uint32_t>(kByteSlots)) {
      for (uint32_t i = 0; i < n_esc_lane; ++i) {
        const uint32_t ent = slots[i * 64];
        dst[i] = (static_cast<uint32_t>(table[ent & 0xFFu]) << 16) | mod_chunk(ent >> 8, chunk_mod);
      }
    } else {
      // more escapes than slots: walk the bytes again, writing them out
      uint32_t n2 = 0;
      byte_walk<K, 16, true>(x, c_in, sb0, lut, remw, a.n, 0u, nullptr, nullptr, 0u, table,
                             chunk_mod, dst, n2);
    }
  }
}

// The byte tables into LDS, one entry of each per thread of the 256-thread
// block.
__device__ __forceinline__ void load_byte_tables(uint4* lut, uint32_t* spread) {
  const uint32_t t = threadIdx.x;
  lut[t] = *reinterpret_cast<const uint4*>(kByteTables.lut[t]);
  spread[t] = kByteTables.spread[t];
  __syncthreads();
}

// Up to 16 tensors per launch: tensor i owns the launch's jobs
// [first_job[i], first_job[i+1]). Their escape exponents share one pool.
constexpr int kMaxDecodeBatch = 16;
constexpr int kEscPool = 1024;
struct RiceBatch {
  RiceArgs item[kMaxDecodeBatch];
  uint32_t first_job[kMaxDecodeBatch + 1];
  int32_t count;
  uint8_t pool[kEscPool];
};
static_assert(sizeof(RiceBatch) <= 4096, "kernel arguments of one decode launch");

// One wave per job (job g of the launch is wave g). The tensor's arguments
// are read in place from the argument segment (an index into a by-value
// argument array would be copied to scratch memory). The job's bounds, then
// its words, are requested before any other work.
__global__ __launch_bounds__(256, BINADE_DECODE_MIN_WAVES) void rice_to_r4_batch_kernel(RiceBatch b) {
  __shared__ __align__(16) uint32_t lds[kWavesPerBlock][kWaveWords];
  __shared__ uint4 lut[256];
  __shared__ uint32_t spread[256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t g = uniform(blockIdx.x * kWavesPerBlock + static_cast<uint32_t>(wave));
  const bool live = g < b.first_job[b.count];
  int i = 0;
#pragma unroll
  for (int t = 1; t < kMaxDecodeBatch; ++t)
    if (t < b.count && g >= b.first_job[t]) i = t;
  i = uniform(i);
  const size_t off = offsetof(RiceBatch, item) + static_cast<size_t>(i) * sizeof(RiceArgs);
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const RiceArgs& a = *(const RiceArgs*)(kp + off);
  // table[r] for 15 <= r < n (every lookup is of an escape whose rank was
  // checked against n)
  const uint8_t* table = (const uint8_t*)kp + a.esc_tbl - 15;
  Job job;
  JobLoads L;
  bool bytes = false;
  if (live) {
    job_of(a, static_cast<int64_t>(g - b.first_job[i]), job);
    job_bounds(a, job, lane, L);
    bytes = a.k == 1u && a.n >= 15u && (job.cnt == 1 || a.unit >= 128u) && L.B > L.A &&
            L.B - L.A <= kByteMaxBits;
    if (bytes) job_words(a, job, lane, L);
  }
  load_byte_tables(lut, spread);
  if (!live) return;
  if (bytes) {
    decode_job_bytes<1>(a, table, job, L, lane, lds[wave], lut, spread);
    return;
  }
  // general path: each run of the job
  for (int r = 0; r < 2; ++r) {
    Run run;
    if (!run_of(a, job, r, run)) break;
    Prefetch pf;
    prefetch_bounds(a, run, pf);
    prefetch_words(a, run, lane, pf);
    decode_run(a, table, run, pf, lane, lds[wave], lds[wave] + (kStageWords + 4),
               lds[wave] + kGeneralWords + lane);
    wave_sync();   // the next run reuses the same LDS
  }
}


// ------------------------------------------------------------ streamed path
// The byte table walked over long spans. One wave decodes a span of
// consecutive row-chunks, which the format keeps contiguous in weights, in
// unary bits and in escapes, in rounds of 64 * 8 * kSpl unary bits: lane l
// takes the round's bits [8 kSpl l, 8 kSpl (l + 1)), requested one round
// ahead; a wave prefix sum of their one bits places its codes and a wave
// prefix maximum of the last one bits gives the zeros carried into it; the
// byte walk then ORs the nibbles into an LDS buffer that holds the codes not
// yet written. Whole batches of 64 tiles leave the buffer in R4 order with
// their remainder bits; the unfinished tiles move to its front. The span's
// bounds, escape count and setup are paid once per span instead of once per
// 4096 weights. Every row-chunk start inside the span is checked in the round
// that holds its previous weight's code: the lane holding that code's one
// bit gets the start as its limit (its escapes before it are counted), and a
// scalar pass compares the one bit's position with the chunk's anchor and
// the escapes before it with the chunk's escape prefix.
#ifndef BINADE_STREAM_SPL
#define BINADE_STREAM_SPL 8
#endif
constexpr int kSpl = BINADE_STREAM_SPL;            // unary bytes per lane and round
constexpr int kSplWords = kSpl / 4;
constexpr uint32_t kRoundBits = 64u * 8u * kSpl;   // unary bits per round
#ifndef BINADE_STREAM_WAVES
#define BINADE_STREAM_WAVES 4
#endif
constexpr int kStreamWaves = BINADE_STREAM_WAVES;  // waves per block
// LDS per wave (words): the nibble buffer (the unfinished tile, then up to
// one code per bit of a round, and the 64-bit OR's spill word), two escape
// counters and the escape slots of each lane, and the remainder words of the
// round's codes (a rare escape reads its bit there)
constexpr int kSNibWords = 4 + static_cast<int>(kRoundBits / 8) + 4;
constexpr int kSCtr = kSNibWords;
constexpr int kSSlots = kSCtr + 128;
constexpr int kSRemWords = static_cast<int>(kRoundBits / 32) + 8;
constexpr int kSRem = kSSlots + kByteSlots * 64;
constexpr int kSWaveWords = kSRem + kSRemWords;
constexpr int kRemRegs = (kSRemWords + 63) / 64;   // remainder words per lane and round
constexpr int kFlushRegs = static_cast<int>(kRoundBits / 32 / 64);   // tile batches per round
static_assert(kSpl == 8 || kSpl == 16, "two or four unary words per lane and round");
static_assert(kSNibWords % 4 == 0, "16-byte aligned LDS regions");
static_assert(kSRemWords % 8 == 0 && kSRemWords >= kRoundBits / 32 + 1, "remainder stage");
static_assert(kStreamWaves * kSWaveWords * 4 + 256 * 20 <= 64 * 1024, "LDS per block");

struct StreamArgs {
  const uint32_t* unary;
  const uint32_t* rem;
  const uint64_t* anchor;
  const uint32_t* esc_pre;
  uint8_t* nib;
  uint32_t* esc;
  uint32_t* status;
  uint64_t unary_words;
  uint32_t n_esc;         // side-list entries (< 2^32)
  uint32_t total;         // rows * cols (< 2^31)
  uint32_t cols;          // >= 128
  uint32_t C;             // row-chunks per row
  uint32_t n_chunks;      // rows * C
  uint32_t cols_recip;    // ceil(2^32 / cols)
  uint32_t span_chunks;   // row-chunks per span
  uint32_t n;             // ranks in the table
  uint32_t esc_tbl;       // byte offset of rank 15's exponent from the arguments
};

// A buffer resource over bytes [base, base + bytes): loads beyond it return
// zero and access nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_span(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Which check of the streamed path set the status word (a debugging build
// only; BINADE_STREAM_DEBUG adds bit 8 + site).
__device__ __forceinline__ uint32_t stream_site(int site) {
#ifdef BINADE_STREAM_DEBUG
  return 1u << (8 + site);
#else
  (void)site;
  return 0u;
#endif
}

// w / cols for w < 2^31: the reciprocal's quotient is exact or one too large.
__device__ __forceinline__ uint32_t div_cols(uint32_t w, const StreamArgs& a) {
  uint32_t q = __umulhi(w, a.cols_recip);
  if (q * a.cols > w) --q;
  return q;
}

// Column of weight w inside its row-chunk.
__device__ __forceinline__ uint32_t col_in_chunk(uint32_t w, const StreamArgs& a) {
  return (w - div_cols(w, a) * a.cols) & (kChunk - 1u);
}

// Weight index of row-chunk c's first weight (c <= n_chunks).
__device__ __forceinline__ uint32_t chunk_weight(uint32_t c, const StreamArgs& a) {
  if (c >= a.n_chunks) return a.total;
  const uint32_t row = c / a.C;
  return row * a.cols + (c - row * a.C) * static_cast<uint32_t>(kChunk);
}

// The row-chunk starts of a span, one after the other (uniform).
struct ChunkCursor {
  uint32_t w;      // weight index of the start
  uint32_t c;      // its row-chunk
  uint32_t col;    // its column in its row
};
__device__ __forceinline__ void next_chunk(ChunkCursor& k, const StreamArgs& a) {
  k.c += 1u;
  const uint32_t step = min(static_cast<uint32_t>(kChunk), a.cols - k.col);
  k.w += step;
  k.col += step;
  if (k.col == a.cols) k.col = 0u;
}

// The byte walk of one lane over its kSpl bytes (x: bit 0 first). As
// byte_walk with k = 1, the codes indexed from the nibble buffer's start;
// a rare escape reads its remainder bit from the staged words remw, code
// idx's word being remw[idx / 32 + roff].
template <bool kEmit>
__device__ __forceinline__ void stream_walk(const uint32_t (&x)[kSplWords], int32_t c,
                                            uint32_t sb, const uint4* lut, const uint32_t* remw,
                                            int32_t roff, uint32_t n, uint32_t nb,
                                            uint32_t* ctr, uint32_t* slots, uint32_t limit,
                                            const uint8_t* table, const StreamArgs& a,
                                            uint32_t wbase, uint32_t* dst, uint32_t& n_esc) {
  constexpr int kGroup = 4;
#pragma unroll
  for (int j0 = 0; j0 < kSpl; j0 += kGroup) {
    uint4 e[kGroup];
#pragma unroll
    for (int jj = 0; jj < kGroup; ++jj) {
      const int j = j0 + jj;
      e[jj] = lut[__builtin_amdgcn_ubfe(x[j >> 2], 8 * (j & 3), 8)];
    }
#pragma unroll
    for (int jj = 0; jj < kGroup; ++jj) {
      const int32_t t = static_cast<int32_t>(e[jj].y) + c;     // first code's q << 1
      if (t >= 14) {
        // rare: the first code may be an escape
        const uint32_t idx = sb >> 2;
        const uint32_t rb = (remw[static_cast<int32_t>(idx >> 5) + roff] >> (idx & 31u)) & 1u;
        const uint32_t rank = static_cast<uint32_t>(t) | rb;
        if (rank >= 15u) {
          if (kEmit) {
            if (rank < n)
              dst[n_esc++] =
                  (static_cast<uint32_t>(table[rank]) << 16) | col_in_chunk(wbase + idx, a);
          } else {
            const uint32_t pos = lds_add_rtn(ctr, rank < n ? 1u : kBadRank) & ~kBadRank;
            if (pos < static_cast<uint32_t>(kByteSlots)) slots[pos * 64] = (idx << 8) | (rank & 0xFFu);
            if (idx < limit) lds_add_rtn(ctr + 64, 1u);
          }
        }
      }
      if (!kEmit) {
        const uint32_t v = e[jj].x | static_cast<uint32_t>(min(max(t, 0), 15));
        const uint64_t w = static_cast<uint64_t>(v) << (sb & 31u);
        uint32_t addr;
        asm("v_bfe_u32 %0, %1, 5, 27\n\tv_lshl_add_u32 %0, %0, 2, %2"
            : "=&v"(addr)
            : "v"(sb), "v"(nb));
        lds_or(addr, static_cast<uint32_t>(w));
        lds_or(addr + 4u, static_cast<uint32_t>(w >> 32));
      }
      c = min(c + 16, static_cast<int32_t>(e[jj].w));
      sb += e[jj].z;
    }
  }
}

// Nibbles of 8 weights in weight order -> R4 order (weight i in byte i % 4,
// high nibble for i >= 4): the low nibbles come from bytes 0, 1 of n and of
// n >> 4, the high ones from bytes 1, 2 of n >> 4 and 2, 3 of n.
__device__ __forceinline__ uint32_t r4_order(uint32_t n) {
  const uint32_t r = n >> 4;
  const uint32_t lo = __builtin_amdgcn_perm(r, n, 0x05010400u);
  const uint32_t hi = __builtin_amdgcn_perm(r, n, 0x03060205u);
  return (lo & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);
}

// One tile of the nibble buffer in R4 order with its remainder word.
__device__ __forceinline__ uint4 r4_tile(uint4 nn, uint32_t rw, const uint32_t* spread) {
  uint4 o;
  o.x = r4_order(nn.x) | spread[rw & 0xFFu];
  o.y = r4_order(nn.y) | spread[(rw >> 8) & 0xFFu];
  o.z = r4_order(nn.z) | spread[(rw >> 16) & 0xFFu];
  o.w = r4_order(nn.w) | spread[rw >> 24];
  return o;
}

// The uniform facts of a span.
struct Span {
  uint64_t A, B;        // its unary bits [A, B)
  uint64_t R0;          // A rounded down to 64 bits: the first round's first bit
  uint32_t W0, W1;      // its weights [W0, W1)
  uint32_t E0, E1;      // its escapes [E0, E1)
  uint32_t ntiles;      // (W1 - W0) / 32
  uint32_t c0;          // its first row-chunk
};

// The state a span's rounds carry (uniform).
struct SpanState {
  uint32_t r;           // the round's first bit, from R0
  int32_t prev_last;    // last one bit before the round, from the round's first bit
  uint32_t last_one;    // one past the last one bit seen, from R0 (0: none)
  uint32_t P;           // codes before the round
  uint32_t T;           // first tile not yet written
  uint32_t esc_done;    // escapes written
  ChunkCursor next;     // the next row-chunk start to check
};

// Resources of a span: its unary words from R0 on and its remainder words.
struct SpanRes {
  __amdgpu_buffer_rsrc_t unary;
  __amdgpu_buffer_rsrc_t rem;
  uint64_t anchor;      // lane i: anchor of row-chunk c0 + i (i < span_chunks <= 64)
  uint32_t esc_pre;     // lane i: its escape prefix
};

// The lane's two unary words of the round starting r bits after R0 (zero
// past the span's words). The offset goes in the range-checked operand.
__device__ __forceinline__ void round_words(const SpanRes& rs, uint32_t r, uint32_t lane_off,
                                            uint32_t (&x)[kSplWords]) {
  if (kSplWords == 2) {
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  rs.unary, lane_off + (r >> 3), 0, 0));
    x[0] = v.x;
    x[kSplWords - 1] = v.y;
  } else {
    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs.unary, lane_off + (r >> 3), 0, 0));
    x[0] = v.x;
    x[1] = v.y;
    x[2 % kSplWords] = v.z;
    x[3 % kSplWords] = v.w;
  }
}

// The remainder word of span tile t (zero past the span).
__device__ __forceinline__ uint32_t tile_rem(const SpanRes& rs, uint32_t t) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs.rem, 4u * t, 0, 0);
}

// The remainder words of span tiles t0 + 64 q + lane.
__device__ __forceinline__ void round_rems(const SpanRes& rs, uint32_t t0, uint32_t lane,
                                           uint32_t (&r)[kRemRegs]) {
#pragma unroll
  for (int q = 0; q < kRemRegs; ++q) r[q] = tile_rem(rs, t0 + 64u * q + lane);
}

// Round status: go on, the span's last round is done, or corrupt planes
// (the status word is set).
enum : int { kRoundNext = 0, kRoundLast = 1, kRoundBad = 2 };

// One round of a span. xr, rr: this round's unary and remainder words
// (already requested); the next round's are requested into xn, rn.
__device__ __forceinline__ int stream_round(const StreamArgs& a, const Span& sp, const SpanRes& rs,
                                            SpanState& st, const uint32_t (&xr)[kSplWords],
                                            uint32_t (&xn)[kSplWords],
                                            const uint32_t (&rr)[kRemRegs],
                                            uint32_t (&rn)[kRemRegs], const uint8_t* table,
                                            int lane, uint32_t* lds, const uint4* lut,
                                            const uint32_t* spread) {
  uint32_t* nibw = lds;
  uint32_t* ctr = lds + kSCtr + lane;
  uint32_t* slots = lds + kSSlots + lane;
  uint32_t* remw = lds + kSRem;
  const uint32_t r = st.r;
  const uint32_t T = st.T;
  const uint32_t P = st.P;
  const uint64_t R = sp.R0 + r;
  const uint32_t lane_u = static_cast<uint32_t>(lane);
  // the remainder words of the round's codes: span tiles T + i at remw[i]
  // (T = P / 32: only the unfinished tile is carried from round to round).
  // A rare escape reads its bit there, and the tiles written at the end of
  // the round take their remainder words from there.
#pragma unroll
  for (int q = 0; q < kRemRegs; ++q)
    if (64 * q + lane < kSRemWords) remw[64 * q + lane] = rr[q];
  ctr[0] = 0u;
  ctr[64] = 0u;
  uint32_t x[kSplWords];
#pragma unroll
  for (int q = 0; q < kSplWords; ++q) x[q] = xr[q];
  const int32_t lbit = static_cast<int32_t>(8 * kSpl) * lane;   // lane's first bit, from R
  if (R < sp.A && lane == 0) {
    // the span's first bits sit in lane 0's words
    const uint32_t skip = static_cast<uint32_t>(sp.A - R);        // < 64
    x[0] &= skip >= 32u ? 0u : 0xFFFFFFFFu << skip;
    x[1] &= skip <= 32u ? 0xFFFFFFFFu : 0xFFFFFFFFu << (skip - 32u);   // skip < 64
  }
  const bool last_round = R + kRoundBits >= sp.B;
  if (last_round) {
    // the span ends in this round: clear the bits from B on
    const int32_t keep = static_cast<int32_t>(sp.B - R) - lbit;   // lane bits inside the span
#pragma unroll
    for (int q = 0; q < kSplWords; ++q) {
      const int32_t k = keep - 32 * q;
      x[q] &= k <= 0 ? 0u : (k >= 32 ? 0xFFFFFFFFu : (1u << k) - 1u);
    }
  }
  uint32_t pc = 0;
#pragma unroll
  for (int q = 0; q < kSplWords; ++q) pc += __popc(x[q]);
  // the next round's words
  round_words(rs, r + kRoundBits, 4u * kSplWords * lane_u, xn);

  // ---- where the lane's codes go and the zeros carried into it
  const uint32_t incl = wave_inclusive_sum(pc);
  const uint32_t n_round = lane63(incl);
  const uint32_t s_first = P + incl - pc;          // span index of the lane's first code
  int32_t top = 0;
#pragma unroll
  for (int q = 0; q < kSplWords; ++q)
    if (x[q]) top = 32 * q + 31 - static_cast<int32_t>(__clz(x[q]));
  const int32_t last = pc ? lbit + top : st.prev_last;
  const int32_t mx = wave_inclusive_max(last);
  const int32_t prev = wave_shift_up(mx, st.prev_last);
  const int32_t c_in = (lbit - prev - 1) << 1;
  const int32_t round_last = static_cast<int32_t>(lane63(static_cast<uint32_t>(mx)));
  // the next round's remainder words
  round_rems(rs, (P + n_round) >> 5, lane_u, rn);

  // ---- row-chunk starts X whose previous code X - 1 ends in this round:
  // the lane holding that code counts its escapes before X
  uint32_t limit = 0;
  {
    ChunkCursor k = st.next;
    while (k.w < sp.W1 && k.w - sp.W0 <= P + n_round) {
      const uint32_t X = k.w - sp.W0;
      const uint32_t L = __popcll(__ballot(incl <= X - 1u - P));   // lane holding code X - 1
      if (lane_u == L) limit = X;
      next_chunk(k, a);
    }
  }

  // ---- the walk
  const uint32_t base = 32u * T;                   // span index of the buffer's first code
  const int32_t roff = 0;   // T == P / 32
  const uint32_t nb = lds_address(nibw);
  uint32_t unused = 0;
  wave_sync();
  // lanes without a one bit (past the span's end in its last round) would
  // all OR into one word: they skip the walk
  if (pc != 0u)
    stream_walk<false>(x, c_in, 4u * (s_first - base), lut, remw, roff, a.n, nb, ctr, slots,
                       limit != 0u ? limit - base : 0u, table, a, sp.W0 + base, nullptr, unused);
  const uint32_t cw = ctr[0];
  const uint32_t n_esc_lane = cw & ~kBadRank;
  if (__any((cw & kBadRank) != 0u) || P + n_round > sp.W1 - sp.W0) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM | stream_site(1), lane);
    return kRoundBad;
  }

  // ---- escapes: their places in the side list
  uint32_t before, total;
  if (__ballot(n_esc_lane > 1u) == 0) {
    const uint64_t has = __ballot(n_esc_lane != 0u);
    before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(has >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(has), 0u));
    total = __popcll(has);
  } else {
    const uint32_t esc_incl = wave_inclusive_sum(n_esc_lane);
    before = esc_incl - n_esc_lane;
    total = lane63(esc_incl);
  }
  if (sp.E1 - sp.E0 - st.esc_done < total) {
    flag(a.status, BINADE_DEV_CORRUPT_ESC | stream_site(2), lane);
    return kRoundBad;
  }

  // ---- the chunk starts of this round against their anchors and escape
  // prefixes (scalar, from the lane holding each start's previous code)
  {
    const uint32_t n_before = ctr[64];
    uint32_t bad = 0;
    ChunkCursor k = st.next;
    while (k.w < sp.W1 && k.w - sp.W0 <= P + n_round) {
      const uint32_t X = k.w - sp.W0;
      const uint32_t L = __popcll(__ballot(incl <= X - 1u - P));
      // (readlane returns an int: widen through uint32_t)
      const uint32_t sl = static_cast<uint32_t>(__builtin_amdgcn_readlane(s_first, L));
      const uint32_t el = static_cast<uint32_t>(__builtin_amdgcn_readlane(before, L)) +
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(n_before, L));
      const uint32_t ci = k.c - sp.c0;   // < span_chunks
      const uint64_t ia =
          (static_cast<uint64_t>(static_cast<uint32_t>(
               __builtin_amdgcn_readlane(static_cast<uint32_t>(rs.anchor >> 32), ci))) << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(rs.anchor), ci));
      const uint32_t ie = static_cast<uint32_t>(__builtin_amdgcn_readlane(rs.esc_pre, ci));
      // the one bit ending code X - 1: bit p of lane L's bits, with X - 1 - sl
      // one bits below it
      const uint64_t p = ia - 1u - (R + 8u * kSpl * L);
      bool ok = p < 8u * kSpl;
      uint32_t below = 0;
#pragma unroll
      for (int q = 0; q < kSplWords; ++q) {
        const uint32_t wq = static_cast<uint32_t>(__builtin_amdgcn_readlane(x[q], L));
        const uint64_t lo = 32u * q;
        if (p >= lo + 32u) {
          below += __popc(wq);
        } else if (p >= lo) {
          const uint32_t b = static_cast<uint32_t>(p - lo);
          ok = ok && ((wq >> b) & 1u) != 0u;
          below += __popc(wq & ((1u << b) - 1u));
        }
      }
      if (!ok || below != X - 1u - sl)
        bad |= BINADE_DEV_CORRUPT_STREAM | stream_site(12);
      if (ie != sp.E0 + st.esc_done + el) bad |= BINADE_DEV_CORRUPT_ESC;
      next_chunk(k, a);
    }
    st.next = k;
    if (bad != 0u) {
      flag(a.status, bad | stream_site(3), lane);
      return kRoundBad;
    }
  }

  if (n_esc_lane > 0u) {
    uint32_t* dst = a.esc + (sp.E0 + st.esc_done + before);
    if (n_esc_lane <= static_cast<uint32_t>(kByteSlots)) {
      for (uint32_t i = 0; i < n_esc_lane; ++i) {
        const uint32_t ent = slots[i * 64];
        dst[i] = (static_cast<uint32_t>(table[ent & 0xFFu]) << 16) |
                 col_in_chunk(sp.W0 + base + (ent >> 8), a);
      }
    } else {
      uint32_t n2 = 0;
      stream_walk<true>(x, c_in, 4u * (s_first - base), lut, remw, roff, a.n, 0u, nullptr,
                        nullptr, 0u, table, a, sp.W0 + base, dst, n2);
    }
  }
  st.esc_done += total;
  st.P = P + n_round;
  if (n_round > 0u) st.last_one = r + static_cast<uint32_t>(round_last) + 1u;
  st.prev_last = round_last - static_cast<int32_t>(kRoundBits);
  st.r = r + kRoundBits;
  wave_sync();

  // ---- the finished tiles to R4 (at most kRoundBits / 32: a round adds at
  // most one code per bit to an unfinished tile); the unfinished one to the
  // front
  const uint32_t done = (st.P >> 5) - T;
  uint8_t* out = a.nib + (sp.W0 >> 1) + 16ull * T;
#pragma unroll
  for (int q = 0; q < kFlushRegs; ++q) {
    if (64u * q >= done) break;   // uniform
    if (64u * q + lane_u < done)
      *reinterpret_cast<uint4*>(out + 16u * (64u * q + lane_u)) =
          r4_tile(reinterpret_cast<const uint4*>(nibw)[64 * q + lane], remw[64 * q + lane], spread);
  }
  st.T = T + done;
  const uint4 cv = reinterpret_cast<const uint4*>(nibw)[done];
  wave_sync();
  // the next round ORs into zeros past the unfinished tile
  if (lane == 0) reinterpret_cast<uint4*>(nibw)[0] = cv;
#pragma unroll
  for (int q = 0; q < (kSNibWords / 4 - 1 + 63) / 64; ++q)
    if (1 + q * 64 + lane < kSNibWords / 4)
      reinterpret_cast<uint4*>(nibw)[1 + q * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);
  wave_sync();
  return last_round ? kRoundLast : kRoundNext;
}

__device__ void stream_span(const StreamArgs& a, const uint8_t* table, const Span& sp,
                            int lane, uint32_t* lds, const uint4* lut,
                            const uint32_t* spread) {
  const uint32_t nw = sp.W1 - sp.W0;                 // codes of the span, a multiple of 32
  // a valid code has at most 128 bits (rank <= 255 at k = 1)
  if (sp.B < sp.A + nw || sp.B > a.unary_words * 32ull || sp.B - sp.A > 128ull * nw) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM | stream_site(4), lane);
    return;
  }
  if (sp.E1 < sp.E0 || sp.E1 > a.n_esc) {
    flag(a.status, BINADE_DEV_CORRUPT_ESC | stream_site(5), lane);
    return;
  }
  uint32_t* nibw = lds;
#pragma unroll
  for (int q = 0; q < (kSNibWords / 4 + 63) / 64; ++q)
    if (q * 64 + lane < kSNibWords / 4)
      reinterpret_cast<uint4*>(nibw)[q * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);

  SpanRes rs;
  const uint64_t wR = sp.R0 >> 5;
  rs.unary = buffer_span(a.unary + wR, static_cast<uint32_t>(4u * (((sp.B + 31u) >> 5) - wR)));
  rs.rem = buffer_span(a.rem + (sp.W0 >> 5), 4u * sp.ntiles);
  {
    const uint32_t i = min(static_cast<uint32_t>(lane), a.span_chunks - 1u);
    const uint32_t c = min(sp.c0 + i, a.n_chunks);
    rs.anchor = a.anchor[c];
    rs.esc_pre = a.esc_pre[c];
  }
  SpanState st;
  st.r = 0;
  st.prev_last = static_cast<int32_t>(sp.A - sp.R0) - 1;   // the bit before the span
  st.last_one = 0;
  st.P = 0;
  st.T = 0;
  st.esc_done = 0;
  st.next.c = sp.c0;
  st.next.w = sp.W0;
  st.next.col = sp.W0 - div_cols(sp.W0, a) * a.cols;
  next_chunk(st.next, a);
  // two sets of word registers in turn: a round reads one while the next
  // round's words arrive in the other (no copy of a register in flight)
  const uint32_t lane_u = static_cast<uint32_t>(lane);
  uint32_t xa[kSplWords], xb[kSplWords], ra[kRemRegs], rb[kRemRegs];
  round_words(rs, 0u, 4u * kSplWords * lane_u, xa);
  round_rems(rs, 0u, lane_u, ra);
  int s;
  while (true) {
    s = stream_round(a, sp, rs, st, xa, xb, ra, rb, table, lane, lds, lut, spread);
    if (s != kRoundNext) break;
    s = stream_round(a, sp, rs, st, xb, xa, rb, ra, table, lane, lds, lut, spread);
    if (s != kRoundNext) break;
  }
  if (s == kRoundBad) return;
  if (st.P != nw || sp.R0 + st.last_one != sp.B) {
    flag(a.status, BINADE_DEV_CORRUPT_STREAM | stream_site(6), lane);
    return;
  }
  if (st.esc_done != sp.E1 - sp.E0) {
    flag(a.status, BINADE_DEV_CORRUPT_ESC | stream_site(7), lane);
    return;
  }
  // the last tiles (fewer than 64)
  const uint32_t t = st.T + lane_u;
  if (t < sp.ntiles) {
    const uint32_t rw = tile_rem(rs, t);
    *reinterpret_cast<uint4*>(a.nib + (sp.W0 >> 1) + 16ull * t) =
        r4_tile(reinterpret_cast<const uint4*>(nibw)[lane], rw, spread);
  }
}

struct StreamBatch {
  StreamArgs item[kMaxDecodeBatch];
  uint32_t first_job[kMaxDecodeBatch + 1];
  int32_t count;
  uint8_t pool[kEscPool];
};
static_assert(sizeof(StreamBatch) <= 4096, "kernel arguments of one streamed launch");

// The work of one wave: span `span` of the tensor a (when live), after the
// block has put the byte tables in LDS.
__device__ __forceinline__ void stream_wave(const StreamArgs& a, const uint8_t* table,
                                            uint32_t span, bool live,
                                            uint32_t (&lds)[kStreamWaves][kSWaveWords],
                                            uint4* lut, uint32_t* spread) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  Span sp{};
  if (live) {
    const uint32_t c0 = span * a.span_chunks;
    const uint32_t c1 = min(c0 + a.span_chunks, a.n_chunks);
    sp.A = uniform64(static_cast<int64_t>(a.anchor[c0]));
    sp.B = uniform64(static_cast<int64_t>(a.anchor[c1]));
    sp.E0 = uniform(a.esc_pre[c0]);
    sp.E1 = uniform(a.esc_pre[c1]);
    sp.R0 = sp.A & ~63ull;
    sp.W0 = chunk_weight(c0, a);
    sp.W1 = chunk_weight(c1, a);
    sp.ntiles = (sp.W1 - sp.W0) >> 5;
    sp.c0 = c0;
  }
  for (uint32_t t = threadIdx.x; t < 512u; t += 64u * kStreamWaves) {
    if (t < 256u)
      lut[t] = *reinterpret_cast<const uint4*>(kByteTables.lut[t]);
    else
      spread[t - 256u] = kByteTables.spread[t - 256u];
  }
  __syncthreads();
  if (!live) return;
  stream_span(a, table, sp, lane, lds[wave], lut, spread);
}

// One wave per span (span s of tensor i is wave first_job[i] + s).
__global__ __launch_bounds__(64 * kStreamWaves) void rice_stream_kernel(StreamBatch b) {
  __shared__ __align__(16) uint32_t lds[kStreamWaves][kSWaveWords];
  __shared__ uint4 lut[256];
  __shared__ uint32_t spread[256];
  const uint32_t g = uniform(blockIdx.x * kStreamWaves + (threadIdx.x >> 6));
  const bool live = g < b.first_job[b.count];
  int i = 0;
#pragma unroll
  for (int t = 1; t < kMaxDecodeBatch; ++t)
    if (t < b.count && g >= b.first_job[t]) i = t;
  i = uniform(i);
  const size_t off = offsetof(StreamBatch, item) + static_cast<size_t>(i) * sizeof(StreamArgs);
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const StreamArgs a = *(const StreamArgs*)(kp + off);   // uniform: held in SGPRs
  const uint8_t* table = (const uint8_t*)kp + a.esc_tbl - 15;
  stream_wave(a, table, g - b.first_job[i], live, lds, lut, spread);
}

// A decode plan in device memory: its tensors' spans in one launch. The
// plan holds first_job[count + 1] at first_off, StreamArgs[count] at
// items_off and the escape exponents their esc_tbl offsets point at; the
// status word comes with the launch.
struct PlanLaunch {
  const uint8_t* plan;
  uint32_t* status;
  uint32_t count;       // >= 1
  uint32_t spans;       // first_job[count]
  uint32_t first_off;
  uint32_t items_off;
};

// One wave per span of the plan; the wave finds its tensor by a binary
// search of first_job (uniform scalar loads).
__global__ __launch_bounds__(64 * kStreamWaves) void rice_plan_kernel(PlanLaunch p) {
  __shared__ __align__(16) uint32_t lds[kStreamWaves][kSWaveWords];
  __shared__ uint4 lut[256];
  __shared__ uint32_t spread[256];
  const uint32_t g = uniform(blockIdx.x * kStreamWaves + (threadIdx.x >> 6));
  const bool live = g < p.spans;
  const uint32_t* first = reinterpret_cast<const uint32_t*>(p.plan + p.first_off);
  uint32_t lo = 0, hi = p.count;   // first[lo] <= g < first[hi] for a live wave
  while (hi - lo > 1u) {
    const uint32_t mid = (lo + hi) >> 1;
    if (g >= uniform(first[mid])) lo = mid;
    else hi = mid;
  }
  lo = uniform(lo);
  StreamArgs a = *reinterpret_cast<const StreamArgs*>(p.plan + p.items_off +
                                                      static_cast<size_t>(lo) * sizeof(StreamArgs));
  a.status = p.status;
  const uint8_t* table = p.plan + a.esc_tbl - 15;
  stream_wave(a, table, g - uniform(first[lo]), live, lds, lut, spread);
}

}  // namespace
}  // namespace binade

using namespace binade;

namespace {

// Checks one format 2 -> R4 request and fills its kernel arguments and the
// host-visible R4 fields. Returns the number of jobs (waves) or a status.
int64_t prepare_decode(const binade_rice* in, binade_r4* out, uint32_t* dev_status,
                       RiceArgs& a) {
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
  if (n_chunks >= (1ll << 31)) return BINADE_EUNSUPPORTED;

  out->rows = in->rows;
  out->cols = in->cols;
  out->sm = in->sm;
  out->esc_pre = in->esc_pre;
  out->n_esc = in->n_esc;
  for (int r = 0; r < 16; ++r)
    out->lut[r] = (r < 15 && static_cast<uint32_t>(r) < in->n) ? in->exp_of_rank[r] : 0;

  a = RiceArgs{};
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
  a.chunks_per_row = static_cast<uint32_t>(C);
  auto recip = [](uint64_t d) {   // ceil(2^32 / d), d >= 2
    return static_cast<uint32_t>(((1ull << 32) + d - 1) / d);
  };
  if (C > 1) {
    // jobs: two row-chunks of one row (the last one alone when C is odd)
    const int64_t P = (C + 1) / 2;
    a.pairs_per_row = static_cast<uint32_t>(P);
    a.p_recip = P > 1 ? recip(static_cast<uint64_t>(P)) : 0u;
    a.sub_rows = 1;
    a.sub_len = BINADE_CHUNK;
    a.unit = BINADE_CHUNK;
    a.unit_recip = 1u << 21;   // 2^32 / 2048, exact
    a.jobs = in->rows * P;
  } else {
    // jobs: 2G whole rows, runs of G = 2048 / cols rows
    const int64_t G = BINADE_CHUNK / in->cols;
    a.job_rows = static_cast<uint32_t>(2 * G);
    a.sub_rows = static_cast<uint32_t>(G);
    a.sub_len = static_cast<int32_t>(G * in->cols);
    a.unit = static_cast<uint32_t>(in->cols);
    a.unit_recip = in->cols > 1 ? recip(static_cast<uint64_t>(in->cols)) : 0u;
    a.jobs = (in->rows + 2 * G - 1) / (2 * G);
  }
  return a.jobs;
}

}  // namespace

namespace {

int32_t launch_batch(const RiceBatch& b, hipStream_t stream) {
  const uint32_t total = b.first_job[b.count];
  if (total == 0) return BINADE_OK;
  const int64_t blocks = (static_cast<int64_t>(total) + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(rice_to_r4_batch_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * kWavesPerBlock), 0, stream, b);
  return launch_status();
}

// Decode plans: a 32-byte header (PlanHeader), first_job[count + 1], the
// tensors' StreamArgs (status cleared), then their escape exponents.
constexpr uint32_t kPlanMagic = 0x31505242u;   // "BRP1"
constexpr int32_t kMaxPlanTensors = 1 << 16;
struct PlanHeader {
  uint32_t magic;
  int32_t count;
  uint32_t spans;
  uint32_t first_off;
  uint32_t items_off;
  uint32_t pool_off;
  uint32_t bytes;       // bytes written, escape exponents included
  uint32_t reserved;
};
static_assert(sizeof(PlanHeader) == 32, "plan header");

struct PlanLayout {
  uint32_t first_off, items_off, pool_off, max_bytes;
};

PlanLayout plan_layout(int32_t count) {
  PlanLayout l;
  l.first_off = sizeof(PlanHeader);
  l.items_off = (l.first_off + 4u * static_cast<uint32_t>(count + 1) + 7u) & ~7u;
  l.pool_off = l.items_off + static_cast<uint32_t>(count) * static_cast<uint32_t>(sizeof(StreamArgs));
  l.max_bytes = l.pool_off + 241u * static_cast<uint32_t>(count);
  return l;
}

int32_t launch_plan(const PlanLaunch& p, hipStream_t stream) {
  if (p.spans == 0) return BINADE_OK;
  const int64_t blocks = (static_cast<int64_t>(p.spans) + kStreamWaves - 1) / kStreamWaves;
  hipLaunchKernelGGL(rice_plan_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * kStreamWaves), 0, stream, p);
  return launch_status();
}

int32_t launch_stream(const StreamBatch& b, hipStream_t stream) {
  const uint32_t total = b.first_job[b.count];
  if (total == 0) return BINADE_OK;
  const int64_t blocks = (static_cast<int64_t>(total) + kStreamWaves - 1) / kStreamWaves;
  hipLaunchKernelGGL(rice_stream_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * kStreamWaves), 0, stream, b);
  return launch_status();
}

// Weights per span: a launch of up to 16 tensors, and a plan's single
// launch (whose waves follow each other for the whole model, so that longer
// spans pay their setup less often with no launch tail after each group).
#ifndef BINADE_STREAM_SPAN
#define BINADE_STREAM_SPAN 16384
#endif
#ifndef BINADE_PLAN_SPAN
#define BINADE_PLAN_SPAN 32768
#endif

// The streamed path takes tensors of the byte-table kind (Rice k = 1, a table
// of at least 15 ranks) whose row-chunk starts are at least 128 weights apart
// and whose weight indices fit 31 bits. Fills its arguments from a checked
// request and returns the span count.
int64_t prepare_stream(const binade_rice* in, const RiceArgs& r, StreamArgs& s,
                       int64_t span_weights = BINADE_STREAM_SPAN) {
  // rows shorter than 1024 weights start a chunk every few hundred codes,
  // which the per-job kernel checks more cheaply
  if (in->k != 1 || in->n < 15 || in->cols < 1024) return 0;
  const int64_t tail = in->cols % BINADE_CHUNK;
  if (tail != 0 && tail < 128) return 0;
  if (in->rows * in->cols >= (1ll << 31) || in->unary_words < 1) return 0;
  s = StreamArgs{};
  s.unary = r.unary;
  s.rem = r.rem;
  s.anchor = r.anchor;
  s.esc_pre = r.esc_pre;
  s.nib = r.nib;
  s.esc = r.esc;
  s.status = r.status;
  s.unary_words = r.unary_words;
  s.n_esc = static_cast<uint32_t>(r.n_esc);
  s.total = static_cast<uint32_t>(in->rows * in->cols);
  s.cols = static_cast<uint32_t>(in->cols);
  s.C = r.chunks_per_row;
  s.n_chunks = static_cast<uint32_t>(r.n_chunks);
  s.cols_recip = static_cast<uint32_t>(((1ull << 32) + s.cols - 1) / s.cols);
  const int64_t per = s.C > 1 ? span_weights / BINADE_CHUNK : span_weights / in->cols;
  s.span_chunks = static_cast<uint32_t>(per > 64 ? 64 : per > 1 ? per : 1);
  s.n = r.n;
  return (r.n_chunks + s.span_chunks - 1) / s.span_chunks;
}

}  // namespace

extern "C" int32_t binade_rice_to_r4(const binade_rice* in, binade_r4* out,
                                     uint32_t* dev_status, void* stream) {
  return binade_rice_to_r4_batch(in, out, 1, dev_status, stream);
}

extern "C" int32_t binade_rice_to_r4_batch(const binade_rice* in, binade_r4* out,
                                           int32_t count, uint32_t* dev_status,
                                           void* stream) {
  if (count < 0 || (count > 0 && (in == nullptr || out == nullptr))) return BINADE_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // two launches fill side by side: the streamed kernel's tensors and the
  // job kernel's; each launch holds up to 16 tensors, their escape exponents
  // and fewer than 2^31 waves
  RiceBatch b{};
  StreamBatch sbat{};
  int n = 0, sn = 0;
  uint64_t jobs = 0, spans = 0;
  uint32_t pool = 0, spool = 0;   // bytes of the escape pools in use
  for (int32_t i = 0; i < count; ++i) {
    RiceArgs a;
    const int64_t nj = prepare_decode(&in[i], &out[i], dev_status, a);
    if (nj < 0) return static_cast<int32_t>(nj);
    const uint32_t esc_bytes = in[i].n > 15 ? in[i].n - 15 : 0;   // <= 241
    StreamArgs sa;
    const int64_t ns = prepare_stream(&in[i], a, sa);
    if (ns > 0) {
      if (sn == kMaxDecodeBatch || spool + esc_bytes > static_cast<uint32_t>(kEscPool) ||
          spans + static_cast<uint64_t>(ns) >= (1ull << 31)) {
        sbat.first_job[sn] = static_cast<uint32_t>(spans);
        sbat.count = sn;
        const int32_t s = launch_stream(sbat, st);
        if (s != BINADE_OK) return s;
        sbat = StreamBatch{};
        sn = 0;
        spans = 0;
        spool = 0;
      }
      if (static_cast<uint64_t>(ns) >= (1ull << 31)) return BINADE_EUNSUPPORTED;
      for (uint32_t r = 0; r < esc_bytes; ++r) sbat.pool[spool + r] = in[i].exp_of_rank[15 + r];
      sa.esc_tbl = static_cast<uint32_t>(offsetof(StreamBatch, pool)) + spool;
      spool += esc_bytes;
      sbat.item[sn] = sa;
      sbat.first_job[sn] = static_cast<uint32_t>(spans);
      spans += static_cast<uint64_t>(ns);
      ++sn;
      continue;
    }
    if (n == kMaxDecodeBatch || pool + esc_bytes > static_cast<uint32_t>(kEscPool) ||
        jobs + static_cast<uint64_t>(nj) >= (1ull << 31)) {
      b.first_job[n] = static_cast<uint32_t>(jobs);
      b.count = n;
      const int32_t s = launch_batch(b, st);
      if (s != BINADE_OK) return s;
      b = RiceBatch{};
      n = 0;
      jobs = 0;
      pool = 0;
    }
    if (static_cast<uint64_t>(nj) >= (1ull << 31)) return BINADE_EUNSUPPORTED;
    for (uint32_t r = 0; r < esc_bytes; ++r) b.pool[pool + r] = in[i].exp_of_rank[15 + r];
    a.esc_tbl = static_cast<uint32_t>(offsetof(RiceBatch, pool)) + pool;
    pool += esc_bytes;
    b.item[n] = a;
    b.first_job[n] = static_cast<uint32_t>(jobs);
    jobs += static_cast<uint64_t>(nj);
    ++n;
  }
  if (n > 0) {
    b.first_job[n] = static_cast<uint32_t>(jobs);
    b.count = n;
    const int32_t s = launch_batch(b, st);
    if (s != BINADE_OK) return s;
  }
  if (sn > 0) {
    sbat.first_job[sn] = static_cast<uint32_t>(spans);
    sbat.count = sn;
    return launch_stream(sbat, st);
  }
  return BINADE_OK;
}

extern "C" int64_t binade_rice_plan_bytes(int32_t count) {
  if (count < 0 || count > kMaxPlanTensors) return BINADE_EINVAL;
  return plan_layout(count).max_bytes;
}

extern "C" int32_t binade_rice_to_r4_plan(const binade_rice* in, binade_r4* out,
                                          int32_t count, void* plan, int64_t plan_bytes) {
  if (count < 0 || count > kMaxPlanTensors || plan == nullptr ||
      (count > 0 && (in == nullptr || out == nullptr)))
    return BINADE_EINVAL;
  const PlanLayout l = plan_layout(count);
  if (plan_bytes < static_cast<int64_t>(l.max_bytes)) return BINADE_EINVAL;
  uint8_t* base = static_cast<uint8_t*>(plan);
  std::memset(base, 0, l.pool_off);
  uint32_t* first = reinterpret_cast<uint32_t*>(base + l.first_off);
  uint64_t spans = 0;
  uint32_t pool = 0;
  for (int32_t i = 0; i < count; ++i) {
    RiceArgs a;
    const int64_t nj = prepare_decode(&in[i], &out[i], nullptr, a);
    if (nj < 0) return static_cast<int32_t>(nj);
    StreamArgs sa;
    const int64_t ns = prepare_stream(&in[i], a, sa, BINADE_PLAN_SPAN);
    if (ns <= 0 || spans + static_cast<uint64_t>(ns) >= (1ull << 31)) return BINADE_EUNSUPPORTED;
    const uint32_t esc_bytes = in[i].n > 15 ? in[i].n - 15 : 0;   // <= 241
    std::memcpy(base + l.pool_off + pool, in[i].exp_of_rank + 15, esc_bytes);
    sa.esc_tbl = l.pool_off + pool;
    sa.status = nullptr;
    pool += esc_bytes;
    first[i] = static_cast<uint32_t>(spans);
    std::memcpy(base + l.items_off + static_cast<size_t>(i) * sizeof(StreamArgs), &sa, sizeof sa);
    spans += static_cast<uint64_t>(ns);
  }
  first[count] = static_cast<uint32_t>(spans);
  PlanHeader h{};
  h.magic = kPlanMagic;
  h.count = count;
  h.spans = static_cast<uint32_t>(spans);
  h.first_off = l.first_off;
  h.items_off = l.items_off;
  h.pool_off = l.pool_off;
  h.bytes = l.pool_off + pool;
  std::memcpy(base, &h, sizeof h);
  return BINADE_OK;
}

extern "C" int32_t binade_rice_to_r4_run(const void* host_plan, const void* dev_plan,
                                         uint32_t* dev_status, void* stream) {
  if (host_plan == nullptr) return BINADE_EINVAL;
  PlanHeader h;
  std::memcpy(&h, host_plan, sizeof h);
  if (h.magic != kPlanMagic || h.count < 0 || h.count > kMaxPlanTensors) return BINADE_EINVAL;
  const PlanLayout l = plan_layout(h.count);
  if (h.first_off != l.first_off || h.items_off != l.items_off || h.pool_off != l.pool_off)
    return BINADE_EINVAL;
  if (h.count == 0 || h.spans == 0) return BINADE_OK;
  if (dev_plan == nullptr || (reinterpret_cast<uintptr_t>(dev_plan) & 7u) != 0)
    return BINADE_EINVAL;
  PlanLaunch p;
  p.plan = static_cast<const uint8_t*>(dev_plan);
  p.status = dev_status;
  p.count = static_cast<uint32_t>(h.count);
  p.spans = h.spans;
  p.first_off = h.first_off;
  p.items_off = h.items_off;
  return launch_plan(p, static_cast<hipStream_t>(stream));
}
