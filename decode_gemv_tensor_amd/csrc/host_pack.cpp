// Host half of libbinade: exponent table, plane sizes and the format 2
// (Rice) packer.
//
// "Binade" package page (pypi.org/project/binade), intro: sign and mantissa
// bits are kept unchanged in a byte, the exponent is stored as its rank
// among the tensor's exponents ordered by frequency, and the ranks are
// stored in Rice codes. Section "How it works": one table per tensor;
// format 2 is the Rice format.
//
// Packing is offline work (the pages run it as a command-line step), so it
// lives on the host; the device kernels start from its planes.
#include <algorithm>
#include <array>
#include <cstring>
#include <numeric>
#include <queue>
#include <utility>
#include <vector>

#include "binade.h"
#include "binade_internal.h"

namespace {

// Appends bit fields to a little-endian u32 word array through a 64-bit
// accumulator. Bits beyond the final position stay zero.
class BitSink {
 public:
  BitSink(uint32_t* words, uint64_t cap_words) : w_(words), cap_(cap_words) {}

  // Append `n` zero bits followed by nothing (n may be large).
  bool zeros(uint64_t n) {
    while (n > 0) {
      const uint32_t take = static_cast<uint32_t>(std::min<uint64_t>(n, 32));
      if (!put(0, take)) return false;
      n -= take;
    }
    return true;
  }

  // Append the low `n` bits of v (n <= 32), least significant first.
  bool put(uint32_t v, uint32_t n) {
    if (n == 0) return true;
    acc_ |= static_cast<uint64_t>(v & mask(n)) << fill_;
    fill_ += n;
    pos_ += n;
    if (fill_ >= 32) {
      if (out_ >= cap_) return false;
      w_[out_++] = static_cast<uint32_t>(acc_);
      acc_ >>= 32;
      fill_ -= 32;
    }
    return true;
  }

  bool flush() {
    if (fill_ > 0) {
      if (out_ >= cap_) return false;
      w_[out_++] = static_cast<uint32_t>(acc_);
      acc_ = 0;
      fill_ = 0;
    }
    for (uint64_t i = out_; i < cap_; ++i) w_[i] = 0;  // padding
    return true;
  }

  uint64_t position() const { return pos_; }

 private:
  static uint32_t mask(uint32_t n) { return n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u); }
  uint32_t* w_;
  uint64_t cap_;
  uint64_t out_ = 0;
  uint64_t acc_ = 0;
  uint32_t fill_ = 0;
  uint64_t pos_ = 0;
};

inline uint32_t exponent_of(uint16_t b) { return (b >> 7) & 0xFFu; }

}  // namespace

extern "C" int32_t binade_build_table(const uint16_t* w, int64_t n,
                                      binade_table* out) {
  if (w == nullptr || out == nullptr || n <= 0) return BINADE_EINVAL;
  std::array<uint64_t, 256> hist{};
  for (int64_t i = 0; i < n; ++i) ++hist[exponent_of(w[i])];

  std::array<uint16_t, 256> order;
  std::iota(order.begin(), order.end(), 0);
  // most frequent first; equal counts: smaller exponent first
  std::sort(order.begin(), order.end(), [&](uint16_t a, uint16_t b) {
    if (hist[a] != hist[b]) return hist[a] > hist[b];
    return a < b;
  });

  std::memset(out, 0, sizeof(*out));
  for (int e = 0; e < 256; ++e) out->rank_of_exp[e] = 0xFFFF;
  uint32_t present = 0;
  for (int r = 0; r < 256; ++r) {
    const uint16_t e = order[r];
    if (hist[e] == 0) break;
    out->exp_of_rank[r] = static_cast<uint8_t>(e);
    out->rank_of_exp[e] = static_cast<uint16_t>(r);
    out->count_of_rank[r] = hist[e];
    ++present;
  }
  out->n = present;
  out->k = binade::best_rice_k(out->count_of_rank, present);
  return BINADE_OK;
}

namespace binade {

uint64_t rice_unary_bits(const uint64_t* count_of_rank, uint32_t n,
                         uint32_t k) {
  uint64_t bits = 0;
  for (uint32_t r = 0; r < n; ++r) bits += count_of_rank[r] * ((r >> k) + 1u);
  return bits;
}

uint32_t best_rice_k(const uint64_t* count_of_rank, uint32_t n) {
  uint64_t total_w = 0;
  for (uint32_t r = 0; r < n; ++r) total_w += count_of_rank[r];
  uint32_t best = 0;
  uint64_t best_bits = ~0ull;
  for (uint32_t k = 0; k <= 7; ++k) {
    const uint64_t bits = rice_unary_bits(count_of_rank, n, k) + k * total_w;
    if (bits < best_bits) {  // strict: ties keep the smaller k
      best_bits = bits;
      best = k;
    }
  }
  return best;
}

}  // namespace binade

extern "C" int32_t binade_sizes_of(const binade_table* t, int64_t rows,
                                   int64_t cols, binade_sizes* out) {
  if (t == nullptr || out == nullptr || rows <= 0 || cols <= 0 || t->n == 0 ||
      t->n > 256 || t->k > 7)
    return BINADE_EINVAL;
  const uint64_t nw = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols);
  uint64_t counted = 0, esc = 0;
  for (uint32_t r = 0; r < t->n; ++r) {
    counted += t->count_of_rank[r];
    if (r >= 15) esc += t->count_of_rank[r];
  }
  // the table may describe a different tensor than rows x cols only if the
  // counts disagree; sizes are only meaningful for the tensor it was built on
  if (counted != nw) return BINADE_EINVAL;
  out->n_weights = nw;
  out->n_chunks = static_cast<uint64_t>(rows) *
                  static_cast<uint64_t>((cols + BINADE_CHUNK - 1) / BINADE_CHUNK);
  out->unary_bits = binade::rice_unary_bits(t->count_of_rank, t->n, t->k);
  out->unary_words = (out->unary_bits + 31) / 32 + 2;
  out->rem_words = (nw * t->k + 31) / 32 + 2;
  out->n_esc = esc;
  out->nib_bytes = nw / 2;
  return BINADE_OK;
}

extern "C" int32_t binade_pack_rice(const uint16_t* w, int64_t rows,
                                    int64_t cols, const binade_table* t,
                                    binade_rice* out) {
  if (w == nullptr || t == nullptr || out == nullptr || rows <= 0 ||
      cols <= 0 || t->n == 0 || t->n > 256 || t->k > 7)
    return BINADE_EINVAL;
  if (out->sm == nullptr || out->unary == nullptr || out->anchor == nullptr ||
      out->esc_pre == nullptr || (t->k > 0 && out->rem == nullptr))
    return BINADE_EINVAL;
  const uint32_t k = t->k;
  const int64_t cpr = (cols + BINADE_CHUNK - 1) / BINADE_CHUNK;

  BitSink unary(out->unary, out->unary_words);
  BitSink rem(out->rem, k > 0 ? out->rem_words : 0);
  uint64_t esc = 0;
  for (int64_t row = 0; row < rows; ++row) {
    const uint16_t* src = w + row * cols;
    uint8_t* sm = out->sm + row * cols;
    for (int64_t c0 = 0; c0 < cols; c0 += BINADE_CHUNK) {
      const int64_t chunk = row * cpr + c0 / BINADE_CHUNK;
      out->anchor[chunk] = unary.position();
      out->esc_pre[chunk] = static_cast<uint32_t>(esc);
      const int64_t c1 = std::min<int64_t>(cols, c0 + BINADE_CHUNK);
      for (int64_t c = c0; c < c1; ++c) {
        const uint16_t b = src[c];
        const uint16_t rank = t->rank_of_exp[exponent_of(b)];
        if (rank == 0xFFFF || rank >= t->n) return BINADE_EINVAL;
        sm[c] = static_cast<uint8_t>(((b >> 8) & 0x80u) | (b & 0x7Fu));
        if (!unary.zeros(rank >> k) || !unary.put(1u, 1)) return BINADE_ENOSPACE;
        if (k > 0 && !rem.put(rank, k)) return BINADE_ENOSPACE;
        esc += rank >= 15;
      }
    }
  }
  if (!unary.flush() || (k > 0 && !rem.flush())) return BINADE_ENOSPACE;
  const int64_t nchunks = rows * cpr;
  out->anchor[nchunks] = unary.position();
  out->esc_pre[nchunks] = static_cast<uint32_t>(esc);
  out->rows = rows;
  out->cols = cols;
  out->k = k;
  out->n = t->n;
  std::memcpy(out->exp_of_rank, t->exp_of_rank, sizeof(out->exp_of_rank));
  out->unary_bits = unary.position();
  out->n_esc = esc;
  return BINADE_OK;
}

// ---------------------------------------------------------------- format 1
// "Binade" package page, "How it works": format 1 stores a fixed code width
// per 128-weight tile, with escapes. The layout is the one binade.h states.

namespace {

constexpr int64_t kTile = 128;

// The width of a tile of `len` ranks with the fewest code and escape bits,
// len * w + 8 * (ranks >= 2^w - 1); width 0 only when every rank is 0; ties
// to the smaller width. Ranks are counted once, by value.
int tile_width(const uint16_t* ranks, int64_t len) {
  std::array<int64_t, 257> at_least{};   // ranks >= v, for v = 0..256
  for (int64_t i = 0; i < len; ++i) ++at_least[ranks[i]];
  for (int v = 255; v >= 0; --v) at_least[v] += at_least[v + 1];
  int best = at_least[1] == 0 ? 0 : -1;
  int64_t best_bits = 0;
  for (int w = 1; w <= 8; ++w) {
    const int64_t bits = len * w + 8 * at_least[(1 << w) - 1];
    if (best < 0 || bits < best_bits) {
      best = w;
      best_bits = bits;
    }
  }
  return best;
}

}  // namespace

extern "C" int32_t binade_f1_sizes_of(int64_t rows, int64_t cols,
                                      binade_f1_sizes* out) {
  if (out == nullptr || rows <= 0 || cols <= 0) return BINADE_EINVAL;
  const uint64_t nw = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols);
  out->n_weights = nw;
  out->n_tiles = static_cast<uint64_t>(rows) * static_cast<uint64_t>((cols + kTile - 1) / kTile);
  out->n_chunks = static_cast<uint64_t>(rows) *
                  static_cast<uint64_t>((cols + BINADE_CHUNK - 1) / BINADE_CHUNK);
  out->code_words = nw * 8 / 32 + 2;
  out->esc_cap = nw;
  return BINADE_OK;
}

extern "C" int32_t binade_pack_f1(const uint16_t* w, int64_t rows, int64_t cols,
                                  const binade_table* t, binade_f1* out) {
  if (w == nullptr || t == nullptr || out == nullptr || rows <= 0 ||
      cols <= 0 || t->n == 0 || t->n > 256)
    return BINADE_EINVAL;
  if (out->sm == nullptr || out->width == nullptr || out->codes == nullptr ||
      out->anchor == nullptr || out->f1_pre == nullptr || out->esc_pre == nullptr ||
      (out->esc_cap > 0 && out->esc_rank == nullptr))
    return BINADE_EINVAL;
  const int64_t tpr = (cols + kTile - 1) / kTile;
  const int64_t cpr = (cols + BINADE_CHUNK - 1) / BINADE_CHUNK;
  BitSink codes(out->codes, out->code_words);
  uint64_t n_f1 = 0, n_r4 = 0;
  uint16_t ranks[kTile];
  for (int64_t row = 0; row < rows; ++row) {
    const uint16_t* src = w + row * cols;
    uint8_t* sm = out->sm + row * cols;
    for (int64_t tile = 0; tile < tpr; ++tile) {
      const int64_t c0 = tile * kTile;
      const int64_t len = std::min<int64_t>(kTile, cols - c0);
      if (c0 % BINADE_CHUNK == 0) {
        const int64_t chunk = row * cpr + c0 / BINADE_CHUNK;
        out->anchor[chunk] = codes.position();
        out->f1_pre[chunk] = static_cast<uint32_t>(n_f1);
        out->esc_pre[chunk] = static_cast<uint32_t>(n_r4);
      }
      for (int64_t i = 0; i < len; ++i) {
        const uint16_t b = src[c0 + i];
        const uint16_t r = t->rank_of_exp[exponent_of(b)];
        if (r == 0xFFFF || r >= t->n) return BINADE_EINVAL;
        ranks[i] = r;
        sm[c0 + i] = static_cast<uint8_t>(((b >> 8) & 0x80u) | (b & 0x7Fu));
        n_r4 += r >= 15;
      }
      const int wt = tile_width(ranks, len);
      out->width[row * tpr + tile] = static_cast<uint8_t>(wt);
      if (wt == 0) continue;
      const uint32_t escape = (1u << wt) - 1u;
      for (int64_t i = 0; i < len; ++i) {
        if (ranks[i] >= escape) {
          if (n_f1 >= out->esc_cap) return BINADE_ENOSPACE;
          out->esc_rank[n_f1++] = static_cast<uint8_t>(ranks[i]);
          if (!codes.put(escape, static_cast<uint32_t>(wt))) return BINADE_ENOSPACE;
        } else if (!codes.put(ranks[i], static_cast<uint32_t>(wt))) {
          return BINADE_ENOSPACE;
        }
      }
    }
  }
  if (!codes.flush()) return BINADE_ENOSPACE;
  const int64_t nchunks = rows * cpr;
  out->anchor[nchunks] = codes.position();
  out->f1_pre[nchunks] = static_cast<uint32_t>(n_f1);
  out->esc_pre[nchunks] = static_cast<uint32_t>(n_r4);
  out->rows = rows;
  out->cols = cols;
  out->n = t->n;
  std::memcpy(out->exp_of_rank, t->exp_of_rank, sizeof(out->exp_of_rank));
  out->code_bits = codes.position();
  out->n_f1esc = n_f1;
  out->n_esc = n_r4;
  return BINADE_OK;
}

// ---------------------------------------------------------------- Huffman
// "Lossless BF16 weight compression" page, intro and "Best measured
// configuration": the comparison codec. The layout is the one binade.h
// states for binade_huff.

namespace {

constexpr int kHuffMaxLen = 31;

// Code lengths by Huffman's construction: a min-heap of (weight, id), the
// two lightest merged into node 256 + m at merge m.
int32_t huff_lengths(const std::array<uint64_t, 256>& counts, uint8_t* len) {
  using Node = std::pair<uint64_t, int>;
  std::priority_queue<Node, std::vector<Node>, std::greater<Node>> heap;
  std::array<int, 511> parent;
  parent.fill(-1);
  int present = 0;
  for (int e = 0; e < 256; ++e) {
    len[e] = 0;
    if (counts[e]) {
      heap.push({counts[e], e});
      ++present;
    }
  }
  if (present == 0) return BINADE_EINVAL;
  if (present == 1) {
    len[heap.top().second] = 1;
    return BINADE_OK;
  }
  int next = 256;
  while (heap.size() > 1) {
    const Node a = heap.top();
    heap.pop();
    const Node b = heap.top();
    heap.pop();
    parent[a.second] = parent[b.second] = next;
    heap.push({a.first + b.first, next++});
  }
  for (int e = 0; e < 256; ++e) {
    if (!counts[e]) continue;
    int d = 0;
    for (int p = parent[e]; p >= 0; p = parent[p]) ++d;
    if (d > kHuffMaxLen) return BINADE_EUNSUPPORTED;
    len[e] = static_cast<uint8_t>(d);
  }
  return BINADE_OK;
}

// Canonical codes: exponents in (length, exponent) order take consecutive
// values; a longer length shifts the running value left.
std::array<uint32_t, 256> huff_codes(const uint8_t* len) {
  std::array<uint32_t, 256> code{};
  std::vector<std::pair<int, int>> order;   // (length, exponent)
  for (int e = 0; e < 256; ++e)
    if (len[e]) order.push_back({len[e], e});
  std::sort(order.begin(), order.end());
  uint32_t c = 0;
  int prev = 0;
  for (const auto& le : order) {
    if (prev) c <<= (le.first - prev);
    code[le.second] = c++;
    prev = le.first;
  }
  return code;
}

std::array<uint64_t, 256> exponent_counts(const uint16_t* w, int64_t n) {
  std::array<uint64_t, 256> c{};
  for (int64_t i = 0; i < n; ++i) ++c[exponent_of(w[i])];
  return c;
}

}  // namespace

extern "C" int32_t binade_huff_lengths(const uint16_t* w, int64_t n, uint8_t* len,
                                       uint64_t* stream_cap) {
  if (w == nullptr || n <= 0 || len == nullptr) return BINADE_EINVAL;
  const auto counts = exponent_counts(w, n);
  const int32_t s = huff_lengths(counts, len);
  if (s != BINADE_OK) return s;
  if (stream_cap != nullptr) {
    uint64_t bits = 0;
    for (int e = 0; e < 256; ++e) bits += counts[e] * len[e];
    const uint64_t blocks = (static_cast<uint64_t>(n) + BINADE_HUFF_BLOCK - 1) / BINADE_HUFF_BLOCK;
    *stream_cap = (bits + 7) / 8 + blocks + 8;
  }
  return BINADE_OK;
}

extern "C" int32_t binade_huff_pack(const uint16_t* w, binade_huff* out) {
  if (w == nullptr || out == nullptr || out->n <= 0 || out->sm == nullptr ||
      out->stream == nullptr || out->block_len == nullptr || out->group_off == nullptr)
    return BINADE_EINVAL;
  const int64_t n = out->n;
  const auto code = huff_codes(out->len);
  std::memset(out->stream, 0, out->stream_cap);
  uint64_t pos = 0;   // bit position, MSB-first within bytes
  const int64_t blocks = (n + BINADE_HUFF_BLOCK - 1) / BINADE_HUFF_BLOCK;
  for (int64_t b = 0; b < blocks; ++b) {
    const uint64_t start = pos;
    if (b % BINADE_HUFF_GROUP == 0) out->group_off[b / BINADE_HUFF_GROUP] = pos >> 3;
    const int64_t i1 = std::min<int64_t>(n, (b + 1) * BINADE_HUFF_BLOCK);
    for (int64_t i = b * BINADE_HUFF_BLOCK; i < i1; ++i) {
      const uint32_t e = exponent_of(w[i]);
      const int l = out->len[e];
      if (l == 0 || l > kHuffMaxLen) return BINADE_EINVAL;
      out->sm[i] = static_cast<uint8_t>(((w[i] >> 8) & 0x80u) | (w[i] & 0x7Fu));
      if ((pos + l + 7) / 8 > out->stream_cap) return BINADE_ENOSPACE;
      for (int j = l - 1; j >= 0; --j, ++pos)
        if ((code[e] >> j) & 1u) out->stream[pos >> 3] |= static_cast<uint8_t>(0x80u >> (pos & 7));
    }
    pos = (pos + 7) & ~7ull;
    out->block_len[b] = static_cast<uint8_t>((pos - start) >> 3);
  }
  out->group_off[(blocks + BINADE_HUFF_GROUP - 1) / BINADE_HUFF_GROUP] = pos >> 3;
  out->stream_bytes = pos >> 3;
  return BINADE_OK;
}

extern "C" const char* binade_status_str(int32_t s) {
  switch (s) {
    case BINADE_OK: return "ok";
    case BINADE_EINVAL: return "invalid argument";
    case BINADE_ECORRUPT: return "corrupt planes";
    case BINADE_EUNSUPPORTED: return "unsupported shape or alignment";
    case BINADE_EHIP: return "HIP runtime error";
    case BINADE_ENOSPACE: return "output buffer too small";
    default: return "unknown status";
  }
}
