// Runs the library's host packers (binade_build_table, binade_sizes_of,
// binade_pack_rice; binade_f1_sizes_of, binade_pack_f1; binade_huff_lengths,
// binade_huff_pack) on many shapes and bit distributions with buffers of
// exactly the size the library reports (or the pack needed), plus their
// error paths. Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py;
// any out-of-bounds access, leak or undefined operation aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "binade.h"

static int fail(const char* what, int64_t rows, int64_t cols, int32_t s) {
  std::fprintf(stderr, "%s failed: %lldx%lld status %d\n", what, (long long)rows, (long long)cols, s);
  return 1;
}

static int run(const std::vector<uint16_t>& w, int64_t rows, int64_t cols) {
  binade_table t;
  int32_t s = binade_build_table(w.data(), rows * cols, &t);
  if (s != BINADE_OK) return fail("build_table", rows, cols, s);
  binade_sizes z;
  s = binade_sizes_of(&t, rows, cols, &z);
  if (s != BINADE_OK) return fail("sizes_of", rows, cols, s);
  // exact-size heap buffers: one word past the end is a sanitizer report
  uint8_t* sm = new uint8_t[z.n_weights];
  uint32_t* unary = new uint32_t[z.unary_words];
  uint32_t* rem = t.k ? new uint32_t[z.rem_words] : nullptr;
  uint64_t* anchor = new uint64_t[z.n_chunks + 1];
  uint32_t* esc_pre = new uint32_t[z.n_chunks + 1];
  binade_rice r{};
  r.sm = sm; r.unary = unary; r.unary_words = z.unary_words;
  r.rem = rem; r.rem_words = t.k ? z.rem_words : 0;
  r.anchor = anchor; r.esc_pre = esc_pre;
  s = binade_pack_rice(w.data(), rows, cols, &t, &r);
  int bad = s != BINADE_OK ? fail("pack_rice", rows, cols, s) : 0;
  if (!bad && (r.unary_bits != z.unary_bits || r.n_esc != z.n_esc))
    bad = fail("pack_rice sizes", rows, cols, -100);
  // too little room: ENOSPACE, no write past the buffers
  if (!bad && z.unary_words > 3) {
    r.unary_words = z.unary_words - 3;
    s = binade_pack_rice(w.data(), rows, cols, &t, &r);
    if (s != BINADE_ENOSPACE) bad = fail("pack_rice short unary", rows, cols, s);
  }
  delete[] sm; delete[] unary; delete[] rem; delete[] anchor; delete[] esc_pre;
  return bad;
}

// Format 1: the capacities binade_f1_sizes_of reports, then buffers of
// exactly the words and escapes the first pack used, then one word and one
// escape fewer (ENOSPACE, no write past the buffers).
static int run_f1(const std::vector<uint16_t>& w, int64_t rows, int64_t cols) {
  binade_table t;
  int32_t s = binade_build_table(w.data(), rows * cols, &t);
  if (s != BINADE_OK) return fail("build_table", rows, cols, s);
  binade_f1_sizes z;
  s = binade_f1_sizes_of(rows, cols, &z);
  if (s != BINADE_OK) return fail("f1_sizes_of", rows, cols, s);
  std::vector<uint8_t> sm(z.n_weights), width(z.n_tiles);
  std::vector<uint64_t> anchor(z.n_chunks + 1);
  std::vector<uint32_t> f1_pre(z.n_chunks + 1), esc_pre(z.n_chunks + 1);
  auto pack = [&](uint64_t words, uint64_t escs, binade_f1& f) {
    uint32_t* codes = new uint32_t[words ? words : 1];
    uint8_t* esc = escs ? new uint8_t[escs] : nullptr;
    f = binade_f1{};
    f.sm = sm.data(); f.width = width.data(); f.codes = codes; f.code_words = words;
    f.esc_rank = esc; f.esc_cap = escs; f.anchor = anchor.data();
    f.f1_pre = f1_pre.data(); f.esc_pre = esc_pre.data();
    const int32_t rc = binade_pack_f1(w.data(), rows, cols, &t, &f);
    delete[] codes; delete[] esc;
    return rc;
  };
  binade_f1 f;
  s = pack(z.code_words, z.esc_cap, f);
  if (s != BINADE_OK) return fail("pack_f1", rows, cols, s);
  const uint64_t words = (f.code_bits + 31) / 32, escs = f.n_f1esc;
  binade_f1 g;
  s = pack(words, escs, g);
  if (s != BINADE_OK || g.code_bits != f.code_bits || g.n_f1esc != f.n_f1esc)
    return fail("pack_f1 exact", rows, cols, s);
  if (words > 0 && pack(words - 1, escs, g) != BINADE_ENOSPACE)
    return fail("pack_f1 short codes", rows, cols, -101);
  if (escs > 0 && pack(words, escs - 1, g) != BINADE_ENOSPACE)
    return fail("pack_f1 short escapes", rows, cols, -102);
  return 0;
}

// Huffman: lengths and the capacity they report, a pack into exactly that,
// then into the bytes the stream needs minus one (ENOSPACE).
static int run_huff(const std::vector<uint16_t>& w) {
  const int64_t n = static_cast<int64_t>(w.size());
  binade_huff h{};
  h.n = n;
  uint64_t cap = 0;
  int32_t s = binade_huff_lengths(w.data(), n, h.len, &cap);
  if (s != BINADE_OK) return fail("huff_lengths", n, 0, s);
  const int64_t blocks = (n + BINADE_HUFF_BLOCK - 1) / BINADE_HUFF_BLOCK;
  const int64_t groups = (blocks + BINADE_HUFF_GROUP - 1) / BINADE_HUFF_GROUP;
  std::vector<uint8_t> sm(n), block_len(blocks);
  std::vector<uint64_t> group_off(groups + 1);
  auto pack = [&](uint64_t c, binade_huff& o) {
    uint8_t* stream = new uint8_t[c ? c : 1];
    o = h;
    o.sm = sm.data(); o.stream = stream; o.stream_cap = c;
    o.block_len = block_len.data(); o.group_off = group_off.data();
    const int32_t rc = binade_huff_pack(w.data(), &o);
    delete[] stream;
    return rc;
  };
  binade_huff o;
  s = pack(cap, o);
  if (s != BINADE_OK) return fail("huff_pack", n, 0, s);
  if (o.stream_bytes > 0 && pack(o.stream_bytes - 1, o) != BINADE_ENOSPACE)
    return fail("huff_pack short stream", n, 0, -103);
  return 0;
}

int main() {
  std::mt19937_64 rng(7);
  int bad = 0;
  const int64_t shapes[][2] = {{1, 1}, {1, 31}, {3, 33}, {5, 2048}, {4, 2049}, {2, 6144},
                               {7, 4160}, {64, 100}, {130, 128}};
  for (auto& sh : shapes) {
    const int64_t rows = sh[0], cols = sh[1];
    for (int dist = 0; dist < 3; ++dist) {
      std::vector<uint16_t> w(rows * cols);
      for (auto& v : w) {
        uint64_t u = rng();
        if (dist == 0) v = (uint16_t)u;                                  // any pattern
        else if (dist == 1) v = (uint16_t)(((u >> 8) & 0x807F) | ((118 + (u % 9)) << 7));  // few exponents
        else v = (uint16_t)(((u >> 8) & 0x807F) | ((60 + (u % 130)) << 7));             // many exponents
      }
      bad |= run(w, rows, cols);
      bad |= run_f1(w, rows, cols);
      bad |= run_huff(w);
    }
  }
  std::vector<uint16_t> all(65536);
  for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
  bad |= run(all, 256, 256);
  bad |= run_f1(all, 256, 256);
  bad |= run_huff(all);
  {
    // a Fibonacci histogram: a code longer than 31 bits is refused
    std::vector<uint16_t> fib;
    uint64_t a = 1, b = 1;
    for (int e = 0; e < 34; ++e) {
      for (uint64_t i = 0; i < a && fib.size() < 20000000; ++i) fib.push_back((uint16_t)((e + 1) << 7));
      const uint64_t c = a + b;
      a = b;
      b = c;
    }
    uint8_t len[256];
    uint64_t cap = 0;
    if (binade_huff_lengths(fib.data(), (int64_t)fib.size(), len, &cap) != BINADE_EUNSUPPORTED)
      bad |= fail("huff_lengths deep tree", (int64_t)fib.size(), 0, -104);
  }
  // argument errors
  binade_table t{};
  if (binade_build_table(nullptr, 4, &t) != BINADE_EINVAL) bad |= fail("null w", 0, 0, 0);
  if (binade_build_table(all.data(), 0, &t) != BINADE_EINVAL) bad |= fail("n = 0", 0, 0, 0);
  binade_sizes z;
  if (binade_sizes_of(&t, -1, 4, &z) != BINADE_EINVAL) bad |= fail("rows < 0", 0, 0, 0);
  for (int32_t s = -6; s <= 1; ++s)
    if (binade_status_str(s) == nullptr) bad |= fail("status_str", 0, 0, s);
  std::printf(bad ? "host packer: FAILED\n" : "host packer: ok\n");
  return bad;
}
