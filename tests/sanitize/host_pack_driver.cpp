// Runs the library's host packer (binade_build_table, binade_sizes_of,
// binade_pack_rice) on many shapes and bit distributions with buffers of
// exactly the size binade_sizes_of reports, plus its error paths. Built with
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
    }
  }
  std::vector<uint16_t> all(65536);
  for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
  bad |= run(all, 256, 256);
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
