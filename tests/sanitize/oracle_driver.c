/* Runs every oracle function (table, both file formats, R4, the GEMV, GEMM
 * and MoE replays, the MoE epilogue, the Huffman codec) on many shapes with
 * buffers of exactly the sizes its callers use, including corrupt streams. Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitizers.py; any out-of-bounds access, leak or undefined
 * operation aborts the run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_build_table(const uint16_t *w, int64_t n, uint32_t *n_present, uint8_t *exp_of_rank, uint64_t *count_of_rank);
uint64_t oracle_rice_code_bits(const uint64_t *count_of_rank, uint32_t n, int k);
int oracle_rice_k(const uint64_t *count_of_rank, uint32_t n);
int oracle_pack_rice(const uint16_t *w, int64_t rows, int64_t cols, const uint8_t *exp_of_rank, uint32_t n, int k,
                     uint8_t *sm, uint32_t *unary, int64_t unary_words, uint32_t *rem, int64_t rem_words,
                     uint64_t *anchor, uint32_t *esc_pre, uint64_t *unary_bits_out);
int oracle_rice_decode(int64_t rows, int64_t cols, int k, const uint8_t *exp_of_rank, uint32_t n, const uint8_t *sm,
                       const uint32_t *unary, uint64_t unary_bits, const uint32_t *rem, const uint64_t *anchor,
                       const uint32_t *esc_pre, uint16_t *out);
int oracle_make_r4(const uint16_t *w, int64_t rows, int64_t cols, const uint8_t *exp_of_rank, uint32_t n,
                   uint8_t *lut16, uint8_t *nib, uint32_t *esc_pre, uint32_t *esc, int64_t esc_cap, int64_t *n_esc_out);
int oracle_r4_unpack(int64_t rows, int64_t cols, const uint8_t *lut16, const uint8_t *sm, const uint8_t *nib,
                     const uint32_t *esc_pre, const uint32_t *esc, int64_t n_esc, uint16_t *out);
int oracle_gemv_replay(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *x, float *y);
int oracle_gemm_replay(const uint16_t *w, int64_t N, int64_t K, const uint16_t *x, int64_t M, float *y);
int oracle_moe_replay(const uint16_t *experts, int64_t n_experts, int64_t N, int64_t K, const uint16_t *x,
                      int x_per_slot, const int32_t *idx, int64_t n_tokens, int64_t top_k, float *y);
float oracle_mfma_step(const uint16_t *a, const uint16_t *b, float c);
int oracle_pack_f1(const uint16_t *w, int64_t rows, int64_t cols, const uint8_t *exp_of_rank, uint32_t n,
                   uint8_t *sm, uint8_t *width, uint32_t *codes, int64_t code_words, uint8_t *esc, int64_t esc_cap,
                   uint64_t *anchor, uint32_t *f1_pre, uint32_t *esc_pre, uint64_t *code_bits_out,
                   int64_t *n_f1esc_out);
int oracle_f1_decode(int64_t rows, int64_t cols, const uint8_t *exp_of_rank, uint32_t n, const uint8_t *sm,
                     const uint8_t *width, const uint32_t *codes, uint64_t code_bits, const uint8_t *esc,
                     int64_t n_f1esc, const uint64_t *anchor, const uint32_t *f1_pre, const uint32_t *esc_pre,
                     uint16_t *out);
void oracle_silu_mul(const float *gate, const float *up, int64_t n, float *out);
int oracle_moe_combine(const float *y, const float *weights, int64_t n_tokens, int top_k, int64_t n, float *out);
int oracle_huff_lengths(const uint64_t *counts, uint8_t *len);
int oracle_huff_pack(const uint16_t *w, int64_t n, const uint8_t *len, uint8_t *sm, uint8_t *stream, int64_t cap,
                     uint8_t *block_len, uint64_t *group_off, uint64_t *bytes_out);
int oracle_huff_decode(int64_t n, const uint8_t *len, const uint8_t *sm, const uint8_t *stream,
                       int64_t stream_bytes, const uint8_t *block_len, const uint64_t *group_off, uint16_t *out);

static uint64_t state = 88172645463325252ull;
static uint64_t next(void) { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return state; }

static int check(int64_t rows, int64_t cols, int dist) {
  int64_t n = rows * cols, i, cpr = (cols + 2047) / 2048, nch = rows * cpr, nesc = 0;
  uint16_t *w = malloc(n * 2), *back = malloc(n * 2);
  uint32_t np = 0;
  uint8_t eor[256];
  uint64_t cor[256], ubits = 0;
  int k, rc, bad = 0;
  for (i = 0; i < n; ++i) {
    uint64_t u = next();
    w[i] = dist == 0 ? (uint16_t)u : (uint16_t)(((u >> 8) & 0x807F) | ((118 + u % 9) << 7));
  }
  rc = oracle_build_table(w, n, &np, eor, cor);
  k = oracle_rice_k(cor, np);
  {
    int64_t ubits_max = (int64_t)oracle_rice_code_bits(cor, np, k) - (int64_t)n * k;
    int64_t uw = ubits_max / 32 + 1, rw = (n * k + 31) / 32 + 1;
    uint8_t *sm = malloc(n);
    uint32_t *unary = malloc(uw * 4), *rem = malloc(rw * 4), *epre = malloc((nch + 1) * 4);
    uint64_t *anchor = malloc((nch + 1) * 8);
    rc |= oracle_pack_rice(w, rows, cols, eor, np, k, sm, unary, uw, rem, rw, anchor, epre, &ubits);
    rc |= oracle_rice_decode(rows, cols, k, eor, np, sm, unary, ubits, rem, anchor, epre, back);
    if (rc || memcmp(back, w, n * 2)) bad = 1;
    /* corrupt: flip unary bits; decode must report it without reading past the planes */
    unary[0] ^= 0x5u;
    if (uw > 2) unary[uw / 2] ^= 0x80000001u;
    if (oracle_rice_decode(rows, cols, k, eor, np, sm, unary, ubits, rem, anchor, epre, back) == 0 && ubits > 40) bad = 1;
    free(sm); free(unary); free(rem); free(epre); free(anchor);
  }
  if (cols % 32 == 0) {
    uint8_t lut[16], *nib = malloc(n / 2), *sm = malloc(n);
    uint32_t *epre = malloc((nch + 1) * 4), *esc = malloc((n ? n : 1) * 4);
    uint16_t *x = malloc(2 * cols * 2);   /* one vector per token of the gather */
    float *y = malloc(rows * 4);
    for (i = 0; i < n; ++i) sm[i] = (uint8_t)(((w[i] >> 8) & 0x80) | (w[i] & 0x7F));
    rc = oracle_make_r4(w, rows, cols, eor, np, lut, nib, epre, esc, n, &nesc);
    rc |= oracle_r4_unpack(rows, cols, lut, sm, nib, epre, esc, nesc, back);
    if (rc || memcmp(back, w, n * 2)) bad = 1;
    for (i = 0; i < 2 * cols; ++i) x[i] = (uint16_t)(0x3C00 + next() % 0x700);
    rc = oracle_gemv_replay(w, rows, cols, x, y);
    if (dist && rows >= 2 && cols >= 64) {
      int32_t idx[4] = {0, 1, 1, 0};
      float *ym = malloc(4 * (rows / 2) * 4);
      rc |= oracle_moe_replay(w, 2, rows / 2, cols, x, 0, idx, 2, 2, ym);
      free(ym);
    }
    if (dist) {
      int64_t M = 3;
      uint16_t *X = malloc(M * cols * 2);
      float *Y = malloc(M * rows * 4);
      for (i = 0; i < M * cols; ++i) X[i] = (uint16_t)(next() & 0xBFFF);
      rc |= oracle_gemm_replay(w, rows, cols, X, M, Y);
      free(X); free(Y);
    }
    if (rc) bad = 1;
    free(nib); free(sm); free(epre); free(esc); free(x); free(y);
  }
  {
    /* format 1: pack into the capacities its callers use, then decode from
     * exactly the words and escapes the pack wrote (plus the one word of
     * look-ahead its callers append) */
    int64_t tpr = (cols + 127) / 128, cw = n * 8 / 32 + 2, nf1 = 0, used;
    uint64_t cbits = 0;
    uint8_t *sm = malloc(n), *width = malloc(rows * tpr), *esc = malloc(n ? n : 1);
    uint32_t *codes = malloc(cw * 4), *f1p = malloc((nch + 1) * 4), *epre = malloc((nch + 1) * 4);
    uint64_t *anchor = malloc((nch + 1) * 8);
    rc = oracle_pack_f1(w, rows, cols, eor, np, sm, width, codes, cw, esc, n, anchor, f1p, epre, &cbits, &nf1);
    if (rc) bad = 1;
    used = (int64_t)((cbits + 31) / 32) + 1;
    {
      uint32_t *c2 = malloc(used * 4);
      uint8_t *e2 = malloc(nf1 ? nf1 : 1);
      memcpy(c2, codes, (used - 1) * 4);
      c2[used - 1] = 0;
      memcpy(e2, esc, nf1);
      if (!rc && (oracle_f1_decode(rows, cols, eor, np, sm, width, c2, cbits, e2, nf1, anchor, f1p, epre, back) ||
                  memcmp(back, w, n * 2)))
        bad = 1;
      /* corrupt: a width above 8 must be reported */
      if (rows * tpr > 0) {
        width[0] = 9;
        if (oracle_f1_decode(rows, cols, eor, np, sm, width, c2, cbits, e2, nf1, anchor, f1p, epre, back) == 0)
          bad = 1;
      }
      free(c2); free(e2);
    }
    free(sm); free(width); free(esc); free(codes); free(f1p); free(epre); free(anchor);
  }
  {
    /* Huffman: lengths, a pack into the stream bytes the codes need plus
     * one per block (its callers' capacity), a decode from exactly the
     * bytes written, and a corrupt block length */
    uint64_t cnt[256], bits = 0, sb = 0;
    uint8_t len[256];
    int64_t nb = (n + 63) / 64, ng = (nb + 127) / 128, cap;
    memset(cnt, 0, sizeof cnt);
    for (i = 0; i < n; ++i) ++cnt[(w[i] >> 7) & 0xFF];
    if (n > 0) {
      rc = oracle_huff_lengths(cnt, len);
      for (i = 0; i < 256; ++i) bits += cnt[i] * len[i];
      cap = (int64_t)((bits + 7) / 8) + nb;
      {
        uint8_t *sm = malloc(n), *stream = malloc(cap), *bl = malloc(nb);
        uint64_t *go = malloc((ng + 1) * 8);
        rc |= oracle_huff_pack(w, n, len, sm, stream, cap, bl, go, &sb);
        if (rc || oracle_huff_decode(n, len, sm, stream, (int64_t)sb, bl, go, back) || memcmp(back, w, n * 2))
          bad = 1;
        bl[0] ^= 1u;
        if (oracle_huff_decode(n, len, sm, stream, (int64_t)sb, bl, go, back) == 0) bad = 1;
        free(sm); free(stream); free(bl); free(go);
      }
    }
  }
  free(w); free(back);
  if (bad) fprintf(stderr, "oracle failed at %lldx%lld dist %d\n", (long long)rows, (long long)cols, dist);
  return bad;
}

int main(void) {
  static const int64_t shapes[][2] = {{1, 1}, {1, 31}, {3, 32}, {5, 2048}, {4, 2080}, {2, 6144}, {7, 4160}, {64, 96}, {130, 128}};
  int bad = 0, s, d, t;
  uint16_t a[32], b[32];
  for (s = 0; s < (int)(sizeof shapes / sizeof shapes[0]); ++s)
    for (d = 0; d < 2; ++d) bad |= check(shapes[s][0], shapes[s][1], d);
  for (t = 0; t < 20000; ++t) {   /* steps over every exponent range, finite operands */
    int k;
    float c;
    uint32_t cu = (uint32_t)next();
    for (k = 0; k < 32; ++k) {
      a[k] = (uint16_t)(next() & 0xBFFF);                 /* finite */
      b[k] = (uint16_t)next();
      if (((b[k] >> 7) & 0xFF) == 0xFF) b[k] &= 0xBFFF;   /* finite */
    }
    if (((cu >> 23) & 0xFF) == 0xFF) cu &= 0xBFFFFFFFu;
    memcpy(&c, &cu, 4);
    (void)oracle_mfma_step(a, b, c);
  }
  {
    /* MoE epilogue: activation and combine over exact-size buffers */
    float g[257], u[257], h[257], yv[3 * 4 * 33], wt[3 * 4], out[3 * 33];
    int j;
    for (j = 0; j < 257; ++j) {
      uint32_t bits = (uint32_t)next();
      if (((bits >> 23) & 0xFF) == 0xFF) bits &= 0xBFFFFFFFu;   /* finite */
      memcpy(&g[j], &bits, 4);
      u[j] = (float)((int)(next() % 2001) - 1000) / 7.0f;
    }
    oracle_silu_mul(g, u, 257, h);
    for (j = 0; j < 3 * 4 * 33; ++j) yv[j] = (float)((int)(next() % 2001) - 1000) / 3.0f;
    for (j = 0; j < 12; ++j) wt[j] = (float)(next() % 1000) / 1000.0f;
    if (oracle_moe_combine(yv, wt, 3, 4, 33, out)) bad = 1;
    if (oracle_moe_combine(yv, wt, 3, 0, 33, out) == 0) bad = 1;   /* top_k 0: EINVAL */
  }
  printf(bad ? "oracle: FAILED\n" : "oracle: ok\n");
  return bad;
}
