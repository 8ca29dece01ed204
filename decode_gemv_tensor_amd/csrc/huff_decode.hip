// The Huffman comparison decoder: canonical Huffman codes of the exponent
// byte, blocks of 64 symbols, back to bf16 weights.
//
// "Lossless BF16 weight compression" page (WeightLab), intro and "Best
// measured configuration": the exponent field entropy coded with canonical
// Huffman, sign and mantissa raw; one thread per block of 64 symbols, 128
// threads per thread block, each block's start found by a prefix sum over
// 8-bit block lengths, codes looked up in a table. The layout is the one
// binade.h states for binade_huff.
//
// On gfx950: a workgroup of 128 threads (two waves) takes groups of 128
// blocks in turn (persistent). Per group: a wave prefix sum (DPP) of the
// 8-bit lengths, joined across the two waves through LDS, gives each
// thread its block's first byte; the group's bytes (a few KiB) are copied
// into LDS with coalesced loads, byte-swapped to MSB-first words; each
// thread then decodes its 64 codes from a 64-bit bit buffer: the next 11
// bits index a 2048-entry table (symbol and length) in LDS, longer codes
// walk the canonical first-code-per-length table. Each 8 outputs leave as
// one 16-byte store. The tables are built once per call by a one-block
// kernel into the workspace.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

constexpr int kLutBits = 11;
constexpr int kLut = 1 << kLutBits;
constexpr int kMaxLen = 31;
constexpr int kHuffThreads = BINADE_HUFF_GROUP;   // one thread per block of a group
// A group's stream words staged in LDS (4 KiB: up to 4 bits per symbol on
// average; a longer group reads its words from memory)
constexpr int kStageWords = 1024;
// Words past the staged ones that a block's reads can reach: a block of 64
// codes of at most 31 bits spans at most 62 words beyond its first two, so
// the top-up read stays inside the array even on a corrupt stream (where
// the extra words are stale and the block is flagged by its length check).
constexpr int kStagePad = 64;

// Workspace layout (bytes)
constexpr int kWsLut = 0;                        // u16[2048]: symbol | length << 8 (0: longer)
constexpr int kWsFirst = kWsLut + 2 * kLut;      // u32[32]: canonical first code per length
constexpr int kWsCount = kWsFirst + 4 * 32;      // u32[32]: codes per length
constexpr int kWsBase = kWsCount + 4 * 32;       // u32[32]: index of the first symbol of a length
constexpr int kWsSorted = kWsBase + 4 * 32;      // u8[256]: symbols by (length, exponent)
constexpr int kWsBytes = kWsSorted + 256;

struct HuffTables {
  uint8_t len[256];
};

__global__ __launch_bounds__(256) void huff_tables_kernel(HuffTables t, uint8_t* ws) {
  __shared__ uint32_t count[kMaxLen + 2], first[kMaxLen + 2], base[kMaxLen + 2];
  __shared__ uint32_t wave_count[4][kMaxLen + 1];   // exponents of each length per wave
  __shared__ uint8_t sorted[256];
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  if (e < kMaxLen + 2) count[e] = 0;
  if (e < 4 * (kMaxLen + 1)) (&wave_count[0][0])[e] = 0;
  const uint32_t le = t.len[e];
  // the lanes of this wave with the same length as this lane (a ballot per
  // bit of the 5-bit length)
  uint64_t same = ~0ull;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const uint64_t m = __ballot((le >> b) & 1u);
    same &= ((le >> b) & 1u) ? m : ~m;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t in_wave = static_cast<uint32_t>(__popcll(same & below));
  __syncthreads();
  if (le) {
    atomicAdd(&count[le], 1u);
    if (in_wave == 0) wave_count[wave][le] = static_cast<uint32_t>(__popcll(same));
  }
  __syncthreads();
  if (e == 0) {
    uint32_t code = 0, idx = 0;
    for (int l = 1; l <= kMaxLen; ++l) {
      code = (l == 1) ? 0u : (code + count[l - 1]) << 1;
      first[l] = code;
      base[l] = idx;
      idx += count[l];
    }
  }
  __syncthreads();
  if (le) {
    // exponents of the same length before e: earlier waves', then this one's
    uint32_t before = in_wave;
    for (int w = 0; w < wave; ++w) before += wave_count[w][le];
    sorted[base[le] + before] = static_cast<uint8_t>(e);
  }
  __syncthreads();
  uint16_t* lut = reinterpret_cast<uint16_t*>(ws + kWsLut);
  // the table's lengths' counts and first codes, read once (wave-uniform)
  uint32_t cnt_l[kLutBits + 1], fst_l[kLutBits + 1], bas_l[kLutBits + 1];
#pragma unroll
  for (int l = 1; l <= kLutBits; ++l) {
    cnt_l[l] = count[l];
    fst_l[l] = first[l];
    bas_l[l] = base[l];
  }
#pragma unroll
  for (int q = 0; q < kLut / 256; ++q) {
    const uint32_t x = static_cast<uint32_t>(e + 256 * q);
    // the shortest length whose codes hold x's prefix (none: a longer code)
    uint32_t idx = 0, len = 0;
#pragma unroll
    for (int l = kLutBits; l >= 1; --l) {
      const uint32_t d = (x >> (kLutBits - l)) - fst_l[l];
      if (d < cnt_l[l]) {
        idx = bas_l[l] + d;
        len = static_cast<uint32_t>(l);
      }
    }
    lut[x] = len ? static_cast<uint16_t>(sorted[idx] | (len << 8)) : static_cast<uint16_t>(0);
  }
  if (e < 32) {
    reinterpret_cast<uint32_t*>(ws + kWsFirst)[e] = e <= kMaxLen ? first[e] : 0u;
    reinterpret_cast<uint32_t*>(ws + kWsCount)[e] = e <= kMaxLen ? count[e] : 0u;
    reinterpret_cast<uint32_t*>(ws + kWsBase)[e] = e <= kMaxLen ? base[e] : 0u;
  }
  ws[kWsSorted + e] = sorted[e];
}

struct HuffArgs {
  const uint8_t* sm;
  const uint8_t* stream;
  const uint8_t* block_len;
  const uint64_t* group_off;
  const uint8_t* ws;
  uint16_t* out;
  uint32_t* status;
  int64_t n;
  int64_t blocks;
  int64_t groups;
  uint32_t stream_words;   // whole 4-byte words the stream buffer holds
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ uint32_t bswap32(uint32_t v) {
  return __builtin_amdgcn_perm(0u, v, 0x00010203u);   // bytes 3,2,1,0: MSB-first bit order
}

__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {   // inclusive, 64 lanes
  constexpr int kRowShr = 0x110, kBcast15 = 0x142, kBcast31 = 0x143;
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 8, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0u, v, kBcast31, 0xC, 0xF, false);
  return v;
}

// The decode tables and the group's staged words in LDS.
struct HuffLds {
  const uint16_t* lut;
  const uint32_t* first;
  const uint32_t* count;
  const uint32_t* base;
  const uint8_t* sorted;
  const uint32_t* stage;
};

// One block's cnt codes from the bit buffer at word wi0 (skip bits in):
// each code is one table lookup (a rare longer code walks the canonical
// table, behind a wave-uniform test); the buffer tops up from the next word
// without a branch when fewer than 32 bits are left. kStaged: words from
// LDS, else from memory. kFull: every block of the wave holds 64 codes (no
// per-code test of the count).
template <bool kStaged, bool kFull>
__device__ __forceinline__ void decode_block(const HuffLds& L, __amdgpu_buffer_rsrc_t rs, uint32_t w0,
                                             uint32_t wi0, uint32_t skip, int cnt,
                                             const uint32_t (&smw)[16], uint16_t* po,
                                             uint32_t& used, bool& bad) {
  auto word = [&](uint32_t i) -> uint32_t {
    return kStaged ? L.stage[i] : bswap32(__builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (w0 + i), 0, 0));
  };
  uint32_t wi = wi0;
  uint64_t buf = ((static_cast<uint64_t>(word(wi)) << 32) | word(wi + 1)) << skip;
  uint32_t avail = 64u - skip;
  wi += 2;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 8 * q + k;
      if (kFull || i < cnt) {
        const uint32_t ent = L.lut[static_cast<uint32_t>(buf >> (64 - kLutBits))];
        uint32_t l = ent >> 8, sym = ent & 0xFFu;
        if (__any(l == 0u)) {
          if (l == 0u) {   // a code longer than the table: the canonical walk
            bool found = false;
            for (uint32_t ll = kLutBits + 1; ll <= kMaxLen; ++ll) {
              const uint32_t c = static_cast<uint32_t>(buf >> (64 - ll));
              if (L.count[ll] && c - L.first[ll] < L.count[ll]) {
                sym = L.sorted[L.base[ll] + c - L.first[ll]];
                l = ll;
                found = true;
                break;
              }
            }
            if (!found) {
              bad = true;
              l = 1;
            }
          }
        }
        buf <<= l;
        avail -= l;
        used += l;
        if (kStaged) {
          // top up from the next word when fewer than 32 bits are left
          const uint32_t nw = L.stage[wi];
          const bool need = avail < 32u;
          buf |= need ? static_cast<uint64_t>(nw) << (32u - avail) : 0ull;
          wi += need ? 1u : 0u;
          avail += need ? 32u : 0u;
        } else if (avail < 32u) {
          buf |= static_cast<uint64_t>(word(wi++)) << (32u - avail);
          avail += 32u;
        }
        const uint32_t sm = (smw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const uint32_t bf = ((sm & 0x80u) << 8) | (sym << 7) | (sm & 0x7Fu);
        o[k >> 1] |= bf << (16 * (k & 1));
      }
    }
    if (kFull || cnt == BINADE_HUFF_BLOCK) {
      reinterpret_cast<uint4*>(po)[q] = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (8 * q + k < cnt) po[8 * q + k] = static_cast<uint16_t>(o[k >> 1] >> (16 * (k & 1)));
    }
  }
}

__global__ __launch_bounds__(kHuffThreads) void huff_decode_kernel(HuffArgs a) {
  __shared__ uint16_t lut[kLut];
  __shared__ uint32_t first[32], count[32], base[32];
  __shared__ uint8_t sorted[256];
  __shared__ uint32_t stage[kStageWords + kStagePad];
  __shared__ uint32_t wave_total[2];
  const uint32_t tid = threadIdx.x;
  for (int i = tid; i < kLut / 2; i += kHuffThreads)
    reinterpret_cast<uint32_t*>(lut)[i] = reinterpret_cast<const uint32_t*>(a.ws + kWsLut)[i];
  if (tid < 32) {
    first[tid] = reinterpret_cast<const uint32_t*>(a.ws + kWsFirst)[tid];
    count[tid] = reinterpret_cast<const uint32_t*>(a.ws + kWsCount)[tid];
    base[tid] = reinterpret_cast<const uint32_t*>(a.ws + kWsBase)[tid];
  }
  for (int i = tid; i < 256; i += kHuffThreads) sorted[i] = a.ws[kWsSorted + i];
  const __amdgpu_buffer_rsrc_t rs = span(a.stream, 4u * a.stream_words);
  const __amdgpu_buffer_rsrc_t rsm = span(a.sm, static_cast<uint32_t>(a.n));

  for (int64_t g = blockIdx.x; g < a.groups; g += gridDim.x) {
    __syncthreads();   // tables ready; the previous group's stage is consumed
    // Every load of the group is issued before any is waited on: the block
    // lengths, the group's stream words (located by the group offsets alone,
    // checked against the lengths' sum below) and the sign/mantissa bytes.
    const uint64_t A = a.group_off[g], Aend = a.group_off[g + 1];
    const int64_t b = g * kHuffThreads + tid;
    const uint32_t blen = b < a.blocks ? a.block_len[b] : 0u;
    const bool span_ok = Aend >= A && Aend + 8 <= 4ull * a.stream_words;
    // the group's stream words, from the word holding its first byte, plus
    // two words of look-ahead
    const uint32_t w0 = static_cast<uint32_t>(A >> 2);
    const uint64_t nwords = span_ok ? ((Aend + 3) >> 2) - w0 + 2u : 0u;
    const bool staged = nwords <= static_cast<uint64_t>(kStageWords);
    uint32_t sw[kStageWords / kHuffThreads];
#pragma unroll
    for (int j = 0; j < kStageWords / kHuffThreads; ++j) {
      const uint32_t i = tid + kHuffThreads * j;
      sw[j] = staged && i < nwords ? __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (w0 + i), 0, 0) : 0u;
    }
    const int64_t sym0 = b * BINADE_HUFF_BLOCK;
    const int64_t left = a.n - sym0;
    const int cnt = left <= 0 ? 0 : left < BINADE_HUFF_BLOCK ? static_cast<int>(left) : BINADE_HUFF_BLOCK;
    // the block's 64 sign/mantissa bytes
    uint32_t smw[16];
    if (cnt == BINADE_HUFF_BLOCK) {
      const uint4* ps = reinterpret_cast<const uint4*>(a.sm + sym0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 q = ps[v];
        smw[4 * v] = q.x;
        smw[4 * v + 1] = q.y;
        smw[4 * v + 2] = q.z;
        smw[4 * v + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t v = 0;
        if (cnt > 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            v |= __builtin_amdgcn_raw_buffer_load_b8(rsm, static_cast<uint32_t>(sym0) + 4 * i + k, 0, 0)
                 << (8 * k);
        }
        smw[i] = v;
      }
    }
    // block offsets within the group: a scan of the lengths over the two waves
    uint32_t incl = wave_scan(blen);
    if ((tid & 63) == 63) wave_total[tid >> 6] = incl;
#pragma unroll
    for (int j = 0; j < kStageWords / kHuffThreads; ++j) {
      const uint32_t i = tid + kHuffThreads * j;
      if (staged && i < nwords) stage[i] = bswap32(sw[j]);
    }
    __syncthreads();
    if (tid >= 64) incl += wave_total[0];
    const uint32_t off = incl - blen;
    const uint32_t gbytes = wave_total[0] + wave_total[1];   // the group's bytes
    bool bad = !span_ok || Aend - A != gbytes;
    if (bad) {
      if (tid == 0 && a.status) atomicOr(a.status, BINADE_DEV_CORRUPT_STREAM);
      continue;
    }
    if (cnt == 0) continue;
    // bit buffer: the next bits at the top of a 64-bit value
    const uint64_t p = A + off;   // the block's first byte
    const uint32_t wi0 = static_cast<uint32_t>(p >> 2) - w0;
    const uint32_t skip = static_cast<uint32_t>(p & 3u) * 8u;
    uint32_t used = 0;
    uint16_t* po = a.out + sym0;
    const HuffLds L{lut, first, count, base, sorted, stage};
    if (staged) {
      if (__all(cnt == BINADE_HUFF_BLOCK))
        decode_block<true, true>(L, rs, w0, wi0, skip, cnt, smw, po, used, bad);
      else
        decode_block<true, false>(L, rs, w0, wi0, skip, cnt, smw, po, used, bad);
    } else {
      decode_block<false, false>(L, rs, w0, wi0, skip, cnt, smw, po, used, bad);
    }
    if (bad || (used + 7u) / 8u != blen) {
      if (a.status) atomicOr(a.status, BINADE_DEV_CORRUPT_STREAM);
    }
  }
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int64_t binade_huff_workspace_bytes(void) { return kWsBytes; }

extern "C" int32_t binade_huff_decode(const binade_huff* in, uint16_t* out, void* workspace,
                                      uint32_t* dev_status, void* stream) {
  if (in == nullptr || out == nullptr || workspace == nullptr || in->n <= 0 ||
      in->sm == nullptr || in->stream == nullptr || in->block_len == nullptr ||
      in->group_off == nullptr)
    return BINADE_EINVAL;
  for (int e = 0; e < 256; ++e)
    if (in->len[e] > kMaxLen) return BINADE_EINVAL;
  if (!aligned16(out) || !aligned16(in->sm) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(in->stream) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(in->group_off) & 7u) != 0)
    return BINADE_EUNSUPPORTED;
  if (in->stream_cap < in->stream_bytes + 8 || in->stream_cap / 4 > 0xFFFFFFFFull ||
      in->n > 0x7FFFFFFFll)
    return BINADE_EUNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  HuffTables t;
  for (int e = 0; e < 256; ++e) t.len[e] = in->len[e];
  hipLaunchKernelGGL(huff_tables_kernel, dim3(1), dim3(256), 0, s, t,
                     static_cast<uint8_t*>(workspace));
  int32_t st = launch_status();
  if (st != BINADE_OK) return st;
  HuffArgs a{};
  a.sm = in->sm;
  a.stream = in->stream;
  a.block_len = in->block_len;
  a.group_off = in->group_off;
  a.ws = static_cast<const uint8_t*>(workspace);
  a.out = out;
  a.status = dev_status;
  a.n = in->n;
  a.blocks = (in->n + BINADE_HUFF_BLOCK - 1) / BINADE_HUFF_BLOCK;
  a.groups = (a.blocks + BINADE_HUFF_GROUP - 1) / BINADE_HUFF_GROUP;
  a.stream_words = static_cast<uint32_t>(in->stream_cap / 4);
  // one workgroup per group (the loop covers grids past the launch limit)
  const int64_t grid = a.groups < (1ll << 30) ? a.groups : (1ll << 30);
  hipLaunchKernelGGL(huff_decode_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kHuffThreads), 0,
                     s, a);
  return launch_status();
}
