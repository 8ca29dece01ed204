// The exponent table and the format 2 (Rice) pack on the GPU: the same
// bytes binade_build_table and binade_pack_rice write on the host.
//
// "Binade" package page (pypi.org/project/binade), intro and "How it
// works": one table per tensor ranks the exponents by how often they occur;
// format 2 stores each weight's sign+mantissa byte and the Rice code of its
// exponent's rank; "Use": packing is a separate step before load. Doing it
// on the GPU keeps a large stack's weights in device memory from start to
// R4.
//
// Table: a histogram kernel (per-block LDS counts, then one 64-bit atomic
// add per bin), and one block that ranks the 256 exponents by count
// (descending, smaller exponent first on ties) and picks the Rice k with the
// fewest bits (ties to the smaller k).
//
// Pack, one wave per row-chunk of 2048 columns (lane l: columns 32l .. +31
// of the chunk):
//  1. count: sm bytes and remainder bits are written where they belong
//     (fixed positions); the chunk's unary bits and escapes are summed;
//  2. scan: block sums of 1024 chunks, a single-block scan of those, then
//     each block's chunks get their anchors and escape prefixes;
//  3. write: a wave prefix sum of the lanes' unary bits places each lane;
//     the chunk's bits are ORed together in LDS (one bit per weight) and
//     stored as words, the two words a chunk may share with its neighbours
//     by atomic OR into the zeroed plane.
#include <hip/hip_runtime.h>

#include <cstddef>

#include "binade.h"
#include "device_common.h"

namespace binade {
namespace {

using namespace dev;

constexpr int kPackWaves = 4;
constexpr int kScanBlock = 1024;       // chunks per scan block
constexpr int kStreamWords = 2048;     // LDS words per wave for a job's unary bits
constexpr int kHistCopies = 64;        // histogram copies per block (one per lane)

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, uint64_t words) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
       i += stride)
    p[i] = 0u;
}

// ---------------------------------------------------------------- table
__global__ __launch_bounds__(256) void hist_kernel(const uint16_t* w, int64_t n,
                                                   unsigned long long* counts) {
  // kHistCopies counts per bin, lane l adding into copy l % kHistCopies:
  // the lanes of one instruction never hit the same word, and lanes that hit
  // the same bin fall in different banks (bin e, copy k at word
  // e * (kHistCopies + 1) + k). Two 16-byte loads per thread are in flight
  // before their counts are added.
  constexpr int kStride = kHistCopies + 1;
  __shared__ uint32_t h[256 * kStride];
  uint32_t* mine = h + threadIdx.x % kHistCopies;
  for (int e = threadIdx.x; e < 256 * kStride; e += blockDim.x) h[e] = 0u;
  __syncthreads();
  auto add8 = [&](const uint4 v) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      atomicAdd(&mine[((d[i] >> 7) & 0xFFu) * kStride], 1u);
      atomicAdd(&mine[((d[i] >> 23) & 0xFFu) * kStride], 1u);
    }
  };
  const int64_t groups = n >> 3;   // 8 weights per 16-byte load
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const uint4* w4 = reinterpret_cast<const uint4*>(w);
  int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; g + stride < groups; g += 2 * stride) {
    const uint4 v0 = w4[g], v1 = w4[g + stride];
    add8(v0);
    add8(v1);
  }
  if (g < groups) add8(w4[g]);
  if (blockIdx.x == 0)
    for (int64_t i = (groups << 3) + threadIdx.x; i < n; i += blockDim.x)
      atomicAdd(&mine[((w[i] >> 7) & 0xFFu) * kStride], 1u);
  __syncthreads();
  const int e = threadIdx.x;
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < kHistCopies; ++k) c += h[e * kStride + k];
  if (c) atomicAdd(&counts[e], static_cast<unsigned long long>(c));
}

__global__ __launch_bounds__(256) void table_kernel(const unsigned long long* counts,
                                                    binade_table* t) {
  __shared__ unsigned long long pc[256];   // counts of the present exponents (any order)
  __shared__ uint32_t pe[256];             // and those exponents
  __shared__ unsigned long long by_rank[256];
  __shared__ unsigned long long bits_k[8];
  __shared__ uint32_t n_present;
  const int e = threadIdx.x;
  const unsigned long long ce = counts[e];
  by_rank[e] = 0ull;
  if (e == 0) n_present = 0u;
  __syncthreads();
  if (ce) {
    const uint32_t slot = atomicAdd(&n_present, 1u);
    pc[slot] = ce;
    pe[slot] = static_cast<uint32_t>(e);
  }
  __syncthreads();
  const uint32_t np = n_present;
  // rank = present exponents before e in (count desc, exponent asc) order;
  // it depends only on the counts, not on the slots' order
  uint32_t rank = 0;
  for (uint32_t o = 0; o < np; ++o) {
    const unsigned long long co = pc[o];
    rank += (co > ce || (co == ce && pe[o] < static_cast<uint32_t>(e))) ? 1u : 0u;
  }
  if (ce) by_rank[rank] = ce;
  __syncthreads();
  const uint32_t n = n_present;
  t->rank_of_exp[e] = ce ? static_cast<uint16_t>(rank) : static_cast<uint16_t>(0xFFFF);
  if (ce) t->exp_of_rank[rank] = static_cast<uint8_t>(e);
  if (static_cast<uint32_t>(e) >= n) t->exp_of_rank[e] = 0;
  t->count_of_rank[e] = by_rank[e];
  if (e < 8) {
    unsigned long long bits = 0, total = 0;
    for (uint32_t r = 0; r < n; ++r) {
      bits += by_rank[r] * ((r >> e) + 1u);
      total += by_rank[r];
    }
    bits_k[e] = bits + static_cast<unsigned long long>(e) * total;
  }
  __syncthreads();
  if (e == 0) {
    uint32_t best = 0;
    for (uint32_t k = 1; k < 8; ++k)
      if (bits_k[k] < bits_k[best]) best = k;   // strict: ties keep the smaller k
    t->n = n;
    t->k = best;
  }
}

// ---------------------------------------------------------------- pack
struct PackArgs {
  const uint16_t* w;
  uint8_t* sm;
  uint32_t* unary;
  uint32_t* rem;
  uint64_t* anchor;
  uint32_t* esc_pre;
  uint32_t* chunk_bits;
  uint32_t* chunk_esc;
  unsigned long long* block_bits;   // per scan block: sum, then exclusive offset
  uint32_t* block_esc;
  uint32_t* status;
  uint64_t unary_cap;               // words the unary plane holds
  uint64_t expect_bits;             // the table's unary bits for this tensor
  uint64_t expect_esc;
  int64_t rows;
  int64_t chunks;
  int64_t jobs;
  int32_t cols;
  uint32_t C;                       // chunks per row
  uint32_t G, L;                    // C == 1: rows per job, lanes per row (cols / 32)
  uint32_t lane_recip;              // C == 1, L > 1: ceil(2^32 / L), lane / L = mulhi(lane, lane_recip)
  uint32_t k, n;
  uint16_t rank_of_exp[256];
};

__device__ __forceinline__ void pack_flag(uint32_t* status, uint32_t bits) {
  if (status != nullptr) atomicOr(status, bits);
}

// The lane's 32 weights (columns 32t .. 32t+31 of row `row`) and their
// ranks, when live.
__device__ __forceinline__ void lane_ranks(const PackArgs& a, const uint16_t* rk, int64_t row,
                                           uint32_t t, uint32_t (&b)[16], uint32_t (&r)[32],
                                           bool& bad) {
  const uint4* p = reinterpret_cast<const uint4*>(a.w + row * a.cols + 32 * t);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint4 q = p[v];
    b[4 * v] = q.x;
    b[4 * v + 1] = q.y;
    b[4 * v + 2] = q.z;
    b[4 * v + 3] = q.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t r0 = rk[(b[i] >> 7) & 0xFFu], r1 = rk[(b[i] >> 23) & 0xFFu];
    bad = bad || r0 >= a.n || r1 >= a.n;   // absent exponents hold 0xFFFF
    r[2 * i] = r0 < 256u ? r0 : 0u;
    r[2 * i + 1] = r1 < 256u ? r1 : 0u;
  }
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

__device__ __forceinline__ uint32_t lane_scan(uint32_t v) {   // inclusive
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const uint32_t o = __shfl_up(v, s, 64);
    if ((threadIdx.x & 63u) >= static_cast<uint32_t>(s)) v += o;
  }
  return v;
}

// A job is one row-chunk when rows are longer than a chunk (C > 1), else G
// whole rows (one chunk each) on L = cols / 32 lanes apiece. The lane's row,
// its tile within the row, whether it holds weights, its row within the
// job, and the job's first chunk.
struct PackLane {
  int64_t row;
  uint32_t t, rl;
  bool live;
  int64_t c0;
};

__device__ __forceinline__ PackLane pack_lane(const PackArgs& a, uint32_t j, uint32_t lane) {
  PackLane p;
  if (a.C > 1) {
    const uint32_t row = j / a.C;
    const uint32_t q = j - row * a.C;
    p.row = row;
    p.t = q * 64u + lane;
    p.rl = 0;
    p.live = p.t < (static_cast<uint32_t>(a.cols) >> 5);
    p.c0 = j;
  } else {
    const int64_t row0 = static_cast<int64_t>(j) * a.G;
    p.rl = a.L == 1u ? lane : __umulhi(lane, a.lane_recip);   // lane / L
    p.t = lane - p.rl * a.L;
    p.row = row0 + p.rl;
    p.live = p.rl < a.G && p.row < a.rows;
    p.c0 = row0;
  }
  return p;
}

__global__ __launch_bounds__(64 * kPackWaves) void pack_count_kernel(PackArgs args) {
  __shared__ uint16_t rk[256];
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const PackArgs& a = *(const PackArgs*)kp;
  rk[threadIdx.x] = a.rank_of_exp[threadIdx.x];
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t j = blockIdx.x * kPackWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (j >= a.jobs) return;
  const PackLane pl = pack_lane(a, j, lane);
  uint32_t b[16], r[32];
  bool bad = false;
  uint32_t bits = 0, esc = 0;
  if (pl.live) {
    lane_ranks(a, rk, pl.row, pl.t, b, r, bad);
    uint32_t sm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = b[2 * i + h];
        const uint32_t s0 = ((x >> 8) & 0x80u) | (x & 0x7Fu);
        const uint32_t s1 = ((x >> 24) & 0x80u) | ((x >> 16) & 0x7Fu);
        o |= (s0 | (s1 << 8)) << (16 * h);
      }
      sm[i] = o;
    }
    uint4* ps = reinterpret_cast<uint4*>(a.sm + pl.row * a.cols + 32 * pl.t);
    ps[0] = make_uint4(sm[0], sm[1], sm[2], sm[3]);
    ps[1] = make_uint4(sm[4], sm[5], sm[6], sm[7]);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      bits += (r[i] >> a.k) + 1u;
      esc += r[i] >= 15u ? 1u : 0u;
    }
    if (a.k > 0) {
      // the lane's 32 remainders: k whole words from word (row*J + t) * k
      const uint32_t k = a.k, mask = (1u << k) - 1u;
      uint32_t* pr = a.rem + (static_cast<uint64_t>(pl.row) * (a.cols >> 5) + pl.t) * k;
      uint64_t acc = 0;
      uint32_t fill = 0, out = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        acc |= static_cast<uint64_t>(r[i] & mask) << fill;
        fill += k;
        if (fill >= 32) {
          pr[out++] = static_cast<uint32_t>(acc);
          acc >>= 32;
          fill -= 32;
        }
      }
    }
  }
  if (a.C > 1) {
    bits = wave_sum(bits);
    esc = wave_sum(esc);
    if (lane == 0) {
      a.chunk_bits[j] = bits;
      a.chunk_esc[j] = esc;
    }
  } else {
    // one chunk per row: the row's sums from the wave's prefix sums, written
    // by the row's last lane
    const uint32_t ib = lane_scan(bits), ie = lane_scan(esc);
    const uint32_t first = pl.rl * a.L;
    const uint32_t src = first > 0 ? first - 1u : 0u;
    const uint32_t pb = __shfl(ib, static_cast<int>(src), 64);
    const uint32_t pe = __shfl(ie, static_cast<int>(src), 64);
    if (pl.live && pl.t + 1 == a.L) {
      a.chunk_bits[pl.row] = ib - (first > 0 ? pb : 0u);
      a.chunk_esc[pl.row] = ie - (first > 0 ? pe : 0u);
    }
  }
  if (__any(bad) && lane == 0) pack_flag(a.status, BINADE_DEV_CORRUPT_STREAM);
}

// Inclusive sum over the block's 256 threads (Hillis-Steele in LDS).
template <typename T>
__device__ __forceinline__ T block_incl(T v, T* s) {
  s[threadIdx.x] = v;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const T o = threadIdx.x >= static_cast<uint32_t>(d) ? s[threadIdx.x - d] : T(0);
    __syncthreads();
    v += o;
    s[threadIdx.x] = v;
    __syncthreads();
  }
  return v;
}

// Sums of each scan block's chunks (4 per thread).
__global__ __launch_bounds__(256) void block_sums_kernel(PackArgs a) {
  __shared__ unsigned long long sb[256];
  __shared__ uint32_t se[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanBlock + 4 * threadIdx.x;
  unsigned long long bits = 0;
  uint32_t esc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (base + i < a.chunks) {
      bits += a.chunk_bits[base + i];
      esc += a.chunk_esc[base + i];
    }
  bits = block_incl(bits, sb);
  esc = block_incl(esc, se);
  if (threadIdx.x == 255) {
    a.block_bits[blockIdx.x] = bits;
    a.block_esc[blockIdx.x] = esc;
  }
}

// One block: block sums -> exclusive offsets (in place), and the totals.
__global__ __launch_bounds__(256) void block_offsets_kernel(PackArgs a, int64_t nb) {
  __shared__ unsigned long long sb[256];
  __shared__ uint32_t se[256];
  unsigned long long carry_b = 0;
  uint32_t carry_e = 0;
  for (int64_t base = 0; base < nb; base += 256) {
    const int64_t i = base + threadIdx.x;
    const unsigned long long vb = i < nb ? a.block_bits[i] : 0ull;
    const uint32_t ve = i < nb ? a.block_esc[i] : 0u;
    const unsigned long long ib = block_incl(vb, sb);
    const uint32_t ie = block_incl(ve, se);
    if (i < nb) {
      a.block_bits[i] = carry_b + ib - vb;
      a.block_esc[i] = carry_e + ie - ve;
    }
    carry_b += sb[255];
    carry_e += se[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.anchor[a.chunks] = carry_b;
    a.esc_pre[a.chunks] = carry_e;
    if (carry_b != a.expect_bits || carry_e != a.expect_esc)
      pack_flag(a.status, BINADE_DEV_CORRUPT_STREAM);   // the table is not this tensor's
  }
}

// Each chunk's anchor and escape prefix.
__global__ __launch_bounds__(256) void chunk_offsets_kernel(PackArgs a) {
  __shared__ unsigned long long sb[256];
  __shared__ uint32_t se[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanBlock + 4 * threadIdx.x;
  uint32_t cb[4], ce[4];
  unsigned long long bits = 0;
  uint32_t esc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cb[i] = base + i < a.chunks ? a.chunk_bits[base + i] : 0u;
    ce[i] = base + i < a.chunks ? a.chunk_esc[base + i] : 0u;
    bits += cb[i];
    esc += ce[i];
  }
  const unsigned long long ib = block_incl(bits, sb);
  const uint32_t ie = block_incl(esc, se);
  unsigned long long pb = a.block_bits[blockIdx.x] + ib - bits;
  uint32_t pe = a.block_esc[blockIdx.x] + ie - esc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (base + i < a.chunks) {
      a.anchor[base + i] = pb;
      a.esc_pre[base + i] = pe;
      pb += cb[i];
      pe += ce[i];
    }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__global__ __launch_bounds__(64 * kPackWaves) void pack_unary_kernel(PackArgs args) {
  __shared__ uint16_t rk[256];
  __shared__ uint32_t stream[kPackWaves][kStreamWords];
  const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const PackArgs& a = *(const PackArgs*)kp;
  rk[threadIdx.x] = a.rank_of_exp[threadIdx.x];
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t j = blockIdx.x * kPackWaves + wave;
  if (j >= a.jobs) return;
  const PackLane pl = pack_lane(a, j, lane);
  uint32_t b[16], r[32];
  bool bad = false;
  uint32_t bits = 0;
  if (pl.live) {
    lane_ranks(a, rk, pl.row, pl.t, b, r, bad);
#pragma unroll
    for (int i = 0; i < 32; ++i) bits += (r[i] >> a.k) + 1u;
  }
  // the job's chunks are consecutive in the stream: one bit range from the
  // first chunk's anchor
  const uint32_t incl = lane_scan(bits);
  const uint32_t total = __shfl(incl, 63, 64);
  const uint64_t A = a.anchor[pl.c0];
  const uint32_t s0 = static_cast<uint32_t>(A & 31u);
  const uint64_t w0 = A >> 5;
  const uint32_t nwords = (s0 + total + 31u) >> 5;
  uint32_t pos = s0 + incl - bits;   // the lane's first bit, from word w0
  if (nwords <= static_cast<uint32_t>(kStreamWords)) {
    uint32_t* s = stream[wave];
    for (uint32_t i = lane; i < nwords; i += 64u) s[i] = 0u;
    wave_sync_lds();
    if (pl.live) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        pos += r[i] >> a.k;
        atomicOr(&s[pos >> 5], 1u << (pos & 31u));
        ++pos;
      }
    }
    wave_sync_lds();
    for (uint32_t i = lane; i < nwords; i += 64u) {
      const uint32_t v = s[i];
      if (w0 + i >= a.unary_cap) {   // more bits than the table promised: not this tensor's table
        pack_flag(a.status, BINADE_DEV_CORRUPT_STREAM);
      } else if (i == 0 || i + 1 == nwords) {
        if (v) atomicOr(a.unary + w0 + i, v);   // may be shared with a neighbouring job
      } else {
        a.unary[w0 + i] = v;
      }
    }
  } else if (pl.live) {
    // a job of very long codes: its one bits straight into the plane
#pragma unroll 1
    for (int i = 0; i < 32; ++i) {
      pos += r[i] >> a.k;
      if (w0 + (pos >> 5) < a.unary_cap)
        atomicOr(a.unary + w0 + (pos >> 5), 1u << (pos & 31u));
      else
        pack_flag(a.status, BINADE_DEV_CORRUPT_STREAM);
      ++pos;
    }
  }
}

uint64_t pack_chunks(int64_t rows, int64_t cols) {
  return static_cast<uint64_t>(rows) * static_cast<uint64_t>((cols + BINADE_CHUNK - 1) / BINADE_CHUNK);
}

uint32_t zero_blocks(uint64_t words) {
  const uint64_t b = (words + 255) / 256;
  return static_cast<uint32_t>(b < 4096 ? b : 4096);
}

}  // namespace
}  // namespace binade

using namespace binade;

extern "C" int64_t binade_pack_gpu_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  const uint64_t chunks = pack_chunks(rows, cols);
  const uint64_t nb = (chunks + kScanBlock - 1) / kScanBlock;
  const uint64_t bytes = 8 * chunks + 12 * nb + 256;
  return static_cast<int64_t>(bytes > 2048 ? bytes : 2048);   // >= the table's 256 counts
}

extern "C" int32_t binade_build_table_gpu(const uint16_t* w, int64_t n, void* workspace,
                                          binade_table* table, void* stream) {
  if (w == nullptr || n <= 0 || workspace == nullptr || table == nullptr) return BINADE_EINVAL;
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(table) & 7u) != 0)
    return BINADE_EUNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  auto* counts = static_cast<unsigned long long*>(workspace);
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(counts), static_cast<uint64_t>(512));
  int32_t st = launch_status();
  if (st != BINADE_OK) return st;
  const int64_t groups = n >> 3;
  int64_t blocks = (groups + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  hipLaunchKernelGGL(hist_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, w, n,
                     counts);
  st = launch_status();
  if (st != BINADE_OK) return st;
  hipLaunchKernelGGL(table_kernel, dim3(1), dim3(256), 0, s, counts, table);
  return launch_status();
}

extern "C" int32_t binade_pack_rice_gpu(const uint16_t* w, int64_t rows, int64_t cols,
                                        const binade_table* t, binade_rice* out,
                                        void* workspace, uint32_t* dev_status, void* stream) {
  if (w == nullptr || t == nullptr || out == nullptr || workspace == nullptr || rows <= 0 ||
      cols <= 0)
    return BINADE_EINVAL;
  if (cols % 32 != 0 || cols > (1 << 30)) return BINADE_EUNSUPPORTED;
  binade_sizes sz;
  int32_t st = binade_sizes_of(t, rows, cols, &sz);
  if (st != BINADE_OK) return st;
  if (out->sm == nullptr || out->unary == nullptr || out->anchor == nullptr ||
      out->esc_pre == nullptr || (t->k > 0 && out->rem == nullptr))
    return BINADE_EINVAL;
  if (out->unary_words < sz.unary_words || (t->k > 0 && out->rem_words < sz.rem_words))
    return BINADE_ENOSPACE;
  if (!aligned16(w) || !aligned16(out->sm) || (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(out->anchor) & 7u) != 0)
    return BINADE_EUNSUPPORTED;
  const uint64_t chunks = pack_chunks(rows, cols);
  if (chunks >= (1ull << 31) || sz.n_esc > 0xFFFFFFFFull) return BINADE_EUNSUPPORTED;
  const uint64_t nb = (chunks + kScanBlock - 1) / kScanBlock;

  PackArgs a{};
  a.w = w;
  a.sm = out->sm;
  a.unary = out->unary;
  a.rem = t->k > 0 ? out->rem : nullptr;
  a.anchor = out->anchor;
  a.esc_pre = out->esc_pre;
  char* ws = static_cast<char*>(workspace);
  a.block_bits = reinterpret_cast<unsigned long long*>(ws);
  a.chunk_bits = reinterpret_cast<uint32_t*>(ws + 8 * nb);
  a.chunk_esc = a.chunk_bits + chunks;
  a.block_esc = a.chunk_esc + chunks;
  a.status = dev_status;
  a.unary_cap = out->unary_words;
  a.expect_bits = sz.unary_bits;
  a.expect_esc = sz.n_esc;
  a.rows = rows;
  a.chunks = static_cast<int64_t>(chunks);
  a.cols = static_cast<int32_t>(cols);
  a.C = static_cast<uint32_t>((cols + BINADE_CHUNK - 1) / BINADE_CHUNK);
  if (a.C > 1) {
    a.jobs = static_cast<int64_t>(chunks);
  } else {
    a.L = static_cast<uint32_t>(cols / 32);
    a.G = 64u / a.L;
    a.lane_recip = a.L > 1 ? static_cast<uint32_t>(((1ull << 32) + a.L - 1) / a.L) : 0u;
    a.jobs = (rows + a.G - 1) / a.G;
  }
  a.k = t->k;
  a.n = t->n;
  for (int e = 0; e < 256; ++e) a.rank_of_exp[e] = t->rank_of_exp[e];

  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_words_kernel, dim3(zero_blocks(out->unary_words)), dim3(256), 0, s,
                     out->unary, out->unary_words);
  if ((st = launch_status()) != BINADE_OK) return st;
  if (t->k > 0) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(zero_blocks(out->rem_words)), dim3(256), 0, s,
                       out->rem, out->rem_words);
    if ((st = launch_status()) != BINADE_OK) return st;
  }
  const dim3 wave_grid(static_cast<uint32_t>((a.jobs + kPackWaves - 1) / kPackWaves));
  hipLaunchKernelGGL(pack_count_kernel, wave_grid, dim3(64 * kPackWaves), 0, s, a);
  if ((st = launch_status()) != BINADE_OK) return st;
  hipLaunchKernelGGL(block_sums_kernel, dim3(static_cast<uint32_t>(nb)), dim3(256), 0, s, a);
  if ((st = launch_status()) != BINADE_OK) return st;
  hipLaunchKernelGGL(block_offsets_kernel, dim3(1), dim3(256), 0, s, a, static_cast<int64_t>(nb));
  if ((st = launch_status()) != BINADE_OK) return st;
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(static_cast<uint32_t>(nb)), dim3(256), 0, s, a);
  if ((st = launch_status()) != BINADE_OK) return st;
  hipLaunchKernelGGL(pack_unary_kernel, wave_grid, dim3(64 * kPackWaves), 0, s, a);
  if ((st = launch_status()) != BINADE_OK) return st;

  out->rows = rows;
  out->cols = cols;
  out->k = t->k;
  out->n = t->n;
  for (int e = 0; e < 256; ++e) out->exp_of_rank[e] = t->exp_of_rank[e];
  out->unary_bits = sz.unary_bits;
  out->n_esc = sz.n_esc;
  return BINADE_OK;
}
