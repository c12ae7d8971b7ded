// BCR layouts: the chunk budget, chunk scores, the rows of whole chunks, and
// grown spans.  [Budgeted Cache Repair for Cross-Context KV-Cache Reuse:
// §3 "The layouts" (BCR-chunk, BCR-grow, BCR-single) and "The repair" (a
// group of rows scores the mean of its rows); §4.3 (tau = 0.25); App. A.2
// "The policy" step 2, "The random control" and Table 8; App. B Algorithm 1]
//
// chunk means: one thread per chunk sums the chunk's scores in fp64 in row
// order, divides by the chunk's own length and rounds once to fp32, so the
// ranking of chunks is decided on exactly the values the definition gives.
//
// expand: one block per score row.  A block scan over the listed chunks'
// lengths gives each chunk its place in the compacted row list; the block
// then writes rows and padding together and sets the mask bits with atomics.
//
// grow: one 1024-thread block per score row.  Every seed of the greedy walk
// is one of the b best rows (all rows ranked above a seed are taken already,
// and fewer than b are taken), so the block finds the b best with the radix
// search of the top-b selection, sorts them best first in LDS (bitonic, 64-bit
// keys: score descending, then index ascending), flags the seeds that can
// only span themselves (both neighbours below tau times the seed), and stages
// the row's scores and a chosen-row bitmap in LDS.  One wave then walks the
// seeds: a run of flagged seeds is taken 64 at a time (a bit test per lane
// and a prefix count against the budget); a seed that may grow holds a
// 64-row window of candidate rows on each side in registers and takes whole
// runs of rows per comparison (see grow_walk), so a long span costs a few
// ballots per 64 rows and a short one a single LDS round trip.
#include <type_traits>

#include "common.h"
#include "host_util.h"
#include "select_common.h"

namespace kvfix {

// ---------------------------------------------------------------------------
// chunk means
// ---------------------------------------------------------------------------

constexpr int kMeanBlock = 256;

__global__ __launch_bounds__(kMeanBlock) void chunk_means_kernel(const float* __restrict__ scores,
                                                                 int64_t total, int n, int B,
                                                                 int nc,
                                                                 float* __restrict__ means) {
  const int64_t c = (int64_t)blockIdx.x * kMeanBlock + threadIdx.x;
  if (c >= total) return;
  const int r = (int)(c / nc), i = (int)(c % nc);
  const int lo = i * B, hi = min(lo + B, n);
  const float* p = scores + (int64_t)r * n;
  double acc = 0.0;
  int j = lo;
  for (; j + 8 <= hi; j += 8) {                     // loads in batches, adds in row order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += (double)v[u];
  }
  for (; j < hi; ++j) acc += (double)p[j];
  means[c] = (float)(acc / (double)(hi - lo));
}

// ---------------------------------------------------------------------------
// expand chunks into rows
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kSelBlock) void expand_chunks_kernel(
    const int32_t* __restrict__ chunk_idx, int c, int n, int B, int words,
    int32_t* __restrict__ idx, int32_t* __restrict__ counts, uint32_t* __restrict__ mask) {
  __shared__ uint32_t scan[160];
  __shared__ int32_t s_first[kSelBlock], s_off[kSelBlock];
  const int row = blockIdx.x, t = threadIdx.x;
  const int nc = (int)(((int64_t)n + B - 1) / B);
  const int32_t* ci = chunk_idx + (int64_t)row * c;
  int32_t* out = idx + (int64_t)row * c * B;
  uint32_t* m = mask + (int64_t)row * words;
  for (int w = t; w < words; w += kSelBlock) m[w] = 0u;
  __syncthreads();
  uint32_t base = 0;
  for (int q0 = 0; q0 < c; q0 += kSelBlock) {       // the listed chunks, 1024 at a time
    const int q = q0 + t;
    int first = 0, len = 0;
    if (q < c) {
      const int k = ci[q];
      if (k >= 0 && k < nc) {                        // an id out of range lists no rows
        first = k * B;
        len = min(B, n - first);
      }
    }
    uint32_t tot;
    const uint32_t off = base + block_exclusive_scan((uint32_t)len, scan, &tot);
    s_first[t] = first;
    s_off[t] = (int32_t)off;
    __syncthreads();
    // the tile's rows, spread over the block: slot k belongs to the last
    // chunk whose offset is <= k (binary search over the tile's offsets)
    const int tile = min(kSelBlock, c - q0);
    for (uint32_t k = base + t; k < base + tot; k += kSelBlock) {
      int lo = 0, hi = tile - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((uint32_t)s_off[mid] <= k) lo = mid; else hi = mid - 1;
      }
      const int j = s_first[lo] + (int)(k - (uint32_t)s_off[lo]);
      out[k] = j;
      atomicOr(&m[j >> 5], 1u << (j & 31));
    }
    base += tot;
    __syncthreads();
  }
  for (int64_t k = (int64_t)base + t; k < (int64_t)c * B; k += kSelBlock) out[k] = -1;
  if (t == 0) counts[row] = (int32_t)base;
}

// ---------------------------------------------------------------------------
// grow
// ---------------------------------------------------------------------------

// Dynamic LDS of the grow kernel:
//   [0, a_bytes)                 radix histograms, then the sort keys, then
//                                the row's scores (when they fit)
//   [a_bytes, +4 words)          chosen-row bitmap
//   [.., +4 b)                   the b seeds, best first
struct GrowShape {
  int32_t P;                 // sort length: b rounded up to a power of two
  int32_t scores_in_lds;
  uint32_t a_bytes, bytes;
};

__host__ __device__ inline uint32_t align16u(uint64_t x) { return (uint32_t)((x + 15) & ~15ull); }

inline GrowShape grow_shape(int n, int b, bool scores_in_lds) {
  GrowShape g;
  int P = 1;
  while (P < b) P <<= 1;
  g.P = P;
  g.scores_in_lds = scores_in_lds;
  uint64_t a = (uint64_t)kSelWaves * 256 * 4;
  if ((uint64_t)P * 8 > a) a = (uint64_t)P * 8;
  if (scores_in_lds && (uint64_t)n * 4 > a) a = (uint64_t)n * 4;
  g.a_bytes = align16u(a);
  const uint64_t words = ((uint64_t)n + 31) / 32;
  const uint64_t total = (uint64_t)g.a_bytes + align16u(words * 4) + align16u((uint64_t)b * 4);
  g.bytes = total > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)total;
  return g;
}

__device__ __forceinline__ float lane_float(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Set bits lo..hi (inclusive) of the bitmap; called by one whole wave.
__device__ __forceinline__ void mark_rows(uint32_t* bits, int lo, int hi, int lane) {
  const int w0 = lo >> 5, w1 = hi >> 5;
  for (int w = w0 + lane; w <= w1; w += kWave) {
    const int a = max(lo, w << 5) - (w << 5), z = min(hi, (w << 5) + 31) - (w << 5);
    const uint32_t m = (z == 31 ? 0xFFFFFFFFu : ((1u << (z + 1)) - 1u)) & ~((1u << a) - 1u);
    bits[w] |= m;
  }
}

// Bit 31 of a seed entry: the seed spans itself alone whatever is chosen
// around it (both neighbours score below tau times the seed, or lie outside
// the row).
constexpr uint32_t kSingle = 0x80000000u;
// Steps a span takes one row at a time before it switches to whole runs.
constexpr int kRawSteps = 16;

__device__ __forceinline__ int ones_from(uint64_t m, int i) {   // consecutive set bits from bit i
  const uint64_t inv = ~(m >> i);
  return inv == 0 ? kWave - i : min((int)__builtin_ctzll(inv), kWave - i);
}

// One side of a growing span: a window of the 64 rows next to it (lane k:
// the k-th row outward), whether each may join (a run of ones ending at the
// first row that may not), how many are taken, and the running minimum of
// the side's scores (prefix minima, computed when both sides are alive).
struct Side {
  float v, pm;
  uint64_t ok;
  int i;
  float carry;               // minimum of the side's rows before this window
  bool have_pm;
};

// The greedy walk over the seeds (one wave; every branch is wave-uniform).
//
// A span takes, at each step, the higher of the two rows just outside it
// (the left one on a tie).  While both sides can grow this is the merge of
// the two sides' sequences of scores; taking the larger head each time is
// the same as merging the sequences' running minima (non-increasing), with
// ties to the left, because a row above its side's running minimum follows
// the row that set that minimum without the other side's head changing.  So
// each comparison takes a whole run of rows: from the left side every row
// whose running minimum is >= the right head, or from the right side every
// row whose running minimum is > the left head.
__device__ __forceinline__ void grow_walk(const float* A, uint32_t* bits,
                                          const uint32_t* seeds, int n, int b, double tau,
                                          int lane) {
  const uint64_t below = (1ull << lane) - 1ull;
  int left = b;
  for (int k0 = 0; k0 < b && left > 0; k0 += kWave) {
    const int kn = min(kWave, b - k0);
    const uint32_t e = lane < kn ? seeds[k0 + lane] : kSingle;
    const int my_s = (int)(e & ~kSingle);
    const float my_a = lane < kn ? A[my_s] : 0.0f;
    const uint64_t singles = __ballot((e & kSingle) != 0u);
    int q = 0;
    while (q < kn && left > 0) {
      // seeds q .. p-1 span themselves: take the ones not chosen yet, in order
      const int p = min(kn, q + ones_from(singles, q));
      if (p > q) {
        const bool mine = lane >= q && lane < p;
        const bool free_row = mine && !((bits[my_s >> 5] >> (my_s & 31)) & 1u);
        const uint64_t fr = __ballot(free_row);
        const bool take = free_row && __popcll(fr & below) < left;
        if (take) atomicOr(&bits[my_s >> 5], 1u << (my_s & 31));
        left -= min(__popcll(fr), left);
        q = p;
        continue;
      }
      // seed q may grow; its windows are read with its chosen bit (one round trip)
      const int s = __builtin_amdgcn_readlane(my_s, q);
      const double thr = tau * (double)lane_float(my_a, q);
      ++q;
      Side L, R;
      auto load = [&](Side& S, int first, int dir) {
        const int j = first + dir * lane;
        bool ok = j >= 0 && j < n;
        const float v = ok ? A[j] : 0.0f;
        ok = ok && !((bits[j >> 5] >> (j & 31)) & 1u) && (double)v >= thr;
        S.v = v;
        S.ok = __ballot(ok);
        S.i = 0;
        S.have_pm = false;
      };
      // running minima of a side from its current head on (rows taken
      // before the head are not part of the sequence still to merge)
      auto prefix_min = [&](Side& S) {
        if (S.have_pm) return;
        float m = lane < S.i ? __int_as_float(0x7f800000) : S.v;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const float y = __shfl_up(m, off);
          if (lane >= off) m = fminf(m, y);
        }
        S.pm = fminf(m, S.carry);
        S.have_pm = true;
      };
      load(R, s + 1, 1);
      load(L, s - 1, -1);
      const uint32_t wbits = __builtin_amdgcn_readfirstlane(bits[s >> 5]);
      if ((wbits >> (s & 31)) & 1u) continue;      // taken by an earlier span
      --left;
      int lo = s, hi = s, raw = 0;
      bool runs = false;
      L.carry = R.carry = __int_as_float(0x7f800000);   // +inf
      while (left > 0) {
        const bool la = (L.ok >> L.i) & 1u, ra = (R.ok >> R.i) & 1u;
        if (!la && !ra) break;
        bool take_left;
        int k;
        if (la && ra && !runs && raw < kRawSteps) {
          // the first steps of a span one row at a time, on the raw scores
          take_left = lane_float(L.v, L.i) >= lane_float(R.v, R.i);
          k = 1;
          ++raw;
        } else if (la && ra) {
          if (!runs) {                                 // from here on: whole runs
            runs = true;
            L.have_pm = R.have_pm = false;
          }
          prefix_min(L);
          prefix_min(R);
          const float xh = lane_float(L.pm, L.i), yh = lane_float(R.pm, R.i);
          take_left = xh >= yh;
          k = take_left ? ones_from(__ballot(L.pm >= yh) & L.ok, L.i)
                        : ones_from(__ballot(R.pm > xh) & R.ok, R.i);
        } else {
          take_left = la;                              // one side left: take its run
          k = take_left ? ones_from(L.ok, L.i) : ones_from(R.ok, R.i);
        }
        k = min(k, left);
        left -= k;
        Side& S = take_left ? L : R;
        if (take_left) lo -= k; else hi += k;
        S.i += k;
        if (S.i == kWave) {                            // window used up: the next 64 rows
          const float carry = S.have_pm ? lane_float(S.pm, kWave - 1) : S.carry;
          if (take_left) load(L, lo - 1, -1); else load(R, hi + 1, 1);
          S.carry = carry;
        }
      }
      mark_rows(bits, lo, hi, lane);
    }
  }
}

__global__ __launch_bounds__(kSelBlock) void select_grow_kernel(const float* __restrict__ scores,
                                                                int n, int b, double tau,
                                                                int32_t* __restrict__ idx,
                                                                uint32_t* __restrict__ mask,
                                                                int words, GrowShape G) {
  extern __shared__ __attribute__((aligned(16))) unsigned char glds[];
  __shared__ uint64_t scan64[160];
  __shared__ uint32_t ctab[2 * kCompactTab];
  __shared__ uint32_t sh[3];
  uint32_t* hist = reinterpret_cast<uint32_t*>(glds);
  uint64_t* keys = reinterpret_cast<uint64_t*>(glds);
  float* s_scores = reinterpret_cast<float*>(glds);
  uint32_t* bits = reinterpret_cast<uint32_t*>(glds + G.a_bytes);
  uint32_t* seeds = reinterpret_cast<uint32_t*>(glds + G.a_bytes + align16u((uint64_t)words * 4));
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* sc = scores + (int64_t)row * n;
  int32_t* out_idx = idx + (int64_t)row * b;
  uint32_t* out_mask = mask + (int64_t)row * words;
  const bool in_regs = n <= kSelBlock * kSelRegKeys;

  // 1. the b best rows
  uint32_t key[kSelRegKeys];
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kSelRegKeys; ++q) {
      const int j = t + q * kSelBlock;
      key[q] = j < n ? order_key(sc[j]) : 0u;
    }
  }
  uint32_t T, need_eq, eq_total;
  radix_threshold(key, in_regs, sc, n, b, hist, sh, &T, &need_eq, &eq_total);
  compact_topb(key, in_regs, sc, n, b, T, need_eq, eq_total, ctab,
               [&](uint32_t pos, int j, uint32_t k) {   // best score first, then the lower index
                 keys[pos] = ((uint64_t)(~k) << 32) | (uint32_t)j;
               },
               [](int, uint32_t) {});
  for (int i = b + t; i < G.P; i += kSelBlock) keys[i] = ~0ull;
  __syncthreads();

  // 2. bitonic sort of the P keys, ascending
  for (int kk = 2; kk <= G.P; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < G.P / 2; i += kSelBlock) {
        const int lo = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
        const int hi = lo | jj;
        const uint64_t x = keys[lo], y = keys[hi];
        const bool up = (lo & kk) == 0;
        if ((x > y) == up) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < b; i += kSelBlock) {
    const int sd = (int)(uint32_t)(keys[i] & 0xFFFFFFFFull);
    const double thr = tau * (double)sc[sd];
    const bool grows = (sd > 0 && (double)sc[sd - 1] >= thr) ||
                       (sd + 1 < n && (double)sc[sd + 1] >= thr);
    seeds[i] = (uint32_t)sd | (grows ? 0u : kSingle);
  }
  __syncthreads();

  // 3. stage the scores (the keys are dead), clear the bitmap
  if (G.scores_in_lds)
    for (int j = t; j < n; j += kSelBlock) s_scores[j] = sc[j];
  for (int w = t; w < words; w += kSelBlock) bits[w] = 0u;
  __syncthreads();

  // 4. the walk
  // (two call sites, so that each reads its scores through a typed pointer:
  // LDS or global, never a generic one)
  if (wave == 0) {
    if (G.scores_in_lds)
      grow_walk(s_scores, bits, seeds, n, b, tau, lane);
    else
      grow_walk(sc, bits, seeds, n, b, tau, lane);
  }
  __syncthreads();

  // 5. mask and ascending indices from the bitmap
  uint64_t base = 0;
  for (int w0 = 0; w0 < words; w0 += kSelBlock) {
    const int w = w0 + t;
    const uint32_t v = w < words ? bits[w] : 0u;
    if (w < words) out_mask[w] = v;
    uint64_t tot;
    uint64_t pos = base + block_exclusive_scan64((uint64_t)__popc(v), scan64, &tot);
    for (uint32_t x = v; x; x &= x - 1) {
      if (pos < (uint64_t)b) out_idx[pos] = (w << 5) + __ffs(x) - 1;
      ++pos;
    }
    base += tot;
  }
}

static int max_lds_per_block() {
  static std::atomic<int> cached{0};
  int v = cached.load();
  if (v == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0)
      v = 65536;
    cached.store(v);
  }
  return v;
}

}  // namespace kvfix

using namespace kvfix;

extern "C" int64_t kvfix_chunk_budget(int64_t n_tokens, int32_t chunk, int64_t rho_num,
                                      int64_t rho_den, int32_t rule) {
  // bounds that keep every product below 2^62
  if (n_tokens < 0 || chunk < 1 || rho_den < 1 || rho_num < 0 || rho_num > rho_den ||
      rho_den > ((int64_t)1 << 30) || n_tokens > ((int64_t)1 << 31))
    return -1;
  const int64_t nc = (n_tokens + chunk - 1) / chunk;
  // round(x / y) for x, y >= 0, a half rounding up: floor((2x + y) / 2y)
  auto round_div = [](int64_t x, int64_t y) { return (2 * x + y) / (2 * y); };
  int64_t c;
  if (rule == KVFIX_BUDGET_SKIP) {
    // skip when M < 2B or rho M < B, else round(rho M / B)
    if (n_tokens < 2 * (int64_t)chunk || rho_num * n_tokens < (int64_t)chunk * rho_den) return 0;
    c = round_div(rho_num * n_tokens, rho_den * (int64_t)chunk);
  } else if (rule == KVFIX_BUDGET_AT_LEAST_ONE) {
    c = round_div(rho_num * nc, rho_den);
    if (c < 1) c = 1;
  } else {
    return -1;
  }
  return c < nc ? c : nc;
}

extern "C" kvfix_status kvfix_chunk_means(const float* scores, int32_t n_rows, int32_t n,
                                          int32_t chunk, float* means, void* stream) {
  if (n_rows < 0 || n < 0 || chunk < 1) return KVFIX_ERR_ARG;
  if (n_rows == 0 || n == 0) return KVFIX_OK;
  if (scores == nullptr || means == nullptr) return KVFIX_ERR_ARG;
  const int nc = (int)(((int64_t)n + chunk - 1) / chunk);
  const int64_t total = (int64_t)n_rows * nc;
  const int64_t blocks = (total + kMeanBlock - 1) / kMeanBlock;
  if (blocks > kMaxGrid) return KVFIX_ERR_ARG;
  chunk_means_kernel<<<dim3((unsigned)blocks), dim3(kMeanBlock), 0, (hipStream_t)stream>>>(
      scores, total, n, chunk, nc, means);
  return launch_status();
}

extern "C" kvfix_status kvfix_expand_chunks(const int32_t* chunk_idx, int32_t n_rows, int32_t c,
                                            int32_t n, int32_t chunk, int32_t* idx,
                                            int32_t* counts, uint32_t* mask, void* stream) {
  if (n_rows < 0 || c < 0 || n < 0 || chunk < 1) return KVFIX_ERR_ARG;
  if ((int64_t)c * chunk > ((int64_t)1 << 31) - 1) return KVFIX_ERR_ARG;
  if (n_rows == 0) return KVFIX_OK;
  if (counts == nullptr || (n > 0 && mask == nullptr) ||
      (c > 0 && (chunk_idx == nullptr || idx == nullptr)))
    return KVFIX_ERR_ARG;
  if (n_rows > kMaxGrid) return KVFIX_ERR_ARG;
  const int words = (int)ceil_div(n, 32);
  expand_chunks_kernel<<<dim3((unsigned)n_rows), dim3(kSelBlock), 0, (hipStream_t)stream>>>(
      chunk_idx, c, n, chunk, words, idx, counts, mask);
  return launch_status();
}

extern "C" kvfix_status kvfix_select_grow(const float* scores, int32_t n_rows, int32_t n,
                                          int32_t b, double tau, int32_t* idx, uint32_t* mask,
                                          void* stream) {
  if (n_rows < 0 || n < 0 || b < 0 || b > n || !(tau == tau)) return KVFIX_ERR_ARG;
  if (n_rows == 0 || n == 0) return KVFIX_OK;
  if (scores == nullptr || mask == nullptr || (b > 0 && idx == nullptr)) return KVFIX_ERR_ARG;
  if (n_rows > kMaxGrid) return KVFIX_ERR_ARG;
  const int limit = max_lds_per_block() - 8192;     // room for the static LDS
  GrowShape G = grow_shape(n, b, true);
  if (G.bytes > (uint32_t)limit) G = grow_shape(n, b, false);
  if (G.bytes > (uint32_t)limit) return KVFIX_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&select_grow_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)G.bytes) != hipSuccess)
    return KVFIX_ERR_HIP;
  const int words = (int)ceil_div(n, 32);
  select_grow_kernel<<<dim3((unsigned)n_rows), dim3(kSelBlock), G.bytes, (hipStream_t)stream>>>(
      scores, n, b, tau, idx, mask, words, G);
  return launch_status();
}
