// Rotary re-alignment, probe-mean fit and fused correction apply.
//
// rope_shift : a1, stand-alone batched rotation of a key plane.
// fit_mean   : a5, mu[l][s][h] = mean over probes of fresh - align(reuse) - A B,
//              plus the exact copy of the fresh probe rows into the output.
// apply      : a6, out_j = round(align(reuse_j) + w_j mu + A_j B) for non-probes.
//
// Work split: one "unit" is a (layer, segment, head); its rows are the tokens.
// rope_shift and apply give each 256-thread block a chunk of one unit's rows,
// so the block's rotary table (fp64 sincos, one per segment) and its mu / B
// constants live in LDS and registers for the whole chunk.  fit_mean gives
// each block one whole unit and reduces in a fixed order (deterministic).
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "host_util.h"

namespace kvfix {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
// Rows per block of the streaming kernels (the block stages per-row data
// for that many rows in LDS).
constexpr int kRowsPerBlock = 2048;

// Wait until every vector-memory load this wave issued has returned.  Placed
// after a batch of row loads, it lets the following stores issue back to back
// (across per-row branches the compiler cannot count outstanding loads and
// would otherwise wait for every earlier store before each store).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
constexpr int kMaxRowsPerBlock = kRowsPerBlock;

// ---------------------------------------------------------------------------
// rope_shift
// ---------------------------------------------------------------------------

struct RopeShiftParams {
  DPlane src, dst;
  RopeArgs rope;
  int32_t S, H, n, chunks, rows_per_block;
};

template <typename T, int HD, int STYLE>
__global__ __launch_bounds__(kBlock) void rope_shift_kernel(RopeShiftParams P) {
  using M = RowMap<T, HD, STYLE>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW, U = 4;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane % G, rw = lane / G;
  const int chunk = blockIdx.x % P.chunks;
  int unit = blockIdx.x / P.chunks;
  const int h = unit % P.H; unit /= P.H;
  const int s = unit % P.S;
  const int l = unit / P.S;
  const int j_begin = chunk * P.rows_per_block;
  const int j_end = min(P.n, j_begin + P.rows_per_block);

  __shared__ double tc[HD / 2], ts[HD / 2];
  __shared__ int32_t spin[kMaxRowsPerBlock + 1], spout[kMaxRowsPerBlock + 1];
  rope_table<HD, double>(P.rope, P.rope.delta[s], tc, ts);
  const int pin0 = stage_pages(P.src, s, j_begin, j_end, spin);
  const int pout0 = stage_pages(P.dst, s, j_begin, j_end, spout);
  __syncthreads();
  double cs[V], sn[V];
#pragma unroll
  for (int m = 0; m < V; ++m) { cs[m] = tc[g * V + m]; sn[m] = ts[g * V + m]; }

  constexpr int kStep = kWavesPerBlock * RPW;
  for (int j0 = j_begin + wave * RPW + rw; j0 < j_end; j0 += kStep * U) {
    vu4 r0[U], r1[U];
    int64_t oo[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kStep;
      live[u] = j < j_end;
      int64_t io = -1;
      oo[u] = -1;
      if (live[u]) {
        io = row_offset_staged(P.src, l, s, h, j, spin, pin0);
        oo[u] = row_offset_staged(P.dst, l, s, h, j, spout, pout0);
        live[u] = io >= 0 && oo[u] >= 0;
      }
      if (live[u]) {
        const T* row = reinterpret_cast<const T*>(P.src.data) + io;
        r0[u] = ld16(row + M::off0(g));
        r1[u] = ld16(row + M::off1(g));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      double p0[V], p1[V], a[V], b[V];
      Cd::unpack(r0[u], p0);
      Cd::unpack(r1[u], p1);
      parts_to_pairs<STYLE, V>(p0, p1, a, b);
      rotate_pairs<V>(a, b, cs, sn);
      pairs_to_parts<STYLE, V>(a, b, p0, p1);
      T* row = reinterpret_cast<T*>(P.dst.data) + oo[u];
      st16(row + M::off0(g), Cd::pack(p0));
      st16(row + M::off1(g), Cd::pack(p1));
    }
  }
}

// ---------------------------------------------------------------------------
// fit_mean: two stages.  Stage 1 gives each block a slice of <= kFitRows
// probe rows of one (layer, segment, head); the block scatters the fresh rows
// and writes, in fp64, the sum of fresh - align(reuse) over its slice and the
// sum of the slice's rank-state rows A_j.  Stage 2 adds a unit's slices in
// slice order and forms mu = (sum(fresh - align(reuse)) - (sum A_j) B) / b,
// which is the mean of fresh - align(reuse) - A_j B by linearity.
// Fixed order throughout.
// ---------------------------------------------------------------------------

constexpr int kFitRows = 256;
constexpr int kFitMaxRank = 8;
// A partial row: HD residual sums, kFitMaxRank sums of rank-state rows, and
// the number of probe-set members (indices inside [0, n)) of the slice.
__host__ __device__ constexpr int fit_row_width(int hd) { return hd + kFitMaxRank + 1; }

struct FitParams {
  DPlane fresh, reuse, out;
  int32_t has_out, fresh_by_slot;
  const int32_t* idx;
  int32_t b, parts;
  DLowRank lr;
  RopeArgs rope;
  double* partial;          // [units][parts][kFitRowWidth(HD)]
  int32_t S, H, n;
  int32_t idx_heads;        // 1: idx [S][b]; H: idx [S][H][b] (per head)
  const int32_t* cover;     // rank state only for rows j < cover[s] (NULL: all)
};

template <typename T, int HD, int STYLE>
__global__ __launch_bounds__(kBlock) void fit_partial_kernel(FitParams P) {
  using M = PartMap<T, HD, STYLE>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW, U = 4;
  constexpr int PW = fit_row_width(HD);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane % G, rw = lane / G;
  const int part = blockIdx.x % P.parts;
  int unit = blockIdx.x / P.parts;
  const int h = unit % P.H; unit /= P.H;
  const int s = unit % P.S;
  const int l = unit / P.S;
  const int k_begin = part * kFitRows;
  const int k_end = min(P.b, k_begin + kFitRows);
  const int nk = k_end - k_begin;

  __shared__ double tc[HD / 2], ts[HD / 2];
  __shared__ double red[kWavesPerBlock][HD];
  __shared__ int32_t sj[kFitRows], spf[kFitRows], spr[kFitRows], spo[kFitRows];
  if constexpr (STYLE != kStyleNone) rope_table<HD, double>(P.rope, P.rope.delta[s], tc, ts);
  // Stage the slice's probe indices and their page ids.  Thread t < nk also
  // loads the rank-state row of slot t now (summed after the main loop), so
  // that load shares a memory round trip with the staging.
  const int32_t* idx = P.idx + ((int64_t)s * P.idx_heads + (P.idx_heads > 1 ? h : 0)) * P.b;
  const int cov = P.cover ? P.cover[s] : P.n;
  const int rank = P.lr.rank;
  double* outp = P.partial + (int64_t)blockIdx.x * PW;
  float arow[kFitMaxRank];
#pragma unroll
  for (int k = 0; k < kFitMaxRank; ++k) arow[k] = 0.0f;
  int member = 0;
  {
    const int i = threadIdx.x;
    if (i < nk) {
      const int k = k_begin + i;
      const int j = idx[k];
      const bool ok = j >= 0 && j < P.n;            // an index out of range is padding
      member = ok;
      sj[i] = ok ? j : -1;
      spf[i] = ok ? page_of(P.fresh, s, P.fresh_by_slot ? k : j) : -1;
      spr[i] = ok ? page_of(P.reuse, s, j) : -1;
      spo[i] = ok && P.has_out ? page_of(P.out, s, j) : 0;
      if (ok && rank > 0 && j < cov) {                // no rank state past the covered prefix
        const float* Ar = P.lr.A + l * P.lr.sA_layer + s * P.lr.sA_seg + h * P.lr.sA_head +
                          (int64_t)j * rank;
#pragma unroll
        for (int kk = 0; kk < kFitMaxRank; ++kk) arow[kk] = kk < rank ? Ar[kk] : 0.0f;
      }
    }
  }
  const int members = __syncthreads_count(member);
  static_assert(kFitRows <= kBlock, "one probe row per thread in the rank-state sum");
  double cs[V], ss[V];
  if constexpr (STYLE != kStyleNone) {
    const bool first_half = STYLE == kStyleHalf && g < M::X;
#pragma unroll
    for (int m = 0; m < V; ++m) {
      cs[m] = tc[M::pair(g, m)];
      ss[m] = first_half ? -ts[M::pair(g, m)] : ts[M::pair(g, m)];
    }
  }
  double acc[V];
#pragma unroll
  for (int m = 0; m < V; ++m) acc[m] = 0.0;

  constexpr int kStep = kWavesPerBlock * RPW;
  for (int i0 = wave * RPW + rw; i0 < nk; i0 += kStep * U) {
    vu4 f[U], q[U];
    int64_t oo[U];
    bool live[U];
    // unconditional loads (a dead slot reads the plane's first vector)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kStep;
      const int j = i < nk ? sj[i] : -1;
      int64_t fo = -1, ro = -1;
      oo[u] = -1;
      if (j >= 0) {
        fo = row_offset_page(P.fresh, l, s, h, P.fresh_by_slot ? k_begin + i : j, spf[i]);
        ro = row_offset_page(P.reuse, l, s, h, j, spr[i]);
        if (P.has_out) oo[u] = row_offset_page(P.out, l, s, h, j, spo[i]);
      }
      live[u] = j >= 0 && fo >= 0 && ro >= 0 && (!P.has_out || oo[u] >= 0);
      const T* fp = reinterpret_cast<const T*>(P.fresh.data) + (live[u] ? fo + M::dim(g, 0) : 0);
      const T* rp = reinterpret_cast<const T*>(P.reuse.data) + (live[u] ? ro + M::dim(g, 0) : 0);
      f[u] = ld16(fp);
      q[u] = ld16(rp);
    }
    wait_loads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vu4 pr = q[u];
      if constexpr (STYLE == kStyleHalf) pr = partner16<M::X>(q[u]);
      if (!live[u]) continue;
      double x[V], pv[V], fr[V];
      Cd::unpack(q[u], x);
      if constexpr (STYLE == kStyleHalf) Cd::unpack(pr, pv);
      if constexpr (STYLE != kStyleNone) rotate_part<STYLE, V>(x, pv, cs, ss);
      Cd::unpack(f[u], fr);
#pragma unroll
      for (int m = 0; m < V; ++m) acc[m] += fr[m] - x[m];
      if (P.has_out) st16(reinterpret_cast<T*>(P.out.data) + oo[u] + M::dim(g, 0), f[u]);
    }
  }
  // Sum of the slice's rank-state rows (one row per thread): fixed-order
  // butterfly over the wave, then the waves in index order.
  __shared__ double redA[kWavesPerBlock][kFitMaxRank];
  if (rank > 0) {
    for (int k = 0; k < rank; ++k) {
      double a = (double)arow[k];
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) a += __shfl_xor(a, off);
      if (lane == 0) redA[wave][k] = a;
    }
  }
  // Fixed-order reduction: butterfly over the rows of a wave, then the waves
  // in index order.
#pragma unroll
  for (int off = G; off < kWave; off <<= 1)
#pragma unroll
    for (int m = 0; m < V; ++m) acc[m] += __shfl_xor(acc[m], off);
  if (rw == 0) {
#pragma unroll
    for (int m = 0; m < V; ++m) red[wave][M::dim(g, m)] = acc[m];
  }
  __syncthreads();
  for (int d = threadIdx.x; d < HD; d += kBlock) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) t += red[w][d];
    outp[d] = t;
  }
  if (threadIdx.x < kFitMaxRank) {
    double a = 0.0;
    if ((int)threadIdx.x < rank) {
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) a += redA[w][threadIdx.x];
    }
    outp[HD + threadIdx.x] = a;
  }
  if (threadIdx.x == 0) outp[HD + kFitMaxRank] = (double)members;
}

// mu[unit][d] = (sum_p partial[p][d] - sum_k (sum_p partial[p][HD + k]) B[k][d]) / members,
// members = the number of probe-set members over all slices (mu = 0 for none)
struct FitFinishParams {
  const double* partial;
  DLowRank lr;
  float* mu;
  int32_t parts, hd, b, S, H;
};

__global__ void fit_finish_kernel(FitFinishParams F) {
  __shared__ double sA[kFitMaxRank];
  const int unit = blockIdx.x;
  const int pw = fit_row_width(F.hd);
  __shared__ double s_members;
  const double* pp = F.partial + (int64_t)unit * F.parts * pw;
  if (threadIdx.x < kFitMaxRank) {
    double a = 0.0;
    for (int p = 0; p < F.parts; ++p) a += pp[(int64_t)p * pw + F.hd + threadIdx.x];
    sA[threadIdx.x] = a;
  }
  if (threadIdx.x == 0) {
    double c = 0.0;
    for (int p = 0; p < F.parts; ++p) c += pp[(int64_t)p * pw + F.hd + kFitMaxRank];
    s_members = c;
  }
  __syncthreads();
  const double members = s_members;
  const int h = unit % F.H, s = (unit / F.H) % F.S, l = unit / (F.H * F.S);
  const float* Bp = F.lr.rank > 0 ? F.lr.B + l * F.lr.sB_layer + s * F.lr.sB_seg + h * F.lr.sB_head
                                  : nullptr;
  for (int d = threadIdx.x; d < F.hd; d += blockDim.x) {
    double t = 0.0;
    for (int p = 0; p < F.parts; ++p) t += pp[(int64_t)p * pw + d];
    double ab = 0.0;
    for (int k = 0; k < F.lr.rank; ++k) ab = fma(sA[k], (double)Bp[k * F.hd + d], ab);
    F.mu[(int64_t)unit * F.hd + d] = members > 0.0 ? (float)((t - ab) / members) : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// apply
// ---------------------------------------------------------------------------
//
// The rows are cut into chunks of CH rows (one batch of U rows per lane).  On
// dense planes each block takes one chunk, in address order, so the chunks
// in flight cover neighbouring bytes; on paged pools a block takes a run of
// about 32 consecutive chunks, fetching each next chunk's page ids while it
// works on the current one.  Chunks are numbered segment-major, so a block
// recomputes its rotary table only when the segment changes.
//
// Per chunk, a block issues its row loads first, then the chunk's set-up
// loads (probe bits, weights, rank-state rows; the lane's mean and B
// values), so both share one memory round trip; the per-row data goes
// through LDS (double-buffered: one barrier per chunk).
//
// bf16 planes with head_dim 128 take the rank-r term on the matrix cores: a
// wave's U x RPW = 16 rows form one 16 x 16 x 4 fp32 MFMA tile per 16-dim
// slice, with the tile's columns permuted so that each lane receives exactly
// the 8 contiguous dims it holds (see apply_kernel), and the rotated row plus
// the weighted mean as the accumulator input.

constexpr int kApplyBlock = 256;
constexpr int kApplyWaves = kApplyBlock / kWave;
constexpr int kApplyU = 4;
constexpr int kPagedChunksPerBlock = 32;

// Rows per chunk for storage type T and head_dim HD (host and device).
__host__ __device__ constexpr int apply_chunk_rows(int vec, int hd) {
  return kApplyWaves * (kWave / (hd / vec)) * kApplyU;
}

struct ApplyParams {
  DPlane in, out;
  const uint32_t* mask;
  const float* scores;
  float w_lo, w_hi;
  const float* mu;
  DLowRank lr;
  RopeArgs rope;
  int32_t S, L, H, n, cpu, mask_words;
  int32_t per_head;            // mask [S][H][words] and scores [S][H][n]
  const int32_t* cover;        // rows j >= cover[s] are only re-aligned (NULL: none)
  // Chunk order: c = ((s L + l) X + x) Y + y, where (x, y) = (head, chunk
  // of tokens) or, when a head's rows are farther apart than a token's
  // (paged pools, token-major layouts), (chunk of tokens, head), so that the
  // chunks in flight together cover neighbouring bytes.  Block b takes the
  // per_block chunks from b per_block on, one after another (a paged pool
  // then reuses its rotary table across them).
  int32_t h_inner;
  int32_t per_block;
  int32_t a_vec;               // A rows may be read as whole 16-byte vectors
  int32_t b_vec;               // B rows may be read as whole 16-byte vectors
};

// Rank-state left factor of one row: MAXR values (zero past the rank).
template <int MAXR, typename C>
__device__ __forceinline__ void load_a_row(const float* Ar, int rank, bool vec, C* out) {
  if constexpr (MAXR >= 4) {
    if (vec) {
#pragma unroll
      for (int q = 0; q < MAXR / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(Ar + 4 * q);
        out[4 * q] = (C)v.x; out[4 * q + 1] = (C)v.y; out[4 * q + 2] = (C)v.z; out[4 * q + 3] = (C)v.w;
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < MAXR; ++k) out[k] = k < rank ? (C)Ar[k] : (C)0;
}

// N consecutive floats (N a multiple of 4 when vec) from global memory.
template <int N, typename C>
__device__ __forceinline__ void load_floats(const float* p, bool vec, C* out) {
  if constexpr (N % 4 == 0) {
    if (vec) {
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(p + 4 * q);
        out[4 * q] = (C)v.x; out[4 * q + 1] = (C)v.y; out[4 * q + 2] = (C)v.z; out[4 * q + 3] = (C)v.w;
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < N; ++k) out[k] = (C)p[k];
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T, typename C, int HD, int STYLE, int MAXR, bool PAGED>
__device__ __forceinline__ void apply_body(const ApplyParams& P) {
  using M = PartMap<T, HD, STYLE>;
  using Cc = Codec<T, C>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW, U = kApplyU;
  constexpr int kStep = kApplyWaves * RPW;          // rows per block per batch step
  constexpr int CH = kStep * U;                     // rows per chunk
  static_assert(CH == apply_chunk_rows(V, HD), "chunk size");
  static_assert(CH <= kApplyBlock, "one thread per chunk row in the set-up");
  constexpr int R = MAXR > 0 ? MAXR : 1;
  constexpr int RS = MAXR > 0 ? (MAXR + 3) / 4 * 4 : 1;   // LDS row stride of A
  constexpr int KB = (MAXR + 3) / 4;                      // MFMA k-blocks
  constexpr bool kMfma = std::is_same<T, bf16_t>::value && std::is_same<C, float>::value &&
                         HD == 128 && MAXR > 0;
  static_assert(!kMfma || (V == 8 && G == 16 && RPW == 4 && U == 4), "MFMA tile shape");
  constexpr int NW = CH >= 32 ? CH / 32 : 1;        // probe-bit words per chunk
  static_assert(CH % 32 == 0 || 32 % CH == 0, "chunks start on a word or inside one");

  __shared__ C tab_c[2][HD / 2], tab_s[2][HD / 2];
  __shared__ __attribute__((aligned(16))) float sa[2][MAXR > 0 ? CH * RS : 1];
  __shared__ float sw[2][CH];

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t / kWave;
  const int g = lane % G, rw = lane / G;
  const int i_first = wave * RPW + rw;
  const int rank = P.lr.rank;
  const int64_t in_step = (int64_t)kStep * P.in.s_token;
  const int64_t out_step = (int64_t)kStep * P.out.s_token;
  int cur_s = -1, gen = 0;
  const bool first_half = STYLE == kStyleHalf && g < M::X;
  // Chunk coordinates (block-uniform).  The block steps to the next chunk
  // digit by digit with carries: no division in the loop.
  struct Pos { int k, h, l, s; };
  const int r0 = P.h_inner ? P.H : P.cpu, r1 = P.h_inner ? P.cpu : P.H;
  auto advance = [&](Pos p) {
    int d0 = P.h_inner ? p.h : p.k, d1 = P.h_inner ? p.k : p.h;
    int cy = ++d0 >= r0; if (cy) d0 = 0;
    d1 += cy;
    cy = d1 >= r1; if (cy) d1 = 0;
    p.l += cy;
    cy = p.l >= P.L; if (cy) p.l = 0;
    p.s += cy;
    p.h = P.h_inner ? d0 : d1;
    p.k = P.h_inner ? d1 : d0;
    return p;
  };
  // Probe bits of a chunk: NW words, uniform over the block (scalar loads),
  // fetched one chunk ahead so that the row loads can skip probe rows.
  auto chunk_words = [&](Pos p, uint32_t* w) {
#pragma unroll
    for (int qq = 0; qq < NW; ++qq) w[qq] = 0u;
    if (P.mask == nullptr || p.s >= P.S) return;
    const int wb = (p.k * CH) >> 5;
#pragma unroll
    for (int qq = 0; qq < NW; ++qq)
      if (wb + qq < P.mask_words)
        w[qq] = P.mask[((int64_t)p.s * (P.per_head ? P.H : 1) + (P.per_head ? p.h : 0)) *
                           P.mask_words + wb + qq];
  };
  Pos pos;
  {
    unsigned q = blockIdx.x * (unsigned)P.per_block;     // below 2^31 (host check)
    const int d0 = (int)(q % (unsigned)r0); q /= (unsigned)r0;
    const int d1 = (int)(q % (unsigned)r1); q /= (unsigned)r1;
    pos.l = (int)(q % (unsigned)P.L);
    pos.s = (int)(q / (unsigned)P.L);
    pos.h = P.h_inner ? d0 : d1;
    pos.k = P.h_inner ? d1 : d0;
  }
  uint32_t mw[NW];
  chunk_words(pos, mw);
  // Page ids of this lane's rows of a chunk (paged planes), also fetched one
  // chunk ahead, so a paged chunk issues its row loads as early as a dense one.
  auto chunk_pages = [&](Pos p, int32_t* pi, int32_t* po) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = p.k * CH + i_first + u * kStep;
      const bool ok = p.s < P.S && j < P.n;
      pi[u] = ok ? page_of(P.in, p.s, j) : 0;
      po[u] = ok ? page_of(P.out, p.s, j) : 0;
    }
  };
  int32_t pgi[PAGED ? U : 1], pgo[PAGED ? U : 1];
  if constexpr (PAGED) chunk_pages(pos, pgi, pgo);
  // rotary frequency of table entry t (parked in LDS: written and read by
  // thread t only), and the current segment's shift
  __shared__ double sfreq[STYLE != kStyleNone ? HD / 2 : 1];
  if (STYLE != kStyleNone && t < HD / 2) sfreq[t] = P.rope.inv_freq[t];
  int64_t delta_cur = STYLE != kStyleNone && pos.s < P.S ? P.rope.delta[pos.s] : 0;

  // Dense planes take exactly one chunk per block (the launcher's grid).
  // The rotating MFMA instance then compiles the body once, with no
  // next-chunk fetches: the loop's state would spill its scalar registers
  // and leave it at four waves per SIMD.  The other dense instances keep
  // the loop (run once); compiled straight, they measured slower.
  constexpr bool kOne = !PAGED && kMfma && STYLE != kStyleNone;
  int it = 0;
  for (; pos.s < P.S && it < (kOne ? 1 : P.per_block); ++it) {
    const int buf = it & 1;
    const int k = pos.k, h = pos.h, l = pos.l, s = pos.s;
    const int j_begin = k * CH;
    const int j_end = min(P.n, j_begin + CH);
    const int nrows = j_end - j_begin;
    // A new segment needs its rotary table.  It is computed after the
    // chunk's loads are issued (their latency covers it) and published by
    // the chunk's barrier; its shift was fetched one chunk ahead.
    const bool new_seg = STYLE != kStyleNone && s != cur_s;      // uniform over the block
    if (new_seg) ++gen;
    const Pos next = kOne ? pos : advance(pos);
    uint32_t mw_next[NW];
    if constexpr (!kOne) chunk_words(next, mw_next);
    int64_t delta_next = 0;
    if constexpr (!kOne)
      if (STYLE != kStyleNone && next.s < P.S && next.s != s) delta_next = P.rope.delta[next.s];
    // live rows of this lane: in range and not a probe
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i_first + u * kStep;
      const int bit = (CH >= 32 ? i : (j_begin & 31) + i);
      live[u] = i < nrows && ((mw[bit >> 5 < NW ? bit >> 5 : 0] >> (bit & 31)) & 1u) == 0;
    }

    // Row loads are unconditional (no branch between them, so they all stay
    // in flight together): a row past the chunk reads the plane's first
    // vector instead, an address that always exists and stays in cache.
    // Probe rows are loaded too and simply not stored.
    vu4 r0[U];
    // Dense planes: this lane's first row of the chunk; its further rows
    // are kStep rows apart.
    const int64_t jf = j_begin + i_first;
    const T* ip0 = reinterpret_cast<const T*>(P.in.data) + (int64_t)l * P.in.s_layer +
                   (int64_t)s * P.in.s_seg + (int64_t)h * P.in.s_head + jf * P.in.s_token +
                   M::dim(g, 0);
    T* op0 = reinterpret_cast<T*>(P.out.data) + (int64_t)l * P.out.s_layer +
             (int64_t)s * P.out.s_seg + (int64_t)h * P.out.s_head + jf * P.out.s_token +
             M::dim(g, 0);
    int64_t po[PAGED ? U : 1];            // paged: output row offsets
    if constexpr (!PAGED) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        r0[u] = ld16(live[u] ? ip0 + u * in_step : reinterpret_cast<const T*>(P.in.data));
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j_begin + i_first + u * kStep;
        const int64_t io = live[u] ? row_offset_page(P.in, l, s, h, j, pgi[u]) : -1;
        const int64_t oo = live[u] ? row_offset_page(P.out, l, s, h, j, pgo[u]) : -1;
        live[u] = live[u] && io >= 0 && oo >= 0;          // a bad page id skips the row
        r0[u] = ld16(reinterpret_cast<const T*>(P.in.data) + (live[u] ? io + M::dim(g, 0) : 0));
        po[u] = oo + M::dim(g, 0);
      }
    }
    int32_t pgi_next[PAGED ? U : 1], pgo_next[PAGED ? U : 1];
    if constexpr (PAGED) chunk_pages(next, pgi_next, pgo_next);

    // Set-up loads: this thread's chunk row (weight, rank-state row) and the
    // lane's per-unit mean and B values.
    float wt = 1.0f;
    if (P.scores && t < nrows)
      wt = P.scores[((int64_t)s * (P.per_head ? P.H : 1) + (P.per_head ? h : 0)) * P.n +
                    j_begin + t];
    const int cov = P.cover ? P.cover[s] : P.n;
    float arow[R];
#pragma unroll
    for (int kk = 0; kk < R; ++kk) arow[kk] = 0.0f;
    if constexpr (MAXR > 0) {
      if (t < nrows) {
        const float* Ar = P.lr.A + l * P.lr.sA_layer + s * P.lr.sA_seg + h * P.lr.sA_head +
                          (int64_t)(j_begin + t) * rank;
        load_a_row<MAXR>(Ar, rank, P.a_vec, arow);
      }
    }
    const int64_t ubase = (((int64_t)l * P.S + s) * P.H + h) * HD;
    C mu[V];
    load_floats<V>(P.mu + ubase + M::dim(g, 0), true, mu);
    const float* Bp = MAXR > 0 ? P.lr.B + l * P.lr.sB_layer + s * P.lr.sB_seg + h * P.lr.sB_head
                               : nullptr;
    // MFMA operand: lane supplies B[4 kb + lane / 16][8 (lane % 16) + n], n < 8.
    float Bm[kMfma ? KB : 1][kMfma ? 8 : 1];
    // VALU operand: B[k][dims of this lane].
    C Bv[kMfma ? 1 : R][kMfma ? 1 : V];
    if constexpr (kMfma) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int kr = 4 * kb + lane / 16;
        if (kr < rank) load_floats<8>(Bp + kr * HD + 8 * (lane % 16), P.b_vec, Bm[kb]);
        else
#pragma unroll
          for (int n = 0; n < 8; ++n) Bm[kb][n] = 0.0f;
      }
    } else if constexpr (MAXR > 0) {
#pragma unroll
      for (int kk = 0; kk < MAXR; ++kk) {
        if (kk < rank) load_floats<V>(Bp + kk * HD + M::dim(g, 0), P.b_vec, Bv[kk]);
        else
#pragma unroll
          for (int m = 0; m < V; ++m) Bv[kk][m] = (C)0;
      }
    }
    if (new_seg && t < HD / 2) {
      if constexpr (std::is_same<C, float>::value) {     // fp32 table (bf16 planes)
        float sv, cv;
        rope_sincos_f32((double)delta_cur * sfreq[t], &sv, &cv);
        tab_c[gen & 1][t] = cv;
        tab_s[gen & 1][t] = sv;
      } else {
        double sv, cv;
        rope_sincos((double)delta_cur * sfreq[t], &sv, &cv);
        tab_c[gen & 1][t] = (C)cv;
        tab_s[gen & 1][t] = (C)sv;
      }
    }
    if (t < nrows) {
      // w = clamp(score) (1 without scores); past the covered prefix neither
      // the mean nor the rank term applies: w = 0 and A row = 0
      const bool covered = j_begin + t < cov;
      sw[buf][t] = !covered ? 0.0f : P.scores ? fminf(fmaxf(wt, P.w_lo), P.w_hi) : 1.0f;
      if constexpr (MAXR > 0) {
#pragma unroll
        for (int kk = 0; kk < RS; ++kk)
          sa[buf][t * RS + kk] = kk < MAXR && covered ? arow[kk] : 0.0f;
      }
    }
    __syncthreads();
    if (new_seg) cur_s = s;
    // This lane's cos / signed sin (read from the block's table for the
    // segment each chunk, so they hold no registers across the loads).
    C cs[V], ss[V];
    if constexpr (STYLE != kStyleNone) {
#pragma unroll
      for (int m = 0; m < V; ++m) {
        cs[m] = tab_c[gen & 1][M::pair(g, m)];
        const C sv = tab_s[gen & 1][M::pair(g, m)];
        ss[m] = first_half ? -sv : sv;
      }
    }

    // Output row of batch row u (dense: op0 + u out_step; paged: looked up).
    auto out_row = [&](int u) -> T* {
      if constexpr (PAGED) return reinterpret_cast<T*>(P.out.data) + po[u];
      else return op0 + u * out_step;
    };
    wait_loads();

    if constexpr (kMfma) {
      // Accumulator input: rotated row plus weighted mean; lane holds
      // acc[m][u] = element m of its 8 dims for batch row u.
      f32x4 acc[V];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        vu4 pr = r0[u];
        if constexpr (STYLE == kStyleHalf) pr = partner16<M::X>(r0[u]);
        C x[V], pv[V];
        Cc::unpack(r0[u], x);
        if constexpr (STYLE == kStyleHalf) Cc::unpack(pr, pv);
        if constexpr (STYLE != kStyleNone) rotate_part<STYLE, V>(x, pv, cs, ss);
        const C w = (C)sw[buf][i_first + u * kStep];
#pragma unroll
        for (int m = 0; m < V; ++m) acc[m][u] = fma(w, mu[m], x[m]);
        // one row at a time: keeps the unpacked rows out of registers together
        __builtin_amdgcn_sched_barrier(0);
      }
      // Tile row r = 4 (lane / 16) + u holds chunk row i_first + u kStep of
      // the lane group lane / 16; as an A operand, lane supplies tile row
      // lane % 16, i.e. chunk row wave RPW + (lane % 16) / 4 + ((lane % 16) % 4) kStep.
      const int arow_i = wave * RPW + (lane % 16) / 4 + ((lane % 16) % 4) * kStep;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float a = sa[buf][arow_i * RS + 4 * kb + lane / 16];
#pragma unroll
        for (int m = 0; m < V; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Bm[kb][m], acc[m], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!live[u]) continue;
        C y[V];
#pragma unroll
        for (int m = 0; m < V; ++m) y[m] = acc[m][u];
        st16(out_row(u), Cc::pack(y));
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // the partner exchange runs on every lane of the wave (both halves of
        // a row are live or dead together)
        vu4 pr = r0[u];
        if constexpr (STYLE == kStyleHalf) pr = partner16<M::X>(r0[u]);
        if (!live[u]) continue;
        const int i = i_first + u * kStep;
        C x[V], pv[V];
        Cc::unpack(r0[u], x);
        if constexpr (STYLE == kStyleHalf) Cc::unpack(pr, pv);
        if constexpr (STYLE != kStyleNone) rotate_part<STYLE, V>(x, pv, cs, ss);
        const C w = (C)sw[buf][i];
        C Av[R];
        if constexpr (MAXR > 0) {
#pragma unroll
          for (int kk = 0; kk < MAXR; ++kk) Av[kk] = (C)sa[buf][i * RS + kk];
        }
#pragma unroll
        for (int m = 0; m < V; ++m) {
          C y = fma(w, mu[m], x[m]);
          if constexpr (MAXR > 0) {
#pragma unroll
            for (int kk = 0; kk < MAXR; ++kk) y = fma(Av[kk], Bv[kk][m], y);
          }
          x[m] = y;
        }
        st16(out_row(u), Cc::pack(x));
      }
    }
    if constexpr (kOne) break;
#pragma unroll
    for (int qq = 0; qq < NW; ++qq) mw[qq] = mw_next[qq];
    if constexpr (PAGED) {
#pragma unroll
      for (int u = 0; u < U; ++u) { pgi[u] = pgi_next[u]; pgo[u] = pgo_next[u]; }
    }
    if (next.s != s) delta_cur = delta_next;
    pos = next;
  }
}

// Register budget: the bf16 / hd 128 / rank <= 4 instances fit in 128 VGPRs
// without spilling (4 waves per SIMD, so 4 resident blocks per CU); the other
// instances keep the compiler's own choice.
template <typename T, int HD, int MAXR, bool PAGED>
constexpr bool apply_occ4() {
  return std::is_same<T, bf16_t>::value && HD == 128 && MAXR <= 4;
}

template <typename T, typename C, int HD, int STYLE, int MAXR, bool PAGED>
__global__ __launch_bounds__(kApplyBlock) __attribute__((amdgpu_waves_per_eu(4)))
void apply_kernel(ApplyParams P) {
  apply_body<T, C, HD, STYLE, MAXR, PAGED>(P);
}

template <typename T, typename C, int HD, int STYLE, int MAXR, bool PAGED>
__global__ __launch_bounds__(kApplyBlock) void apply_kernel_wide(ApplyParams P) {
  apply_body<T, C, HD, STYLE, MAXR, PAGED>(P);
}

// ---------------------------------------------------------------------------
// Dispatch helpers: (dtype, head_dim, style, rank) -> template instance.
// ---------------------------------------------------------------------------

template <template <typename, int, int> class F, typename... A>
kvfix_status dispatch_t_hd_style(int32_t dtype, int32_t hd, int style, A&&... args) {
#define KVFIX_CASE(T_, HD_, ST_)                                          \
  if (dtype == (std::is_same<T_, float>::value ? KVFIX_F32 : KVFIX_BF16) && \
      hd == HD_ && style == ST_)                                          \
    return F<T_, HD_, ST_>::run(args...);
#define KVFIX_STYLES(T_, HD_)         \
  KVFIX_CASE(T_, HD_, kStyleNone)     \
  KVFIX_CASE(T_, HD_, kStyleHalf)     \
  KVFIX_CASE(T_, HD_, kStyleInter)
  KVFIX_STYLES(float, 64) KVFIX_STYLES(float, 128) KVFIX_STYLES(float, 256)
  KVFIX_STYLES(bf16_t, 64) KVFIX_STYLES(bf16_t, 128) KVFIX_STYLES(bf16_t, 256)
#undef KVFIX_STYLES
#undef KVFIX_CASE
  return KVFIX_ERR_UNSUPPORTED;
}

template <typename T, int HD, int STYLE>
struct RopeShiftLaunch {
  static kvfix_status run(const RopeShiftParams& P, int64_t grid, hipStream_t st) {
    if constexpr (STYLE == kStyleNone) {
      return KVFIX_ERR_ARG;
    } else {
      rope_shift_kernel<T, HD, STYLE><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P);
      return launch_status();
    }
  }
};

template <typename T, int HD, int STYLE>
struct FitLaunch {
  static kvfix_status run(const FitParams& P, int64_t grid, hipStream_t st) {
    fit_partial_kernel<T, HD, STYLE><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P);
    return launch_status();
  }
};

template <typename T, int HD, int STYLE>
struct ApplyLaunch {
  using C = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
  // Dense planes: one block per chunk.  Paged pools: about 32 consecutive chunks
  // per block, and never fewer blocks than the chip holds at once (resident
  // blocks per CU of this instance x CUs) unless there are fewer chunks.
  template <int R, bool PG>
  static void launch(ApplyParams P, int64_t n_chunks, hipStream_t st) {
    // only the chosen instance is compiled
    auto kern = [] {
      if constexpr (apply_occ4<T, HD, R, PG>()) return apply_kernel<T, C, HD, STYLE, R, PG>;
      else return apply_kernel_wide<T, C, HD, STYLE, R, PG>;
    }();
    static const int per_cu = [&] {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kApplyBlock, 0) != hipSuccess ||
          nb < 1)
        nb = 1;
      return nb;
    }();
    const int64_t resident = (int64_t)per_cu * device_cus();
    // Dense planes: one block per chunk, dispatched in address order (the
    // hardware then streams HBM like a plain one-pass copy).  Paged pools:
    // runs of about kPagedChunksPerBlock consecutive chunks per block (and
    // never fewer blocks than the chip holds at once), so each block's page
    // ids are fetched a chunk ahead and its rotary table serves the run.
    int64_t blocks = !PG ? n_chunks : n_chunks / kPagedChunksPerBlock;
    if (blocks < resident) blocks = resident;
    if (blocks > n_chunks) blocks = n_chunks;
    const int64_t per = (n_chunks + blocks - 1) / blocks;
    const int64_t grid = (n_chunks + per - 1) / per;
    P.per_block = (int32_t)per;
    kern<<<dim3((unsigned)grid), dim3(kApplyBlock), 0, st>>>(P);
  }
  template <bool PG>
  static void go(const ApplyParams& P, int rank_var, int64_t grid, hipStream_t st) {
    switch (rank_var) {
      case 0: launch<0, PG>(P, grid, st); break;
      case 2: launch<2, PG>(P, grid, st); break;
      case 4: launch<4, PG>(P, grid, st); break;
      default: launch<8, PG>(P, grid, st); break;
    }
  }
  static kvfix_status run(const ApplyParams& P, int rank_var, int64_t grid, hipStream_t st) {
    if (P.in.page_table || P.out.page_table) go<true>(P, rank_var, grid, st);
    else go<false>(P, rank_var, grid, st);
    return launch_status();
  }
};

}  // namespace kvfix

using namespace kvfix;

extern "C" kvfix_status kvfix_rope_shift(const kvfix_plane* src, const kvfix_plane* dst,
                                         const kvfix_rope* rope, void* stream) {
  KVFIX_TRY(check_plane(src));
  KVFIX_TRY(check_plane(dst));
  KVFIX_TRY(same_rows(src, dst));
  if (src->n_layers != dst->n_layers || rope == nullptr) return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(rope, src->head_dim));
  const int64_t units = (int64_t)src->n_layers * src->n_segs * src->n_heads;
  if (units == 0 || src->n_tokens == 0) return KVFIX_OK;
  RopeShiftParams P;
  P.src = make_dplane(*src);
  P.dst = make_dplane(*dst);
  P.rope = make_rope_args(rope, src->head_dim);
  P.S = src->n_segs; P.H = src->n_heads; P.n = src->n_tokens;
  P.rows_per_block = kRowsPerBlock;
  P.chunks = (int32_t)ceil_div(src->n_tokens, kRowsPerBlock);
  const int64_t grid = units * P.chunks;
  if (grid > kMaxGrid) return KVFIX_ERR_ARG;
  return dispatch_t_hd_style<RopeShiftLaunch>(src->dtype, src->head_dim, rope->style, P, grid,
                                              (hipStream_t)stream);
}

static int fit_parts(int32_t b) { return b > 0 ? (b + kFitRows - 1) / kFitRows : 1; }

extern "C" size_t kvfix_fit_mean_workspace(int32_t n_layers, int32_t n_segs, int32_t n_heads,
                                           int32_t head_dim, int32_t b) {
  if (n_layers < 0 || n_segs < 0 || n_heads < 0 || head_dim < 0 || b < 0) return 0;
  return (size_t)n_layers * n_segs * n_heads * fit_parts(b) * fit_row_width(head_dim) *
         sizeof(double);
}

extern "C" kvfix_status kvfix_fit_mean_ex(const kvfix_plane* fresh, int32_t fresh_by_slot,
                                          const kvfix_plane* reuse, const kvfix_plane* out,
                                          const int32_t* idx, int32_t b, const kvfix_rope* rope,
                                          const kvfix_lowrank* lowrank,
                                          const kvfix_granularity* opt, float* mu, void* ws,
                                          size_t ws_bytes, void* stream) {
  KVFIX_TRY(check_plane(fresh));
  KVFIX_TRY(check_plane(reuse));
  if (out) {
    KVFIX_TRY(check_plane(out));
    KVFIX_TRY(same_rows(out, reuse));
    if (out->n_layers != reuse->n_layers) return KVFIX_ERR_ARG;
  }
  if (mu == nullptr) return KVFIX_ERR_ARG;
  if (fresh->dtype != reuse->dtype || fresh->head_dim != reuse->head_dim ||
      fresh->n_heads != reuse->n_heads || fresh->n_segs != reuse->n_segs ||
      fresh->n_layers != reuse->n_layers)
    return KVFIX_ERR_ARG;
  if (b < 0) return KVFIX_ERR_ARG;                // b: the width of each index list
  if (b > 0 && idx == nullptr) return KVFIX_ERR_ARG;
  if (fresh_by_slot ? fresh->n_tokens < b : fresh->n_tokens != reuse->n_tokens)
    return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(rope, reuse->head_dim));
  KVFIX_TRY(check_lowrank(lowrank));
  if (opt && opt->per_head != 0 && opt->per_head != 1) return KVFIX_ERR_ARG;
  const int64_t units = (int64_t)reuse->n_layers * reuse->n_segs * reuse->n_heads;
  if (units == 0) return KVFIX_OK;
  const size_t need = kvfix_fit_mean_workspace(reuse->n_layers, reuse->n_segs, reuse->n_heads,
                                               reuse->head_dim, b);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return KVFIX_ERR_ARG;
  const int parts = fit_parts(b);
  const int64_t grid = units * parts;
  if (grid > kMaxGrid) return KVFIX_ERR_ARG;
  FitParams P;
  P.fresh = make_dplane(*fresh);
  P.reuse = make_dplane(*reuse);
  P.out = out ? make_dplane(*out) : make_dplane(*reuse);
  P.has_out = out != nullptr;
  P.fresh_by_slot = fresh_by_slot != 0;
  P.idx = idx;
  P.b = b;
  P.parts = parts;
  P.lr = make_dlowrank(lowrank);
  P.rope = make_rope_args(rope, reuse->head_dim);
  P.partial = static_cast<double*>(ws);
  P.S = reuse->n_segs; P.H = reuse->n_heads; P.n = reuse->n_tokens;
  P.idx_heads = opt && opt->per_head ? reuse->n_heads : 1;
  P.cover = opt ? opt->cover : nullptr;
  hipStream_t st = (hipStream_t)stream;
  const int style = rope ? rope->style : kStyleNone;
  KVFIX_TRY(dispatch_t_hd_style<FitLaunch>(reuse->dtype, reuse->head_dim, style, P, grid, st));
  FitFinishParams F;
  F.partial = P.partial;
  F.lr = P.lr;
  F.mu = mu;
  F.parts = parts; F.hd = reuse->head_dim; F.b = b; F.S = P.S; F.H = P.H;
  fit_finish_kernel<<<dim3((unsigned)units), dim3(128), 0, st>>>(F);
  return launch_status();
}

extern "C" kvfix_status kvfix_fit_mean(const kvfix_plane* fresh, int32_t fresh_by_slot,
                                       const kvfix_plane* reuse, const kvfix_plane* out,
                                       const int32_t* idx, int32_t b, const kvfix_rope* rope,
                                       const kvfix_lowrank* lowrank, float* mu, void* ws,
                                       size_t ws_bytes, void* stream) {
  return kvfix_fit_mean_ex(fresh, fresh_by_slot, reuse, out, idx, b, rope, lowrank, nullptr, mu,
                           ws, ws_bytes, stream);
}

extern "C" kvfix_status kvfix_apply_ex(const kvfix_plane* reuse, const kvfix_plane* out,
                                       const uint32_t* mask, const float* scores, float w_lo,
                                       float w_hi, const float* mu, const kvfix_lowrank* lowrank,
                                       const kvfix_rope* rope, const kvfix_granularity* opt,
                                       void* stream) {
  KVFIX_TRY(check_plane(reuse));
  KVFIX_TRY(check_plane(out));
  KVFIX_TRY(same_rows(reuse, out));
  if (reuse->n_layers != out->n_layers || mu == nullptr) return KVFIX_ERR_ARG;
  if (scores && !(w_lo <= w_hi)) return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(rope, reuse->head_dim));
  KVFIX_TRY(check_lowrank(lowrank));
  if (opt && opt->per_head != 0 && opt->per_head != 1) return KVFIX_ERR_ARG;
  const int64_t units = (int64_t)reuse->n_layers * reuse->n_segs * reuse->n_heads;
  if (units == 0 || reuse->n_tokens == 0) return KVFIX_OK;
  if (!aligned16(mu)) return KVFIX_ERR_ALIGN;
  ApplyParams P;
  P.in = make_dplane(*reuse);
  P.out = make_dplane(*out);
  P.mask = mask;
  P.scores = scores;
  P.w_lo = w_lo;
  P.w_hi = w_hi;
  P.mu = mu;
  P.lr = make_dlowrank(lowrank);
  P.a_vec = P.lr.rank > 0 && aligned16(P.lr.A) && (P.lr.sA_layer * 4) % 16 == 0 &&
            (P.lr.sA_seg * 4) % 16 == 0 && (P.lr.sA_head * 4) % 16 == 0 && (P.lr.rank * 4) % 16 == 0;
  P.b_vec = P.lr.rank > 0 && aligned16(P.lr.B) && (P.lr.sB_layer * 4) % 16 == 0 &&
            (P.lr.sB_seg * 4) % 16 == 0 && (P.lr.sB_head * 4) % 16 == 0;
  P.rope = make_rope_args(rope, reuse->head_dim);
  P.S = reuse->n_segs; P.L = reuse->n_layers; P.H = reuse->n_heads; P.n = reuse->n_tokens;
  P.mask_words = (int32_t)ceil_div(reuse->n_tokens, 32);
  P.per_head = opt ? opt->per_head : 0;
  P.cover = opt ? opt->cover : nullptr;
  const int ch = apply_chunk_rows(reuse->dtype == KVFIX_F32 ? 4 : 8, reuse->head_dim);
  P.cpu = (reuse->n_tokens + ch - 1) / ch;
  const int64_t n_chunks = units * P.cpu;
  // heads innermost when a token's heads sit closer together than a head's
  // tokens (a paged pool, a token-major layout)
  P.h_inner = reuse->s_head < reuse->s_token;
  if (n_chunks > kMaxGrid) return KVFIX_ERR_ARG;
  const int64_t grid = n_chunks;        // the launcher derives the grid from the chunk count
  const int style = rope ? rope->style : kStyleNone;
  return dispatch_t_hd_style<ApplyLaunch>(reuse->dtype, reuse->head_dim, style, P,
                                          rank_variant(P.lr.rank), grid, (hipStream_t)stream);
}

extern "C" kvfix_status kvfix_apply(const kvfix_plane* reuse, const kvfix_plane* out,
                                    const uint32_t* mask, const float* scores, float w_lo,
                                    float w_hi, const float* mu, const kvfix_lowrank* lowrank,
                                    const kvfix_rope* rope, void* stream) {
  return kvfix_apply_ex(reuse, out, mask, scores, w_lo, w_hi, mu, lowrank, rope, nullptr, stream);
}

// ---------------------------------------------------------------------------
// kvfix_fit_mean_noalloc: the fit with its slice partials in a file-scope
// device array instead of a caller workspace, for callers that cannot
// allocate.  Every GPU the library runs on holds its own copy of the array
// (KVFIX_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code the
// array's name is only a stand-in: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and that address is
// what the kernels receive.  Every call on a device shares its array, so
// calls that overlap on one device race; nothing in it needs to start at
// zero (each slice writes its own partial before the finisher reads it).
// ---------------------------------------------------------------------------

namespace kvfix {

static __device__ __align__(256) unsigned char scratch[KVFIX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;

// Device address of this device's `scratch`, or nullptr on a HIP error.
static void* scratch_address() {
  static std::atomic<void*> addr[kMaxScratchDevices];
  static std::mutex lock;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> guard(lock);
  p = addr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    addr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace kvfix

extern "C" kvfix_status kvfix_fit_mean_noalloc(const kvfix_plane* fresh, int32_t fresh_by_slot,
                                               const kvfix_plane* reuse, const kvfix_plane* out,
                                               const int32_t* idx, int32_t b,
                                               const kvfix_rope* rope,
                                               const kvfix_lowrank* lowrank, float* mu,
                                               void* stream) {
  if (reuse == nullptr || b < 0) return KVFIX_ERR_ARG;
  if (reuse->n_layers < 0 || reuse->n_segs < 0 || reuse->n_heads < 0 || reuse->head_dim < 0)
    return KVFIX_ERR_ARG;
  const size_t need = kvfix_fit_mean_workspace(reuse->n_layers, reuse->n_segs, reuse->n_heads,
                                               reuse->head_dim, b);
  if (need > (size_t)KVFIX_NOALLOC_SCRATCH_BYTES) return KVFIX_ERR_CAPACITY;
  void* ws = scratch_address();
  if (ws == nullptr) return KVFIX_ERR_HIP;
  return kvfix_fit_mean_ex(fresh, fresh_by_slot, reuse, out, idx, b, rope, lowrank, nullptr, mu,
                           ws, (size_t)KVFIX_NOALLOC_SCRATCH_BYTES, stream);
}
