// L2 divergence score (a2) and top-b selection (a4).
//
// score: one 256-thread block per (segment, RPW tokens), up to 8 such groups
// per block on rotated planes.  The four waves split the KV heads; each lane accumulates (fresh - align(reuse))^2 of its
// pairs in fp64, lanes of a row reduce by a fixed butterfly, the waves add in
// index order, and sqrt is rounded once to fp32.
//
// select: one 1024-thread block per row.  Scores become order-preserving
// 32-bit keys (NaN lowest, -0 = +0).  Four 8-bit radix passes (LDS integer
// histograms, wave-aggregated increments) find the key T of the b-th largest
// element and how many elements equal to T are still needed; then the
// compaction keeps every key > T and the lowest-index keys == T, placing
// each by wave ballots and a scanned table of per-wave counts, and writes
// indices in ascending order and the bitmask word by word.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "host_util.h"
#include "select_common.h"

namespace kvfix {

constexpr int kScoreBlock = 256;
constexpr int kScoreGroupsMax = 8;      // 8-token groups (RPW rows) per block, at most
constexpr int kScoreMinBlocks = 2048;   // fewer groups per block below this many blocks

struct ScoreParams {
  DPlane fresh, reuse;
  int32_t fl, rl;                 // layer read in each plane
  RopeArgs rope;
  float* scores;                  // [S][n], or [S][H][n] per head
  int32_t S, H, n, tok_blocks;
  int32_t groups;                 // row groups per block (1..kScoreGroupsMax)
  int32_t per_head;
};

// Rotated planes: a block takes `groups` consecutive groups of RPW tokens of
// one segment, so the segment's rotary table is built once per block, after
// the loads of the block's first rows have been issued.
template <typename T, int HD, int STYLE>
__global__ __launch_bounds__(kScoreBlock) void score_l2_kernel(ScoreParams P) {
  static_assert(STYLE != kStyleNone, "unrotated planes take score_l2_plain_kernel");
  constexpr int MS = STYLE;
  using M = RowMap<T, HD, MS>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW;
  constexpr int W = kScoreBlock / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // (uniform)
  const int g = lane % G, rw = lane / G;
  const int grp0 = (blockIdx.x % P.tok_blocks) * P.groups;
  const int s = blockIdx.x / P.tok_blocks;

  __shared__ double tc[HD / 2], ts[HD / 2];
  __shared__ double part[kScoreGroupsMax][W][RPW];
  // the row pair (fresh, reuse) of token j, head h: four 16-byte pieces
  const DPlane pf = P.fresh, pr = P.reuse;
  const int fl = P.fl, rl = P.rl, n = P.n;
  auto load = [&](int j, int h, vu4* r) {
    const int64_t fo = j < n ? row_offset(pf, fl, s, h, j) : -1;
    const int64_t ro = j < n ? row_offset(pr, rl, s, h, j) : -1;
    if (fo < 0 || ro < 0) return false;
    const T* fr = reinterpret_cast<const T*>(pf.data) + fo;
    const T* rr = reinterpret_cast<const T*>(pr.data) + ro;
    r[0] = ld16(fr + M::off0(g));
    r[1] = ld16(fr + M::off1(g));
    r[2] = ld16(rr + M::off0(g));
    r[3] = ld16(rr + M::off1(g));
    return true;
  };
  // the block's first rows are requested before the table is built
  vu4 r[4];
  bool ok = wave < P.H && load(grp0 * RPW + rw, wave, r);
  rope_table<HD, double>(P.rope, P.rope.delta[s], tc, ts);
  __syncthreads();
  double cs[V], sn[V];
#pragma unroll
  for (int m = 0; m < V; ++m) { cs[m] = tc[g * V + m]; sn[m] = ts[g * V + m]; }

#pragma unroll 1
  for (int gi = 0; gi < P.groups; ++gi) {
    const int j = (grp0 + gi) * RPW + rw;
    // Every lane runs the head loop (the per-head sums reduce across lanes
    // inside it); a lane past n or on a bad page id adds nothing.
    double acc = 0.0;
#pragma unroll 1
    for (int h = wave; h < P.H; h += W) {
      if (gi > 0 || h != wave) ok = load(j, h, r);     // (else already in)
      double hacc = 0.0;
      if (ok) {
        double p0[V], p1[V], fa[V], fb[V], ra[V], rb[V];
        Cd::unpack(r[0], p0);
        Cd::unpack(r[1], p1);
        parts_to_pairs<MS, V>(p0, p1, fa, fb);
        Cd::unpack(r[2], p0);
        Cd::unpack(r[3], p1);
        parts_to_pairs<MS, V>(p0, p1, ra, rb);
        rotate_pairs<V>(ra, rb, cs, sn);
#pragma unroll
        for (int m = 0; m < V; ++m) {
          const double da = fa[m] - ra[m], db = fb[m] - rb[m];
          hacc = fma(da, da, hacc);
          hacc = fma(db, db, hacc);
        }
      }
      if (P.per_head) {                            // uniform: this head's score of row j
#pragma unroll
        for (int off = 1; off < G; off <<= 1) hacc += __shfl_xor(hacc, off);
        if (g == 0 && j < P.n) P.scores[((int64_t)s * P.H + h) * P.n + j] = (float)sqrt(hacc);
      } else {
        acc += hacc;
      }
    }
    if (!P.per_head) {
#pragma unroll
      for (int off = 1; off < G; off <<= 1) acc += __shfl_xor(acc, off);
      if (g == 0) part[gi][wave][rw] = acc;
    }
  }
  if (P.per_head) return;                          // (uniform over the block)
  __syncthreads();
  // the waves' head sums of each row, added in wave order
  if ((int)threadIdx.x < P.groups * RPW) {
    const int gi = threadIdx.x / RPW, r = threadIdx.x % RPW;
    const int jj = (grp0 + gi) * RPW + r;
    if (jj < P.n) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < W; ++w) t += part[gi][w][r];
      P.scores[(int64_t)s * P.n + jj] = (float)sqrt(t);
    }
  }
}

// Unrotated planes (no table to share): one group of RPW tokens per block.
template <typename T, int HD>
__global__ __launch_bounds__(kScoreBlock) void score_l2_plain_kernel(ScoreParams P) {
  constexpr int MS = kStyleHalf;          // (any pairing: nothing is rotated)
  using M = RowMap<T, HD, MS>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW;
  constexpr int W = kScoreBlock / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane % G, rw = lane / G;
  const int tb = blockIdx.x % P.tok_blocks;
  const int s = blockIdx.x / P.tok_blocks;
  const int j = tb * RPW + rw;

  __shared__ double part[W][RPW];

  // Every lane runs the head loop (the per-head sums reduce across lanes
  // inside it); a lane past n or on a bad page id adds nothing.
  double acc = 0.0;
  for (int h = wave; h < P.H; h += W) {
    const int64_t fo = j < P.n ? row_offset(P.fresh, P.fl, s, h, j) : -1;
    const int64_t ro = j < P.n ? row_offset(P.reuse, P.rl, s, h, j) : -1;
    double hacc = 0.0;
    if (fo >= 0 && ro >= 0) {
      const T* fr = reinterpret_cast<const T*>(P.fresh.data) + fo;
      const T* rr = reinterpret_cast<const T*>(P.reuse.data) + ro;
      const vu4 f0 = ld16(fr + M::off0(g)), f1 = ld16(fr + M::off1(g));
      const vu4 q0 = ld16(rr + M::off0(g)), q1 = ld16(rr + M::off1(g));
      double p0[V], p1[V], fa[V], fb[V], ra[V], rb[V];
      Cd::unpack(f0, p0);
      Cd::unpack(f1, p1);
      parts_to_pairs<MS, V>(p0, p1, fa, fb);
      Cd::unpack(q0, p0);
      Cd::unpack(q1, p1);
      parts_to_pairs<MS, V>(p0, p1, ra, rb);
#pragma unroll
      for (int m = 0; m < V; ++m) {
        const double da = fa[m] - ra[m], db = fb[m] - rb[m];
        hacc = fma(da, da, hacc);
        hacc = fma(db, db, hacc);
      }
    }
    if (P.per_head) {                              // uniform: this head's score of row j
#pragma unroll
      for (int off = 1; off < G; off <<= 1) hacc += __shfl_xor(hacc, off);
      if (g == 0 && j < P.n) P.scores[((int64_t)s * P.H + h) * P.n + j] = (float)sqrt(hacc);
    } else {
      acc += hacc;
    }
  }
  if (P.per_head) return;                          // (uniform over the block)
#pragma unroll
  for (int off = 1; off < G; off <<= 1) acc += __shfl_xor(acc, off);
  if (g == 0) part[wave][rw] = acc;
  __syncthreads();
  if (threadIdx.x < RPW) {
    const int jj = tb * RPW + threadIdx.x;
    if (jj < P.n) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < W; ++w) t += part[w][threadIdx.x];
      P.scores[(int64_t)s * P.n + jj] = (float)sqrt(t);
    }
  }
}

template <typename T, int HD, int STYLE>
struct ScoreLaunch {
  static kvfix_status run(const ScoreParams& P, hipStream_t st) {
    constexpr int MS = STYLE == kStyleNone ? kStyleHalf : STYLE;
    constexpr int RPW = RowMap<T, HD, MS>::RPW;
    ScoreParams Q = P;
    // Several row groups per block only where they share a rotary table.
    const int64_t groups_total = (int64_t)((P.n + RPW - 1) / RPW) * P.S;
    Q.groups = STYLE == kStyleNone
                   ? 1
                   : (int)std::max<int64_t>(
                         1, std::min<int64_t>(kScoreGroupsMax, groups_total / kScoreMinBlocks));
    Q.tok_blocks = (int32_t)ceil_div(ceil_div(P.n, RPW), Q.groups);
    const int64_t grid = (int64_t)Q.tok_blocks * P.S;
    if (grid > kMaxGrid) return KVFIX_ERR_ARG;
    if constexpr (STYLE == kStyleNone)
      score_l2_plain_kernel<T, HD><<<dim3((unsigned)grid), dim3(kScoreBlock), 0, st>>>(Q);
    else
      score_l2_kernel<T, HD, STYLE><<<dim3((unsigned)grid), dim3(kScoreBlock), 0, st>>>(Q);
    return launch_status();
  }
};

// ---------------------------------------------------------------------------
// top-b selection
// ---------------------------------------------------------------------------

// One block per row.  Keys j = t + 1024 q live in registers (read once).
// Four 8-bit radix passes over per-wave LDS histograms find the b-th largest
// key T and how many keys equal to T are still needed; the compaction then
// places every kept key by wave ballots and a scanned table of per-wave
// counts, so indices come out ascending and the lowest-index keys equal to
// T are the ones taken.
template <int KR>
__global__ __launch_bounds__(kSelBlock) void select_topb_kernel(const float* __restrict__ scores,
                                                                int n, int b,
                                                                int32_t* __restrict__ idx,
                                                                uint32_t* __restrict__ mask,
                                                                int words) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t ctab[2 * kCompactTab];
  __shared__ uint32_t sh[3];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const float* sc = scores + (int64_t)row * n;
  int32_t* out_idx = idx + (int64_t)row * b;
  uint32_t* out_mask = mask + (int64_t)row * words;
  const bool in_regs = n <= kSelBlock * KR;

  uint32_t key[KR];
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const int j = t + q * kSelBlock;
      key[q] = j < n ? order_key(sc[j]) : 0u;
    }
  }
  uint32_t T, need_eq, eq_total;
  radix_threshold<KR>(key, in_regs, sc, n, b, &hist[0][0], sh, &T, &need_eq, &eq_total);

  compact_topb<KR>(key, in_regs, sc, n, b, T, need_eq, eq_total, ctab,
                   [&](uint32_t pos, int j, uint32_t) { out_idx[pos] = j; },
                   [&](int w, uint32_t bits) { out_mask[w] = bits; });
}

}  // namespace kvfix

using namespace kvfix;

extern "C" kvfix_status kvfix_score_ex(const kvfix_plane* fresh, int32_t fresh_layer,
                                       const kvfix_plane* reuse, int32_t reuse_layer,
                                       const kvfix_rope* rope, const kvfix_granularity* opt,
                                       float* scores, void* stream) {
  KVFIX_TRY(check_plane(fresh));
  KVFIX_TRY(check_plane(reuse));
  KVFIX_TRY(same_rows(fresh, reuse));
  if (scores == nullptr) return KVFIX_ERR_ARG;
  if (fresh_layer < 0 || fresh_layer >= fresh->n_layers || reuse_layer < 0 ||
      reuse_layer >= reuse->n_layers)
    return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(rope, reuse->head_dim));
  if (opt && opt->per_head != 0 && opt->per_head != 1) return KVFIX_ERR_ARG;
  if (reuse->n_segs == 0 || reuse->n_tokens == 0 || reuse->n_heads == 0) return KVFIX_OK;
  ScoreParams P;
  P.fresh = make_dplane(*fresh);
  P.reuse = make_dplane(*reuse);
  P.fl = fresh_layer;
  P.rl = reuse_layer;
  P.rope = make_rope_args(rope, reuse->head_dim);
  P.scores = scores;
  P.S = reuse->n_segs; P.H = reuse->n_heads; P.n = reuse->n_tokens;
  P.tok_blocks = 0;
  P.per_head = opt ? opt->per_head : 0;
  const int style = rope ? rope->style : kStyleNone;
  // The dispatcher lives with the correction kernels; replicate it here.
#define KVFIX_SCASE(T_, HD_, ST_)                                              \
  if (reuse->dtype == (std::is_same<T_, float>::value ? KVFIX_F32 : KVFIX_BF16) && \
      reuse->head_dim == HD_ && style == ST_)                                  \
    return ScoreLaunch<T_, HD_, ST_>::run(P, (hipStream_t)stream);
#define KVFIX_SSTYLES(T_, HD_) \
  KVFIX_SCASE(T_, HD_, kStyleNone) KVFIX_SCASE(T_, HD_, kStyleHalf) KVFIX_SCASE(T_, HD_, kStyleInter)
  KVFIX_SSTYLES(float, 64) KVFIX_SSTYLES(float, 128) KVFIX_SSTYLES(float, 256)
  KVFIX_SSTYLES(bf16_t, 64) KVFIX_SSTYLES(bf16_t, 128) KVFIX_SSTYLES(bf16_t, 256)
#undef KVFIX_SSTYLES
#undef KVFIX_SCASE
  return KVFIX_ERR_UNSUPPORTED;
}

extern "C" kvfix_status kvfix_score(const kvfix_plane* fresh, int32_t fresh_layer,
                                    const kvfix_plane* reuse, int32_t reuse_layer,
                                    const kvfix_rope* rope, float* scores, void* stream) {
  return kvfix_score_ex(fresh, fresh_layer, reuse, reuse_layer, rope, nullptr, scores, stream);
}

extern "C" kvfix_status kvfix_select_topb(const float* scores, int32_t n_rows, int32_t n,
                                          int32_t b, int32_t* idx, uint32_t* mask,
                                          void* stream) {
  if (n_rows < 0 || n < 0 || b < 0 || b > n) return KVFIX_ERR_ARG;
  if (n_rows == 0 || n == 0) return KVFIX_OK;
  if (scores == nullptr || mask == nullptr || (b > 0 && idx == nullptr)) return KVFIX_ERR_ARG;
  if (n_rows > kMaxGrid) return KVFIX_ERR_ARG;
  const int words = (int)ceil_div(n, 32);
  // register keys per thread: the fewest columns (a power of two) that hold
  // the row; longer rows stream from memory through the 32-column path
  const int cols = (int)ceil_div(n, kSelBlock);
  const dim3 grid((unsigned)n_rows), block(kSelBlock);
  hipStream_t st = (hipStream_t)stream;
  if (cols <= 1) select_topb_kernel<1><<<grid, block, 0, st>>>(scores, n, b, idx, mask, words);
  else if (cols <= 2) select_topb_kernel<2><<<grid, block, 0, st>>>(scores, n, b, idx, mask, words);
  else if (cols <= 4) select_topb_kernel<4><<<grid, block, 0, st>>>(scores, n, b, idx, mask, words);
  else if (cols <= 8) select_topb_kernel<8><<<grid, block, 0, st>>>(scores, n, b, idx, mask, words);
  else if (cols <= 16) select_topb_kernel<16><<<grid, block, 0, st>>>(scores, n, b, idx, mask, words);
  else select_topb_kernel<kSelRegKeys><<<grid, block, 0, st>>>(scores, n, b, idx, mask, words);
  return launch_status();
}
