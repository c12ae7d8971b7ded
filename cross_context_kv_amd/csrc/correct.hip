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
#include <type_traits>

#include "common.h"
#include "host_util.h"

namespace kvfix {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

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
  rope_table<HD, double>(P.rope, P.rope.delta[s], tc, ts);
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
        io = row_offset(P.src, l, s, h, j);
        oo[u] = row_offset(P.dst, l, s, h, j);
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
// fit_mean
// ---------------------------------------------------------------------------

struct FitParams {
  DPlane fresh, reuse, out;
  int32_t has_out, fresh_by_slot, rotate;
  const int32_t* idx;
  int32_t b;
  DLowRank lr;
  RopeArgs rope;
  float* mu;
  int32_t S, H, n;
};

template <typename T, int HD, int STYLE, int MAXR>
__global__ __launch_bounds__(kBlock) void fit_mean_kernel(FitParams P) {
  constexpr int MS = STYLE == kStyleNone ? kStyleHalf : STYLE;
  using M = RowMap<T, HD, MS>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW, U = 2;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane % G, rw = lane / G;
  int unit = blockIdx.x;
  const int h = unit % P.H; unit /= P.H;
  const int s = unit % P.S;
  const int l = unit / P.S;

  __shared__ double tc[HD / 2], ts[HD / 2];
  __shared__ double part[kWavesPerBlock][HD];
  if constexpr (STYLE != kStyleNone) rope_table<HD, double>(P.rope, P.rope.delta[s], tc, ts);

  // Rank-state right factor B (zero past the rank).
  double Ba[MAXR > 0 ? MAXR : 1][V], Bb[MAXR > 0 ? MAXR : 1][V];
  const float* Arow_base = nullptr;
  if constexpr (MAXR > 0) {
    const float* Bp = P.lr.B + l * P.lr.sB_layer + s * P.lr.sB_seg + h * P.lr.sB_head;
    Arow_base = P.lr.A + l * P.lr.sA_layer + s * P.lr.sA_seg + h * P.lr.sA_head;
#pragma unroll
    for (int k = 0; k < MAXR; ++k)
#pragma unroll
      for (int m = 0; m < V; ++m) {
        const bool on = k < P.lr.rank;
        Ba[k][m] = on ? (double)Bp[k * HD + M::dim_a(g, m)] : 0.0;
        Bb[k][m] = on ? (double)Bp[k * HD + M::dim_b(g, m)] : 0.0;
      }
  }
  __syncthreads();
  double cs[V], sn[V];
  if constexpr (STYLE != kStyleNone) {
#pragma unroll
    for (int m = 0; m < V; ++m) { cs[m] = tc[g * V + m]; sn[m] = ts[g * V + m]; }
  }

  double acc_a[V], acc_b[V];
#pragma unroll
  for (int m = 0; m < V; ++m) { acc_a[m] = 0.0; acc_b[m] = 0.0; }

  const int32_t* idx = P.idx + (int64_t)s * P.b;
  constexpr int kStep = kWavesPerBlock * RPW;
  for (int k0 = wave * RPW + rw; k0 < P.b; k0 += kStep * U) {
    vu4 f0[U], f1[U], q0[U], q1[U];
    int jj[U];
    int64_t oo[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * kStep;
      live[u] = k < P.b;
      jj[u] = 0;
      oo[u] = -1;
      if (live[u]) {
        const int j = idx[k];
        jj[u] = j;
        live[u] = j >= 0 && j < P.n;   // an index out of range is dropped, never followed
      }
      if (live[u]) {
        const int j = jj[u];
        const int64_t fo = row_offset(P.fresh, l, s, h, P.fresh_by_slot ? k : j);
        const int64_t ro = row_offset(P.reuse, l, s, h, j);
        if (P.has_out) oo[u] = row_offset(P.out, l, s, h, j);
        live[u] = fo >= 0 && ro >= 0 && (!P.has_out || oo[u] >= 0);
        if (live[u]) {
          const T* fr = reinterpret_cast<const T*>(P.fresh.data) + fo;
          const T* rr = reinterpret_cast<const T*>(P.reuse.data) + ro;
          f0[u] = ld16(fr + M::off0(g));
          f1[u] = ld16(fr + M::off1(g));
          q0[u] = ld16(rr + M::off0(g));
          q1[u] = ld16(rr + M::off1(g));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      double p0[V], p1[V], fa[V], fb[V], ra[V], rb[V];
      Cd::unpack(f0[u], p0);
      Cd::unpack(f1[u], p1);
      parts_to_pairs<MS, V>(p0, p1, fa, fb);
      Cd::unpack(q0[u], p0);
      Cd::unpack(q1[u], p1);
      parts_to_pairs<MS, V>(p0, p1, ra, rb);
      if constexpr (STYLE != kStyleNone) rotate_pairs<V>(ra, rb, cs, sn);
      double ab_a[V], ab_b[V];
#pragma unroll
      for (int m = 0; m < V; ++m) { ab_a[m] = 0.0; ab_b[m] = 0.0; }
      if constexpr (MAXR > 0) {
        const float* Ar = Arow_base + (int64_t)jj[u] * P.lr.rank;
#pragma unroll
        for (int kk = 0; kk < MAXR; ++kk) {
          const double a = kk < P.lr.rank ? (double)Ar[kk] : 0.0;
#pragma unroll
          for (int m = 0; m < V; ++m) {
            ab_a[m] = fma(a, Ba[kk][m], ab_a[m]);
            ab_b[m] = fma(a, Bb[kk][m], ab_b[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < V; ++m) {
        acc_a[m] += (fa[m] - ra[m]) - ab_a[m];
        acc_b[m] += (fb[m] - rb[m]) - ab_b[m];
      }
      if (P.has_out) {
        T* orow = reinterpret_cast<T*>(P.out.data) + oo[u];
        st16(orow + M::off0(g), f0[u]);
        st16(orow + M::off1(g), f1[u]);
      }
    }
  }

  // Fixed-order reduction: butterfly over the rows of a wave, then the waves
  // in index order.
#pragma unroll
  for (int off = G; off < kWave; off <<= 1) {
#pragma unroll
    for (int m = 0; m < V; ++m) {
      acc_a[m] += __shfl_xor(acc_a[m], off);
      acc_b[m] += __shfl_xor(acc_b[m], off);
    }
  }
  if (rw == 0) {
#pragma unroll
    for (int m = 0; m < V; ++m) {
      part[wave][M::dim_a(g, m)] = acc_a[m];
      part[wave][M::dim_b(g, m)] = acc_b[m];
    }
  }
  __syncthreads();
  for (int d = threadIdx.x; d < HD; d += kBlock) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) t += part[w][d];
    const double mean = P.b > 0 ? t / (double)P.b : 0.0;
    P.mu[(((int64_t)l * P.S + s) * P.H + h) * HD + d] = (float)mean;
  }
}

// ---------------------------------------------------------------------------
// apply
// ---------------------------------------------------------------------------

struct ApplyParams {
  DPlane in, out;
  const uint32_t* mask;
  const float* scores;
  float w_lo, w_hi;
  const float* mu;
  DLowRank lr;
  RopeArgs rope;
  int32_t S, H, n, chunks, rows_per_block, mask_words;
};

template <typename T, typename C, int HD, int STYLE, int MAXR>
__global__ __launch_bounds__(kBlock) void apply_kernel(ApplyParams P) {
  constexpr int MS = STYLE == kStyleNone ? kStyleHalf : STYLE;
  using M = RowMap<T, HD, MS>;
  using Cc = Codec<T, C>;
  constexpr int V = M::V, G = M::G, RPW = M::RPW, U = 4;
  constexpr int R = MAXR > 0 ? MAXR : 1;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane % G, rw = lane / G;
  const int chunk = blockIdx.x % P.chunks;
  int unit = blockIdx.x / P.chunks;
  const int h = unit % P.H; unit /= P.H;
  const int s = unit % P.S;
  const int l = unit / P.S;
  const int j_begin = chunk * P.rows_per_block;
  const int j_end = min(P.n, j_begin + P.rows_per_block);

  __shared__ C tc[HD / 2], ts[HD / 2];
  if constexpr (STYLE != kStyleNone) rope_table<HD, C>(P.rope, P.rope.delta[s], tc, ts);

  // Per-unit constants: mean residual and rank-state right factor.
  const int64_t ubase = (((int64_t)l * P.S + s) * P.H + h) * HD;
  C mua[V], mub[V];
#pragma unroll
  for (int m = 0; m < V; ++m) {
    mua[m] = (C)P.mu[ubase + M::dim_a(g, m)];
    mub[m] = (C)P.mu[ubase + M::dim_b(g, m)];
  }
  C Ba[R][V], Bb[R][V];
  const float* Arow_base = nullptr;
  if constexpr (MAXR > 0) {
    const float* Bp = P.lr.B + l * P.lr.sB_layer + s * P.lr.sB_seg + h * P.lr.sB_head;
    Arow_base = P.lr.A + l * P.lr.sA_layer + s * P.lr.sA_seg + h * P.lr.sA_head;
#pragma unroll
    for (int k = 0; k < MAXR; ++k)
#pragma unroll
      for (int m = 0; m < V; ++m) {
        const bool on = k < P.lr.rank;
        Ba[k][m] = on ? (C)Bp[k * HD + M::dim_a(g, m)] : (C)0;
        Bb[k][m] = on ? (C)Bp[k * HD + M::dim_b(g, m)] : (C)0;
      }
  }
  __syncthreads();
  C cs[V], sn[V];
  if constexpr (STYLE != kStyleNone) {
#pragma unroll
    for (int m = 0; m < V; ++m) { cs[m] = tc[g * V + m]; sn[m] = ts[g * V + m]; }
  }

  const uint32_t* mrow = P.mask ? P.mask + (int64_t)s * P.mask_words : nullptr;
  const float* srow = P.scores ? P.scores + (int64_t)s * P.n : nullptr;
  constexpr int kStep = kWavesPerBlock * RPW;
  for (int j0 = j_begin + wave * RPW + rw; j0 < j_end; j0 += kStep * U) {
    vu4 r0[U], r1[U];
    int64_t oo[U];
    bool live[U];
    C w[U];
    C Av[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kStep;
      live[u] = j < j_end;
      oo[u] = -1;
      w[u] = (C)1;
      if (live[u] && mrow) live[u] = ((mrow[j >> 5] >> (j & 31)) & 1u) == 0;
      int64_t io = -1;
      if (live[u]) {
        io = row_offset(P.in, l, s, h, j);
        oo[u] = row_offset(P.out, l, s, h, j);
        live[u] = io >= 0 && oo[u] >= 0;
      }
      if (live[u]) {
        const T* row = reinterpret_cast<const T*>(P.in.data) + io;
        r0[u] = ld16(row + M::off0(g));
        r1[u] = ld16(row + M::off1(g));
        if (srow) w[u] = (C)fminf(fmaxf(srow[j], P.w_lo), P.w_hi);
        if constexpr (MAXR > 0) {
          const float* Ar = Arow_base + (int64_t)j * P.lr.rank;
#pragma unroll
          for (int k = 0; k < MAXR; ++k) Av[u][k] = k < P.lr.rank ? (C)Ar[k] : (C)0;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      C p0[V], p1[V], a[V], b[V];
      Cc::unpack(r0[u], p0);
      Cc::unpack(r1[u], p1);
      parts_to_pairs<MS, V>(p0, p1, a, b);
      if constexpr (STYLE != kStyleNone) rotate_pairs<V>(a, b, cs, sn);
#pragma unroll
      for (int m = 0; m < V; ++m) {
        C xa = a[m] + w[u] * mua[m];
        C xb = b[m] + w[u] * mub[m];
        if constexpr (MAXR > 0) {
#pragma unroll
          for (int k = 0; k < MAXR; ++k) {
            xa += Av[u][k] * Ba[k][m];
            xb += Av[u][k] * Bb[k][m];
          }
        }
        a[m] = xa;
        b[m] = xb;
      }
      pairs_to_parts<MS, V>(a, b, p0, p1);
      T* row = reinterpret_cast<T*>(P.out.data) + oo[u];
      st16(row + M::off0(g), Cc::pack(p0));
      st16(row + M::off1(g), Cc::pack(p1));
    }
  }
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
  static kvfix_status run(const FitParams& P, int rank_var, int64_t grid, hipStream_t st) {
    switch (rank_var) {
      case 0: fit_mean_kernel<T, HD, STYLE, 0><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
      case 2: fit_mean_kernel<T, HD, STYLE, 2><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
      case 4: fit_mean_kernel<T, HD, STYLE, 4><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
      default: fit_mean_kernel<T, HD, STYLE, 8><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
    }
    return launch_status();
  }
};

template <typename T, int HD, int STYLE>
struct ApplyLaunch {
  using C = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
  static kvfix_status run(const ApplyParams& P, int rank_var, int64_t grid, hipStream_t st) {
    switch (rank_var) {
      case 0: apply_kernel<T, C, HD, STYLE, 0><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
      case 2: apply_kernel<T, C, HD, STYLE, 2><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
      case 4: apply_kernel<T, C, HD, STYLE, 4><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
      default: apply_kernel<T, C, HD, STYLE, 8><<<dim3((unsigned)grid), dim3(kBlock), 0, st>>>(P); break;
    }
    return launch_status();
  }
};

// Rows per block: 256 for streaming kernels (64 KB of bf16 hd-128 rows).
constexpr int kRowsPerBlock = 256;

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
  P.chunks = (src->n_tokens + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t grid = units * P.chunks;
  if (grid > kMaxGrid) return KVFIX_ERR_ARG;
  return dispatch_t_hd_style<RopeShiftLaunch>(src->dtype, src->head_dim, rope->style, P, grid,
                                              (hipStream_t)stream);
}

extern "C" kvfix_status kvfix_fit_mean(const kvfix_plane* fresh, int32_t fresh_by_slot,
                                       const kvfix_plane* reuse, const kvfix_plane* out,
                                       const int32_t* idx, int32_t b, const kvfix_rope* rope,
                                       const kvfix_lowrank* lowrank, float* mu, void* stream) {
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
  if (b < 0 || b > reuse->n_tokens) return KVFIX_ERR_ARG;
  if (b > 0 && idx == nullptr) return KVFIX_ERR_ARG;
  if (fresh_by_slot ? fresh->n_tokens < b : fresh->n_tokens != reuse->n_tokens)
    return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(rope, reuse->head_dim));
  KVFIX_TRY(check_lowrank(lowrank));
  const int64_t units = (int64_t)reuse->n_layers * reuse->n_segs * reuse->n_heads;
  if (units == 0) return KVFIX_OK;
  if (units > kMaxGrid) return KVFIX_ERR_ARG;
  FitParams P;
  P.fresh = make_dplane(*fresh);
  P.reuse = make_dplane(*reuse);
  P.out = out ? make_dplane(*out) : make_dplane(*reuse);
  P.has_out = out != nullptr;
  P.fresh_by_slot = fresh_by_slot != 0;
  P.rotate = rope != nullptr;
  P.idx = idx;
  P.b = b;
  P.lr = make_dlowrank(lowrank);
  P.rope = make_rope_args(rope, reuse->head_dim);
  P.mu = mu;
  P.S = reuse->n_segs; P.H = reuse->n_heads; P.n = reuse->n_tokens;
  const int style = rope ? rope->style : kStyleNone;
  return dispatch_t_hd_style<FitLaunch>(reuse->dtype, reuse->head_dim, style, P,
                                        rank_variant(P.lr.rank), units, (hipStream_t)stream);
}

extern "C" kvfix_status kvfix_apply(const kvfix_plane* reuse, const kvfix_plane* out,
                                    const uint32_t* mask, const float* scores, float w_lo,
                                    float w_hi, const float* mu, const kvfix_lowrank* lowrank,
                                    const kvfix_rope* rope, void* stream) {
  KVFIX_TRY(check_plane(reuse));
  KVFIX_TRY(check_plane(out));
  KVFIX_TRY(same_rows(reuse, out));
  if (reuse->n_layers != out->n_layers || mu == nullptr) return KVFIX_ERR_ARG;
  if (scores && !(w_lo <= w_hi)) return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(rope, reuse->head_dim));
  KVFIX_TRY(check_lowrank(lowrank));
  const int64_t units = (int64_t)reuse->n_layers * reuse->n_segs * reuse->n_heads;
  if (units == 0 || reuse->n_tokens == 0) return KVFIX_OK;
  ApplyParams P;
  P.in = make_dplane(*reuse);
  P.out = make_dplane(*out);
  P.mask = mask;
  P.scores = scores;
  P.w_lo = w_lo;
  P.w_hi = w_hi;
  P.mu = mu;
  P.lr = make_dlowrank(lowrank);
  P.rope = make_rope_args(rope, reuse->head_dim);
  P.S = reuse->n_segs; P.H = reuse->n_heads; P.n = reuse->n_tokens;
  P.mask_words = (reuse->n_tokens + 31) / 32;
  P.rows_per_block = kRowsPerBlock;
  P.chunks = (reuse->n_tokens + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t grid = units * P.chunks;
  if (grid > kMaxGrid) return KVFIX_ERR_ARG;
  const int style = rope ? rope->style : kStyleNone;
  return dispatch_t_hd_style<ApplyLaunch>(reuse->dtype, reuse->head_dim, style, P,
                                          rank_variant(P.lr.rank), grid, (hipStream_t)stream);
}
