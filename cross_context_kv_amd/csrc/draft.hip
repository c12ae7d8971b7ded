// Draft attention-mass score (a3) on MFMA.
//
// a[s][j] = sum over layers l >= first, query heads h and draft rows t of
// softmax_j( q'(s,l,h,t) . k(l,s,g(h),j) ),  q' = R(-delta_s) q / sqrt(hd),
// g(h) = h / (Hq / H).  Rotating the query instead of every key gives the
// same logits (q . R(d) k = R(-d) q . k) and leaves K untouched in HBM.
//
// logits : one 256-thread block per (s, l, KV head g, chunk of 1024 keys).
//          The block's query tile (the group x n_draft rows that read head g,
//          <= 16 rows) is rotated and scaled in fp64 and split into three
//          bf16 parts hi + mid + lo (together fp32-accurate); each wave runs
//          v_mfma_f32_16x16x32_bf16 over 16 key tiles (3 parts x 4 k-steps per
//          tile).  Logits go to the workspace, in base-2 units.  Each lane
//          keeps a running (max, sum exp) per query row over its own keys;
//          the 16 lanes of a row and the 4 waves are combined once, at the
//          end of the chunk.
// mass   : one 256-thread block per (s, split of the query rows, 1024 keys).
//          The block first forms each of its rows' maximum M and 1/Z from
//          the chunk statistics (fp64, fixed order), then every thread adds
//          exp(x - M) / Z over the split's rows for four keys (16-byte
//          non-temporal loads, sixteen rows in flight), in fp64, in row order.  The exponentials
//          are the hardware's base-2 exponential (within about one unit of
//          2^-24 relative for these arguments, which are <= 0).
// total  : per key, the splits added in split order, rounded once to fp32.
#include <type_traits>

#include "common.h"
#include "host_util.h"

namespace kvfix {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDraftHD = 128;
constexpr int kDraftBlock = 256;
constexpr int kTilesPerWave = 16;
constexpr int kDraftChunk = (kDraftBlock / kWave) * kTilesPerWave * 16;   // 1024 keys
constexpr int kMassKeys = 1024;          // keys per mass block (4 per thread)
constexpr int kMassRowsMax = 64;         // query rows per mass block (one split)
constexpr int kMassUnroll = 16;          // rows in flight per thread

struct DraftParams {
  const bf16_t* q;          // [S][L][Hq][T][hd]
  DPlane k;
  RopeArgs rope;
  float* logits;            // [S*Lf*Hq*T][ldl]
  float2* stats;            // [S*Lf*Hq*T][n_chunks]
  int32_t S, L, first, Hq, H, T, group, qr, n, n_chunks;
  int64_t ldl;              // logit row pitch (floats)
};

__device__ __forceinline__ bf16_t bf16_bits_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Logits are kept in base-2 units, x = log2(e) q'.k (the query is scaled by
// log2(e) / sqrt(hd)), so that softmax_j = 2^(x_j - M) / sum 2^(x - M) and
// every exponential is one v_exp_f32.

// Merge running softmax statistics (m, s): s holds sum 2^(x - m).
__device__ __forceinline__ void stat_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;                       // both empty
  s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - mn)) +
      (m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f(m2 - mn));
  m = mn;
}

// Key tiles: a wave's 16-key tile (4 KiB) is loaded with each instruction
// covering 1 KiB of consecutive bytes (lane L: key 4 i + L / 16 of the tile,
// bytes 16 (L % 16) ..), written to a wave-private LDS buffer, and read back
// in the MFMA operand layout (lane L: key L % 16, 16-byte chunk 4 m + L / 16
// for k-step m).  Chunk c of key j sits at slot j * 16 + (c ^ j), so that
// both the writes and the operand reads touch 16 different slots per key
// row.  Loading the operand layout directly would read 64-byte pieces of 16
// rows per instruction, which streams HBM markedly slower.  Planes whose
// token rows are not head_dim apart, and paged pools, load per key instead.
template <int STYLE, bool CONTIG>
__global__ __launch_bounds__(kDraftBlock) void draft_logits_kernel(DraftParams P) {
  constexpr int HD = kDraftHD;
  __shared__ double tc[HD / 2], ts[HD / 2];
  __shared__ __attribute__((aligned(16))) bf16_t qs[3][16][HD];   // hi, mid, lo parts of the query tile
  __shared__ float wstat[4][16][2];
  __shared__ vu4 ktile[CONTIG ? 4 : 1][CONTIG ? 256 : 1];         // one 16-key tile per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Lf = P.L - P.first;
  int u = blockIdx.x;
  const int chunk = u % P.n_chunks; u /= P.n_chunks;
  const int g = u % P.H; u /= P.H;
  const int lf = u % Lf;
  const int s = u / Lf;
  const int l = P.first + lf;
  const int key_base = chunk * kDraftChunk + wave * (kTilesPerWave * 16);
  const bool full = (chunk + 1) * kDraftChunk <= P.n;     // uniform: no key past n
  const int akq = lane >> 4;
  const int jl = key_base + (lane & 15);                  // this lane's operand key, tile 0

  constexpr int TG = 4;                                   // tiles loaded together
  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(P.k.data);
  // contiguous tiles: the wave's first key row; lane L reads 16 bytes at
  // element 8 L of each 1 KiB piece
  const bf16_t* kw = kbase;
  int64_t tstep = 0;
  if constexpr (CONTIG) {
    kw += (int64_t)l * P.k.s_layer + (int64_t)s * P.k.s_seg + (int64_t)g * P.k.s_head +
          (int64_t)key_base * HD + 8 * lane;
    tstep = 16 * HD;
  }
  auto load_group = [&](int tt0, vu4 (&B)[TG][4]) {
#pragma unroll
    for (int q = 0; q < TG; ++q) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if constexpr (CONTIG) {
          const int j = key_base + (tt0 + q) * 16 + 4 * kk + akq;      // key this lane reads
          B[q][kk] = (full || j < P.n) ? ld16(kw + (tt0 + q) * tstep + kk * 512)
                                       : vu4{0u, 0u, 0u, 0u};
        } else {
          const int j = jl + (tt0 + q) * 16;
          const int64_t off = j < P.n ? row_offset(P.k, l, s, g, j) : -1;
          B[q][kk] = off >= 0 ? ld16(kbase + off + kk * 32 + 8 * akq) : vu4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  // The first key tiles' loads go out before the query tile is prepared.
  vu4 B[TG][4];
  load_group(0, B);

  // rotary table for a shift of -delta: cos stays, sin flips sign
  if (tid < HD / 2) {
    double sv, cv;
    rope_sincos((double)P.rope.delta[s] * P.rope.inv_freq[tid], &sv, &cv);
    tc[tid] = cv;
    ts[tid] = -sv;
  }
  __syncthreads();
  // query tile: rows r < qr are (head g*group + r / T, draft row r % T),
  // scaled by log2(e) / sqrt(hd)
  const double scale = 1.4426950408889634074 / sqrt((double)HD);
  const bf16_t* qbase = P.q + ((((int64_t)s * P.L + l) * P.Hq + (int64_t)g * P.group) * P.T) * HD;
  for (int job = tid; job < 16 * (HD / 2); job += kDraftBlock) {
    const int r = job / (HD / 2), i = job % (HD / 2);
    const int da = STYLE == kStyleInter ? 2 * i : i;
    const int db = STYLE == kStyleInter ? 2 * i + 1 : i + HD / 2;
    double ya = 0.0, yb = 0.0;
    if (r < P.qr) {
      const bf16_t* qr = qbase + (int64_t)r * HD;
      const double xa = (double)__uint_as_float((uint32_t)qr[da] << 16);
      const double xb = (double)__uint_as_float((uint32_t)qr[db] << 16);
      ya = (xa * tc[i] - xb * ts[i]) * scale;
      yb = (xb * tc[i] + xa * ts[i]) * scale;
    }
    const double y2[2] = {ya, yb};
    const int d2[2] = {da, db};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      // three-term split: hi + mid + lo reproduces y to about 2^-24 relative
      const bf16_t hi = bf16_bits_rne((float)y2[e]);
      const double r1 = y2[e] - (double)__uint_as_float((uint32_t)hi << 16);
      const bf16_t mid = bf16_bits_rne((float)r1);
      const double r2 = r1 - (double)__uint_as_float((uint32_t)mid << 16);
      const bf16_t lo = bf16_bits_rne((float)r2);
      qs[0][r][d2[e]] = hi;
      qs[1][r][d2[e]] = mid;
      qs[2][r][d2[e]] = lo;
    }
  }
  __syncthreads();

  // A operands: lane holds row (lane % 16), dims kk*32 + 8*(lane/16) .. +8
  const int arow = lane & 15;
  bf16x8 A[3][4];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      A[p][kk] = *reinterpret_cast<const bf16x8*>(&qs[p][arow][kk * 32 + 8 * akq]);

  // running statistics of this lane's keys for its 4 rows
  float m_run[4], s_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }
  const int64_t qrow0 = (((int64_t)s * Lf + lf) * P.Hq + (int64_t)g * P.group) * P.T;
  // this lane's logit row pointers (its 4 rows, at its key of tile 0)
  float* lrow[4];
  bool rv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (lane >> 4) + i;
    rv[i] = r < P.qr;
    lrow[i] = P.logits + (qrow0 + r) * P.ldl + jl;
  }

  // Operand of tile q for k-step m (contiguous tiles: through the wave's LDS buffer).
  vu4* kt = ktile[CONTIG ? wave : 0];
  const int jo = lane & 15;                                // operand key of this lane
  for (int tt0 = 0; tt0 < kTilesPerWave; tt0 += TG) {
    if (tt0 > 0) load_group(tt0, B);
    f32x4 acc[TG];
#pragma unroll
    for (int q = 0; q < TG; ++q) {
      acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      vu4 Bo[4];
      if constexpr (CONTIG) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int kq = 4 * kk + akq;                     // key (in the tile) of B[q][kk]
          kt[kq * 16 + ((lane & 15) ^ kq)] = B[q][kk];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);               // lgkmcnt(0): the tile is in LDS
#pragma unroll
        for (int m = 0; m < 4; ++m) Bo[m] = kt[jo * 16 + ((4 * m + akq) ^ jo)];
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) Bo[m] = B[q][m];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int p = 2; p >= 0; --p)
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[p][kk], __builtin_bit_cast(bf16x8, Bo[kk]),
                                                          acc[q], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < TG; ++q) {
      // lane holds rows 4*(lane/16)+i of key jl + (tt0 + q) * 16
      if (!full && jl + (tt0 + q) * 16 >= P.n) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc[q][i];
        if (rv[i]) lrow[i][(tt0 + q) * 16] = x;
        // one exponential per logit, e = 2^-|x - m|: a new maximum
        // rescales the sum, any other logit adds to it (m = -inf: s = 1)
        const float d = x - m_run[i];
        const float e = __builtin_amdgcn_exp2f(-fabsf(d));
        s_run[i] = d > 0.f ? fmaf(s_run[i], e, 1.0f) : s_run[i] + e;
        m_run[i] = fmaxf(m_run[i], x);
      }
    }
  }

  // combine the 16 lanes of each row (fixed butterfly), then the waves
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float m2 = __shfl_xor(m_run[i], off), s2 = __shfl_xor(s_run[i], off);
      stat_merge(m_run[i], s_run[i], m2, s2);
    }
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wstat[wave][4 * (lane >> 4) + i][0] = m_run[i];
      wstat[wave][4 * (lane >> 4) + i][1] = s_run[i];
    }
  }
  __syncthreads();
  if (tid < P.qr) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wstat[w][tid][0]);
    float Z = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (wstat[w][tid][0] != -INFINITY)
        Z += wstat[w][tid][1] * __builtin_amdgcn_exp2f(wstat[w][tid][0] - M);
    P.stats[(qrow0 + tid) * P.n_chunks + chunk] = make_float2(M, Z);
  }
}

// Mass of a split of the segment's query rows over kMassKeys keys (logits in
// base-2 units).
//   partial[s][split][j] = sum over rows r of the split of 2^(x_rj - M_r) / Z_r
// with M_r = the row's maximum over its chunks and Z_r = sum over chunks of
// their sums rescaled to M_r (fp64, chunk order), both formed here first.
struct MassParams {
  const float* logits;      // [S][qps][ldl]
  const float2* stats;      // [S][qps][n_chunks]
  double* partial;          // [S][splits][ldl]
  int32_t qps, n, n_chunks, splits, rows_per_split, key_blocks;
  int64_t ldl;
};

__global__ __launch_bounds__(256) void draft_mass_kernel(MassParams P) {
  __shared__ float sM[kMassRowsMax], sZ[kMassRowsMax];
  // Splits run last first: the logits written last (the last layers) are
  // the likeliest to be still in the last-level cache.
  int u = blockIdx.x;
  const int kb = u % P.key_blocks; u /= P.key_blocks;
  const int split = P.splits - 1 - u % P.splits;
  const int s = u / P.splits;
  const int r0 = split * P.rows_per_split;
  const int nr = min(P.qps - r0, P.rows_per_split);
  const int j0 = kb * kMassKeys + 4 * threadIdx.x;
  const float* lg = P.logits + ((int64_t)s * P.qps + r0) * P.ldl;
  const bool full = j0 + 3 < P.n;                  // ldl is a multiple of 64
  if ((int)threadIdx.x < nr) {
    const float2* st = P.stats + ((int64_t)s * P.qps + r0 + threadIdx.x) * P.n_chunks;
    float M = -INFINITY;
    for (int c = 0; c < P.n_chunks; ++c) M = fmaxf(M, st[c].x);
    double Z = 0.0;
    for (int c = 0; c < P.n_chunks; ++c)
      if (st[c].x != -INFINITY) Z += (double)st[c].y * exp2((double)st[c].x - (double)M);
    sM[threadIdx.x] = M;
    sZ[threadIdx.x] = (float)(1.0 / Z);
  }
  __syncthreads();
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (j0 < P.n) {
    int r = 0;
    for (; r + kMassUnroll <= nr; r += kMassUnroll) {
      float4 x[kMassUnroll];
#pragma unroll
      for (int e = 0; e < kMassUnroll; ++e) {
        const float* p = lg + (int64_t)(r + e) * P.ldl + j0;
        if (full) x[e] = __builtin_bit_cast(float4, ld16(p));     // read once: non-temporal
        else {
          x[e].x = p[0];
          x[e].y = j0 + 1 < P.n ? p[1] : 0.f;
          x[e].z = j0 + 2 < P.n ? p[2] : 0.f;
          x[e].w = j0 + 3 < P.n ? p[3] : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < kMassUnroll; ++e) {
        const float M = sM[r + e], iz = sZ[r + e];
        acc[0] += (double)(__builtin_amdgcn_exp2f(x[e].x - M) * iz);
        acc[1] += (double)(__builtin_amdgcn_exp2f(x[e].y - M) * iz);
        acc[2] += (double)(__builtin_amdgcn_exp2f(x[e].z - M) * iz);
        acc[3] += (double)(__builtin_amdgcn_exp2f(x[e].w - M) * iz);
      }
    }
    for (; r < nr; ++r) {
      const float* p = lg + (int64_t)r * P.ldl + j0;
      const float M = sM[r], iz = sZ[r];
      acc[0] += (double)(__builtin_amdgcn_exp2f(p[0] - M) * iz);
      if (j0 + 1 < P.n) acc[1] += (double)(__builtin_amdgcn_exp2f(p[1] - M) * iz);
      if (j0 + 2 < P.n) acc[2] += (double)(__builtin_amdgcn_exp2f(p[2] - M) * iz);
      if (j0 + 3 < P.n) acc[3] += (double)(__builtin_amdgcn_exp2f(p[3] - M) * iz);
    }
    double* out = P.partial + ((int64_t)s * P.splits + split) * P.ldl + j0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j0 + e < P.n) out[e] = acc[e];
  }
}

// a[s][j] = the splits' partial masses added in split order, rounded to fp32.
__global__ void draft_total_kernel(const double* partial, int S, int splits, int n, int64_t ldl,
                                   float* scores) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)S * n) return;
  const int s = (int)(i / n), j = (int)(i % n);
  const double* p = partial + (int64_t)s * splits * ldl + j;
  double t = 0.0;
  int k = 0;
  for (; k + 8 <= splits; k += 8) {               // eight loads in flight, added in order
    double x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = p[(int64_t)(k + e) * ldl];
#pragma unroll
    for (int e = 0; e < 8; ++e) t += x[e];
  }
  for (; k < splits; ++k) t += p[(int64_t)k * ldl];
  scores[i] = (float)t;
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Query rows per segment are cut into splits of at most kMassRowsMax rows.
inline int mass_splits(int64_t qps) { return (int)((qps + kMassRowsMax - 1) / kMassRowsMax); }

// Row pitch (floats) of the logits and of the partial masses: n rounded up
// to 64 plus 64, so rows are 256-byte aligned and never a power of two apart
// (rows a power of two apart fall on the same memory channels).
inline int64_t logit_pitch(int64_t n) { return (n + 63) / 64 * 64 + 64; }

}  // namespace kvfix

using namespace kvfix;

extern "C" size_t kvfix_score_draft_workspace(int32_t n_segs, int32_t n_layers, int32_t first_layer,
                                              int32_t n_q_heads, int32_t n_draft, int32_t n_tokens) {
  if (n_segs < 0 || n_layers < 0 || first_layer < 0 || n_q_heads < 0 || n_draft < 0 ||
      n_tokens < 0)
    return 0;
  const int64_t lf = n_layers > first_layer ? n_layers - first_layer : 0;
  const int64_t qps = lf * n_q_heads * n_draft;
  const size_t rows = (size_t)n_segs * qps;
  const size_t chunks = ((size_t)n_tokens + kDraftChunk - 1) / kDraftChunk;
  const size_t splits = qps > 0 ? (size_t)mass_splits(qps) : 1;
  const size_t ldl = (size_t)logit_pitch(n_tokens);
  return al256(rows * ldl * 4) + al256(rows * chunks * 8) + al256((size_t)n_segs * splits * ldl * 8);
}

extern "C" kvfix_status kvfix_score_draft(const void* q, int32_t n_q_heads, int32_t n_draft,
                                          const kvfix_plane* k, int32_t first_layer,
                                          const kvfix_rope* rope, float* scores, void* ws,
                                          size_t ws_bytes, void* stream) {
  KVFIX_TRY(check_plane(k));
  if (k->dtype != KVFIX_BF16 || k->head_dim != kDraftHD) return KVFIX_ERR_UNSUPPORTED;
  if (q == nullptr || scores == nullptr || rope == nullptr) return KVFIX_ERR_ARG;
  if (!aligned16(q)) return KVFIX_ERR_ALIGN;
  KVFIX_TRY(check_rope(rope, k->head_dim));
  if (n_draft <= 0 || n_q_heads <= 0 || k->n_heads <= 0 || n_q_heads % k->n_heads != 0)
    return KVFIX_ERR_ARG;
  const int32_t group = n_q_heads / k->n_heads;
  if (group * n_draft > 16) return KVFIX_ERR_UNSUPPORTED;
  if (first_layer < 0 || first_layer > k->n_layers) return KVFIX_ERR_ARG;
  const int32_t S = k->n_segs, L = k->n_layers, n = k->n_tokens;
  if (S == 0 || n == 0) return KVFIX_OK;
  const size_t need = kvfix_score_draft_workspace(S, L, first_layer, n_q_heads, n_draft, n);
  if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255))
    return KVFIX_ERR_ARG;
  const int32_t Lf = L - first_layer;
  const int64_t qps = (int64_t)Lf * n_q_heads * n_draft;
  const int64_t rows = (int64_t)S * qps;
  const int32_t n_chunks = (int32_t)ceil_div(n, kDraftChunk);
  const int splits = qps > 0 ? mass_splits(qps) : 1;
  const int key_blocks = (int)ceil_div(n, kMassKeys);
  // every grid size is checked before the first launch
  const int64_t lgrid = (int64_t)S * Lf * k->n_heads * n_chunks;
  const int64_t mgrid = (int64_t)S * splits * key_blocks;
  const int64_t tgrid = ((int64_t)S * n + 255) / 256;
  if (lgrid > kMaxGrid || mgrid > kMaxGrid || tgrid > kMaxGrid || qps > 0x7fffffff)
    return KVFIX_ERR_ARG;
  const int64_t ldl = logit_pitch(n);
  char* w = static_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(w);
  float2* stats = reinterpret_cast<float2*>(w + al256((size_t)rows * ldl * 4));
  double* partial = reinterpret_cast<double*>(w + al256((size_t)rows * ldl * 4) +
                                              al256((size_t)rows * n_chunks * 8));
  hipStream_t st = (hipStream_t)stream;
  if (rows > 0) {
    DraftParams P;
    P.q = static_cast<const bf16_t*>(q);
    P.k = make_dplane(*k);
    P.rope = make_rope_args(rope, k->head_dim);
    P.logits = logits;
    P.stats = stats;
    P.S = S; P.L = L; P.first = first_layer; P.Hq = n_q_heads; P.H = k->n_heads; P.T = n_draft;
    P.group = group; P.qr = group * n_draft; P.n = n; P.n_chunks = n_chunks; P.ldl = ldl;
    const dim3 lg((unsigned)lgrid), lb(kDraftBlock);
    // contiguous key rows (dense, token stride = head_dim): 1 KiB loads
    const bool contig = k->page_table == nullptr && k->s_token == kDraftHD;
    if (rope->style == KVFIX_ROPE_HALF) {
      if (contig) draft_logits_kernel<kStyleHalf, true><<<lg, lb, 0, st>>>(P);
      else draft_logits_kernel<kStyleHalf, false><<<lg, lb, 0, st>>>(P);
    } else {
      if (contig) draft_logits_kernel<kStyleInter, true><<<lg, lb, 0, st>>>(P);
      else draft_logits_kernel<kStyleInter, false><<<lg, lb, 0, st>>>(P);
    }
    KVFIX_TRY(launch_status());
    MassParams M;
    M.logits = logits; M.stats = stats; M.partial = partial;
    M.qps = (int32_t)qps; M.n = n; M.n_chunks = n_chunks; M.splits = splits;
    M.rows_per_split = kMassRowsMax; M.key_blocks = key_blocks; M.ldl = ldl;
    draft_mass_kernel<<<dim3((unsigned)mgrid), dim3(256), 0, st>>>(M);
    KVFIX_TRY(launch_status());
    draft_total_kernel<<<dim3((unsigned)tgrid), dim3(256), 0, st>>>(partial, S, splits, n, ldl,
                                                                     scores);
  } else {
    // no query rows (first_layer == n_layers): every mass is 0 (no split is read)
    draft_total_kernel<<<dim3((unsigned)tgrid), dim3(256), 0, st>>>(partial, S, 0, n, ldl, scores);
  }
  return launch_status();
}
