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
//          tile).  Logits go to the workspace; an online (max, sum exp) per
//          row and chunk goes beside them.
// norm   : per query row, combine the chunk statistics (fp64, fixed order)
//          into the row maximum M and 1/Z.
// mass   : per (s, 64 keys), sum exp(x - M) / Z over every query row of the
//          segment in fp64, in a fixed order; round once to fp32.
#include "common.h"
#include "host_util.h"

namespace kvfix {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDraftHD = 128;
constexpr int kDraftBlock = 256;
constexpr int kTilesPerWave = 16;
constexpr int kDraftChunk = (kDraftBlock / kWave) * kTilesPerWave * 16;   // 1024 keys
constexpr int kMassKeys = 64;

struct DraftParams {
  const bf16_t* q;          // [S][L][Hq][T][hd]
  DPlane k;
  RopeArgs rope;
  float* logits;            // [S*Lf*Hq*T][n]
  float2* stats;            // [S*Lf*Hq*T][n_chunks]
  int32_t S, L, first, Hq, H, T, group, qr, n, n_chunks;
};

__device__ __forceinline__ bf16_t bf16_bits_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Three waves per SIMD: the instance fits in 168 VGPRs without spilling
// (the compiler's own choice, 176, leaves two).
template <int STYLE>
__global__ __launch_bounds__(kDraftBlock) __attribute__((amdgpu_waves_per_eu(3)))
void draft_logits_kernel(DraftParams P) {
  constexpr int HD = kDraftHD;
  __shared__ double tc[HD / 2], ts[HD / 2];
  __shared__ __attribute__((aligned(16))) bf16_t qs[3][16][HD];   // hi, mid, lo parts of the query tile
  __shared__ float wstat[4][16][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Lf = P.L - P.first;
  int u = blockIdx.x;
  const int chunk = u % P.n_chunks; u /= P.n_chunks;
  const int g = u % P.H; u /= P.H;
  const int lf = u % Lf;
  const int s = u / Lf;
  const int l = P.first + lf;

  // rotary table for a shift of -delta: cos stays, sin flips sign
  if (tid < HD / 2) {
    double sv, cv;
    rope_sincos((double)P.rope.delta[s] * P.rope.inv_freq[tid], &sv, &cv);
    tc[tid] = cv;
    ts[tid] = -sv;
  }
  __syncthreads();
  // query tile: rows r < qr are (head g*group + r / T, draft row r % T)
  const double scale = 1.0 / sqrt((double)HD);
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
  const int arow = lane & 15, akq = lane >> 4;
  bf16x8 A[3][4];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      A[p][kk] = *reinterpret_cast<const bf16x8*>(&qs[p][arow][kk * 32 + 8 * akq]);

  float m_run[4], s_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }
  const int64_t qrow0 = (((int64_t)s * Lf + lf) * P.Hq + (int64_t)g * P.group) * P.T;
  const int key_base = chunk * kDraftChunk + wave * (kTilesPerWave * 16);

  constexpr int TG = 4;                                   // tiles loaded together
  for (int tt0 = 0; tt0 < kTilesPerWave; tt0 += TG) {
    vu4 B[TG][4];
    int jj[TG];
#pragma unroll
    for (int q = 0; q < TG; ++q) {
      const int j = key_base + (tt0 + q) * 16 + (lane & 15);
      jj[q] = j;
      const int64_t off = j < P.n ? row_offset(P.k, l, s, g, j) : -1;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (off >= 0)
          B[q][kk] = ld16(reinterpret_cast<const bf16_t*>(P.k.data) + off + kk * 32 + 8 * akq);
        else
          B[q][kk] = vu4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < TG; ++q) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, B[q][kk]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2][kk], b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][kk], b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][kk], b, acc, 0, 0, 0);
      }
      // lane holds rows 4*(lane/16)+i of key jj[q]
      const bool kvalid = jj[q] < P.n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * (lane >> 4) + i;
        const float x = acc[i];
        if (kvalid && r < P.qr) P.logits[(qrow0 + r) * (int64_t)P.n + jj[q]] = x;
        float tmax = kvalid ? x : -INFINITY;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
        const float m_new = fmaxf(m_run[i], tmax);
        float e = (kvalid && m_new != -INFINITY) ? expf(x - m_new) : 0.f;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) e += __shfl_xor(e, off);
        const float keep = (m_run[i] == -INFINITY) ? 0.f : expf(m_run[i] - m_new);
        s_run[i] = s_run[i] * keep + e;
        m_run[i] = m_new;
      }
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
      if (wstat[w][tid][0] != -INFINITY) Z += wstat[w][tid][1] * expf(wstat[w][tid][0] - M);
    P.stats[(qrow0 + tid) * P.n_chunks + chunk] = make_float2(M, Z);
  }
}

// Per query row: M = max over chunks, Z = sum of chunk sums rescaled to M.
__global__ void draft_norm_kernel(const float2* stats, int rows, int n_chunks, float2* norm) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const float2* st = stats + (int64_t)r * n_chunks;
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, st[c].x);
  double Z = 0.0;
  for (int c = 0; c < n_chunks; ++c)
    if (st[c].x != -INFINITY) Z += (double)st[c].y * exp((double)st[c].x - (double)M);
  norm[r] = make_float2(M, (float)(1.0 / Z));
}

// a[s][j] = sum over the segment's query rows of exp(x - M) / Z.
__global__ __launch_bounds__(256) void draft_mass_kernel(const float* logits, const float2* norm,
                                                         int qps, int n, float* scores) {
  __shared__ double part[4][kMassKeys];
  const int blocks_per_seg = (n + kMassKeys - 1) / kMassKeys;
  const int s = blockIdx.x / blocks_per_seg;
  const int j = (blockIdx.x % blocks_per_seg) * kMassKeys + (threadIdx.x % kMassKeys);
  const int rg = threadIdx.x / kMassKeys;
  double acc = 0.0;
  if (j < n) {
    const float* lg = logits + (int64_t)s * qps * n + j;
    const float2* nm = norm + (int64_t)s * qps;
    int q = rg;
    for (; q + 12 < qps; q += 16) {
      const float x0 = lg[(int64_t)q * n], x1 = lg[(int64_t)(q + 4) * n];
      const float x2 = lg[(int64_t)(q + 8) * n], x3 = lg[(int64_t)(q + 12) * n];
      const float2 n0 = nm[q], n1 = nm[q + 4], n2 = nm[q + 8], n3 = nm[q + 12];
      acc += (double)(expf(x0 - n0.x) * n0.y);
      acc += (double)(expf(x1 - n1.x) * n1.y);
      acc += (double)(expf(x2 - n2.x) * n2.y);
      acc += (double)(expf(x3 - n3.x) * n3.y);
    }
    for (; q < qps; q += 4) {
      const float2 nq = nm[q];
      acc += (double)(expf(lg[(int64_t)q * n] - nq.x) * nq.y);
    }
  }
  part[rg][threadIdx.x % kMassKeys] = acc;
  __syncthreads();
  if (threadIdx.x < kMassKeys && j < n) {
    const double t = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] +
                     part[3][threadIdx.x];
    scores[(int64_t)s * n + j] = (float)t;
  }
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace kvfix

using namespace kvfix;

extern "C" size_t kvfix_score_draft_workspace(int32_t n_segs, int32_t n_layers, int32_t first_layer,
                                              int32_t n_q_heads, int32_t n_draft, int32_t n_tokens) {
  if (n_segs < 0 || n_layers < 0 || first_layer < 0 || n_q_heads < 0 || n_draft < 0 ||
      n_tokens < 0)
    return 0;
  const int64_t lf = n_layers > first_layer ? n_layers - first_layer : 0;
  const size_t rows = (size_t)n_segs * lf * n_q_heads * n_draft;
  const size_t chunks = ((size_t)n_tokens + kDraftChunk - 1) / kDraftChunk;
  return al256(rows * n_tokens * 4) + al256(rows * chunks * 8) + al256(rows * 8);
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
  const int64_t rows = (int64_t)S * Lf * n_q_heads * n_draft;
  const int32_t n_chunks = (n + kDraftChunk - 1) / kDraftChunk;
  char* w = static_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(w);
  float2* stats = reinterpret_cast<float2*>(w + al256((size_t)rows * n * 4));
  float2* norm = reinterpret_cast<float2*>(w + al256((size_t)rows * n * 4) +
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
    P.group = group; P.qr = group * n_draft; P.n = n; P.n_chunks = n_chunks;
    const int64_t grid = (int64_t)S * Lf * k->n_heads * n_chunks;
    if (grid > kMaxGrid) return KVFIX_ERR_ARG;
    if (rope->style == KVFIX_ROPE_HALF)
      draft_logits_kernel<kStyleHalf><<<dim3((unsigned)grid), dim3(kDraftBlock), 0, st>>>(P);
    else
      draft_logits_kernel<kStyleInter><<<dim3((unsigned)grid), dim3(kDraftBlock), 0, st>>>(P);
    KVFIX_TRY(launch_status());
    draft_norm_kernel<<<dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st>>>(
        stats, (int)rows, n_chunks, norm);
    KVFIX_TRY(launch_status());
  }
  const int64_t qps = (int64_t)Lf * n_q_heads * n_draft;
  const int64_t mgrid = (int64_t)S * ((n + kMassKeys - 1) / kMassKeys);
  if (mgrid > kMaxGrid || qps > 0x7fffffff) return KVFIX_ERR_ARG;
  draft_mass_kernel<<<dim3((unsigned)mgrid), dim3(256), 0, st>>>(logits, norm, (int)qps, n,
                                                                  scores);
  return launch_status();
}
