// Anchor-blended low-rank correction and the reliability gate.
//
// [KVCMAS eq. 7-8: each anchor of a placeholder slot stores rank-r factors
//  A B of its base cache and of its delta correction; the correction is the
//  weighted sum of the anchors' deltas.  App. A.3 "Reliability Gate" eq. 9-11,
//  "Correction Weighting and Positional Alignment" and "Variable Segment
//  Lengths".]
//
// Two passes over the source segment:
//   match  reconstructs every eligible anchor's base rows A_v B_v with bf16
//          MFMA and, per (layer, plane, token), takes the mean absolute
//          distance to the source row over all heads (keys first turned to
//          canonical positions) and the softmax over anchors (T = 1): the
//          token-wise weights.  On the value plane the same pass accumulates
//          the squared distances over the gate prefix.  A finish kernel forms
//          the weights from the head sums and pre-adds the gate partials; a
//          one-block gate kernel turns those into the gate distances, the
//          normalized entropy and the decision.
//   apply  reconstructs the delta rows A_v B_v with MFMA (each anchor's
//          operands staged in LDS three anchors ahead), blends them with the
//          token weights in fp32 and adds them to the re-aligned source:
//          keys R(p_t - p_s) x + R(p_t) delta, values x + delta; rows past
//          the covered prefix are only re-aligned.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, K = 32 = the rank).  The output
// tile is 16 features x 16 tokens: operand A holds 16 rows of the transposed
// right factor (feature x rank), operand B the left-factor rows of 16 tokens.
// Output row m of feature tile c (c = 0..7 over one 128-dim head) is mapped to
// dim 64 (c / 4) + 16 (m / 4) + 4 (c % 4) + m % 4, so that output lane group
// g (lanes 16g..16g+15, rows 4g..4g+3) ends up holding dims [16g, 16g+16) and
// [64+16g, 64+16g+16) of its token: two 32-byte pieces of the source row, and
// both members of every rotary pair in either pairing.
#include <algorithm>
#include <initializer_list>

#include "common.h"
#include "host_util.h"

namespace kvfix {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAnchorMax = KVFIX_ANCHOR_MAX;
constexpr int kRank = KVFIX_ANCHOR_RANK;
constexpr int kHD = 128;
constexpr int kTiles = 8;                       // 16-dim MFMA tiles per head
constexpr int kMatchWaves = 4, kMatchBands = 2;
constexpr int kMatchTokens = kMatchWaves * kMatchBands * 16;    // 128
constexpr int kApplyWaves = 4, kApplyBands = 4;
constexpr int kApplyThreads = kApplyWaves * 64;
constexpr int kApplyTokens = kApplyWaves * kApplyBands * 16;    // 256
constexpr int kSlice = kTiles * 16 * kRank;   // one head's right factor, bf16 elements (8 KiB)
constexpr int kXcds = 8;
constexpr int64_t kMaxOffset = int64_t(1) << 23;   // rotary angles stay accurate below this

__device__ __forceinline__ int tile_dim(int c, int m) {
  return (c >> 2) * 64 + (m >> 2) * 16 + (c & 3) * 4 + (m & 3);
}

// Factor slabs of one pool: A [V][L][2][n_max][r], Bt [V][L][2][D][r].
struct Pool {
  const bf16_t* a;
  const bf16_t* bt;
  int64_t n_max;
  int32_t L, D;
  int32_t len[kAnchorMax];
};

__device__ __forceinline__ const bf16_t* a_row(const Pool& G, int v, int l, int p, int j) {
  return G.a + ((((int64_t)v * G.L + l) * 2 + p) * G.n_max + j) * kRank;
}
__device__ __forceinline__ const bf16_t* bt_row(const Pool& G, int v, int l, int p, int f) {
  return G.bt + ((((int64_t)v * G.L + l) * 2 + p) * G.D + f) * kRank;
}

// Factor rows are re-read by many blocks: ordinary (cached) loads.
// LDS position (bf16 elements) of 16-byte chunk q (rank coefficients 8q..8q+7)
// of MFMA row m of feature tile c in a staged right-factor slice.  A wave's
// operand read for one tile (lanes: q = lane group, m = lane in group) then
// covers one contiguous KiB, and the XOR spreads the staging writes (four
// chunks of one row, several rows) over the banks.
__device__ __forceinline__ int slice_chunk(int c, int q, int m) {
  return ((c * 4 + q) * 16 + (m ^ (q << 2))) * 8;
}

// Layer-plane pairs on XCDs: XCD x takes layers x, x + 8, ..., each with its
// key plane then its value plane, so every XCD holds both planes' work (the
// key plane's rotations and the value plane's squares cost differently) and
// one pair's blocks share that XCD's L2.  Local slot q of XCD x is layer
// (q / 2) * 8 + x, plane q % 2.
__host__ __device__ __forceinline__ int xcd_pair(int q, int xcd) {
  return 2 * ((q >> 1) * kXcds + xcd) + (q & 1);
}
inline int64_t pair_slots(int64_t L) { return 2 * ((L + kXcds - 1) / kXcds) * kXcds; }

__device__ __forceinline__ bf16x8 ld_op(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, ld16_cached(p));
}

// Wait until at most N of this thread's vector memory operations are
// outstanding and its LDS operations are done, then meet the block.  The
// compiler may not move memory accesses across it; unlike __syncthreads it
// does not wait for every direct-to-LDS load in flight.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global-to-LDS loads of one head's right-factor slice (anchor v,
// layer l, plane p, head h) into an LDS stage in MFMA operand order: slice
// chunk k * 256 + tid holds rank chunk q of feature row tile_dim(c, m), the
// inverse of slice_chunk.  Two loads per thread of a 256-thread block.
constexpr int kSliceLoads = kSlice * 2 / (16 * 256);
__device__ __forceinline__ void stage_slice(const Pool& G, int v, int l, int p, int h, char* st,
                                            int tid, int wave) {
#pragma unroll
  for (int k = 0; k < kSliceLoads; ++k) {
    const int u = k * 256 + tid, c = u >> 6, q = (u >> 4) & 3, m = (u & 15) ^ (q << 2);
    const bf16_t* src = bt_row(G, v, l, p, h * kHD + tile_dim(c, m)) + 8 * q;
    __builtin_amdgcn_global_load_lds(src, to_lds(st + (k * 256 + wave * 64) * 16), 16, 0, 0);
  }
}

// Keeps the compiler from moving memory accesses across this point, so that
// loads are issued in the order the stage barriers count them.
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }


// The lane's 32 dims of row (l, seg, h, j) as four raw 16-byte pieces:
// dims [16g, 16g+8), [16g+8, 16g+16), [64+16g, ..+8), [64+16g+8, ..+16).
// Zeros for a row outside the segment or on a bad page.
__device__ __forceinline__ void load_lane_raw(const DPlane& S, int l, int seg, int h, int j, int n,
                                              int g, vu4* r) {
  const int64_t off = j < n ? row_offset(S, l, seg, h, j) : -1;
  if (off < 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = vu4{0u, 0u, 0u, 0u};
    return;
  }
  const bf16_t* row = reinterpret_cast<const bf16_t*>(S.data) + off;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = ld16(row + (q >> 1) * 64 + 16 * g + 8 * (q & 1));
}

// Raw pieces -> fp32: x[0..15] = dims [16g, 16g+16), x[16..31] = dims
// [64+16g, 64+16g+16).
__device__ __forceinline__ void unpack_lane(const vu4* r, float* x) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[8 * q + 2 * w] = bf16_lo(r[q][w]);
      x[8 * q + 2 * w + 1] = bf16_hi(r[q][w]);
    }
}

// The lane's 32 dims of the row at element offset off, rounded to bf16.
__device__ __forceinline__ void store_lane_at(const DPlane& O, int64_t off, int g, const float* y) {
  bf16_t* row = reinterpret_cast<bf16_t*>(O.data) + off;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      vu4 u;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        u[w] = pack_bf16x2(y[16 * part + 8 * q + 2 * w], y[16 * part + 8 * q + 2 * w + 1]);
      // an ordinary store: the four lane groups of a token write a row's
      // 64-byte lines in two instructions, which L2 merges before writing back
      *reinterpret_cast<vu4*>(row + part * 64 + 16 * g + 8 * q) = u;
    }
  }
}

// Rotate the lane's 32 dims by the table's angles (cos tc, sin ts per pair).
template <int STYLE>
__device__ __forceinline__ void rotate_lane(float* x, const float* tc, const float* ts, int g) {
  if (STYLE == kStyleHalf) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = 16 * g + e;
      const float a = x[e], b = x[16 + e], c = tc[q], s = ts[q];
      x[e] = fmaf(a, c, -(b * s));
      x[16 + e] = fmaf(b, c, a * s);
    }
  } else {
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int q = 32 * part + 8 * g + e / 2;
        const float a = x[16 * part + e], b = x[16 * part + e + 1], c = tc[q], s = ts[q];
        x[16 * part + e] = fmaf(a, c, -(b * s));
        x[16 * part + e + 1] = fmaf(b, c, a * s);
      }
    }
  }
}

// The same rotation, negated: -(rotated x), bit for bit (the sign goes on the
// table operands, and round-to-nearest-even is symmetric).
template <int STYLE>
__device__ __forceinline__ void rotate_lane_neg(float* x, const float* tc, const float* ts,
                                                int g) {
  if (STYLE == kStyleHalf) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = 16 * g + e;
      const float a = x[e], b = x[16 + e], c = tc[q], s = ts[q];
      x[e] = fmaf(a, -c, b * s);
      x[16 + e] = fmaf(b, -c, -(a * s));
    }
  } else {
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int q = 32 * part + 8 * g + e / 2;
        const float a = x[16 * part + e], b = x[16 * part + e + 1], c = tc[q], s = ts[q];
        x[16 * part + e] = fmaf(a, -c, b * s);
        x[16 * part + e + 1] = fmaf(b, -c, -(a * s));
      }
    }
  }
}

// x + (x of lane ^ 16), then + (that of lane ^ 32): the sum over a token
// column's four lane groups, in the same order in every lane.  The swaps run
// on the vector ALU (no LDS round trip); each lane adds its own value and its
// partner's, and addition commutes, so both lanes of a pair get the same bits.
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// ----------------------------------------------------------------------------
// match: token weights and gate partial sums
// ----------------------------------------------------------------------------

struct MatchParams {
  DPlane src[2];
  Pool G;
  RopeArgs rope;
  int64_t src_off;
  int32_t seg, n, H, V;
  uint32_t elig, gate_set;
  int32_t cover, k_gate;
  int32_t n_pairs, n_tiles;
  int32_t n_list[2];               // anchors computed per plane, in order,
  uint64_t list[2];                // 4 bits per anchor id
  int32_t hpb, HG;   // heads per block (1 or 2), head groups H / hpb
  float* part1;      // [L][2][V][HG][n] sums of |source - A_v B_v| over a block's heads
  double* gpart;     // [L][n_tiles][HG][V] the gate prefix's squared sums per block
};

// One block = 128 tokens (4 waves x 2 bands of 16) of one (layer, plane,
// head).  Blocks of one (layer, plane) run on one XCD with the heads of a
// token tile next to each other, so the left-factor rows of the tile are read
// from HBM once and from L2 by every head.  The head's source rows sit in
// registers as fp32 (keys rotated by -src_off to canonical positions),
// negated, and serve as the MFMA accumulator input, so the MFMA returns
// A_v B_v - x directly.  Per listed anchor: the head's right-factor slice is
// staged in LDS (two buffers, one barrier per anchor, the next anchor's slice
// and left rows loaded while the current one computes; indices clamped at
// the end so every load is unconditional); absolute values (and squares on
// the value plane) are summed per lane, added across the four lane groups of
// a token column in a fixed order, and written as the head's sums.
// Sum over the 16 lanes of a lane group, by DPP within rows of 16: lanes
// i ^ 1, i ^ 2, then the row rotated by 4 and by 8.  Lane 16 g holds its
// group's total (the order is fixed).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum_row16(float x) {
  x += dpp_f32<0xb1>(x);       // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4e>(x);       // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x124>(x);      // row_ror 4
  x += dpp_f32<0x128>(x);      // row_ror 8
  return x;
}

template <int STYLE, bool GATE, int HPB>
__device__ __forceinline__ void match_body(const MatchParams& P, int l, int hg, int tile,
                                           bf16_t* sbt, float* tc, float* ts, float* gw,
                                           float* hsum) {
  constexpr int p = GATE ? 1 : 0;
  if (STYLE != kStyleNone) rope_table<kHD, float>(P.rope, -P.src_off, tc, ts);
  __syncthreads();

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int j0 = tile * kMatchTokens, jw = j0 + wave * kMatchBands * 16;
  const int lim = GATE ? max(P.cover, P.k_gate) : P.cover;
  const int nl = P.n_list[p];
  const uint64_t list = P.list[p];
  const int V = P.V, n = P.n;
  double* gpart = P.gpart + (((int64_t)l * P.n_tiles + tile) * P.HG + hg) * V;
  if (j0 >= lim || nl == 0) {                 // block-uniform: no barrier follows
    if (GATE && tid < V) gpart[tid] = 0.0;    // no prefix rows here
    return;
  }
  auto anchor = [&](int i) { return (int)((list >> (4 * min(i, nl - 1))) & 15u); };
  // The block's heads one after the other; a token's sums over them are
  // added in head order (a non-final head parks them in LDS, written and
  // read back by the same lane) and written once per anchor.
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh) {
  const int h = hg * HPB + hh;
  const bool last_head = hh == HPB - 1;

  float nx[kMatchBands][32];
#pragma unroll
  for (int b = 0; b < kMatchBands; ++b) {
    vu4 xr[4];
    load_lane_raw(P.src[p], l, P.seg, h, jw + 16 * b + t, n, g, xr);
    if (STYLE != kStyleNone) {
      unpack_lane(xr, nx[b]);
      rotate_lane_neg<STYLE>(nx[b], tc, ts, g);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) xr[q][w] ^= 0x80008000u;     // both halves negated
      unpack_lane(xr, nx[b]);
    }
  }

  // Every per-anchor load is a uniform base (the anchor's slice, its left
  // row of the tile's first token) plus a lane offset computed here once.
  // The staged slice's LDS positions are per lane and fixed as well.
  int spos[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int u = tid + 256 * k2, f = u >> 2, q = u & 3;
    const int c = ((f >> 6) << 2) | ((f >> 2) & 3), m = (((f >> 4) & 3) << 2) | (f & 3);
    spos[k2] = slice_chunk(c, q, m);
  }
  auto stage_load = [&](int v, vu4* r) {
    const char* src = reinterpret_cast<const char*>(bt_row(P.G, v, l, p, h * kHD));
    r[0] = ld16_cached(src + 16 * tid);
    r[1] = ld16_cached(src + 16 * (tid + 256));
  };
  auto stage_store = [&](const vu4* r, bf16_t* buf) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) *reinterpret_cast<vu4*>(buf + spos[k2]) = r[k2];
  };
  // Rows are clamped to the slab's last row, so every load stays inside the
  // pool; a row an anchor does not store only feeds a sum that no later step
  // reads (tokens past its length never use that anchor).
  const int last = (int)P.G.n_max - 1;        // a listed anchor stores >= 1 row
  const int jb = min(j0, last);
  uint32_t oa[kMatchBands];
#pragma unroll
  for (int b = 0; b < kMatchBands; ++b)
    oa[b] = (uint32_t)((min(jw + 16 * b + t, last) - jb) * kRank * 2 + 16 * g);
  auto load_a = [&](int v, bf16x8* a) {
    const char* base = reinterpret_cast<const char*>(a_row(P.G, v, l, p, jb));
#pragma unroll
    for (int b = 0; b < kMatchBands; ++b) a[b] = __builtin_bit_cast(bf16x8, ld16_cached(base + oa[b]));
  };
  auto compute = [&](const bf16_t* buf, const bf16x8* a, int i) {
    const int v = anchor(i);
    bf16x8 bop[kTiles];
#pragma unroll
    for (int c = 0; c < kTiles; ++c)
      bop[c] = *reinterpret_cast<const bf16x8*>(buf + slice_chunk(c, g, t));
    float* o1 = P.part1 + ((((int64_t)l * 2 + p) * V + v) * P.HG + hg) * n;
    // Both bands' products of a tile are issued before either is summed, so
    // one band's sums cover the other band's MFMA latency.  Per band the
    // sums still run over the tiles in order.
    float s1[kMatchBands][4], s2[kMatchBands][4];
#pragma unroll
    for (int b = 0; b < kMatchBands; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) s1[b][e] = s2[b][e] = 0.0f;
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      f32x4 d[kMatchBands];
#pragma unroll
      for (int b = 0; b < kMatchBands; ++b) {
        const f32x4 cx = {nx[b][4 * c], nx[b][4 * c + 1], nx[b][4 * c + 2], nx[b][4 * c + 3]};
        d[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop[c], a[b], cx, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < kMatchBands; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s1[b][e] += fabsf(d[b][e]);
          if (GATE) s2[b][e] = fmaf(d[b][e], d[b][e], s2[b][e]);
        }
    }
    // the wave's squared sums over its prefix rows (bands in order, then
    // the 16 token columns), kept in LDS until the block adds its waves
    float q = 0.0f;
#pragma unroll
    for (int b = 0; b < kMatchBands; ++b) {
      float c1 = sum_lane_groups((s1[b][0] + s1[b][1]) + (s1[b][2] + s1[b][3]));
      const int j = jw + 16 * b + t;
      if (GATE) {
        const float c2 = sum_lane_groups((s2[b][0] + s2[b][1]) + (s2[b][2] + s2[b][3]));
        q += j < P.k_gate ? c2 : 0.0f;
      }
      float* hs = hsum + i * kMatchTokens + wave * kMatchBands * 16 + 16 * b + t;
      if (hh > 0) c1 = *hs + c1;                    // the block's earlier heads first
      if (g == 0) {
        if (!last_head) *hs = c1;
        else if (j < n) o1[j] = c1;
      }
    }
    if (GATE) {
      q = sum_row16(q);
      if (lane == 0) gw[i * kMatchWaves + wave] = hh > 0 ? gw[i * kMatchWaves + wave] + q : q;
    }
  };

  vu4 sr[2];
  bf16x8 a0[kMatchBands], a1[kMatchBands];
  stage_load(anchor(0), sr);
  load_a(anchor(0), a0);
  stage_store(sr, sbt);
  __syncthreads();
  for (int i = 0; i < nl; i += 2) {
    stage_load(anchor(i + 1), sr);
    load_a(anchor(i + 1), a1);
    compute(sbt, a0, i);
    stage_store(sr, sbt + kSlice);
    __syncthreads();
    stage_load(anchor(i + 2), sr);
    load_a(anchor(i + 2), a0);
    if (i + 1 < nl) compute(sbt + kSlice, a1, i + 1);
    stage_store(sr, sbt);
    __syncthreads();
  }
  }                                            // heads
  // (the loop's last barrier orders the waves' partials before this)
  if (GATE && tid < V) {
    double d = 0.0;                   // 0 for anchors outside the gate set
    if ((P.gate_set >> tid) & 1u)     // (all listed: the prefix is not empty)
      for (int i = 0; i < nl; ++i)
        if (anchor(i) == tid)
          for (int w = 0; w < kMatchWaves; ++w) d += (double)gw[i * kMatchWaves + w];
    gpart[tid] = d;
  }
}

template <int STYLE, int HPB>
__global__ __launch_bounds__(kMatchWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void anchor_match_kernel(MatchParams P) {
  __shared__ __attribute__((aligned(16))) bf16_t sbt[2 * kSlice];
  __shared__ float tc[kHD / 2], ts[kHD / 2];
  __shared__ float gw[kAnchorMax * kMatchWaves];
  __shared__ float hsum[kAnchorMax * kMatchTokens];
  const int id = blockIdx.x, xcd = id % kXcds, k = id / kXcds;
  const int hg = k % P.HG, k2 = k / P.HG;
  const int tile = k2 % P.n_tiles;
  const int pair = xcd_pair(k2 / P.n_tiles, xcd);
  if (pair >= P.n_pairs) return;
  const int l = pair >> 1;
  if ((pair & 1) == 0)
    match_body<STYLE, false, HPB>(P, l, hg, tile, sbt, tc, ts, gw, hsum);
  else
    match_body<kStyleNone, true, HPB>(P, l, hg, tile, sbt, tc, ts, gw, hsum);
}

// Per token: the head sums added in head order give the distance sums;
// weights = softmax over E of minus the mean absolute distance (T = 1).
constexpr int kFinishTokens = 256;

static_assert(kFinishTokens == 2 * kMatchTokens, "a finish block covers two match tiles");

struct FinishParams {
  const float* part1;
  int32_t n, H, V;
  uint32_t elig;
  int32_t cover;
  float D;                         // features per token row (all heads)
  float* w;                        // [L][2][V][n]
  const double* gpart;             // [L][n_match_tiles][H][V] from the match
  int32_t n_match_tiles, n_tiles;
  double* gsum;                    // [L][n_tiles][V]
};

// On the value plane a block also adds the gate partials of its two match
// tiles, tile by tile and head by head, into one partial per anchor.
__global__ __launch_bounds__(kFinishTokens) void anchor_finish_kernel(FinishParams P) {
  const int tile = blockIdx.x, p = blockIdx.y & 1, l = blockIdx.y >> 1;
  const int j = tile * kFinishTokens + threadIdx.x;
  const int V = P.V, H = P.H, n = P.n;
  if (p == 1 && (int)threadIdx.x < V) {
    double d = 0.0;
    for (int tt = 2 * tile; tt < min(2 * tile + 2, P.n_match_tiles); ++tt)
      for (int hh = 0; hh < H; ++hh)
        d += P.gpart[(((int64_t)l * P.n_match_tiles + tt) * H + hh) * V + threadIdx.x];
    P.gsum[((int64_t)l * P.n_tiles + tile) * V + threadIdx.x] = d;
  }
  if (j >= n) return;
  float* wr = P.w + ((int64_t)l * 2 + p) * V * n + j;
  if (j >= P.cover) {
    for (int v = 0; v < V; ++v) wr[(int64_t)v * n] = 0.0f;
    return;
  }
  // Sums over heads, head by head (fixed order); the anchors' loads of one
  // head are independent and issued together.
  const float* base = P.part1 + ((int64_t)l * 2 + p) * V * H * n;
  float s[kAnchorMax];
#pragma unroll
  for (int v = 0; v < kAnchorMax; ++v) s[v] = 0.0f;
  for (int hh = 0; hh < H; ++hh) {
    float x[kAnchorMax];
#pragma unroll
    for (int v = 0; v < kAnchorMax; ++v)
      x[v] = (v < V && ((P.elig >> v) & 1u)) ? base[((int64_t)v * H + hh) * n + j] : 0.0f;
#pragma unroll
    for (int v = 0; v < kAnchorMax; ++v) s[v] += x[v];
  }
  float m = INFINITY;
#pragma unroll
  for (int v = 0; v < kAnchorMax; ++v)
    if (v < V && ((P.elig >> v) & 1u)) m = fminf(m, s[v] / P.D);
  float sum = 0.0f;
#pragma unroll
  for (int v = 0; v < kAnchorMax; ++v)
    if (v < V && ((P.elig >> v) & 1u)) sum += expf(m - s[v] / P.D);
#pragma unroll
  for (int v = 0; v < kAnchorMax; ++v)
    if (v < V) wr[(int64_t)v * n] = ((P.elig >> v) & 1u) ? expf(m - s[v] / P.D) / sum : 0.0f;
}

// Gate finish: d_v = sqrt of the summed partials (fp64, fixed order), then
// g = softmax(-d), Hbar = -sum g log2 g / log2 |A_k| clamped to [0, 1], and
// the decision Hbar <= tau with at least two compared anchors.
__global__ __launch_bounds__(1024) void anchor_gate_kernel(const double* part, int n_parts, int V,
                                                           uint32_t gate_set, double tau,
                                                           double* gate, int32_t* accept) {
  __shared__ double sd[kAnchorMax];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < V) {
    double s = 0.0;
    int i = lane;
    for (; i + 7 * 64 < n_parts; i += 8 * 64) {   // eight loads in flight, added in order
      double x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = part[(int64_t)(i + 64 * e) * V + wave];
#pragma unroll
      for (int e = 0; e < 8; ++e) s += x[e];
    }
    for (; i < n_parts; i += 64) s += part[(int64_t)i * V + wave];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sd[wave] = ((gate_set >> wave) & 1u) ? sqrt(s) : __builtin_nan("");
  }
  __syncthreads();
  if (wave != 0) return;
  // the exponentials and logarithms one anchor per lane; the sums in anchor
  // order by lane 0
  __shared__ double se[kAnchorMax], sl[kAnchorMax];
  int na = 0;
  double dmin = INFINITY;
  for (int v = 0; v < V; ++v) {
    if ((gate_set >> v) & 1u) {
      ++na;
      dmin = fmin(dmin, sd[v]);
    }
  }
  if (lane < V) gate[lane] = sd[lane];
  if (na < 2) {
    if (lane == 0) {
      gate[V] = __builtin_nan("");
      *accept = 0;
    }
    return;
  }
  const bool in = lane < V && ((gate_set >> lane) & 1u);
  const double ev = in ? exp(dmin - sd[lane]) : 0.0;
  if (lane < V) se[lane] = ev;
  __builtin_amdgcn_wave_barrier();
  double sum = 0.0;
  for (int v = 0; v < V; ++v)
    if ((gate_set >> v) & 1u) sum += se[v];
  if (lane < V) {
    const double gv = ev / sum;
    sl[lane] = in && gv > 0.0 ? gv * log2(gv) : 0.0;
  }
  __builtin_amdgcn_wave_barrier();
  if (lane != 0) return;
  double hsum = 0.0;
  for (int v = 0; v < V; ++v) {
    if (!((gate_set >> v) & 1u)) continue;
    const double gv = se[v] / sum;
    if (gv > 0.0) hsum += sl[v];
  }
  double hbar = -hsum / log2((double)na);
  hbar = fmin(1.0, fmax(0.0, hbar));
  gate[V] = hbar;
  *accept = hbar <= tau ? 1 : 0;
}

// ----------------------------------------------------------------------------
// apply: blended deltas added to the re-aligned source
// ----------------------------------------------------------------------------

struct AnchorApplyParams {
  DPlane src[2], out[2];
  Pool G;
  RopeArgs rope;
  int64_t src_off, tgt_off;
  int32_t seg, n, H, V;
  uint32_t elig;
  int32_t cover;
  int32_t n_pairs, n_tiles;
  int32_t n_list;                  // the eligible anchors, in order,
  uint64_t list;                   // 4 bits per anchor id
  const float* w;    // [L][2][V][n]
};

// One anchor's operands for an apply block, staged in LDS: the head's
// right-factor slice in MFMA operand order, the left rows of the block's
// tokens and their weights.
constexpr int kStageBt = kSlice * 2;                    // 8 KiB
constexpr int kStageA = kApplyTokens * kRank * 2;       // 16 KiB
constexpr int kStageW = kApplyThreads * 4;              // 1 KiB
constexpr int kStageBytes = kStageBt + kStageA + kStageW;
constexpr int kApplyStages = 3;
constexpr int kApplyPages = kApplyTokens + 1;           // page ids a tile can span
// Direct global-to-LDS loads per thread and anchor (slice chunks, row
// chunks, one weight): the in-order count that the pipeline waits on.
constexpr int kALoads = kStageA / (16 * kApplyThreads);
constexpr int kStageLoads = kSliceLoads + kALoads + 1;
static_assert(kApplyThreads == 256 && kALoads * 16 * kApplyThreads == kStageA, "stage loads");

template <int STYLE, bool PAGED>
__device__ __forceinline__ void apply_body(const AnchorApplyParams& P, int l, int p, int h,
                                           int tile, char* stages, float* tab, int32_t* pages) {
  float *tc1 = tab, *ts1 = tab + 64, *tc2 = tab + 128, *ts2 = tab + 192;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = tile * kApplyTokens, jw = j0 + wave * kApplyBands * 16;
  f32x4 acc[kApplyBands][kTiles];
#pragma unroll
  for (int b = 0; b < kApplyBands; ++b)
#pragma unroll
    for (int c = 0; c < kTiles; ++c) acc[b][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // The eligible anchors in order, three stages deep: anchor i + 2's
  // operands are loaded into LDS while anchor i computes, one barrier per
  // anchor.  Token indices are clamped to the covered prefix, so every load
  // is in bounds; rows past the prefix get weight 0.
  const int nl = P.n_list;
  const bool run = j0 < P.cover && nl > 0;
  const int last = P.cover - 1;
  const float* wl = P.w + ((int64_t)l * 2 + p) * P.V * P.n;
  // Each lane's byte offsets from an anchor's slice, the tile's first left
  // row and first weight, the same for every anchor (and small: inside one
  // head's slice or one tile): a staging load is then the anchor's uniform
  // base plus a 32-bit lane offset.  Slice chunk k * 256 + tid holds rank
  // chunk q of feature row tile_dim(c, m) (the inverse of slice_chunk); left
  // rows go token-major, 4 chunks per token; every thread loads one weight,
  // so that every wave counts the same loads (threads past the tile's tokens
  // repeat the last ones).
  uint32_t ob[kSliceLoads], oa[kALoads];
#pragma unroll
  for (int k = 0; k < kSliceLoads; ++k) {
    const int u = k * 256 + tid, c = u >> 6, q = (u >> 4) & 3, m = (u & 15) ^ (q << 2);
    ob[k] = (uint32_t)(((h * kHD + tile_dim(c, m)) * kRank + 8 * q) * 2);
  }
#pragma unroll
  for (int k = 0; k < kALoads; ++k) {
    const int u = k * kApplyThreads + tid;
    oa[k] = (uint32_t)(((min(j0 + (u >> 2), last) - j0) * kRank + 8 * (u & 3)) * 2);
  }
  const uint32_t ow = (uint32_t)((min(j0 + tid % kApplyTokens, last) - j0) * 4);
  auto issue = [&](int i) {
    const int v = (int)((P.list >> (4 * i)) & 15u);
    char* st = stages + (i % kApplyStages) * kStageBytes;
    const char* bt = reinterpret_cast<const char*>(bt_row(P.G, v, l, p, 0));
    const char* ar = reinterpret_cast<const char*>(a_row(P.G, v, l, p, j0));
    const char* wr = reinterpret_cast<const char*>(wl + (int64_t)v * P.n + j0);
#pragma unroll
    for (int k = 0; k < kSliceLoads; ++k)
      __builtin_amdgcn_global_load_lds(bt + ob[k], to_lds(st + (k * 256 + wave * 64) * 16), 16, 0, 0);
#pragma unroll
    for (int k = 0; k < kALoads; ++k)
      __builtin_amdgcn_global_load_lds(
          ar + oa[k], to_lds(st + kStageBt + (k * kApplyThreads + wave * 64) * 16), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(wr + ow, to_lds(st + kStageBt + kStageA + wave * 64 * 4), 4,
                                     0, 0);
  };
  // Row addresses.  A paged plane's page ids for the tile are staged in LDS
  // before the first anchor (covered by its barrier), so no row address
  // waits on a global load once stores are in flight.
  const DPlane& S = P.src[p];
  const DPlane& O = P.out[p];
  int first_s = 0, first_o = 0;
  if (PAGED) {
    const int j1 = min(j0 + kApplyTokens, P.n);
    first_s = stage_pages(S, P.seg, j0, j1, pages);
    first_o = stage_pages(O, P.seg, j0, j1, pages + kApplyPages);
  }
  auto src_off = [&](int b) -> int64_t {
    const int j = min(jw + 16 * b + t, P.n - 1);
    if (PAGED) return row_offset_staged(S, l, P.seg, h, j, pages, first_s);
    return (int64_t)l * S.s_layer + (int64_t)P.seg * S.s_seg + (int64_t)h * S.s_head +
           (int64_t)j * S.s_token;
  };
  auto out_off = [&](int b) -> int64_t {
    const int j = jw + 16 * b + t;
    if (j >= P.n) return -1;
    if (PAGED) return row_offset_staged(O, l, P.seg, h, j, pages + kApplyPages, first_o);
    return (int64_t)l * O.s_layer + (int64_t)P.seg * O.s_seg + (int64_t)h * O.s_head +
           (int64_t)j * O.s_token;
  };
  auto load_band = [&](int b, vu4* r) {
    const bf16_t* row = reinterpret_cast<const bf16_t*>(S.data) + max(src_off(b), int64_t(0));
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = ld16(row + (q >> 1) * 64 + 16 * g + 8 * (q & 1));
  };
  // Source rows of two bands in flight; the first two bands are loaded at
  // the top of the last anchor, behind its products.
  vu4 xr[2][4];
  if (run) {
    issue(0);
    if (nl > 1) issue(1);
  }
  if (STYLE != kStyleNone) {
    rope_table<kHD, float>(P.rope, P.tgt_off - P.src_off, tc1, ts1);
    rope_table<kHD, float>(P.rope, P.tgt_off, tc2, ts2);
  }
  if (run) {
    for (int i = 0; i < nl; ++i) {
      if (i + 1 < nl)
        stage_barrier<kStageLoads>();
      else
        stage_barrier<0>();
      if (i + 2 < nl) issue(i + 2);
      if (i + 1 == nl) {
        load_band(0, xr[0]);
        load_band(1, xr[1]);
      }
      const char* st = stages + (i % kApplyStages) * kStageBytes;
      const bf16_t* sb = reinterpret_cast<const bf16_t*>(st);
      const bf16_t* sa = reinterpret_cast<const bf16_t*>(st + kStageBt);
      const float* sw = reinterpret_cast<const float*>(st + kStageBt + kStageA);
      bf16x8 aop[kApplyBands];
      float wv[kApplyBands];
#pragma unroll
      for (int b = 0; b < kApplyBands; ++b) {
        const int r = wave * kApplyBands * 16 + 16 * b + t;
        aop[b] = *reinterpret_cast<const bf16x8*>(sa + r * kRank + 8 * g);
        wv[b] = jw + 16 * b + t < P.cover ? sw[r] : 0.0f;
      }
      // Tile-major: each right-factor tile is read once and serves the four
      // bands.  Product k + 1 is issued before product k is weighted into
      // its accumulator (two temporaries), so the matrix unit and the vector
      // unit overlap instead of each vector step waiting out a product.
      bf16x8 bop = *reinterpret_cast<const bf16x8*>(sb + slice_chunk(0, g, t));
      f32x4 d[2];
      d[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop, aop[0], f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                     0, 0, 0);
#pragma unroll
      for (int k = 0; k < kTiles * kApplyBands; ++k) {
        const int c = k / kApplyBands, b = k % kApplyBands;
        if (k + 1 < kTiles * kApplyBands) {
          const int c1 = (k + 1) / kApplyBands, b1 = (k + 1) % kApplyBands;
          if (b1 == 0) bop = *reinterpret_cast<const bf16x8*>(sb + slice_chunk(c1, g, t));
          d[(k + 1) & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              bop, aop[b1], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[b][c][e] = fmaf(wv[b], d[k & 1][e], acc[b][c][e]);
      }
    }
    // Nothing is in flight here (the last anchor waited for everything);
    // saying so lets the epilogue's waits count its own loads exactly.
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
  } else {
    __syncthreads();
  }

  // Epilogue.  The source loads are unconditional (a row past the end reads
  // the last row; in a paged plane a row on a bad page reads element 0 and is
  // zeroed) and one band ahead, and only the store depends on the row, so no
  // band's loads wait for an earlier band's stores (loads and stores share
  // one in-order counter).
  if (!run) load_band(0, xr[0]);
#pragma unroll
  for (int b = 0; b < kApplyBands; ++b) {
    if (b + 1 < kApplyBands && !(run && b == 0)) load_band(b + 1, xr[(b + 1) & 1]);
    const bool valid = !PAGED || src_off(b) >= 0;
    float x[32], dl[32];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = valid ? xr[b & 1][q][w] : 0u;
        x[8 * q + 2 * w] = bf16_lo(u);
        x[8 * q + 2 * w + 1] = bf16_hi(u);
      }
#pragma unroll
    for (int c = 0; c < kTiles; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) dl[4 * c + e] = acc[b][c][e];
    if (STYLE != kStyleNone) {
      rotate_lane<STYLE>(x, tc1, ts1, g);
      rotate_lane<STYLE>(dl, tc2, ts2, g);
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] += dl[e];
    const int64_t oq = out_off(b);
    if (oq >= 0) store_lane_at(O, oq, g, x);
  }
}

// Blocks of one (layer, plane) run on one XCD and walk its heads fastest, so
// the delta left factors and weights of a token tile are read from HBM once
// and reused from L2 by every head.
template <int STYLE, bool PAGED>
__global__ __launch_bounds__(kApplyWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void anchor_apply_kernel(AnchorApplyParams P) {
  __shared__ __attribute__((aligned(16))) char stages[kApplyStages * kStageBytes];
  __shared__ float tab[4 * (kHD / 2)];
  __shared__ int32_t pages[PAGED ? 2 * kApplyPages : 1];
  const int id = blockIdx.x, xcd = id % kXcds, k = id / kXcds;
  const int h = k % P.H, k2 = k / P.H;
  const int tile = k2 % P.n_tiles;
  const int pair = xcd_pair(k2 / P.n_tiles, xcd);
  if (pair >= P.n_pairs) return;
  const int l = pair >> 1;
  if ((pair & 1) == 0)
    apply_body<STYLE, PAGED>(P, l, 0, h, tile, stages, tab, pages);
  else
    apply_body<kStyleNone, PAGED>(P, l, 1, h, tile, stages, tab, pages);
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

struct Eligible {
  uint32_t elig = 0, gate_set = 0;
  int32_t cover = 0, k_gate = 0;
};

// E and the covered prefix [KVCMAS App. A.3 "Variable Segment Lengths"]: the
// anchors storing the whole segment, else those storing the longest prefix;
// the gate set A_k: anchors storing at least k tokens (k clamped to [0, n]).
Eligible eligible(const kvfix_anchor_pool* pool, int32_t n, int64_t k_gate) {
  Eligible e;
  int32_t longest = 0;
  for (int v = 0; v < pool->n_anchors; ++v) longest = std::max(longest, pool->lengths[v]);
  for (int v = 0; v < pool->n_anchors; ++v)
    if (pool->lengths[v] >= n) e.elig |= 1u << v;
  if (e.elig) {
    e.cover = n;
  } else if (longest > 0) {
    e.cover = longest;
    for (int v = 0; v < pool->n_anchors; ++v)
      if (pool->lengths[v] == longest) e.elig |= 1u << v;
  }
  e.k_gate = (int32_t)std::min<int64_t>(std::max<int64_t>(k_gate, 0), n);
  for (int v = 0; v < pool->n_anchors; ++v)
    if (pool->lengths[v] >= e.k_gate) e.gate_set |= 1u << v;
  return e;
}

kvfix_status check_pool(const kvfix_anchor_pool* pool) {
  if (pool == nullptr) return KVFIX_ERR_ARG;
  if (pool->n_anchors < 0 || pool->n_anchors > kAnchorMax || pool->n_max < 0) return KVFIX_ERR_ARG;
  if (pool->rank != kRank) return KVFIX_ERR_UNSUPPORTED;
  if (pool->n_anchors == 0) return KVFIX_OK;
  if (pool->lengths == nullptr || pool->a == nullptr || pool->bt == nullptr) return KVFIX_ERR_ARG;
  if (!aligned16(pool->a) || !aligned16(pool->bt)) return KVFIX_ERR_ALIGN;
  for (int v = 0; v < pool->n_anchors; ++v)
    if (pool->lengths[v] < 0 || pool->lengths[v] > pool->n_max) return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

kvfix_status check_anchor_planes(const kvfix_plane* k, const kvfix_plane* v, int32_t seg) {
  KVFIX_TRY(check_plane(k));
  KVFIX_TRY(check_plane(v));
  KVFIX_TRY(same_rows(k, v));
  if (k->n_layers != v->n_layers) return KVFIX_ERR_ARG;
  if (k->dtype != KVFIX_BF16 || k->head_dim != kHD) return KVFIX_ERR_UNSUPPORTED;
  if (seg < 0 || seg >= k->n_segs) return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

kvfix_status check_rotary(double theta, int32_t style, std::initializer_list<int64_t> offsets) {
  if (style != KVFIX_ROPE_HALF && style != KVFIX_ROPE_INTERLEAVED) return KVFIX_ERR_ARG;
  if (!(theta > 0.0) || !isfinite(theta)) return KVFIX_ERR_ARG;
  for (int64_t o : offsets)
    if (o > kMaxOffset || o < -kMaxOffset) return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

Pool make_pool(const kvfix_anchor_pool* pool, int32_t L, int32_t D) {
  Pool G;
  memset(&G, 0, sizeof(G));
  G.a = static_cast<const bf16_t*>(pool->a);
  G.bt = static_cast<const bf16_t*>(pool->bt);
  G.n_max = pool->n_max;
  G.L = L;
  G.D = D;
  for (int v = 0; v < pool->n_anchors; ++v) G.len[v] = pool->lengths[v];
  return G;
}

RopeArgs rope_freqs(double theta, int32_t style) {
  kvfix_rope r;
  r.theta = theta;
  r.style = style;
  r.delta = nullptr;
  return make_rope_args(&r, kHD);
}

// Workspace: the distance sums of both planes per block's heads, the gate's
// partial sums per match block (layer, 128-token tile, head group, anchor)
// and per finish block (layer, 256-token tile, anchor).
struct MatchWs {
  size_t part1, gpart, gsum, total;
};

// Heads per match block: two when the head count is even.
int match_hpb(int64_t H) { return H % 2 == 0 ? 2 : 1; }

MatchWs match_ws(int64_t L, int64_t H, int64_t n, int64_t V) {
  MatchWs w;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const int64_t HG = H > 0 ? H / match_hpb(H) : 0;
  w.part1 = up((size_t)(L * 2 * V * HG * n) * sizeof(float));
  w.gpart = up((size_t)(L * ((n + kMatchTokens - 1) / kMatchTokens) * HG * V) * sizeof(double));
  w.gsum = up((size_t)(L * ((n + kFinishTokens - 1) / kFinishTokens) * V) * sizeof(double));
  w.total = w.part1 + w.gpart + w.gsum + 256;
  return w;
}

}  // namespace
}  // namespace kvfix

using namespace kvfix;

extern "C" size_t kvfix_anchor_match_workspace(int32_t n_layers, int32_t n_heads,
                                               int32_t n_tokens, int32_t n_anchors) {
  if (n_layers < 0 || n_heads < 0 || n_tokens < 0 || n_anchors < 0) return 0;
  return match_ws(n_layers, n_heads, n_tokens, n_anchors).total;
}

extern "C" kvfix_status kvfix_anchor_match(const kvfix_plane* src_k, const kvfix_plane* src_v,
                                           int32_t seg, const kvfix_anchor_pool* base,
                                           int64_t src_off, double theta, int32_t rope_style,
                                           int64_t k_gate, double tau, float* weights,
                                           double* gate, int32_t* accept, void* ws,
                                           size_t ws_bytes, void* stream) {
  KVFIX_TRY(check_anchor_planes(src_k, src_v, seg));
  KVFIX_TRY(check_pool(base));
  KVFIX_TRY(check_rotary(theta, rope_style, {src_off}));
  if (gate == nullptr || accept == nullptr || ws == nullptr) return KVFIX_ERR_ARG;
  if (!(tau == tau)) return KVFIX_ERR_ARG;
  const int32_t L = src_k->n_layers, n = src_k->n_tokens, V = base->n_anchors;
  const int32_t H = src_k->n_heads;
  if (V > 0 && n > 0 && L > 0 && weights == nullptr) return KVFIX_ERR_ARG;
  const MatchWs W = match_ws(L, H, n, V);
  if (ws_bytes < W.total) return KVFIX_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return KVFIX_ERR_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  const Eligible e = eligible(base, n, k_gate);
  char* wsb = static_cast<char*>(ws);
  double* gpart = reinterpret_cast<double*>(wsb + W.part1);
  double* gsum = reinterpret_cast<double*>(wsb + W.part1 + W.gpart);
  const int32_t n_tiles = (int32_t)ceil_div(n, kMatchTokens);
  const int32_t n_fin = (int32_t)ceil_div(n, kFinishTokens);

  if (V > 0 && n > 0 && L > 0 && H > 0) {
    MatchParams P;
    memset(&P, 0, sizeof(P));
    P.src[0] = make_dplane(*src_k);
    P.src[1] = make_dplane(*src_v);
    P.G = make_pool(base, L, H * kHD);
    P.rope = rope_freqs(theta, rope_style);
    P.src_off = src_off;
    P.seg = seg;
    P.n = n;
    P.H = H;
    P.hpb = match_hpb(H);
    P.HG = H / P.hpb;
    P.V = V;
    P.elig = e.elig;
    P.gate_set = e.gate_set;
    P.cover = e.cover;
    P.k_gate = e.k_gate;
    P.n_pairs = 2 * L;
    P.n_tiles = n_tiles;
    for (int v = 0; v < V; ++v) {
      const bool in_e = (e.elig >> v) & 1u;
      const bool in_gate = e.k_gate > 0 && ((e.gate_set >> v) & 1u);
      if (in_e) P.list[0] |= (uint64_t)v << (4 * P.n_list[0]++);
      if (in_e || in_gate) P.list[1] |= (uint64_t)v << (4 * P.n_list[1]++);
    }
    P.part1 = reinterpret_cast<float*>(wsb);
    P.gpart = gpart;
    const int64_t grid = (int64_t)P.HG * P.n_tiles * pair_slots(L);
    if (grid > kMaxGrid) return KVFIX_ERR_ARG;
    const dim3 gd((unsigned)grid), bd(kMatchWaves * 64);
    if (rope_style == KVFIX_ROPE_HALF) {
      if (P.hpb == 2) anchor_match_kernel<kStyleHalf, 2><<<gd, bd, 0, st>>>(P);
      else anchor_match_kernel<kStyleHalf, 1><<<gd, bd, 0, st>>>(P);
    } else {
      if (P.hpb == 2) anchor_match_kernel<kStyleInter, 2><<<gd, bd, 0, st>>>(P);
      else anchor_match_kernel<kStyleInter, 1><<<gd, bd, 0, st>>>(P);
    }
    KVFIX_TRY(launch_status());

    FinishParams F;
    F.part1 = P.part1;
    F.n = n;
    F.H = P.HG;                     // the head sums come per head group
    F.V = V;
    F.elig = e.elig;
    F.cover = e.cover;
    F.D = (float)(H * kHD);
    F.w = weights;
    F.gpart = gpart;
    F.n_match_tiles = n_tiles;
    F.n_tiles = n_fin;
    F.gsum = gsum;
    anchor_finish_kernel<<<dim3((unsigned)n_fin, (unsigned)(2 * L)), dim3(kFinishTokens), 0,
                           st>>>(F);
    KVFIX_TRY(launch_status());
  }
  const int n_parts = (V > 0 && n > 0 && H > 0) ? L * n_fin : 0;
  anchor_gate_kernel<<<dim3(1), dim3(1024), 0, st>>>(gsum, n_parts, V, e.gate_set, tau, gate,
                                                      accept);
  return launch_status();
}

extern "C" kvfix_status kvfix_anchor_apply(const kvfix_plane* src_k, const kvfix_plane* src_v,
                                           int32_t seg, const kvfix_anchor_pool* delta,
                                           const float* weights, int64_t src_off,
                                           int64_t tgt_off, double theta, int32_t rope_style,
                                           const kvfix_plane* out_k, const kvfix_plane* out_v,
                                           void* stream) {
  KVFIX_TRY(check_anchor_planes(src_k, src_v, seg));
  KVFIX_TRY(check_anchor_planes(out_k, out_v, seg));
  KVFIX_TRY(same_rows(src_k, out_k));
  if (src_k->n_layers != out_k->n_layers) return KVFIX_ERR_ARG;
  KVFIX_TRY(check_pool(delta));
  KVFIX_TRY(check_rotary(theta, rope_style, {src_off, tgt_off, tgt_off - src_off}));
  const int32_t L = src_k->n_layers, n = src_k->n_tokens, V = delta->n_anchors;
  const Eligible e = eligible(delta, n, 0);
  if (e.elig != 0 && weights == nullptr) return KVFIX_ERR_ARG;
  if (L == 0 || n == 0 || src_k->n_heads == 0) return KVFIX_OK;

  AnchorApplyParams P;
  memset(&P, 0, sizeof(P));
  P.src[0] = make_dplane(*src_k);
  P.src[1] = make_dplane(*src_v);
  P.out[0] = make_dplane(*out_k);
  P.out[1] = make_dplane(*out_v);
  P.G = make_pool(delta, L, src_k->n_heads * kHD);
  P.rope = rope_freqs(theta, rope_style);
  P.src_off = src_off;
  P.tgt_off = tgt_off;
  P.seg = seg;
  P.n = n;
  P.H = src_k->n_heads;
  P.V = V;
  P.elig = e.elig;
  P.cover = e.cover;
  P.n_pairs = 2 * L;
  P.n_tiles = (int32_t)ceil_div(n, kApplyTokens);
  for (int v = 0; v < V; ++v)
    if ((e.elig >> v) & 1u) P.list |= (uint64_t)v << (4 * P.n_list++);
  P.w = weights;
  const int64_t grid = (int64_t)P.H * P.n_tiles * pair_slots(L);
  if (grid > kMaxGrid) return KVFIX_ERR_ARG;
  const hipStream_t st = (hipStream_t)stream;
  const dim3 gd((unsigned)grid), bd(kApplyWaves * 64);
  const bool paged = P.src[0].page_table || P.src[1].page_table || P.out[0].page_table ||
                     P.out[1].page_table;
  if (rope_style == KVFIX_ROPE_HALF) {
    if (paged)
      anchor_apply_kernel<kStyleHalf, true><<<gd, bd, 0, st>>>(P);
    else
      anchor_apply_kernel<kStyleHalf, false><<<gd, bd, 0, st>>>(P);
  } else {
    if (paged)
      anchor_apply_kernel<kStyleInter, true><<<gd, bd, 0, st>>>(P);
    else
      anchor_apply_kernel<kStyleInter, false><<<gd, bd, 0, st>>>(P);
  }
  return launch_status();
}
