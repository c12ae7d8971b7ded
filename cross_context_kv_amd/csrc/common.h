// Shared device helpers for the kvfix HIP kernels (gfx950, wave64).
//
// Lane-to-row map.  A row is head_dim contiguous elements of one (layer,
// segment, head, token).  G = HD / (2 V) lanes serve one row, V being the
// elements in 16 bytes (8 bf16 or 4 fp32).  Each lane moves two 16-byte parts
// of its row and owns V rotary pairs entirely, so a rotation never needs a
// cross-lane exchange:
//   rotate-half : part 0 = dims [gV, gV+V), part 1 = dims [HD/2+gV, HD/2+gV+V);
//                 pair m = (part0[m], part1[m])
//   interleaved : parts 0,1 = dims [2gV, 2gV+2V); pair m = (dim 2gV+2m, 2gV+2m+1)
// In both cases pair m of lane g has frequency index gV + m.
// A wave covers RPW = 64 / G rows per step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvfix.h"

namespace kvfix {

constexpr int kWave = 64;
constexpr int kStyleNone = -1;   // value plane: no rotation
constexpr int kStyleHalf = KVFIX_ROPE_HALF;
constexpr int kStyleInter = KVFIX_ROPE_INTERLEAVED;
constexpr int kMaxHeadDim = 256;

typedef uint16_t bf16_t;          // bfloat16 storage (bit pattern)
typedef uint32_t vu4 __attribute__((ext_vector_type(4)));   // one 16-byte vector

// Immediate of s_waitcnt: at most vm vector memory operations (6 bits, split
// over bits 3:0 and 15:14) and lgkm LDS / scalar operations (4 bits) left in
// flight; export count not waited on.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// An LDS address as a wave-uniform 32-bit offset, the form a direct
// global-to-LDS load takes.
typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ __forceinline__ lds_ptr to_lds(void* p) {
  return (lds_ptr)(uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)p);
}

// Device view of a plane (element strides; byte base pointer).
struct DPlane {
  char* data;
  int64_t s_layer, s_seg, s_head, s_token, s_page;
  const int32_t* page_table;
  int32_t page_size, pages_per_seg;
  int64_t n_pool_pages;
};

inline DPlane make_dplane(const kvfix_plane& p) {
  DPlane d;
  d.data = static_cast<char*>(p.data);
  d.s_layer = p.s_layer; d.s_seg = p.s_seg; d.s_head = p.s_head; d.s_token = p.s_token;
  d.s_page = p.s_page; d.page_table = p.page_table; d.page_size = p.page_size;
  d.pages_per_seg = p.pages_per_seg; d.n_pool_pages = p.n_pool_pages;
  return d;
}

// Element offset of row (l, s, h, j), or -1 if its page id is out of range.
__device__ __forceinline__ int64_t row_offset(const DPlane& p, int l, int s, int h, int j) {
  if (p.page_table == nullptr)
    return (int64_t)l * p.s_layer + (int64_t)s * p.s_seg + (int64_t)h * p.s_head +
           (int64_t)j * p.s_token;
  const int page = p.page_table[(int64_t)s * p.pages_per_seg + j / p.page_size];
  if (page < 0 || (int64_t)page >= p.n_pool_pages) return -1;
  return (int64_t)l * p.s_layer + (int64_t)page * p.s_page +
         (int64_t)(j % p.page_size) * p.s_token + (int64_t)h * p.s_head;
}

// Page ids of tokens [j0, j1) of segment s, staged in LDS by the whole block,
// so that a row address never waits on a dependent global load.  `first` is
// the first page index covered; the block calls __syncthreads() afterwards.
__device__ __forceinline__ int stage_pages(const DPlane& p, int s, int j0, int j1, int32_t* lds) {
  if (p.page_table == nullptr || j1 <= j0) return 0;
  const int first = j0 / p.page_size, last = (j1 - 1) / p.page_size;
  const int32_t* pt = p.page_table + (int64_t)s * p.pages_per_seg;
  for (int i = threadIdx.x; i <= last - first; i += blockDim.x) lds[i] = pt[first + i];
  return first;
}

// Element offset of row (l, s, h, j) using staged page ids (or the dense
// formula); -1 for an out-of-range page id.
__device__ __forceinline__ int64_t row_offset_staged(const DPlane& p, int l, int s, int h, int j,
                                                    const int32_t* lds, int first) {
  if (p.page_table == nullptr)
    return (int64_t)l * p.s_layer + (int64_t)s * p.s_seg + (int64_t)h * p.s_head +
           (int64_t)j * p.s_token;
  const int page = lds[j / p.page_size - first];
  if (page < 0 || (int64_t)page >= p.n_pool_pages) return -1;
  return (int64_t)l * p.s_layer + (int64_t)page * p.s_page +
         (int64_t)(j % p.page_size) * p.s_token + (int64_t)h * p.s_head;
}

// Page id of token j of segment s (read directly; for staging loops).
__device__ __forceinline__ int32_t page_of(const DPlane& p, int s, int j) {
  return p.page_table ? p.page_table[(int64_t)s * p.pages_per_seg + j / p.page_size] : 0;
}

// Element offset of row (l, s, h, j) given its page id (ignored for dense
// planes); -1 for an out-of-range page id.
__device__ __forceinline__ int64_t row_offset_page(const DPlane& p, int l, int s, int h, int j,
                                                  int32_t page) {
  if (p.page_table == nullptr)
    return (int64_t)l * p.s_layer + (int64_t)s * p.s_seg + (int64_t)h * p.s_head +
           (int64_t)j * p.s_token;
  if (page < 0 || (int64_t)page >= p.n_pool_pages) return -1;
  return (int64_t)l * p.s_layer + (int64_t)page * p.s_page +
         (int64_t)(j % p.page_size) * p.s_token + (int64_t)h * p.s_head;
}

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<bf16_t> { static constexpr int N = 8; };

template <typename T, int HD, int STYLE>
struct RowMap {
  static constexpr int V = Vec<T>::N;
  static constexpr int G = HD / (2 * V);
  static constexpr int RPW = kWave / G;
  static_assert(G >= 1 && G <= kWave && (kWave % G) == 0, "unsupported head_dim");
  __device__ static constexpr int off0(int g) { return STYLE == kStyleInter ? 2 * g * V : g * V; }
  __device__ static constexpr int off1(int g) {
    return STYLE == kStyleInter ? 2 * g * V + V : HD / 2 + g * V;
  }
  __device__ static constexpr int dim_a(int g, int m) {
    return STYLE == kStyleInter ? 2 * g * V + 2 * m : g * V + m;
  }
  __device__ static constexpr int dim_b(int g, int m) {
    return STYLE == kStyleInter ? 2 * g * V + 2 * m + 1 : HD / 2 + g * V + m;
  }
};

// One-part lane map: G1 = HD / V lanes serve a row, lane g owning dims
// [gV, gV + V) (one 16-byte part).  For rotate-half, lanes g < X hold the
// first components of pairs (g mod X)V .. +V and lanes g >= X the second
// ones, X = HD / (2V); a lane's rotation partner is lane g ^ X.  For
// interleaved pairs, element m pairs with m ^ 1 inside the lane.  Halving
// the dims per lane halves the per-lane constants (mean, rank-state right
// factor, cos/sin), which keeps the streaming kernels at high occupancy.
template <typename T, int HD, int STYLE>
struct PartMap {
  static constexpr int V = Vec<T>::N;
  static constexpr int G = HD / V;
  static constexpr int RPW = kWave / G;
  static constexpr int X = HD / (2 * V);
  static_assert(G >= 2 && G <= kWave && (kWave % G) == 0, "unsupported head_dim");
  __device__ static constexpr int dim(int g, int m) { return g * V + m; }
  // rotary pair index of element m of lane g
  __device__ static constexpr int pair(int g, int m) {
    return STYLE == kStyleInter ? (g * V + m) / 2 : (g % X) * V + m;
  }
};

// Exchange a 16-byte value with lane ^ X (rotation partner).  X = 8 stays
// inside a 16-lane DPP row (row_ror:8); other distances use a lane shuffle.
template <int X>
__device__ __forceinline__ vu4 partner16(vu4 v) {
  vu4 r;
  if constexpr (X == 8) {
    r.x = __builtin_amdgcn_mov_dpp((int)v.x, 0x128, 0xf, 0xf, false);
    r.y = __builtin_amdgcn_mov_dpp((int)v.y, 0x128, 0xf, 0xf, false);
    r.z = __builtin_amdgcn_mov_dpp((int)v.z, 0x128, 0xf, 0xf, false);
    r.w = __builtin_amdgcn_mov_dpp((int)v.w, 0x128, 0xf, 0xf, false);
  } else {
    r.x = __shfl_xor((int)v.x, X);
    r.y = __shfl_xor((int)v.y, X);
    r.z = __shfl_xor((int)v.z, X);
    r.w = __shfl_xor((int)v.w, X);
  }
  return r;
}

// Rotate one lane's V elements (x) by the cos/sin of their pairs.
// Rotate-half: p holds the partner lane's elements; ss is -sin on lanes that
// hold first components and +sin on the others, so every element becomes
// x*cos + p*ss (the same operations, in the same order, as rotate_pairs).
// Interleaved: pairs are (x[2i], x[2i+1]) inside the lane; c, s indexed by m.
template <int STYLE, int V, typename C>
__device__ __forceinline__ void rotate_part(C* x, const C* p, const C* c, const C* ss) {
  if constexpr (STYLE == kStyleInter) {
#pragma unroll
    for (int m = 0; m < V; m += 2) {
      const C a = x[m], b = x[m + 1];
      x[m] = fma(a, c[m], -(b * ss[m]));
      x[m + 1] = fma(b, c[m], a * ss[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < V; ++m) x[m] = fma(x[m], c[m], p[m] * ss[m]);
  }
}

// ---------------------------------------------------------------------------
// 16-byte vector codecs
// ---------------------------------------------------------------------------

__device__ __forceinline__ vu4 ld16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const vu4*>(p));
}
__device__ __forceinline__ vu4 ld16_cached(const void* p) {
  return *reinterpret_cast<const vu4*>(p);
}
__device__ __forceinline__ void st16(void* p, vu4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<vu4*>(p));
}

// Completes the load that produced v here, once.  vmcnt counts stores as
// well as loads, so a loop that reads registers loaded before it would
// otherwise wait, every iteration, for all of its own earlier stores.
__device__ __forceinline__ void settle(vu4& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 bits, round to nearest even (one gfx950
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// double -> float rounded to odd: exact results pass through; inexact ones
// are truncated and get their last bit set.  Rounding that float to bf16
// (nearest even) then equals a single rounding of the double to bf16.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  float f = __double2float_rz(d);
  if ((double)f != d && d == d) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f;
}

template <typename C> __device__ __forceinline__ float to_bf16_input(C x);
template <> __device__ __forceinline__ float to_bf16_input<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_bf16_input<double>(double x) {
  return f64_to_f32_odd(x);
}

// Unpack 16 bytes of T into V compute values.
template <typename T, typename C> struct Codec;

template <typename C> struct Codec<bf16_t, C> {
  static constexpr int V = 8;
  __device__ static __forceinline__ void unpack(vu4 v, C* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = (C)bf16_lo(w[i]);
      x[2 * i + 1] = (C)bf16_hi(w[i]);
    }
  }
  __device__ static __forceinline__ vu4 pack(const C* x) {
    vu4 v;
    v.x = pack_bf16x2(to_bf16_input<C>(x[0]), to_bf16_input<C>(x[1]));
    v.y = pack_bf16x2(to_bf16_input<C>(x[2]), to_bf16_input<C>(x[3]));
    v.z = pack_bf16x2(to_bf16_input<C>(x[4]), to_bf16_input<C>(x[5]));
    v.w = pack_bf16x2(to_bf16_input<C>(x[6]), to_bf16_input<C>(x[7]));
    return v;
  }
};

template <typename C> struct Codec<float, C> {
  static constexpr int V = 4;
  __device__ static __forceinline__ void unpack(vu4 v, C* x) {
    x[0] = (C)__uint_as_float(v.x);
    x[1] = (C)__uint_as_float(v.y);
    x[2] = (C)__uint_as_float(v.z);
    x[3] = (C)__uint_as_float(v.w);
  }
  __device__ static __forceinline__ vu4 pack(const C* x) {
    vu4 v;
    v.x = __float_as_uint((float)x[0]);
    v.y = __float_as_uint((float)x[1]);
    v.z = __float_as_uint((float)x[2]);
    v.w = __float_as_uint((float)x[3]);
    return v;
  }
};

// Split the two 16-byte parts of a lane into its V pairs (a[m], b[m]).
template <int STYLE, int V, typename C>
__device__ __forceinline__ void parts_to_pairs(const C* p0, const C* p1, C* a, C* b) {
  if constexpr (STYLE == kStyleInter) {
#pragma unroll
    for (int m = 0; m < V; ++m) {
      const int e0 = 2 * m, e1 = 2 * m + 1;
      a[m] = e0 < V ? p0[e0] : p1[e0 - V];
      b[m] = e1 < V ? p0[e1] : p1[e1 - V];
    }
  } else {
#pragma unroll
    for (int m = 0; m < V; ++m) { a[m] = p0[m]; b[m] = p1[m]; }
  }
}

template <int STYLE, int V, typename C>
__device__ __forceinline__ void pairs_to_parts(const C* a, const C* b, C* p0, C* p1) {
  if constexpr (STYLE == kStyleInter) {
#pragma unroll
    for (int m = 0; m < V; ++m) {
      const int e0 = 2 * m, e1 = 2 * m + 1;
      if (e0 < V) p0[e0] = a[m]; else p1[e0 - V] = a[m];
      if (e1 < V) p0[e1] = b[m]; else p1[e1 - V] = b[m];
    }
  } else {
#pragma unroll
    for (int m = 0; m < V; ++m) { p0[m] = a[m]; p1[m] = b[m]; }
  }
}

// Rotate the pairs forward by the angles whose cos/sin are given.  The
// operation order is spelled out (explicit fma, contraction off in the
// build), so every kernel that rotates rounds identically.
template <int V, typename C>
__device__ __forceinline__ void rotate_pairs(C* a, C* b, const C* c, const C* s) {
#pragma unroll
  for (int m = 0; m < V; ++m) {
    const C x = a[m], y = b[m];
    a[m] = fma(x, c[m], -(y * s[m]));
    b[m] = fma(y, c[m], x * s[m]);
  }
}

// Host-side argument block carrying the rotary inverse frequencies
// theta^(-2i/hd), computed on the host in fp64 (same formula as the angles'
// definition) so that every kernel uses identical frequencies.
struct RopeArgs {
  const int64_t* delta;
  double inv_freq[kMaxHeadDim / 2];
};

// sin and cos of a rotary angle x in fp64, small enough in code and
// registers to sit inside streaming loops.  Cody-Waite reduction: k =
// nearest integer to x 2/pi, r = x - k pi/2 with pi/2 split into two 30-bit
// parts and a remainder, so k P1 and k P2 are exact for |k| < 2^23 (|x| up to
// about 1.3e7 rad, i.e. shifts up to 2^23 positions); then the Taylor series
// of sin and cos on |r| <= pi/4, through r^19 and r^20 (truncation below
// 1e-22), and the quadrant k mod 4.  Within about one unit of 2^-53 of the
// exact values.  Host-callable too, so a CPU test can check it against libm.
__host__ __device__ __forceinline__ void rope_sincos(double x, double* sp, double* cp) {
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
  constexpr double kP1 = 0x1.921fb54000000p+0;     // pi/2, first 30 bits
  constexpr double kP2 = 0x1.10b4611800000p-30;    // next 30 bits
  constexpr double kP3 = 0x1.313198a2e0370p-61;    // remainder
  const double k = rint(x * kTwoOverPi);
  double r = fma(-k, kP1, x);
  r = fma(-k, kP2, r);
  r = fma(-k, kP3, r);
  const double r2 = r * r;
  // (-1)^i / (2i+1)!, i = 1..9 and (-1)^i / (2i)!, i = 1..10
  constexpr double s3 = -1.0 / 6, s5 = 1.0 / 120, s7 = -1.0 / 5040, s9 = 1.0 / 362880,
                   s11 = -1.0 / 39916800, s13 = 1.0 / 6227020800.0,
                   s15 = -1.0 / 1307674368000.0, s17 = 1.0 / 355687428096000.0,
                   s19 = -1.0 / 121645100408832000.0;
  constexpr double c2 = -1.0 / 2, c4 = 1.0 / 24, c6 = -1.0 / 720, c8 = 1.0 / 40320,
                   c10 = -1.0 / 3628800, c12 = 1.0 / 479001600.0,
                   c14 = -1.0 / 87178291200.0, c16 = 1.0 / 20922789888000.0,
                   c18 = -1.0 / 6402373705728000.0, c20 = 1.0 / 2432902008176640000.0;
  double ps = fma(s19, r2, s17);
  ps = fma(ps, r2, s15); ps = fma(ps, r2, s13); ps = fma(ps, r2, s11); ps = fma(ps, r2, s9);
  ps = fma(ps, r2, s7); ps = fma(ps, r2, s5); ps = fma(ps, r2, s3);
  const double sr = fma(r * r2, ps, r);
  double pc = fma(c20, r2, c18);
  pc = fma(pc, r2, c16); pc = fma(pc, r2, c14); pc = fma(pc, r2, c12); pc = fma(pc, r2, c10);
  pc = fma(pc, r2, c8); pc = fma(pc, r2, c6); pc = fma(pc, r2, c4); pc = fma(pc, r2, c2);
  const double cr = fma(r2, pc, 1.0);
  const int q = (int)((int64_t)k & 3);
  *sp = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
  *cp = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}

// sin and cos of a rotary angle x for fp32 tables: the same Cody-Waite
// reduction in fp64 (so a large x loses nothing), then the Taylor series of
// sin and cos on |r| <= pi/4 in fp32 through r^11 and r^12 (truncation below
// 2e-12), and the quadrant.  Within about two units of 2^-24 of the exact
// values, at a fraction of the fp64 series' cost.  Host-callable too.
__host__ __device__ __forceinline__ void rope_sincos_f32(double x, float* sp, float* cp) {
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
  constexpr double kP1 = 0x1.921fb54000000p+0;
  constexpr double kP2 = 0x1.10b4611800000p-30;
  constexpr double kP3 = 0x1.313198a2e0370p-61;
  const double k = rint(x * kTwoOverPi);
  double rd = fma(-k, kP1, x);
  rd = fma(-k, kP2, rd);
  rd = fma(-k, kP3, rd);
  const float r = (float)rd, r2 = r * r;
  float ps = fmaf(-1.0f / 39916800.0f, r2, 1.0f / 362880.0f);
  ps = fmaf(ps, r2, -1.0f / 5040.0f);
  ps = fmaf(ps, r2, 1.0f / 120.0f);
  ps = fmaf(ps, r2, -1.0f / 6.0f);
  const float sr = fmaf(r * r2, ps, r);
  float pc = fmaf(1.0f / 479001600.0f, r2, -1.0f / 3628800.0f);
  pc = fmaf(pc, r2, 1.0f / 40320.0f);
  pc = fmaf(pc, r2, -1.0f / 720.0f);
  pc = fmaf(pc, r2, 1.0f / 24.0f);
  pc = fmaf(pc, r2, -0.5f);
  const float cr = fmaf(r2, pc, 1.0f);
  const int q = (int)((int64_t)k & 3);
  *sp = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
  *cp = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}

// Fill cos/sin of the HD/2 pair angles for a shift of delta positions into
// LDS (fp64 angle and sincos, stored in C).  Called by the whole block;
// followed by __syncthreads() at the call site.
template <int HD, typename C>
__device__ __forceinline__ void rope_table(const RopeArgs& r, int64_t delta, C* tc, C* ts) {
  for (int t = threadIdx.x; t < HD / 2; t += blockDim.x) {
    const double phi = (double)delta * r.inv_freq[t];
    double sv, cv;
    rope_sincos(phi, &sv, &cv);
    tc[t] = (C)cv;
    ts[t] = (C)sv;
  }
}

}  // namespace kvfix
