// Shared pieces of the row selections: order-preserving keys, a block scan
// and the radix search for the b-th largest key of a row.
#pragma once

#include "common.h"

namespace kvfix {

constexpr int kSelBlock = 1024;
constexpr int kSelWaves = kSelBlock / 64;
constexpr int kSelRegKeys = 32;        // keys held in registers per thread (n <= 32768)

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;                                   // NaN ranks lowest
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix of a per-thread count over the block (integer, so order
// does not matter): wave prefix by shuffles, then the wave totals.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds,
                                                        uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint32_t wt = lane < kSelWaves ? lds[lane] : 0u;
    uint32_t wi = wt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(wi, off);
      if (lane >= off) wi += y;
    }
    if (lane < kSelWaves) lds[64 + lane] = wi - wt;        // exclusive prefix of wave totals
    if (lane == kSelWaves - 1) lds[128] = wi;
  }
  __syncthreads();
  const uint32_t r = lds[64 + wave] + incl - v;
  *total = lds[128];
  __syncthreads();
  return r;
}

// Radix search over the order keys of one row of n elements for the key T of
// the b-th largest (four 8-bit passes over per-wave LDS integer histograms)
// and the number of elements equal to T that the b largest include (the
// lowest-index ones).  Keys come from registers (key[q] is the key of
// element t + 1024 q) when in_regs, else from sc.  hist: kSelWaves * 256
// words of LDS; sh: 2 words of LDS.  Every thread of the 1024-thread block
// calls it; it returns with the block synchronised.  b == 0 gives need_eq 0.
__device__ __forceinline__ void radix_threshold(const uint32_t* key, bool in_regs,
                                                const float* __restrict__ sc, int n, int b,
                                                uint32_t* hist, uint32_t* sh, uint32_t* T_out,
                                                uint32_t* need_eq_out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) { sh[0] = 0; sh[1] = (uint32_t)b; }
  __syncthreads();
  uint32_t prefix = 0, pmask = 0;
  if (b > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = lane; i < 256; i += 64) hist[wave * 256 + i] = 0;
      __syncthreads();
      if (in_regs) {
#pragma unroll
        for (int q = 0; q < kSelRegKeys; ++q) {
          const int j = t + q * kSelBlock;
          if (j < n && (key[q] & pmask) == prefix) atomicAdd(&hist[wave * 256 + ((key[q] >> shift) & 255u)], 1u);
        }
      } else {
        for (int j = t; j < n; j += kSelBlock) {
          const uint32_t k = order_key(sc[j]);
          if ((k & pmask) == prefix) atomicAdd(&hist[wave * 256 + ((k >> shift) & 255u)], 1u);
        }
      }
      __syncthreads();
      if (t < 256) {                                       // fold the wave histograms
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) c += hist[w * 256 + t];
        hist[t] = c;
      }
      __syncthreads();
      if (t < 64) {
        // lane L owns bins 255-4L .. 252-4L (descending); find the bin that
        // holds the need-th largest key by a prefix over the lanes
        const uint32_t need = sh[1];
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * t - i]; sum += c[i]; }
        uint32_t incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off);
          if (t >= off) incl += y;
        }
        const uint32_t excl = incl - sum;
        if (excl < need && need <= incl) {
          uint32_t above = excl;
          int d = 255 - 4 * t - 3;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (above + c[i] >= need) { d = 255 - 4 * t - i; break; }
            above += c[i];
          }
          sh[1] = need - above;
          sh[0] = prefix | ((uint32_t)d << shift);
        }
      }
      __syncthreads();
      prefix = sh[0];
      pmask |= 255u << shift;
    }
  }
  *T_out = sh[0];
  *need_eq_out = b > 0 ? sh[1] : 0u;
  __syncthreads();
}

}  // namespace kvfix
