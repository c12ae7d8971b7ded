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

// The same for 64-bit values (two 32-bit counts packed in one value).
// lds: 129 words of 64 bits.
__device__ __forceinline__ uint64_t block_exclusive_scan64(uint64_t v, uint64_t* lds,
                                                          uint64_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint64_t wt = lane < kSelWaves ? lds[lane] : 0ull;
    uint64_t wi = wt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t y = __shfl_up(wi, off);
      if (lane >= off) wi += y;
    }
    if (lane < kSelWaves) lds[64 + lane] = wi - wt;
    if (lane == kSelWaves - 1) lds[128] = wi;
  }
  __syncthreads();
  const uint64_t r = lds[64 + wave] + incl - v;
  *total = lds[128];
  __syncthreads();
  return r;
}

// One histogram increment per lane with valid set, aggregated over the wave
// for the first valid lane's bin (near-equal scores put most lanes in one
// bin, where per-lane LDS atomics would serialise).
__device__ __forceinline__ void hist_add(uint32_t* whist, uint32_t bin, bool valid, int lane) {
  const uint64_t vm = __ballot(valid);
  if (vm == 0ull) return;
  const int first = (int)__builtin_ctzll(vm);
  const uint32_t lead = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
  const uint64_t same = __ballot(valid && bin == lead);
  if (lane == first) atomicAdd(&whist[lead], (uint32_t)__popcll(same));
  if (valid && bin != lead) atomicAdd(&whist[bin], 1u);
}

// Radix search over the order keys of one row of n elements for the key T of
// the b-th largest (four 8-bit passes over per-wave LDS integer histograms)
// and the number of elements equal to T that the b largest include (the
// lowest-index ones).  Keys come from registers (key[q] is the key of
// element t + 1024 q) when in_regs, else from sc.  hist: kSelWaves * 256
// words of LDS.  Every thread of the 1024-thread block
// calls it; it returns with the block synchronised.  b == 0 gives need_eq 0.
// eq_total_out: the number of keys equal to T (all of them are kept when it
// equals need_eq).  sh: 3 words of LDS.  KR: the register keys per thread
// (n <= 1024 KR when in_regs); a short row compiles only the columns it has.
template <int KR = kSelRegKeys>
__device__ __forceinline__ void radix_threshold(const uint32_t* key, bool in_regs,
                                                const float* __restrict__ sc, int n, int b,
                                                uint32_t* hist, uint32_t* sh, uint32_t* T_out,
                                                uint32_t* need_eq_out, uint32_t* eq_total_out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) { sh[0] = 0; sh[1] = (uint32_t)b; sh[2] = 0; }
  __syncthreads();
  uint32_t prefix = 0, pmask = 0;
  if (b > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = lane; i < 256; i += 64) hist[wave * 256 + i] = 0;
      __syncthreads();
      if (in_regs) {
        const int cols = (n + kSelBlock - 1) / kSelBlock;   // columns holding keys
#pragma unroll
        for (int q = 0; q < KR; ++q) {
          if (q < cols) {
            const int j = t + q * kSelBlock;
            hist_add(hist + wave * 256, (key[q] >> shift) & 255u,
                     j < n && (key[q] & pmask) == prefix, lane);
          }
        }
      } else {
        for (int j0 = 0; j0 < n; j0 += kSelBlock) {          // whole waves take part
          const int j = j0 + t;
          const uint32_t k = j < n ? order_key(sc[j]) : 0u;
          hist_add(hist + wave * 256, (k >> shift) & 255u, j < n && (k & pmask) == prefix, lane);
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
          uint32_t above = excl, in_bin = c[3];
          int d = 255 - 4 * t - 3;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (above + c[i] >= need) { d = 255 - 4 * t - i; in_bin = c[i]; break; }
            above += c[i];
          }
          sh[1] = need - above;
          sh[0] = prefix | ((uint32_t)d << shift);
          sh[2] = in_bin;                                  // after the last pass: keys == T
        }
      }
      __syncthreads();
      prefix = sh[0];
      pmask |= 255u << shift;
    }
  }
  *T_out = sh[0];
  *need_eq_out = b > 0 ? sh[1] : 0u;
  *eq_total_out = b > 0 ? sh[2] : 0u;
  __syncthreads();
}

// Exclusive prefix, in place, of the 512 counts tab[0..512) in index order;
// tab[512] receives the total.  Wave 0 works (8 entries per lane); the
// caller synchronises the block before and after.
__device__ __forceinline__ void scan512(uint32_t* tab, int t) {
  if (t >= 64) return;
  uint32_t c[8], sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { c[i] = tab[8 * t + i]; sum += c[i]; }
  uint32_t incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (t >= off) incl += y;
  }
  uint32_t run = incl - sum;
#pragma unroll
  for (int i = 0; i < 8; ++i) { tab[8 * t + i] = run; run += c[i]; }
  if (t == 63) tab[512] = incl;
}

constexpr int kCompactTab = 520;       // words of each of the two count tables

// Compaction of the b largest in index order, after radix_threshold: keys
// > T, and the first need_eq keys == T in index order.  Keys stay in the
// strided layout of the radix passes (key q of thread t is element
// 1024 q + t of a block of 32768; longer rows take several blocks), so every
// read is coalesced.  A key's place among keys == T, and its output
// position, are the count of such keys in earlier (column, wave) pairs, from
// a scanned LDS table, plus a popcount of the wave's ballot below the lane.
// emit(pos, j, key) receives every kept key; word(w, bits) every mask word
// (all ceil(n/32) words).  tab: 2 x kCompactTab words of LDS.  Every thread
// of the 1024-thread block calls it; it returns with the block synchronised.
template <int KR = kSelRegKeys, typename Emit, typename Word>
__device__ __forceinline__ void compact_topb(const uint32_t* key_regs, bool in_regs,
                                             const float* __restrict__ sc, int n, int b,
                                             uint32_t T, uint32_t need_eq, uint32_t eq_total,
                                             uint32_t* tab, Emit emit, Word word) {
  // every key == T kept (no tie straddles the b-th place): keep iff key >= T
  const bool all_eq = b > 0 && need_eq == eq_total;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  const int words = (n + 31) >> 5;
  constexpr int kSpan = kSelBlock * KR;
  uint32_t* teq = tab;
  uint32_t* tkeep = tab + kCompactTab;
  uint32_t eq_carry = 0, pos_carry = 0;
  for (int base = 0; base < n; base += kSpan) {
    const int cols = min(KR, (n - base + kSelBlock - 1) / kSelBlock);
    uint32_t key[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const int j = base + q * kSelBlock + t;
      key[q] = in_regs ? key_regs[q] : (q < cols && j < n ? order_key(sc[j]) : 0u);
    }
    auto is_eq = [&](int q) { return b > 0 && base + q * kSelBlock + t < n && key[q] == T; };
    // keys == T per (column, wave), when their rank decides
    if (!all_eq) {
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        const uint64_t em = q < cols ? __ballot(is_eq(q)) : 0ull;
        if (lane == 0) teq[q * kSelWaves + wave] = (uint32_t)__popcll(em);
      }
      __syncthreads();
      scan512(teq, t);
      __syncthreads();
    }
    auto keep = [&](int q) {
      if (all_eq) return base + q * kSelBlock + t < n && key[q] >= T;
      const bool e = is_eq(q);
      const uint64_t em = __ballot(e);
      const uint32_t rank = eq_carry + teq[q * kSelWaves + wave] + (uint32_t)__popcll(em & below);
      return (b > 0 && base + q * kSelBlock + t < n && key[q] > T) || (e && rank < need_eq);
    };
    // kept keys per (column, wave)
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const uint64_t km = q < cols ? __ballot(keep(q)) : 0ull;
      if (lane == 0) tkeep[q * kSelWaves + wave] = (uint32_t)__popcll(km);
    }
    __syncthreads();
    scan512(tkeep, t);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      if (q >= cols) continue;
      const bool k = keep(q);
      const uint64_t km = __ballot(k);
      const int j = base + q * kSelBlock + t;
      const uint32_t pos = pos_carry + tkeep[q * kSelWaves + wave] + (uint32_t)__popcll(km & below);
      if (k && pos < (uint32_t)b) emit(pos, j, key[q]);
      const int w = (base + q * kSelBlock + wave * 64) >> 5;   // the wave's two mask words
      if (lane == 0 && w < words) word(w, (uint32_t)km);
      if (lane == 32 && w + 1 < words) word(w + 1, (uint32_t)(km >> 32));
    }
    if (!all_eq) eq_carry += teq[512];
    pos_carry += tkeep[512];
    __syncthreads();                                       // the tables are reused
  }
}

}  // namespace kvfix
