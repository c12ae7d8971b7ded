// Host-side argument checks and launch helpers shared by the kvfix entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "common.h"

namespace kvfix {

#define KVFIX_TRY(expr)                        \
  do {                                         \
    const kvfix_status st_ = (expr);           \
    if (st_ != KVFIX_OK) return st_;           \
  } while (0)

inline kvfix_status launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVFIX_OK : KVFIX_ERR_HIP;
}

inline int elem_size(int32_t dtype) { return dtype == KVFIX_F32 ? 4 : 2; }

inline bool hd_supported(int32_t hd) { return hd == 64 || hd == 128 || hd == 256; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validate one plane description.  Shapes may be empty (a zero extent makes
// every call on it a no-op).
inline kvfix_status check_plane(const kvfix_plane* p) {
  if (p == nullptr) return KVFIX_ERR_ARG;
  const bool empty = p->n_layers == 0 || p->n_segs == 0 || p->n_heads == 0 || p->n_tokens == 0;
  if (p->data == nullptr && !empty) return KVFIX_ERR_ARG;   // an empty plane needs no memory
  if (p->dtype != KVFIX_F32 && p->dtype != KVFIX_BF16) return KVFIX_ERR_UNSUPPORTED;
  if (!hd_supported(p->head_dim)) return KVFIX_ERR_UNSUPPORTED;
  if (p->n_layers < 0 || p->n_segs < 0 || p->n_heads < 0 || p->n_tokens < 0)
    return KVFIX_ERR_ARG;
  if (p->s_layer < 0 || p->s_seg < 0 || p->s_head < 0 || p->s_token < 0) return KVFIX_ERR_ARG;
  const int64_t es = elem_size(p->dtype);
  if (p->data != nullptr && !aligned16(p->data)) return KVFIX_ERR_ALIGN;
  if ((p->s_layer * es) % 16 || (p->s_seg * es) % 16 || (p->s_head * es) % 16 ||
      (p->s_token * es) % 16)
    return KVFIX_ERR_ALIGN;
  if (p->page_table != nullptr) {
    if (p->page_size <= 0 || p->n_pool_pages <= 0 || p->s_page < 0) return KVFIX_ERR_ARG;
    if ((int64_t)p->pages_per_seg * p->page_size < p->n_tokens) return KVFIX_ERR_ARG;
    if ((p->s_page * es) % 16) return KVFIX_ERR_ALIGN;
  }
  return KVFIX_OK;
}

// Two planes that must describe the same logical shape (layers may differ
// where a call reads one layer of each).
inline kvfix_status same_rows(const kvfix_plane* a, const kvfix_plane* b) {
  if (a->dtype != b->dtype || a->head_dim != b->head_dim || a->n_heads != b->n_heads ||
      a->n_segs != b->n_segs || a->n_tokens != b->n_tokens)
    return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

inline kvfix_status check_rope(const kvfix_rope* r, int32_t head_dim) {
  if (r == nullptr) return KVFIX_OK;
  if (r->delta == nullptr) return KVFIX_ERR_ARG;
  if (r->style != KVFIX_ROPE_HALF && r->style != KVFIX_ROPE_INTERLEAVED) return KVFIX_ERR_ARG;
  if (!(r->theta > 0.0) || !isfinite(r->theta)) return KVFIX_ERR_ARG;
  if (head_dim > kMaxHeadDim) return KVFIX_ERR_UNSUPPORTED;
  return KVFIX_OK;
}

// Frequencies of the hd/2 rotary pairs, theta^(-2i/hd), in fp64.
inline RopeArgs make_rope_args(const kvfix_rope* r, int32_t head_dim) {
  RopeArgs a;
  memset(&a, 0, sizeof(a));
  if (r == nullptr) return a;
  a.delta = r->delta;
  for (int i = 0; i < head_dim / 2; ++i) a.inv_freq[i] = pow(r->theta, -2.0 * i / head_dim);
  return a;
}

inline kvfix_status check_lowrank(const kvfix_lowrank* lr) {
  if (lr == nullptr || lr->rank == 0) return KVFIX_OK;
  if (lr->rank < 0 || lr->rank > 8) return KVFIX_ERR_UNSUPPORTED;
  if (lr->A == nullptr || lr->B == nullptr) return KVFIX_ERR_ARG;
  if (lr->sA_layer < 0 || lr->sA_seg < 0 || lr->sA_head < 0 || lr->sB_layer < 0 ||
      lr->sB_seg < 0 || lr->sB_head < 0)
    return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

// Rank-r state as kernels see it.
struct DLowRank {
  const float* A;
  const float* B;
  int32_t rank;
  int64_t sA_layer, sA_seg, sA_head, sB_layer, sB_seg, sB_head;
};

inline DLowRank make_dlowrank(const kvfix_lowrank* lr) {
  DLowRank d;
  memset(&d, 0, sizeof(d));
  if (lr == nullptr || lr->rank == 0) return d;
  d.A = lr->A; d.B = lr->B; d.rank = lr->rank;
  d.sA_layer = lr->sA_layer; d.sA_seg = lr->sA_seg; d.sA_head = lr->sA_head;
  d.sB_layer = lr->sB_layer; d.sB_seg = lr->sB_seg; d.sB_head = lr->sB_head;
  return d;
}

// Rank rounded up to a compiled kernel variant.
inline int rank_variant(int r) { return r == 0 ? 0 : r <= 2 ? 2 : r <= 4 ? 4 : 8; }

constexpr int64_t kMaxGrid = 0x7fffffffLL;

// ceil(a / b) for a >= 0 and b > 0, in 64 bits: token counts near 2^31 do
// not wrap (a + b - 1 would overflow int32).
constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, cached per device id.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace kvfix
