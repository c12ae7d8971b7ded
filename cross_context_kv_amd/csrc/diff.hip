// Master-mirror block-sparse diff: encode (a8) and fused restore (a9).
//
// A block is (agent a, layer l, token block beta): the rows of tokens
// [beta*bt, min(n, beta*bt + bt)) of every head.  One table per agent holds
// the fp64 cos/sin of its rotary shift (tiny pre-kernel into the workspace).
//
// encode
//   flag  : one 256-thread block per (l, beta).  For every agent it streams
//           the sibling's K and V rows once, re-aligns K into the master frame
//           in fp64, compares with the master (|x - m| > eps) and or-reduces
//           the block; the master rows stay hot in L2 across the agents.
//   rows  : one wave per (a, l): ballots the flags into mask words and counts.
//   scan  : one block: exclusive prefix of the counts -> offsets, status.
//   pack  : one block per packed slot (slots past the total exit): finds its
//           (a, l, beta) from the offsets and mask, re-reads the sibling block,
//           writes the re-aligned K (one rounding) and V, and beta.
// decode
//   one 256-thread block per (l, beta): for every agent, each row comes from
//   the agent's packed block if listed, else from the master (L2-hot), K is
//   rotated forward in fp64 and rounded once, and the row is written to the
//   agent's output.  No dense mirror is ever materialised.
#include <type_traits>

#include "common.h"
#include "host_util.h"

namespace kvfix {

constexpr int kDiffBlock = 256;

// tab[s * HD/2 + t] = (cos, sin) of delta[s] * inv_freq[t]
__global__ void rope_table_kernel(RopeArgs r, int half, int n_segs, double2* tab) {
  const int s = blockIdx.x;
  if (s >= n_segs) return;
  const double d = (double)r.delta[s];
  for (int t = threadIdx.x; t < half; t += blockDim.x) {
    double sv, cv;
    rope_sincos(d * r.inv_freq[t], &sv, &cv);
    tab[(int64_t)s * half + t] = make_double2(cv, sv);
  }
}

struct DiffShape {
  DPlane mk, mv, sk, sv;     // master (one segment) and siblings (n_agents segments)
  int32_t A, L, H, n, bt, nb, words;
  float eps;
};

template <int HD, int V>
__device__ __forceinline__ void load_table(const double2* tab, int seg, int g, double* cs,
                                           double* sn) {
#pragma unroll
  for (int m = 0; m < V; ++m) {
    const double2 e = tab[(int64_t)seg * (HD / 2) + g * V + m];
    cs[m] = e.x;
    sn[m] = e.y;
  }
}

// Agents handled per pass over a block's master rows: their rotary tables
// sit in LDS, and the master rows are read from HBM once per pass.
constexpr int kAgentGroup = 16;
constexpr int kMaxBlockTokens = 64;      // the largest diff block (validated on the host)

// Copy the tables of agents [a0, a0 + na) into LDS (whole block).
template <int HD>
__device__ __forceinline__ void stage_tables(const double2* tab, int a0, int na,
                                             double2 (*stab)[HD / 2]) {
  for (int i = threadIdx.x; i < na * (HD / 2); i += blockDim.x)
    stab[i / (HD / 2)][i % (HD / 2)] = tab[(int64_t)(a0 + i / (HD / 2)) * (HD / 2) + i % (HD / 2)];
}

template <int V>
__device__ __forceinline__ void lds_table(const double2* row, int g, double* cs, double* sn) {
#pragma unroll
  for (int m = 0; m < V; ++m) {
    const double2 e = row[g * V + m];
    cs[m] = e.x;
    sn[m] = e.y;
  }
}

template <typename T, int HD, int STYLE>
__global__ __launch_bounds__(kDiffBlock) __attribute__((amdgpu_waves_per_eu(3)))
void diff_flag_kernel(DiffShape D, const double2* tab, uint8_t* flags) {
  using M = RowMap<T, HD, STYLE>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPB = kDiffBlock / G;
  __shared__ double2 stab[kAgentGroup][HD / 2];
  __shared__ uint32_t sover;
  const int g = threadIdx.x % G, rr = threadIdx.x / G;
  const int beta = blockIdx.x % D.nb;
  const int l = blockIdx.x / D.nb;
  const int t0 = beta * D.bt;
  const int tb = min(D.bt, D.n - t0);           // valid tokens of this block
  const int rows = D.H * tb;
  const double eps = (double)D.eps;
  for (int a0 = 0; a0 < D.A; a0 += kAgentGroup) {
    const int na = min(kAgentGroup, D.A - a0);
    __syncthreads();                            // the previous group is done with stab, sover
    stage_tables<HD>(tab, a0, na, stab);
    if (threadIdx.x == 0) sover = 0;
    __syncthreads();
    uint32_t over = 0;                          // bit a: agent a0 + a differs on my rows
    for (int r = rr; r < rows; r += RPB) {
      const int h = r / tb, t = t0 + r % tb;
      // the master row, once per group of agents
      const T* mkp = reinterpret_cast<const T*>(D.mk.data) + row_offset(D.mk, l, 0, h, t);
      const T* mvp = reinterpret_cast<const T*>(D.mv.data) + row_offset(D.mv, l, 0, h, t);
      const vu4 mk0 = ld16(mkp + M::off0(g)), mk1 = ld16(mkp + M::off1(g));
      const vu4 mv0 = ld16(mvp + M::off0(g)), mv1 = ld16(mvp + M::off1(g));
      // the next agent's rows load while this agent's compare (the last
      // agent loads its own rows again)
      auto load_agent = [&](int a, vu4* r) {
        const T* sk = reinterpret_cast<const T*>(D.sk.data) + row_offset(D.sk, l, a0 + a, h, t);
        const T* sv = reinterpret_cast<const T*>(D.sv.data) + row_offset(D.sv, l, a0 + a, h, t);
        r[0] = ld16(sk + M::off0(g)); r[1] = ld16(sk + M::off1(g));
        r[2] = ld16(sv + M::off0(g)); r[3] = ld16(sv + M::off1(g));
      };
      vu4 nxt[4];
      load_agent(0, nxt);
      for (int a = 0; a < na; ++a) {
        const vu4 k0 = nxt[0], k1 = nxt[1], v0 = nxt[2], v1 = nxt[3];
        load_agent(a + 1 < na ? a + 1 : a, nxt);
        double cs[V], sn[V];
        lds_table<V>(stab[a], g, cs, sn);
        double p0[V], p1[V], xa[V], xb[V], ma[V], mb[V];
        Cd::unpack(k0, p0);
        Cd::unpack(k1, p1);
        parts_to_pairs<STYLE, V>(p0, p1, xa, xb);
        rotate_pairs<V>(xa, xb, cs, sn);
        Cd::unpack(mk0, p0);
        Cd::unpack(mk1, p1);
        parts_to_pairs<STYLE, V>(p0, p1, ma, mb);
        bool d = false;
#pragma unroll
        for (int m = 0; m < V; ++m) d |= (fabs(xa[m] - ma[m]) > eps) | (fabs(xb[m] - mb[m]) > eps);
        double q0[V], q1[V];
        Cd::unpack(v0, p0);
        Cd::unpack(v1, p1);
        Cd::unpack(mv0, q0);
        Cd::unpack(mv1, q1);
#pragma unroll
        for (int m = 0; m < V; ++m) d |= (fabs(p0[m] - q0[m]) > eps) | (fabs(p1[m] - q1[m]) > eps);
        over |= (uint32_t)d << a;
      }
    }
    if (over) atomicOr(&sover, over);
    __syncthreads();
    if ((int)threadIdx.x < na)
      flags[((int64_t)(a0 + threadIdx.x) * D.L + l) * D.nb + beta] = (sover >> threadIdx.x) & 1u;
  }
}

// Empty group: offsets all zero and status OK (a kernel, not a memset, so a
// captured graph replays it correctly).
__global__ void diff_empty_kernel(int64_t* offsets, int64_t n, int32_t* status) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    offsets[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = KVFIX_OK;
}

// One wave per (agent, layer) row: mask words and the row's count.
__global__ __launch_bounds__(64) void diff_rows_kernel(const uint8_t* flags, int nb, int words,
                                                       uint32_t* mask, int64_t* counts) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const uint8_t* f = flags + (int64_t)row * nb;
  uint32_t* mrow = mask + (int64_t)row * words;
  int64_t count = 0;
  for (int base = 0; base < nb; base += 64) {
    const int beta = base + lane;
    const bool on = beta < nb && f[beta] != 0;
    const uint64_t bal = __ballot(on);
    count += __popcll(bal);
    if (lane == 0 && base / 32 < words) mrow[base / 32] = (uint32_t)bal;
    if (lane == 32 && base / 32 + 1 < words) mrow[base / 32 + 1] = (uint32_t)(bal >> 32);
  }
  if (lane == 0) counts[row] = count;
}

// Exclusive prefix of the per-row counts (single block, fixed order).
__global__ __launch_bounds__(1024) void diff_scan_kernel(const int64_t* counts, int rows,
                                                         int64_t* offsets, int64_t capacity,
                                                         int32_t* status) {
  __shared__ int64_t part[1024];
  __shared__ int64_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < rows; base += 1024) {
    const int i = base + t;
    const int64_t v = i < rows ? counts[i] : 0;
    part[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int64_t add = t >= off ? part[t - off] : 0;
      __syncthreads();
      part[t] += add;
      __syncthreads();
    }
    if (i < rows) offsets[i] = carry + part[t] - v;
    __syncthreads();
    if (t == 0) carry += part[1023];
    __syncthreads();
  }
  if (t == 0) {
    offsets[rows] = carry;
    *status = carry > capacity ? KVFIX_ERR_CAPACITY : KVFIX_OK;
  }
}

struct PackParams {
  DiffShape D;
  const int64_t* offsets;
  const uint32_t* mask;
  int32_t* block_idx;
  char* vals_k;
  char* vals_v;
  int64_t capacity;
};

template <typename T, int HD, int STYLE>
__global__ __launch_bounds__(kDiffBlock) void diff_pack_kernel(PackParams P, const double2* tab) {
  using M = RowMap<T, HD, STYLE>;
  using Cd = Codec<T, double>;
  constexpr int V = M::V, G = M::G, RPB = kDiffBlock / G;
  const DiffShape& D = P.D;
  const int64_t slot = blockIdx.x;
  const int rows_al = D.A * D.L;
  const int64_t total = P.offsets[rows_al];
  if (slot >= total || slot >= P.capacity) return;
  // (agent, layer) row holding this slot: last row with offsets[row] <= slot.
  int lo = 0, hi = rows_al - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (P.offsets[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  const int row = lo;
  int64_t k = slot - P.offsets[row];
  // the k-th set bit of the row's mask
  const uint32_t* mrow = P.mask + (int64_t)row * D.words;
  int beta = 0;
  for (int w = 0; w < D.words; ++w) {
    uint32_t bits = mrow[w];
    const int c = __popc(bits);
    if (k < c) {
      for (int i = 0; i < k; ++i) bits &= bits - 1;
      beta = w * 32 + __ffs(bits) - 1;
      break;
    }
    k -= c;
  }
  const int a = row / D.L, l = row % D.L;
  if (threadIdx.x == 0) P.block_idx[slot] = beta;
  const int g = threadIdx.x % G, rr = threadIdx.x / G;
  const int t0 = beta * D.bt;
  const int tb = min(D.bt, D.n - t0);
  double cs[V], sn[V];
  load_table<HD, V>(tab, a, g, cs, sn);
  T* vk = reinterpret_cast<T*>(P.vals_k) + slot * (int64_t)D.H * D.bt * HD;
  T* vv = reinterpret_cast<T*>(P.vals_v) + slot * (int64_t)D.H * D.bt * HD;
  for (int r = rr; r < D.H * tb; r += RPB) {
    const int h = r / tb, t = r % tb;
    const T* sk = reinterpret_cast<const T*>(D.sk.data) + row_offset(D.sk, l, a, h, t0 + t);
    const T* sv = reinterpret_cast<const T*>(D.sv.data) + row_offset(D.sv, l, a, h, t0 + t);
    double p0[V], p1[V], xa[V], xb[V];
    Cd::unpack(ld16(sk + M::off0(g)), p0);
    Cd::unpack(ld16(sk + M::off1(g)), p1);
    parts_to_pairs<STYLE, V>(p0, p1, xa, xb);
    rotate_pairs<V>(xa, xb, cs, sn);
    pairs_to_parts<STYLE, V>(xa, xb, p0, p1);
    T* ok = vk + ((int64_t)h * D.bt + t) * HD;
    T* ov = vv + ((int64_t)h * D.bt + t) * HD;
    st16(ok + M::off0(g), Cd::pack(p0));
    st16(ok + M::off1(g), Cd::pack(p1));
    st16(ov + M::off0(g), ld16(sv + M::off0(g)));
    st16(ov + M::off1(g), ld16(sv + M::off1(g)));
  }
}

struct DecodeParams {
  DPlane mk, mv, ok, ov;
  const uint32_t* mask;
  const int64_t* offsets;
  const char* vals_k;
  const char* vals_v;
  int64_t capacity;
  int32_t A, L, H, n, bt, nb, words;
};

// Wait until at most N of this wave's vector memory operations are in
// flight (LDS operations not waited on); memory accesses stay on their side.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 15));
  asm volatile("" ::: "memory");
}

// Element offset of row (l, s, h, j) of a plane known to be dense.
__device__ __forceinline__ int64_t dense_offset(const DPlane& p, int l, int s, int h, int j) {
  return (int64_t)l * p.s_layer + (int64_t)s * p.s_seg + (int64_t)h * p.s_head +
         (int64_t)j * p.s_token;
}

// Direct-to-LDS loads of this wave's master rows (K and V, two 16-byte
// pieces each per lane) for head h, token j of a dense master: piece q of
// lane L lands at ring[q * 64 + L].
template <typename T, typename M>
__device__ __forceinline__ void master_dma(const DecodeParams& P, int l, int h, int j, int g,
                                           vu4* ring) {
  const T* mkp = reinterpret_cast<const T*>(P.mk.data) + dense_offset(P.mk, l, 0, h, j);
  const T* mvp = reinterpret_cast<const T*>(P.mv.data) + dense_offset(P.mv, l, 0, h, j);
  const void* src[4] = {mkp + M::off0(g), mkp + M::off1(g), mvp + M::off0(g), mvp + M::off1(g)};
#pragma unroll
  for (int q = 0; q < 4; ++q) __builtin_amdgcn_global_load_lds(src[q], to_lds(ring + 64 * q), 16, 0, 0);
}

// The same for an agent's packed rows (diff slot `slot`, head h, token t of
// the block).
template <typename T, typename M, int HD>
__device__ __forceinline__ void vals_dma(const DecodeParams& P, int64_t slot, int h, int t, int g,
                                         vu4* ring) {
  const int64_t e = ((slot * P.H + h) * (int64_t)P.bt + t) * HD;
  const T* pk = reinterpret_cast<const T*>(P.vals_k) + e;
  const T* pv = reinterpret_cast<const T*>(P.vals_v) + e;
  const void* src[4] = {pk + M::off0(g), pk + M::off1(g), pv + M::off0(g), pv + M::off1(g)};
#pragma unroll
  for (int q = 0; q < 4; ++q) __builtin_amdgcn_global_load_lds(src[q], to_lds(ring + 64 * q), 16, 0, 0);
}

// Wait until every vector memory operation of this wave issued before its
// last `younger` ones is complete (the wait allows 2^k - 1 operations in
// flight for the largest such count not above `younger`, at most 63).
__device__ __forceinline__ void wait_vm_behind(int younger) {
  if (younger >= 63) wait_vm<63>();
  else if (younger >= 31) wait_vm<31>();
  else if (younger >= 15) wait_vm<15>();
  else if (younger >= 7) wait_vm<7>();
  else if (younger >= 3) wait_vm<3>();
  else wait_vm<0>();
}

template <typename T, int HD, int STYLE, bool RING, bool PAGED_OUT>
__global__ __launch_bounds__(kDiffBlock) void diff_decode_kernel(DecodeParams P,
                                                                 const double2* tab) {
  // Values are rotated in fp32 for bf16 storage (one rounding to bf16, as in
  // apply) and in fp64 for fp32 storage.
  using C = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
  using M = RowMap<T, HD, STYLE>;
  using Cd = Codec<T, C>;
  constexpr int V = M::V, G = M::G, RPB = kDiffBlock / G;
  __shared__ double2 stab[kAgentGroup][HD / 2];
  __shared__ int64_t sslot[kAgentGroup];       // packed slot of the agent's block, or -1
  // page ids of the group's output rows (paged output planes: the slot
  // mapping), staged once per group so that no store waits on a table read
  __shared__ int32_t spk[PAGED_OUT ? kAgentGroup * kMaxBlockTokens : 1];
  __shared__ int32_t spv[PAGED_OUT ? kAgentGroup * kMaxBlockTokens : 1];
  // dense master planes: each wave's master rows of the next pass and the packed
  // rows of the pass's first agent with a diff block, loaded straight into
  // LDS (four 16-byte pieces per lane each); the group's agents in the order
  // the passes take them, agents without a diff block first
  __shared__ vu4 mring[RING ? kDiffBlock / 64 : 1][4][64];
  __shared__ vu4 dring[RING ? kDiffBlock / 64 : 1][4][64];
  __shared__ int32_t sorder[kAgentGroup];
  __shared__ int32_t sndiff;
  const int g = threadIdx.x % G, rr = threadIdx.x / G;
  const int beta = blockIdx.x % P.nb;
  const int l = blockIdx.x / P.nb;
  const int t0 = beta * P.bt;
  const int tb = min(P.bt, P.n - t0);
  const int rows = P.H * tb;
  for (int a0 = 0; a0 < P.A; a0 += kAgentGroup) {
    const int na = min(kAgentGroup, P.A - a0);
    __syncthreads();                            // the previous group is done with stab, sslot
    stage_tables<HD>(tab, a0, na, stab);
    if ((int)threadIdx.x < na) {
      const int arow = (a0 + threadIdx.x) * P.L + l;
      const uint32_t* mrow = P.mask + (int64_t)arow * P.words;
      int64_t slot = -1;
      if ((mrow[beta >> 5] >> (beta & 31)) & 1u) {
        int64_t before = 0;
        for (int w = 0; w < (beta >> 5); ++w) before += __popc(mrow[w]);
        before += __popc(mrow[beta >> 5] & ((1u << (beta & 31)) - 1u));
        slot = P.offsets[arow] + before;
        if (slot >= P.capacity) slot = -1;      // never read past the packed values
      }
      sslot[threadIdx.x] = slot;
    }
    if (PAGED_OUT) {
      for (int i = threadIdx.x; i < na * tb; i += kDiffBlock) {
        const int a = i / tb, t = i % tb;
        spk[a * kMaxBlockTokens + t] = page_of(P.ok, a0 + a, t0 + t);
        spv[a * kMaxBlockTokens + t] = page_of(P.ov, a0 + a, t0 + t);
      }
    }
    __syncthreads();
    if (RING) {
      if (threadIdx.x == 0) {
        int k = 0, nd = 0;
        for (int a = 0; a < na; ++a)
          if (sslot[a] < 0) sorder[k++] = a;
        for (int a = 0; a < na; ++a)
          if (sslot[a] >= 0) { sorder[k++] = a; ++nd; }
        sndiff = nd;
      }
      __syncthreads();
    }
    // Dense master planes: loads and stores share one in-order counter, so a load
    // issued behind stores cannot be waited for without waiting for them.
    // A pass's master rows are therefore loaded into the wave's LDS ring at
    // the start of the previous pass, before its stores (at least 4 * na:
    // K and V, two pieces each, per agent), and the packed rows of the
    // pass's first agent with a diff block at the start of the pass, before
    // the stores of the agents without one, which go first.  A dense output
    // issues 4 stores per agent; a paged one skips a store where no lane has
    // a valid row, so its waits count the stores the wave has issued since
    // (loads are not counted, which only makes a wait stricter).  Paged
    // master planes load every row in place.
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nd = RING ? sndiff : 0;
    if (RING && rr < rows) master_dma<T, M>(P, l, rr / tb, t0 + rr % tb, g, &mring[wave][0][0]);
    int since_m = 0, since_d = 0;   // stores issued since the master / packed-row loads
    for (int r = rr, pass = 0; r < rows; r += RPB, ++pass) {
      const int h = r / tb, t = r % tb;
      // the master row, once per group of agents
      vu4 mk0, mk1, mv0, mv1;
      if (RING) {
        wait_vm_behind(pass == 0 ? 0 : PAGED_OUT ? since_m : 4 * na);
        mk0 = mring[wave][0][lane]; mk1 = mring[wave][1][lane];
        mv0 = mring[wave][2][lane]; mv1 = mring[wave][3][lane];
        // the rings are this wave's and this lane's: once the reads are done
        // (the packed rows' in the previous pass too) they take new rows
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (nd > 0) vals_dma<T, M, HD>(P, sslot[sorder[na - nd]], h, t, g, &dring[wave][0][0]);
        since_d = 0;
        if (r + RPB < rows)
          master_dma<T, M>(P, l, (r + RPB) / tb, t0 + (r + RPB) % tb, g, &mring[wave][0][0]);
        since_m = 0;
      } else {
        const T* mkp = reinterpret_cast<const T*>(P.mk.data) + row_offset(P.mk, l, 0, h, t0 + t);
        const T* mvp = reinterpret_cast<const T*>(P.mv.data) + row_offset(P.mv, l, 0, h, t0 + t);
        mk0 = ld16(mkp + M::off0(g)); mk1 = ld16(mkp + M::off1(g));
        mv0 = ld16(mvp + M::off0(g)); mv1 = ld16(mvp + M::off1(g));
        settle(mk0); settle(mk1); settle(mv0); settle(mv1);
      }
      for (int i = 0; i < na; ++i) {
        const int a = RING ? sorder[i] : i;     // uniform over the block
        const int64_t slot = sslot[a];
        vu4 k0 = mk0, k1 = mk1, v0 = mv0, v1 = mv1;
        if (RING && i == na - nd) {
          // the first agent with a diff block: its rows are in the ring,
          // behind the stores of the agents without one
          wait_vm_behind(PAGED_OUT ? since_d : 4 * (na - nd));
          k0 = dring[wave][0][lane]; k1 = dring[wave][1][lane];
          v0 = dring[wave][2][lane]; v1 = dring[wave][3][lane];
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        } else if (slot >= 0) {
          const int64_t e = ((slot * P.H + h) * (int64_t)P.bt + t) * HD;
          const T* pk = reinterpret_cast<const T*>(P.vals_k) + e;
          const T* pv = reinterpret_cast<const T*>(P.vals_v) + e;
          k0 = ld16(pk + M::off0(g));
          k1 = ld16(pk + M::off1(g));
          v0 = ld16(pv + M::off0(g));
          v1 = ld16(pv + M::off1(g));
          // consumed on this path, so that no later iteration waits on them
          settle(k0); settle(k1); settle(v0); settle(v1);
        }
        double csd[V], snd[V];
        lds_table<V>(stab[a], g, csd, snd);
        C cs[V], sn[V];
#pragma unroll
        for (int m = 0; m < V; ++m) { cs[m] = (C)csd[m]; sn[m] = (C)snd[m]; }
        C p0[V], p1[V], xa[V], xb[V];
        Cd::unpack(k0, p0);
        Cd::unpack(k1, p1);
        parts_to_pairs<STYLE, V>(p0, p1, xa, xb);
        rotate_pairs<V>(xa, xb, cs, sn);
        pairs_to_parts<STYLE, V>(xa, xb, p0, p1);
        const int64_t ko =
            PAGED_OUT ? row_offset_page(P.ok, l, a0 + a, h, t0 + t, spk[a * kMaxBlockTokens + t])
                      : dense_offset(P.ok, l, a0 + a, h, t0 + t);
        const int64_t vo =
            PAGED_OUT ? row_offset_page(P.ov, l, a0 + a, h, t0 + t, spv[a * kMaxBlockTokens + t])
                      : dense_offset(P.ov, l, a0 + a, h, t0 + t);
        if (!PAGED_OUT || ko >= 0) {
          T* dk = reinterpret_cast<T*>(P.ok.data) + ko;
          st16(dk + M::off0(g), Cd::pack(p0));
          st16(dk + M::off1(g), Cd::pack(p1));
        }
        if (!PAGED_OUT || vo >= 0) {
          T* dv = reinterpret_cast<T*>(P.ov.data) + vo;
          st16(dv + M::off0(g), v0);
          st16(dv + M::off1(g), v1);
        }
        if (RING && PAGED_OUT) {
          const int issued = 2 * (__ballot(ko >= 0) != 0) + 2 * (__ballot(vo >= 0) != 0);
          since_m += issued;
          since_d += issued;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// master selection (TD §4.2, reuse plan output): the request with the lowest
// total deviation.  Wave w sums the scores of requests w, w + 16, ... in
// fp64 in the order the definition fixes: lane k sums whole 64-token blocks
// in token order, then the block sums are added in block order; thread 0
// then takes the lowest total, ties to the lower index, a NaN total last.
// ---------------------------------------------------------------------------

constexpr int kMasterBlock = 1024;

__global__ __launch_bounds__(kMasterBlock) void select_master_kernel(const float* __restrict__ scores,
                                                                     int A, int n,
                                                                     double* __restrict__ totals,
                                                                     int32_t* __restrict__ master) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nblk = (n + 63) / 64;
  for (int a = wave; a < A; a += kMasterBlock / kWave) {
    const float* p = scores + (int64_t)a * n;
    double total = 0.0;
    for (int b0 = 0; b0 < nblk; b0 += kWave) {
      // lane k: the sum of block b0 + k, its tokens in order
      const int bk = b0 + lane;
      double blk = 0.0;
      if (bk < nblk) {
        const int j0 = bk * 64, j1 = min(j0 + 64, n);
        for (int j = j0; j < j1; j += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = j + u < j1 ? p[j + u] : 0.0f;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (j + u < j1) blk += (double)v[u];
        }
      }
      // the block sums, in block order
      const int cnt = min(kWave, nblk - b0);
      for (int k = 0; k < cnt; ++k) {
        const uint64_t bits = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                  (int)(uint32_t)__double_as_longlong(blk), k) |
                              (uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                  (int)(uint32_t)(__double_as_longlong(blk) >> 32), k)
                                  << 32;
        total += __longlong_as_double((long long)bits);
      }
    }
    if (lane == 0) totals[a] = total;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    double bv = totals[0];
    for (int a = 1; a < A; ++a) {
      const double v = totals[a];
      if (v < bv || (bv != bv && v == v)) { bv = v; best = a; }
    }
    *master = best;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline size_t table_bytes(int32_t n_agents, int32_t head_dim) {
  return align256((size_t)n_agents * (head_dim / 2) * sizeof(double2));
}

template <template <typename, int, int> class F, typename... Args>
kvfix_status dispatch_rot(int32_t dtype, int32_t hd, int style, Args&&... args) {
#define KVFIX_DCASE(T_, HD_, ST_)                                            \
  if (dtype == (std::is_same<T_, float>::value ? KVFIX_F32 : KVFIX_BF16) &&   \
      hd == HD_ && style == ST_)                                            \
    return F<T_, HD_, ST_>::run(args...);
#define KVFIX_DSTYLES(T_, HD_) KVFIX_DCASE(T_, HD_, kStyleHalf) KVFIX_DCASE(T_, HD_, kStyleInter)
  KVFIX_DSTYLES(float, 64) KVFIX_DSTYLES(float, 128) KVFIX_DSTYLES(float, 256)
  KVFIX_DSTYLES(bf16_t, 64) KVFIX_DSTYLES(bf16_t, 128) KVFIX_DSTYLES(bf16_t, 256)
#undef KVFIX_DSTYLES
#undef KVFIX_DCASE
  return KVFIX_ERR_UNSUPPORTED;
}

template <typename T, int HD, int STYLE>
struct FlagLaunch {
  static kvfix_status run(const DiffShape& D, const double2* tab, uint8_t* flags, hipStream_t st) {
    diff_flag_kernel<T, HD, STYLE>
        <<<dim3((unsigned)((int64_t)D.L * D.nb)), dim3(kDiffBlock), 0, st>>>(D, tab, flags);
    return launch_status();
  }
};

template <typename T, int HD, int STYLE>
struct PackLaunch {
  static kvfix_status run(const PackParams& P, const double2* tab, hipStream_t st) {
    diff_pack_kernel<T, HD, STYLE>
        <<<dim3((unsigned)P.capacity), dim3(kDiffBlock), 0, st>>>(P, tab);
    return launch_status();
  }
};

template <typename T, int HD, int STYLE>
struct DecodeLaunch {
  static kvfix_status run(const DecodeParams& P, const double2* tab, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)P.L * P.nb)), block(kDiffBlock);
    // the LDS rings need dense master planes; paged outputs take staged page ids
    const bool ring = !P.mk.page_table && !P.mv.page_table;
    const bool paged_out = P.ok.page_table || P.ov.page_table;
    if (ring && !paged_out)
      diff_decode_kernel<T, HD, STYLE, true, false><<<grid, block, 0, st>>>(P, tab);
    else if (ring)
      diff_decode_kernel<T, HD, STYLE, true, true><<<grid, block, 0, st>>>(P, tab);
    else
      diff_decode_kernel<T, HD, STYLE, false, true><<<grid, block, 0, st>>>(P, tab);
    return launch_status();
  }
};

// Shape checks shared by encode and decode: masters hold one segment, the
// siblings / outputs n_agents; everything else agrees.
inline kvfix_status check_group(const kvfix_plane* mk, const kvfix_plane* mv,
                                const kvfix_plane* sk, const kvfix_plane* sv) {
  KVFIX_TRY(check_plane(mk));
  KVFIX_TRY(check_plane(mv));
  KVFIX_TRY(check_plane(sk));
  KVFIX_TRY(check_plane(sv));
  if (mk->n_segs != 1 || mv->n_segs != 1) return KVFIX_ERR_ARG;
  const kvfix_plane* all[4] = {mk, mv, sk, sv};
  for (const kvfix_plane* p : all) {
    if (p->dtype != mk->dtype || p->head_dim != mk->head_dim || p->n_heads != mk->n_heads ||
        p->n_tokens != mk->n_tokens || p->n_layers != mk->n_layers)
      return KVFIX_ERR_ARG;
  }
  if (sk->n_segs != sv->n_segs) return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

inline kvfix_status check_diff(const kvfix_diff* d) {
  if (d == nullptr || d->offsets == nullptr) return KVFIX_ERR_ARG;
  if (d->block_tokens < 1 || d->block_tokens > kMaxBlockTokens || d->capacity_blocks < 0)
    return KVFIX_ERR_ARG;
  if (d->capacity_blocks > 0 && (d->block_idx == nullptr || d->vals_k == nullptr ||
                                 d->vals_v == nullptr))
    return KVFIX_ERR_ARG;
  if (!aligned16(d->vals_k) || !aligned16(d->vals_v)) return KVFIX_ERR_ALIGN;
  if (d->capacity_blocks > kMaxGrid) return KVFIX_ERR_ARG;
  return KVFIX_OK;
}

}  // namespace kvfix

using namespace kvfix;

extern "C" size_t kvfix_diff_encode_workspace(int32_t n_agents, int32_t n_layers,
                                              int32_t n_tokens, int32_t block_tokens) {
  if (n_agents < 0 || n_layers < 0 || n_tokens < 0 || block_tokens < 1) return 0;
  const size_t nb = ((size_t)n_tokens + block_tokens - 1) / block_tokens;
  const size_t rows = (size_t)n_agents * n_layers;
  return table_bytes(n_agents, kMaxHeadDim) + align256(rows * nb) + align256(rows * 8);
}

extern "C" size_t kvfix_diff_decode_workspace(int32_t n_agents, int32_t head_dim) {
  if (n_agents < 0 || head_dim < 0) return 0;
  return table_bytes(n_agents, head_dim > kMaxHeadDim ? kMaxHeadDim : head_dim);
}

extern "C" kvfix_status kvfix_diff_encode(const kvfix_plane* master_k, const kvfix_plane* master_v,
                                          const kvfix_plane* sib_k, const kvfix_plane* sib_v,
                                          const kvfix_rope* to_master, float eps,
                                          const kvfix_diff* out, int32_t* dev_status, void* ws,
                                          size_t ws_bytes, void* stream) {
  KVFIX_TRY(check_group(master_k, master_v, sib_k, sib_v));
  KVFIX_TRY(check_diff(out));
  if (to_master == nullptr || dev_status == nullptr || !(eps >= 0.0f)) return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(to_master, master_k->head_dim));
  const int32_t A = sib_k->n_segs, L = sib_k->n_layers, n = sib_k->n_tokens;
  const int32_t bt = out->block_tokens;
  const int32_t nb = (int32_t)ceil_div(n, bt), words = (int32_t)ceil_div(nb, 32);
  if ((int64_t)A * L > 0x7fffffff / 2) return KVFIX_ERR_ARG;
  if ((int64_t)A * L * words > 0 && out->mask == nullptr) return KVFIX_ERR_ARG;
  const size_t need = kvfix_diff_encode_workspace(A, L, n, bt);
  if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255)) return KVFIX_ERR_ARG;
  if ((int64_t)L * nb > kMaxGrid) return KVFIX_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  double2* tab = reinterpret_cast<double2*>(w);
  uint8_t* flags = reinterpret_cast<uint8_t*>(w + table_bytes(A, kMaxHeadDim));
  int64_t* counts = reinterpret_cast<int64_t*>(w + table_bytes(A, kMaxHeadDim) +
                                               align256((size_t)A * L * nb));
  if (A == 0 || L == 0 || n == 0) {
    const int64_t cnt = (int64_t)A * L + 1;
    diff_empty_kernel<<<dim3((unsigned)((cnt + 255) / 256 > 1024 ? 1024 : (cnt + 255) / 256)),
                        dim3(256), 0, st>>>(out->offsets, cnt, dev_status);
    return launch_status();
  }
  const RopeArgs rope = make_rope_args(to_master, master_k->head_dim);
  rope_table_kernel<<<dim3(A), dim3(64), 0, st>>>(rope, master_k->head_dim / 2, A, tab);
  KVFIX_TRY(launch_status());
  DiffShape D;
  D.mk = make_dplane(*master_k); D.mv = make_dplane(*master_v);
  D.sk = make_dplane(*sib_k); D.sv = make_dplane(*sib_v);
  D.A = A; D.L = L; D.H = sib_k->n_heads; D.n = n; D.bt = bt; D.nb = nb; D.words = words;
  D.eps = eps;
  KVFIX_TRY(dispatch_rot<FlagLaunch>(master_k->dtype, master_k->head_dim, to_master->style, D,
                                     (const double2*)tab, flags, st));
  diff_rows_kernel<<<dim3((unsigned)(A * L)), dim3(64), 0, st>>>(flags, nb, words, out->mask,
                                                                 counts);
  KVFIX_TRY(launch_status());
  diff_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(counts, A * L, out->offsets,
                                                   out->capacity_blocks, dev_status);
  KVFIX_TRY(launch_status());
  if (out->capacity_blocks == 0) return KVFIX_OK;
  PackParams P;
  P.D = D;
  P.offsets = out->offsets;
  P.mask = out->mask;
  P.block_idx = out->block_idx;
  P.vals_k = static_cast<char*>(out->vals_k);
  P.vals_v = static_cast<char*>(out->vals_v);
  P.capacity = out->capacity_blocks;
  return dispatch_rot<PackLaunch>(master_k->dtype, master_k->head_dim, to_master->style, P,
                                  (const double2*)tab, st);
}

extern "C" kvfix_status kvfix_diff_decode(const kvfix_plane* master_k, const kvfix_plane* master_v,
                                          const kvfix_diff* diff, const kvfix_rope* from_master,
                                          const kvfix_plane* out_k, const kvfix_plane* out_v,
                                          void* ws, size_t ws_bytes, void* stream) {
  KVFIX_TRY(check_group(master_k, master_v, out_k, out_v));
  KVFIX_TRY(check_diff(diff));
  if (from_master == nullptr) return KVFIX_ERR_ARG;
  KVFIX_TRY(check_rope(from_master, master_k->head_dim));
  const int32_t A = out_k->n_segs, L = out_k->n_layers, n = out_k->n_tokens;
  const int32_t bt = diff->block_tokens;
  const int32_t nb = (int32_t)ceil_div(n, bt), words = (int32_t)ceil_div(nb, 32);
  if (A == 0 || L == 0 || n == 0 || out_k->n_heads == 0) return KVFIX_OK;
  if (diff->mask == nullptr) return KVFIX_ERR_ARG;
  const size_t need = kvfix_diff_decode_workspace(A, master_k->head_dim);
  if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255)) return KVFIX_ERR_ARG;
  if ((int64_t)L * nb > kMaxGrid) return KVFIX_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  double2* tab = reinterpret_cast<double2*>(ws);
  const RopeArgs rope = make_rope_args(from_master, master_k->head_dim);
  rope_table_kernel<<<dim3(A), dim3(64), 0, st>>>(rope, master_k->head_dim / 2, A, tab);
  KVFIX_TRY(launch_status());
  DecodeParams P;
  P.mk = make_dplane(*master_k); P.mv = make_dplane(*master_v);
  P.ok = make_dplane(*out_k); P.ov = make_dplane(*out_v);
  P.mask = diff->mask;
  P.offsets = diff->offsets;
  P.vals_k = static_cast<const char*>(diff->vals_k);
  P.vals_v = static_cast<const char*>(diff->vals_v);
  P.capacity = diff->capacity_blocks;
  P.A = A; P.L = L; P.H = out_k->n_heads; P.n = n; P.bt = bt; P.nb = nb; P.words = words;
  return dispatch_rot<DecodeLaunch>(master_k->dtype, master_k->head_dim, from_master->style, P,
                                    (const double2*)tab, st);
}

extern "C" kvfix_status kvfix_select_master(const float* scores, int32_t n_agents, int32_t n,
                                            double* totals, int32_t* master, void* stream) {
  if (n_agents < 1 || n < 0 || (scores == nullptr && n > 0) || totals == nullptr ||
      master == nullptr)
    return KVFIX_ERR_ARG;
  select_master_kernel<<<dim3(1), dim3(kMasterBlock), 0, (hipStream_t)stream>>>(
      scores, n_agents, n, totals, master);
  return launch_status();
}
