// Router top-k, routing weights and the fused expert-id -> slot remap with
// batch-LRU victim choice, in one workgroup: four wavefronts, or eight for a
// step of many picks (each wavefront routes one row at a time), or a single
// wavefront for a one-row step.
//
// Method: the slot cache of page "GLM 5.3 Testing: HBM Expert Allocation"
// (section "What the slot cache is": ids are mapped to slots on the device
// before the expert launch, a miss takes the least-recently-used victim slot,
// more than 16 rows bypass), doing in one kernel what that page's section "The
// build" spread over a dozen small framework ops.  Occupancy follows an LRU clock
// (page "GB300 GLM 5.3 Testing", section "Expert allocation vs a cache").
// Router ties break by a stable expert order (page "TensorFold GLM-5.3
// explained", exact-decoding rule).
//
// Bookkeeping rules (the pages leave these open; one launch maps a whole step,
// so they are per step):
//   P  = the M*k picks in (row, rank) order, p = 0..M*k-1
//   U  = unique experts of P in first-occurrence order; hits = resident ones
//   bypass when M > 16 or |U| - (pinned hits) > S - P (P pinned slots; |U| > S
//          without pins): the cache is untouched, the step counter still
//          advances, resident experts are read from their slots and the
//          others from the backing store (the pages' bypass reads
//          non-resident experts: page "GB300 GLM 5.3 Testing", section on
//          sizing the context window); a prefill step with a staging area
//          copies those into HBM staging blobs first, G per group
//   pinned slots [0, P) hold fixed experts and are never victims
//   candidates = slots not holding a hit, ascending (key, slot); empty slots
//          have key -1; the i-th miss (first-occurrence order) takes the i-th
//   key[slot(e)] = t * (16 * k) + last position of e in P, for every e in U
#include "internal.h"

#include <climits>

namespace sc {
namespace {

// Steps of at least kRouteWidePicks picks (eight rows of top-8) route on eight
// wavefronts: twice the rows in flight, at the cost of wider barriers.
constexpr int kRouteWideThreads = 512;
constexpr int kRouteWidePicks = 64;
// One-row steps of at most kRouteOneMaxK picks that cannot bypass route on one
// wavefront (k_route_one); the victim search takes one wavefront minimum per miss.
constexpr int kRouteOneMaxK = 16;

__device__ __forceinline__ uint64_t order_key(float z, int e) {
  // Larger key = earlier pick: logit descending, then expert id ascending.
  // NaN sorts below -inf; -0 and +0 compare equal.  Key 0 marks "taken".
  uint32_t u = __float_as_uint(z);
  uint32_t ord;
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) {
    ord = 1u;
  } else {
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Cross-lane reductions on the DPP path (no LDS round trip): quad
// permutations and the half-row / row mirrors reduce each 16-lane row, two
// row broadcasts fold the rows into lane 63, which readlane makes uniform.
// Lanes of a row that the row mask leaves out read `OLD` instead of a
// neighbour: the identity of the reduction (0 for max and sum, all ones for min).
template <int CTRL, int ROWS, uint32_t OLD = 0u>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)OLD, (int)v, CTRL, ROWS, 0xF, false);
}

template <bool MAX, int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_step_u64(uint64_t v) {
  constexpr uint32_t ID = MAX ? 0u : 0xFFFFFFFFu;
  const uint64_t o = ((uint64_t)dpp_u32<CTRL, ROWS, ID>((uint32_t)(v >> 32)) << 32) |
                     dpp_u32<CTRL, ROWS, ID>((uint32_t)v);
  if (MAX) return o > v ? o : v;
  return o < v ? o : v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  return ((uint64_t)hi << 32) | lo;
}

// Max (MAX) or min over the wavefront, returned as a uniform value.
template <bool MAX>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t v) {
  v = dpp_step_u64<MAX, 0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v = dpp_step_u64<MAX, 0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v = dpp_step_u64<MAX, 0x141, 0xF>(v);   // row_half_mirror
  v = dpp_step_u64<MAX, 0x140, 0xF>(v);   // row_mirror
  v = dpp_step_u64<MAX, 0x142, 0xA>(v);   // row_bcast:15 -> rows 1, 3
  v = dpp_step_u64<MAX, 0x143, 0xC>(v);   // row_bcast:31 -> rows 2, 3
  return readlane_u64(v, 63);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = dpp_u32<CTRL, ROWS>(v);
  return o > v ? o : v;
}

// Unsigned 32-bit maximum over the wavefront, uniform result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1, 0xF>(v);
  v = dpp_max_u32<0x4E, 0xF>(v);
  v = dpp_max_u32<0x141, 0xF>(v);
  v = dpp_max_u32<0x140, 0xF>(v);
  v = dpp_max_u32<0x142, 0xA>(v);
  v = dpp_max_u32<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add_f32(float v) {
  return v + __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v)));
}

// Sum over the wavefront in a fixed order, returned as a uniform value.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = dpp_add_f32<0xB1, 0xF>(v);
  v = dpp_add_f32<0x4E, 0xF>(v);
  v = dpp_add_f32<0x141, 0xF>(v);
  v = dpp_add_f32<0x140, 0xF>(v);
  v = dpp_add_f32<0x142, 0xA>(v);
  v = dpp_add_f32<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Exclusive rank of `pred` among the block's NT threads in thread order.
template <int NT>
__device__ __forceinline__ int block_rank(bool pred, int* s_wc, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t mask = __ballot(pred);
  int in_wave = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) s_wc[wave] = __popcll(mask);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int c = s_wc[w];
    if (w < wave) base += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + in_wave;
}

// Exclusive scan of s_in[0..n) into s_out (n <= 4 * NT); returns the total.
template <int NT>
__device__ __forceinline__ int block_scan(const int* s_in, int* s_out, int n, int* s_wc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int idx = 4 * tid + i;
    v[i] = idx < n ? s_in[idx] : 0;
    sum += v[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wc[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) base += s_wc[w];
    tot += s_wc[w];
  }
  int ex = base + incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int idx = 4 * tid + i;
    if (idx < n) s_out[idx] = ex;
    ex += v[i];
  }
  __syncthreads();
  return tot;
}

struct RouteArgs {
  Shape sh;
  LayerDev L;
  Workspace W;
  const float* logits;
  int M;
  uint64_t* span;
};

// Router for one row on one wavefront: lane l holds the keys of experts
// l, l+64, ... sorted by (logit descending, id ascending).  Each round takes
// the wavefront maximum of the lanes' head order words (32-bit); equal heads
// are settled by the lowest expert id, and the owner lane pops its head.
// Lane j < k returns the j-th pick and its logit.  z holds the lane's
// logits (load_row).
template <int EPL>
__device__ __forceinline__ void load_row(const float* row, int E, int lane, float (&z)[EPL]) {
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    z[i] = e < E ? row[e] : 0.0f;
  }
}

template <int EPL>
__device__ __forceinline__ void route_row(const float (&z)[EPL], int E, int k, int lane, int* pick, float* logit) {
  uint64_t keys[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    keys[i] = e < E ? order_key(z[i], e) : 0ull;
  }
#pragma unroll
  for (int i = 1; i < EPL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j)
      if (keys[j] > keys[j - 1]) {
        const uint64_t tmp = keys[j];
        keys[j] = keys[j - 1];
        keys[j - 1] = tmp;
      }
  int my_e = 0;
  uint32_t my_ord = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t h_ord = (uint32_t)(keys[0] >> 32);
    const uint32_t h_inv = (uint32_t)keys[0];            // 0xFFFFFFFF - expert id
    const uint32_t best = wave_max_u32(h_ord);
    const uint64_t tied = __ballot(keys[0] != 0ull && h_ord == best);
    uint32_t win_inv;
    if (__popcll(tied) == 1) {
      win_inv = (uint32_t)__builtin_amdgcn_readlane((int)h_inv, (int)__ffsll((unsigned long long)tied) - 1);
    } else {
      win_inv = wave_max_u32(((tied >> lane) & 1ull) ? h_inv : 0u);   // lowest id among the tied heads
    }
    if (keys[0] != 0ull && h_ord == best && h_inv == win_inv) {
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) keys[i] = keys[i + 1];
      keys[EPL - 1] = 0ull;
    }
    if (lane == j) {
      my_e = (int)(0xFFFFFFFFu - win_inv);
      my_ord = best;
    }
  }
  // the logit back from its order key (NaN keys carry ord 1; -0 was folded into +0)
  const uint32_t zb = (my_ord & 0x80000000u) ? (my_ord & 0x7FFFFFFFu) : ~my_ord;
  *pick = my_e;
  *logit = my_ord == 1u ? __uint_as_float(0x7FC00000u) : __uint_as_float(zb);
}

// Routing weight of lane j's pick (j < k): softmax over the k chosen logits,
// in the limits for non-finite picks (+inf picks share the weight, a NaN or
// -inf leading logit gives every pick 1/k).  zj is route_row's logit.
__device__ __forceinline__ float pick_weight(float zj, int k, int lane) {
  const bool act = lane < k;
  if (!act) zj = 0.0f;
  const bool is_nan = zj != zj;
  const bool pinf = act && zj == INFINITY;
  const int npinf = __popcll(__ballot(pinf));
  const float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zj), 0));
  if (npinf > 0) return pinf ? 1.0f / (float)npinf : 0.0f;
  if (z0 != z0 || z0 == -INFINITY) return 1.0f / (float)k;
  const float ex = (act && !is_nan) ? expf(zj - z0) : 0.0f;
  const float sum = wave_sum_f32(ex);
  return ex / sum;
}

// Bookkeeping of a step of at most 16 rows and 64 picks (cached, or a bypass
// when its experts do not fit) on one wavefront, once its rows are routed and
// the picks and the state snapshot are in LDS: pick p on lane p, unique
// expert u on lane u.  The rules and every value written are those of the
// block-wide passes of k_route_remap, without its block barriers.
__device__ __forceinline__ void remap_small(const RouteArgs& a, int M, int P, const int* s_pick, int* s_first,
                                         int* s_last, int* s_uidx, int* s_uexp, const int* s_e2s,
                                         const int* s_s2e, const long long* s_key, uint8_t* s_ref, int64_t t,
                                         uint64_t ev_head, uint64_t (&cnt)[C_N]) {
  const int lane = threadIdx.x & 63;
  const int E = a.sh.E, k = a.sh.k, S = a.L.S, Pn = a.L.P;
  const int64_t B = a.sh.blob;
  const uint64_t below = (1ull << lane) - 1ull;

  // unique experts in first-occurrence order (the LDS operations of one
  // wavefront take effect in program order)
  const bool act = lane < P;
  const int e = act ? s_pick[lane] : 0;
  if (act) {
    atomicMin(&s_first[e], lane);
    atomicMax(&s_last[e], lane);
  }
  const bool first = act && s_first[e] == lane;
  const uint64_t fm = __ballot(first);
  const int U = __popcll(fm);
  if (first) {
    const int r = __popcll(fm & below);
    s_uexp[r] = e;
    s_uidx[e] = r;
  }

  // residency against the slot map
  const bool uact = lane < U;
  const int ue = uact ? s_uexp[lane] : 0;
  int sl = uact ? s_e2s[ue] : -1;
  if (uact && (sl < -1 || sl >= S)) {
    atomicOr(a.L.error, 1u);
    sl = -1;
  }
  const bool miss = uact && sl < 0;
  const uint64_t mm = __ballot(miss);
  const int nmiss = __popcll(mm), mrank = __popcll(mm & below);
  const int npin = __popcll(__ballot(uact && sl >= 0 && sl < Pn));
  const bool bypass = U - npin > S - Pn;
  const int nres = U - nmiss;
  int nevict = 0;
  if (!bypass) {
    if (nmiss > 0) {
      // victims: the nmiss least (key, slot) among unpinned slots not hit,
      // one wavefront minimum per miss over packed (key + 2, slot)
      for (int c = lane; c < S; c += 64) s_ref[c] = 0;
      if (uact && sl >= 0) s_ref[sl] = 1;
      constexpr int SPL = kMaxSlots / 64;
      uint64_t ck[SPL];
#pragma unroll
      for (int q = 0; q < SPL; ++q) {
        const int c = lane + 64 * q;
        ck[q] = (c >= Pn && c < S && !s_ref[c]) ? (((uint64_t)(s_key[c] + 2) << 11) | (uint64_t)c) : ~0ull;
      }
      int my_victim = -1;
      for (int i = 0; i < nmiss; ++i) {
        uint64_t loc = ~0ull;
#pragma unroll
        for (int q = 0; q < SPL; ++q) loc = ck[q] < loc ? ck[q] : loc;
        const uint64_t g = wave_reduce_u64<false>(loc);
#pragma unroll
        for (int q = 0; q < SPL; ++q)
          if (ck[q] == g) ck[q] = ~0ull;
        if (lane == i) my_victim = g == ~0ull ? -1 : (int)(g & 0x7FFull);
      }
      const int v = __shfl(my_victim, miss ? mrank : 0);
      int old = -1;
      if (miss) {
        if (v < 0 || v >= S) {
          // no victim (cannot happen while |U| <= S): read this expert from the
          // backing store, leave the maps alone, and make the fill skip it
          atomicOr(a.L.error, 4u);
          a.W.miss_src[mrank] = nullptr;
          a.W.miss_dst[mrank] = nullptr;
        } else {
          old = s_s2e[v];
          if (old >= E) {
            atomicOr(a.L.error, 2u);
            old = -1;
          }
          if (old >= 0) a.L.e2s[old] = -1;
          a.L.e2s[ue] = v;
          a.L.s2e[v] = ue;
          sl = v;
          sc_event ev;
          ev.step = t;
          ev.expert = ue;
          ev.slot = v;
          ev.evicted = old;
          ev.reserved = 0;
          a.L.events[(ev_head + (uint64_t)mrank) % (uint64_t)a.L.ev_cap] = ev;
          a.W.miss_src[mrank] = a.L.backing + (size_t)ue * B;
          a.W.miss_dst[mrank] = a.L.slots + (size_t)v * B;
        }
      }
      nevict = __popcll(__ballot(old >= 0));
    }
    // stamp the clock, publish slot pointers and the resident-first order
    if (uact) {
      a.W.uniq_order[miss ? nres + mrank : lane - mrank] = lane;
      if (sl >= 0) {
        a.L.key[sl] = t * (int64_t)(kCachedRows * k) + (int64_t)s_last[ue];
        a.W.uniq_ptr[lane] = a.L.slots + (size_t)sl * B;
      } else {
        a.W.uniq_ptr[lane] = a.L.backing + (size_t)ue * B;
      }
    }
  } else if (uact) {
    // bypass: resident experts from their slots, the others read in place from the backing store
    a.W.uniq_ptr[lane] = sl >= 0 ? a.L.slots + (size_t)sl * B : a.L.backing + (size_t)ue * B;
    a.W.uniq_order[lane] = lane;
  }
  if (uact) a.W.uniq_expert[lane] = ue;

  // picks grouped by unique expert (CSR), ascending pick order
  if (U == P) {
    if (act) {
      a.W.pick_u[lane] = lane;
      a.W.uniq_picks[lane] = lane;
      a.W.uniq_off[lane] = lane;
    }
  } else {
    const int up = act ? s_uidx[e] : -1;
    int r = 0, c = 0;
    for (int u = 0; u < U; ++u) {
      const uint64_t m = __ballot(up == u);
      if (up == u) r = __popcll(m & below);
      if (lane == u) c = __popcll(m);
    }
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int ex = incl - c;
    const int base = __shfl(ex, up >= 0 ? up : 0);
    if (act) {
      a.W.pick_u[lane] = up;
      a.W.uniq_picks[base + r] = lane;
    }
    if (uact) a.W.uniq_off[lane] = ex;
  }

  if (lane == 0) {
    a.W.uniq_off[U] = P;
    a.W.hdr[H_UNIQUE] = U;
    a.W.hdr[H_MISS] = bypass ? 0 : nmiss;
    a.W.hdr[H_BYPASS] = bypass ? 1 : 0;
    a.W.hdr[H_ROWS] = M;
    a.W.hdr[H_RESIDENT] = U - nmiss;
    a.W.hdr[H_STAGED] = 0;
    cnt[C_STEPS] += 1;
    if (bypass) {
      cnt[C_BYPASS] += 1;
      cnt[C_BYPASS_BYTES] += (uint64_t)nmiss * (uint64_t)B;
    } else {
      cnt[C_PICKS] += (uint64_t)P;
      cnt[C_LOOKUPS] += (uint64_t)U;
      cnt[C_HITS] += (uint64_t)(U - nmiss);
      cnt[C_MISSES] += (uint64_t)nmiss;
      cnt[C_EVICT] += (uint64_t)nevict;
      cnt[C_FILLED] += (uint64_t)nmiss * (uint64_t)B;
      *a.L.ev_head = ev_head + (uint64_t)nmiss;
    }
#pragma unroll
    for (int c = 0; c < C_N; ++c) a.L.counters[c] = cnt[c];
    *a.L.step = t + 1;
  }
}

template <int EPL, int NT>
__global__ __launch_bounds__(NT) void k_route_remap(RouteArgs a) {
  constexpr int SPT = kMaxSlots / NT;   // slots per thread
  constexpr int XPT = kMaxExperts / NT; // experts per thread
  __shared__ __attribute__((aligned(16))) int s_pick[kMaxPicks];
  __shared__ int s_first[kMaxExperts];   // first pick position per expert; later pick counts
  __shared__ int s_last[kMaxExperts];
  __shared__ int s_uidx[kMaxExperts];
  __shared__ int s_uexp[kMaxExperts];
  __shared__ int s_uslot[kMaxExperts];
  __shared__ int s_umiss[kMaxExperts];   // miss rank per unique (-1 - rank among resident ones); later CSR offsets
  __shared__ int s_victim[kMaxSlots];
  __shared__ int s_e2s[kMaxExperts];     // snapshot of the slot map
  __shared__ int s_s2e[kMaxSlots];
  __shared__ long long s_key[kMaxSlots]; // snapshot of the clock, then candidate keys
  __shared__ uint8_t s_ref[kMaxSlots];
  __shared__ int s_wc[NT / 64];
  __shared__ unsigned long long s_wmin[NT / 64];
  __shared__ int s_nevict;
  __shared__ long long s_t;
  __shared__ unsigned long long s_evh;

  span_start(a.span);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.sh.E, k = a.sh.k, M = a.M, S = a.L.S;
  const int P = M * k;
  // The clock and the event head are read by one thread and passed on
  // through LDS once the rows are routed: a uniform value loaded here would
  // be moved to scalar registers at once, making every later load wait for it.
  uint64_t cnt[C_N];
  int64_t t0 = 0;
  uint64_t evh0 = 0;
  if (tid == 0) {
#pragma unroll
    for (int c = 0; c < C_N; ++c) cnt[c] = a.L.counters[c];
    t0 = *a.L.step;
    evh0 = *a.L.ev_head;
  }

  // Layer state and the first logits rows are loaded up front; the state
  // goes to LDS once the rows are routed, so the two latencies overlap.
  int r_e2s[XPT], r_s2e[SPT];
  int64_t r_key[SPT];
#pragma unroll
  for (int q = 0; q < XPT; ++q) {
    const int e = tid + q * NT;
    r_e2s[q] = e < E ? a.L.e2s[e] : -1;
  }
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    const int sl = tid + q * NT;
    r_s2e[q] = sl < S ? a.L.s2e[sl] : -1;
    r_key[q] = sl < S ? a.L.key[sl] : -1;
  }

  // ---- router: one row per wavefront, up to four rows' logits in flight ----
  constexpr int NW = NT / 64;
  constexpr int RD = 4;                         // rows in flight per wavefront
  float zr[RD][EPL];
#pragma unroll
  for (int d = 0; d < RD; ++d)
    if (wave + d * NW < M) load_row<EPL>(a.logits + (size_t)(wave + d * NW) * E, E, lane, zr[d]);
  for (int m0 = wave; m0 < M; m0 += RD * NW) {
#pragma unroll
    for (int d = 0; d < RD; ++d) {
      const int m = m0 + d * NW;
      if (m >= M) break;
      int my_e;
      float zj;
      route_row<EPL>(zr[d], E, k, lane, &my_e, &zj);
      if (m + RD * NW < M) load_row<EPL>(a.logits + (size_t)(m + RD * NW) * E, E, lane, zr[d]);
      const float w = pick_weight(zj, k, lane);
      if (lane < k) {
        s_pick[m * k + lane] = my_e;
        a.W.pick_expert[m * k + lane] = my_e;
        a.W.pick_w[m * k + lane] = w;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < XPT; ++q) {
    const int e = tid + q * NT;
    if (e < E) {
      s_e2s[e] = r_e2s[q];
      s_first[e] = INT_MAX;
      s_last[e] = -1;
    }
  }
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    const int sl = tid + q * NT;
    if (sl < S) {
      s_s2e[sl] = r_s2e[q];
      s_key[sl] = (long long)r_key[q];
    }
  }
  if (tid == 0) {
    s_nevict = 0;
    s_t = t0;
    s_evh = evh0;
  }
  __syncthreads();
  const int64_t t = s_t;
  const uint64_t ev_head = s_evh;
  if (P <= 64 && M <= kCachedRows) {
    if (wave == 0) remap_small(a, M, P, s_pick, s_first, s_last, s_uidx, s_uexp, s_e2s, s_s2e, s_key, s_ref, t,
                               ev_head, cnt);
    span_end(a.span);
    return;
  }

  // ---- unique experts in first-occurrence order ----------------------------
  for (int p = tid; p < P; p += NT) {
    atomicMin(&s_first[s_pick[p]], p);
    atomicMax(&s_last[s_pick[p]], p);
  }
  __syncthreads();
  int U = 0;
  for (int base = 0; base < P; base += NT) {
    const int p = base + tid;
    const int e = p < P ? s_pick[p] : 0;
    const bool f = p < P && s_first[e] == p;
    int tot;
    const int r = block_rank<NT>(f, s_wc, &tot);
    if (f) {
      s_uexp[U + r] = e;
      s_uidx[e] = U + r;
    }
    U += tot;
  }
  __syncthreads();

  const int64_t B = a.sh.blob;
  const int Pn = a.L.P;
  // ---- residency against the slot map (bypass steps use it too) -----------
  for (int u = tid; u < U; u += NT) {
    int sl = s_e2s[s_uexp[u]];
    if (sl < -1 || sl >= S) {
      atomicOr(a.L.error, 1u);
      sl = -1;
    }
    s_uslot[u] = sl;
  }
  __syncthreads();
  int nmiss = 0, npin = 0;
  for (int base = 0; base < U; base += NT) {
    const int u = base + tid;
    const bool ms = u < U && s_uslot[u] < 0;
    const bool pn = u < U && s_uslot[u] >= 0 && s_uslot[u] < Pn;
    int tot, tot_pin;
    const int r = block_rank<NT>(ms, s_wc, &tot);
    (void)block_rank<NT>(pn, s_wc, &tot_pin);
    // a miss stores its rank among misses; a resident expert -1 - its rank
    // among resident ones (r counts the misses before u in either case)
    if (u < U) s_umiss[u] = ms ? nmiss + r : -1 - (u - (nmiss + r));
    nmiss += tot;
    npin += tot_pin;
  }
  __syncthreads();
  const bool bypass = (M > kCachedRows) || (U - npin > S - Pn);
  if (!bypass) {
    if (nmiss > 0) {
      // ---- victims: the nmiss least (key, slot) among slots not hit ---------
      for (int sl = tid; sl < S; sl += NT) s_ref[sl] = 0;
      __syncthreads();
      for (int u = tid; u < U; u += NT)
        if (s_uslot[u] >= 0) s_ref[s_uslot[u]] = 1;
      __syncthreads();
      if (nmiss <= 8) {
        // a few misses: repeated block minimum over packed (key + 2, slot);
        // keys are >= -1, so a candidate packs to >= 2^11 and ~0 means "none"
        uint64_t ck[SPT];
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
          const int sl = tid + q * NT;
          ck[q] = (sl >= Pn && sl < S && !s_ref[sl]) ? (((uint64_t)(s_key[sl] + 2) << 11) | (uint64_t)sl) : ~0ull;
        }
        for (int i = 0; i < nmiss; ++i) {
          uint64_t loc = ~0ull;
#pragma unroll
          for (int q = 0; q < SPT; ++q) loc = ck[q] < loc ? ck[q] : loc;
          const uint64_t wm = wave_reduce_u64<false>(loc);
          if (lane == 0) s_wmin[wave] = wm;
          __syncthreads();
          uint64_t g = s_wmin[0];
#pragma unroll
          for (int w = 1; w < NT / 64; ++w) g = s_wmin[w] < g ? s_wmin[w] : g;
#pragma unroll
          for (int q = 0; q < SPT; ++q)
            if (ck[q] == g) ck[q] = ~0ull;
          if (tid == 0) s_victim[i] = g == ~0ull ? -1 : (int)(g & 0x7FFull);
          __syncthreads();
        }
      } else {
        // many misses: rank every candidate by (key, slot)
        for (int sl = tid; sl < S; sl += NT) {
          if (s_ref[sl] || sl < Pn) s_key[sl] = (long long)LLONG_MAX;
          s_victim[sl] = -1;
        }
        __syncthreads();
        for (int sl = tid; sl < S; sl += NT) {
          if (s_ref[sl] || sl < Pn) continue;
          const long long ks = s_key[sl];
          int r = 0;
          for (int s2 = 0; s2 < S; ++s2) {
            const long long k2 = s_key[s2];
            r += (k2 < ks) || (k2 == ks && s2 < sl);
          }
          if (r < nmiss) s_victim[r] = sl;
        }
      }
      __syncthreads();
      // ---- apply the misses: evict, remap, log, queue the fills ------------
      for (int u = tid; u < U; u += NT) {
        const int i = s_umiss[u];
        if (i < 0) continue;
        const int e = s_uexp[u];
        const int sl = s_victim[i];
        if (sl < 0 || sl >= S) {
          // no victim (cannot happen while |U| <= S): read this expert from the
          // backing store, leave the maps alone, and make the fill skip it
          atomicOr(a.L.error, 4u);
          s_uslot[u] = -1;
          a.W.miss_src[i] = nullptr;
          a.W.miss_dst[i] = nullptr;
          continue;
        }
        int old = s_s2e[sl];
        if (old >= E) {
          atomicOr(a.L.error, 2u);
          old = -1;
        }
        if (old >= 0) {
          a.L.e2s[old] = -1;
          atomicAdd(&s_nevict, 1);
        }
        a.L.e2s[e] = sl;
        a.L.s2e[sl] = e;
        s_uslot[u] = sl;
        sc_event ev;
        ev.step = t;
        ev.expert = e;
        ev.slot = sl;
        ev.evicted = old;
        ev.reserved = 0;
        a.L.events[(ev_head + (uint64_t)i) % (uint64_t)a.L.ev_cap] = ev;
        a.W.miss_src[i] = a.L.backing + (size_t)e * B;
        a.W.miss_dst[i] = a.L.slots + (size_t)sl * B;
      }
      __syncthreads();
    }
    // ---- stamp the clock, publish slot pointers and the resident-first order
    const int nres = U - nmiss;
    for (int u = tid; u < U; u += NT) {
      const int sl = s_uslot[u], i = s_umiss[u];
      a.W.uniq_order[i >= 0 ? nres + i : -1 - i] = u;
      if (sl < 0) {
        a.W.uniq_ptr[u] = a.L.backing + (size_t)s_uexp[u] * B;
        continue;
      }
      a.L.key[sl] = t * (int64_t)(kCachedRows * k) + (int64_t)s_last[s_uexp[u]];
      a.W.uniq_ptr[u] = a.L.slots + (size_t)sl * B;
    }
  } else if (staged_step(a.W, M)) {
    // staged prefill: resident experts from their slots; the i-th non-resident
    // one is copied into staging blob i % G by group i / G.  uniq_order lists
    // the resident experts, then the staged ones in staging order.
    const int G = a.W.stage_n, nres = U - nmiss;
    for (int u = tid; u < U; u += NT) {
      const int sl = s_uslot[u], i = s_umiss[u];
      if (sl >= 0) {
        a.W.uniq_ptr[u] = a.L.slots + (size_t)sl * B;
        a.W.uniq_order[-1 - i] = u;
      } else {
        uint8_t* dst = a.W.stage + (size_t)(i % G) * B;
        a.W.uniq_ptr[u] = dst;
        a.W.miss_src[i] = a.L.backing + (size_t)s_uexp[u] * B;
        a.W.miss_dst[i] = dst;
        a.W.uniq_order[nres + i] = u;
      }
    }
  } else {
    // bypass: resident experts from their slots, the others read in place from the backing store
    for (int u = tid; u < U; u += NT) {
      const int sl = s_uslot[u];
      a.W.uniq_ptr[u] = sl >= 0 ? a.L.slots + (size_t)sl * B : a.L.backing + (size_t)s_uexp[u] * B;
      a.W.uniq_order[u] = u;
    }
  }
  for (int u = tid; u < U; u += NT) a.W.uniq_expert[u] = s_uexp[u];

  // ---- picks grouped by unique expert (CSR), ascending pick order ---------
  if (U == P) {
    // every pick is its own unique expert, in pick order
    for (int p = tid; p < P; p += NT) {
      a.W.pick_u[p] = p;
      a.W.uniq_picks[p] = p;
      a.W.uniq_off[p] = p;
    }
  } else {
    int* s_cnt = s_first;   // free after the unique pass
    int* s_off = s_umiss;   // free after the miss pass
    __syncthreads();
    for (int u = tid; u < U; u += NT) s_cnt[u] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += NT) {
      const int u = s_uidx[s_pick[p]];
      atomicAdd(&s_cnt[u], 1);
      a.W.pick_u[p] = u;
    }
    __syncthreads();
    block_scan<NT>(s_cnt, s_off, U, s_wc);
    for (int p = tid; p < P; p += NT) {
      const int e = s_pick[p];
      // rank of p among the picks of e: earlier picks of e, four per LDS read
      int r = 0, q = 0;
      const int4* pk4 = reinterpret_cast<const int4*>(s_pick);
      for (; q + 4 <= p; q += 4) {
        const int4 v = pk4[q >> 2];
        r += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
      }
      for (; q < p; ++q) r += s_pick[q] == e;
      a.W.uniq_picks[s_off[s_uidx[e]] + r] = p;
    }
    for (int u = tid; u < U; u += NT) a.W.uniq_off[u] = s_off[u];
  }

  if (tid == 0) {
    a.W.uniq_off[U] = P;
    a.W.hdr[H_UNIQUE] = U;
    a.W.hdr[H_MISS] = bypass ? 0 : nmiss;     // a bypass step fills nothing
    a.W.hdr[H_BYPASS] = bypass ? 1 : 0;
    a.W.hdr[H_ROWS] = M;
    a.W.hdr[H_RESIDENT] = U - nmiss;
    a.W.hdr[H_STAGED] = bypass && staged_step(a.W, M) ? nmiss : 0;
    cnt[C_STEPS] += 1;
    if (bypass) {
      cnt[C_BYPASS] += 1;
      cnt[C_BYPASS_BYTES] += (uint64_t)nmiss * (uint64_t)B;   // its non-resident experts
    } else {
      cnt[C_PICKS] += (uint64_t)P;
      cnt[C_LOOKUPS] += (uint64_t)U;
      cnt[C_HITS] += (uint64_t)(U - nmiss);
      cnt[C_MISSES] += (uint64_t)nmiss;
      cnt[C_EVICT] += (uint64_t)s_nevict;
      cnt[C_FILLED] += (uint64_t)nmiss * (uint64_t)B;
      *a.L.ev_head = ev_head + (uint64_t)nmiss;
    }
#pragma unroll
    for (int c = 0; c < C_N; ++c) a.L.counters[c] = cnt[c];
    *a.L.step = t + 1;
  }
  span_end(a.span);
}

// One-row steps on one wavefront.  A row's k picks are distinct experts, so
// the unique experts are the picks in rank order, every expert has one pick
// and the CSR lists are the identity; with k <= S - P the step cannot bypass.
// Lane j < k owns pick j.  Without block barriers or the general kernel's
// unique and CSR passes, the step's critical path is the logits load, the
// top-k rounds and the stores; the bookkeeping rules and every value written
// are the general kernel's.
template <int EPL, int SPL>
__global__ __launch_bounds__(64) void k_route_one(RouteArgs a) {
  __shared__ int s_e2s[kMaxExperts];
  __shared__ int s_s2e[kMaxSlots];
  __shared__ uint8_t s_ref[kMaxSlots];

  span_start(a.span);
  const int lane = threadIdx.x;
  const int E = a.sh.E, k = a.sh.k, S = a.L.S, Pn = a.L.P;
  const int64_t t = *a.L.step;
  const uint64_t ev_head = *a.L.ev_head;
  uint64_t cnt[C_N];
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < C_N; ++c) cnt[c] = a.L.counters[c];
  }
  // Every load is issued unconditionally (indices clamped into range, the
  // values past the end replaced afterwards): loads under a branch let the
  // compiler wait for each one inside its branch, one memory latency apiece.
  int r_e2s[EPL], r_s2e[SPL];
  int64_t r_key[SPL];
  float z[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = min(lane + 64 * q, E - 1);
    r_e2s[q] = a.L.e2s[e];
    z[q] = a.logits[e];
  }
#pragma unroll
  for (int q = 0; q < SPL; ++q) {
    const int sl = min(lane + 64 * q, S - 1);
    r_s2e[q] = a.L.s2e[sl];
    r_key[q] = a.L.key[sl];
  }
#pragma unroll
  for (int q = 0; q < EPL; ++q)
    if (lane + 64 * q >= E) {
      r_e2s[q] = -1;
      z[q] = 0.0f;
    }
#pragma unroll
  for (int q = 0; q < SPL; ++q)
    if (lane + 64 * q >= S) {
      r_s2e[q] = -1;
      r_key[q] = -1;
    }
  int e;
  float zj;
  route_row<EPL>(z, E, k, lane, &e, &zj);
  const float w = pick_weight(zj, k, lane);
  const bool act = lane < k;
#pragma unroll
  for (int q = 0; q < EPL; ++q)
    if (lane + 64 * q < E) s_e2s[lane + 64 * q] = r_e2s[q];
#pragma unroll
  for (int q = 0; q < SPL; ++q)
    if (lane + 64 * q < S) {
      s_s2e[lane + 64 * q] = r_s2e[q];
      s_ref[lane + 64 * q] = 0;
    }
  __syncthreads();

  // residency; a miss's rank among misses, a hit's among hits, in pick order
  int sl = act ? s_e2s[e] : -1;
  if (act && (sl < -1 || sl >= S)) {
    atomicOr(a.L.error, 1u);
    sl = -1;
  }
  const bool miss = act && sl < 0;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t mmask = __ballot(miss);
  const int nmiss = __popcll(mmask);
  const int mrank = __popcll(mmask & below);
  const int nres = k - nmiss;
  int nevict = 0;
  if (nmiss > 0) {
    // victims: the nmiss least (key, slot) among unpinned slots not hit;
    // packed as (key + 2, slot) with keys >= -1, ~0 meaning "none"
    if (act && !miss) s_ref[sl] = 1;
    __syncthreads();
    uint64_t ck[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
      const int c = lane + 64 * q;
      ck[q] = (c >= Pn && c < S && !s_ref[c]) ? (((uint64_t)(r_key[q] + 2) << 11) | (uint64_t)c) : ~0ull;
    }
    int my_victim = -1;
    for (int i = 0; i < nmiss; ++i) {
      uint64_t loc = ~0ull;
#pragma unroll
      for (int q = 0; q < SPL; ++q) loc = ck[q] < loc ? ck[q] : loc;
      const uint64_t g = wave_reduce_u64<false>(loc);
#pragma unroll
      for (int q = 0; q < SPL; ++q)
        if (ck[q] == g) ck[q] = ~0ull;
      if (lane == i) my_victim = g == ~0ull ? -1 : (int)(g & 0x7FFull);
    }
    const int v = __shfl(my_victim, miss ? mrank : 0);
    int old = -1;
    if (miss) {
      if (v < 0 || v >= S) {
        // no victim (cannot happen while the maps are consistent): read this
        // expert from the backing store and make the fill skip it
        atomicOr(a.L.error, 4u);
        a.W.miss_src[mrank] = nullptr;
        a.W.miss_dst[mrank] = nullptr;
      } else {
        old = s_s2e[v];
        if (old >= E) {
          atomicOr(a.L.error, 2u);
          old = -1;
        }
        if (old >= 0) a.L.e2s[old] = -1;
        a.L.e2s[e] = v;
        a.L.s2e[v] = e;
        sl = v;
        sc_event ev;
        ev.step = t;
        ev.expert = e;
        ev.slot = v;
        ev.evicted = old;
        ev.reserved = 0;
        a.L.events[(ev_head + (uint64_t)mrank) % (uint64_t)a.L.ev_cap] = ev;
        a.W.miss_src[mrank] = a.L.backing + (size_t)e * a.sh.blob;
        a.W.miss_dst[mrank] = a.L.slots + (size_t)v * a.sh.blob;
      }
    }
    nevict = __popcll(__ballot(old >= 0));
  }
  if (act) {
    const int64_t B = a.sh.blob;
    a.W.pick_expert[lane] = e;
    a.W.pick_w[lane] = w;
    a.W.uniq_order[miss ? nres + mrank : lane - mrank] = lane;
    if (sl >= 0) {
      a.L.key[sl] = t * (int64_t)(kCachedRows * k) + (int64_t)lane;
      a.W.uniq_ptr[lane] = a.L.slots + (size_t)sl * B;
    } else {
      a.W.uniq_ptr[lane] = a.L.backing + (size_t)e * B;
    }
    a.W.uniq_expert[lane] = e;
    a.W.pick_u[lane] = lane;
    a.W.uniq_picks[lane] = lane;
    a.W.uniq_off[lane] = lane;
  }
  if (lane == 0) {
    a.W.uniq_off[k] = k;
    a.W.hdr[H_UNIQUE] = k;
    a.W.hdr[H_MISS] = nmiss;
    a.W.hdr[H_BYPASS] = 0;
    a.W.hdr[H_ROWS] = 1;
    a.W.hdr[H_RESIDENT] = nres;
    a.W.hdr[H_STAGED] = 0;
    cnt[C_STEPS] += 1;
    cnt[C_PICKS] += (uint64_t)k;
    cnt[C_LOOKUPS] += (uint64_t)k;
    cnt[C_HITS] += (uint64_t)nres;
    cnt[C_MISSES] += (uint64_t)nmiss;
    cnt[C_EVICT] += (uint64_t)nevict;
    cnt[C_FILLED] += (uint64_t)nmiss * (uint64_t)a.sh.blob;
    *a.L.ev_head = ev_head + (uint64_t)nmiss;
#pragma unroll
    for (int c = 0; c < C_N; ++c) a.L.counters[c] = cnt[c];
    *a.L.step = t + 1;
  }
  span_end(a.span);
}

}  // namespace

template <int NT>
static hipError_t launch_route_nt(int epl, const RouteArgs& a, hipStream_t st, KEvents ev) {
  const dim3 g(1), b(NT);
  if (epl <= 1) return sc_launch(k_route_remap<1, NT>, g, b, st, ev, a);
  if (epl <= 2) return sc_launch(k_route_remap<2, NT>, g, b, st, ev, a);
  if (epl <= 4) return sc_launch(k_route_remap<4, NT>, g, b, st, ev, a);
  if (epl <= 8) return sc_launch(k_route_remap<8, NT>, g, b, st, ev, a);
  return sc_launch(k_route_remap<16, NT>, g, b, st, ev, a);
}

template <int SPL>
static hipError_t launch_route_one_spl(int epl, const RouteArgs& a, hipStream_t st, KEvents ev) {
  const dim3 g(1), b(64);
  if (epl <= 1) return sc_launch(k_route_one<1, SPL>, g, b, st, ev, a);
  if (epl <= 2) return sc_launch(k_route_one<2, SPL>, g, b, st, ev, a);
  if (epl <= 4) return sc_launch(k_route_one<4, SPL>, g, b, st, ev, a);
  if (epl <= 8) return sc_launch(k_route_one<8, SPL>, g, b, st, ev, a);
  return sc_launch(k_route_one<16, SPL>, g, b, st, ev, a);
}

hipError_t launch_route(const Shape& sh, const LayerDev& L, const Workspace& W,
                        const float* logits, int M, hipStream_t st, KEvents ev) {
  RouteArgs a;
  a.sh = sh;
  a.L = L;
  a.W = W;
  a.logits = logits;
  a.M = M;
  a.span = ev.span_for(1);
  const int epl = (sh.E + 63) / 64;
  if (M == 1 && sh.k <= kRouteOneMaxK && sh.k <= L.S - L.P)
    return L.S <= 128 ? launch_route_one_spl<2>(epl, a, st, ev)
         : L.S <= 256 ? launch_route_one_spl<4>(epl, a, st, ev) : launch_route_one_spl<16>(epl, a, st, ev);
  if (M * sh.k >= kRouteWidePicks) return launch_route_nt<kRouteWideThreads>(epl, a, st, ev);
  return launch_route_nt<kRouteThreads>(epl, a, st, ev);
}

}  // namespace sc
