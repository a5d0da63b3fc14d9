// Router top-k, routing weights and the fused expert-id -> slot remap with
// batch-LRU victim choice, in one workgroup of four wavefronts.
//
// Method: the slot cache of page "GLM 5.3 Testing: HBM Expert Allocation"
// (section "What the slot cache is": ids are mapped to slots on the device
// before the expert launch, a miss takes the least-recently-used victim slot,
// more than 16 rows bypass), replacing the "dozen tiny torch ops" of that
// page's section "The build" with one kernel.  Occupancy is a live LRU clock
// (page "GB300 GLM 5.3 Testing", section "Expert allocation vs a cache").
// Router ties break by a stable expert order (page "TensorFold GLM-5.3
// explained", exact-decoding rule).
//
// Bookkeeping rules (the pages leave these open; one launch maps a whole step,
// so they are per step):
//   P  = the M*k picks in (row, rank) order, p = 0..M*k-1
//   U  = unique experts of P in first-occurrence order; hits = resident ones
//   bypass when M > 16 or |U| > S: the cache is untouched, blobs are read
//          from the backing store, the step counter still advances
//   candidates = slots not holding a hit, ascending (key, slot); empty slots
//          have key -1; the i-th miss (first-occurrence order) takes the i-th
//   key[slot(e)] = t * (16 * k) + last position of e in P, for every e in U
#include "internal.h"

#include <climits>

namespace sc {
namespace {

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Exclusive rank of `pred` among the block's threads in thread order.
__device__ __forceinline__ int block_rank(bool pred, int* s_wc, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t mask = __ballot(pred);
  int in_wave = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) s_wc[wave] = __popcll(mask);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) {
    int c = s_wc[w];
    if (w < wave) base += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + in_wave;
}

// Exclusive scan of s_in[0..n) into s_out (n <= 4 * blockDim); returns the total.
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
  for (int w = 0; w < kRouteThreads / 64; ++w) {
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
};

__global__ __launch_bounds__(kRouteThreads) void k_route_remap(RouteArgs a) {
  __shared__ int s_pick[kMaxPicks];
  __shared__ int s_first[kMaxExperts];
  __shared__ int s_last[kMaxExperts];
  __shared__ int s_uidx[kMaxExperts];
  __shared__ int s_uexp[kMaxExperts];
  __shared__ int s_uslot[kMaxExperts];
  __shared__ int s_umiss[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_ref[kMaxSlots];
  __shared__ int s_victim[kMaxSlots];
  __shared__ long long s_ckey[kMaxSlots];
  __shared__ int s_wc[kRouteThreads / 64];
  __shared__ int s_nevict;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.sh.E, k = a.sh.k, M = a.M, S = a.L.S;
  const int P = M * k;
  const int64_t t = *a.L.step;
  const uint64_t ev_head = *a.L.ev_head;

  // ---- router: one row per wavefront -------------------------------------
  constexpr int EPL = kMaxExperts / 64;
  const int epl = (E + 63) / 64;
  for (int m = wave; m < M; m += kRouteThreads / 64) {
    const float* z = a.logits + (size_t)m * E;
    uint64_t keys[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int e = lane + 64 * i;
      keys[i] = (i < epl && e < E) ? order_key(z[e], e) : 0ull;
    }
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t loc = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) loc = keys[i] > loc ? keys[i] : loc;
      uint64_t best = wave_max_u64(loc);
      int eb = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i == eb) keys[i] = 0ull;
      if (lane == j) my_e = eb;
    }
    // weights: softmax over the k chosen logits (limits for non-finite picks)
    const bool act = lane < k;
    float zj = act ? z[my_e] : 0.0f;
    const bool is_nan = zj != zj;
    const bool pinf = act && zj == INFINITY;
    const int npinf = __popcll(__ballot(pinf));
    const float z0 = __shfl(zj, 0);
    float w;
    if (npinf > 0) {
      w = pinf ? 1.0f / (float)npinf : 0.0f;
    } else if (z0 != z0 || z0 == -INFINITY) {
      w = 1.0f / (float)k;
    } else {
      float ex = (act && !is_nan) ? expf(zj - z0) : 0.0f;
      float sum = wave_sum_f32(ex);
      w = ex / sum;
    }
    if (act) {
      s_pick[m * k + lane] = my_e;
      a.W.pick_expert[m * k + lane] = my_e;
      a.W.pick_w[m * k + lane] = w;
    }
  }
  for (int e = tid; e < E; e += kRouteThreads) {
    s_first[e] = INT_MAX;
    s_last[e] = -1;
  }
  if (tid == 0) s_nevict = 0;
  __syncthreads();

  // ---- unique experts in first-occurrence order ----------------------------
  for (int p = tid; p < P; p += kRouteThreads) {
    atomicMin(&s_first[s_pick[p]], p);
    atomicMax(&s_last[s_pick[p]], p);
  }
  __syncthreads();
  int U = 0;
  for (int base = 0; base < P; base += kRouteThreads) {
    int p = base + tid;
    int e = p < P ? s_pick[p] : 0;
    bool f = p < P && s_first[e] == p;
    int tot;
    int r = block_rank(f, s_wc, &tot);
    if (f) {
      s_uexp[U + r] = e;
      s_uidx[e] = U + r;
    }
    U += tot;
  }
  __syncthreads();

  const bool bypass = (M > kCachedRows) || (U > S);
  const int64_t B = a.sh.blob;
  int nmiss = 0;
  if (!bypass) {
    // ---- hit test against the slot map ------------------------------------
    for (int u = tid; u < U; u += kRouteThreads) {
      int s = a.L.e2s[s_uexp[u]];
      if (s < -1 || s >= S) {
        atomicOr(a.L.error, 1u);
        s = -1;
      }
      s_uslot[u] = s;
    }
    __syncthreads();
    for (int base = 0; base < U; base += kRouteThreads) {
      int u = base + tid;
      bool ms = u < U && s_uslot[u] < 0;
      int tot;
      int r = block_rank(ms, s_wc, &tot);
      if (u < U) s_umiss[u] = ms ? nmiss + r : -1;
      nmiss += tot;
    }
    __syncthreads();
    if (nmiss > 0) {
      // ---- victims: candidates ranked by (key, slot) -----------------------
      for (int s = tid; s < S; s += kRouteThreads) s_ref[s] = 0;
      __syncthreads();
      for (int u = tid; u < U; u += kRouteThreads)
        if (s_uslot[u] >= 0) s_ref[s_uslot[u]] = 1;
      __syncthreads();
      for (int s = tid; s < S; s += kRouteThreads)
        s_ckey[s] = s_ref[s] ? (long long)LLONG_MAX : (long long)a.L.key[s];
      __syncthreads();
      for (int s = tid; s < S; s += kRouteThreads) {
        if (s_ref[s]) continue;
        const long long ks = s_ckey[s];
        int r = 0;
        for (int s2 = 0; s2 < S; ++s2) {
          long long k2 = s_ckey[s2];
          r += (k2 < ks) || (k2 == ks && s2 < s);
        }
        if (r < nmiss) s_victim[r] = s;
      }
      __syncthreads();
      // ---- apply the misses: evict, remap, log, queue the fills ------------
      for (int u = tid; u < U; u += kRouteThreads) {
        int i = s_umiss[u];
        if (i < 0) continue;
        int e = s_uexp[u];
        int s = s_victim[i];
        int old = a.L.s2e[s];
        if (old >= E) {
          atomicOr(a.L.error, 2u);
          old = -1;
        }
        if (old >= 0) {
          a.L.e2s[old] = -1;
          atomicAdd(&s_nevict, 1);
        }
        a.L.e2s[e] = s;
        a.L.s2e[s] = e;
        s_uslot[u] = s;
        sc_event ev;
        ev.step = t;
        ev.expert = e;
        ev.slot = s;
        ev.evicted = old;
        ev.reserved = 0;
        a.L.events[(ev_head + (uint64_t)i) % (uint64_t)a.L.ev_cap] = ev;
        a.W.miss_src[i] = a.L.backing + (size_t)e * B;
        a.W.miss_dst[i] = a.L.slots + (size_t)s * B;
      }
      __syncthreads();
    }
    // ---- stamp the clock, publish slot pointers ----------------------------
    for (int u = tid; u < U; u += kRouteThreads) {
      int s = s_uslot[u];
      a.L.key[s] = t * (int64_t)(kCachedRows * k) + (int64_t)s_last[s_uexp[u]];
      a.W.uniq_ptr[u] = a.L.slots + (size_t)s * B;
    }
  } else {
    for (int u = tid; u < U; u += kRouteThreads)
      a.W.uniq_ptr[u] = a.L.backing + (size_t)s_uexp[u] * B;
  }
  for (int u = tid; u < U; u += kRouteThreads) {
    int e = s_uexp[u];
    a.W.uniq_expert[u] = e;
    a.W.uniq_gs[2 * u] = a.L.gs[2 * e];
    a.W.uniq_gs[2 * u + 1] = a.L.gs[2 * e + 1];
    s_cnt[u] = 0;
  }
  __syncthreads();

  // ---- picks grouped by unique expert (CSR), ascending pick order ---------
  for (int p = tid; p < P; p += kRouteThreads) {
    int u = s_uidx[s_pick[p]];
    atomicAdd(&s_cnt[u], 1);
    a.W.pick_u[p] = u;
  }
  __syncthreads();
  block_scan(s_cnt, s_off, U, s_wc);
  for (int p = tid; p < P; p += kRouteThreads) {
    const int e = s_pick[p];
    int r = 0;
    for (int q = 0; q < p; ++q) r += s_pick[q] == e;
    a.W.uniq_picks[s_off[s_uidx[e]] + r] = p;
  }
  for (int u = tid; u < U; u += kRouteThreads) a.W.uniq_off[u] = s_off[u];
  __syncthreads();

  if (tid == 0) {
    a.W.uniq_off[U] = P;
    a.W.hdr[H_UNIQUE] = U;
    a.W.hdr[H_MISS] = nmiss;
    a.W.hdr[H_BYPASS] = bypass ? 1 : 0;
    a.W.hdr[H_ROWS] = M;
    uint64_t* c = a.L.counters;
    c[C_STEPS] += 1;
    if (bypass) {
      c[C_BYPASS] += 1;
      c[C_BYPASS_BYTES] += (uint64_t)U * (uint64_t)B;
    } else {
      c[C_PICKS] += (uint64_t)P;
      c[C_LOOKUPS] += (uint64_t)U;
      c[C_HITS] += (uint64_t)(U - nmiss);
      c[C_MISSES] += (uint64_t)nmiss;
      c[C_EVICT] += (uint64_t)s_nevict;
      c[C_FILLED] += (uint64_t)nmiss * (uint64_t)B;
      *a.L.ev_head = ev_head + (uint64_t)nmiss;
    }
    *a.L.step = t + 1;
  }
}

}  // namespace

hipError_t launch_route(const Shape& sh, const LayerDev& L, const Workspace& W,
                        const float* logits, int M, hipStream_t st) {
  RouteArgs a;
  a.sh = sh;
  a.L = L;
  a.W = W;
  a.logits = logits;
  a.M = M;
  hipLaunchKernelGGL(k_route_remap, dim3(1), dim3(kRouteThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sc
