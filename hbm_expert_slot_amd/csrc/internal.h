// Internal definitions shared by the host runtime and the kernels of libslotcache.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "slotcache.h"

namespace sc {

constexpr int kMaxExperts = 1024;
constexpr int kMaxSlots = 1024;
constexpr int kMaxRows = 256;
constexpr int kMaxTopK = 32;
constexpr int kMaxPicks = 2048;        // max_rows * top_k
constexpr int kRouteThreads = 256;
constexpr int kGemvThreads = 256;
constexpr int kCachedRows = SC_BYPASS_ROWS;

enum Counter {
  C_STEPS = 0, C_BYPASS, C_PICKS, C_LOOKUPS, C_HITS, C_MISSES, C_EVICT, C_FILLED, C_BYPASS_BYTES, C_N
};

// Workspace header words.
// H_RESIDENT / H_STAGED: a staged prefill step's resident and staged unique experts.
enum Hdr { H_UNIQUE = 0, H_MISS = 1, H_BYPASS = 2, H_ROWS = 3, H_RESIDENT = 4, H_STAGED = 5, H_WORDS = 64 };

// Device view of one layer: its maps, clock, counters, event ring, slots,
// the backing bank it reads and that bank's global-scale table.
struct LayerDev {
  int32_t* e2s;            // [E]   slot of expert or -1
  int32_t* s2e;            // [S]   expert in slot or -1
  int64_t* key;            // [S]   LRU clock stamp, -1 = empty
  int64_t* step;           // step counter
  uint64_t* counters;      // [C_N]
  uint32_t* error;         // device error word
  uint64_t* ev_head;       // events ever logged
  sc_event* events;        // [ev_cap] ring
  uint8_t* slots;          // S blobs, stride blob_bytes
  const uint8_t* backing;  // device-mapped view of the host bank, E blobs
  const float* gs;         // [E][2] (w13, w2)
  int32_t S;
  int32_t ev_cap;
  int32_t P;               // pinned slots [0, P): fixed experts, never victims
};

// Per-call scratch shared by all layers of a handle.
struct Workspace {
  int32_t* hdr;                 // [H_WORDS]
  int32_t* pick_expert;         // [Pmax]  (row, rank) order
  float* pick_w;                // [Pmax]
  int32_t* pick_u;              // [Pmax]  unique index of each pick
  int32_t* uniq_expert;         // [Pmax]
  const uint8_t** uniq_ptr;     // [Pmax]  blob each unique expert is read from
  int32_t* uniq_off;            // [Pmax + 1] CSR offsets into uniq_picks
  int32_t* uniq_picks;          // [Pmax]  picks grouped by unique expert, ascending
  const uint8_t** miss_src;     // [Pmax]
  uint8_t** miss_dst;           // [Pmax]
  float* h;                     // [Pmax][I]  SiLU(gate) * up, per pick
  float* part;                  // [Pmax][H]  down projection, per pick
  int32_t* uniq_order;          // [Pmax]  the uniques found resident, then the others: misses in miss order
                                //         (cached step), staged ones in staging order (staged prefill);
                                //         unique order on other bypass steps
  uint8_t* stage;               // [stage_n] blobs: prefill staging area (null when stage_n == 0)
  int32_t stage_n;              // G, experts per prefill group (0: no staging)
};

// A step of M rows is staged when it is a prefill chunk and the workspace has
// a staging area.
__host__ __device__ inline bool staged_step(const Workspace& W, int M) { return M > kCachedRows && W.stage_n > 0; }
// Groups enqueued for a staged step: enough for min(M*k, E) staged experts.
inline int stage_groups(const Workspace& W, int M, int k, int E) {
  const int maxu = M * k < E ? M * k : E;
  return (maxu + W.stage_n - 1) / W.stage_n;
}

// Positions [lo, hi) of group `g` in uniq_order: the resident experts and the
// first G staged ones form group 0, staged ones g*G .. g*G+G-1 group g.
__device__ __forceinline__ void group_range(const int32_t* hdr, int g, int G, int& lo, int& hi) {
  const int nres = hdr[H_RESIDENT], ns = hdr[H_STAGED];
  const int end = ns < (g + 1) * G ? ns : (g + 1) * G;
  lo = g == 0 ? 0 : nres + g * G;
  hi = nres + end;
  if (hi < lo) hi = lo;
}

struct Shape {
  int32_t H, I, E, k;
  int64_t blob;                 // B_e
  int64_t off_w13s, off_w2c, off_w2s;   // part offsets inside a blob
};

inline Shape make_shape(int H, int I, int E, int k) {
  Shape s;
  s.H = H; s.I = I; s.E = E; s.k = k;
  int64_t w13c = (int64_t)2 * I * (H / 2);
  int64_t w13s = (int64_t)2 * I * (H / 16);
  int64_t w2c = (int64_t)H * (I / 2);
  int64_t w2s = (int64_t)H * (I / 16);
  s.off_w13s = w13c;
  s.off_w2c = w13c + w13s;
  s.off_w2s = w13c + w13s + w2c;
  s.blob = w13c + w13s + w2c + w2s;
  return s;
}

// Optional start/stop events of one launch (both null: a plain launch).  With
// events the kernel is launched through hipExtLaunchKernelGGL, which stamps
// the events at the kernel's own start and end.  `span`, when set, receives
// the launch's execution stamps (see span_start / span_end).
struct KEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  uint64_t* span = nullptr;
  int span_blocks = 0;       // blocks the span region holds
  // the stamps region for a launch of `blocks` blocks (null if it would not fit)
  uint64_t* span_for(long blocks) const { return blocks <= span_blocks ? span : nullptr; }
};

// Execution stamps of one launch, in ticks of the device's constant wall clock
// (s_memrealtime): block b writes its start to span[b * kSpanSlots] and each
// of its wavefronts w its end, after its memory operations have completed, to
// span[b * kSpanSlots + 1 + w].  Kernels of a timed step write them; the host
// keeps the stamps not older than the step's routing kernel start.
constexpr int kSpanSlots = 5;   // start + one end per wavefront (at most 4 per block)
// b: the block's index in the launch, or in its part of a launch whose blocks
// do two jobs (the stamps of each job go to a region of their own).
__device__ __forceinline__ void span_start(uint64_t* span, unsigned b) {
  if (span && threadIdx.x == 0) span[(size_t)b * kSpanSlots] = (uint64_t)wall_clock64();
}
__device__ __forceinline__ void span_end(uint64_t* span, unsigned b) {
  if (span) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wavefront's stores are done
    if ((threadIdx.x & 63) == 0)
      span[(size_t)b * kSpanSlots + 1 + (threadIdx.x >> 6)] = (uint64_t)wall_clock64();
  }
}
__device__ __forceinline__ void span_start(uint64_t* span) { span_start(span, blockIdx.x); }
__device__ __forceinline__ void span_end(uint64_t* span) { span_end(span, blockIdx.x); }

template <typename F, typename... Args>
inline hipError_t sc_launch(F kernel, dim3 grid, dim3 block, hipStream_t st, KEvents ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  return hipGetLastError();
}

// True when the gate/up (K = H) or down (K = I) kernels are compiled for K.
bool gemv_supported(int K, bool gateup);

// Enqueue the phases of one step.  Each returns hipSuccess or the launch error.
hipError_t launch_route(const Shape& sh, const LayerDev& L, const Workspace& W,
                        const float* logits, int M, hipStream_t st, KEvents ev);
// group: -1 for a whole step (the step's misses / all its unique experts),
// g >= 0 for group g of a staged prefill step.
hipError_t launch_fill(const Shape& sh, const Workspace& W, int group, hipStream_t st, KEvents ev);
// mfma: the matrix-core kernels serve M >= SC_MFMA_MIN_ROWS_GATEUP (gate/up) and
// SC_MFMA_MIN_ROWS_DOWN (down); off: the streaming kernels for every M.
hipError_t launch_gateup(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x, int M,
                         bool mfma, int group, hipStream_t st, KEvents ev);
// Overlapped fill of a one-row step (SC_FLAG_OVERLAP_FILL), two launches in
// place of launch_fill + launch_gateup.  The first shares its blocks between
// the copy of the step's misses (stamps in ev_fill's region) and the gate/up
// products of the experts the copy does not write (stamps in ev's region, and
// ev's events bracket the launch); the second computes the copied experts'
// gate/up once the copy is done (no stamps).  Both read the step's expert
// order from the remap: experts it found resident first, then the misses.
hipError_t launch_fill_gateup(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x,
                              hipStream_t st, KEvents ev_fill, KEvents ev);
hipError_t launch_gateup_filled(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x,
                                hipStream_t st);
hipError_t launch_down(const Shape& sh, const Workspace& W, const float* gs, int M, bool mfma, int group,
                       hipStream_t st, KEvents ev);
hipError_t launch_combine(const Shape& sh, const Workspace& W, float* y, int M, hipStream_t st,
                          KEvents ev);

}  // namespace sc
