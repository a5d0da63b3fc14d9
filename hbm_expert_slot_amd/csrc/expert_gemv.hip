// Miss fill, NVFP4 expert products and the weighted top-k combine.
//
// Pages: a miss copies the expert's weight row and scale row into its victim
// slot before the expert launch (page "GLM 5.3 Testing: HBM Expert
// Allocation", section "What the slot cache is"); the copy is an SM-driven
// kernel and its cost is host-link bytes (same page, section "The build";
// page "GB300 GLM 5.3 Testing", section "E1 v2").  The expert products are the
// routed gate/up ("w13") and down ("w2") NVFP4 matrices, combined in fp32 and
// reduced once (page "GLM 5.3 Testing: HBM Expert Allocation", section "A
// correction first"; page "glm53 - GLM-5.3-Flash (NVFP4)", prefill-groups
// knob).
//
// GEMV layout (decode rows are few, so the products are HBM-bandwidth bound):
// one wavefront owns a run of output rows of one unique expert.  Each lane
// owns 32 consecutive K-elements of a row per 2048-wide chunk (16 B of FP4
// codes and 2 B of E4M3 block scales, coalesced across the wavefront), keeps
// the matching activation slice in registers for every row of the run, and
// the lanes of a row are summed with cross-lane shuffles.  FP4 pairs are
// widened by the gfx950 convert instructions; gate/up uses bf16 dot2 on the
// bf16 activations (exact products, fp32 accumulate), down uses fp32 FMAs on
// the fp32 intermediate.  The E4M3 block scale multiplies each 16-element
// block sum; the fp32 global scale multiplies the row sum.
#include "internal.h"

#include <type_traits>

namespace sc {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

template <int K>
struct Geo {
  static constexpr int NSEG = K >= 2048 ? K / 2048 : 1;   // 2048-wide chunks per row
  static constexpr int LPR = K >= 2048 ? 64 : K / 32;     // lanes per row
  static constexpr int RPW = 64 / LPR;                    // rows per wavefront step
  static_assert(K % 32 == 0, "K must be a multiple of 32");
  static_assert(K >= 2048 ? (K % 2048 == 0) : (64 % (K / 32) == 0), "unsupported K");
};

struct GemvArgs {
  const int32_t* hdr;
  const uint8_t* const* uniq_ptr;
  const int32_t* uniq_expert;
  const float* gs;       // [E][2] global scales of the layer's bank
  const int32_t* uniq_off;
  const int32_t* uniq_picks;
  const void* operand;   // gate/up: bf16 x [M][H]; down: h [P][I], 4 bytes per element
  float* out;            // gate/up: h [P][I];      down: part [P][H]
  int rows;              // output rows per expert: I (gate/up) or H (down)
  int k;                 // top-k: pick p belongs to row p / k
  int up_row0;           // gate/up: first up row (I)
  int split_h;           // gate/up: write h split for the matrix-core down product (see store_h)
  int64_t code_off;      // offset of the code rows inside a blob
  int64_t scale_off;     // offset of the scale rows inside a blob
  uint64_t* span;        // execution stamps of a timed step, else null
  const int32_t* order;  // staged prefill: unique experts in group order
  int group;             // -1: every unique expert; g >= 0: group g of a staged step
  int G;                 // experts per staged group
};

// The unique experts a launch computes: positions [lo, lo + n) of `order`, or
// all U in their own order when the launch is not one group of a staged step.
__device__ __forceinline__ void launch_uniques(const GemvArgs& a, int U, int& lo, int& n) {
  if (a.group < 0) {
    lo = 0;
    n = U;
  } else {
    int hi;
    group_range(a.hdr, a.group, a.G, lo, hi);
    n = hi - lo;
  }
}
__device__ __forceinline__ int unique_at(const GemvArgs& a, int lo, int j) {
  return a.group < 0 ? j : a.order[lo + j];
}

// SiLU from the hardware exponential and reciprocal (v_exp_f32 of -g log2(e),
// v_rcp_f32: a few ulps in all, far inside the fp32 accumulation error of g
// and u).  Below about g = -88 the exponential is +inf and the result -0.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// h as the matrix-core down product reads it: each group of 8 elements is 16
// bytes of bf16 high parts then 16 bytes of bf16 low parts (hi = bf16(v), lo =
// bf16(v - hi)), so a pick's row keeps the 4 bytes per element of fp32 h.
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}
__device__ __forceinline__ void store_h(float* row, int r, float v, bool split) {
  if (!split) {
    row[r] = v;
    return;
  }
  __bf16 hi, lo;
  split_bf16(v, hi, lo);
  __bf16* grp = reinterpret_cast<__bf16*>(row) + (r / 8) * 16 + (r % 8);
  grp[0] = hi;
  grp[8] = lo;
}

// Loads through global-address-space pointers: blob pointers come from memory,
// so without the cast the compiler emits flat loads (which also count against
// the LDS counter and force conservative waits).  Device-mapped pinned host
// memory is global memory to the GPU as well.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const uint16_t g_u16;
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  const u32x4 v = *(g_u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Weight streams are read once per step: the nontemporal hint keeps them from
// displacing the activations and partial results in the caches (measured a
// few per cent faster on the 113 MB gate/up stream).
__device__ __forceinline__ uint4 ld16_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((g_u32x4*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The block scales are streamed once per step as well.
__device__ __forceinline__ uint32_t ld2(const uint8_t* p) { return __builtin_nontemporal_load((g_u16*)(p)); }

// Wavefront index as a uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Widen the eight FP4 values of one dword (byte j holds elements 2j, 2j+1,
// the even one in the low nibble) to bf16 or fp32 pairs.  The byte selector
// of the convert instruction must be an immediate.
__device__ __forceinline__ void fp4x8_bf16(uint32_t c, bf16x2 (&w)[4]) {
  w[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 0);
  w[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 1);
  w[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 2);
  w[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 3);
}

__device__ __forceinline__ void fp4x8_f32(uint32_t c, f32x2 (&w)[4]) {
  w[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  w[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  w[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  w[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
}

// The two E4M3 block scales in bytes 0 and 1 of sc, widened by one
// instruction (the conversion is exact).
__device__ __forceinline__ f32x2 scales2(uint32_t sc) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)sc, false); }

// v_dot2_f32_bf16 with an inline zero accumulator: the builtin's form first
// zeroes a register with a move.  Same operation and result.
__device__ __forceinline__ float dot2_bf16_z(bf16x2 a, bf16x2 b) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// A row's running sum over its chunks: acc + b0 s0 + b1 s1, where b0 and b1
// are one lane's sums over the two 16-element blocks of its 32 elements of one
// chunk (codes q, 16 B; block scales in bytes 0 and 1 of sc; bf16 activation
// pairs xv[16]).  A row's sum starts from -0, so the first chunk adds exactly
// b0 s0 + b1 s1 rounded as the fused multiply-adds round it.
__device__ __forceinline__ float seg_dot_bf16(const uint4& q, uint32_t sc, const uint32_t* xv, float acc_in) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  float b[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float acc = 0.0f;
#pragma unroll
    for (int dw = 0; dw < 2; ++dw) {
      bf16x2 w[4];
      fp4x8_bf16(d[blk * 2 + dw], w);
#pragma unroll
      for (int sel = 0; sel < 4; ++sel) {
        bf16x2 xx = __builtin_bit_cast(bf16x2, xv[(blk * 2 + dw) * 4 + sel]);
        acc = dw == 0 && sel == 0 ? dot2_bf16_z(w[sel], xx) : __builtin_amdgcn_fdot2_f32_bf16(w[sel], xx, acc, false);
      }
    }
    b[blk] = acc;
  }
  const f32x2 sw = scales2(sc);
  const float s0 = sw.x, s1 = sw.y;
  return fmaf(b[1], s1, fmaf(b[0], s0, acc_in));
}

// Same with fp32 activations hv[32].
__device__ __forceinline__ float seg_dot_f32(const uint4& q, uint32_t sc, const float* hv, float acc_in) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  float b[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float acc = 0.0f;
#pragma unroll
    for (int dw = 0; dw < 2; ++dw) {
      f32x2 w[4];
      fp4x8_f32(d[blk * 2 + dw], w);
#pragma unroll
      for (int sel = 0; sel < 4; ++sel) {
        const int e = ((blk * 2 + dw) * 4 + sel) * 2;
        acc = fmaf(w[sel].x, hv[e], acc);
        acc = fmaf(w[sel].y, hv[e + 1], acc);
      }
    }
    b[blk] = acc;
  }
  const f32x2 sw = scales2(sc);
  const float s0 = sw.x, s1 = sw.y;
  return fmaf(b[1], s1, fmaf(b[0], s0, acc_in));
}

// Sum NV values per lane over the LPR lanes of a row group with a transposed
// butterfly: while more than one value is left, each step trades half of the
// values with the partner lane, so a lane ends up holding the group sum of one
// value, index (lane % LPR) / (LPR / NV).
//
// The exchanges stay in registers.  Steps 32 and 16 use the gfx950 lane-swap
// instructions (v_permlane32_swap / v_permlane16_swap: the upper 32 lanes, or
// the odd 16-lane rows, of one register trade places with the lower lanes, or
// even rows, of another), so one instruction exchanges a pair of values; steps
// 8, 4, 2 and 1 read the partner through DPP: row mirror (lane ^ 15), half-row
// mirror (lane ^ 7) and two quad permutes (lane ^ 2, lane ^ 1).  Every step
// pairs lanes that differ in bit O, both partners add the same two numbers,
// and the six pairings span all lane bits: each value is summed over its row
// group by the same tree whatever NV is, and every lane that holds it holds
// the same bits.
template <int O>
__device__ __forceinline__ float dpp_partner(float v) {
  constexpr int ctrl = O == 8 ? 0x140 : O == 4 ? 0x141 : O == 2 ? 0x4E : 0xB1;
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), ctrl, 0xF, 0xF, false));
}

// a, b -> the step-O pair sums: lanes below bit O hold a's sum, lanes above it b's
template <int O>
__device__ __forceinline__ float swap_add(float a, float b) {
  static_assert(O == 32 || O == 16, "lane swaps exist for 32 and 16");
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int O, int C>
struct XRed {
  __device__ static __forceinline__ void run(float* v, int lane) {
    if constexpr (O == 0) {
      return;
    } else {
      if constexpr (O >= 16) {
#pragma unroll
        for (int i = 0; i < (C > 1 ? C / 2 : 1); ++i) v[i] = swap_add<O>(v[i], v[C > 1 ? i + C / 2 : 0]);
      } else if constexpr (C > 1) {
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int i = 0; i < C / 2; ++i) {
          const float send = up ? v[i] : v[i + C / 2];
          const float keep = up ? v[i + C / 2] : v[i];
          v[i] = keep + dpp_partner<O>(send);
        }
      } else {
        v[0] += dpp_partner<O>(v[0]);
      }
      XRed<O / 2, (C > 1 ? C / 2 : 1)>::run(v, lane);
    }
  }
};

// Streaming GEMV.  Each unique expert's row steps are split into `wpu`
// contiguous runs, one per wavefront (task); a wavefront keeps the operand
// slices of up to MR picks in registers and walks its run R row steps at a
// time, issuing the next R steps' code and scale loads (a second register
// set) before it sums the current ones; the compiler's waits let those loads
// overlap the current steps' first products (see load()).
//
// SINGLE: a one-row step.  Its k picks are k distinct experts, so U = k and
// pick u is unique expert u (the remap's CSR lists are the identity): the
// kernel takes U from the launch instead of the header and skips the CSR
// lookups, so a wavefront's first weight loads wait for one pointer load only
// and its activation loads for none.
//
// PART (one-row gate/up only) splits a step around its fill: 1 = the experts
// the fill does not write (the copy runs beside them), 2 = the ones it writes,
// taken from the remap's resident-first order once the copy is done.
template <int K, int MR, int R, bool GATEUP, bool SINGLE = false, int PART = 0>
struct Gemv {
  using G = Geo<K>;
  static constexpr int NSEG = G::NSEG, LPR = G::LPR, RPW = G::RPW;
  static constexpr int OPW = GATEUP ? 16 : 32;
  static constexpr int NM = GATEUP ? 2 : 1;
  static constexpr int NV = R * MR;
  static_assert(NV <= LPR, "too many values for the row group");

  struct Buf {
    uint4 q[R][NM][NSEG];
    uint32_t sc[R][NM][NSEG];
  };

  // Row step of the task's i-th step: base + i * stride.  The loads of one
  // stage carry no branches (with one branch per row the compiler waited for
  // every outstanding load before the stage's first product): a row step past
  // the end of the run re-reads the run's last row step, and process() stores
  // nothing for it.  The loop below skips the next stage's loads at the end of
  // a run, so the compiler waits for them too before the current stage's last
  // products; a branch-free steady state that keeps them in flight measured
  // slower (more registers: two wavefronts per SIMD for gate/up).
  __device__ static __forceinline__ void load(Buf& b, const uint8_t* code_base, const uint8_t* scale_base,
                                              int i, int n, int base, int stride, int rsub, int up_row0) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int step = i + j < n ? i + j : n - 1;
      const int r = (base + step * stride) * RPW + rsub;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const size_t row = (size_t)(r + m * up_row0);
#pragma unroll
        for (int c = 0; c < NSEG; ++c) {
          b.q[j][m][c] = ld16_stream(code_base + row * (K / 2) + c * 1024);
          b.sc[j][m][c] = ld2(scale_base + row * (K / 16) + c * 128);
        }
      }
    }
  }

  // seg_dot_f32 with the codes already widened: w[4 * dw + sel] from dword dw
  __device__ static __forceinline__ float blocks_dot_f32(const f32x2 (&w)[16], float s0, float s1, const float* hv,
                                                        float acc_in) {
    float bsum[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc = fmaf(w[blk * 8 + e].x, hv[2 * (blk * 8 + e)], acc);
        acc = fmaf(w[blk * 8 + e].y, hv[2 * (blk * 8 + e) + 1], acc);
      }
      bsum[blk] = acc;
    }
    return fmaf(bsum[1], s1, fmaf(bsum[0], s0, acc_in));
  }

  // hq: the one-row gate/up's pending sums (see below); unused otherwise
  __device__ static __forceinline__ void process(const Buf& b, const uint32_t (&opw)[MR][NSEG][OPW],
                                                 const int (&pk)[MR], int nc, int i, int n, int base,
                                                 int stride, int lane, int rsub, float gs, const GemvArgs& a,
                                                 float& hq) {
    float v0[NV], v1[NV];
    if constexpr (!GATEUP && MR > 1) {
      // down with several picks: each row's codes are widened once and serve
      // every pick (same products and order as seg_dot_f32)
#pragma unroll
      for (int e = 0; e < NV; ++e) v0[e] = -0.0f;
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int c = 0; c < NSEG; ++c) {
          const uint32_t d[4] = {b.q[j][0][c].x, b.q[j][0][c].y, b.q[j][0][c].z, b.q[j][0][c].w};
          f32x2 w[16];
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            f32x2 t[4];
            fp4x8_f32(d[dw], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) w[4 * dw + e] = t[e];
          }
          const f32x2 sw = scales2(b.sc[j][0][c]);
          const float s0 = sw.x, s1 = sw.y;
#pragma unroll
          for (int mi = 0; mi < MR; ++mi)
            if (mi < nc)
              v0[j * MR + mi] = blocks_dot_f32(w, s0, s1, reinterpret_cast<const float*>(opw[mi][c]), v0[j * MR + mi]);
          // one row's widened codes live at a time
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int mi = 0; mi < MR; ++mi) {
        float acc0 = -0.0f, acc1 = -0.0f;
        if (mi < nc) {
#pragma unroll
          for (int c = 0; c < NSEG; ++c) {
            if (GATEUP) {
              acc0 = seg_dot_bf16(b.q[j][0][c], b.sc[j][0][c], opw[mi][c], acc0);
              acc1 = seg_dot_bf16(b.q[j][NM - 1][c], b.sc[j][NM - 1][c], opw[mi][c], acc1);
            } else {
              acc0 = seg_dot_f32(b.q[j][0][c], b.sc[j][0][c], reinterpret_cast<const float*>(opw[mi][c]), acc0);
            }
          }
        }
        v0[j * MR + mi] = acc0;
        v1[j * MR + mi] = acc1;
      }
    }
    }
    if constexpr (GATEUP && NV == 1 && LPR == 64) {
      // one row over the whole wavefront: its gate and up sums are reduced
      // together (each by the same tree as alone), lanes 0-31 ending with the
      // gate sum and lanes 32-63 with the up sum
      float gu[2] = {v0[0], v1[0]};
      XRed<32, 2>::run(gu, lane);
      // Row step i's gate sum waits in lane i % 32 of hq and its up sum in
      // lane 32 + i % 32; every 32 row steps, and after the run's last, lanes
      // 0-31 take SiLU(gate) * up of the row steps they hold and store them
      // together (the rows are consecutive).
      const int t = i & 31;
      hq = (lane & 31) == t ? gu[0] : hq;
      if (t == 31 || i + 1 >= n) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(hq), __float_as_uint(hq), false, false);
        const float g = __uint_as_float(sw[0]), u = __uint_as_float(sw[1]);   // lanes 0-31: own and lane + 32
        if (lane <= t && nc > 0)
          store_h(a.out + (size_t)pk[0] * a.rows, base + (i - t + lane) * stride, silu_f32(g * gs) * (u * gs),
                  !SINGLE && a.split_h);
      }
      return;
    }
    if constexpr (!GATEUP && MR == 1) {
      // a lane holds the sum of row step i + j, j = (lane % LPR) / (LPR / NV):
      // one store for the stage's R rows
      XRed<LPR / 2, NV>::run(v0, lane);
      const int g = lane % LPR;
      const int j = g / (LPR / NV);
      if (g % (LPR / NV) == 0 && nc > 0 && i + j < n)
        a.out[(size_t)pk[0] * a.rows + (base + (i + j) * stride) * RPW + rsub] = v0[0] * gs;
      return;
    }
    XRed<LPR / 2, NV>::run(v0, lane);
    if (GATEUP) XRed<LPR / 2, NV>::run(v1, lane);
    const int g = lane % LPR;
    if (g % (LPR / NV) == 0) {
      const int idx = g / (LPR / NV);
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
          if (idx == j * MR + mi && mi < nc && i + j < n) {
            const int r = (base + (i + j) * stride) * RPW + rsub;
            if (GATEUP)
              store_h(a.out + (size_t)pk[mi] * a.rows, r, silu_f32(v0[0] * gs) * (v1[0] * gs),
                      !SINGLE && a.split_h);   // one-row steps never run the matrix cores
            else
              a.out[(size_t)pk[mi] * a.rows + r] = v0[0] * gs;
          }
        }
      }
    }
  }

  // vblock / vgrid: this block and the launch's block count, or those of the
  // launch's product blocks when it shares them with a copy.
  __device__ static __forceinline__ void run(const GemvArgs& a, int vblock, int vgrid) {
    static_assert(!SINGLE || MR == 1, "one-row steps have one pick per expert");
    static_assert(PART == 0 || (SINGLE && GATEUP), "only one-row gate/up steps are split");
    int lo = 0, U = a.k;
    if (!SINGLE) launch_uniques(a, a.hdr[H_UNIQUE], lo, U);
    // filled experts: the last nf of the resident-first order
    int nf = PART != 0 ? a.hdr[H_MISS] : 0;
    nf = nf < 0 ? 0 : nf > a.k ? a.k : nf;
    if (PART == 2) {
      lo = a.k - nf;
      U = nf;
    }
    if (U <= 0) return;
    const int lane = threadIdx.x & 63;
    const int seg = lane % LPR, rsub = lane / LPR;
    const int nwaves = vgrid * (kGemvThreads / 64);
    const int gw = vblock * (kGemvThreads / 64) + wave_id();
    const int spu = a.rows / RPW;
    int wpu = nwaves / U;
    if (wpu < 1) wpu = 1;
    if (wpu > spu) wpu = spu;
    // contiguous runs: the first `rem` tasks of an expert take q + 1 row steps, the others q
    const int q = spu / wpu, rem = spu - q * wpu;
    const int ntask = U * wpu;
    for (int task = gw; task < ntask; task += nwaves) {
      const int j = task / wpu, sub = task - (task / wpu) * wpu;
      const int u = PART == 2 ? a.order[lo + j] : SINGLE ? j : unique_at(a, lo, j);
      // a task owns row steps base + i * stride, i < n
      const int base = sub * q + (sub < rem ? sub : rem), stride = 1;
      const int n = q + (sub < rem ? 1 : 0);
      if (n <= 0) continue;
      const uint8_t* blob = a.uniq_ptr[u];
      const float gs = a.gs[2 * a.uniq_expert[u] + (GATEUP ? 0 : 1)];
      if (PART == 1 && nf > 0) {
        // part 1 keeps every expert's share of the waves, so an all-hit step
        // (nf = 0) runs as the plain kernel does; a filled expert's waves sit out
        bool filled = false;
        for (int i = a.k - nf; i < a.k; ++i) filled |= a.order[i] == u;
        if (filled) continue;
      }
      const int off0 = SINGLE ? u : a.uniq_off[u], off1 = SINGLE ? u + 1 : a.uniq_off[u + 1];
      const uint8_t* code_base = blob + a.code_off + seg * 16;
      const uint8_t* scale_base = blob + a.scale_off + seg * 2;
      for (int c0 = off0; c0 < off1; c0 += MR) {
        const int nc = off1 - c0 < MR ? off1 - c0 : MR;
        Buf A, B;
        load(A, code_base, scale_base, 0, n, base, stride, rsub, a.up_row0);
        int pk[MR];
        uint32_t opw[MR][NSEG][OPW];
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
          pk[mi] = SINGLE ? c0 : (mi < nc ? a.uniq_picks[c0 + mi] : 0);
#pragma unroll
          for (int c = 0; c < NSEG; ++c) {
            const int e0 = c * 2048 + seg * 32;
            const uint4* src;
            if (GATEUP)
              src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.operand) +
                                                   (size_t)(SINGLE ? 0 : pk[mi] / a.k) * K + e0);
            else
              src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.operand) +
                                                   (size_t)pk[mi] * K + e0);
#pragma unroll
            for (int v = 0; v < OPW / 4; ++v) {
              uint4 t = mi < nc ? src[v] : make_uint4(0u, 0u, 0u, 0u);
              opw[mi][c][4 * v + 0] = t.x;
              opw[mi][c][4 * v + 1] = t.y;
              opw[mi][c][4 * v + 2] = t.z;
              opw[mi][c][4 * v + 3] = t.w;
            }
          }
        }
        float hq = 0.0f;
        int i = 0;
        while (true) {
          if (i + R < n) load(B, code_base, scale_base, i + R, n, base, stride, rsub, a.up_row0);
          process(A, opw, pk, nc, i, n, base, stride, lane, rsub, gs, a, hq);
          i += R;
          if (i >= n) break;
          if (i + R < n) load(A, code_base, scale_base, i + R, n, base, stride, rsub, a.up_row0);
          process(B, opw, pk, nc, i, n, base, stride, lane, rsub, gs, a, hq);
          i += R;
          if (i >= n) break;
        }
      }
    }
  }
};

// Streaming GEMVs for steps of two to four rows.  The weights stream as in
// the one-row kernels (a lane owns 32 K-elements per 2048-wide chunk; the next
// row steps' loads are issued before the current ones are summed), each
// chunk's codes are widened once (gate/up to bf16 pairs, down to fp32), and
// every pick of the expert is computed from them.  A step of M rows gives an
// expert at most M picks (a row's top-k experts are distinct), so the operand
// rows (x or h) of an expert's at most kSharedPicks picks sit in LDS, loaded
// once per block task and shared by the block's four wavefronts: a block task
// is a run of one expert's row steps, split among the wavefronts.  A row's products, its block-scale
// products and its cross-lane sums are those of the one-row kernel, in the
// same order, so each row's bits do not depend on how many rows the step has.
// In LDS, operand piece v (16 bytes) of lane `seg` in a chunk sits in slot
// v ^ sw(seg) of the lane's run, so eight neighbouring lanes reading their
// v-th pieces hit eight different bank groups.
constexpr int kSharedPicks = 4;

template <int K, int R, bool GATEUP>
struct GemvShared {
  using G = Geo<K>;
  static constexpr int NSEG = G::NSEG, LPR = G::LPR, RPW = G::RPW;
  static constexpr int NM = GATEUP ? 2 : 1;
  static constexpr int MRX = kSharedPicks;
  static constexpr int EB = GATEUP ? 2 : 4;             // operand bytes per element
  static constexpr int ROWB = K * EB;                   // operand bytes per pick
  static constexpr int PPL = 32 * EB / 16;              // 16-byte pieces per lane and chunk
  static constexpr int NV = R * MRX;
  static constexpr int LDS_B = MRX * ROWB;
  static_assert(NV <= LPR, "too many values for the row group");

  using Buf = typename Gemv<K, 1, R, GATEUP>::Buf;

  __device__ static __forceinline__ int sw(int seg) { return EB == 2 ? ((seg >> 1) & 3) : (seg & 7); }
  // byte offset of piece v of lane seg, chunk c, pick slot m
  __device__ static __forceinline__ int lpos(int m, int c, int seg, int v) {
    return m * ROWB + c * (2048 * EB) + seg * (PPL * 16) + 16 * (v ^ sw(seg));
  }

  // the operand rows of picks c0 .. c0 + nc - 1 into LDS (all threads of the block)
  __device__ static __forceinline__ void stage_operand(const GemvArgs& a, uint8_t* lds, int c0, int nc) {
    constexpr int PPR_ = ROWB / 16;                     // pieces per operand row
    const int total = nc * PPR_;
    for (int P = threadIdx.x; P < total; P += kGemvThreads) {
      const int m = P / PPR_, q = P - m * PPR_;
      const int p = a.uniq_picks[c0 + m];
      const uint8_t* row = static_cast<const uint8_t*>(a.operand) +
                           (GATEUP ? (size_t)(p / a.k) * K * 2 : (size_t)p * K * 4);
      const int byte = 16 * q;
      const int c = byte / (2048 * EB), rem = byte - c * (2048 * EB);
      const int seg = rem / (PPL * 16), v = (rem / 16) % PPL;
      *reinterpret_cast<uint4*>(lds + lpos(m, c, seg, v)) = ld16(row + byte);
    }
  }

  // the lane's 32 operand elements of chunk c of pick slot m
  __device__ static __forceinline__ void xread(const uint8_t* lds, int m, int c, int seg, uint32_t (&xv)[16 * EB / 2]) {
#pragma unroll
    for (int v = 0; v < PPL; ++v) {
      const uint4 t = *reinterpret_cast<const uint4*>(lds + lpos(m, c, seg, v));
      xv[4 * v + 0] = t.x;
      xv[4 * v + 1] = t.y;
      xv[4 * v + 2] = t.z;
      xv[4 * v + 3] = t.w;
    }
  }

  // seg_dot_bf16 with the codes already widened: w[4 * dw + sel] from dword dw
  __device__ static __forceinline__ float blocks_dot(const bf16x2 (&w)[16], float s0, float s1, const uint32_t* xv,
                                                     float acc_in) {
    float bsum[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16x2 xx = __builtin_bit_cast(bf16x2, xv[blk * 8 + e]);
        acc = e == 0 ? dot2_bf16_z(w[blk * 8 + e], xx) : __builtin_amdgcn_fdot2_f32_bf16(w[blk * 8 + e], xx, acc, false);
      }
      bsum[blk] = acc;
    }
    return fmaf(bsum[1], s1, fmaf(bsum[0], s0, acc_in));
  }

  __device__ static __forceinline__ void process(const Buf& b, const uint8_t* lds, const int (&pk)[MRX], int nc, int i,
                                                 int n, int base, int lane, int rsub, float gs, const GemvArgs& a) {
    const int seg = lane % LPR;
    float v0[NV], v1[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      v0[e] = -0.0f;
      v1[e] = -0.0f;
    }
    if constexpr (GATEUP) {
      // each chunk's codes are widened once, then used by every pick
#pragma unroll
      for (int c = 0; c < NSEG; ++c) {
        bf16x2 wg[R][16], wu[R][16];
        float sg[R][2], su[R][2];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const uint32_t dg[4] = {b.q[j][0][c].x, b.q[j][0][c].y, b.q[j][0][c].z, b.q[j][0][c].w};
          const uint32_t du[4] = {b.q[j][1][c].x, b.q[j][1][c].y, b.q[j][1][c].z, b.q[j][1][c].w};
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            bf16x2 t[4];
            fp4x8_bf16(dg[dw], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) wg[j][4 * dw + e] = t[e];
            fp4x8_bf16(du[dw], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) wu[j][4 * dw + e] = t[e];
          }
          const f32x2 g2 = scales2(b.sc[j][0][c]), u2 = scales2(b.sc[j][1][c]);
          sg[j][0] = g2.x;
          sg[j][1] = g2.y;
          su[j][0] = u2.x;
          su[j][1] = u2.y;
        }
#pragma unroll
        for (int m = 0; m < MRX; ++m) {
          if (m < nc) {
            uint32_t xv[16];
            xread(lds, m, c, seg, xv);
#pragma unroll
            for (int j = 0; j < R; ++j) {
              v0[j * MRX + m] = blocks_dot(wg[j], sg[j][0], sg[j][1], xv, v0[j * MRX + m]);
              v1[j * MRX + m] = blocks_dot(wu[j], su[j][0], su[j][1], xv, v1[j * MRX + m]);
            }
          }
        }
      }
    } else {
      // the stage's R rows are widened to fp32 once per chunk; each pick's
      // operand slice is read from LDS once per chunk and serves the R rows
#pragma unroll
      for (int c = 0; c < NSEG; ++c) {
        f32x2 w[R][16];
        float s0[R], s1[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const uint32_t d[4] = {b.q[j][0][c].x, b.q[j][0][c].y, b.q[j][0][c].z, b.q[j][0][c].w};
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            f32x2 t[4];
            fp4x8_f32(d[dw], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) w[j][4 * dw + e] = t[e];
          }
          const f32x2 sw = scales2(b.sc[j][0][c]);
          s0[j] = sw.x;
          s1[j] = sw.y;
        }
#pragma unroll
        for (int m = 0; m < MRX; ++m) {
          if (m < nc) {
            uint32_t xv[32];
            xread(lds, m, c, seg, xv);
#pragma unroll
            for (int j = 0; j < R; ++j)
              v0[j * MRX + m] = Gemv<K, 1, R, false>::blocks_dot_f32(w[j], s0[j], s1[j],
                                                                    reinterpret_cast<const float*>(xv),
                                                                    v0[j * MRX + m]);
          }
        }
      }
    }
    XRed<LPR / 2, NV>::run(v0, lane);
    if (GATEUP) XRed<LPR / 2, NV>::run(v1, lane);
    const int g = lane % LPR;
    if (g % (LPR / NV) == 0) {
      const int idx = g / (LPR / NV);
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int m = 0; m < MRX; ++m) {
          if (idx == j * MRX + m && m < nc && i + j < n) {
            const int r = (base + i + j) * RPW + rsub;
            if (GATEUP)
              store_h(a.out + (size_t)pk[m] * a.rows, r, silu_f32(v0[0] * gs) * (v1[0] * gs), a.split_h);
            else
              a.out[(size_t)pk[m] * a.rows + r] = v0[0] * gs;
          }
        }
      }
    }
  }

  __device__ static __forceinline__ void run(const GemvArgs& a, uint8_t* lds) {
    const int U = a.hdr[H_UNIQUE];
    if (U <= 0) return;
    const int lane = threadIdx.x & 63, w = wave_id();
    const int seg = lane % LPR, rsub = lane / LPR;
    const int spu = a.rows / RPW;                 // row steps per expert
    int tpe = (int)gridDim.x / U;                 // block tasks per expert
    if (tpe < 1) tpe = 1;
    if (tpe > spu) tpe = spu;
    const int ntask = U * tpe;
    int prev_u = -1;
    for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
      const int u = task / tpe, sub = task - u * tpe;
      // the task's row steps [t0, t1), then the wavefront's share [base, base + n)
      const int t0 = (int)((long)spu * sub / tpe), t1 = (int)((long)spu * (sub + 1) / tpe);
      const int per = (t1 - t0 + 3) / 4;
      const int base = t0 + w * per;
      int n = t1 - base;
      n = n < 0 ? 0 : n > per ? per : n;
      const uint8_t* blob = a.uniq_ptr[u];
      const float gs = a.gs[2 * a.uniq_expert[u] + (GATEUP ? 0 : 1)];
      const int off0 = a.uniq_off[u], off1 = a.uniq_off[u + 1];
      const int nc = off1 - off0 < MRX ? off1 - off0 : MRX;     // at most MRX on the steps this kernel serves
      const uint8_t* code_base = blob + a.code_off + seg * 16;
      const uint8_t* scale_base = blob + a.scale_off + seg * 2;
      Buf A, B;
      if (n > 0) Gemv<K, 1, R, GATEUP>::load(A, code_base, scale_base, 0, n, base, 1, rsub, a.up_row0);
      if (u != prev_u) {
        __syncthreads();                          // the block is done with the previous operands
        stage_operand(a, lds, off0, nc);
        __syncthreads();
        prev_u = u;
      }
      int pk[MRX];
#pragma unroll
      for (int m = 0; m < MRX; ++m) pk[m] = m < nc ? a.uniq_picks[off0 + m] : 0;
      if (n <= 0) continue;
      int i = 0;
      while (true) {
        if (i + R < n) Gemv<K, 1, R, GATEUP>::load(B, code_base, scale_base, i + R, n, base, 1, rsub, a.up_row0);
        process(A, lds, pk, nc, i, n, base, lane, rsub, gs, a);
        i += R;
        if (i >= n) break;
        if (i + R < n) Gemv<K, 1, R, GATEUP>::load(A, code_base, scale_base, i + R, n, base, 1, rsub, a.up_row0);
        process(B, lds, pk, nc, i, n, base, lane, rsub, gs, a);
        i += R;
        if (i >= n) break;
      }
    }
  }
};

template <int K, int R, bool GATEUP>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_shared(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GemvShared<K, R, GATEUP>::LDS_B];
  span_start(a.span);
  GemvShared<K, R, GATEUP>::run(a, lds);
  span_end(a.span);
}

template <int K, int MR, int R, bool GATEUP, bool SINGLE>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvArgs a) {
  span_start(a.span);
  Gemv<K, MR, R, GATEUP, SINGLE>::run(a, blockIdx.x, gridDim.x);
  span_end(a.span);
}

// ---------------------------------------------------------------------------
// Matrix-core path for steps with several rows per expert (draft / verify
// batches).  For every 128-wide K tile a wavefront decodes the FP4 codes of
// 16 weight rows into bf16 pre-multiplied by their E4M3 block scale (exact: a
// code has at most 2 significant bits and a scale 4, so the product fits
// bf16's 8) and issues four v_mfma_f32_16x16x32_bf16 against up to 16 picks.
// Lane layout of that instruction (checked on the device): A lane l = row
// l%16, k = 8*(l/16)+j; B lane l = k = 8*(l/16)+j, column l%16; D lane l, j =
// row 4*(l/16)+j, column l%16.  Lane group g = l/16 therefore takes elements
// [32g, 32g+32) of the K tile -- 16 bytes of codes and 2 bytes of scales --
// and dword d of those codes is its slice of the d-th MFMA.  The down
// projection's fp32 operand is split into bf16 high and low parts (two
// MFMAs), keeping about 16 bits.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ bf16x8 fp4x8_scaled_bf16(uint32_t c, float s) {
  f32x2 w[4];
  fp4x8_f32(c, w);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (__bf16)(w[i].x * s);
    r[2 * i + 1] = (__bf16)(w[i].y * s);
  }
  return r;
}

__device__ __forceinline__ bf16x8 bf16x8_from_words(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// The weights are staged through LDS.  Loaded in the MFMA layout directly (16
// rows x 64 bytes per instruction) they peaked at about 4.5 TB/s in a
// pure-read test, against 6.8 TB/s for loads of whole cache lines.  A task is
// 16 * RT weight rows of one unique expert (gate/up: RT 16-row tiles of gate
// and the matching tiles of up) against NCP of its picks per pass.  K is walked
// in stages of KC elements: the stage's weight rows are loaded
// row-contiguously (whole 128-byte lines per row) into registers, together
// with the stage's operand slices (x or h) of the NCP pick columns, written to
// the wavefront's LDS buffer and read back in the MFMA lane layout while the
// next stage's loads (TWO: the next two stages') are in flight, so the operand
// waits no longer than the weights do.  In LDS, 16-byte piece c of weight row
// j sits in slot c ^ (j mod PPR) of its row, and operand chunk o of column n
// in slot o ^ (n mod 8) of its column, so the lanes of one read hit different
// bank groups.  Columns past the pass's picks load the last pick's operand
// (their loads coalesce with its own): the products of one column do not mix
// with the others', and only the picks' columns are stored; MFMA columns
// NCP..15 repeat columns 0..NCP-1.  (Direct-to-LDS loads cannot be prefetched
// this way: the compiler waits for all of them before any LDS read.)
template <int K, bool GATEUP, int RT, int KCW, int NCP, bool TWO>
struct GemvMfmaL {
  static constexpr int NM = GATEUP ? 2 : 1;
  static constexpr int NROW = 16 * RT * NM;            // weight rows per task
  static constexpr int KC = K < KCW ? K : KCW;         // K elements per stage
  static constexpr int NS = K / KC;                    // stages
  static constexpr int PPR = KC / 32;                  // 16-byte code pieces per row and stage
  static constexpr int CPL = NROW * PPR / 64;          // code pieces per lane and stage
  static constexpr int SPR = KC / 64;                  // scale dwords per row and stage
  static constexpr int SPL = NROW * SPR / 64;          // scale dwords per lane and stage
  static constexpr int CODE_B = NROW * KC / 2;
  static constexpr int W_B = CODE_B + NROW * KC / 16;  // weight bytes per stage
  static constexpr int EB = GATEUP ? 2 : 4;            // operand bytes per element (h: bf16 high + low)
  static constexpr int OCH = KC * EB / 16;             // 16-byte operand chunks per column and stage
  static constexpr int XPL = NCP * OCH / 64;           // operand chunks per lane and stage
  static constexpr int TCH = 128 * EB / 64;            // operand chunks a lane reads per K tile
  static constexpr int STAGE_B = W_B + NCP * OCH * 16;
  static constexpr int NKT = KC / 128;                 // K tiles per stage
  static_assert(K % KC == 0 && KC % 128 == 0 && CPL >= 1 && SPL >= 1 && XPL >= 1, "unsupported K");
  static_assert(OCH % 8 == 0, "the operand swizzle permutes groups of 8 chunks");

  struct Regs {
    uint4 c[CPL];
    uint32_t s[SPL];
    uint4 x[XPL];
  };

  // global row of task row j (a ragged task re-reads its last tile)
  __device__ static __forceinline__ size_t grow(const GemvArgs& a, int tile0, int nt, int j) {
    const int rt = j / (16 * NM), m = (j / 16) % NM, n = j % 16;
    const int tile = tile0 + (rt < nt ? rt : nt - 1);
    return (size_t)(tile * 16 + n + m * a.up_row0);
  }

  // xsrc: the operand row of the lane's column (lane mod 16); the lane loads
  // its chunks lane / 16 + 4 i of the stage
  __device__ static __forceinline__ void gload(Regs& r, const GemvArgs& a, const uint8_t* blob, const uint8_t* xsrc,
                                               int tile0, int nt, int stage, int lane) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int L = 64 * i + lane, j = L / PPR, slot = L % PPR;
      const int c = slot ^ (j % PPR);
      r.c[i] = ld16_stream(blob + a.code_off + grow(a, tile0, nt, j) * (K / 2) + stage * (KC / 2) + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int D = 64 * i + lane, j = D / SPR, dw = D % SPR;
      r.s[i] = *(const __attribute__((address_space(1))) uint32_t*)(blob + a.scale_off + grow(a, tile0, nt, j) * (K / 16) +
                                                                   stage * (KC / 16) + 4 * dw);
    }
    const uint8_t* xs = xsrc + (size_t)stage * (KC * EB) + 16 * (lane / NCP);
#pragma unroll
    for (int i = 0; i < XPL; ++i) r.x[i] = ld16(xs + (64 / NCP) * 16 * i);
  }

  __device__ static __forceinline__ void lstore(const Regs& r, uint8_t* buf, int lane) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int L = 64 * i + lane, j = L / PPR, slot = L % PPR;
      *reinterpret_cast<uint4*>(buf + j * (KC / 2) + 16 * slot) = r.c[i];
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int D = 64 * i + lane, j = D / SPR, dw = D % SPR;
      *reinterpret_cast<uint32_t*>(buf + CODE_B + j * (KC / 16) + 4 * dw) = r.s[i];
    }
    const int n = lane % NCP;
#pragma unroll
    for (int i = 0; i < XPL; ++i) {
      const int o = lane / NCP + (64 / NCP) * i;
      *reinterpret_cast<uint4*>(buf + W_B + (n * OCH + (o ^ (n & 7))) * 16) = r.x[i];
    }
  }

  // the products of K tile kt' of the stage in buf
  __device__ static __forceinline__ void tile(const uint8_t* buf, int ktp, f32x4 (&acc)[RT][NM], int g, int n) {
    uint4 x[TCH];
    const int nn = n % NCP;    // columns NCP.. repeat the first ones; their products are not stored
#pragma unroll
    for (int v = 0; v < TCH; ++v) {
      const int o = TCH * (4 * ktp + g) + v;
      x[v] = *reinterpret_cast<const uint4*>(buf + W_B + (nn * OCH + (o ^ (nn & 7))) * 16);
    }
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (GATEUP) {
        bh[q] = bf16x8_from_words(x[q]);
      } else {
        // h arrives split (store_h): 8 high parts, then their 8 low parts
        bh[q] = bf16x8_from_words(x[2 * q]);
        bl[q] = bf16x8_from_words(x[2 * q + 1]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int j = (rt * NM + m) * 16 + n;
        const int slot = (4 * ktp + g) ^ (j % PPR);
        const uint4 q4 = *reinterpret_cast<const uint4*>(buf + j * (KC / 2) + 16 * slot);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(buf + CODE_B + j * (KC / 16) + 8 * ktp + 2 * g);
        const f32x2 sw = scales2(sc);
        const float s0 = sw.x, s1 = sw.y;
        const uint32_t d[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8 av = fp4x8_scaled_bf16(d[q], q < 2 ? s0 : s1);
          acc[rt][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[q], acc[rt][m], 0, 0, 0);
          if (!GATEUP) acc[rt][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[q], acc[rt][m], 0, 0, 0);
        }
      }
    }
  }

  // LDS writes of this wavefront are complete and ordered before its later reads
  __device__ static __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // One LDS buffer per wavefront: a stage's writes follow the reads of the
  // stage before in the wavefront's own program order, and the LDS serves a
  // wavefront's accesses in that order.
  __device__ static __forceinline__ void run(const GemvArgs& a, uint8_t* lds) {
    int lo, U;
    launch_uniques(a, a.hdr[H_UNIQUE], lo, U);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int nwaves = gridDim.x * (kGemvThreads / 64);
    const int w = wave_id();
    const int gw = blockIdx.x * (kGemvThreads / 64) + w;
    uint8_t* buf = lds + (size_t)w * STAGE_B;
    const int ntiles = a.rows / 16;
    const int tpu = (ntiles + RT - 1) / RT;     // tasks per unique expert
    const int ntask = U * tpu;
    for (int task = gw; task < ntask; task += nwaves) {
      const int u = unique_at(a, lo, task / tpu), tg = task - (task / tpu) * tpu;
      const int tile0 = tg * RT;
      const int nt = ntiles - tile0 < RT ? ntiles - tile0 : RT;
      const uint8_t* blob = a.uniq_ptr[u];
      const float gs = a.gs[2 * a.uniq_expert[u] + (GATEUP ? 0 : 1)];
      const int off0 = a.uniq_off[u], off1 = a.uniq_off[u + 1];
      for (int c0 = off0; c0 < off1; c0 += NCP) {
        const int nc = off1 - c0 < NCP ? off1 - c0 : NCP;
        const bool live = n < nc;
        const int p = a.uniq_picks[c0 + (live ? n : nc - 1)];
        const int ln = lane % NCP;    // the column whose operand this lane loads
        const int pl = a.uniq_picks[c0 + (ln < nc ? ln : nc - 1)];
        const uint8_t* xsrc = static_cast<const uint8_t*>(a.operand) +
                              (GATEUP ? (size_t)(pl / a.k) * K * 2 : (size_t)pl * K * 4);
        f32x4 acc[RT][NM];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int m = 0; m < NM; ++m) acc[rt][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (TWO) {
        // two register stages in flight: RA and RB hold stages st + 1 and st + 2.
        // The steady-state loop issues its loads unconditionally (a skipped
        // load on one path makes the compiler wait for every load on both).
        Regs RA, RB;
        gload(RA, a, blob, xsrc, tile0, nt, 0, lane);
        lstore(RA, buf, lane);
        if (NS > 1) gload(RA, a, blob, xsrc, tile0, nt, 1, lane);
        if (NS > 2) gload(RB, a, blob, xsrc, tile0, nt, 2, lane);
        lds_sync();
        int st = 0;
        for (; st + 4 < NS; st += 2) {
#pragma unroll
          for (int ktp = 0; ktp < NKT; ++ktp) tile(buf, ktp, acc, g, n);
          lstore(RA, buf, lane);
          gload(RA, a, blob, xsrc, tile0, nt, st + 3, lane);
          lds_sync();
#pragma unroll
          for (int ktp = 0; ktp < NKT; ++ktp) tile(buf, ktp, acc, g, n);
          lstore(RB, buf, lane);
          gload(RB, a, blob, xsrc, tile0, nt, st + 4, lane);
          lds_sync();
        }
        // the last stages (at most four)
        while (true) {
#pragma unroll
          for (int ktp = 0; ktp < NKT; ++ktp) tile(buf, ktp, acc, g, n);
          if (st + 1 >= NS) break;
          lstore(RA, buf, lane);
          if (st + 3 < NS) gload(RA, a, blob, xsrc, tile0, nt, st + 3, lane);
          lds_sync();
          ++st;
#pragma unroll
          for (int ktp = 0; ktp < NKT; ++ktp) tile(buf, ktp, acc, g, n);
          if (st + 1 >= NS) break;
          lstore(RB, buf, lane);
          if (st + 3 < NS) gload(RB, a, blob, xsrc, tile0, nt, st + 3, lane);
          lds_sync();
          ++st;
        }
        } else {
        Regs R;
        gload(R, a, blob, xsrc, tile0, nt, 0, lane);
        lstore(R, buf, lane);
        if (NS > 1) gload(R, a, blob, xsrc, tile0, nt, 1, lane);
        lds_sync();
        for (int st = 0; st < NS; ++st) {
#pragma unroll
          for (int ktp = 0; ktp < NKT; ++ktp) tile(buf, ktp, acc, g, n);
          if (st + 1 < NS) {
            lstore(R, buf, lane);
            if (st + 2 < NS) gload(R, a, blob, xsrc, tile0, nt, st + 2, lane);
            lds_sync();
          }
        }
        }
        if (live) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if (rt >= nt) break;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              v[j] = GATEUP ? silu_f32(acc[rt][0][j] * gs) * (acc[rt][NM - 1][j] * gs) : acc[rt][0][j] * gs;
            const int r0 = (tile0 + rt) * 16 + 4 * g;      // r0 % 8 is 0 or 4
            float* row = a.out + (size_t)p * a.rows;
            if (GATEUP && a.split_h) {
              bf16x4 hi4, lo4;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                __bf16 h, l;
                split_bf16(v[j], h, l);
                hi4[j] = h;
                lo4[j] = l;
              }
              __bf16* grp = reinterpret_cast<__bf16*>(row) + (r0 / 8) * 16 + (r0 % 8);
              *reinterpret_cast<bf16x4*>(grp) = hi4;
              *reinterpret_cast<bf16x4*>(grp + 8) = lo4;
            } else {
              *reinterpret_cast<float4*>(row + r0) = make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
        // the next task's first stage overwrites the buffer this one has read
        lds_sync();
      }
    }
  }
};

// The matrix-core form for larger steps' down product: the weights are staged
// through two LDS buffers per wavefront as above, and each lane reads its
// pick column's operand slice from global memory one K tile ahead.  Tasks of
// 64 rows against 16 columns read the operand once per 64 weight rows.
constexpr int kLdsStageK = 256;

template <int K, bool GATEUP, int RT>
struct GemvMfmaX {
  static constexpr int NM = GATEUP ? 2 : 1;
  static constexpr int NROW = 16 * RT * NM;            // weight rows per task
  static constexpr int KC = K < kLdsStageK ? K : kLdsStageK;   // K elements per stage
  static constexpr int NS = K / KC;                    // stages
  static constexpr int PPR = KC / 32;                  // 16-byte code pieces per row and stage
  static constexpr int CPL = NROW * PPR / 64;          // code pieces per lane and stage
  static constexpr int SPR = KC / 64;                  // scale dwords per row and stage
  static constexpr int SPL = NROW * SPR / 64;          // scale dwords per lane and stage
  static constexpr int CODE_B = NROW * KC / 2;
  static constexpr int STAGE_B = CODE_B + NROW * KC / 16;
  static constexpr int NKT = KC / 128;                 // K tiles per stage
  static constexpr int NX = GATEUP ? 4 : 8;            // 16-byte operand loads per lane and K tile
  static_assert(K % KC == 0 && KC % 128 == 0 && CPL >= 1 && SPL >= 1, "unsupported K");
  static_assert(NKT == 1 || NKT % 2 == 0, "operand double buffer assumes an even tile count per stage");

  struct Regs {
    uint4 c[CPL];
    uint32_t s[SPL];
  };

  // global row of task row j (a ragged task re-reads its last tile)
  __device__ static __forceinline__ size_t grow(const GemvArgs& a, int tile0, int nt, int j) {
    const int rt = j / (16 * NM), m = (j / 16) % NM, n = j % 16;
    const int tile = tile0 + (rt < nt ? rt : nt - 1);
    return (size_t)(tile * 16 + n + m * a.up_row0);
  }

  __device__ static __forceinline__ void gload(Regs& r, const GemvArgs& a, const uint8_t* blob, int tile0, int nt,
                                               int stage, int lane) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int L = 64 * i + lane, j = L / PPR, slot = L % PPR;
      const int c = slot ^ (j % PPR);
      r.c[i] = ld16_stream(blob + a.code_off + grow(a, tile0, nt, j) * (K / 2) + stage * (KC / 2) + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int D = 64 * i + lane, j = D / SPR, dw = D % SPR;
      r.s[i] = *(const __attribute__((address_space(1))) uint32_t*)(blob + a.scale_off + grow(a, tile0, nt, j) * (K / 16) +
                                                                   stage * (KC / 16) + 4 * dw);
    }
  }

  __device__ static __forceinline__ void lstore(const Regs& r, uint8_t* buf, int lane) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int L = 64 * i + lane, j = L / PPR, slot = L % PPR;
      *reinterpret_cast<uint4*>(buf + j * (KC / 2) + 16 * slot) = r.c[i];
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int D = 64 * i + lane, j = D / SPR, dw = D % SPR;
      *reinterpret_cast<uint32_t*>(buf + CODE_B + j * (KC / 16) + 4 * dw) = r.s[i];
    }
  }

  // operand elements [128 kt + 32 g, +32) of the lane's pick (zero for an idle column)
  __device__ static __forceinline__ void xload(uint4 (&x)[NX], const uint8_t* xsrc, bool live, int kt, int g) {
    const uint8_t* src = xsrc + (size_t)(128 * kt + 32 * g) * (GATEUP ? 2 : 4);
#pragma unroll
    for (int v = 0; v < NX; ++v) {
      const uint4 t = ld16(src + 16 * v);
      x[v] = make_uint4(live ? t.x : 0u, live ? t.y : 0u, live ? t.z : 0u, live ? t.w : 0u);
    }
  }

  // the products of K tile kt' of the stage in buf
  __device__ static __forceinline__ void tile(const uint8_t* buf, int ktp, const uint4 (&x)[NX], f32x4 (&acc)[RT][NM],
                                              int g, int n) {
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (GATEUP) {
        bh[q] = bf16x8_from_words(x[q]);
      } else {
        // h arrives split (store_h): 8 high parts, then their 8 low parts
        bh[q] = bf16x8_from_words(x[2 * q]);
        bl[q] = bf16x8_from_words(x[2 * q + 1]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int j = (rt * NM + m) * 16 + n;
        const int slot = (4 * ktp + g) ^ (j % PPR);
        const uint4 q4 = *reinterpret_cast<const uint4*>(buf + j * (KC / 2) + 16 * slot);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(buf + CODE_B + j * (KC / 16) + 8 * ktp + 2 * g);
        const f32x2 sw = scales2(sc);
        const float s0 = sw.x, s1 = sw.y;
        const uint32_t d[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8 av = fp4x8_scaled_bf16(d[q], q < 2 ? s0 : s1);
          acc[rt][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[q], acc[rt][m], 0, 0, 0);
          if (!GATEUP) acc[rt][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[q], acc[rt][m], 0, 0, 0);
        }
      }
    }
  }

  // LDS writes of this wavefront are complete and ordered before its later reads
  __device__ static __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  __device__ static __forceinline__ void run(const GemvArgs& a, uint8_t* lds) {
    int lo, U;
    launch_uniques(a, a.hdr[H_UNIQUE], lo, U);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int nwaves = gridDim.x * (kGemvThreads / 64);
    const int w = wave_id();
    const int gw = blockIdx.x * (kGemvThreads / 64) + w;
    uint8_t* buf0 = lds + (size_t)w * 2 * STAGE_B;
    uint8_t* buf1 = buf0 + STAGE_B;
    const int ntiles = a.rows / 16;
    const int tpu = (ntiles + RT - 1) / RT;     // tasks per unique expert
    const int ntask = U * tpu;
    for (int task = gw; task < ntask; task += nwaves) {
      const int u = unique_at(a, lo, task / tpu), tg = task - (task / tpu) * tpu;
      const int tile0 = tg * RT;
      const int nt = ntiles - tile0 < RT ? ntiles - tile0 : RT;
      const uint8_t* blob = a.uniq_ptr[u];
      const float gs = a.gs[2 * a.uniq_expert[u] + (GATEUP ? 0 : 1)];
      const int off0 = a.uniq_off[u], off1 = a.uniq_off[u + 1];
      for (int c0 = off0; c0 < off1; c0 += 16) {
        const int nc = off1 - c0 < 16 ? off1 - c0 : 16;
        const bool live = n < nc;
        const int p = a.uniq_picks[c0 + (live ? n : nc - 1)];
        const uint8_t* xsrc = static_cast<const uint8_t*>(a.operand) +
                              (GATEUP ? (size_t)(p / a.k) * K * 2 : (size_t)p * K * 4);
        f32x4 acc[RT][NM];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int m = 0; m < NM; ++m) acc[rt][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        Regs R;
        uint4 xa[NX], xb[NX];
        gload(R, a, blob, tile0, nt, 0, lane);
        xload(xa, xsrc, live, 0, g);
        lstore(R, buf0, lane);
        if (NS > 1) gload(R, a, blob, tile0, nt, 1, lane);
        lds_sync();
        for (int st = 0; st < NS; ++st) {
          const uint8_t* cur = (st & 1) ? buf1 : buf0;
#pragma unroll
          for (int ktp = 0; ktp < NKT; ++ktp) {
            const int kt = st * NKT + ktp;
            // even tiles use xa, odd ones xb; the next tile's operand loads go to the other
            if ((ktp & 1) == 0) {
              if (kt + 1 < NS * NKT) xload(xb, xsrc, live, kt + 1, g);
              tile(cur, ktp, xa, acc, g, n);
            } else {
              if (kt + 1 < NS * NKT) xload(xa, xsrc, live, kt + 1, g);
              tile(cur, ktp, xb, acc, g, n);
            }
          }
          if (NKT == 1) {
            // one tile per stage: the next stage's operand is in xb; move it to xa
#pragma unroll
            for (int v = 0; v < NX; ++v) xa[v] = xb[v];
          }
          if (st + 1 < NS) {
            lstore(R, (st & 1) ? buf0 : buf1, lane);
            if (st + 2 < NS) gload(R, a, blob, tile0, nt, st + 2, lane);
            lds_sync();
          }
        }
        if (live) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if (rt >= nt) break;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              v[j] = GATEUP ? silu_f32(acc[rt][0][j] * gs) * (acc[rt][NM - 1][j] * gs) : acc[rt][0][j] * gs;
            const int r0 = (tile0 + rt) * 16 + 4 * g;      // r0 % 8 is 0 or 4
            float* row = a.out + (size_t)p * a.rows;
            if (GATEUP && a.split_h) {
              bf16x4 hi4, lo4;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                __bf16 h, l;
                split_bf16(v[j], h, l);
                hi4[j] = h;
                lo4[j] = l;
              }
              __bf16* grp = reinterpret_cast<__bf16*>(row) + (r0 / 8) * 16 + (r0 % 8);
              *reinterpret_cast<bf16x4*>(grp) = hi4;
              *reinterpret_cast<bf16x4*>(grp + 8) = lo4;
            } else {
              *reinterpret_cast<float4*>(row + r0) = make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
        // the next task's first stage overwrites buf0, which this one may still be reading
        lds_sync();
      }
    }
  }
};


// Matrix-core task shapes, by the number NCP of pick columns a pass computes.
// Steps of up to 8 rows (NCP = 8): gate/up tasks are one gate and one up tile
// with two register stages in flight; down tasks are two tiles (32 rows) with
// one.  Larger steps (NCP = 16; an expert has up to 16 picks on a cached step):
// gate/up as above with one register stage; down tasks are four tiles (64
// rows) whose operand comes from global memory one K tile ahead (GemvMfmaX),
// which halves the operand traffic per weight byte.  All stages are 256 wide.
// Each wavefront's LDS holds 8.5 to 18 KiB, so that two or three blocks of
// four wavefronts fit a compute unit, as many as their registers allow.
constexpr int kMfmaStage = 256;
template <int K, bool GATEUP, int NCP>
using MfmaTask = typename std::conditional<
    GATEUP, GemvMfmaL<K, true, 1, kMfmaStage, NCP, NCP == 8>,
    typename std::conditional<NCP == 8, GemvMfmaL<K, false, 2, kMfmaStage, 8, false>,
                              GemvMfmaX<K, false, 4>>::type>::type;
// 16-row tiles per task
constexpr int mfma_tiles(bool gateup, int ncp) { return gateup ? 1 : ncp == 8 ? 2 : 4; }

template <int K, bool GATEUP, int NCP>
constexpr int mfma_lds_bytes() {
  return (kGemvThreads / 64) * (!GATEUP && NCP == 16 ? 2 : 1) * MfmaTask<K, GATEUP, NCP>::STAGE_B;
}

template <int K, bool GATEUP, int NCP>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_mfma_lds(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[mfma_lds_bytes<K, GATEUP, NCP>()];
  span_start(a.span);
  MfmaTask<K, GATEUP, NCP>::run(a, lds);
  span_end(a.span);
}


// Copies the step's missed blobs (host-mapped pinned memory -> HBM slots), or
// one group of a staged prefill step's experts into the staging blobs (group
// >= 0).  The copies' 16-byte chunks form one index space so every thread
// keeps four loads in flight across blob boundaries; with nothing to copy it
// exits.  Entries whose destination is null (a miss the remap could not
// place) are skipped.
// The copy runs over `vgrid` blocks of 256 threads, of which this is `vblock`.
__device__ __forceinline__ void fill_body(const int32_t* hdr, const uint8_t* const* src, uint8_t* const* dst,
                                          long n16, int group, int G, int vblock, int vgrid) {
  int first = 0, count = hdr[H_MISS];
  if (group >= 0) {
    const int ns = hdr[H_STAGED];
    first = group * G;
    count = ns < first + G ? ns - first : G;
    if (count < 0) count = 0;
  }
  src += first;
  dst += first;
  const long total = (long)count * n16;
  const long stride = (long)vgrid * blockDim.x;
  long o = (long)vblock * blockDim.x + threadIdx.x;
  for (; o + 3 * stride < total; o += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long g = o + j * stride, i = g / n16;
      if (dst[i]) v[j] = ld16(src[i] + (g - i * n16) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long g = o + j * stride, i = g / n16;
      if (dst[i]) *reinterpret_cast<uint4*>(dst[i] + (g - i * n16) * 16) = v[j];
    }
  }
  for (; o < total; o += stride) {
    const long i = o / n16;
    if (dst[i]) *reinterpret_cast<uint4*>(dst[i] + (o - i * n16) * 16) = ld16(src[i] + (o - i * n16) * 16);
  }
}

__global__ __launch_bounds__(256) void k_fill(const int32_t* hdr, const uint8_t* const* src,
                                               uint8_t* const* dst, long n16, int group, int G, uint64_t* span) {
  span_start(span);
  fill_body(hdr, src, dst, n16, group, G, blockIdx.x, gridDim.x);
  span_end(span);
}

// Overlapped fill of a one-row step.  The copy is bound by the host link, and
// a concurrent HBM stream does not slow it, so the experts it does not write
// are computed while it runs: blocks [0, nb_fill) copy the misses into their
// slots (first, so that they start at once), the others compute gate/up for
// the resident experts.  The copied experts' gate/up follows in
// k_gemv_filled.  The pages name asynchronous miss fills as what could cut
// the copy's cost ("GB300 GLM 5.3 Testing", September 13 update of
// "Speculation: what is holding the GB300 back, and what probably wins next").
struct FillArgs {
  const int32_t* hdr;
  const uint8_t* const* src;
  uint8_t* const* dst;
  long n16;
  uint64_t* span;
};

template <int K>
__global__ __launch_bounds__(kGemvThreads) void k_fill_gateup(FillArgs f, GemvArgs a, int nb_fill) {
  const int b = blockIdx.x;
  if (b < nb_fill) {
    span_start(f.span, b);
    fill_body(f.hdr, f.src, f.dst, f.n16, -1, 0, b, nb_fill);
    span_end(f.span, b);
  } else {
    span_start(a.span, b - nb_fill);
    Gemv<K, 1, 1, true, true, 1>::run(a, b - nb_fill, gridDim.x - nb_fill);
    span_end(a.span, b - nb_fill);
  }
}

template <int K>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_filled(GemvArgs a) {
  Gemv<K, 1, 1, true, true, 2>::run(a, blockIdx.x, gridDim.x);
}

// y[m][r] = sum over j = 0..k-1 of w[m][j] * part[m*k + j][r], in rank order.
__global__ __launch_bounds__(256) void k_combine(const float* part, const float* w, float* y,
                                                  int M, int k, int H, uint64_t* span) {
  span_start(span);
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx < (long)M * H) {
    const int m = (int)(idx / H), r = (int)(idx - (long)m * H);
    const float* pp = part + (size_t)m * k * H + r;
    const float* wm = w + m * k;
    float acc = 0.0f;
    int j = 0;
    // eight partial loads in flight at a time; the sum keeps rank order
    for (; j + 8 <= k; j += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = pp[(size_t)(j + i) * H];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(wm[j + i], v[i], acc);
    }
    for (; j < k; ++j) acc = fmaf(wm[j], pp[(size_t)j * H], acc);
    y[idx] = acc;
  }
  span_end(span);
}

typedef void (*GemvFn)(GemvArgs);

// Row steps per pipeline stage: as many as the row group can reduce at once, at most 4 for down (measured
// against 2 and 8 on the GLM layer at M = 1: 12.7 against 13.6 and 13.3 us), 1 for gate/up.
template <int K, int MR, bool GATEUP>
constexpr int stage_rows() {
  constexpr int lim = Geo<K>::LPR / MR;
  constexpr int want = GATEUP ? 1 : MR > 2 ? 2 : 4;
  return want < lim ? want : lim;
}

template <int K, int MR, bool GATEUP, bool SINGLE>
GemvFn gemv_fn() {
  return k_gemv<K, MR, stage_rows<K, MR, GATEUP>(), GATEUP, SINGLE>;
}

// MR = 0 selects the one-row variant (one pick per expert, U = k).
template <bool GATEUP, int MR>
GemvFn pick_gemv(int K) {
  constexpr int mr = MR == 0 ? 1 : MR;
  constexpr bool single = MR == 0;
  switch (K) {
    case 128: return GATEUP ? nullptr : gemv_fn<128, mr, GATEUP, single>();
    case 256: return gemv_fn<256, mr, GATEUP, single>();
    case 512: return gemv_fn<512, mr, GATEUP, single>();
    case 1024: return gemv_fn<1024, mr, GATEUP, single>();
    case 2048: return gemv_fn<2048, mr, GATEUP, single>();
    case 4096: return gemv_fn<4096, mr, GATEUP, single>();
    case 6144: return gemv_fn<6144, mr, GATEUP, single>();
    case 8192: return gemv_fn<8192, mr, GATEUP, single>();
    default: return nullptr;
  }
}

int rows_per_wave(int K) { return K >= 2048 ? 1 : 2048 / K; }
int stage_rows_rt(int K, int MR, bool gateup) {
  const int lpr = K >= 2048 ? 64 : K / 32;
  const int want = gateup ? 1 : MR > 2 ? 2 : 4;
  return want < lpr / MR ? want : lpr / MR;
}

// Enough wavefronts for about two pipeline stages each, capped per kernel.
int gemv_blocks(long stages, int cap) {
  long blocks = (stages + 7) / 8;
  if (blocks < 1) blocks = 1;
  if (blocks > cap) blocks = cap;
  return (int)blocks;
}

// The gate/up kernels hold about 152 VGPRs, three wavefronts per SIMD: 768
// blocks of four wavefronts are all resident at once.  With 1024 the last 256
// blocks only started once the first ones had finished (about 12 us in) and
// streamed alone at the end (GLM layer, M=1: 21.2 against 20.6 us).
constexpr int kGateupBlocks = 768;
// Copy blocks.  Two per compute unit (8 MiB of host reads in flight) move
// 56.0 GB/s over the host link against 55.5 with one per compute unit (GLM
// layer, M=1, miss steps; 1% off the mean step).  A launch that shares its
// compute units with gate/up products (the overlapped fill) takes one per
// compute unit, so that the products keep two of their three wave slots.
constexpr int kFillBlocks = 512;
constexpr int kFillBlocksShared = 256;
constexpr int kDownBlocks = 512;
// Shared-operand streaming kernels (steps of 2 to 4 rows): 146 to 153 VGPRs
// and 32 to 48 KiB of LDS, three blocks per compute unit, so 768 blocks are
// all resident (down at M = 4 with 512 blocks: 44.6 against 36.4 us).
constexpr int kSharedBlocks = 768;

int mr_for(int M) { return M == 1 ? 1 : 2; }

// Rows per step from which each product runs on the matrix cores (all-hit GLM
// layer, drafted rows, µs per kernel, streaming against matrix cores): gate/up
// 45 / 56 at M = 2, 65 / 58 at 3, 80 / 73 at 4; down 39 / 39 at M = 2, 62 / 41
// at 3.  The two-pick streaming kernels hold 300-480 VGPRs (one wavefront per
// SIMD).
constexpr int kMfmaMinRowsGateup = SC_MFMA_MIN_ROWS_GATEUP;
constexpr int kMfmaMinRowsDown = SC_MFMA_MIN_ROWS_DOWN;

template <bool GATEUP, int NCP>
GemvFn pick_mfma_n(int K) {
  switch (K) {
    case 128: return GATEUP ? nullptr : k_gemv_mfma_lds<128, GATEUP, NCP>;
    case 256: return k_gemv_mfma_lds<256, GATEUP, NCP>;
    case 512: return k_gemv_mfma_lds<512, GATEUP, NCP>;
    case 1024: return k_gemv_mfma_lds<1024, GATEUP, NCP>;
    case 2048: return k_gemv_mfma_lds<2048, GATEUP, NCP>;
    case 4096: return k_gemv_mfma_lds<4096, GATEUP, NCP>;
    case 6144: return k_gemv_mfma_lds<6144, GATEUP, NCP>;
    case 8192: return k_gemv_mfma_lds<8192, GATEUP, NCP>;
    default: return nullptr;
  }
}
// Pick columns per matrix-core pass for a step of M rows (a cached step gives
// an expert at most M picks).
int mfma_columns(int M) { return M <= 8 ? 8 : 16; }
template <bool GATEUP>
GemvFn pick_mfma(int K, int ncp) { return ncp == 8 ? pick_mfma_n<GATEUP, 8>(K) : pick_mfma_n<GATEUP, 16>(K); }

// One wavefront per task (RT 16-row tiles of one expert), at most cap blocks.
constexpr int kMfmaBlocksGateup = 768;
constexpr int kMfmaBlocksDown = 512;
int mfma_blocks(long maxu, int rows, int rt, int cap) {
  const long tasks = maxu * ((rows / 16 + rt - 1) / rt);
  long blocks = (tasks + 3) / 4;
  if (blocks < 1) blocks = 1;
  if (blocks > cap) blocks = cap;
  return (int)blocks;
}

// Shared-operand streaming kernels (steps of 2 .. kSharedPicks rows): row
// steps per pipeline stage as the one-row kernels take them, within what the
// row group can reduce for kSharedPicks picks; null where the operand rows of
// kSharedPicks picks would not fit 64 KiB of LDS.
template <int K, bool GATEUP>
constexpr int shared_rows() {
  constexpr int lim = Geo<K>::LPR / kSharedPicks;
  constexpr int want = GATEUP ? 1 : 2;
  return want < lim ? want : lim;
}
template <int K, bool GATEUP>
GemvFn shared_fn() {
  if constexpr (GemvShared<K, shared_rows<K, GATEUP>(), GATEUP>::LDS_B > 65536) return nullptr;
  else return k_gemv_shared<K, shared_rows<K, GATEUP>(), GATEUP>;
}
template <bool GATEUP>
GemvFn pick_shared(int K) {
  switch (K) {
    case 128: return GATEUP ? nullptr : shared_fn<128, GATEUP>();
    case 256: return shared_fn<256, GATEUP>();
    case 512: return shared_fn<512, GATEUP>();
    case 1024: return shared_fn<1024, GATEUP>();
    case 2048: return shared_fn<2048, GATEUP>();
    case 4096: return shared_fn<4096, GATEUP>();
    case 6144: return shared_fn<6144, GATEUP>();
    case 8192: return shared_fn<8192, GATEUP>();
    default: return nullptr;
  }
}
// A step of 2 .. kSharedPicks rows gives each expert at most M picks (cached or bypass).
bool shared_step(int M, int group) { return M >= 2 && M <= kSharedPicks && group < 0; }

}  // namespace

bool gemv_supported(int K, bool gateup) {
  return gateup ? pick_gemv<true, 0>(K) != nullptr : pick_gemv<false, 0>(K) != nullptr;
}

hipError_t launch_fill(const Shape& sh, const Workspace& W, int group, hipStream_t st, KEvents ev) {
  return sc_launch(k_fill, dim3(kFillBlocks), dim3(256), st, ev, (const int32_t*)W.hdr,
                   (const uint8_t* const*)W.miss_src, (uint8_t* const*)W.miss_dst, (long)(sh.blob / 16), group,
                   (int)W.stage_n, ev.span_for(kFillBlocks));
}

static GemvArgs base_args(const Workspace& W, const float* gs, int group) {
  GemvArgs a;
  a.hdr = W.hdr;
  a.uniq_ptr = W.uniq_ptr;
  a.uniq_expert = W.uniq_expert;
  a.gs = gs;
  a.uniq_off = W.uniq_off;
  a.uniq_picks = W.uniq_picks;
  a.span = nullptr;
  a.order = W.uniq_order;
  a.group = group;
  a.G = W.stage_n;
  a.split_h = 0;
  return a;
}

static GemvArgs gateup_args(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x, int group) {
  GemvArgs a = base_args(W, gs, group);
  a.operand = x;
  a.out = W.h;
  a.rows = sh.I;
  a.k = sh.k;
  a.up_row0 = sh.I;
  a.code_off = 0;
  a.scale_off = sh.off_w13s;
  return a;
}

hipError_t launch_gateup(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x, int M,
                         bool mfma, int group, hipStream_t st, KEvents ev) {
  GemvArgs a = gateup_args(sh, W, gs, x, group);
  a.split_h = mfma && M >= kMfmaMinRowsDown;   // the down product of this step runs on the matrix cores
  const long maxu = (long)(M * sh.k < sh.E ? M * sh.k : sh.E);
  if (shared_step(M, group) && pick_shared<true>(sh.H)) {
    const int blocks = gemv_blocks(maxu * (sh.I / rows_per_wave(sh.H)), kSharedBlocks);
    a.span = ev.span_for(blocks);
    return sc_launch(pick_shared<true>(sh.H), dim3(blocks), dim3(kGemvThreads), st, ev, a);
  }
  if (mfma && M >= kMfmaMinRowsGateup) {
    const int ncp = mfma_columns(M);
    GemvFn fn = pick_mfma<true>(sh.H, ncp);
    if (!fn) return hipErrorInvalidValue;
    const int blocks = mfma_blocks(maxu, sh.I, mfma_tiles(true, ncp), kMfmaBlocksGateup);
    a.span = ev.span_for(blocks);
    return sc_launch(fn, dim3(blocks), dim3(kGemvThreads), st, ev, a);
  }
  const int mr = mr_for(M);
  GemvFn fn = M == 1 ? pick_gemv<true, 0>(sh.H) : pick_gemv<true, 2>(sh.H);
  if (!fn) return hipErrorInvalidValue;
  const long stages = maxu * (sh.I / rows_per_wave(sh.H)) / stage_rows_rt(sh.H, mr, true);
  const int blocks = gemv_blocks(stages, kGateupBlocks);
  a.span = ev.span_for(blocks);
  return sc_launch(fn, dim3(blocks), dim3(kGemvThreads), st, ev, a);
}

typedef void (*FillGateupFn)(FillArgs, GemvArgs, int);

static FillGateupFn pick_fill_gateup(int K) {
  switch (K) {
    case 256: return k_fill_gateup<256>;
    case 512: return k_fill_gateup<512>;
    case 1024: return k_fill_gateup<1024>;
    case 2048: return k_fill_gateup<2048>;
    case 4096: return k_fill_gateup<4096>;
    case 6144: return k_fill_gateup<6144>;
    case 8192: return k_fill_gateup<8192>;
    default: return nullptr;
  }
}

static GemvFn pick_gemv_filled(int K) {
  switch (K) {
    case 256: return k_gemv_filled<256>;
    case 512: return k_gemv_filled<512>;
    case 1024: return k_gemv_filled<1024>;
    case 2048: return k_gemv_filled<2048>;
    case 4096: return k_gemv_filled<4096>;
    case 6144: return k_gemv_filled<6144>;
    case 8192: return k_gemv_filled<8192>;
    default: return nullptr;
  }
}

// Product blocks of a one-row gate/up launch (as launch_gateup picks them).
static int one_row_gateup_blocks(const Shape& sh) {
  const long maxu = sh.k < sh.E ? sh.k : sh.E;
  return gemv_blocks(maxu * (sh.I / rows_per_wave(sh.H)) / stage_rows_rt(sh.H, 1, true), kGateupBlocks);
}

hipError_t launch_fill_gateup(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x,
                              hipStream_t st, KEvents ev_fill, KEvents ev) {
  FillGateupFn fn = pick_fill_gateup(sh.H);
  if (!fn) return hipErrorInvalidValue;
  GemvArgs a = gateup_args(sh, W, gs, x, -1);
  // the product blocks fit beside the copy blocks (three blocks per compute
  // unit at this kernel's registers), so none waits for the copy to end
  int blocks = one_row_gateup_blocks(sh);
  if (blocks > kGateupBlocks - kFillBlocksShared) blocks = kGateupBlocks - kFillBlocksShared;
  a.span = ev.span_for(blocks);
  FillArgs f;
  f.hdr = W.hdr;
  f.src = W.miss_src;
  f.dst = W.miss_dst;
  f.n16 = (long)(sh.blob / 16);
  f.span = ev_fill.span_for(kFillBlocksShared);
  return sc_launch(fn, dim3(kFillBlocksShared + blocks), dim3(kGemvThreads), st, ev, f, a, kFillBlocksShared);
}

hipError_t launch_gateup_filled(const Shape& sh, const Workspace& W, const float* gs, const uint16_t* x,
                                hipStream_t st) {
  GemvFn fn = pick_gemv_filled(sh.H);
  if (!fn) return hipErrorInvalidValue;
  return sc_launch(fn, dim3(one_row_gateup_blocks(sh)), dim3(kGemvThreads), st, KEvents(),
                   gateup_args(sh, W, gs, x, -1));
}

hipError_t launch_down(const Shape& sh, const Workspace& W, const float* gs, int M, bool mfma, int group,
                       hipStream_t st, KEvents ev) {
  GemvArgs a = base_args(W, gs, group);
  a.operand = W.h;
  a.out = W.part;
  a.rows = sh.H;
  a.k = sh.k;
  a.up_row0 = 0;
  a.code_off = sh.off_w2c;
  a.scale_off = sh.off_w2s;
  const long maxu = (long)(M * sh.k < sh.E ? M * sh.k : sh.E);
  if (mfma && M >= kMfmaMinRowsDown) {
    const int ncp = mfma_columns(M);
    GemvFn fn = pick_mfma<false>(sh.I, ncp);
    if (!fn) return hipErrorInvalidValue;
    const int blocks = mfma_blocks(maxu, sh.H, mfma_tiles(false, ncp), kMfmaBlocksDown);
    a.span = ev.span_for(blocks);
    return sc_launch(fn, dim3(blocks), dim3(kGemvThreads), st, ev, a);
  }
  if (shared_step(M, group)) {
    if (GemvFn fn = pick_shared<false>(sh.I)) {
      const int blocks = gemv_blocks(maxu * (sh.H / rows_per_wave(sh.I)), kSharedBlocks);
      a.span = ev.span_for(blocks);
      return sc_launch(fn, dim3(blocks), dim3(kGemvThreads), st, ev, a);
    }
    if (GemvFn fn = pick_gemv<false, 4>(sh.I)) {
      // operand rows too large for LDS: four picks' slices in registers
      const int blocks = gemv_blocks(maxu * (sh.H / rows_per_wave(sh.I)) / stage_rows_rt(sh.I, 4, false), kDownBlocks);
      a.span = ev.span_for(blocks);
      return sc_launch(fn, dim3(blocks), dim3(kGemvThreads), st, ev, a);
    }
  }
  const int mr = mr_for(M);
  GemvFn fn = M == 1 ? pick_gemv<false, 0>(sh.I) : pick_gemv<false, 2>(sh.I);
  if (!fn) return hipErrorInvalidValue;
  const long stages = maxu * (sh.H / rows_per_wave(sh.I)) / stage_rows_rt(sh.I, mr, false);
  const int blocks = gemv_blocks(stages, kDownBlocks);
  a.span = ev.span_for(blocks);
  return sc_launch(fn, dim3(blocks), dim3(kGemvThreads), st, ev, a);
}

hipError_t launch_combine(const Shape& sh, const Workspace& W, float* y, int M, hipStream_t st,
                          KEvents ev) {
  const long n = (long)M * sh.H;
  const long blocks = (n + 255) / 256;
  return sc_launch(k_combine, dim3((unsigned)blocks), dim3(256), st, ev, (const float*)W.part,
                   (const float*)W.pick_w, y, M, sh.k, sh.H, ev.span_for(blocks));
}

}  // namespace sc
