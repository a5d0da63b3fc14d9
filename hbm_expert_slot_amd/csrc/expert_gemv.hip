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
  const float* uniq_gs;
  const int32_t* uniq_off;
  const int32_t* uniq_picks;
  const void* operand;   // gate/up: bf16 x [M][H]; down: fp32 h [P][I]
  float* out;            // gate/up: h [P][I];      down: part [P][H]
  int rows;              // output rows per expert: I (gate/up) or H (down)
  int k;                 // top-k: pick p belongs to row p / k
  int up_row0;           // gate/up: first up row (I)
  int64_t code_off;      // offset of the code rows inside a blob
  int64_t scale_off;     // offset of the scale rows inside a blob
};

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

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

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum over one lane's 32 elements of one chunk: codes q (16 B), two block
// scales in sc (bytes 0, 1), bf16 activation pairs xv[16].
__device__ __forceinline__ float seg_dot_bf16(const uint4& q, uint32_t sc, const uint32_t* xv) {
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
        acc = __builtin_amdgcn_fdot2_f32_bf16(w[sel], xx, acc, false);
      }
    }
    b[blk] = acc;
  }
  const float s0 = __builtin_amdgcn_cvt_f32_fp8(sc, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8(sc, 1);
  return fmaf(b[1], s1, b[0] * s0);
}

// Same with fp32 activations hv[32].
__device__ __forceinline__ float seg_dot_f32(const uint4& q, uint32_t sc, const float* hv) {
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
  const float s0 = __builtin_amdgcn_cvt_f32_fp8(sc, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8(sc, 1);
  return fmaf(b[1], s1, b[0] * s0);
}

template <int K, int MR, bool GATEUP>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvArgs a) {
  using G = Geo<K>;
  constexpr int NSEG = G::NSEG, LPR = G::LPR, RPW = G::RPW;
  constexpr int OPW = GATEUP ? 16 : 32;   // operand words per lane per chunk
  const int U = a.hdr[H_UNIQUE];
  const int lane = threadIdx.x & 63;
  const int seg = lane % LPR, rsub = lane / LPR;
  const long nwaves = (long)gridDim.x * (kGemvThreads / 64);
  const long gw = (long)blockIdx.x * (kGemvThreads / 64) + (threadIdx.x >> 6);
  const int spu = a.rows / RPW;
  const long items = (long)U * spu;
  const long per = (items + nwaves - 1) / nwaves;
  long it = gw * per;
  const long end = items < it + per ? items : it + per;

  while (it < end) {
    const int u = (int)(it / spu);
    const long uend = end < (long)(u + 1) * spu ? end : (long)(u + 1) * spu;
    const uint8_t* blob = a.uniq_ptr[u];
    const float gs = a.uniq_gs[2 * u + (GATEUP ? 0 : 1)];
    const int off0 = a.uniq_off[u], off1 = a.uniq_off[u + 1];
    for (int c0 = off0; c0 < off1; c0 += MR) {
      const int nc = off1 - c0 < MR ? off1 - c0 : MR;
      int pk[MR];
      uint32_t opw[MR][NSEG][OPW];
#pragma unroll
      for (int mi = 0; mi < MR; ++mi) {
        pk[mi] = mi < nc ? a.uniq_picks[c0 + mi] : 0;
        if (mi < nc) {
#pragma unroll
          for (int c = 0; c < NSEG; ++c) {
            const int e0 = c * 2048 + seg * 32;
            const uint4* src;
            if (GATEUP) {
              const int m = pk[mi] / a.k;
              src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.operand) +
                                                   (size_t)m * K + e0);
            } else {
              src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.operand) +
                                                   (size_t)pk[mi] * K + e0);
            }
#pragma unroll
            for (int v = 0; v < OPW / 4; ++v) {
              uint4 t = src[v];
              opw[mi][c][4 * v + 0] = t.x;
              opw[mi][c][4 * v + 1] = t.y;
              opw[mi][c][4 * v + 2] = t.z;
              opw[mi][c][4 * v + 3] = t.w;
            }
          }
        } else {
#pragma unroll
          for (int c = 0; c < NSEG; ++c)
#pragma unroll
            for (int v = 0; v < OPW; ++v) opw[mi][c][v] = 0u;
        }
      }
      for (long i2 = it; i2 < uend; ++i2) {
        const int r = (int)(i2 - (long)u * spu) * RPW + rsub;
        if (GATEUP) {
          const uint8_t* cg = blob + a.code_off + (size_t)r * (K / 2) + seg * 16;
          const uint8_t* cu = blob + a.code_off + (size_t)(a.up_row0 + r) * (K / 2) + seg * 16;
          const uint8_t* sg = blob + a.scale_off + (size_t)r * (K / 16) + seg * 2;
          const uint8_t* su = blob + a.scale_off + (size_t)(a.up_row0 + r) * (K / 16) + seg * 2;
          uint4 qg[NSEG], qu[NSEG];
          uint32_t scg[NSEG], scu[NSEG];
#pragma unroll
          for (int c = 0; c < NSEG; ++c) {
            qg[c] = *reinterpret_cast<const uint4*>(cg + c * 1024);
            qu[c] = *reinterpret_cast<const uint4*>(cu + c * 1024);
            scg[c] = *reinterpret_cast<const uint16_t*>(sg + c * 128);
            scu[c] = *reinterpret_cast<const uint16_t*>(su + c * 128);
          }
          float ag[MR], au[MR];
#pragma unroll
          for (int mi = 0; mi < MR; ++mi) {
            ag[mi] = 0.0f;
            au[mi] = 0.0f;
            if (mi < nc) {
#pragma unroll
              for (int c = 0; c < NSEG; ++c) {
                ag[mi] += seg_dot_bf16(qg[c], scg[c], opw[mi][c]);
                au[mi] += seg_dot_bf16(qu[c], scu[c], opw[mi][c]);
              }
            }
            ag[mi] = group_sum<LPR>(ag[mi]);
            au[mi] = group_sum<LPR>(au[mi]);
          }
          if (seg == 0) {
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
              if (mi < nc)
                a.out[(size_t)pk[mi] * a.rows + r] = silu_f32(ag[mi] * gs) * (au[mi] * gs);
          }
        } else {
          const uint8_t* cd = blob + a.code_off + (size_t)r * (K / 2) + seg * 16;
          const uint8_t* sd = blob + a.scale_off + (size_t)r * (K / 16) + seg * 2;
          uint4 qd[NSEG];
          uint32_t scd[NSEG];
#pragma unroll
          for (int c = 0; c < NSEG; ++c) {
            qd[c] = *reinterpret_cast<const uint4*>(cd + c * 1024);
            scd[c] = *reinterpret_cast<const uint16_t*>(sd + c * 128);
          }
          float ad[MR];
#pragma unroll
          for (int mi = 0; mi < MR; ++mi) {
            ad[mi] = 0.0f;
            if (mi < nc) {
#pragma unroll
              for (int c = 0; c < NSEG; ++c)
                ad[mi] += seg_dot_f32(qd[c], scd[c], reinterpret_cast<const float*>(opw[mi][c]));
            }
            ad[mi] = group_sum<LPR>(ad[mi]);
          }
          if (seg == 0) {
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
              if (mi < nc) a.out[(size_t)pk[mi] * a.rows + r] = ad[mi] * gs;
          }
        }
      }
    }
    it = uend;
  }
}

__global__ __launch_bounds__(256) void k_fill(const int32_t* hdr, const uint8_t* const* src,
                                               uint8_t* const* dst, long n16) {
  const int nmiss = hdr[H_MISS];
  const long stride = (long)gridDim.x * blockDim.x;
  const long t0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = 0; i < nmiss; ++i) {
    const uint4* s = reinterpret_cast<const uint4*>(src[i]);
    uint4* d = reinterpret_cast<uint4*>(dst[i]);
    long o = t0;
    for (; o + 3 * stride < n16; o += 4 * stride) {   // four 16-byte loads in flight
      const uint4 v0 = s[o], v1 = s[o + stride], v2 = s[o + 2 * stride], v3 = s[o + 3 * stride];
      d[o] = v0;
      d[o + stride] = v1;
      d[o + 2 * stride] = v2;
      d[o + 3 * stride] = v3;
    }
    for (; o < n16; o += stride) d[o] = s[o];
  }
}

__global__ __launch_bounds__(256) void k_combine(const float* part, const float* w, float* y,
                                                  int M, int k, int H) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)M * H) return;
  const int m = (int)(idx / H), r = (int)(idx - (long)m * H);
  float acc = 0.0f;
  for (int j = 0; j < k; ++j) acc = fmaf(w[m * k + j], part[(size_t)(m * k + j) * H + r], acc);
  y[idx] = acc;
}

typedef void (*GemvFn)(GemvArgs);

template <bool GATEUP, int MR>
GemvFn pick_gemv(int K) {
  switch (K) {
    case 128: return GATEUP ? nullptr : k_gemv<128, MR, GATEUP>;
    case 256: return k_gemv<256, MR, GATEUP>;
    case 512: return k_gemv<512, MR, GATEUP>;
    case 1024: return k_gemv<1024, MR, GATEUP>;
    case 2048: return k_gemv<2048, MR, GATEUP>;
    case 4096: return k_gemv<4096, MR, GATEUP>;
    case 6144: return k_gemv<6144, MR, GATEUP>;
    case 8192: return k_gemv<8192, MR, GATEUP>;
    default: return nullptr;
  }
}

int rows_per_wave(int K) { return K >= 2048 ? 1 : 2048 / K; }

int gemv_blocks(long items) {
  long waves = (items + 3) / 4;   // at least four row-steps per wavefront
  long blocks = (waves + 3) / 4;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  return (int)blocks;
}

int mr_for(int M) { return M == 1 ? 1 : 2; }

}  // namespace

bool gemv_supported(int K, bool gateup) {
  return gateup ? pick_gemv<true, 1>(K) != nullptr : pick_gemv<false, 1>(K) != nullptr;
}

hipError_t launch_fill(const Shape& sh, const Workspace& W, hipStream_t st) {
  hipLaunchKernelGGL(k_fill, dim3(512), dim3(256), 0, st, W.hdr, W.miss_src, W.miss_dst,
                     (long)(sh.blob / 16));
  return hipGetLastError();
}

hipError_t launch_gateup(const Shape& sh, const Workspace& W, const uint16_t* x, int M,
                         hipStream_t st) {
  GemvArgs a;
  a.hdr = W.hdr;
  a.uniq_ptr = W.uniq_ptr;
  a.uniq_gs = W.uniq_gs;
  a.uniq_off = W.uniq_off;
  a.uniq_picks = W.uniq_picks;
  a.operand = x;
  a.out = W.h;
  a.rows = sh.I;
  a.k = sh.k;
  a.up_row0 = sh.I;
  a.code_off = 0;
  a.scale_off = sh.off_w13s;
  const int mr = mr_for(M);
  GemvFn fn = mr == 1 ? pick_gemv<true, 1>(sh.H) : pick_gemv<true, 2>(sh.H);
  if (!fn) return hipErrorInvalidValue;
  const long maxu = (long)(M * sh.k < sh.E ? M * sh.k : sh.E);
  const int blocks = gemv_blocks(maxu * (sh.I / rows_per_wave(sh.H)));
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kGemvThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_down(const Shape& sh, const Workspace& W, int M, hipStream_t st) {
  GemvArgs a;
  a.hdr = W.hdr;
  a.uniq_ptr = W.uniq_ptr;
  a.uniq_gs = W.uniq_gs;
  a.uniq_off = W.uniq_off;
  a.uniq_picks = W.uniq_picks;
  a.operand = W.h;
  a.out = W.part;
  a.rows = sh.H;
  a.k = sh.k;
  a.up_row0 = 0;
  a.code_off = sh.off_w2c;
  a.scale_off = sh.off_w2s;
  const int mr = mr_for(M);
  GemvFn fn = mr == 1 ? pick_gemv<false, 1>(sh.I) : pick_gemv<false, 2>(sh.I);
  if (!fn) return hipErrorInvalidValue;
  const long maxu = (long)(M * sh.k < sh.E ? M * sh.k : sh.E);
  const int blocks = gemv_blocks(maxu * (sh.H / rows_per_wave(sh.I)));
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kGemvThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& sh, const Workspace& W, float* y, int M, hipStream_t st) {
  const long n = (long)M * sh.H;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, W.part,
                     W.pick_w, y, M, sh.k, sh.H);
  return hipGetLastError();
}

}  // namespace sc
