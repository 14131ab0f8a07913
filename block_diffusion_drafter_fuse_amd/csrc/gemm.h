// MFMA GEMM  C[m, f] = sum_k A[m, k] * W[f, k]  with fused epilogues.
//
// W is a "virtual" weight: the concatenation of up to kMaxSeg [rows, K]
// matrices (e.g. [W_q; W_kb; W_vb]).  A is [M, K] with K optionally split into
// segments at separate addresses (the L tapped target layers of the fusion
// step, concatenated along features without a copy).
//
// Each wave owns FM x FN MFMA tiles (16 tokens x 16 features each): W rows are
// the 16-row MFMA A operand, activation rows the 16-column B operand, so a lane
// ends up holding 4 consecutive features of one token.  Operands are loaded
// straight from global memory with 16-byte loads (W is streamed once, A is
// small and cache-resident).  A work-group holds WM x WN x WK waves; the WK
// waves split K and are reduced through LDS in a fixed order (deterministic).
//
// Paired epilogues (RoPE, SwiGLU) need feature f and its partner f + P in the
// same lane: with a pair distance P, 16-feature groups 2i and 2i+1 map to
// features (first half) and (first half + P).
#pragma once
#include "common.h"

namespace dfl {

template <typename T>
struct WOperand {
  const T* ptr[kMaxSeg];
  int end[kMaxSeg];  // cumulative row counts
  int nseg;
  int pair;     // 0 or the pair distance P (a multiple of 16)
  int ngroups;  // virtual rows / 16

  __device__ __forceinline__ int feature_of_group(int gi) const {
    if (pair == 0) return gi * 16;
    const int pi = gi >> 1, half = gi & 1;
    const int per = pair >> 4;
    return (pi / per) * 2 * pair + (pi % per) * 16 + half * pair;
  }
  __device__ __forceinline__ const T* row(int f, int K) const {
    int s = 0;
    while (s + 1 < nseg && f >= end[s]) ++s;
    const int r = f - (s ? end[s - 1] : 0);
    return ptr[s] + (size_t)r * K;
  }
};

template <typename T>
struct AOperand {
  const T* ptr[kMaxKSeg];
  int nk;    // K segments
  int kseg;  // columns per segment (multiple of the MFMA k-step)
  int lda;   // row stride (elements)
  int M;     // rows
};

template <typename T, int FM, int FN, int WM, int WN, int WK, int U, class Epi>
__global__ __launch_bounds__(64 * WM * WN * WK) void gemm_kernel(const WOperand<T> w,
                                                                  const AOperand<T> a,
                                                                  const Epi epi) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  static_assert(!Epi::kPaired || (FN % 2 == 0), "paired epilogue needs even FN");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wk = wave % WK;
  const int wn = (wave / WK) % WN;
  const int wm = wave / (WK * WN);
  const int r16 = lane & 15, kg = lane >> 4;

  const int gpb = FN * WN;
  const int tiles_n = (w.ngroups + gpb - 1) / gpb;
  const int bn = blockIdx.x % tiles_n;
  const int bm = blockIdx.x / tiles_n;
  const int m0 = (bm * WM + wm) * 16 * FM;
  const int g0 = (bn * WN + wn) * FN;
  const int K = a.nk * a.kseg;

  const T* wp[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int gi = g0 + fn;
    const int f = gi < w.ngroups ? w.feature_of_group(gi) + r16 : r16;
    wp[fn] = w.row(f, K) + kg * EPL;
  }
  int arow[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + fm * 16 + r16;
    arow[fm] = m < a.M ? m : a.M - 1;
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nks = a.kseg / KS;
  const int nfull = (nks / U) * U;
  for (int s = 0; s < a.nk; ++s) {
    const T* ap[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) ap[fm] = a.ptr[s] + (size_t)arow[fm] * a.lda + kg * EPL;
    const T* wps[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wps[fn] = wp[fn] + (size_t)s * a.kseg;

    for (int ks = wk * U; ks + U <= nfull; ks += WK * U) {
      uint4 wf[U][FN], af[U][FM];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) wf[u][fn] = ld16_stream(wps[fn] + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[u][fm] = ld16(ap[fm] + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::step(wf[u][fn], af[u][fm], acc[fm][fn]);
    }
    for (int ks = nfull + wk; ks < nks; ks += WK) {
      uint4 wf[FN], af[FM];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) wf[fn] = ld16_stream(wps[fn] + ks * KS);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) af[fm] = ld16(ap[fm] + ks * KS);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::step(wf[fn], af[fm], acc[fm][fn]);
    }
  }

  if constexpr (WK > 1) {
    __shared__ f32x4_t red[WM * WN][WK - 1][FM * FN][64];
    const int wmn = wm * WN + wn;
    if (wk > 0) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) red[wmn][wk - 1][fm * FN + fn][lane] = acc[fm][fn];
    }
    __syncthreads();
    if (wk != 0) return;
    for (int j = 0; j < WK - 1; ++j)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] += red[wmn][j][fm * FN + fn][lane];
  }

#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + fm * 16 + r16;
    if (m >= a.M) continue;
    if constexpr (Epi::kPaired) {
#pragma unroll
      for (int fn = 0; fn < FN; fn += 2) {
        const int gi = g0 + fn;
        if (gi >= w.ngroups) continue;
        epi.pair(m, w.feature_of_group(gi) + 4 * kg, acc[fm][fn], acc[fm][fn + 1]);
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int gi = g0 + fn;
        if (gi >= w.ngroups) continue;
        epi.single(m, w.feature_of_group(gi) + 4 * kg, acc[fm][fn]);
      }
    }
  }
}

// ---------------------------------------------------------------- epilogues

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
  v.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
  *reinterpret_cast<uint2*>(p) = v;
}

// out[m, f..f+3] = acc (fp32)
struct EpiStoreF32 {
  static constexpr bool kPaired = false;
  float* out;
  int ldo;
  __device__ __forceinline__ void single(int m, int f, f32x4_t v) const {
    *reinterpret_cast<f32x4_t*>(out + (size_t)m * ldo + f) = v;
  }
};

// x[m, f..f+3] += acc (fp32 residual stream)
struct EpiResidual {
  static constexpr bool kPaired = false;
  float* x;
  int ldx;
  __device__ __forceinline__ void single(int m, int f, f32x4_t v) const {
    f32x4_t* p = reinterpret_cast<f32x4_t*>(x + (size_t)m * ldx + f);
    *p = *p + v;
  }
};

// h[m, f] = SiLU(gate) * up, gate rows first, up rows at +I
template <typename T>
struct EpiSwiGLU {
  static constexpr bool kPaired = true;
  T* h;
  int ldh;
  __device__ __forceinline__ void pair(int m, int f, f32x4_t g, f32x4_t u) const {
    store4<T>(h + (size_t)m * ldh + f, silu(g[0]) * u[0], silu(g[1]) * u[1], silu(g[2]) * u[2],
              silu(g[3]) * u[3]);
  }
};

// Rotate-half RoPE of a channel pair (c, c + hd/2) at table row `pos`.
__device__ __forceinline__ void rope4(const float2* tab, int half, int pos, int c, int use, f32x4_t& a,
                                      f32x4_t& b) {
  if (!use) return;
  const float2* t = tab + (size_t)pos * half + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 cs = t[i];
    const float x1 = a[i], x2 = b[i];
    a[i] = x1 * cs.x - x2 * cs.y;
    b[i] = x2 * cs.x + x1 * cs.y;
  }
}

// Block projections: virtual weight [W_q; W_kb; W_vb], pair distance hd/2.
// Q and K_b are rotated at absolute position ctx[r] + j and stored row-major;
// V_b is stored transposed per (request, kv head): vbT[((r*Hkv+g)*hd + d)*BP + j].
template <typename T>
struct EpiQKV {
  static constexpr bool kPaired = true;
  T* q;
  T* kb;
  T* vbT;
  const float2* rope;
  int Hq, Hkv, hd, BP, use_rope;
  DraftMeta meta;
  __device__ __forceinline__ void pair(int m, int f, f32x4_t a, f32x4_t b) const {
    const int B = meta.B;
    const int r = m / B, j = m - r * B;
    const int qd = Hq * hd, kd = Hkv * hd, half = hd >> 1;
    const int c = f % hd;  // < hd/2 by the pairing
    if (f < qd + kd) {
      rope4(rope, half, meta.ctx[r] + j, c, use_rope, a, b);
      T* dst = f < qd ? q + (size_t)m * qd + f : kb + (size_t)m * kd + (f - qd);
      store4<T>(dst, a[0], a[1], a[2], a[3]);
      store4<T>(dst + half, b[0], b[1], b[2], b[3]);
    } else {
      const int fv = f - qd - kd;
      const int g = fv / hd;
      T* base = vbT + ((size_t)(r * Hkv + g) * hd + c) * BP + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base[(size_t)i * BP] = from_f<T>(a[i]);
        base[(size_t)(i + half) * BP] = from_f<T>(b[i]);
      }
    }
  }
};

// Context projections of the fusion step: virtual weight
// [W_kc^0; W_vc^0; W_kc^1; W_vc^1; ...], pair distance hd/2.  Keys are rotated
// at their absolute positions and written row-major into the slot's cache;
// values are written transposed (cache layout [Hkv][hd][max_ctx_pad]).
template <typename T>
struct EpiKVAppend {
  static constexpr bool kPaired = true;
  T* pool;
  size_t slot_stride, layer_stride, kv_stride, head_stride;
  const float2* rope;
  int Hkv, hd, ctx_pad, use_rope, row_base;
  FuseMeta meta;
  __device__ __forceinline__ void pair(int m, int f, f32x4_t a, f32x4_t b) const {
    const int per_layer = 2 * Hkv * hd;
    const int layer = f / per_layer;
    int rem = f - layer * per_layer;
    const int isv = rem >= Hkv * hd;
    rem -= isv * Hkv * hd;
    const int g = rem / hd, c = rem - g * hd, half = hd >> 1;
    const int gm = row_base + m;
    const int r = fuse_req_of_row(meta, gm);
    const int pos = meta.pos0[r] + gm - meta.row0[r];
    T* base = pool + (size_t)meta.slot[r] * slot_stride + (size_t)layer * layer_stride +
              (size_t)isv * kv_stride + (size_t)g * head_stride;
    if (!isv) {
      rope4(rope, half, pos, c, use_rope, a, b);
      T* dst = base + (size_t)pos * hd + c;
      store4<T>(dst, a[0], a[1], a[2], a[3]);
      store4<T>(dst + half, b[0], b[1], b[2], b[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base[(size_t)(c + i) * ctx_pad + pos] = from_f<T>(a[i]);
        base[(size_t)(c + half + i) * ctx_pad + pos] = from_f<T>(b[i]);
      }
    }
  }
};

}  // namespace dfl
