// DFlash 2 two-tap dynamic depthwise convolution along the block ("DFlash 2：
// 正确 token 已在候选里", second-insight section):
//
//   y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1},  k_{t,j}[c] = kbase_j[c] + z_t[j][c / 16]
//
// over the block offsets t of one request (x_{-1} = 0: the anchor at offset 0
// has no left neighbour; offset 1 reads the anchor).  The tap corrections
// z_t = [W_0; W_1] x_t run on the GEMM engines with the two taps' rows paired
// (group g of tap 0 beside group g of tap 1).  With few token rows (GEMV
// engines) the tap mix is their epilogue: a lane holds the corrections of
// groups g..g+3 of both taps for token row m, i.e. everything the 64 channels
// 16g..16g+63 of y_m need besides the inputs x_m and x_{m-1}, which it reads.
// With many token rows the corrections are stored and conv_mix_kernel mixes
// the taps (two launches per site).
//  * normed site (attention / FFN input): x is the RMSNorm output, held as
//    T(h * g) with per-16-channel sums of squares of h; the engine passes the
//    row scale of row m, and row m-1's is the one held by the lane a row up
//    in the same 16-row fragment.  y is written in the storage type (the next
//    GEMM's operand).
//  * residual site (attention / FFN output before the residual add): x is
//    the sub-layer output in the storage type; h += y on the fp32 residual
//    stream, and the next RMSNorm's operand T(h * g) and per-16-channel sums
//    of squares are written, as the residual epilogue of the plain layer does.
#pragma once
#include "gemm.h"

namespace dfl {

template <typename T, bool RESID>
struct EpiConvMix {
  static constexpr bool kPaired = true;
  static constexpr bool kRow = false;
  static constexpr bool kScaled = true;
  const T* in;        // [M, D] site input (the GEMM's activation operand)
  const float* ssq;   // normed site: [M, D/16] sums of squares of the unnormalised rows
  float inv_d, eps;
  const T* kbase;     // [2, D]
  int B, D;
  T* y;               // normed site output [M, D]
  float* h;           // residual site: fp32 residual stream [M, D]
  T* u;               // residual site: T(h * g) [M, D]
  const T* g;         // residual site: gain of the next RMSNorm
  float* ssq_out;     // residual site: [M, D/16]

  __device__ __forceinline__ void apply2s(int m, bool valid, int f, f32x4_t z0, f32x4_t z1, float sc) const {
    // row m - 1 sits one lane down in the same 16-row fragment (lane = row + 16 k)
    const int lane = threadIdx.x & 63;
    float scl = __shfl(sc, (lane & 15) ? lane - 1 : lane);
    if (!valid) return;
    const int t = m % B;
    const int G = D >> 4;
    if (!RESID && t > 0 && (lane & 15) == 0) {
      // the fragment starts inside a block (B does not divide 16): reduce row m-1 here
      float s = 0.f;
      for (int j = 0; j < G; ++j) s += ssq[(size_t)(m - 1) * G + j];
      scl = 1.0f / sqrtf(s * inv_d + eps);
    }
    z0 = z0 * sc;
    z1 = z1 * sc;
    const float sct = RESID ? 1.0f : sc;
    const T* xt_row = in + (size_t)m * D;
    const T* xl_row = in + (size_t)(m - 1) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int grp = f + i;
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = grp * 16 + q * 4;
        const f32x4_t xt = load4<T>(xt_row + c) * sct;
        const f32x4_t xl = t > 0 ? load4<T>(xl_row + c) * (RESID ? 1.0f : scl) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        const f32x4_t k0 = load4<T>(kbase + c), k1 = load4<T>(kbase + D + c);
        f32x4_t yv;
#pragma unroll
        for (int e = 0; e < 4; ++e) yv[e] = (k0[e] + z0[i]) * xt[e] + (k1[e] + z1[i]) * xl[e];
        if constexpr (!RESID) {
          store4<T>(y + (size_t)m * D + c, yv[0], yv[1], yv[2], yv[3]);
        } else {
          f32x4_t* hp = reinterpret_cast<f32x4_t*>(h + (size_t)m * D + c);
          const f32x4_t hn = *hp + yv;
          *hp = hn;
          const f32x4_t gg = load4<T>(g + c);
          store4<T>(u + (size_t)m * D + c, hn[0] * gg[0], hn[1] * gg[1], hn[2] * gg[2], hn[3] * gg[3]);
          ss += (hn[0] * hn[0] + hn[1] * hn[1]) + (hn[2] * hn[2] + hn[3] * hn[3]);
        }
      }
      if constexpr (RESID) ssq_out[(size_t)m * G + grp] = ss;
    }
  }
};

// The tap mix as a kernel of its own, after the corrections z were stored by
// the GEMM (many token rows: there the corrections GEMM splits K, and a mix in
// its epilogue would run in the one work-group per tile that sums the splits).
template <typename T>
struct ConvMixArgs {
  const T* in;        // [M, D] site input
  const float* ssq;   // normed site: [M, D/16] sums of squares of the unnormalised rows
  float inv_d, eps;
  const float* z;     // [M, 2 * D/16] tap corrections (tap 0 first)
  const T* kbase;     // [2, D]
  int B, D;
  T* y;               // normed site output [M, D]
  float* h;           // residual site: fp32 residual stream [M, D]
  T* u;               // residual site: T(h * g) [M, D]
  const T* g;         // residual site: gain of the next RMSNorm
  float* ssq_out;     // residual site: [M, D/16]
};

// Row scale 1/sqrt(mean + eps) of row m from its per-16-channel sums of
// squares, reduced by one wave in a fixed order (lane-strided partial sums,
// then a butterfly): no work-group barrier, every wave holds the result.
__device__ __forceinline__ float conv_row_scale(const float* ssq, int m, int nslot, float inv_d, float eps) {
  const float* p = ssq + (size_t)m * nslot;
  float s = 0.f;
  for (int i0 = threadIdx.x & 63; i0 < nslot; i0 += 64 * 8) {  // eight loads in flight, then the sums in order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i0 + 64 * u < nslot ? p[i0 + 64 * u] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + 64 * u < nslot) s += v[u];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  return 1.0f / sqrtf(s * inv_d + eps);
}

// One work-group per block row m = r * B + t (blockDim a multiple of 64, up
// to 1024), one 4-channel vector c = 4 i + 4 blockDim p per thread and pass (a
// 16-channel slot is 4 adjacent lanes).  The first pass's inputs are loaded
// before the row scales are reduced, so the two memory round trips overlap.
template <typename T, bool RESID>
__global__ __launch_bounds__(1024) void conv_mix_kernel(const ConvMixArgs<T> a) {
  const int m = blockIdx.x, t = m % a.B;
  const int D = a.D, G = D >> 4;
  const int step = (int)blockDim.x * 4;
  int c = threadIdx.x * 4;
  f32x4_t xt = {0.f, 0.f, 0.f, 0.f}, xl = {0.f, 0.f, 0.f, 0.f};
  if (c < D) {
    xt = load4<T>(a.in + (size_t)m * D + c);
    if (t > 0) xl = load4<T>(a.in + (size_t)(m - 1) * D + c);
  }
  float sc = 1.0f, scl = 1.0f;
  if (!RESID) {
    sc = conv_row_scale(a.ssq, m, G, a.inv_d, a.eps);
    if (t > 0) scl = conv_row_scale(a.ssq, m - 1, G, a.inv_d, a.eps);
  }
  const float* z = a.z + (size_t)m * 2 * G;
  for (; c < D; c += step) {
    if (c >= step) {  // later passes (D > 4 blockDim)
      xt = load4<T>(a.in + (size_t)m * D + c);
      if (t > 0) xl = load4<T>(a.in + (size_t)(m - 1) * D + c);
    }
    const f32x4_t xs = xt * sc, xls = xl * scl;
    const float z0 = z[c >> 4], z1 = z[G + (c >> 4)];
    const f32x4_t k0 = load4<T>(a.kbase + c), k1 = load4<T>(a.kbase + D + c);
    f32x4_t y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (k0[i] + z0) * xs[i] + (k1[i] + z1) * xls[i];
    if constexpr (!RESID) {
      store4<T>(a.y + (size_t)m * D + c, y[0], y[1], y[2], y[3]);
    } else {
      f32x4_t* hp = reinterpret_cast<f32x4_t*>(a.h + (size_t)m * D + c);
      const f32x4_t hn = *hp + y;
      *hp = hn;
      const f32x4_t gg = load4<T>(a.g + c);
      store4<T>(a.u + (size_t)m * D + c, hn[0] * gg[0], hn[1] * gg[1], hn[2] * gg[2], hn[3] * gg[3]);
      float ss = hn[0] * hn[0] + hn[1] * hn[1] + hn[2] * hn[2] + hn[3] * hn[3];
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if ((threadIdx.x & 3) == 0) a.ssq_out[(size_t)m * G + (c >> 4)] = ss;
    }
  }
}

}  // namespace dfl
