// DFlash 2 two-tap dynamic depthwise convolution along the block ("DFlash 2：
// 正确 token 已在候选里", second-insight section):
//
//   y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1},  k_{t,j}[c] = kbase_j[c] + z_t[j][c / 16]
//
// over the block offsets t of one request (x_{-1} = 0: the anchor at offset 0
// has no left neighbour; offset 1 reads the anchor).  z_t = [W_0; W_1] x_t
// comes from the GEMM engine (one output per 16 channels and tap); this
// kernel mixes the taps.  Two forms:
//  * normed site (attention / FFN input): x is the RMSNorm output, held as
//    T(h * g) with per-16-channel sums of squares of h; the row scales of
//    rows t and t-1 are completed here, the convolved rows y are written in
//    the storage type (the next GEMM's operand);
//  * residual site (attention / FFN output before the residual add): x is
//    the sub-layer output in the storage type; h += y on the fp32 residual
//    stream, and the next RMSNorm's operand T(h * g) and per-16-channel sums
//    of squares are written, as the residual epilogue of the plain layer does.
#pragma once
#include "gemm.h"

namespace dfl {

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

// Row scale 1/sqrt(mean + eps) of row m from its per-16-channel sums of squares.
template <int NT>
__device__ __forceinline__ float conv_row_scale(const float* ssq, int m, int nslot, float inv_d, float eps,
                                                float* red) {
  float s = 0.f;
  for (int i = threadIdx.x; i < nslot; i += NT) s += ssq[(size_t)m * nslot + i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  __syncthreads();
  return 1.0f / sqrtf(t * inv_d + eps);
}

// One 256-thread work-group per block row m = r * B + t; thread i handles the
// 4-channel vectors c = 4 i + 1024 p (a 16-channel slot is 4 adjacent lanes).
template <typename T, bool RESID>
__global__ __launch_bounds__(256) void conv_mix_kernel(const ConvMixArgs<T> a) {
  __shared__ float red[4];
  const int m = blockIdx.x, t = m % a.B;
  const int D = a.D, G = D >> 4;
  float sc = 1.0f, scl = 1.0f;
  if (!RESID) {
    sc = conv_row_scale<256>(a.ssq, m, G, a.inv_d, a.eps, red);
    if (t > 0) scl = conv_row_scale<256>(a.ssq, m - 1, G, a.inv_d, a.eps, red);
  }
  const float* z = a.z + (size_t)m * 2 * G;
  for (int c = threadIdx.x * 4; c < D; c += 1024) {
    const f32x4_t xt = load4<T>(a.in + (size_t)m * D + c) * sc;
    const f32x4_t xl = t > 0 ? load4<T>(a.in + (size_t)(m - 1) * D + c) * scl : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float z0 = z[c >> 4], z1 = z[G + (c >> 4)];
    const f32x4_t k0 = load4<T>(a.kbase + c), k1 = load4<T>(a.kbase + D + c);
    f32x4_t y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (k0[i] + z0) * xt[i] + (k1[i] + z1) * xl[i];
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
