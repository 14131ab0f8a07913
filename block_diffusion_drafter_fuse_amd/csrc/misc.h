// Small kernels: block assembly, RMSNorm, RoPE table, acceptance scan, cache
// read-back.
#pragma once
#include "common.h"

namespace dfl {

// Block assembly: row r*B + j of the fp32 residual stream is the anchor's
// token embedding (j == 0) or the shared mask embedding (j > 0).
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* embed, const T* e_mask, const int* anchor,
                                                    int B, int D, int V, float* x) {
  const int m = blockIdx.x;
  const int r = m / B, j = m - r * B;
  const T* src;
  if (j == 0) {
    int a = anchor[r];
    a = a < 0 ? 0 : (a >= V ? V - 1 : a);
    src = embed + (size_t)a * D;
  } else {
    src = e_mask;
  }
  for (int d = threadIdx.x; d < D; d += 256) x[(size_t)m * D + d] = to_f<T>(src[d]);
}

// y[mo] = x[mi] * rsqrt(mean(x[mi]^2) + eps) * g, output in the storage type.
// skip_anchor: output row mo = r*(B-1) + (j-1) reads input row r*B + j.
template <typename T, typename TI>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TI* x, const T* g, T* y, int D, float eps,
                                                      int skip_anchor, int B) {
  const int mo = blockIdx.x;
  int mi = mo;
  if (skip_anchor) {
    const int r = mo / (B - 1);
    mi = r * B + (mo - r * (B - 1)) + 1;
  }
  const TI* xr = x + (size_t)mi * D;
  float ss = 0.f;
  for (int d = threadIdx.x; d < D; d += 256) {
    const float v = to_f<TI>(xr[d]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)D + eps);
  for (int d = threadIdx.x; d < D; d += 256)
    y[(size_t)mo * D + d] = from_f<T>(to_f<TI>(xr[d]) * inv * to_f<T>(g[d]));
}

// RoPE table: tab[pos][i] = (cos, sin)(pos * base^(-2i/hd)), computed in
// double and rounded to float.
__global__ void rope_table_kernel(float2* tab, int npos, int half, double base, int hd) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= npos * half) return;
  const int pos = idx / half, i = idx - pos * half;
  const double inv = pow(base, -(2.0 * i) / (double)hd);
  const double ang = (double)pos * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// Greedy acceptance, one thread per request.
__global__ void accept_kernel(int n_req, int B, const int* cand, int cand_stride, const int* target,
                              int* tau, int* bonus) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_req) return;
  const int* c = cand + (size_t)r * (B - 1) * cand_stride;
  const int* t = target + (size_t)r * B;
  int n = 0;
  while (n < B - 1 && c[(size_t)n * cand_stride] == t[n]) ++n;
  tau[r] = n + 1;
  bonus[r] = t[n];
}

// Read back cached K/V of one (slot, layer) into fp32 [Hkv][n][hd].
template <typename T>
__global__ void read_cache_kernel(const T* kbase, const T* vtbase, size_t head_stride, int ctx_pad,
                                  int hd, int Hkv, int pos0, int n, float* kout, float* vout) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int total = Hkv * n * hd;
  if (idx >= total) return;
  const int g = idx / (n * hd);
  const int rem = idx - g * n * hd;
  const int p = rem / hd, d = rem - p * hd;
  kout[idx] = to_f<T>(kbase[(size_t)g * head_stride + (size_t)(pos0 + p) * hd + d]);
  vout[idx] = to_f<T>(vtbase[(size_t)g * head_stride + (size_t)d * ctx_pad + pos0 + p]);
}

}  // namespace dfl
