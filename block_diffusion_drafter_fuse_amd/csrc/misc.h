// Small kernels: block assembly, RMSNorm, RoPE table, acceptance scan, cache
// read-back.
#pragma once
#include "common.h"

namespace dfl {

// Block assembly: row r*B + j of the fp32 residual stream is the anchor's
// token embedding (j == 0) or the shared mask embedding (j > 0).  Also writes
// the first layer's normed-input operand u = T(x * g) and per-16-feature sums
// of squares (the RMSNorm is completed by the consuming GEMM).
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* embed, const T* e_mask, const int* anchor,
                                                    const T* g, int B, int D, int V, float* x, T* u,
                                                    float* ssq) {
  const int m = blockIdx.x;
  const int r = m / B, j = m - r * B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* src;
  if (j == 0) {
    int a = anchor[r];
    a = a < 0 ? 0 : (a >= V ? V - 1 : a);
    src = embed + (size_t)a * D;
  } else {
    src = e_mask;
  }
  const int nslot = D >> 4;
  for (int c = wave; c < (D >> 6); c += 4) {
    const int d = c * 64 + lane;
    const float v = to_f<T>(src[d]);
    x[(size_t)m * D + d] = v;
    u[(size_t)m * D + d] = from_f<T>(v * to_f<T>(g[d]));
    float ss = v * v;
    for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
    if ((lane & 15) == 0) ssq[(size_t)m * nslot + (d >> 4)] = ss;
  }
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

// Read back cached K/V of one (slot, layer) into fp32 [Hkv][n][hd]; values
// are stored in 64-key tiles [pos/64][hd][64] per head.
template <typename T>
__global__ void read_cache_kernel(const T* kbase, const T* vtbase, size_t head_stride, int hd, int Hkv,
                                  int pos0, int n, float* kout, float* vout) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int total = Hkv * n * hd;
  if (idx >= total) return;
  const int g = idx / (n * hd);
  const int rem = idx - g * n * hd;
  const int p = rem / hd, d = rem - p * hd;
  kout[idx] = to_f<T>(kbase[(size_t)g * head_stride + (size_t)(pos0 + p) * hd + d]);
  const int pos = pos0 + p;
  vout[idx] = to_f<T>(vtbase[(size_t)g * head_stride + ((size_t)(pos >> 6) * hd + d) * 64 + (pos & 63)]);
}

}  // namespace dfl
