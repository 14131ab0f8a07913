// Small kernels: block assembly, RMSNorm, RoPE table, acceptance scan, cache
// read-back.
#pragma once
#include "common.h"
#include "gemm.h"

namespace dfl {

// Block assembly: row r*B + j of the fp32 residual stream is the anchor's
// token embedding (j == 0), a DFlow relay row stored for the request's slot
// (2 <= j < 2 + relay n), or the shared mask embedding.  Also writes the first
// layer's normed-input operand u = T(x * g) and per-16-feature sums of squares
// (the RMSNorm is completed by the consuming GEMM).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf2f((bf16_t)(w[i] & 0xffff));
    v[2 * i + 1] = bf2f((bf16_t)(w[i] >> 16));
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
}
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&v)[8]) {
  uint4 q;
  q.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  q.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  q.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  q.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = q;
}

// One work-group per block row; thread t handles features 8t .. 8t+7 (and
// +8*blockDim ...), all loads of a thread issued before any store.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* embed, const T* e_mask, const int* anchor,
                                                    const T* g, int B, int D, int V, float* x, T* u,
                                                    float* ssq, const DraftRelay rl) {
  constexpr int PT = 2;  // 8-feature groups per thread and pass (D <= 4096 in one pass)
  const int m = blockIdx.x;
  const int r = m / B, j = m - r * B;
  const T* src = nullptr;
  const float* rsrc = nullptr;
  if (j == 0) {
    int a = anchor[r];
    a = a < 0 ? 0 : (a >= V ? V - 1 : a);
    src = embed + (size_t)a * D;
  } else if (rl.rows && j >= 2 && j < 2 + rl.n[r]) {
    rsrc = rl.rows + ((size_t)rl.slot[r] * B + j) * D;
  } else {
    src = e_mask;
  }
  const int nslot = D >> 4;
  const int ngrp = D >> 3;
  for (int g0 = 0; g0 < ngrp; g0 += PT * blockDim.x) {
    float v[PT][8], gg[PT][8];
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int gi = g0 + q * blockDim.x + threadIdx.x;
      if (gi < ngrp) {
        if (rsrc)
          load8<float>(rsrc + gi * 8, v[q]);
        else
          load8<T>(src + gi * 8, v[q]);
        load8<T>(g + gi * 8, gg[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int gi = g0 + q * blockDim.x + threadIdx.x;
      // partner thread (gi ^ 1) holds the other half of the 16-feature slot;
      // ngrp is even and pairs never straddle the bound
      float ss = 0.f, un[8];
      if (gi < ngrp) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ss += v[q][i] * v[q][i];
          un[i] = v[q][i] * gg[q][i];
        }
      }
      ss += __shfl_xor(ss, 1);
      if (gi < ngrp) {
        store8<float>(x + (size_t)m * D + gi * 8, v[q]);
        store8<T>(u + (size_t)m * D + gi * 8, un);
        if ((gi & 1) == 0) ssq[(size_t)m * nslot + (gi >> 1)] = ss;
      }
    }
  }
}

// DFlow relay, per relay row m (one work-group): completes the RMSNorm of the
// shared fusion projection (hc holds T(z * g_c), fssq the per-16-feature sums
// of squares of z), then writes the relay MLP input row
// [E(bonus); E(first rejection); h] (K = 3D, storage dtype) and LN(h) in fp32
// (population variance, eps 1e-5, no affine).  The row of T(z * g_c) is read
// once, 4 features per thread and pass, and held in registers for the mean,
// the variance and the writes (D <= 4 * 256 * kRelayMaxPass).
constexpr int kRelayMaxPass = 16;

template <typename T>
__global__ __launch_bounds__(256) void relay_assemble_kernel(const T* hc, const float* fssq, int D, float eps,
                                                             const T* embed, int V, const int* bonus,
                                                             const int* cand, int cand_stride, int Bm1,
                                                             const RelayMeta rm, T* in, float* lnh) {
  const int m = blockIdx.x;
  const int r = relay_req_of_row(rm, m);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[3][4];
  const int nslot = D >> 4;
  f32x4_t hv[kRelayMaxPass];
#pragma unroll
  for (int p = 0; p < kRelayMaxPass; ++p) {
    const int c = (tid + 256 * p) * 4;
    hv[p] = c < D ? load4<T>(hc + (size_t)m * D + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // mean of z^2 from the slot sums
  float ss = 0.f;
  for (int i = tid; i < nslot; i += 256) ss += fssq[(size_t)m * nslot + i];
  ss = wave_sum(ss);
  if (lane == 0) red[0][wave] = ss;
  __syncthreads();
  const float rs = rsqrtf((red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)D + eps);
  // mean and variance of h = T(z*g) * rs (padding lanes hold zeros and are
  // left out of the variance)
  float s1 = 0.f;
#pragma unroll
  for (int p = 0; p < kRelayMaxPass; ++p) {
    hv[p] = hv[p] * rs;
    s1 += (hv[p][0] + hv[p][1]) + (hv[p][2] + hv[p][3]);
  }
  s1 = wave_sum(s1);
  if (lane == 0) red[1][wave] = s1;
  __syncthreads();
  const float mu = (red[1][0] + red[1][1] + red[1][2] + red[1][3]) / (float)D;
  float s2 = 0.f;
#pragma unroll
  for (int p = 0; p < kRelayMaxPass; ++p) {
    if ((tid + 256 * p) * 4 >= D) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dv = hv[p][e] - mu;
      s2 += dv * dv;
    }
  }
  s2 = wave_sum(s2);
  if (lane == 0) red[2][wave] = s2;
  __syncthreads();
  const float rstd = rsqrtf((red[2][0] + red[2][1] + red[2][2] + red[2][3]) / (float)D + 1e-5f);
  int b = bonus[r], y = cand[((size_t)r * Bm1 + rm.nacc[r]) * cand_stride];
  b = b < 0 ? 0 : (b >= V ? V - 1 : b);
  y = y < 0 ? 0 : (y >= V ? V - 1 : y);
  T* row = in + (size_t)m * 3 * D;
#pragma unroll
  for (int p = 0; p < kRelayMaxPass; ++p) {
    const int c = (tid + 256 * p) * 4;
    if (c >= D) continue;
    const f32x4_t eb = load4<T>(embed + (size_t)b * D + c), ey = load4<T>(embed + (size_t)y * D + c);
    store4<T>(row + c, eb[0], eb[1], eb[2], eb[3]);
    store4<T>(row + D + c, ey[0], ey[1], ey[2], ey[3]);
    store4<T>(row + 2 * D + c, hv[p][0], hv[p][1], hv[p][2], hv[p][3]);
    *reinterpret_cast<f32x4_t*>(lnh + (size_t)m * D + c) = (hv[p] - mu) * rstd;
  }
}

// DFlash 2 path selector.  select_tables_kernel: one work-group per (request,
// drafted position t) stages the k previous-token rows of A (the anchor's row
// alone for t = 0), the k candidate rows of B and the gate g_t in LDS, then
// thread (i, j) forms S_t(a_i, b_j) = U_t(b_j) + <A(a_i) * g_t, B(b_j)>.
// select_walk_kernel: one wave per request walks the greedy best successors
// (ties to the lower rank).
constexpr int kSelMaxT = 15, kSelMaxK = 16, kSelMaxR = 256;

template <typename T>
__global__ __launch_bounds__(256) void select_tables_kernel(const int* anchor, const int* cand, const float* ul,
                                                            int k, int Tn, const T* ta, const T* tb, int R,
                                                            const float* gates, int V, float* tables) {
  // rows of A * g_t and of B, 16-byte aligned, read back 4 features at a time
  __shared__ __align__(16) float sa[kSelMaxK][kSelMaxR + 4];
  __shared__ __align__(16) float sb[kSelMaxK][kSelMaxR + 4];
  const int r = blockIdx.x, t = blockIdx.y;
  const int na = t == 0 ? 1 : k;
  const float* g = gates + ((size_t)r * Tn + t) * R;
  const int cpr = R / 4;  // 4-feature chunks per row
  for (int e = threadIdx.x; e < (na + k) * cpr; e += blockDim.x) {
    const int row = e / cpr, c = (e - row * cpr) * 4;
    int id;
    if (row < na) id = t == 0 ? anchor[r] : cand[((size_t)r * Tn + t - 1) * k + row];
    else id = cand[((size_t)r * Tn + t) * k + row - na];
    id = id < 0 ? 0 : (id >= V ? V - 1 : id);
    f32x4_t v = load4<T>((row < na ? ta : tb) + (size_t)id * R + c);
    if (row < na) v = v * *reinterpret_cast<const f32x4_t*>(g + c);
    *reinterpret_cast<f32x4_t*>(row < na ? &sa[row][c] : &sb[row - na][c]) = v;
  }
  __syncthreads();
  const int i = threadIdx.x / k, j = threadIdx.x - i * k;
  if (i >= k) return;
  const int ia = t == 0 ? 0 : i;
  float s = 0.f;
  for (int c = 0; c < R; c += 4) {
    const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(&sa[ia][c]);
    const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(&sb[j][c]);
    s += ((a4[0] * b4[0] + a4[1] * b4[1]) + (a4[2] * b4[2] + a4[3] * b4[3]));
  }
  tables[(((size_t)r * Tn + t) * k + i) * k + j] = ul[((size_t)r * Tn + t) * k + j] + s;
}

__global__ __launch_bounds__(256) void select_walk_kernel(const int* cand, const float* tables, int k, int Tn,
                                                          int* out_path) {
  __shared__ float tab[kSelMaxT * kSelMaxK * kSelMaxK];
  const int r = blockIdx.x;
  const int n = Tn * k * k;
  for (int e = threadIdx.x; e < n; e += blockDim.x) tab[e] = tables[(size_t)r * n + e];
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // one wave: lane j < k holds candidate j of the row; argmax over 16 lanes
  // with ties to the lower rank; lane t keeps the rank chosen at position t,
  // and the candidate ids are gathered after the walk (no global access
  // inside the dependent chain)
  const int lane = threadIdx.x;
  int prev = 0, mine = 0;
  for (int t = 0; t < Tn; ++t) {
    const float* row = tab + (t * k + (t == 0 ? 0 : prev)) * k;
    float v = lane < k ? row[lane] : -INFINITY;
    int bi = lane < k ? lane : kSelMaxK;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float v2 = __shfl_xor(v, o);
      const int i2 = __shfl_xor(bi, o);
      if (v2 > v || (v2 == v && i2 < bi)) {
        v = v2;
        bi = i2;
      }
    }
    prev = __shfl(bi, 0);
    if (lane == t) mine = prev;
  }
  if (lane < Tn) out_path[(size_t)r * Tn + lane] = cand[((size_t)r * Tn + lane) * k + mine];
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
// are stored in kVTile-key tiles [pos/kVTile][hd][kVTile] per head.
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
  vout[idx] = to_f<T>(vtbase[(size_t)g * head_stride + ((size_t)(pos / kVTile) * hd + d) * kVTile + (pos % kVTile)]);
}

}  // namespace dfl
