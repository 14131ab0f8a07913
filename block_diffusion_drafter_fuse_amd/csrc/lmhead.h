// Shared LM head with fused per-position top-k.
//
// logits[m, v] = sum_k u[m, k] * W_lm[v, k] for the block offsets 1..B-1 of
// every request.  Logits are never written to memory (unless the debug
// output is requested): each lane keeps a running top-KTOP list, ordered by
// (value descending, id ascending), over the vocabulary rows it produces; the
// lists are merged across lanes and waves in LDS and written per work-group
// as partial lists, which a second kernel merges per row.
#pragma once
#include "common.h"

namespace dfl {

__device__ __forceinline__ bool tk_better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <int K>
__device__ __forceinline__ void tk_insert(float (&lv)[K], int (&li)[K], float v, int id) {
  if (!tk_better(v, id, lv[K - 1], li[K - 1])) return;
  lv[K - 1] = v;
  li[K - 1] = id;
#pragma unroll
  for (int j = K - 1; j > 0; --j) {
    if (tk_better(lv[j], li[j], lv[j - 1], li[j - 1])) {
      const float tv = lv[j];
      lv[j] = lv[j - 1];
      lv[j - 1] = tv;
      const int ti = li[j];
      li[j] = li[j - 1];
      li[j - 1] = ti;
    }
  }
}

template <typename T>
struct LmArgs {
  const T* u;       // [M, D] normed final states of offsets 1..B-1
  const T* w;       // [V, D]
  int M, V, D;
  int tpw;          // 16-row vocab tiles per wave
  float* logits;    // nullable [M, V]
  float* part_v;    // [nchunk][M][KTOP]
  int* part_i;
};

// Work-group: WV waves along the vocabulary, all on the same 16*FM rows.
template <typename T, int FM, int KTOP, int WV, int U>
__global__ __launch_bounds__(64 * WV) void lmhead_kernel(const LmArgs<T> a) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int chunk = blockIdx.x;
  const int m0 = blockIdx.y * 16 * FM;
  const int ntiles = a.V >> 4;
  const int t0 = (chunk * WV + wv) * a.tpw;
  const int t1 = min(ntiles, t0 + a.tpw);

  const T* ap[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + fm * 16 + r16;
    ap[fm] = a.u + (size_t)(m < a.M ? m : a.M - 1) * a.D + kg * EPL;
  }
  float lv[FM][KTOP];
  int li[FM][KTOP];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int k = 0; k < KTOP; ++k) {
      lv[fm][k] = -INFINITY;
      li[fm][k] = 0x7fffffff;
    }

  const int nks = a.D / KS;
  const int nfull = (nks / U) * U;
  for (int t = t0; t < t1; ++t) {
    const T* wp = a.w + (size_t)(t * 16 + r16) * a.D + kg * EPL;
    f32x4_t acc[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[fm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < nfull; ks += U) {
      uint4 wf[U], af[U][FM];
#pragma unroll
      for (int u = 0; u < U; ++u) wf[u] = ld16_stream(wp + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[u][fm] = ld16(ap[fm] + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fm] = MM::step(wf[u], af[u][fm], acc[fm]);
    }
    for (int ks = nfull; ks < nks; ++ks) {
      const uint4 wf = ld16_stream(wp + ks * KS);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) acc[fm] = MM::step(wf, ld16(ap[fm] + ks * KS), acc[fm]);
    }
    const int id0 = t * 16 + 4 * kg;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tk_insert<KTOP>(lv[fm], li[fm], acc[fm][i], id0 + i);
      if (a.logits) {
        const int m = m0 + fm * 16 + r16;
        if (m < a.M) *reinterpret_cast<f32x4_t*>(a.logits + (size_t)m * a.V + id0) = acc[fm];
      }
    }
  }

  // Merge: per row, WV*4 sorted lists -> one; one 16-row group at a time.
  constexpr int NL = WV * 4;
  __shared__ float sv[16][NL][KTOP];
  __shared__ int si[16][NL][KTOP];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int k = 0; k < KTOP; ++k) {
      sv[r16][wv * 4 + kg][k] = lv[fm][k];
      si[r16][wv * 4 + kg][k] = li[fm][k];
    }
    __syncthreads();
    const int row = threadIdx.x;
    const int m = m0 + fm * 16 + row;
    if (row < 16 && m < a.M) {
      int head[NL];
#pragma unroll
      for (int l = 0; l < NL; ++l) head[l] = 0;
      float* ov = a.part_v + ((size_t)chunk * a.M + m) * KTOP;
      int* oi = a.part_i + ((size_t)chunk * a.M + m) * KTOP;
      for (int k = 0; k < KTOP; ++k) {
        int best = -1;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          if (head[l] >= KTOP) continue;
          const float v = sv[row][l][head[l]];
          const int id = si[row][l][head[l]];
          if (best < 0 || tk_better(v, id, bv, bi)) {
            bv = v;
            bi = id;
            best = l;
          }
        }
        ov[k] = bv;
        oi[k] = bi;
#pragma unroll
        for (int l = 0; l < NL; ++l)
          if (l == best) ++head[l];
      }
    }
    __syncthreads();
  }
}

// Second stage: merge nchunk partial lists of one row; 256 threads per row.
// Each thread keeps a top-KTOP list of its share of the candidates; then
// KTOP rounds of a block-wide (value, id) maximum over the list heads.
template <int KTOP>
__global__ __launch_bounds__(256) void topk_merge_kernel(const float* part_v, const int* part_i,
                                                         int nchunk, int M, int top_k, int* out_ids,
                                                         float* out_vals) {
  const int m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float lv[KTOP];
  int li[KTOP];
#pragma unroll
  for (int k = 0; k < KTOP; ++k) {
    lv[k] = -INFINITY;
    li[k] = 0x7fffffff;
  }
  const int total = nchunk * KTOP;
  for (int c = tid; c < total; c += 256) {
    const int ch = c / KTOP, k = c - ch * KTOP;
    const size_t idx = ((size_t)ch * M + m) * KTOP + k;
    tk_insert<KTOP>(lv, li, part_v[idx], part_i[idx]);
  }
  __shared__ float sv[KTOP][256];
  __shared__ int si[KTOP][256];
  __shared__ float wv_[4];
  __shared__ int wi_[4];
#pragma unroll
  for (int k = 0; k < KTOP; ++k) {
    sv[k][tid] = lv[k];
    si[k][tid] = li[k];
  }
  __syncthreads();
  int head = 0;
  for (int k = 0; k < top_k; ++k) {
    float v = head < KTOP ? sv[head][tid] : -INFINITY;
    int id = head < KTOP ? si[head][tid] : 0x7fffffff;
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(v, o);
      const int i2 = __shfl_xor(id, o);
      if (tk_better(v2, i2, v, id)) {
        v = v2;
        id = i2;
      }
    }
    if (lane == 0) {
      wv_[wave] = v;
      wi_[wave] = id;
    }
    __syncthreads();
    float bv = wv_[0];
    int bi = wi_[0];
    for (int w = 1; w < 4; ++w)
      if (tk_better(wv_[w], wi_[w], bv, bi)) {
        bv = wv_[w];
        bi = wi_[w];
      }
    if (head < KTOP && si[head][tid] == bi && sv[head][tid] == bv) ++head;
    if (tid == 0) {
      out_ids[(size_t)m * top_k + k] = bi;
      if (out_vals) out_vals[(size_t)m * top_k + k] = bv;
    }
    __syncthreads();
  }
}

}  // namespace dfl
