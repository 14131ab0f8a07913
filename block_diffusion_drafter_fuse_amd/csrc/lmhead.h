// Shared LM head with fused per-position top-k.
//
// logits[m, v] = sum_k u[m, k] * W_lm[v, k] for the block offsets 1..B-1 of
// every request.  Logits are never written to memory (unless the debug
// output is requested): each lane keeps a running top-KTOP list, ordered by
// (value descending, id ascending), over the vocabulary rows it produces; the
// lists are merged across lanes and waves in LDS and written per work-group
// as partial lists, which a second kernel merges per row.
#pragma once
#include "gemm.h"

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
  AOperand<T> a;    // normed final states; rowmap skips the anchor rows
  NormIn nrm;       // final RMSNorm scale
  const T* w;       // [V, D]
  int V;
  int tpw;          // 64-row vocab groups per wave
  float* logits;    // nullable [M, V]
  float* part_v;    // [nchunk][M][KTOP]
  int* part_i;
};

// Few-token LM head: WV waves per work-group, each wave owns tpw groups of
// 16*FN vocabulary rows (FN MFMA fragments sharing one activation fragment)
// over the full K for one 16-token fragment.
template <typename T, int KTOP, int WV, int FN, int U>
__global__ __launch_bounds__(64 * WV) void lmhead_kernel(const LmArgs<T> p) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int chunk = blockIdx.x;
  const int m0 = blockIdx.y * 16;
  const int D = p.a.kseg;
  const int ngroups = p.V / (16 * FN);
  const int t0 = (chunk * WV + wv) * p.tpw;
  const int t1 = min(ngroups, t0 + p.tpw);
  const int m = m0 + r16;
  const int arow = p.a.row(m < p.a.M ? m : p.a.M - 1);
  const T* ap = p.a.ptr[0] + (size_t)arow * p.a.lda + kg * EPL;
  const float sc = norm_scale(p.nrm, arow, kg);

  float lv[KTOP];
  int li[KTOP];
#pragma unroll
  for (int k = 0; k < KTOP; ++k) {
    lv[k] = -INFINITY;
    li[k] = 0x7fffffff;
  }

  const int nks = D / KS;
  const int nfull = (nks / U) * U;
  for (int t = t0; t < t1; ++t) {
    const T* wp[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wp[fn] = p.w + (size_t)(t * 16 * FN + fn * 16 + r16) * D + kg * EPL;
    f32x4_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < nfull; ks += U) {
      uint4 wf[U][FN], af[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) wf[u][fn] = ld16_stream(wp[fn] + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u) af[u] = ld16(ap + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fn] = MM::step(wf[u][fn], af[u], acc[fn]);
    }
    for (int ks = nfull; ks < nks; ++ks) {
      const uint4 af = ld16(ap + ks * KS);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fn] = MM::step(ld16_stream(wp[fn] + ks * KS), af, acc[fn]);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int id0 = t * 16 * FN + fn * 16 + 4 * kg;
      const f32x4_t v = acc[fn] * sc;
#pragma unroll
      for (int i = 0; i < 4; ++i) tk_insert<KTOP>(lv, li, v[i], id0 + i);
      if (p.logits && m < p.a.M) *reinterpret_cast<f32x4_t*>(p.logits + (size_t)m * p.V + id0) = v;
    }
  }

  // Merge: per row, WV*4 sorted lists -> one.
  constexpr int NL = WV * 4;
  __shared__ float sv[16][NL][KTOP];
  __shared__ int si[16][NL][KTOP];
#pragma unroll
  for (int k = 0; k < KTOP; ++k) {
    sv[r16][wv * 4 + kg][k] = lv[k];
    si[r16][wv * 4 + kg][k] = li[k];
  }
  __syncthreads();
  const int row = threadIdx.x;
  const int mr = m0 + row;
  if (row < 16 && mr < p.a.M) {
    int head[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) head[l] = 0;
    float* ov = p.part_v + ((size_t)chunk * p.a.M + mr) * KTOP;
    int* oi = p.part_i + ((size_t)chunk * p.a.M + mr) * KTOP;
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
}

// Top-1 epilogue for the tiled GEMM: the best (logit, id) of each token over
// the 16*FN vocabulary rows a wave holds, written as that chunk's partial list.
struct EpiTop1 {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = true;
  float* part_v;   // [ceil(V / (16*FN))][M]
  int* part_i;
  float* logits;   // nullable [M, V]
  int M, V;
  template <int FN>
  __device__ __forceinline__ void apply_row(int m, bool mvalid, int nvalid, const int (&fb)[FN],
                                            const f32x4_t (&acc)[FN], float sc, int kg) const {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (j >= nvalid) continue;
      const f32x4_t v = acc[j] * sc;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tk_better(v[i], fb[j] + 4 * kg + i, bv, bi)) {
          bv = v[i];
          bi = fb[j] + 4 * kg + i;
        }
      if (logits && mvalid) *reinterpret_cast<f32x4_t*>(logits + (size_t)m * V + fb[j] + 4 * kg) = v;
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float v2 = __shfl_xor(bv, o);
      const int i2 = __shfl_xor(bi, o);
      if (tk_better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    if (mvalid && nvalid > 0 && (threadIdx.x & 63) < 16) {
      const size_t idx = (size_t)(fb[0] / (16 * FN)) * M + m;
      part_v[idx] = bv;
      part_i[idx] = bi;
    }
  }
};

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
