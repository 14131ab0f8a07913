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
  float* logits;    // nullable [M, V]
  float* part_v;    // [M][nchunk][KTOP]
  int* part_i;
};

// Few-token LM head with the activations staged in LDS: one work-group of
// 16 waves per CU holds the 16 normed rows [16][D] (rows padded by 16 bytes,
// so 16 * (D * sizeof(T) + 16) bytes of LDS, which the host checks against
// the 160 KB of a CU), so the vector-memory path carries only the weight
// stream.  Any D that is a multiple of the MFMA k-step is handled (the k-loop
// is unrolled by U with a remainder loop).  Waves take
// 16*FN-row vocabulary tiles from a per-launch atomic counter (reset by the
// merge kernel) and keep a running top-KTOP per lane; the lists are merged
// per work-group in LDS.  The partial lists depend on which wave took which
// tile, the merged result does not.
template <typename T, int KTOP, int FN, int U>
__global__ __launch_bounds__(1024) void lmhead_lds_kernel(const LmArgs<T> p, int* tile_ctr) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int m0 = blockIdx.y * 16;
  const int D = p.a.kseg;
  const int rowb = D * (int)sizeof(T) + 16;
  // stage the 16 activation rows
  const int cpr = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  for (int i = tid; i < 16 * cpr; i += 1024) {
    const int row = i / cpr, c = i - row * cpr;
    const int m = m0 + row < p.a.M ? m0 + row : p.a.M - 1;
    *reinterpret_cast<uint4*>(lds + row * rowb + c * 16) =
        ld16(reinterpret_cast<const char*>(p.a.ptr[0] + (size_t)p.a.row(m) * p.a.lda) + c * 16);
  }
  const int m = m0 + r16;
  const int arow = p.a.row(m < p.a.M ? m : p.a.M - 1);
  const float sc = norm_scale(p.nrm, arow, kg);
  __syncthreads();

  float lv[KTOP];
  int li[KTOP];
#pragma unroll
  for (int k = 0; k < KTOP; ++k) {
    lv[k] = -INFINITY;
    li[k] = 0x7fffffff;
  }
  const int ntiles = p.V / (16 * FN);
  const int nks = D / KS;
  const char* abase = lds + r16 * rowb + kg * 16;
  for (;;) {
    int t = 0;
    if (lane == 0) t = atomicAdd(tile_ctr + blockIdx.y, 1);
    t = __shfl(t, 0);
    if (t >= ntiles) break;
    const T* wp[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) wp[fn] = p.w + (size_t)(t * 16 * FN + fn * 16 + r16) * D + kg * EPL;
    f32x4_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nks_u = nks - nks % U;  // whole unrolled batches, then the k-steps left over
    for (int ks = 0; ks < nks_u; ks += U) {
      uint4 wf[U][FN], af[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) wf[u][fn] = ld16_stream(wp[fn] + (ks + u) * KS);
#pragma unroll
      for (int u = 0; u < U; ++u) af[u] = *reinterpret_cast<const uint4*>(abase + (ks + u) * 64);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fn] = MM::step(wf[u][fn], af[u], acc[fn]);
    }
    for (int ks = nks_u; ks < nks; ++ks) {
      const uint4 af = *reinterpret_cast<const uint4*>(abase + ks * 64);
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

  // Merge the 64 lists per row (16 waves x 4 lanes) in LDS, one row per thread.
  __syncthreads();
  constexpr int NL = 64;
  float* sv = reinterpret_cast<float*>(lds);
  int* si = reinterpret_cast<int*>(lds + 16 * NL * KTOP * sizeof(float));
#pragma unroll
  for (int k = 0; k < KTOP; ++k) {
    sv[(r16 * NL + wv * 4 + kg) * KTOP + k] = lv[k];
    si[(r16 * NL + wv * 4 + kg) * KTOP + k] = li[k];
  }
  __syncthreads();
  const int mr = m0 + tid;
  if (tid < 16 && mr < p.a.M) {
    // list heads of this row in LDS (a per-thread array indexed at run time
    // would live in scratch memory)
    unsigned char* head = reinterpret_cast<unsigned char*>(lds + 16 * NL * KTOP * 8) + tid * NL;
    for (int l = 0; l < NL; ++l) head[l] = 0;
    float* ov = p.part_v + ((size_t)mr * gridDim.x + blockIdx.x) * KTOP;
    int* oi = p.part_i + ((size_t)mr * gridDim.x + blockIdx.x) * KTOP;
    for (int k = 0; k < KTOP; ++k) {
      int best = -1;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int l = 0; l < NL; ++l) {
        const int h = head[l];
        if (h >= KTOP) continue;
        const float v = sv[(tid * NL + l) * KTOP + h];
        const int id = si[(tid * NL + l) * KTOP + h];
        if (best < 0 || tk_better(v, id, bv, bi)) {
          bv = v;
          bi = id;
          best = l;
        }
      }
      ov[k] = bv;
      oi[k] = bi;
      head[best]++;
    }
  }
}

// Top-1 epilogue for the tiled GEMM: the best (logit, id) of each token over
// the 16*FN vocabulary rows a wave holds, written as that chunk's partial list.
struct EpiTop1 {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = true;
  float* part_v;   // [M][nchunk], chunk = 16*FN vocabulary rows
  int* part_i;
  float* logits;   // nullable [M, V]
  int M, V, nchunk;
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
      const size_t idx = (size_t)m * nchunk + fb[0] / (16 * FN);
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
                                                         int nchunk, int top_k, int* out_ids,
                                                         float* out_vals, int* tile_ctr, int nctr) {
  const int m = blockIdx.x;
  if (m == 0 && (int)threadIdx.x < nctr) tile_ctr[threadIdx.x] = 0;  // LM-head tile counters for the next call
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
    const size_t idx = ((size_t)m * nchunk + ch) * KTOP + k;
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

// Top-1 merge: one 1024-thread work-group per row scans the row's contiguous
// partial list (coalesced), then reduces across the waves in LDS.
__global__ __launch_bounds__(1024) void top1_merge_kernel(const float* part_v, const int* part_i, int nchunk,
                                                          int* out_ids, float* out_vals, int* tile_ctr,
                                                          int nctr) {
  const int m = blockIdx.x;
  if (m == 0 && (int)threadIdx.x < nctr) tile_ctr[threadIdx.x] = 0;  // small LM-head tile counters, next call
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pv = part_v + (size_t)m * nchunk;
  const int* pi = part_i + (size_t)m * nchunk;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // eight entries loaded at a time (one memory round trip per eight, not per
  // entry); the winner does not depend on the order of the comparisons
  for (int c0 = tid; c0 < nchunk; c0 += 1024 * 8) {
    float v[8];
    int ix[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * 1024;
      v[u] = c < nchunk ? pv[c] : -INFINITY;
      ix[u] = c < nchunk ? pi[c] : 0x7fffffff;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (tk_better(v[u], ix[u], bv, bi)) {
        bv = v[u];
        bi = ix[u];
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o);
    const int i2 = __shfl_xor(bi, o);
    if (tk_better(v2, i2, bv, bi)) {
      bv = v2;
      bi = i2;
    }
  }
  __shared__ float wv[16];
  __shared__ int wi[16];
  if (lane == 0) {
    wv[wave] = bv;
    wi[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    const int nw = blockDim.x >> 6;
    for (int w = 1; w < nw; ++w)
      if (tk_better(wv[w], wi[w], bv, bi)) {
        bv = wv[w];
        bi = wi[w];
      }
    out_ids[m] = bi;
    if (out_vals) out_vals[m] = bv;
  }
}

}  // namespace dfl
