// KV-injected bidirectional block attention with split-KV and an in-kernel
// combine.
//
// Per (request r, KV head g) the queries are the G*B rows (head-in-group,
// block offset) of the block; the keys/values are the cached context entries
// of the slot followed by the block's own K_b/V_b.  There is no mask.  The
// context is cut into splits of `chunk` keys plus one split for the block;
// each split is one wave that computes S^T = K Q^T and O^T += V^T P^T with
// MFMA and keeps an online softmax per query column.  The last split of a
// (r, g) to finish (atomic counter, device-scope fences) merges the partial
// (max, sum, O) triples in split order, so the result is deterministic.
//
// Layouts: Q, K_b rows [M, heads*hd]; V_b transposed vbT[(r*Hkv+g)*hd + d][BP];
// cache keys [pos][hd] and values transposed [hd][ctx_pad] per (slot, layer,
// head).  A lane holds 4*NT consecutive keys of one query column, which is
// exactly the key run it needs as the P^T operand of the next MFMA, so no
// shuffles are needed between the two products.
#pragma once
#include "common.h"

namespace dfl {

struct AttnMeta {
  int n_req;
  int ctx[kMaxReq];
  int slot[kMaxReq];
  int nsplit[kMaxReq];     // context splits of request r (the block split comes last)
  int work0[kMaxReq + 1];  // first work item of request r; Hkv*(nsplit+1) items each
};

template <typename T>
struct AttnArgs {
  const T* q;
  const T* kb;
  const T* vbT;
  T* o;
  const T* pool;
  size_t slot_stride, layer_stride, kv_stride, head_stride;
  int ctx_pad, layer;
  int Hq, Hkv, G, B, BP, chunk;
  float scale_log2;  // log2(e) / sqrt(hd)
  float* part_o;     // [work][QF*16][hd]
  float* part_ml;    // [work][QF*16][2]
  int* counters;     // [kMaxReq * Hkv], zero between calls
  AttnMeta meta;
};

template <typename T, int HD, int QF>
__global__ __launch_bounds__(64) void attn_kernel(const AttnArgs<T> a) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;  // keys per P.V step
  constexpr int EPL = MM::EPL;
  constexpr int NT = KS / 16;    // S^T tiles per step
  constexpr int HS = HD / KS;    // k-steps over the head dim
  constexpr int DF = HD / 16;    // output d fragments
  constexpr int QR = QF * 16;    // query rows handled

  const int lane = threadIdx.x;
  const int r16 = lane & 15, kg = lane >> 4;
  const int w = blockIdx.x;
  int r = 0;
  while (r + 1 < a.meta.n_req && w >= a.meta.work0[r + 1]) ++r;
  const int S = a.meta.nsplit[r] + 1;
  const int local = w - a.meta.work0[r];
  const int g = local / S, s = local - g * S;
  const int ctx = a.meta.ctx[r];
  const bool is_block = (s == S - 1);
  const int kbeg = is_block ? 0 : s * a.chunk;
  const int kend = is_block ? a.B : min(ctx, kbeg + a.chunk);
  const int qd = a.Hq * HD, kd = a.Hkv * HD;
  const int GB = a.G * a.B;

  // Query fragments (B operand: columns = query rows).
  uint4 qf[QF][HS];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const int qi = f * 16 + r16;
    const bool valid = qi < GB;
    const int hl = valid ? qi / a.B : 0, j = valid ? qi - hl * a.B : 0;
    const T* qp = a.q + (size_t)(r * a.B + j) * qd + (size_t)(g * a.G + hl) * HD + kg * EPL;
#pragma unroll
    for (int h = 0; h < HS; ++h) qf[f][h] = valid ? ld16(qp + h * KS) : make_uint4(0, 0, 0, 0);
  }

  const T* kbase;
  const T* vtbase;
  int kstride, ldvt;
  if (is_block) {
    kbase = a.kb + (size_t)(r * a.B) * kd + (size_t)g * HD;
    kstride = kd;
    vtbase = a.vbT + (size_t)(r * a.Hkv + g) * HD * a.BP;
    ldvt = a.BP;
  } else {
    const T* hb = a.pool + (size_t)a.meta.slot[r] * a.slot_stride + (size_t)a.layer * a.layer_stride +
                  (size_t)g * a.head_stride;
    kbase = hb;
    kstride = HD;
    vtbase = hb + a.kv_stride;
    ldvt = a.ctx_pad;
  }

  f32x4_t o[DF][QF];
#pragma unroll
  for (int d = 0; d < DF; ++d)
#pragma unroll
    for (int f = 0; f < QF; ++f) o[d][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[QF], lrow[QF];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    mrow[f] = -INFINITY;
    lrow[f] = 0.f;
  }

  for (int k0 = kbeg; k0 < kend; k0 += KS) {
    // S^T[key][q]: A operand rows are keys, permuted so that lane group kg
    // ends up holding keys k0 + kg*4*NT + [0, 4*NT).
    f32x4_t st[NT][QF];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int key = k0 + (r16 >> 2) * (4 * NT) + 4 * t + (r16 & 3);
      const int keyc = key < kend ? key : kend - 1;
      const T* kp = kbase + (size_t)keyc * kstride + kg * EPL;
      uint4 kf[HS];
#pragma unroll
      for (int h = 0; h < HS; ++h) kf[h] = ld16(kp + h * KS);
#pragma unroll
      for (int f = 0; f < QF; ++f) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HS; ++h) c = MM::step(kf[h], qf[f][h], c);
        st[t][f] = c;
      }
    }
    // V^T fragments (A operand rows = d, k = the same key run).
    uint4 vf[DF];
#pragma unroll
    for (int d = 0; d < DF; ++d)
      vf[d] = ld16(vtbase + (size_t)(d * 16 + r16) * ldvt + k0 + kg * (4 * NT));

#pragma unroll
    for (int f = 0; f < QF; ++f) {
      float sv[NT][4];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kg * (4 * NT) + 4 * t + i;
          const float x = key < kend ? st[t][f][i] * a.scale_log2 : -INFINITY;
          sv[t][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[f], mx);
      const float alpha = exp2f(mrow[f] - mnew);
      float ps = 0.f;
      float p[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[t][i] = exp2f(sv[t][i] - mnew);
          ps += p[t][i];
        }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      lrow[f] = lrow[f] * alpha + ps;
      mrow[f] = mnew;
#pragma unroll
      for (int d = 0; d < DF; ++d) o[d][f] *= alpha;
      uint4 pp;
      if constexpr (NT == 1) {
        pp = make_uint4(__float_as_uint(p[0][0]), __float_as_uint(p[0][1]), __float_as_uint(p[0][2]),
                        __float_as_uint(p[0][3]));
      } else {
        pp.x = (uint32_t)f2bf(p[0][0]) | ((uint32_t)f2bf(p[0][1]) << 16);
        pp.y = (uint32_t)f2bf(p[0][2]) | ((uint32_t)f2bf(p[0][3]) << 16);
        pp.z = (uint32_t)f2bf(p[1][0]) | ((uint32_t)f2bf(p[1][1]) << 16);
        pp.w = (uint32_t)f2bf(p[1][2]) | ((uint32_t)f2bf(p[1][3]) << 16);
      }
#pragma unroll
      for (int d = 0; d < DF; ++d) o[d][f] = MM::step(vf[d], pp, o[d][f]);
    }
  }

  // Partial results of this split.
  float* po = a.part_o + (size_t)w * QR * HD;
  float* pml = a.part_ml + (size_t)w * QR * 2;
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const int qrow = f * 16 + r16;
#pragma unroll
    for (int d = 0; d < DF; ++d)
      *reinterpret_cast<f32x4_t*>(po + (size_t)qrow * HD + d * 16 + 4 * kg) = o[d][f];
    if (kg == 0) {
      pml[qrow * 2] = mrow[f];
      pml[qrow * 2 + 1] = lrow[f];
    }
  }
  __threadfence();
  int prev = 0;
  int* ctr = a.counters + r * a.Hkv + g;
  if (lane == 0) prev = atomicAdd(ctr, 1);
  prev = __shfl(prev, 0);
  if (prev != S - 1) return;
  __threadfence();
  if (lane == 0) *ctr = 0;

  // Combine the S splits of (r, g) in split order.
  const int w0 = a.meta.work0[r] + g * S;
  for (int qi = 0; qi < GB; ++qi) {
    const int hl = qi / a.B, j = qi - hl * a.B;
    float M = -INFINITY;
    for (int t = 0; t < S; ++t) M = fmaxf(M, a.part_ml[((size_t)(w0 + t) * QR + qi) * 2]);
    float den = 0.f;
    for (int t = 0; t < S; ++t) {
      const float* ml = a.part_ml + ((size_t)(w0 + t) * QR + qi) * 2;
      den += exp2f(ml[0] - M) * ml[1];
    }
    const float inv = 1.0f / den;
    T* op = a.o + (size_t)(r * a.B + j) * qd + (size_t)(g * a.G + hl) * HD;
    for (int d = lane; d < HD; d += 64) {
      float acc = 0.f;
      for (int t = 0; t < S; ++t) {
        const float mt = a.part_ml[((size_t)(w0 + t) * QR + qi) * 2];
        acc += exp2f(mt - M) * a.part_o[((size_t)(w0 + t) * QR + qi) * HD + d];
      }
      op[d] = from_f<T>(acc * inv);
    }
  }
}

}  // namespace dfl
