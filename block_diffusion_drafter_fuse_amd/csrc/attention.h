// KV-injected bidirectional block attention: split-KV partial kernel plus a
// combine kernel.
//
// Per (request r, KV head g) the queries are the G*B rows (head-in-group,
// block offset) of the block; the keys/values are the cached context entries
// of the slot followed by the block's own K_b/V_b.  There is no mask.  The
// context is cut into splits of `chunk` keys; the last split also takes the
// B block keys.  One work-group per split holds QF waves, one per 16 query
// rows; all waves walk the same keys (shared through L1).  Each wave computes
// S^T = K Q^T and O^T += V^T P^T with MFMA and keeps an online softmax per
// query column, then stores its partial (max, sum, O).  The combine kernel
// merges the splits of every (r, g) in split order, so results are
// deterministic.
//
// Layouts: Q, K_b rows [M, heads*hd]; V_b transposed vbT[(r*Hkv+g)*hd + d][BP];
// cache keys [pos][hd] and values transposed [hd][ctx_pad] per (slot, layer,
// head).  A lane holds 4*NT consecutive keys of one query column, which is
// exactly the key run it needs as the P^T operand of the next MFMA.
#pragma once
#include "common.h"

namespace dfl {

struct AttnMeta {
  int n_req;
  int ctx[kMaxReq];
  int slot[kMaxReq];
  int nsplit[kMaxReq];     // splits of request r (>= 1; the last one takes the block keys)
  int work0[kMaxReq + 1];  // first work item of request r; Hkv*nsplit items each
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
  float* part_o;     // [work][QR][hd]
  float* part_ml;    // [work][QR][2]
  AttnMeta meta;
};

template <typename T, int HD>
struct KeySource {
  const T* kbase;  // key row 0
  int kstride;     // elements between key rows
  const T* vtbase; // V^T row 0 (d = 0)
  int ldvt;        // elements between V^T rows
  int kbeg, kend;  // key range [kbeg, kend), kend > kbeg
};

// Online-softmax attention of one wave's 16 query rows over one key source.
template <typename T, int HD>
__device__ __forceinline__ void attn_source(const KeySource<T, HD>& src, const uint4 (&qf)[HD / Mma<T>::KSTEP],
                                            float scale_log2, int r16, int kg, f32x4_t (&o)[HD / 16],
                                            float& mrow, float& lrow) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  constexpr int NT = KS / 16;
  constexpr int HS = HD / KS;
  constexpr int DF = HD / 16;
  const int kend = src.kend;

  auto load = [&](int k0, uint4 (&kf)[NT][HS], uint4 (&vf)[DF]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int key = k0 + (r16 >> 2) * (4 * NT) + 4 * t + (r16 & 3);
      const int keyc = key < kend ? key : kend - 1;
      const T* kp = src.kbase + (size_t)keyc * src.kstride + kg * EPL;
#pragma unroll
      for (int h = 0; h < HS; ++h) kf[t][h] = ld16(kp + h * KS);
    }
#pragma unroll
    for (int d = 0; d < DF; ++d)
      vf[d] = ld16(src.vtbase + (size_t)(d * 16 + r16) * src.ldvt + k0 + kg * (4 * NT));
  };

  uint4 kf[NT][HS], vf[DF];
  load(src.kbeg, kf, vf);
  for (int k0 = src.kbeg; k0 < kend; k0 += KS) {
    uint4 nkf[NT][HS], nvf[DF];
    const int kn = k0 + KS < kend ? k0 + KS : k0;
    load(kn, nkf, nvf);

    float sv[NT][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < HS; ++h) c = MM::step(kf[t][h], qf[h], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kg * (4 * NT) + 4 * t + i;
        const float x = key < kend ? c[i] * scale_log2 : -INFINITY;
        sv[t][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrow, mx);
    const float alpha = exp2f(mrow - mnew);
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
    lrow = lrow * alpha + ps;
    mrow = mnew;
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
    for (int d = 0; d < DF; ++d) o[d] = MM::step(vf[d], pp, o[d] * alpha);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < HS; ++h) kf[t][h] = nkf[t][h];
#pragma unroll
    for (int d = 0; d < DF; ++d) vf[d] = nvf[d];
  }
}

template <typename T, int HD, int QF>
__global__ __launch_bounds__(64 * QF) void attn_kernel(const AttnArgs<T> a) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  constexpr int HS = HD / KS;
  constexpr int DF = HD / 16;
  constexpr int QR = QF * 16;

  const int lane = threadIdx.x & 63, f = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int w = blockIdx.x;
  int r = 0;
  while (r + 1 < a.meta.n_req && w >= a.meta.work0[r + 1]) ++r;
  const int S = a.meta.nsplit[r];
  const int local = w - a.meta.work0[r];
  const int g = local / S, s = local - g * S;
  const int ctx = a.meta.ctx[r];
  const int qd = a.Hq * HD, kd = a.Hkv * HD;
  const int GB = a.G * a.B;

  // Query fragment of this wave (B operand: columns = query rows).
  uint4 qf[HS];
  {
    const int qi = f * 16 + r16;
    const bool valid = qi < GB;
    const int hl = valid ? qi / a.B : 0, j = valid ? qi - hl * a.B : 0;
    const T* qp = a.q + (size_t)(r * a.B + j) * qd + (size_t)(g * a.G + hl) * HD + kg * EPL;
#pragma unroll
    for (int h = 0; h < HS; ++h) qf[h] = valid ? ld16(qp + h * KS) : make_uint4(0, 0, 0, 0);
  }

  f32x4_t o[DF];
#pragma unroll
  for (int d = 0; d < DF; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.f;

  const int kbeg = s * a.chunk;
  const int kend = min(ctx, kbeg + a.chunk);
  if (kend > kbeg) {
    const T* hb = a.pool + (size_t)a.meta.slot[r] * a.slot_stride + (size_t)a.layer * a.layer_stride +
                  (size_t)g * a.head_stride;
    KeySource<T, HD> src{hb, HD, hb + a.kv_stride, a.ctx_pad, kbeg, kend};
    attn_source<T, HD>(src, qf, a.scale_log2, r16, kg, o, mrow, lrow);
  }
  if (s == S - 1) {
    KeySource<T, HD> src{a.kb + (size_t)(r * a.B) * kd + (size_t)g * HD, kd,
                         a.vbT + (size_t)(r * a.Hkv + g) * HD * a.BP, a.BP, 0, a.B};
    attn_source<T, HD>(src, qf, a.scale_log2, r16, kg, o, mrow, lrow);
  }

  float* po = a.part_o + (size_t)w * QR * HD;
  float* pml = a.part_ml + (size_t)w * QR * 2;
  const int qrow = f * 16 + r16;
#pragma unroll
  for (int d = 0; d < DF; ++d)
    *reinterpret_cast<f32x4_t*>(po + (size_t)qrow * HD + d * 16 + 4 * kg) = o[d];
  if (kg == 0) {
    pml[qrow * 2] = mrow;
    pml[qrow * 2 + 1] = lrow;
  }
}

// Merge the splits of every (r, g): one thread per (query row, 4 channels).
template <typename T, int HD, int QR>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs<T> a) {
  const int GB = a.G * a.B;
  const int per_rg = GB * (HD / 4);
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int rg = t / per_rg;
  if (rg >= a.meta.n_req * a.Hkv) return;
  const int rem = t - rg * per_rg;
  const int qi = rem / (HD / 4), d4 = rem - qi * (HD / 4);
  const int r = rg / a.Hkv, g = rg - r * a.Hkv;
  const int S = a.meta.nsplit[r];
  const int w0 = a.meta.work0[r] + g * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[((size_t)(w0 + s) * QR + qi) * 2]);
  float den = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float* ml = a.part_ml + ((size_t)(w0 + s) * QR + qi) * 2;
    const float e = exp2f(ml[0] - M);
    den += e * ml[1];
    acc += e * *reinterpret_cast<const f32x4_t*>(a.part_o + ((size_t)(w0 + s) * QR + qi) * HD + d4 * 4);
  }
  const float inv = 1.0f / den;
  const int hl = qi / a.B, j = qi - hl * a.B;
  T* op = a.o + (size_t)(r * a.B + j) * (a.Hq * HD) + (size_t)(g * a.G + hl) * HD + d4 * 4;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4_t*>(op) = acc * inv;
  } else {
    uint2 v;
    v.x = (uint32_t)f2bf(acc[0] * inv) | ((uint32_t)f2bf(acc[1] * inv) << 16);
    v.y = (uint32_t)f2bf(acc[2] * inv) | ((uint32_t)f2bf(acc[3] * inv) << 16);
    *reinterpret_cast<uint2*>(op) = v;
  }
}

}  // namespace dfl
