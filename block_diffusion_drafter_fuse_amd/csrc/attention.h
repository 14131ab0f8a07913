// KV-injected bidirectional block attention: split-KV partial kernel plus a
// combine kernel.
//
// Per (request r, KV head g) the queries are the G*B rows (head-in-group,
// block offset) of the block; the keys/values are the cached context entries
// of the slot followed by the block's own K_b/V_b.  There is no mask.  The
// context is cut into splits of `chunk` keys (a multiple of 64); the last
// split also takes the block keys.  One work-group per split holds QF waves,
// one per 16 query rows.  Keys are consumed in stages of 64: the work-group
// copies the stage's K rows and V^T rows into LDS (double buffered, the next
// stage's global loads in flight while the current one is consumed), so every
// K/V byte crosses the vector-memory path once per work-group.  Each wave
// computes S^T = K Q^T and O^T += V^T P^T with MFMA and keeps an online
// softmax per query column, then stores its partial (max, sum, O).  The
// combine kernel merges the splits of every (r, g) in split order, so results
// are deterministic.
//
// Layouts: Q, K_b rows [M, heads*hd]; V_b transposed vbT[(r*Hkv+g)*hd + d][BP]
// with BP = 64 (zero padded); cache keys [pos][hd] and values transposed
// [hd][ctx_pad] per (slot, layer, head).  Within a 16*NT-key MFMA step a lane
// holds 4*NT consecutive keys of one query column, which is exactly the key
// run it needs as the P^T operand of the next MFMA.
#pragma once
#include "common.h"

namespace dfl {

constexpr int kAttnStage = 64;  // keys per LDS stage

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

template <typename T, int HD, int QF>
struct AttnStage {
  static constexpr int KROWB = HD * (int)sizeof(T) + 16;          // padded K row bytes
  static constexpr int VROWB = kAttnStage * (int)sizeof(T) + 16;  // padded V^T row bytes
  static constexpr int KBYTES = kAttnStage * KROWB;
  static constexpr int VBYTES = HD * VROWB;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KCH = HD * (int)sizeof(T) / 16;           // 16-byte chunks per K row
  static constexpr int VCH = kAttnStage * (int)sizeof(T) / 16;   // 16-byte chunks per V^T row
  static constexpr int NCH = kAttnStage * KCH + HD * VCH;        // chunks per stage
  static constexpr int NTH = 64 * QF;
  static constexpr int CPT = (NCH + NTH - 1) / NTH;              // chunks per thread
};

template <typename T, int HD, int QF>
__global__ __launch_bounds__(64 * QF) void attn_kernel(const AttnArgs<T> a) {
  using MM = Mma<T>;
  using SG = AttnStage<T, HD, QF>;
  constexpr int KS = MM::KSTEP;  // keys per P.V step
  constexpr int EPL = MM::EPL;
  constexpr int NT = KS / 16;    // S^T tiles per P.V step
  constexpr int HS = HD / KS;    // k-steps over the head dim
  constexpr int DF = HD / 16;    // output d fragments
  constexpr int QR = QF * 16;
  constexpr int PVS = kAttnStage / KS;  // P.V steps per stage

  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, f = tid >> 6;
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

  // Stages: context keys [kbeg, kend) of this split, then (last split) the block.
  const int kbeg = s * a.chunk;
  const int kend = min(ctx, kbeg + a.chunk);
  const int nctx = kend > kbeg ? (kend - kbeg + kAttnStage - 1) / kAttnStage : 0;
  const int nst = nctx + (s == S - 1 ? 1 : 0);
  const T* hb = a.pool + (size_t)a.meta.slot[r] * a.slot_stride + (size_t)a.layer * a.layer_stride +
                (size_t)g * a.head_stride;
  const T* bkb = a.kb + (size_t)(r * a.B) * kd + (size_t)g * HD;
  const T* bvt = a.vbT + (size_t)(r * a.Hkv + g) * HD * a.BP;

  uint4 stg[SG::CPT];
  // global -> registers for stage i
  auto gload = [&](int i) {
    const bool blk = i >= nctx;
    const int k0 = blk ? 0 : kbeg + i * kAttnStage;
    const int ke = blk ? a.B : kend;
#pragma unroll
    for (int c = 0; c < SG::CPT; ++c) {
      const int ch = tid + c * SG::NTH;
      if (ch < kAttnStage * SG::KCH) {
        const int row = ch / SG::KCH, col = ch - row * SG::KCH;
        int key = k0 + row;
        key = key < ke ? key : ke - 1;
        const T* src = blk ? bkb + (size_t)key * kd : hb + (size_t)key * HD;
        stg[c] = ld16(reinterpret_cast<const char*>(src) + col * 16);
      } else if (ch < SG::NCH) {
        const int vch = ch - kAttnStage * SG::KCH;
        const int d = vch / SG::VCH, col = vch - d * SG::VCH;
        const T* src = blk ? bvt + (size_t)d * a.BP : hb + a.kv_stride + (size_t)d * a.ctx_pad + k0;
        stg[c] = ld16(reinterpret_cast<const char*>(src) + col * 16);
      }
    }
  };
  auto lstore = [&](int buf) {
    char* base = lds + buf * SG::BUF;
#pragma unroll
    for (int c = 0; c < SG::CPT; ++c) {
      const int ch = tid + c * SG::NTH;
      if (ch < kAttnStage * SG::KCH) {
        const int row = ch / SG::KCH, col = ch - row * SG::KCH;
        *reinterpret_cast<uint4*>(base + row * SG::KROWB + col * 16) = stg[c];
      } else if (ch < SG::NCH) {
        const int vch = ch - kAttnStage * SG::KCH;
        const int d = vch / SG::VCH, col = vch - d * SG::VCH;
        *reinterpret_cast<uint4*>(base + SG::KBYTES + d * SG::VROWB + col * 16) = stg[c];
      }
    }
  };

  f32x4_t o[DF];
#pragma unroll
  for (int d = 0; d < DF; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int i = 0; i < nst; ++i) {
    const int buf = i & 1;
    if (i + 1 < nst) gload(i + 1);
    const bool blk = i >= nctx;
    const int klim = blk ? a.B : kend - (kbeg + i * kAttnStage);  // valid keys in this stage
    const char* kl = lds + buf * SG::BUF;
    const char* vl = kl + SG::KBYTES;
#pragma unroll
    for (int p = 0; p < PVS; ++p) {
      const int kb0 = p * KS;  // stage-local first key of this P.V step
      if (kb0 >= klim) break;
      float sv[NT][4];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int krow = kb0 + (r16 >> 2) * (4 * NT) + 4 * t + (r16 & 3);
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HS; ++h)
          c = MM::step(*reinterpret_cast<const uint4*>(kl + krow * SG::KROWB + h * 64 + kg * 16), qf[h], c);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int key = kb0 + kg * (4 * NT) + 4 * t + ii;
          const float x = key < klim ? c[ii] * a.scale_log2 : -INFINITY;
          sv[t][ii] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow, mx);
      const float alpha = exp2f(mrow - mnew);
      float ps = 0.f;
      float pr[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          pr[t][ii] = exp2f(sv[t][ii] - mnew);
          ps += pr[t][ii];
        }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      lrow = lrow * alpha + ps;
      mrow = mnew;
      uint4 pp;
      if constexpr (NT == 1) {
        pp = make_uint4(__float_as_uint(pr[0][0]), __float_as_uint(pr[0][1]), __float_as_uint(pr[0][2]),
                        __float_as_uint(pr[0][3]));
      } else {
        pp.x = (uint32_t)f2bf(pr[0][0]) | ((uint32_t)f2bf(pr[0][1]) << 16);
        pp.y = (uint32_t)f2bf(pr[0][2]) | ((uint32_t)f2bf(pr[0][3]) << 16);
        pp.z = (uint32_t)f2bf(pr[1][0]) | ((uint32_t)f2bf(pr[1][1]) << 16);
        pp.w = (uint32_t)f2bf(pr[1][2]) | ((uint32_t)f2bf(pr[1][3]) << 16);
      }
#pragma unroll
      for (int d = 0; d < DF; ++d) {
        const uint4 vf = *reinterpret_cast<const uint4*>(vl + (d * 16 + r16) * SG::VROWB +
                                                          (kb0 + kg * 4 * NT) * (int)sizeof(T));
        o[d] = MM::step(vf, pp, o[d] * alpha);
      }
    }
    if (i + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
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
