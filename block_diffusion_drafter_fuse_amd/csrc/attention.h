// KV-injected bidirectional block attention: split-KV partial kernel plus a
// combine kernel.
//
// Per (request r, KV head g) the queries are the G*B rows (head-in-group,
// block offset) of the block; the keys/values are the cached context entries
// of the slot followed by the block's own K_b/V_b.  There is no mask.  The
// context is cut into splits of `chunk` keys (a multiple of 64); the last
// split also takes the block keys.  One work-group per split holds QF waves,
// one per 16 query rows.  Keys are consumed in stages of STG (a multiple of the
// cache's V^T tile): a stage's K rows and V^T tiles are copied global -> LDS
// asynchronously (16 bytes per lane, no register round trip) into a ring of
// NBUF buffers, one barrier per stage, so every K/V byte crosses the
// vector-memory path once per work-group.  Each
// wave computes S^T = K Q^T and O^T += V^T P^T with MFMA and keeps an online
// softmax per query column, then stores its partial (max, sum, O).  The
// combine kernel merges the splits of every (r, g) in split order, so results
// are deterministic.  Work-groups are launched longest split first (AttnMeta),
// which packs a ragged batch's splits onto the CUs; the partials keep their
// request-major index.
//
// Layouts: Q, K_b rows [M, heads*hd]; V_b transposed vbT[(r*Hkv+g)*hd + d][64]
// (zero padded past B); cache keys [pos][hd] and values in kVTile-key tiles
// [pos/kVTile][hd][kVTile] per (slot, layer, head), so a stage's V^T is one
// contiguous block.  Within a 16*NT-key MFMA step a lane holds 4*NT consecutive keys of
// one query column, which is exactly the key run it needs as the P^T operand
// of the next MFMA.  LDS rows are unpadded; 16-byte chunk c of row r sits at
// slot c ^ f(r), with f chosen so that the 8 rows one fragment read touches
// per bank cycle land on distinct bank groups.
#pragma once
#include "gemm_tiled.h"

namespace dfl {

constexpr int kAttnStage = 64;  // split lengths are multiples of this (and of every stage size)
constexpr float kAttnSlack = 8.f;  // log2 headroom before a query's reference maximum moves

// Work items (request r, KV head g, split s) are numbered canonically, r-major
// (work0[r] + g * nsplit[r] + s: where the split's partial is stored and the
// combine reads it), but launched longest first so that the short splits of
// a ragged batch fill the gaps at the end: the last splits (rest of the
// context plus the block) of the `nbig` requests at least a full split long,
// in rorder; then every full split, r-major; then the other last splits in
// rorder (requests by descending last-split length, ties by index).
struct AttnMeta {
  int n_req;
  int nbig;
  int ctx[kMaxReq];
  int slot[kMaxReq];
  int nsplit[kMaxReq];     // splits of request r (>= 1; the last one takes the block keys)
  int work0[kMaxReq + 1];  // first work item of request r; Hkv*nsplit items each
  int rorder[kMaxReq];
};

// (request, KV head, split) of launched work-group w, in the order above.
__device__ __forceinline__ void attn_item(const AttnMeta& m, int Hkv, int w, int& r, int& g, int& s) {
  const int nbigw = m.nbig * Hkv;
  const int nfull = m.work0[m.n_req] - m.n_req * Hkv;  // full (non-last) splits of all requests
  if (w < nbigw || w >= nbigw + nfull) {
    const int i = w < nbigw ? w : w - nfull;
    r = m.rorder[i / Hkv];
    g = i - (i / Hkv) * Hkv;
    s = m.nsplit[r] - 1;
  } else {
    // full splits before request r: work0[r] - r * Hkv
    const int j = w - nbigw;
    r = 0;
    while (r + 1 < m.n_req && j >= m.work0[r + 1] - (r + 1) * Hkv) ++r;
    const int nf = m.nsplit[r] - 1;
    const int local = j - (m.work0[r] - r * Hkv);
    g = local / nf;
    s = local - g * nf;
  }
}

template <typename T>
struct AttnArgs {
  const T* q;
  const T* kb;
  const T* vbT;
  T* o;
  const T* pool;
  size_t slot_stride, layer_stride, kv_stride, head_stride;
  int layer;
  int Hq, Hkv, G, B, BP, chunk;
  float scale_log2;  // log2(e) / sqrt(hd)
  float* part_o;     // [work][QR][hd]
  float* part_ml;    // [work][QR][2]
  AttnMeta meta;
};

template <typename T, int HD, int NWV, int NBUF, int STG>
struct AttnStage {
  static_assert(STG % kVTile == 0 && kAttnStage % STG == 0, "stages of whole V^T tiles");
  static constexpr int KRB = HD * (int)sizeof(T);      // K row bytes
  static constexpr int VRB = kVTile * (int)sizeof(T);  // V^T row bytes within a tile
  static constexpr int TILEB = HD * VRB;               // V^T tile bytes
  static constexpr int KBYTES = STG * KRB;
  static constexpr int VBYTES = (STG / kVTile) * TILEB;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KI = KBYTES / 1024;  // copy instructions (1 KB each) per stage
  static constexpr int VI = VBYTES / 1024;
  static constexpr int NIW = (KI + VI) / NWV;  // per wave
  static constexpr int LDS = NBUF * BUF;
  static_assert((KI + VI) % NWV == 0 && KI % NWV == 0, "copy blocks split evenly over the waves");
};

// LDS swizzles.  A 16-byte fragment read is served 16 lanes (256 bytes) per
// cycle, so the 16 rows one read touches at a given chunk must land on 16
// distinct 16-byte slots of the 256-byte bank window.
//
// K rows (KCH chunks of 16 bytes): chunk c of row r sits at c ^ kswz(r).  With
// 256-byte rows every row starts the window, so kswz must differ over the 16
// rows of a read: {4*NT*j + 4t + (0..3)}, j = 0..3 (NT = 2), or 16 consecutive
// rows (NT = 1).  With 128-byte rows two rows share the window (row parity
// picks the half) and 3 bits suffice.
template <int NT, int KCH>
__device__ __forceinline__ int attn_kswz(int row) {
  if constexpr (KCH >= 16) {
    if constexpr (NT == 2) return (row & 3) | (((row >> 3) & 3) << 2);
    return row & 15;
  } else {
    if constexpr (NT == 2) return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
    return (row >> 1) & 7;
  }
}

// V^T rows (head-dim index d) of VCH 16-byte chunks: a read touches rows
// d..d+15 at one chunk.  64-byte rows: four rows share the window (d & 3
// picks the quarter), chunk c at c ^ ((d >> 2) & 3).  128-byte rows: two rows
// share it, chunk c at c ^ ((d >> 1) & 7).
template <int VCH>
__device__ __forceinline__ int attn_vswz(int row) {
  return VCH >= 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// QW: query fragments (16 query rows each) per wave; the QF/QW waves share
// the stage copies, and every K or V^T fragment a wave reads from LDS feeds QW
// MFMAs (the LDS reads per key fall by QW).  WPE: waves per SIMD the register
// allocation must allow.
template <typename T, int HD, int QF, int QW, int NBUF, int STG, int WPE>
__global__ __launch_bounds__(64 * (QF / QW), WPE) void attn_kernel(const AttnArgs<T> a) {
  using MM = Mma<T>;
  constexpr int NWV = QF / QW;
  static_assert(QF % QW == 0, "whole query fragments per wave");
  using SG = AttnStage<T, HD, NWV, NBUF, STG>;
  constexpr int KS = MM::KSTEP;  // keys per P.V step
  constexpr int EPL = MM::EPL;
  constexpr int NT = KS / 16;    // S^T tiles per P.V step
  constexpr int HS = HD / KS;    // k-steps over the head dim
  constexpr int DF = HD / 16;    // output d fragments
  constexpr int QR = QF * 16;
  constexpr int PVS = STG / KS;  // P.V steps per stage
  constexpr int KCH = SG::KRB / 16, VCH = SG::VRB / 16;  // 16-byte chunks per row
  static_assert(KCH >= 8 && VCH >= 4, "swizzle needs 8 chunks per K row, 4 per V^T row");

  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, f = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  int r, g, s;
  attn_item(a.meta, a.Hkv, blockIdx.x, r, g, s);
  const int S = a.meta.nsplit[r];
  const int w = a.meta.work0[r] + g * S + s;  // canonical index of this split's partial
  const int ctx = a.meta.ctx[r];
  const int qd = a.Hq * HD, kd = a.Hkv * HD;
  const int GB = a.G * a.B;

  // Query fragments of this wave (B operands: columns = query rows);
  // fragment q covers query rows 16 (f QW + q) ...
  uint4 qf[QW][HS];
#pragma unroll
  for (int q = 0; q < QW; ++q) {
    const int qi = (f * QW + q) * 16 + r16;
    const bool valid = qi < GB;
    const int hl = valid ? qi / a.B : 0, j = valid ? qi - hl * a.B : 0;
    const T* qp = a.q + (size_t)(r * a.B + j) * qd + (size_t)(g * a.G + hl) * HD + kg * EPL;
#pragma unroll
    for (int h = 0; h < HS; ++h) qf[q][h] = valid ? ld16(qp + h * KS) : make_uint4(0, 0, 0, 0);
  }
  // Padding loads after the query fragments: the compiler waits for a
  // fragment with a count of the loads it issued after it; the padding keeps
  // that count at or above the copies in flight at the first stage (which it
  // does not see), so the first stage does not wait for the whole prologue.
  constexpr int NPAD = (NBUF - 1) * (SG::NIW);
  uint32_t pad[NPAD];
  {
    asm volatile("" ::: "memory");
    const char* pp = reinterpret_cast<const char*>(a.q) + (lane & 7) * 4;
#pragma unroll
    for (int i = 0; i < NPAD; ++i) pad[i] = *reinterpret_cast<const uint32_t*>(pp + i * 64);
    asm volatile("" ::: "memory");
  }

  // Stages: context keys [kbeg, kend) of this split, then (last split) the block.
  const int kbeg = s * a.chunk;
  const int kend = min(ctx, kbeg + a.chunk);
  const int nctx = kend > kbeg ? (kend - kbeg + STG - 1) / STG : 0;
  const int nst = nctx + (s == S - 1 ? 1 : 0);
  const T* hb = a.pool + (size_t)a.meta.slot[r] * a.slot_stride + (size_t)a.layer * a.layer_stride +
                (size_t)g * a.head_stride;
  const T* bkb = a.kb + (size_t)(r * a.B) * kd + (size_t)g * HD;
  const T* bvt = a.vbT + (size_t)(r * a.Hkv + g) * HD * a.BP;

  // Copy of stage i into buffer b: instruction j = f + NWV*ii covers K rows
  // (j < KI) or V^T rows; each lane one 16-byte chunk of one row.
  auto issue = [&](int i, int b) {
    const bool blk = i >= nctx;
    const int k0 = blk ? 0 : kbeg + i * STG;  // multiple of STG
    char* base = lds + b * SG::BUF;
#pragma unroll
    for (int ii = 0; ii < SG::NIW; ++ii) {
      const int j = f + NWV * ii;
      if (j < SG::KI) {
        constexpr int RPI = 1024 / SG::KRB;
        const int row = j * RPI + lane / KCH;
        const int chunk = (lane % KCH) ^ attn_kswz<NT, KCH>(row);
        const T* src = blk ? bkb + (size_t)min(row, a.B - 1) * kd : hb + (size_t)(k0 + row) * HD;
        dma16<true>(reinterpret_cast<const char*>(src) + chunk * 16, base + j * 1024);
      } else {
        constexpr int RPI = 1024 / SG::VRB;
        const int row = (j - SG::KI) * RPI + lane / VCH;  // tile-major V^T row: tile row / HD, d row % HD
        const int d = row % HD;
        const int chunk = (lane % VCH) ^ attn_vswz<VCH>(d);
        // the block has one V^T tile (B <= 16 keys); later tiles of its stage
        // re-read it (their keys are masked)
        const T* src = blk ? bvt + (size_t)d * a.BP : hb + a.kv_stride + ((size_t)(k0 / kVTile) * HD + row) * kVTile;
        dma16<true>(reinterpret_cast<const char*>(src) + chunk * 16, base + j * 1024);
      }
    }
  };

  f32x4_t o[QW][DF];
#pragma unroll
  for (int q = 0; q < QW; ++q)
#pragma unroll
    for (int d = 0; d < DF; ++d) o[q][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[QW], lrow[QW];
#pragma unroll
  for (int q = 0; q < QW; ++q) {
    mrow[q] = -INFINITY;
    lrow[q] = 0.f;
  }

#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nst) issue(p, p);

  int buf = 0;
  for (int i = 0; i < nst; ++i) {
    static_assert(NBUF >= 2 && SG::NIW * (NBUF - 2) < 64, "ring depth");
    wait_items<SG::NIW, NBUF - 2>(min(NBUF - 2, nst - 1 - i));
    ring_barrier();
    if (i + NBUF - 1 < nst) {
      int nb = buf + NBUF - 1;
      nb = nb >= NBUF ? nb - NBUF : nb;
      issue(i + NBUF - 1, nb);
    }
    const bool blk = i >= nctx;
    const int klim = blk ? a.B : kend - (kbeg + i * STG);  // valid keys in this stage
    const char* kl = lds + buf * SG::BUF;
    const char* vl = kl + SG::KBYTES;
    // S^T for every key of the stage first (the MFMA chains interleave; one K
    // fragment read feeds the QW query fragments), then one online-softmax
    // update per query column for the whole stage.  No branch on the valid
    // key count here: masked keys are cheap.
    f32x4_t cs[QW][PVS][NT];
#pragma unroll
    for (int h = 0; h < HS; ++h)
#pragma unroll
      for (int p = 0; p < PVS; ++p)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int krow = p * KS + (r16 >> 2) * (4 * NT) + 4 * t + (r16 & 3);
          const uint4 kf =
              *reinterpret_cast<const uint4*>(kl + krow * SG::KRB + (((h * 4 + kg) ^ attn_kswz<NT, KCH>(krow)) << 4));
#pragma unroll
          for (int q = 0; q < QW; ++q)
            cs[q][p][t] = MM::step(kf, qf[q][h], h == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : cs[q][p][t]);
        }
    float sv[QW][PVS][NT][4];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
      float mx = -INFINITY;
      if (klim >= STG) {  // full stage: no key to mask
#pragma unroll
        for (int p = 0; p < PVS; ++p)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              sv[q][p][t][ii] = cs[q][p][t][ii] * a.scale_log2;
              mx = fmaxf(mx, sv[q][p][t][ii]);
            }
      } else {
#pragma unroll
        for (int p = 0; p < PVS; ++p)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const int key = p * KS + kg * (4 * NT) + 4 * t + ii;
              sv[q][p][t][ii] = key < klim ? cs[q][p][t][ii] * a.scale_log2 : -INFINITY;
              mx = fmaxf(mx, sv[q][p][t][ii]);
            }
      }
      mx = xor32_max(xor16_max(mx));
      // The reference maximum of a query column moves only when a score
      // exceeds it by more than kAttnSlack (log2 units): probabilities are
      // then at most 2^kAttnSlack, and l and O, which share the reference,
      // are rescaled together, so the result is unchanged in exact
      // arithmetic.  The rescale of O is skipped when no column of the wave
      // moves (the common case once the first keys have been seen).
      const bool mv = mx > mrow[q] + kAttnSlack;
      if (__any(mv)) {
        const float mnew = mv ? mx : mrow[q];  // finite: every stage holds a valid key
        const float alpha = __builtin_amdgcn_exp2f(mrow[q] - mnew);
        lrow[q] *= alpha;
        mrow[q] = mnew;
#pragma unroll
        for (int d = 0; d < DF; ++d) o[q][d] *= alpha;
      }
      float ps = 0.f;
#pragma unroll
      for (int p = 0; p < PVS; ++p)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            // hardware exp2: arguments are <= kAttnSlack; results below 2^-126
            // flush to zero, far below the weight of any contributing key
            sv[q][p][t][ii] = __builtin_amdgcn_exp2f(sv[q][p][t][ii] - mrow[q]);
            ps += sv[q][p][t][ii];
          }
      lrow[q] += xor32_sum(xor16_sum(ps));
    }
#pragma unroll
    for (int p = 0; p < PVS; ++p) {
      const int kb0 = p * KS;
      if (kb0 >= klim) break;
      uint4 pp[QW];
#pragma unroll
      for (int q = 0; q < QW; ++q) {
        if constexpr (NT == 1) {
          pp[q] = make_uint4(__float_as_uint(sv[q][p][0][0]), __float_as_uint(sv[q][p][0][1]),
                             __float_as_uint(sv[q][p][0][2]), __float_as_uint(sv[q][p][0][3]));
        } else {
          pp[q].x = (uint32_t)f2bf(sv[q][p][0][0]) | ((uint32_t)f2bf(sv[q][p][0][1]) << 16);
          pp[q].y = (uint32_t)f2bf(sv[q][p][0][2]) | ((uint32_t)f2bf(sv[q][p][0][3]) << 16);
          pp[q].z = (uint32_t)f2bf(sv[q][p][1][0]) | ((uint32_t)f2bf(sv[q][p][1][1]) << 16);
          pp[q].w = (uint32_t)f2bf(sv[q][p][1][2]) | ((uint32_t)f2bf(sv[q][p][1][3]) << 16);
        }
      }
      const int vkey = kb0 + kg * 4 * NT;  // first of this lane's keys
      const char* vt = vl + (vkey / kVTile) * SG::TILEB;
      const int vchunk = (vkey % kVTile) * (int)sizeof(T) / 16;
#pragma unroll
      for (int d = 0; d < DF; ++d) {
        const int vrow = d * 16 + r16;
        const uint4 vf = *reinterpret_cast<const uint4*>(vt + vrow * SG::VRB + ((vchunk ^ attn_vswz<VCH>(vrow)) << 4));
#pragma unroll
        for (int q = 0; q < QW; ++q) o[q][d] = MM::step(vf, pp[q], o[q][d]);
      }
    }
    buf = buf + 1 == NBUF ? 0 : buf + 1;
  }

  {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < NPAD; ++i) x |= pad[i];
    asm volatile("" ::"v"(x));
  }
  float* po = a.part_o + (size_t)w * QR * HD;
  float* pml = a.part_ml + (size_t)w * QR * 2;
#pragma unroll
  for (int q = 0; q < QW; ++q) {
    const int qrow = (f * QW + q) * 16 + r16;
#pragma unroll
    for (int d = 0; d < DF; ++d)
      *reinterpret_cast<f32x4_t*>(po + (size_t)qrow * HD + d * 16 + 4 * kg) = o[q][d];
    if (kg == 0) {
      pml[qrow * 2] = mrow[q];
      pml[qrow * 2 + 1] = lrow[q];
    }
  }
}

// Merge the splits of every (r, g).  SUB consecutive lanes share one
// (query row, 4 channels) output: lane `sub` folds splits sub, sub+SUB, ...
// with a running maximum, then the SUB partial states are merged with
// shuffles in a fixed pattern, so results are deterministic.
template <typename T, int HD, int QR, int SUB>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs<T> a) {
  const int GB = a.G * a.B;
  const int per_rg = GB * (HD / 4);
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const int sub = (int)(t % SUB);
  const long o = t / SUB;
  const int rg = (int)(o / per_rg);
  const bool live = rg < a.meta.n_req * a.Hkv;
  const int rgc = live ? rg : 0;
  const int rem = (int)(o - (long)rgc * per_rg);
  const int qi = live ? rem / (HD / 4) : 0, d4 = live ? rem - qi * (HD / 4) : 0;
  const int r = rgc / a.Hkv, g = rgc - r * a.Hkv;
  const int S = live ? a.meta.nsplit[r] : 0;
  const int w0 = a.meta.work0[r] + g * S;
  float M = -INFINITY, den = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = sub; s < S; s += SUB) {
    const size_t pidx = (size_t)(w0 + s) * QR + qi;
    const float mv = a.part_ml[pidx * 2], lv = a.part_ml[pidx * 2 + 1];
    const f32x4_t ov = *reinterpret_cast<const f32x4_t*>(a.part_o + pidx * HD + d4 * 4);
    const float Mn = fmaxf(M, mv);
    const float rs = exp2f(M - Mn), e = exp2f(mv - Mn);
    den = den * rs + e * lv;
    acc = acc * rs + e * ov;
    M = Mn;
  }
#pragma unroll
  for (int x = 1; x < SUB; x <<= 1) {
    const float M2 = __shfl_xor(M, x);
    const float d2 = __shfl_xor(den, x);
    f32x4_t a2;
#pragma unroll
    for (int i = 0; i < 4; ++i) a2[i] = __shfl_xor(acc[i], x);
    const float Mn = fmaxf(M, M2);
    const float r1 = M == -INFINITY ? 0.f : exp2f(M - Mn);
    const float r2 = M2 == -INFINITY ? 0.f : exp2f(M2 - Mn);
    den = den * r1 + d2 * r2;
    acc = acc * r1 + a2 * r2;
    M = Mn;
  }
  if (!live || sub != 0) return;
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
