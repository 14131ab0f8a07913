// Operands, fused epilogues and the skinny (few-token) MFMA GEMM.
//
//   C[m, f] = s_m * sum_k A[m, k] * W[f, k]
//
// W is a "virtual" weight: the concatenation of up to kMaxSeg [rows, K]
// matrices (e.g. [W_q; W_kb; W_vb]).  A is [M, K] with K optionally split into
// segments at separate addresses (the L tapped target layers of the fusion
// step are read in place).  s_m is an optional per-row RMSNorm scale
// rsqrt(mean(x_m^2) + eps): the producer of A already multiplied x by the
// norm gain and left per-16-feature sums of squares, so the norm costs the
// consumer one short reduction in its epilogue and no extra pass.
//
// MFMA orientation: W rows are the 16-row A operand and activation rows the
// 16-column B operand, so a lane ends up holding 4 consecutive features of one
// token (C[4*(l>>4) + i][l & 15]).
//
// Paired epilogues (RoPE, SwiGLU) need feature f and its partner f + P in one
// lane: with a pair distance P, 16-feature groups 2i and 2i+1 map to features
// (first half) and (first half + P).
#pragma once
#include <type_traits>

#include "common.h"

namespace dfl {

template <typename T>
struct WOperand {
  const T* ptr[kMaxSeg];
  int end[kMaxSeg];  // cumulative row counts
  int nseg;
  int pair;     // 0 or the pair distance P (a multiple of 16)
  int ngroups;  // virtual rows / 16

  __device__ __forceinline__ int feature_of_group(int gi) const {
    if (pair == 0) return gi * 16;
    const int pi = gi >> 1, half = gi & 1;
    const int per = pair >> 4;
    return (pi / per) * 2 * pair + (pi % per) * 16 + half * pair;
  }
  // Row f of the virtual weight.  Segments hold whole 16-row groups, so a
  // caller passes the first row of a group (wave-uniform: the segment search
  // then runs on scalar kernel-argument loads) and adds the row in the group.
  __device__ __forceinline__ const T* row(int f, int K) const {
    int s = 0;
    while (s + 1 < nseg && f >= end[s]) ++s;
    const int r = f - (s ? end[s - 1] : 0);
    return ptr[s] + (size_t)r * K;
  }
};

template <typename T>
struct AOperand {
  const T* ptr[kMaxKSeg];
  int nk;        // K segments
  int kseg;      // columns per segment (multiple of the MFMA k-step)
  int lda;       // row stride (elements)
  int M;         // logical rows
  int rowmap_b;  // 0: identity; B > 1: logical row i reads row (i/(B-1))*B + 1 + i%(B-1)
  long lo_off;   // element offset of the low-half plane (split activations), 0 if none
  __device__ __forceinline__ int row(int i) const {
    if (!rowmap_b) return i;
    const int r = i / (rowmap_b - 1);
    return r * rowmap_b + 1 + (i - r * (rowmap_b - 1));
  }
};

// RMSNorm folded into a consumer: sums of squares per (row, 16-feature slot).
struct NormIn {
  const float* ssq;  // nullable: no row scale
  int nslot;         // D / 16
  float inv_d, eps;
};

// Row scale for this lane's token row `arow` (physical row); all 64 lanes of
// the wave must call it.  The 4 lanes of a token (same l & 15) each sum a
// contiguous quarter of the slots and combine with two butterflies.
__device__ __forceinline__ float norm_scale(const NormIn& n, int arow, int kg) {
  if (!n.ssq) return 1.0f;
  const int q = n.nslot >> 2;  // slots per lane (nslot is a multiple of 4)
  const float* p = n.ssq + (size_t)arow * n.nslot + kg * q;
  float s = 0.f;
  int j = 0;
  // eight independent 16-byte loads in flight per batch (a one-load-at-a-time
  // loop costs a memory latency per 4 slots)
  for (; j + 32 <= q; j += 32) {
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4_t*>(p + j + 4 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (v[u][0] + v[u][1]) + (v[u][2] + v[u][3]);
  }
  for (; j + 4 <= q; j += 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p + j);
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
  for (; j < q; ++j) s += p[j];
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  return 1.0f / sqrtf(s * n.inv_d + n.eps);
}

// Split-K across work-groups: the last work-group of a tile to finish sums
// the partials in split order and runs the epilogue.
struct SplitK {
  int SK;       // splits
  int kps;      // K stages per split
  float* part;  // [tiles][SK][waves][FM * FN * 256]
  int* ctr;     // [tiles] tickets, zero between launches (reset by the last arriver)
  int wstream;  // copy weights with the non-temporal hint (few token tiles share each weight tile)
};

// ---------------------------------------------------------------- helpers

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
  v.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
  *reinterpret_cast<uint2*>(p) = v;
}

template <typename T>
__device__ __forceinline__ f32x4_t load4(const T* p);
template <>
__device__ __forceinline__ f32x4_t load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
template <>
__device__ __forceinline__ f32x4_t load4<bf16_t>(const bf16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4_t{bf2f((bf16_t)(v.x & 0xffff)), bf2f((bf16_t)(v.x >> 16)), bf2f((bf16_t)(v.y & 0xffff)),
                 bf2f((bf16_t)(v.y >> 16))};
}

// x rounded to the storage type, back in float.
template <typename T>
__device__ __forceinline__ float round_to(float x) {
  return to_f<T>(from_f<T>(x));
}

// Sum over the 4 lanes holding one token (fixed butterfly order).
__device__ __forceinline__ float token_sum(float s) {
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  return s;
}

// ---------------------------------------------------------------- epilogues
// Unpaired: apply1(m, valid, f, v) - v holds features f..f+3 of row m (this
// lane's part of one 16-feature fragment).  Paired: apply2(m, valid, f, a, b)
// - a holds features f..f+3, b the partners f+P..f+P+3.  Every lane calls
// the epilogue (shuffles inside); stores are guarded by `valid`.  A paired
// epilogue with kScaled takes apply2s(m, valid, f, a, b, sc) instead: the raw
// sums and the row scale of the folded RMSNorm (1 without a norm) apart.

template <class E, class = void>
struct EpiScaled : std::false_type {};
template <class E>
struct EpiScaled<E, std::void_t<decltype(E::kScaled)>> : std::integral_constant<bool, E::kScaled> {};

template <class Epi>
__device__ __forceinline__ void call_paired(const Epi& epi, int m, bool valid, int f, f32x4_t a, f32x4_t b,
                                            float sc) {
  if constexpr (EpiScaled<Epi>::value)
    epi.apply2s(m, valid, f, a, b, sc);
  else
    epi.apply2(m, valid, f, a * sc, b * sc);
}

// Fusion output: u = T(z * g) (plus the low half z*g - u when lo != 0), and
// per-16-feature sums of squares of z.
template <typename T>
struct EpiNormOut {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = false;
  T* u;
  T* lo;  // nullable low-half plane
  const T* g;
  float* ssq;
  int ld, nslot;
  __device__ __forceinline__ void apply1(int m, bool valid, int f, f32x4_t v) const {
    const float ss = token_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
    if (!valid) return;
    const f32x4_t gg = load4<T>(g + f);
    const f32x4_t y = v * gg;
    store4<T>(u + (size_t)m * ld + f, y[0], y[1], y[2], y[3]);
    if (lo)
      store4<T>(lo + (size_t)m * ld + f, y[0] - round_to<T>(y[0]), y[1] - round_to<T>(y[1]),
                y[2] - round_to<T>(y[2]), y[3] - round_to<T>(y[3]));
    if ((threadIdx.x & 63) < 16) ssq[(size_t)m * nslot + (f >> 4)] = ss;
  }
};

// Residual: x += v; u = T(x * g_next); per-16-feature sums of squares of x.
template <typename T>
struct EpiResidualNorm {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = false;
  float* x;
  T* u;
  const T* g;
  float* ssq;
  int ld, nslot;
  __device__ __forceinline__ void apply1(int m, bool valid, int f, f32x4_t v) const {
    f32x4_t* xp = reinterpret_cast<f32x4_t*>(x + (size_t)m * ld + f);
    const f32x4_t xn = valid ? *xp + v : v;
    const float ss = token_sum(xn[0] * xn[0] + xn[1] * xn[1] + xn[2] * xn[2] + xn[3] * xn[3]);
    if (!valid) return;
    *xp = xn;
    const f32x4_t gg = load4<T>(g + f);
    store4<T>(u + (size_t)m * ld + f, xn[0] * gg[0], xn[1] * gg[1], xn[2] * gg[2], xn[3] * gg[3]);
    if ((threadIdx.x & 63) < 16) ssq[(size_t)m * nslot + (f >> 4)] = ss;
  }
};

// h[m, f] = SiLU(gate) * up; the pair is (gate, up).
template <typename T>
struct EpiSwiGLU {
  static constexpr bool kPaired = true;
  static constexpr bool kRow = false;
  T* h;
  int ldh;
  __device__ __forceinline__ void apply2(int m, bool valid, int f, f32x4_t g, f32x4_t u) const {
    if (!valid) return;
    store4<T>(h + (size_t)m * ldh + f, silu(g[0]) * u[0], silu(g[1]) * u[1], silu(g[2]) * u[2],
              silu(g[3]) * u[3]);
  }
};

// Rotate-half RoPE of channel pairs (c, c + hd/2) at table row `pos`.
__device__ __forceinline__ void rope4(const float2* tab, int half, int pos, int c, int use, f32x4_t& a,
                                      f32x4_t& b) {
  if (!use) return;
  const float2* t = tab + (size_t)pos * half + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 cs = t[i];
    const float x1 = a[i], x2 = b[i];
    a[i] = x1 * cs.x - x2 * cs.y;
    b[i] = x2 * cs.x + x1 * cs.y;
  }
}

// Block projections: virtual weight [W_q; W_kb; W_vb], pair distance hd/2.
// Q and K_b are rotated at absolute position ctx[r] + j and stored row-major;
// V_b is stored transposed per (request, kv head): vbT[((r*Hkv+g)*hd + d)*BP + j].
template <typename T>
struct EpiQKV {
  static constexpr bool kPaired = true;
  static constexpr bool kRow = false;
  T* q;
  T* kb;
  T* vbT;
  const float2* rope;
  int Hq, Hkv, hd, BP, use_rope;
  DraftMeta meta;
  __device__ __forceinline__ void one(int m, int f, f32x4_t a, f32x4_t b) const {
    const int B = meta.B;
    const int r = m / B, j = m - r * B;
    const int qd = Hq * hd, kd = Hkv * hd, half = hd >> 1;
    const int c = f % hd;  // < hd/2 by the pairing
    if (f < qd + kd) {
      rope4(rope, half, meta.ctx[r] + j, c, use_rope, a, b);
      T* dst = f < qd ? q + (size_t)m * qd + f : kb + (size_t)m * kd + (f - qd);
      store4<T>(dst, a[0], a[1], a[2], a[3]);
      store4<T>(dst + half, b[0], b[1], b[2], b[3]);
    } else {
      const int fv = f - qd - kd;
      const int g = fv / hd;
      T* base = vbT + ((size_t)(r * Hkv + g) * hd + c) * BP + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base[(size_t)i * BP] = from_f<T>(a[i]);
        base[(size_t)(i + half) * BP] = from_f<T>(b[i]);
      }
    }
  }
  __device__ __forceinline__ void apply2(int m, bool valid, int f, f32x4_t a, f32x4_t b) const {
    if (valid) one(m, f, a, b);
  }
};

// Context projections of the fusion step: virtual weight
// [W_kc^0; W_vc^0; W_kc^1; W_vc^1; ...], pair distance hd/2.  Keys are rotated
// at their absolute positions and written row-major into the slot's cache;
// values are written transposed in kVTile-key tiles (cache layout
// [Hkv][ctx_pad/kVTile][hd][kVTile]).
template <typename T>
struct EpiKVAppend {
  static constexpr bool kPaired = true;
  static constexpr bool kRow = false;
  T* pool;
  size_t slot_stride, layer_stride, kv_stride, head_stride;
  const float2* rope;
  int Hkv, hd, use_rope, row_base;
  FuseMeta meta;
  __device__ __forceinline__ void one(int m, int f, f32x4_t a, f32x4_t b) const {
    const int per_layer = 2 * Hkv * hd;
    const int layer = f / per_layer;
    int rem = f - layer * per_layer;
    const int isv = rem >= Hkv * hd;
    rem -= isv * Hkv * hd;
    const int g = rem / hd, c = rem - g * hd, half = hd >> 1;
    const int gm = row_base + m;
    const int r = fuse_req_of_row(meta, gm);
    const int pos = meta.pos0[r] + gm - meta.row0[r];
    T* base = pool + (size_t)meta.slot[r] * slot_stride + (size_t)layer * layer_stride +
              (size_t)isv * kv_stride + (size_t)g * head_stride;
    if (!isv) {
      rope4(rope, half, pos, c, use_rope, a, b);
      T* dst = base + (size_t)pos * hd + c;
      store4<T>(dst, a[0], a[1], a[2], a[3]);
      store4<T>(dst + half, b[0], b[1], b[2], b[3]);
    } else {
      T* tile = base + (size_t)(pos / kVTile) * hd * kVTile + (pos % kVTile);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tile[(size_t)(c + i) * kVTile] = from_f<T>(a[i]);
        tile[(size_t)(c + half + i) * kVTile] = from_f<T>(b[i]);
      }
    }
  }
  __device__ __forceinline__ void apply2(int m, bool valid, int f, f32x4_t a, f32x4_t b) const {
    if (valid) one(m, f, a, b);
  }
};

// DFlow relay MLP, first layer: s = T(SiLU(v)).
template <typename T>
struct EpiSiLUOut {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = false;
  T* s;
  int ld;
  __device__ __forceinline__ void apply1(int m, bool valid, int f, f32x4_t v) const {
    if (valid) store4<T>(s + (size_t)m * ld + f, silu(v[0]), silu(v[1]), silu(v[2]), silu(v[3]));
  }
};

// DFlow relay MLP, second layer over the virtual weight w2 with pair distance
// D: a holds beta, b gamma for features f..f+3; x = e_mask + beta * LN(h) +
// gamma is stored (fp32) for the slot's next block at offset 2 + (row index
// within the request).
template <typename T>
struct EpiRelayOut {
  static constexpr bool kPaired = true;
  static constexpr bool kRow = false;
  float* rows;         // [max_slots][B][D]
  const float* lnh;    // [relay rows][D]
  const T* e_mask;
  int B, D;
  RelayMeta meta;
  __device__ __forceinline__ void apply2(int m, bool valid, int f, f32x4_t a, f32x4_t b) const {
    if (!valid) return;
    const int r = relay_req_of_row(meta, m);
    const int j = 2 + m - meta.row0[r];
    float* dst = rows + ((size_t)meta.slot[r] * B + j) * D + f;
    const float* ln = lnh + (size_t)m * D + f;
    f32x4_t x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_f<T>(e_mask[f + i]) + a[i] * ln[i] + b[i];
    *reinterpret_cast<f32x4_t*>(dst) = x;
  }
};

// DFlash 2 selector gate: g = sigmoid(v), fp32.
struct EpiSigmoidOut {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = false;
  float* g;
  int ld;
  __device__ __forceinline__ void apply1(int m, bool valid, int f, f32x4_t v) const {
    if (!valid) return;
    f32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = 1.0f / (1.0f + __expf(-v[i]));
    *reinterpret_cast<f32x4_t*>(g + (size_t)m * ld + f) = o;
  }
};

// Plain store of features f..f+3 of row m in OutT (fp32 or the storage type).
template <typename OutT>
struct EpiStore {
  static constexpr bool kPaired = false;
  static constexpr bool kRow = false;
  OutT* out;
  int ld;
  __device__ __forceinline__ void apply1(int m, bool valid, int f, f32x4_t v) const {
    if (!valid) return;
    store4<OutT>(out + (size_t)m * ld + f, v[0], v[1], v[2], v[3]);
  }
};

// ---------------------------------------------------------------- helpers for the GEMM kernels

template <typename T>
__device__ __forceinline__ const T* a_ptr(const AOperand<T>& a, int arow, int kg, int ks) {
  constexpr int KS = Mma<T>::KSTEP, EPL = Mma<T>::EPL;
  if (a.nk == 1) return a.ptr[0] + (size_t)arow * a.lda + kg * EPL + (size_t)ks * KS;
  const int nks_seg = a.kseg / KS;
  const int seg = ks / nks_seg;
  return a.ptr[seg] + (size_t)arow * a.lda + kg * EPL + (size_t)(ks - seg * nks_seg) * KS;
}

// Epilogue dispatch over a wave's FN fragments of one token row: pairs,
// single fragments, or (kRow) all FN fragments at once.  Fragments j >=
// nvalid lie past the last weight row and are not stored.
template <int FN, class Epi>
__device__ __forceinline__ void run_epilogue(const Epi& epi, int m, bool mvalid, int nvalid, const int (&fb)[FN],
                                             const f32x4_t (&acc)[FN], float sc, int kg) {
  if constexpr (Epi::kRow) {
    epi.template apply_row<FN>(m, mvalid, nvalid, fb, acc, sc, kg);
  } else if constexpr (Epi::kPaired) {
#pragma unroll
    for (int j = 0; j < FN; j += 2)
      call_paired(epi, m, mvalid && j + 1 < nvalid, fb[j] + 4 * kg, acc[j], acc[j + 1], sc);
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) epi.apply1(m, mvalid && j < nvalid, fb[j] + 4 * kg, acc[j] * sc);
  }
}

// ---------------------------------------------------------------- activation-stationary GEMV
//
// Few-token GEMM for the memory-bound case.  A work-group of NW waves (NW =
// blockDim/64 <= 16) walks a range of 16-row weight tiles; wave w owns the
// k-steps [c*NW*KSW + w*KSW, +KSW) of every K chunk c and keeps the matching
// activation fragments in registers, so the vector-memory path carries only
// the weight stream (re-reading activations from L2 costs a third of the
// bandwidth).  Tiles are processed in batches of up to TB: inside a batch the
// waves never synchronise (each writes its partial tile to LDS); one barrier
// per batch, then the partial tiles are summed in wave order and the
// epilogues run spread over the waves (a paired epilogue takes two
// consecutive tiles).
// When K spans several chunks the activations are reloaded per chunk (such
// GEMMs have one or two tiles per work-group).
//
// Work-group placement: with XR false the grid is (tile range, 16-row block)
// and weights stream past L2 (every row block of a tile range reads them
// once).  With XR true (many row blocks against a narrow weight) the grid is
// one-dimensional and the work-groups of a row block all run on one XCD
// (work-group i runs on XCD i mod 8), so each activation block is fetched
// into one L2 only; the weight, which every XCD then reads, is loaded with
// ordinary caching.

template <typename T, int KSW, bool ALO, int TB, bool XR, class Epi>
__global__ __launch_bounds__(1024) void gemv_as_kernel(const WOperand<T> w, const AOperand<T> a,
                                                        const NormIn nrm, const Epi epi, int tiles_per_wg) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  extern __shared__ __align__(16) char lds_raw[];
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds_raw);  // [TB][NW][64]
  const int NW = blockDim.x >> 6;
  // wave index as a scalar: the K segment of an activation fragment is then
  // picked with scalar loads instead of a per-lane load of the argument block
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  int tg = blockIdx.x, mb = blockIdx.y;
  if constexpr (XR) {
    const int nwg = (w.ngroups + tiles_per_wg - 1) / tiles_per_wg;
    const int j = blockIdx.x >> 3, q = j / nwg;
    tg = j - q * nwg;
    mb = q * 8 + (blockIdx.x & 7);
    if (mb * 16 >= a.M) return;
  }
  const int t_begin = tg * tiles_per_wg;
  const int t_end = min(w.ngroups, t_begin + tiles_per_wg);
  if (t_begin >= t_end) return;
  const int m0 = mb * 16;
  const int K = a.nk * a.kseg;
  const int nks = K / KS;
  const int span = NW * KSW;
  const int nchunks = (nks + span - 1) / span;
  const int m = m0 + r16;
  const int arow = a.row(m < a.M ? m : a.M - 1);

  uint4 areg[KSW], alo[KSW];
  auto load_a = [&](int c) {
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const int ks = c * span + wave * KSW + j;
      if (ks < nks) {
        const T* ap = a_ptr(a, arow, kg, ks);
        areg[j] = ld16(ap);
        if constexpr (ALO) alo[j] = ld16(ap + a.lo_off);
      } else {
        areg[j] = make_uint4(0, 0, 0, 0);
        if constexpr (ALO) alo[j] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto wrow = [&](int t) { return w.row(w.feature_of_group(t), K) + (size_t)r16 * K + kg * EPL; };
  auto load_w = [&](const T* wp, int c, uint4 (&wf)[KSW]) {
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const int ks = c * span + wave * KSW + j;
      if constexpr (XR)
        wf[j] = ks < nks ? ld16(wp + (size_t)ks * KS) : make_uint4(0, 0, 0, 0);
      else
        wf[j] = ks < nks ? ld16_stream(wp + (size_t)ks * KS) : make_uint4(0, 0, 0, 0);
    }
  };

  if (nchunks == 1) load_a(0);
  // Row norm: with nslot a multiple of 16 x NW (up to two 16-byte loads per
  // lane) the waves split the slots, each lane loads its share now and the
  // sums meet in LDS at the first barrier, so the scale costs no latency of
  // its own; otherwise every wave reduces the whole row up front.
  __shared__ float nsum[16 * 64];
  const int c4 = nrm.ssq ? nrm.nslot / (16 * NW) : 0;
  const bool nsplit = c4 >= 1 && c4 <= 2 && c4 * 16 * NW == nrm.nslot;
  f32x4_t nv0 = {0.f, 0.f, 0.f, 0.f}, nv1 = {0.f, 0.f, 0.f, 0.f};
  float sc = 1.0f;
  if (nsplit) {
    const float* p = nrm.ssq + (size_t)arow * nrm.nslot + (wave * 4 + kg) * 4 * c4;
    nv0 = *reinterpret_cast<const f32x4_t*>(p);
    if (c4 == 2) nv1 = *reinterpret_cast<const f32x4_t*>(p + 4);
  } else {
    sc = norm_scale(nrm, arow, kg);
  }
  for (int b0 = t_begin; b0 < t_end; b0 += TB) {
    const int bt = min(TB, t_end - b0);
    const int items = bt * nchunks;  // (tile, chunk) in order
    const T* wp = wrow(b0);
    uint4 wcur[KSW];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < items; ++it) {
      const int tl = it / nchunks, c = it - tl * nchunks;
      if (nchunks > 1) load_a(c);
      if (c == 0) wp = wrow(b0 + tl);
      load_w(wp, c, wcur);
#pragma unroll
      for (int j = 0; j < KSW; ++j) {
        acc = MM::step(wcur[j], areg[j], acc);
        if constexpr (ALO) acc = MM::step(wcur[j], alo[j], acc);
      }
      if (c == nchunks - 1) {
        red[(tl * NW + wave) * 64 + lane] = acc;
        acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    const bool first = b0 == t_begin;
    if (nsplit && first)
      nsum[wave * 64 + lane] = ((nv0[0] + nv0[1]) + (nv0[2] + nv0[3])) + ((nv1[0] + nv1[1]) + (nv1[2] + nv1[3]));
    __syncthreads();
    if (nsplit && first) {
      float ss = 0.f;
      for (int w2 = 0; w2 < NW; ++w2) ss += nsum[w2 * 64 + lane];
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      sc = 1.0f / sqrtf(ss * nrm.inv_d + nrm.eps);
    }
    // reduce + epilogue: unit j (a tile, or a pair of tiles) handled by wave j % NW
    constexpr int PT = Epi::kPaired ? 2 : 1;
    for (int j = wave; j * PT < bt; j += NW) {
      f32x4_t sum[PT];
#pragma unroll
      for (int p = 0; p < PT; ++p) {
        const int tl = j * PT + p;
        sum[p] = red[(tl * NW) * 64 + lane];
        for (int w2 = 1; w2 < NW; ++w2) sum[p] += red[(tl * NW + w2) * 64 + lane];
      }
      const int t = b0 + j * PT;
      if constexpr (Epi::kRow) {
        const int fb1[1] = {w.feature_of_group(t)};
        epi.template apply_row<1>(m, m < a.M, 1, fb1, sum, sc, kg);
      } else if constexpr (Epi::kPaired) {
        call_paired(epi, m, m < a.M, w.feature_of_group(t) + 4 * kg, sum[0], sum[1], sc);
      } else {
        epi.apply1(m, m < a.M, w.feature_of_group(t) + 4 * kg, sum[0] * sc);
      }
    }
    __syncthreads();
  }
}

}  // namespace dfl
