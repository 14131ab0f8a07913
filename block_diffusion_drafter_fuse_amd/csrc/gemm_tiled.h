// LDS-staged MFMA GEMM for many tokens (batched drafting, context prefill).
//
// Work-group tile BM tokens x BN features, 4 waves in WM x WN, each wave
// FM x FN fragments of 16 x 16.  Each K stage covers 128 bytes of every row
// (64 bf16 or 32 fp32 = two MFMA k-steps); stages are double-buffered in LDS
// (rows padded by 16 bytes against bank conflicts) with the next stage's
// global loads in flight while the current one is consumed.  With ALO the
// activations come as bf16 hi + lo planes (both staged) and every weight
// fragment feeds two MFMAs.  Blocks are
// ordered so that the work-groups of one XCD walk the M tiles of a weight tile
// back to back, which keeps that weight tile in the XCD's L2.
#pragma once
#include "gemm.h"

namespace dfl {

template <typename T, int BM, int BN, int WM, int WN, bool ALO, class Epi>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const WOperand<T> w, const AOperand<T> a,
                                                         const NormIn nrm, const SplitK sk, const Epi epi,
                                                         int nblocks) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int EPL = MM::EPL;
  constexpr int BKE = 128 / sizeof(T);  // elements per row per stage
  constexpr int KPS = BKE / KS;         // k-steps per stage (2)
  constexpr int ROWB = 128 + 16;        // padded LDS row bytes
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int CPR = 8;                // 16-byte chunks per row per stage
  constexpr int AR = ALO ? 2 * BM : BM; // staged activation rows (hi, then lo)
  constexpr int ACH = AR * CPR / 256;   // A chunks per thread
  constexpr int WCH = BN * CPR / 256;   // W chunks per thread
  static_assert(FN % 2 == 0, "paired epilogues take fragment pairs");
  static_assert(WM * WN == 4, "4 waves");

  extern __shared__ __align__(16) char lds[];
  // stage buffer b: AR activation rows at lds + b*(AR+BN)*ROWB, W rows after them
  auto lA = [&](int b) { return lds + b * (AR + BN) * ROWB; };
  auto lW = [&](int b) { return lds + b * (AR + BN) * ROWB + AR * ROWB; };

  // XCD-grouped block order (grid padded to a multiple of 8).
  const int per_xcd = gridDim.x >> 3;
  const int q = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (q >= nblocks) return;
  const int MT = (a.M + BM - 1) / BM;
  int t = q;
  const int s = t % sk.SK;
  t /= sk.SK;
  const int bm = t % MT, bn = t / MT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.nk * a.kseg;
  const int nst_total = K / BKE;
  const int st0 = s * sk.kps, st1 = min(nst_total, st0 + sk.kps);
  const int ngroups_tile0 = bn * (BN / 16);

  // Global chunk pointers for this thread (row and 16-byte column fixed per chunk).
  const char* gA[ACH];
  const char* gW[WCH];
  int oA[ACH], oW[WCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * 256;
    const int row = c / CPR, col = c % CPR;
    const int plane = row / BM;  // 0: hi, 1: lo
    int m = bm * BM + (row - plane * BM);
    m = m < a.M ? m : a.M - 1;
    gA[i] = reinterpret_cast<const char*>(a.ptr[0] + (size_t)a.row(m) * a.lda + plane * a.lo_off) + col * 16;
    oA[i] = row * ROWB + col * 16;
  }
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + i * 256;
    const int row = c / CPR, col = c % CPR;
    const int gi = ngroups_tile0 + row / 16;
    const int f = gi < w.ngroups ? w.feature_of_group(gi) + (row & 15) : (row & 15);
    gW[i] = reinterpret_cast<const char*>(w.row(f, K)) + col * 16;
    oW[i] = row * ROWB + col * 16;
  }
  // Activation segment base offset for stage st (segments are stage-aligned).
  const int st_per_seg = a.kseg / BKE;
  auto a_off = [&](int st) -> long {
    if (a.nk == 1) return (long)st * 128;
    const int seg = st / st_per_seg;
    return (long)(reinterpret_cast<const char*>(a.ptr[seg]) - reinterpret_cast<const char*>(a.ptr[0])) +
           (long)(st - seg * st_per_seg) * 128;
  };

  uint4 rA[ACH], rW[WCH];
  auto gload = [&](int st) {
    const long ao = a_off(st);
#pragma unroll
    for (int i = 0; i < ACH; ++i) rA[i] = ld16(gA[i] + ao);
#pragma unroll
    for (int i = 0; i < WCH; ++i) rW[i] = ld16_stream(gW[i] + (long)st * 128);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<uint4*>(lA(buf) + oA[i]) = rA[i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) *reinterpret_cast<uint4*>(lW(buf) + oW[i]) = rW[i];
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (st0 < st1) {
    gload(st0);
    lstore(0);
    __syncthreads();
  }
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    const bool more = st + 1 < st1;
    if (more) gload(st + 1);
#pragma unroll
    for (int kk = 0; kk < KPS; ++kk) {
      uint4 af[FM], al[FM], wf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * FM * 16 + i * 16 + r16;
        af[i] = *reinterpret_cast<const uint4*>(lA(buf) + row * ROWB + kk * 64 + kg * 16);
        if constexpr (ALO) al[i] = *reinterpret_cast<const uint4*>(lA(buf) + (BM + row) * ROWB + kk * 64 + kg * 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wf[j] = *reinterpret_cast<const uint4*>(lW(buf) + (wn * FN * 16 + j * 16 + r16) * ROWB + kk * 64 + kg * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = MM::step(wf[j], af[i], acc[i][j]);
          if constexpr (ALO) acc[i][j] = MM::step(wf[j], al[i], acc[i][j]);
        }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  if (sk.SK > 1) {
    const int tile = bn * MT + bm;
    constexpr int WTILE = FM * FN * 256;  // floats per wave
    float* pbase = sk.part + ((size_t)tile * sk.SK) * (4 * WTILE) + wave * WTILE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        *reinterpret_cast<f32x4_t*>(pbase + (size_t)s * (4 * WTILE) + (i * FN + j) * 256 + lane * 4) = acc[i][j];
    __threadfence();
    __syncthreads();
    __shared__ int prev_s;
    if (tid == 0) prev_s = atomicAdd(sk.ctr + tile, 1);
    __syncthreads();
    if (prev_s != sk.SK - 1) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int x = 0; x < sk.SK; ++x)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] += *reinterpret_cast<const f32x4_t*>(pbase + (size_t)x * (4 * WTILE) + (i * FN + j) * 256 +
                                                         lane * 4);
    if (tid == 0) sk.ctr[tile] = 0;
  }

  const int g0 = ngroups_tile0 + wn * FN;
  int fb[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[j] = g0 + j < w.ngroups ? w.feature_of_group(g0 + j) : 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = bm * BM + wm * FM * 16 + i * 16 + r16;
    const int arow = a.row(m < a.M ? m : a.M - 1);
    const float sc = norm_scale(nrm, arow, kg);
    run_epilogue<FN>(epi, m, m < a.M, w.ngroups - g0, fb, acc[i], sc, kg);
  }
}

}  // namespace dfl
