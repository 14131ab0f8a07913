// Row-streaming skinny GEMM: few tokens against a wide weight, HBM-bound.
//
//   C[m, f] = s_m * sum_k A[m, k] * W[f, k]      (operands as in gemm.h)
//
// A work-group of 16 waves owns one 16-token block, one K range and a run of
// 16-row weight tiles.  A tile is streamed through an LDS ring in stages of
// 1 KB per row: in each stage wave w copies 1 KB of tile row w with one
// global -> LDS instruction (64 lanes x 16 contiguous bytes).  Whole-row pieces
// per wave instruction stream from HBM markedly faster than the MFMA operand
// layout (16 rows x 64 bytes per instruction).  The copy permutes the 16-byte
// chunks of row r inside each 128-byte window (chunk c lands at slot
// c ^ (r & 7)), so the fragment reads of 8 rows at one chunk fall on 8
// distinct bank groups.
//
// Each stage holds 16 MFMA k-steps; wave w contracts k-step w against its
// activation fragment, held in registers for the work-group's whole K range
// (loaded once, before the first copy).  Copies run NBUF-1 stages ahead; a
// stage ends with one work-group barrier.  When the last stage of a tile is
// done every wave parks its 16x16 partial in LDS; after the next barrier one
// wave sums the 16 partials in wave order and either runs the epilogue at once
// (row epilogues, which only store) or parks the sum until the stream has
// ended, so that no epilogue load waits behind in-flight copies (the
// vector-memory counter retires in order).
//
// K may be split over work-groups (grid.y = splits x token blocks): each split
// publishes its tile sums with agent-scope stores, takes a ticket, and the
// last one to arrive adds the splits in index order (with two splits, the
// other one to its own) and runs the epilogue.
//
// Paired epilogues (RoPE, SwiGLU, the relay's beta/gamma) use tiles of 8 + 8
// rows: rows 0-7 are features f0..f0+7 and rows 8-15 their partners
// f0+P..f0+P+7, so a tile is self-contained and the partner values sit in lane
// l ^ 32 of the same wave.
#pragma once
#include "gemm_tiled.h"

namespace dfl {

constexpr int kRsStage = 1024;  // bytes of one weight row per stage
constexpr int kRsAH = 16;       // activation fragments held per wave (stages per K range)
constexpr int kRsLdsMax = 160 * 1024;

// Stages per K range the kernel can hold (hi + lo planes take twice the registers).
__host__ __device__ constexpr int gemv_rs_ah(bool alo) { return alo ? kRsAH / 2 : kRsAH; }

// LDS layout: ring [NBUF][16 rows][1 KB]; wave partials [1 or 2][16][1 KB]
// (two buffers when some K range is a single stage: a tile's partials are then
// written in the stage whose barrier the previous tile's sum follows); tile
// sums [tiles][1 KB]; norm partials [16][64] floats.
__host__ __device__ constexpr int gemv_rs_red_bytes(bool red2) { return (red2 ? 2 : 1) * 16 * 1024; }
__host__ __device__ constexpr int gemv_rs_lds(int nbuf, bool red2, int tiles) {
  return nbuf * 16 * kRsStage + gemv_rs_red_bytes(red2) + tiles * 1024 + 16 * 64 * 4;
}

struct RsSplit {
  int nsplit;   // K ranges (grid.y = nsplit x token blocks)
  int nst;      // stages per K range (the last range may be shorter)
  int red2;     // some K range is a single stage: two partial buffers
  float* part;  // [token blocks][ngroups][nsplit][256] tile sums
  int* ctr;     // [token blocks][ngroups] tickets, zero between launches
  int wstream;  // copy weights with the non-temporal hint (few token blocks share them)
};

// NBUF: ring depth.  ALO: activations as hi + lo planes.  PAIR8: 8 + 8 row
// tiles (paired epilogues).  The dynamic LDS size is gemv_rs_lds(NBUF, stages
// per K range, tiles_per_wg).
template <typename T, int NBUF, bool ALO, bool PAIR8, class Epi>
__global__ __launch_bounds__(1024) void gemv_rs_kernel(const WOperand<T> w, const AOperand<T> a,
                                                       const NormIn nrm, const RsSplit sp, const Epi epi,
                                                       int tiles_per_wg) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int SB = kRsStage;
  constexpr int TILE = 16 * SB;
  constexpr int AH = gemv_rs_ah(ALO);
  static_assert(SB / (KS * (int)sizeof(T)) == 16, "one k-step per wave per stage");
  static_assert(PAIR8 == Epi::kPaired, "paired epilogues take 8 + 8 row tiles");
  static_assert(NBUF >= 2, "ring depth");
  extern __shared__ __align__(16) char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(w.ngroups, t_begin + tiles_per_wg);
  if (t_begin >= t_end) return;
  const int ks_id = blockIdx.y % sp.nsplit, mb = blockIdx.y / sp.nsplit;
  const int K = a.nk * a.kseg;
  const int nst_all = K * (int)sizeof(T) / SB;
  const int st0 = ks_id * sp.nst;
  const int nst = min(sp.nst, nst_all - st0);
  if (nst <= 0) return;
  const int ntiles = t_end - t_begin;
  const int G = ntiles * nst;
  char* ring = lds;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + NBUF * TILE);  // wave partials
  const int red_alt = sp.red2 ? 16 * 64 : 0;                     // second buffer (single-stage tiles)
  f32x4_t* res = reinterpret_cast<f32x4_t*>(lds + NBUF * TILE + gemv_rs_red_bytes(sp.red2));  // tile sums
  float* nsum = reinterpret_cast<float*>(lds + NBUF * TILE + gemv_rs_red_bytes(sp.red2) + tiles_per_wg * 1024);
  const int m = mb * 16 + r16;
  const bool mvalid = m < a.M;
  const int arow = a.row(mvalid ? m : a.M - 1);

  // Feature of row `row` of tile t.
  auto feat = [&](int t, int row) -> int {
    if constexpr (PAIR8) {
      const int per = w.pair >> 3;
      const int f0 = (t / per) * 2 * w.pair + (t % per) * 8;
      return row < 8 ? f0 + row : f0 + w.pair + (row - 8);
    } else {
      return t * 16 + row;
    }
  };
  // Copy cursor (all scalar: every wave walks the same stages, and 16 waves
  // share one scalar unit, so the per-stage bookkeeping is kept to a few
  // increments; the tile's row address is looked up once per tile).
  const int swz = lane ^ (wave & 7);  // source chunk of this lane's LDS slot (tile row = wave)
  auto row_src = [&](int tl) {
    return reinterpret_cast<const char*>(w.row(feat(t_begin + tl, wave), K)) + st0 * SB;
  };
  int c_tl = 0, c_s = 0, c_buf = 0;
  const char* c_src = row_src(0);
  char* const c_dst = ring + wave * SB;
  auto issue = [&]() {
    if (sp.wstream)
      dma16<true>(c_src + c_s * SB + (swz << 4), c_dst + c_buf * TILE);
    else
      dma16(c_src + c_s * SB + (swz << 4), c_dst + c_buf * TILE);
    c_buf = c_buf + 1 == NBUF ? 0 : c_buf + 1;
    if (++c_s == nst) {
      c_s = 0;
      if (++c_tl < ntiles) c_src = row_src(c_tl);
    }
  };
  const int roff = r16 * SB + ((((wave << 2) + kg) ^ (r16 & 7)) << 4);

  // Activation fragments of the K range (k-step 16 (st0 + s) + wave), then
  // NBUF - 1 padding loads: the compiler waits for fragment s with a count of
  // the loads it issued after it, and the padding keeps that count at or
  // above the copies in flight (which it does not see), so those waits never
  // drain the ring.
  uint4 ahi[AH], alo[AH];
#pragma unroll
  for (int s = 0; s < AH; ++s) {
    if (s < nst) {
      const T* ap = a_ptr(a, arow, kg, (st0 + s) * 16 + wave);
      ahi[s] = ld16(ap);
      if constexpr (ALO) alo[s] = ld16(ap + a.lo_off);
    }
  }
  // this lane's share of the folded RMSNorm's sums of squares (summed after
  // the stream; issued now so that their latency is hidden)
  constexpr int NQ = 4;
  float qv[NQ];
  const bool q_early = nrm.ssq && nrm.nslot <= 64 * NQ;
  if (q_early) {
    const float* q = nrm.ssq + (size_t)arow * nrm.nslot;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int j = wave * 4 + kg + 64 * i;
      qv[i] = j < nrm.nslot ? q[j] : 0.f;
    }
  }
  asm volatile("" ::: "memory");
  uint32_t pad[NBUF - 1];
  {
    // dwords 128 bytes apart in the first stage of this wave's weight row (not
    // mergeable into one instruction; the copy fetches the same lines next)
    const char* pp = reinterpret_cast<const char*>(w.row(feat(t_begin, wave), K)) + st0 * SB + (lane & 3) * 4;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) pad[i] = *reinterpret_cast<const uint32_t*>(pp + i * 128);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < G) issue();

  // Sum of the 16 wave partials of tile tl in wave order, parked for the
  // epilogue (no epilogue store is issued while copies are in flight: the
  // vector-memory counter retires in order, so it would hold up the ring).
  auto finish = [&](int tl) {
    const f32x4_t* p = red + (tl & 1) * red_alt + lane;
    f32x4_t s = p[0];
#pragma unroll
    for (int w2 = 1; w2 < 16; ++w2) s += p[w2 * 64];
    res[tl * 64 + lane] = s;
  };
  float sc = 1.0f;
  auto epilogue = [&](int tl, f32x4_t v) {
    const int t = t_begin + tl;
    if constexpr (Epi::kRow) {
      const int fb1[1] = {t * 16};
      const f32x4_t acc1[1] = {v};
      epi.template apply_row<1>(m, mvalid, 1, fb1, acc1, sc, kg);
    } else if constexpr (Epi::kPaired) {
      f32x4_t b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = __shfl_xor(v[i], 32);
      call_paired(epi, m, mvalid && kg < 2, feat(t, 4 * (kg & 1)), v, b, sc);
    } else {
      epi.apply1(m, mvalid, t * 16 + 4 * kg, v * sc);
    }
  };

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int left = G - 1;  // stages after the current one
  const char* rd = ring + roff;
  int r_buf = 0;
  for (int tl = 0; tl < ntiles; ++tl) {
#pragma unroll
    for (int s = 0; s < AH; ++s) {
      if (s < nst) {
        // own copy of this stage landed (younger ones may be in flight), then
        // everyone's, and everyone is past the previous stage, whose buffer
        // is refilled
        wait_items<1, NBUF - 2>(min(NBUF - 2, left));
        ring_barrier();
        if (left >= NBUF - 1) issue();
        if (s == 0 && tl > 0 && wave == ((tl - 1) & 15)) finish(tl - 1);
        const uint4 wf = *reinterpret_cast<const uint4*>(rd + r_buf * TILE);
        r_buf = r_buf + 1 == NBUF ? 0 : r_buf + 1;
        --left;
        acc = MM::step(wf, ahi[s], acc);
        if constexpr (ALO) acc = MM::step(wf, alo[s], acc);
        if (s == nst - 1) {
          red[(tl & 1) * red_alt + wave * 64 + lane] = acc;
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) x |= pad[i];
    asm volatile("" ::"v"(x));
  }

  // Row scale of the folded RMSNorm: the waves split the row's slots (slot
  // 4 wave + kg + 64 i for this lane's token) and meet in LDS.
  if (nrm.ssq) {
    float ps = 0.f;
    if (q_early) {
#pragma unroll
      for (int i = 0; i < NQ; ++i) ps += qv[i];
    } else {
      const float* q = nrm.ssq + (size_t)arow * nrm.nslot;
      for (int j = wave * 4 + kg; j < nrm.nslot; j += 64) ps += q[j];
    }
    nsum[wave * 64 + lane] = ps;
  }
  __syncthreads();
  if (wave == ((ntiles - 1) & 15)) finish(ntiles - 1);
  if (nrm.ssq) {
    float ss = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) ss += nsum[w2 * 64 + lane];
    sc = 1.0f / sqrtf(token_sum(ss) * nrm.inv_d + nrm.eps);
  }
  {
    __syncthreads();
    for (int tl = wave; tl < ntiles; tl += 16) {
      f32x4_t v = res[tl * 64 + lane];
      if (sp.nsplit > 1) {
        const int t = t_begin + tl;
        const size_t ti = (size_t)mb * w.ngroups + t;
        float* pt = sp.part + ti * sp.nsplit * 256;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          __hip_atomic_store(pt + ks_id * 256 + c * 64 + lane, v[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_vmcnt<0>();
        int ticket = 0;
        if (lane == 0) ticket = __hip_atomic_fetch_add(sp.ctr + ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __shfl(ticket, 0);
        if (ticket != sp.nsplit - 1) continue;
        if (sp.nsplit == 2) {
          // own + other is the same sum whichever arrived last (addition commutes)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            v[c] += __hip_atomic_load(pt + (1 - ks_id) * 256 + c * 64 + lane, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        } else {
          // the sum runs over every split in index order (the own one read back too)
          v = f32x4_t{0.f, 0.f, 0.f, 0.f};
          for (int x = 0; x < sp.nsplit; ++x)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              v[c] += __hip_atomic_load(pt + x * 256 + c * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) __hip_atomic_store(sp.ctr + ti, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      epilogue(tl, v);
    }
  }
}

}  // namespace dfl
