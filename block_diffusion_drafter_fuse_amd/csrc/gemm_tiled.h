// LDS-staged MFMA GEMM for many tokens (batched drafting, context prefill).
//
// Work-group tile BM tokens x BN features, WM x WN waves, each wave FM x FN
// fragments of 16 x 16.  Each K stage covers 128 bytes of every row
// (64 bf16 or 32 fp32 = two MFMA k-steps).  Stages are copied global -> LDS
// asynchronously (global_load_lds, 16 bytes per lane, no register round
// trip) into a ring of NBUF buffers, so NBUF-1 stages are in flight while one
// is consumed; one work-group barrier per stage.  A stage holds AR activation
// rows then BN weight rows, 128 bytes each, with the 16-byte chunks of row r
// stored at slot (chunk ^ (r & 7)): the copy of one wave instruction stays
// contiguous (8 whole rows) and the fragment reads of 8 lanes (8 rows, one
// chunk) fall on 8 distinct 16-byte bank groups.  K may be split over several
// work-groups: each split publishes its partial tile with device-coherent
// stores and the last one to arrive (atomic ticket) sums them and runs the
// epilogue, with no cache write-back or invalidate.  With ALO the activations
// come as bf16 hi + lo planes (both staged) and every weight fragment feeds
// two MFMAs.  Blocks are ordered so that the work-groups of one XCD walk the
// K splits and M tiles of one weight tile back to back, which keeps that
// weight tile in the XCD's L2.
#pragma once
#include <type_traits>

#include "gemm.h"

namespace dfl {

typedef __attribute__((address_space(3))) void* lds_dst_t;

// Asynchronous copy of 16 bytes per lane from `g` into LDS: lane i's bytes land
// at wave_base + 16 * i (wave_base is wave-uniform).  Counted by vmcnt and
// waited for explicitly (wait_vmcnt): the instruction is issued from inline
// assembly so that the compiler does not put a full vmcnt(0) in front of every
// LDS read that might alias a copy still in flight, which would serialise the
// stage ring.  Nothing else in the kernels that use it keeps a value in m0.
// STREAM: data that few work-groups read (the context K/V; weights shared by at
// most kStreamMaxShare token tiles) is copied with the non-temporal hint, so
// that lines read once do not hold the caches (attention at bs 32: 128 ->
// 107 us per layer; the bs 1 step 0.86 -> 0.80 ms).  Activations, re-read by
// many work-groups from L2, and weights shared by more token tiles (prefill)
// are copied without it: there the hint cost re-reads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool STREAM = false>
__device__ __forceinline__ void dma16(const void* g, char* wave_base) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_dst_t)wave_base);
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(m0v) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0v) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most y * IPI vector-memory instructions of this wave are
// outstanding (y in 0 .. MAXY, runtime; each case a compile-time count).
template <int IPI, int MAXY>
__device__ __forceinline__ void wait_items(int y) {
  if constexpr (MAXY <= 0) {
    wait_vmcnt<0>();
  } else {
    if (y >= MAXY) {
      wait_vmcnt<MAXY * IPI>();
      return;
    }
    wait_items<IPI, MAXY - 1>(y);
  }
}

// Work-group barrier for the stage ring: the wave's LDS reads are complete
// (so a buffer may be refilled after it) and no memory access is moved across.
// Outstanding asynchronous copies are not waited for here.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, int BM, int BN, int WM, int WN, int NBUF, bool ALO, class Epi>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(const WOperand<T> w, const AOperand<T> a,
                                                         const NormIn nrm, const SplitK sk, const Epi epi,
                                                         int nblocks) {
  using MM = Mma<T>;
  constexpr int KS = MM::KSTEP;
  constexpr int BKE = 128 / sizeof(T);  // elements per row per stage
  constexpr int KPS = BKE / KS;         // k-steps per stage (2)
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int AR = ALO ? 2 * BM : BM;  // staged activation rows (hi, then lo)
  constexpr int ROWS = AR + BN;
  constexpr int SBYTES = ROWS * 128;
  constexpr int NWV = WM * WN;
  constexpr int NI = ROWS / (8 * NWV);  // copy instructions per wave per stage (8 rows each)
  constexpr int NIA = AR / (8 * NWV);   // of which activation rows
  static_assert(FN % 2 == 0, "paired epilogues take fragment pairs");
  static_assert(AR % (8 * NWV) == 0 && BN % (8 * NWV) == 0, "stage rows in whole copy blocks");
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  static_assert(NI * (NBUF - 2) < 64, "vmcnt range");

  extern __shared__ __align__(16) char lds[];

  // XCD-grouped block order (grid padded to a multiple of 8).
  const int per_xcd = gridDim.x >> 3;
  const int q = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (q >= nblocks) return;
  const int MT = (a.M + BM - 1) / BM;
  int t = q;
  const int s = t % sk.SK;
  t /= sk.SK;
  const int bm = t % MT, bn = t / MT;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.nk * a.kseg;
  const int nst_total = K / BKE;
  const int st0 = s * sk.kps, st1 = min(nst_total, st0 + sk.kps);
  const int nst = st1 - st0;
  const int ngroups_tile0 = bn * (BN / 16);

  // Copy assignment: instruction i of wave v fills stage rows 8*(NWV*i+v) .. +7;
  // lane l covers row +(l>>3), slot l&7, i.e. chunk (l&7) ^ (l>>3).
  const int crow = lane >> 3, cchunk = (lane & 7) ^ crow;
  const char* src[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = 8 * (NWV * i + wave) + crow;
    if (i < NIA) {
      const int plane = row / BM;  // 0: hi, 1: lo
      int m = bm * BM + (row - plane * BM);
      m = m < a.M ? m : a.M - 1;
      src[i] = reinterpret_cast<const char*>(a.ptr[0] + (size_t)a.row(m) * a.lda + plane * a.lo_off) + cchunk * 16;
    } else {
      // the 16-row group of these 8 rows is wave-uniform (AR is a multiple of 16)
      const int wr = row - AR;
      const int gi = ngroups_tile0 + ((NWV * i + wave) * 8 - AR) / 16;
      const T* g = gi < w.ngroups ? w.row(w.feature_of_group(gi), K) : w.ptr[0];
      src[i] = reinterpret_cast<const char*>(g + (size_t)(wr & 15) * K) + cchunk * 16;
    }
  }
  // Activation segment base offset for stage st (segments are stage-aligned).
  const int st_per_seg = a.kseg / BKE;
  auto a_off = [&](int st) -> long {
    if (a.nk == 1) return (long)st * 128;
    const int seg = st / st_per_seg;
    return (long)(reinterpret_cast<const char*>(a.ptr[seg]) - reinterpret_cast<const char*>(a.ptr[0])) +
           (long)(st - seg * st_per_seg) * 128;
  };
  auto issue = [&](int st, int buf) {
    char* base = lds + buf * SBYTES + wave * 1024;
    const long ao = a_off(st);
    const long wo = (long)st * 128;
    if (sk.wstream) {  // one uniform branch per stage, each copy sequence unrolled
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i < NIA)
          dma16(src[i] + ao, base + i * NWV * 1024);
        else
          dma16<true>(src[i] + wo, base + i * NWV * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(src[i] + (i < NIA ? ao : wo), base + i * NWV * 1024);
    }
  };

  // Fragment read offsets within a stage: row r16 of a 16-row block, chunk kk*4+kg.
  int offk[KPS];
#pragma unroll
  for (int kk = 0; kk < KPS; ++kk) offk[kk] = r16 * 128 + (((kk * 4 + kg) ^ (r16 & 7)) << 4);

#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nst) issue(st0 + p, p);

  // Sum of squares of this thread's row of the folded RMSNorm (TPR threads
  // per row, slots in a fixed order), read while the first stages are in
  // flight, the loads four at a time: as a dependent loop after the stream
  // it cost one memory round trip per 16-byte load at the end of every
  // work-group.  The scale goes to LDS after the stream.
  constexpr int NT = 64 * NWV;
  // threads per row: the largest power of two with TPR * BM <= NT (at least 1)
  constexpr int TPR = NT >= 8 * BM ? 8 : NT >= 4 * BM ? 4 : NT >= 2 * BM ? 2 : 1;
  static_assert(NT / TPR >= BM, "one row per thread group");
  const int srow_row = tid / TPR, srow_sub = tid % TPR;
  float ssum = 0.f;
  if (nrm.ssq) {
    const int m = bm * BM + (srow_row < BM ? srow_row : 0);
    const float* p = nrm.ssq + (size_t)a.row(m < a.M ? m : a.M - 1) * nrm.nslot;
    for (int j0 = srow_sub * 4; j0 < nrm.nslot; j0 += TPR * 4 * 4) {
      f32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * TPR * 4;
        v[u] = j < nrm.nslot ? *reinterpret_cast<const f32x4_t*>(p + j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u * TPR * 4 < nrm.nslot) ssum += (v[u][0] + v[u][1]) + (v[u][2] + v[u][3]);
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) ssum += __shfl_xor(ssum, o);
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int buf = 0;
  for (int k = 0; k < nst; ++k) {
    // Own copies of stage k done (younger stages may stay in flight), then
    // everyone's, and everyone is past stage k-1, whose buffer is refilled next.
    const int younger = min(NBUF - 2, nst - 1 - k);
    if constexpr (NBUF >= 4) {
      if (younger >= 2) wait_vmcnt<2 * NI>();
      else if (younger == 1) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
    } else if constexpr (NBUF == 3) {
      if (younger >= 1) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    ring_barrier();
    if (k + NBUF - 1 < nst) {
      int nb = buf + NBUF - 1;
      nb = nb >= NBUF ? nb - NBUF : nb;
      issue(st0 + k + NBUF - 1, nb);
    }
    const char* b = lds + buf * SBYTES;
#pragma unroll
    for (int kk = 0; kk < KPS; ++kk) {
      uint4 af[FM], al[FM], wf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * FM * 16 + i * 16;
        af[i] = *reinterpret_cast<const uint4*>(b + row * 128 + offk[kk]);
        if constexpr (ALO) al[i] = *reinterpret_cast<const uint4*>(b + (BM + row) * 128 + offk[kk]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wf[j] = *reinterpret_cast<const uint4*>(b + (AR + wn * FN * 16 + j * 16) * 128 + offk[kk]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = MM::step(wf[j], af[i], acc[i][j]);
          if constexpr (ALO) acc[i][j] = MM::step(wf[j], al[i], acc[i][j]);
        }
    }
    if constexpr (std::is_same<T, bf16_t>::value && !ALO && KPS == 2) {
      // Instruction order for the stage: the first k-step's fragment reads,
      // then the second k-step's reads spread between the first k-step's
      // MFMAs (so the LDS works while the matrix cores do), then the rest.
      // Left to itself the compiler waits on each small batch of reads
      // right before the MFMAs that use it.
      constexpr int R = FM + FN, MK = FM * FN, Q = MK / R > 0 ? MK / R : 1;
      constexpr int REST = MK - Q * R > 0 ? MK - Q * R : 0;
      __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < R; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, Q, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MK, 0);
    }
    buf = buf + 1 == NBUF ? 0 : buf + 1;
  }

  if (sk.SK > 1) {
    // Partials are written with agent-scope relaxed stores (coherent across
    // XCDs, no dirty L2 lines), completed (vmcnt) before the ticket is taken;
    // the last arriver reads the other splits with agent-scope loads.
    const int tile = bn * MT + bm;
    constexpr int WTILE = FM * FN * 256;  // floats per wave
    float* pt = sk.part + (size_t)tile * sk.SK * (NWV * WTILE) + wave * WTILE;
    {
      float* ps = pt + (size_t)s * (NWV * WTILE);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            __hip_atomic_store(ps + (i * FN + j) * 256 + c * 64 + lane, acc[i][j][c], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();
    __syncthreads();
    int* ticket = reinterpret_cast<int*>(lds);
    if (tid == 0) *ticket = __hip_atomic_fetch_add(sk.ctr + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*ticket != sk.SK - 1) return;
    if (sk.SK == 2) {
      // two splits: own + other is the same sum whichever arrived last
      // (addition commutes), so only the other split's partial is read
      const float* px = pt + (size_t)(1 - s) * (NWV * WTILE);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[i][j][c] += __hip_atomic_load(px + (i * FN + j) * 256 + c * 64 + lane, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // the sum runs over every split in index order (the own partial is read
      // back too), so the result does not depend on which split arrived last
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int x = 0; x < sk.SK; ++x) {
        const float* px = pt + (size_t)x * (NWV * WTILE);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              acc[i][j][c] += __hip_atomic_load(px + (i * FN + j) * 256 + c * 64 + lane, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (tid == 0) __hip_atomic_store(sk.ctr + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Row scales of the folded RMSNorm, once per work-group: the sums of
  // squares reduced before the stream become the BM rows' scales in LDS (the
  // ring is idle after the stream; a barrier first lets every wave finish
  // its last fragment reads).  Every wave of the work-group then reads its
  // rows' scales from LDS instead of re-reducing the slots per fragment.
  float* srow = reinterpret_cast<float*>(lds + 256);
  if (nrm.ssq) {
    __syncthreads();
    if (srow_sub == 0 && srow_row < BM) srow[srow_row] = 1.0f / sqrtf(ssum * nrm.inv_d + nrm.eps);
    __syncthreads();
  }

  const int g0 = ngroups_tile0 + wn * FN;
  int fb[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[j] = g0 + j < w.ngroups ? w.feature_of_group(g0 + j) : 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int lrow = wm * FM * 16 + i * 16 + r16;
    const int m = bm * BM + lrow;
    const float sc = nrm.ssq ? srow[lrow] : 1.0f;
    run_epilogue<FN>(epi, m, m < a.M, w.ngroups - g0, fb, acc[i], sc, kg);
  }
}

}  // namespace dfl
