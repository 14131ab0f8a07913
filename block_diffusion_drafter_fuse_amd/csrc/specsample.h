// Speculative sampling at temperature T > 0 over fp32 logit rows
// ("DFlash 2：正确 token 已在候选里", introduction and selector section:
// outputs stay lossless through rejection sampling; "DFlash 投机解码", section
// 四: the rejected position is redrawn and the last position gives the bonus
// token).  Draws use blocks of kSsBlock = 16384 ids.  Kernels (grids of
// (vocabulary piece, row) work-groups of 256 threads unless noted):
//
//   ss_draft_mass_kernel     per-piece (max, sum) of l log2(e) / T; the last
//                            work-group of a row merges them into the row's
//                            log-sum-exp and the block masses and picks a
//                            block by inverse CDF
//   ss_stats_kernel          base-2 log-sum-exp of the verifier rows (and of
//                            the drafter rows when the draft call did not hand
//                            them over), then, in the last work-group of a
//                            request, the acceptance scan
//                            r_j q_j(x_j) < p_{j-1}(x_j)
//   ss_resample_mass_kernel  per-piece masses of max(0, p - q) on the rejected
//                            offset and of the verifier row; the last
//                            work-group of a request picks the weights and a
//                            block
//   ss_pick_kernel           Gumbel-max over the chosen block's ids, eight
//                            work-groups per draw (the drafted token, or the
//                            replacement / bonus token)
//
// The two-stage draw is exact: P(block b) = mass_b / S and P(v | b) =
// w_v / mass_b.  Only the chosen block needs generator output (one Philox
// block per 8 ids), so the draws stream the logits at HBM speed.
//
// Per-chunk partials go to the workspace with agent-scope stores (coherent
// across XCDs); the last work-group of a row (ticket) combines them in chunk
// order, so results do not depend on arrival order.  Tickets are returned to
// zero by the work-group that takes the last one.
//
// Random numbers: Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), key (seed, stream),
// counter (v / 8, row, request, 0); entry v uses the top 24 bits k of 32-bit
// half (v % 2 == 0: high) of word (v % 8) / 2, as the uniform (k + 0.5) 2^-24.
// Streams: 0 drafting noise (row = offset - 1, index = token id), 1 acceptance
// (index offset - 1), 2 replacement / bonus noise (index = token id), 3 and 4
// the block choice of drafting (row = offset - 1) and of the replacement /
// bonus (row 0), index 0.
#pragma once
#include "common.h"
#include "gemm_tiled.h"

namespace dfl {

constexpr int kSsThreads = 256;
constexpr int kSsPer = 64;                    // entries per thread of the statistics pass
constexpr int kSsBlock = kSsThreads * kSsPer;  // ids per sampling block (and per statistics work-group)
constexpr int kSsPickParts = kSsBlock / (kSsThreads * 8);  // work-groups of a block draw, 8 ids per thread
constexpr int kSsMaxBlocks = 64;              // block masses are scanned by one wave
constexpr int kSsStreamDraft = 0, kSsStreamAccept = 1, kSsStreamResample = 2;
constexpr int kSsStreamDraftBlock = 3, kSsStreamResampleBlock = 4;

struct SsWork {
  float4* part;  // [rows][npiece] per-piece partials
  float* lse;    // [n_req][2K+1] base-2 log-sum-exp of l log2(e) / T: K drafter rows, then K+1 verifier rows
  int* nacc;     // [n_req] accepted drafts
  int* row_ctr;  // [rows] tickets
  int* req_ctr;  // [n_req] tickets
  int* blk;      // [rows] chosen block of a draw; the replacement draw adds 64 when it samples the residual
};

// hi/lo 64-bit halves of the 128-bit product m * c, from four 32 x 32 -> 64
// multiply-adds (no partial sum overflows 64 bits).
__device__ __forceinline__ void ss_mulhilo64(uint64_t m, uint64_t c, uint64_t& hi, uint64_t& lo) {
  const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32), cl = (uint32_t)c, ch = (uint32_t)(c >> 32);
  const uint64_t p0 = (uint64_t)ml * cl;
  const uint64_t t = (uint64_t)ml * ch + (p0 >> 32);
  const uint64_t u = (uint64_t)mh * cl + (uint32_t)t;
  hi = (uint64_t)mh * ch + (t >> 32) + (u >> 32);
  lo = (uint32_t)p0 | (u << 32);
}

// Philox4x64-10 in place on counter c with key (k0, k1).  Each round takes
// the 128-bit products of words 0 and 2 with the two round multipliers; the
// new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)); the key then advances by the two Weyl constants.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    ss_mulhilo64(M0, c[0], hi0, lo0);
    ss_mulhilo64(M1, c[2], hi1, lo1);
    c[0] = hi1 ^ c[1] ^ k0;
    c[1] = lo1;
    c[2] = hi0 ^ c[3] ^ k1;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// 24-bit draw of entry e (0..7) of a generator block.
__device__ __forceinline__ uint32_t ss_bits(const uint64_t c[4], int e) {
  const uint64_t w = c[e >> 1];
  return (uint32_t)((e & 1) ? w : (w >> 32)) >> 8;
}

// log2 of the exponential draw E = -ln(u), u = (k + 0.5) 2^-24, up to an
// additive constant: returns log2(-log2(u)).  A Gumbel draw is G = -ln(E), so
// ln 2 * (z log2(e) - ss_log2_exp(k)) = z + G - ln(ln 2): keys in base 2 rank
// exactly as l / T + G.  Where 1 - u = e' < 2^-7, u itself is not
// representable in fp32, and -log2(u) comes from the series
// e' (1 + e'/2 + e'^2/3 + e'^3/4) log2(e) with e' exact (relative error below
// 1e-7); elsewhere from the hardware log2 of u (rounded by at most 2^-25
// against 1 - u >= 2^-7: relative error below 4e-6).
__device__ __forceinline__ float ss_log2_exp(uint32_t k) {
  const float u = (float)(2u * k + 1u) * 0x1p-25f;
  const float e = (float)((1u << 25) - 2u * k - 1u) * 0x1p-25f;
  const float ser = e * fmaf(e, fmaf(e, fmaf(e, 0.25f, 0.33333334f), 0.5f), 1.0f) * 1.4426950408889634f;
  const float nl = e < 0x1p-7f ? ser : -__builtin_amdgcn_logf(u);
  return __builtin_amdgcn_logf(nl);
}

// Uniform in (0, 1) as an exact double (the acceptance test runs in double so
// that u < 1 holds strictly).
__device__ __forceinline__ double ss_uniform(uint32_t k) { return ((double)k + 0.5) * 0x1p-24; }

// (value, id) order of a Gumbel-max: larger value, ties to the lower id.
__device__ __forceinline__ bool ss_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Eight consecutive entries v0..v0+7 of a row (v0 % 8 == 0); entries at or
// past V read as -inf.  VEC: the row is 16-byte aligned and V % 4 == 0.
template <bool VEC>
__device__ __forceinline__ void ss_load8(const float* row, int v0, int V, float l[8]) {
  if (VEC) {
    const float4 a = *reinterpret_cast<const float4*>(row + v0);
    const float4 b = v0 + 4 < V ? *reinterpret_cast<const float4*>(row + v0 + 4)
                                : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    l[0] = a.x; l[1] = a.y; l[2] = a.z; l[3] = a.w;
    l[4] = b.x; l[5] = b.y; l[6] = b.z; l[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) l[e] = v0 + e < V ? row[v0 + e] : -INFINITY;
  }
}

__device__ __forceinline__ void ss_wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    if (ss_better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// (max, sum 2^(z - max)) pairs: merge b into a.
__device__ __forceinline__ void ss_lse_merge(float& m, float& s, float om, float os) {
  const float M = fmaxf(m, om);
  const float a = s > 0.f ? s * exp2f(m - M) : 0.f;
  const float b = os > 0.f ? os * exp2f(om - M) : 0.f;
  m = M;
  s = a + b;
}

__device__ __forceinline__ void ss_wave_lse(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss_lse_merge(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
}

// Store this work-group's partial for (row, chunk) from thread 0 and take the
// row's ticket; true in every thread of the work-group that arrives last.
__device__ __forceinline__ bool ss_publish(SsWork w, int row, int chunk, int nchunk, float4 val, int* ctr) {
  __shared__ int tk;
  if (threadIdx.x == 0) {
    float* p = reinterpret_cast<float*>(w.part + (size_t)row * nchunk + chunk);
    __hip_atomic_store(p + 0, val.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, val.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 2, val.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 3, val.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    tk = __hip_atomic_fetch_add(ctr + row, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return tk == nchunk - 1;
}

__device__ __forceinline__ float4 ss_load_part(const SsWork& w, int row, int chunk, int nchunk) {
  const float* p = reinterpret_cast<const float*>(w.part + (size_t)row * nchunk + chunk);
  return make_float4(__hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Work-group (max, sum) merge of the lse pairs; result valid in thread 0.
__device__ __forceinline__ void ss_block_lse(float& m, float& s) {
  __shared__ float sm[kSsThreads / 64], ss[kSsThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  ss_wave_lse(m, s);
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int x = 1; x < kSsThreads / 64; ++x) ss_lse_merge(m, s, sm[x], ss[x]);
}

// Loads the PER entries of this thread (PER a multiple of 8; 8-entry groups, ids
// chunk * 256 * PER + (it * 256 + thread) * 8 + e) scaled by s2 = log2(e) / T,
// and their maximum.  Entries at or past V are -inf.
template <bool VEC, int PER>
__device__ __forceinline__ float ss_load_row(const float* lr, int chunk, int V, float s2, float z[PER]) {
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < PER / 8; ++it) {
    const int v0 = chunk * (kSsThreads * PER) + (it * kSsThreads + (int)threadIdx.x) * 8;
    float l[8];
    if (v0 < V) {
      ss_load8<VEC>(lr, v0, V, l);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) l[e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      z[it * 8 + e] = l[e] * s2;
      m = fmaxf(m, z[it * 8 + e]);
    }
  }
  return m;
}

// sum 2^(z - m) over the thread's entries (0 when every entry is -inf).
template <int PER>
__device__ __forceinline__ float ss_sum_exp2(const float z[PER], float m) {
  float s = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int e = 0; e < PER; ++e) s += __builtin_amdgcn_exp2f(z[e] - m);
  }
  return s;
}

// Inverse CDF over block masses held one per lane of a wave (lanes past the
// last block hold 0): the first block whose inclusive prefix exceeds u times
// the total, never an empty block (should rounding leave no prefix above the
// target, the last block with mass).  All 64 lanes call it; the result is the
// same in every lane.
__device__ __forceinline__ int ss_choose_block(float mass, double u) {
  const int lane = threadIdx.x & 63;
  float cum = mass;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(cum, o);
    if (lane >= o) cum += t;
  }
  const float target = (float)(u * (double)__shfl(cum, 63));
  const unsigned long long over = __ballot(cum > target && mass > 0.f);
  if (over) return __ffsll(over) - 1;
  const unsigned long long pos = __ballot(mass > 0.f);
  return pos ? 63 - __clzll(pos) : 0;
}

// Work-group sums of two values; result valid in thread 0.
__device__ __forceinline__ void ss_block_sum2(float& a, float& b) {
  __shared__ float sa[kSsThreads / 64], sb[kSsThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane == 0) {
    sa[wave] = a;
    sb[wave] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int x = 1; x < kSsThreads / 64; ++x) {
      a += sa[x];
      b += sb[x];
    }
}

// Drafting, first pass.  Grid (npiece, n_req * K), pieces of 256 * PER ids;
// row = r * K + (offset - 1) of logits [n_req][K][V].  The last work-group of
// a row stores the chosen block in blk[row] and, when dlse is given, the
// row's base-2 log-sum-exp of l log2(e) / T (for the verifier).
template <bool VEC, int PER>
__global__ void __launch_bounds__(kSsThreads)
    ss_draft_mass_kernel(const float* __restrict__ logits, int V, int K, int npiece, float s2, uint64_t seed,
                         const int* __restrict__ req_id, SsWork w, float* __restrict__ dlse) {
  static_assert(PER % 8 == 0 && kSsBlock % (kSsThreads * PER) == 0, "whole 8-entry groups, whole pieces per block");
  constexpr int PPB = kSsBlock / (kSsThreads * PER);  // pieces per block
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int r = row / K, off = row - r * K;
  {
    float z[PER];
    float m = ss_load_row<VEC, PER>(logits + (size_t)row * V, chunk, V, s2, z);
    float s = ss_sum_exp2<PER>(z, m);
    ss_block_lse(m, s);
    if (!ss_publish(w, row, chunk, npiece, make_float4(m, s, 0.f, 0.f), w.row_ctr)) return;
  }
  if (threadIdx.x >= 64) return;
  // wave 0 of the last work-group: lane b merges the pieces of block b in
  // piece order, then the block by inverse CDF over the masses
  const int lane = threadIdx.x;
  float bm = -INFINITY, bs = 0.f;
  for (int x = lane * PPB; x < min(npiece, (lane + 1) * PPB); ++x) {
    const float4 q = ss_load_part(w, row, x, npiece);
    ss_lse_merge(bm, bs, q.x, q.y);
  }
  float M = bm, S = bs;
  ss_wave_lse(M, S);  // the same totals in every lane
  const float mass = bs > 0.f ? bs * exp2f(bm - M) : 0.f;
  uint64_t c[4] = {0, (uint64_t)off, (uint64_t)(uint32_t)req_id[r], 0};
  philox4x64_10(c, seed, kSsStreamDraftBlock);
  const int b = ss_choose_block(mass, ss_uniform(ss_bits(c, 0)));
  if (lane == 0) {
    w.blk[row] = b;
    if (dlse) dlse[row] = M + log2f(S);
    __hip_atomic_store(w.row_ctr + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Log-sum-exp of the rows, then the acceptance scan.  With dlse == nullptr
// the grid is (nchunk, n_req * (2K + 1)) and row k of request r is drafter row
// k (offset k + 1) for k < K, verifier row k - K otherwise; with dlse (the
// drafter rows' values from ss_draft_kernel) the grid is (nchunk,
// n_req * (K + 1)) over the verifier rows alone.  s2 = log2(e) / T.
template <bool VEC>
__global__ void __launch_bounds__(kSsThreads)
    ss_stats_kernel(const float* __restrict__ draft, const float* __restrict__ target, const int* __restrict__ cand,
                    const float* __restrict__ dlse, int V, int K, int nchunk, float s2, uint64_t seed,
                    const int* __restrict__ req_id, SsWork w, int* __restrict__ tokens) {
  const int chunk = blockIdx.x, y = blockIdx.y;
  const int R = 2 * K + 1;
  const int RA = dlse ? K + 1 : R;  // rows of a request in this grid
  const int r = y / RA, k = (dlse ? K : 0) + (y - r * RA);  // k: row of the request in 0..2K
  const float* lr = k < K ? draft + ((size_t)r * K + k) * V : target + ((size_t)r * (K + 1) + (k - K)) * V;
  float z[kSsPer];
  float m = ss_load_row<VEC, kSsPer>(lr, chunk, V, s2, z);
  float s = ss_sum_exp2<kSsPer>(z, m);
  ss_block_lse(m, s);
  if (!ss_publish(w, y, chunk, nchunk, make_float4(m, s, 0.f, 0.f), w.row_ctr)) return;
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  // wave 0: merge the row's partials in chunk order
  m = -INFINITY;
  s = 0.f;
  for (int x = lane; x < nchunk; x += 64) {
    const float4 q = ss_load_part(w, y, x, nchunk);
    ss_lse_merge(m, s, q.x, q.y);
  }
  ss_wave_lse(m, s);
  int t = 0;
  if (lane == 0) {
    __hip_atomic_store(w.lse + (size_t)r * R + k, m + log2f(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w.row_ctr + y, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    t = __hip_atomic_fetch_add(w.req_ctr + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  t = __shfl(t, 0);
  if (t != RA - 1) return;
  // last row of request r: lane j < K tests offset j + 1; the accepted count
  // is the number of leading passes
  const uint64_t req = (uint64_t)(uint32_t)req_id[r];
  const float* lse = w.lse + (size_t)r * R;
  int x = -1;
  bool ok = false;
  if (lane < K) {
    x = cand[(size_t)r * K + lane];
    if (x >= 0 && x < V) {  // an id outside the vocabulary is rejected
      uint64_t c[4] = {(uint64_t)(lane >> 3), 0, req, 0};
      philox4x64_10(c, seed, kSsStreamAccept);
      const float ld = draft[((size_t)r * K + lane) * V + x];
      const float lt = target[((size_t)r * (K + 1) + lane) * V + x];
      const float ld2 = dlse ? dlse[(size_t)r * K + lane]
                             : __hip_atomic_load(lse + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float lt2 = __hip_atomic_load(lse + K + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float q = exp2f(fmaf(ld, s2, -ld2)), p = exp2f(fmaf(lt, s2, -lt2));
      ok = ss_uniform(ss_bits(c, lane & 7)) * (double)q < (double)p;
    }
  }
  const unsigned long long rejected = __ballot(lane < K && !ok);
  const int n = rejected ? __ffsll(rejected) - 1 : K;
  if (lane <= K && lane != n) tokens[(size_t)r * (K + 1) + lane] = lane < n ? x : -1;
  if (lane == 0) {
    w.nacc[r] = n;
    __hip_atomic_store(w.req_ctr + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The emitted token after the scan, first pass.  Grid (npiece, n_req),
// pieces of 256 * PER ids.  With n = nacc[r] < K the weights are
// max(0, p_n - q_{n+1}) (verifier row n, drafter row n); with n = K, or a
// residual that rounding left empty, the verifier row's softmax(l / T).  The
// last work-group of a request stores the chosen block in blk[r] (+ 64 when
// the residual is sampled).
template <bool VEC, int PER>
__global__ void __launch_bounds__(kSsThreads)
    ss_resample_mass_kernel(const float* __restrict__ draft, const float* __restrict__ target,
                            const float* __restrict__ dlse, int V, int K, int npiece, float s2, uint64_t seed,
                            const int* __restrict__ req_id, SsWork w) {
  static_assert(PER % 8 == 0 && kSsBlock % (kSsThreads * PER) == 0, "whole 8-entry groups, whole pieces per block");
  constexpr int PPB = kSsBlock / (kSsThreads * PER);
  const int chunk = blockIdx.x, r = blockIdx.y;
  const int R = 2 * K + 1;
  const int n = min(max(w.nacc[r], 0), K);  // written by ss_stats_kernel, in 0..K
  const bool rej = n < K;
  {
    const float lse_t = w.lse[(size_t)r * R + K + n];
    const float lse_d = rej ? (dlse ? dlse[(size_t)r * K + n] : w.lse[(size_t)r * R + n]) : 0.f;
    float zt[PER], zd[PER];  // all loads issued before the arithmetic
    ss_load_row<VEC, PER>(target + ((size_t)r * (K + 1) + n) * V, chunk, V, s2, zt);
    if (rej) ss_load_row<VEC, PER>(draft + ((size_t)r * K + n) * V, chunk, V, s2, zd);
    float ws = 0.f, ps = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float p = exp2f(zt[e] - lse_t);
      ps += p;
      if (rej) ws += fmaxf(p - exp2f(zd[e] - lse_d), 0.f);
    }
    ss_block_sum2(ws, ps);
    if (!ss_publish(w, r, chunk, npiece, make_float4(ws, ps, 0.f, 0.f), w.req_ctr)) return;
  }
  if (threadIdx.x >= 64) return;
  // wave 0 of the last work-group: lane b sums the pieces of block b in piece order
  const int lane = threadIdx.x;
  float qx = 0.f, qy = 0.f;
  for (int x = lane * PPB; x < min(npiece, (lane + 1) * PPB); ++x) {
    const float4 q = ss_load_part(w, r, x, npiece);
    qx += q.x;
    qy += q.y;
  }
  const bool res = rej && wave_sum(qx) > 0.f;
  uint64_t c[4] = {0, 0, (uint64_t)(uint32_t)req_id[r], 0};
  philox4x64_10(c, seed, kSsStreamResampleBlock);
  const int b = ss_choose_block(res ? qx : qy, ss_uniform(ss_bits(c, 0)));
  if (lane == 0) {
    w.blk[r] = b + (res ? kSsMaxBlocks : 0);
    __hip_atomic_store(w.req_ctr + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Gumbel-max over the chosen block of one draw.  Grid (kSsPickParts, draws):
// work-group x of draw d covers ids 2048 x .. 2048 x + 2047 of the block, 8
// per thread (one Philox block); the last of the draw's work-groups (ticket)
// merges their winners in part order.
//   RESAMPLE = false: draw d = row of the drafter logits; cand[d] = the token.
//   RESAMPLE = true:  draw d = request; the weights of blk[d] (see
//   ss_resample_mass_kernel); tokens[d][n] = the token, tau[d] = n + 1.
template <bool VEC, bool RESAMPLE>
__global__ void __launch_bounds__(kSsThreads)
    ss_pick_kernel(const float* __restrict__ draft, const float* __restrict__ target,
                   const float* __restrict__ dlse, int V, int K, float s2, uint64_t seed,
                   const int* __restrict__ req_id, SsWork w, int* __restrict__ out, int* __restrict__ tau) {
  const int part = blockIdx.x, d = blockIdx.y, tid = threadIdx.x;
  const int R = 2 * K + 1;
  const int code = w.blk[d];
  const int b = code % kSsMaxBlocks;
  const bool res = RESAMPLE && code >= kSsMaxBlocks;
  int n = 0, r = d, off = 0;
  const float* la;  // weights' logits: the drafter row, or the verifier row
  const float* lb = nullptr;
  float lse_t = 0.f, lse_d = 0.f;
  if constexpr (RESAMPLE) {
    n = min(max(w.nacc[d], 0), K);
    la = target + ((size_t)d * (K + 1) + n) * V;
    if (res) {
      lb = draft + ((size_t)d * K + n) * V;
      lse_t = w.lse[(size_t)d * R + K + n];
      lse_d = dlse ? dlse[(size_t)d * K + n] : w.lse[(size_t)d * R + n];
    }
  } else {
    r = d / K;
    off = d - r * K;
    la = draft + (size_t)d * V;
  }
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const int v0 = b * kSsBlock + part * (kSsThreads * 8) + tid * 8;
  if (v0 < V) {
    float za[8], zb[8];
    ss_load8<VEC>(la, v0, V, za);
    if (res) ss_load8<VEC>(lb, v0, V, zb);
    uint64_t c[4] = {(uint64_t)(v0 >> 3), (uint64_t)off, (uint64_t)(uint32_t)req_id[r], 0};
    philox4x64_10(c, seed, RESAMPLE ? kSsStreamResample : kSsStreamDraft);
    // ids rise within a thread, so a strict > keeps the lowest id of a tie;
    // entries past V hold -inf and never win
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = ss_log2_exp(ss_bits(c, e));
      float key;
      if (res) {
        const float dd = exp2f(fmaf(za[e], s2, -lse_t)) - exp2f(fmaf(zb[e], s2, -lse_d));
        key = dd > 0.f ? __builtin_amdgcn_logf(dd) - g : -INFINITY;
      } else {
        key = fmaf(za[e], s2, -g);
      }
      if (key > bv) {
        bv = key;
        bi = v0 + e;
      }
    }
  }
  __shared__ float sv[kSsThreads / 64];
  __shared__ int si[kSsThreads / 64];
  ss_wave_argmax(bv, bi);
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0)
    for (int x = 1; x < kSsThreads / 64; ++x)
      if (ss_better(sv[x], si[x], bv, bi)) {
        bv = sv[x];
        bi = si[x];
      }
  int* ctr = RESAMPLE ? w.req_ctr : w.row_ctr;
  if (!ss_publish(w, d, part, kSsPickParts, make_float4(bv, __int_as_float(bi), 0.f, 0.f), ctr)) return;
  if (tid >= 64) return;
  // wave 0 of the last work-group: merge the parts in part order
  bv = -INFINITY;
  bi = 0x7fffffff;
  if (tid < kSsPickParts) {
    const float4 q = ss_load_part(w, d, tid, kSsPickParts);
    bv = q.x;
    bi = __float_as_int(q.y);
  }
  ss_wave_argmax(bv, bi);
  if (tid == 0) {
    const int tok = bv > -INFINITY ? bi : b * kSsBlock;  // no finite key: the block's first id
    if constexpr (RESAMPLE) {
      out[(size_t)d * (K + 1) + n] = tok;
      tau[d] = n + 1;
    } else {
      out[d] = tok;
    }
    __hip_atomic_store(ctr + d, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace dfl
