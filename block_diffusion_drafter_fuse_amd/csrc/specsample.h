// Speculative sampling at temperature T > 0 over fp32 logit rows
// ("DFlash 2：正确 token 已在候选里", introduction and selector section:
// outputs stay lossless through rejection sampling; "DFlash 投机解码", section
// 四: the rejected position is redrawn and the last position gives the bonus
// token).  Three HBM-streaming kernels, each a grid of (vocabulary chunk, row)
// work-groups of 256 threads over 4096 entries:
//
//   ss_draft_kernel     x_j = argmax_v (l_j[v] / T + G_v): Gumbel-max drafting
//   ss_stats_kernel     base-2 log-sum-exp of every drafter and verifier row,
//                       then, in the last work-group of a request, the
//                       acceptance scan r_j q_j(x_j) < p_{j-1}(x_j)
//   ss_resample_kernel  the emitted token after the scan: Gumbel-max over
//                       log max(0, p - q) on the rejected offset, or over the
//                       verifier's last row when every draft was kept
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
// Streams: 0 drafting (row = offset - 1), 1 acceptance (index offset - 1),
// 2 replacement / bonus (index = token id).
#pragma once
#include "common.h"
#include "gemm_tiled.h"

namespace dfl {

constexpr int kSsThreads = 256;
// Vocabulary entries per thread (work-group: 256 times that), measured best
// at 1 and 32 requests of a 151,936-entry vocabulary: drafting (bound by the
// generator's integer arithmetic) 32, row statistics (bound by HBM) 64, the
// replacement draw (one or two rows per request) 8 up to four requests and 16
// beyond.
constexpr int kSsPerDraft = 32;
constexpr int kSsPerStats = 64;
constexpr int kSsPerResampleFew = 8;
constexpr int kSsPerResample = 16;
constexpr int kSsStreamDraft = 0, kSsStreamAccept = 1, kSsStreamResample = 2;

struct SsWork {
  float4* part;  // [rows][nchunk] per-chunk partials
  float* lse;    // [n_req][2K+1] base-2 log-sum-exp of l log2(e) / T: K drafter rows, then K+1 verifier rows
  int* nacc;     // [n_req] accepted drafts
  int* row_ctr;  // [rows] tickets
  int* req_ctr;  // [n_req] tickets
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

// Work-group argmax of (v, i) pairs (x and y of the float4: value, id bits)
// and optionally a second pair (z, w); result valid in thread 0.
template <int NPAIR>
__device__ __forceinline__ void ss_block_argmax(float v[NPAIR], int i[NPAIR]) {
  __shared__ float sv[NPAIR][kSsThreads / 64];
  __shared__ int si[NPAIR][kSsThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    ss_wave_argmax(v[p], i[p]);
    if (lane == 0) {
      sv[p][wave] = v[p];
      si[p][wave] = i[p];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int p = 0; p < NPAIR; ++p)
      for (int x = 1; x < kSsThreads / 64; ++x)
        if (ss_better(sv[p][x], si[p][x], v[p], i[p])) {
          v[p] = sv[p][x];
          i[p] = si[p][x];
        }
  }
}

// Wave 0 merges the nchunk argmax partials of `row` in chunk order; the
// result is valid in lane 0 of wave 0.  NPAIR pairs per partial.
template <int NPAIR>
__device__ __forceinline__ void ss_merge_argmax(const SsWork& w, int row, int nchunk, float v[NPAIR], int i[NPAIR]) {
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    v[p] = -INFINITY;
    i[p] = 0x7fffffff;
  }
  if (threadIdx.x >= 64) return;
  for (int x = threadIdx.x; x < nchunk; x += 64) {
    const float4 q = ss_load_part(w, row, x, nchunk);
    const float qv[2] = {q.x, q.z};
    const int qi[2] = {__float_as_int(q.y), __float_as_int(q.w)};
#pragma unroll
    for (int p = 0; p < NPAIR; ++p)
      if (ss_better(qv[p], qi[p], v[p], i[p])) {
        v[p] = qv[p];
        i[p] = qi[p];
      }
  }
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) ss_wave_argmax(v[p], i[p]);
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

// Loads the PER entries of this thread (in 8-entry groups, ids
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

// Gumbel-max drafting.  Grid (nchunk, n_req * K); row = r * K + (offset - 1)
// of logits [n_req][K][V]; cand[row] = the drafted token.  The pass also
// yields the row's base-2 log-sum-exp, written to dlse[row] when dlse is
// given (the verifier then need not read the drafter rows again for it).
template <bool VEC, int PER>
__global__ void __launch_bounds__(kSsThreads)
    ss_draft_kernel(const float* __restrict__ logits, int V, int K, int nchunk, float s2, uint64_t seed,
                    const int* __restrict__ req_id, SsWork w, int* __restrict__ cand, float* __restrict__ dlse) {
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int r = row / K, off = row - r * K;
  const uint64_t req = (uint64_t)(uint32_t)req_id[r];
  float z[PER];
  float m = ss_load_row<VEC, PER>(logits + (size_t)row * V, chunk, V, s2, z);
  float bv[1] = {-INFINITY};
  int bi[1] = {0x7fffffff};
  // ids rise within a thread, so a strict > keeps the lowest id of a tie;
  // entries past V hold -inf and never win
#pragma unroll
  for (int it = 0; it < PER / 8; ++it) {
    const int v0 = chunk * (kSsThreads * PER) + (it * kSsThreads + (int)threadIdx.x) * 8;
    if (v0 < V) {
      uint64_t c[4] = {(uint64_t)(v0 >> 3), (uint64_t)off, req, 0};
      philox4x64_10(c, seed, kSsStreamDraft);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float key = z[it * 8 + e] - ss_log2_exp(ss_bits(c, e));
        if (key > bv[0]) {
          bv[0] = key;
          bi[0] = v0 + e;
        }
      }
    }
  }
  float s = ss_sum_exp2<PER>(z, m);
  ss_block_argmax<1>(bv, bi);
  ss_block_lse(m, s);
  if (!ss_publish(w, row, chunk, nchunk, make_float4(bv[0], __int_as_float(bi[0]), m, s), w.row_ctr)) return;
  if (threadIdx.x >= 64) return;
  // wave 0: merge the row's partials in chunk order
  bv[0] = -INFINITY;
  bi[0] = 0x7fffffff;
  m = -INFINITY;
  s = 0.f;
  for (int x = threadIdx.x; x < nchunk; x += 64) {
    const float4 q = ss_load_part(w, row, x, nchunk);
    if (ss_better(q.x, __float_as_int(q.y), bv[0], bi[0])) {
      bv[0] = q.x;
      bi[0] = __float_as_int(q.y);
    }
    ss_lse_merge(m, s, q.z, q.w);
  }
  ss_wave_argmax(bv[0], bi[0]);
  ss_wave_lse(m, s);
  if (threadIdx.x == 0) {
    cand[row] = bv[0] > -INFINITY ? bi[0] : 0;  // a row without a finite logit: id 0
    if (dlse) dlse[row] = m + log2f(s);
    __hip_atomic_store(w.row_ctr + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Log-sum-exp of the rows, then the acceptance scan.  With dlse == nullptr
// the grid is (nchunk, n_req * (2K + 1)) and row k of request r is drafter row
// k (offset k + 1) for k < K, verifier row k - K otherwise; with dlse (the
// drafter rows' values from ss_draft_kernel) the grid is (nchunk,
// n_req * (K + 1)) over the verifier rows alone.  s2 = log2(e) / T.
template <bool VEC, int PER>
__global__ void __launch_bounds__(kSsThreads)
    ss_stats_kernel(const float* __restrict__ draft, const float* __restrict__ target, const int* __restrict__ cand,
                    const float* __restrict__ dlse, int V, int K, int nchunk, float s2, uint64_t seed,
                    const int* __restrict__ req_id, SsWork w, int* __restrict__ tokens) {
  const int chunk = blockIdx.x, y = blockIdx.y;
  const int R = 2 * K + 1;
  const int RA = dlse ? K + 1 : R;  // rows of a request in this grid
  const int r = y / RA, k = (dlse ? K : 0) + (y - r * RA);  // k: row of the request in 0..2K
  const float* lr = k < K ? draft + ((size_t)r * K + k) * V : target + ((size_t)r * (K + 1) + (k - K)) * V;
  float z[PER];
  float m = ss_load_row<VEC, PER>(lr, chunk, V, s2, z);
  float s = ss_sum_exp2<PER>(z, m);
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

// The emitted token after the scan.  Grid (nchunk, n_req).  With n = nacc[r]
// < K: Gumbel-max over log max(0, p_n - q_{n+1}) (verifier row n, drafter row
// n); with n = K, or a residual that rounding left empty: Gumbel-max over the
// verifier row's l / T.  tokens[r][n] = that token, tau[r] = n + 1.
template <bool VEC, int PER>
__global__ void __launch_bounds__(kSsThreads)
    ss_resample_kernel(const float* __restrict__ draft, const float* __restrict__ target,
                       const float* __restrict__ dlse, int V, int K, int nchunk, float s2, uint64_t seed,
                       const int* __restrict__ req_id, SsWork w, int* __restrict__ tokens, int* __restrict__ tau) {
  const int chunk = blockIdx.x, r = blockIdx.y;
  const int R = 2 * K + 1;
  const int n = min(max(w.nacc[r], 0), K);  // written by ss_stats_kernel, in 0..K
  const bool rej = n < K;
  const uint64_t req = (uint64_t)(uint32_t)req_id[r];
  const float* lt = target + ((size_t)r * (K + 1) + n) * V;
  const float* ld = draft + ((size_t)r * K + (rej ? n : 0)) * V;
  const float lse_t = w.lse[(size_t)r * R + K + n];
  const float lse_d = rej ? (dlse ? dlse[(size_t)r * K + n] : w.lse[(size_t)r * R + n]) : 0.f;
  // pair 0: residual, pair 1: verifier row
  float bv[2] = {-INFINITY, -INFINITY};
  int bi[2] = {0x7fffffff, 0x7fffffff};
#pragma unroll
  for (int it = 0; it < PER / 8; ++it) {
    const int v0 = chunk * (kSsThreads * PER) + (it * kSsThreads + (int)threadIdx.x) * 8;
    if (v0 >= V) break;
    float a[8], b[8];
    ss_load8<VEC>(lt, v0, V, a);
    if (rej) ss_load8<VEC>(ld, v0, V, b);
    uint64_t c[4] = {(uint64_t)(v0 >> 3), 0, req, 0};
    philox4x64_10(c, seed, kSsStreamResample);
    // base-2 keys (see ss_log2_exp); ids rise within a thread, so strict >
    // keeps the lowest id of a tie; entries past V hold -inf and never win
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = ss_log2_exp(ss_bits(c, e));
      const float tk = fmaf(a[e], s2, -g);
      if (tk > bv[1]) {
        bv[1] = tk;
        bi[1] = v0 + e;
      }
      if (rej) {
        const float d = exp2f(fmaf(a[e], s2, -lse_t)) - exp2f(fmaf(b[e], s2, -lse_d));
        const float rk = d > 0.f ? __builtin_amdgcn_logf(d) - g : -INFINITY;
        if (rk > bv[0]) {
          bv[0] = rk;
          bi[0] = v0 + e;
        }
      }
    }
  }
  ss_block_argmax<2>(bv, bi);
  if (!ss_publish(w, r, chunk, nchunk,
                  make_float4(bv[0], __int_as_float(bi[0]), bv[1], __int_as_float(bi[1])), w.req_ctr))
    return;
  ss_merge_argmax<2>(w, r, nchunk, bv, bi);
  if (threadIdx.x == 0) {
    tokens[(size_t)r * (K + 1) + n] = (rej && bv[0] > -INFINITY) ? bi[0] : (bv[1] > -INFINITY ? bi[1] : 0);
    tau[r] = n + 1;
    __hip_atomic_store(w.req_ctr + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace dfl
