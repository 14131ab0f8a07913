// Host side of the DFlash draft-step library: argument validation, buffer
// carving, launch planning and the C ABI declared in include/dflash_fuse.h.
//
// One launch sequence per call, all on the caller's stream:
//   fuse_ctx:  per row chunk, fusion GEMM (writes T(z*g_c) and row sums of
//              squares) -> context K/V GEMM (RMSNorm scale, RoPE, cache append)
//   draft:     embed (x, T(x*g_attn0), sums of squares), then per layer
//              {QKV GEMM (+norm scale, RoPE), attention + combine,
//               O GEMM (+residual, next norm input), gate/up GEMM (+norm scale,
//               SwiGLU), down GEMM (+residual, next norm input)},
//              LM head with fused top-k (+final norm scale), top-k merge
//   accept:    one scan kernel
// RMSNorm never runs as a separate pass: the producer of a normed operand
// writes x*g and per-64-feature sums of squares, the consumer GEMM scales its
// rows by rsqrt(mean + eps) in the epilogue.
// Per-call request metadata travels in kernel arguments (no host-to-device
// copies), so a call sequence can be captured in a HIP graph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dflash_fuse.h"
#include "attention.h"
#include "common.h"
#include "conv.h"
#include "gemm.h"
#include "gemm_tiled.h"
#include "gemv_stream.h"
#include "lmhead.h"
#include "misc.h"
#include "specsample.h"

using namespace dfl;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

constexpr size_t kAlign = 256;
constexpr int kFuseChunk = 4096;       // rows per fusion launch pair
// Tuning constants of the attention launch (overridable at build time for
// sweeps: -DDFL_ATTN_TARGET_WG=... etc.).
#ifndef DFL_ATTN_TARGET_WG
#define DFL_ATTN_TARGET_WG 480
#endif
#ifndef DFL_ATTN_MIN_CHUNK
#define DFL_ATTN_MIN_CHUNK 128
#endif
#ifndef DFL_ATTN_NBUF
#define DFL_ATTN_NBUF 2
#endif
#ifndef DFL_ATTN_WPE
#define DFL_ATTN_WPE 2
#endif
constexpr int kAttnWorkMax = 4096;     // attention split work items per call
constexpr int kAttnTargetWG = DFL_ATTN_TARGET_WG;  // attention work-groups aimed for
constexpr int kAttnMinChunk = DFL_ATTN_MIN_CHUNK;  // minimum context keys per split
constexpr int kAttnNbuf = DFL_ATTN_NBUF;           // attention K/V ring depth
#ifndef DFL_ATTN_STG
#define DFL_ATTN_STG 64
#endif
#ifndef DFL_ATTN_QW
#define DFL_ATTN_QW 1
#endif
constexpr int kAttnStg = DFL_ATTN_STG;             // attention keys per stage (bf16, head dim 128, G*B 64)
constexpr int kAttnShortSplit = 256;               // splits up to this many keys take 32-key stages
constexpr int kAttnWpe = DFL_ATTN_WPE;             // attention waves per SIMD the registers must allow
constexpr int kAttnQw = DFL_ATTN_QW;   // attention query fragments per wave
constexpr int kSkinnyMaxM = 64;        // rows handled by the skinny GEMM
constexpr int kNarrowMaxGroups = 64;   // weights of at most 1024 rows also take the skinny GEMM
constexpr int kGemvKSW = 8;            // k-steps (activation fragments) per wave in the skinny GEMM
constexpr int kGemvTB = 8;             // skinny GEMM tiles per barrier batch (LDS: TB x waves x 1 KB)
constexpr int kGemvWGs = 256;          // skinny GEMM work-groups per 16-token block
constexpr int kGemvXcds = 8;           // XCDs; work-group i runs on XCD i mod 8
#ifndef DFL_RS_NBUF
#define DFL_RS_NBUF 6
#endif
#ifndef DFL_RS_MAX_SPLIT
#define DFL_RS_MAX_SPLIT 8
#endif
#ifndef DFL_RS_SPLIT_COST
#define DFL_RS_SPLIT_COST 0
#endif
constexpr int kRsNbuf = DFL_RS_NBUF;   // row-streaming GEMV ring depth (stages of 16 KB)
constexpr int kRsMaxSplit = DFL_RS_MAX_SPLIT;  // K ranges of the row-streaming GEMV
constexpr int kRsSplitCost = DFL_RS_SPLIT_COST;  // stage-equivalents charged per extra K range
constexpr int kLmFN = 1, kLmU = 8;     // few-token LM head fragments per wave, unroll
constexpr int kTiledSlots = 256;       // concurrent tiled work-groups (one per CU)
constexpr int kStreamMaxShare = 4;     // token tiles sharing a weight tile that still take streamed copies
constexpr size_t kPartFloats = size_t(16) << 20;  // split-K partials (64 MB)
constexpr int kCounters = 1 << 16;

// Raises a kernel's dynamic-LDS limit to `bytes`, once per device: the
// attribute belongs to the kernel on the device current when it is set, so a
// process driving several GPUs sets it on each.  `done` is the call site's own
// bitmask of devices already set (one per kernel instance).
void set_lds_limit(std::atomic<uint64_t>& done, const void* kern, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);  // no bit to remember it by
    return;
  }
  const uint64_t bit = uint64_t(1) << dev;
  if (done.load(std::memory_order_acquire) & bit) return;
  (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done.fetch_or(bit, std::memory_order_acq_rel);
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }
int ceil_div_l(long long a, long long b) { return (int)((a + b - 1) / b); }

struct Plan {
  // pool
  size_t kv_off, rope_off, relay_off, pool_bytes;
  size_t head_stride, kv_stride, layer_stride, slot_stride;  // elements
  int ctx_pad;
  // workspace
  size_t x_off, u_off, ssq_off, q_off, kb_off, vbt_off, o_off, h_off;
  size_t po_off, pml_off, lmv_off, lmi_off, hc_off, hclo_off, fssq_off, part_off, ctr_off;
  size_t rin_off, rlnh_off, rs_off, sel_off, cv_off, ob_off, zc_off;
  size_t ss_part_off, ss_lse_off, ss_nacc_off, ss_rctr_off, ss_qctr_off, ss_blk_off, ws_bytes;
  int ss_nchunk;  // vocabulary chunks of the sampling kernels
  int relay_rows;  // relay rows one call can hold: max_batch * (B - 2)
  int BP;
  size_t lm_entries;
  int qf;
};

// Tiled GEMM work-group shapes: BM tokens x BN features, WM x WN waves, ring depth.
template <int BM_, int BN_, int WM_, int WN_, int NBUF_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NBUF = NBUF_;
  static constexpr int kFeatPerWave = BN / WN;  // features of one wave's fragment row
};
using TileStd = TileCfg<128, 128, 2, 4, 3>;   // general
using TileS192 = TileCfg<128, 192, 4, 2, 3>;  // general, 32 x 96 per wave, where it fills the CUs better
using TileWide = TileCfg<256, 256, 2, 4, 2>;  // many tokens against a wide weight (and the LM head)
using TileW192 = TileCfg<256, 192, 4, 2, 2>;  // same, 64 x 96 per wave, where it fills the CUs better
// Relative time of one work-group tile (measured on the 512 x 24576 x 4096
// bf16 GEMM with one tile per CU): 256 x 192 takes 0.86 of a 256 x 256 tile.
constexpr double kW192TileCost = 0.86;
using TileLo = TileCfg<64, 128, 2, 4, 3>;     // activations as hi + lo planes
using TileLoWide = TileCfg<128, 256, 2, 4, 2>;  // same, many tokens (every CU filled)
// A narrow weight against many tokens (the convolution's tap corrections,
// 512 x 4096 at the 8B shape): 64 x 64 tiles with K split four ways fill every
// CU; against 64 x 128 tiles split eight ways the last arriver of a tile sums
// 64 KB of partials instead of 256 KB (0.49 -> 0.44 ms of convolution per
// bs 32 step).
using TileNarrow = TileCfg<64, 64, 4, 2, 3>;
constexpr int kWideMinFeatures = 16384;

int elt_size(int dtype) { return dtype == DFLASH_BF16 ? 2 : 4; }

// Few-token LM head: one 16-wave work-group per CU and 16-row block.
int lm_chunks_small(int rowblocks) { return std::max(1, 256 / rowblocks); }
constexpr int kLdsMax = 160 * 1024;  // LDS of one CU
// LDS of the top-k LM head: 16 staged rows, reused for the 16 x 64 x 16 list
// merge and its 16 x 64 list heads.
int lm_small_lds(const dflash_dims& d) {
  return std::max(16 * (d.D * elt_size(d.dtype) + 16), 16 * 64 * 16 * 8 + 16 * 64);
}

// Which GEMM engine serves M rows against a weight of ngroups 16-row groups:
// few rows, or a narrow weight (it stays in L2 across the 16-row blocks),
// take the activation-stationary GEMV; the rest the tiled GEMM.
bool uses_gemv(int M, int ngroups) { return M <= kSkinnyMaxM || ngroups <= kNarrowMaxGroups; }

// Top-1 LM head through the GEMM engines: one partial per 16-row tile (GEMV,
// few rows) or per wave fragment row of the wide tiled GEMM (many rows).
int lm_top1_chunks(int Mlm, int V) {
  return uses_gemv(Mlm, ceil_div(V, 16)) ? ceil_div(V, 16) : ceil_div(V, TileWide::kFeatPerWave);
}

// LM-head partial-list entries a call needs (KTOP = 16 for top_k > 1).
size_t lm_entries_for(int Mlm, int V, int top_k) {
  if (top_k == 1) return (size_t)lm_top1_chunks(Mlm, V) * Mlm;
  return (size_t)lm_chunks_small(ceil_div(Mlm, 16)) * Mlm * 16;
}

int validate_dims(const dflash_dims* d) {
  if (!d) return fail(DFLASH_EINVAL, "dims is NULL");
  if (d->dtype != DFLASH_F32 && d->dtype != DFLASH_BF16)
    return fail(DFLASH_EUNSUPPORTED, "dtype must be DFLASH_F32 or DFLASH_BF16");
  const int vals[] = {d->D, d->L, d->Dt, d->N, d->Hq, d->Hkv, d->hd, d->I, d->V, d->B,
                      d->max_ctx, d->max_slots, d->max_batch};
  for (int v : vals)
    if (v <= 0) return fail(DFLASH_EINVAL, "all dimensions must be positive");
  if (d->hd != 64 && d->hd != 128) return fail(DFLASH_EUNSUPPORTED, "head dim must be 64 or 128");
  if (d->B < 2 || d->B > 16) return fail(DFLASH_EUNSUPPORTED, "block size must be in 2..16");
  if (d->N > kMaxLayers) return fail(DFLASH_EUNSUPPORTED, "at most 16 drafter layers");
  if (d->L > kMaxKSeg) return fail(DFLASH_EUNSUPPORTED, "at most 16 tapped target layers");
  if (d->max_batch > kMaxReq) return fail(DFLASH_EUNSUPPORTED, "max_batch must be <= 64");
  if (d->Hq % d->Hkv) return fail(DFLASH_EINVAL, "Hq must be a multiple of Hkv");
  if ((d->Hq / d->Hkv) * d->B > 64)
    return fail(DFLASH_EUNSUPPORTED, "(Hq/Hkv)*B must be <= 64 (query rows per KV head)");
  if (d->D % 64 || d->Dt % 64 || d->I % 64)
    return fail(DFLASH_EUNSUPPORTED, "D, Dt and I must be multiples of 64");
  if (d->V % 64) return fail(DFLASH_EUNSUPPORTED, "V must be a multiple of 64");
  if (!(d->rms_eps >= 0.f) || !(d->rope_base > 0.f))
    return fail(DFLASH_EINVAL, "rms_eps must be >= 0 and rope_base > 0");
  if ((long long)d->max_ctx > (1 << 24)) return fail(DFLASH_EUNSUPPORTED, "max_ctx too large");
  return DFLASH_OK;
}

void make_plan(const dflash_dims* d, Plan* p) {
  const size_t e = elt_size(d->dtype);
  p->ctx_pad = round_up(d->max_ctx, 64);
  p->head_stride = (size_t)p->ctx_pad * d->hd;
  p->kv_stride = p->head_stride * d->Hkv;
  p->layer_stride = 2 * p->kv_stride;
  p->slot_stride = p->layer_stride * d->N;
  size_t off = 0;
  p->kv_off = off;
  off = align_up(off + p->slot_stride * d->max_slots * e);
  p->rope_off = off;
  off = align_up(off + (size_t)(d->max_ctx + d->B) * (d->hd / 2) * sizeof(float2));
  p->relay_off = off;  // DFlow relay rows [max_slots][B][D] fp32
  off = align_up(off + (size_t)d->max_slots * d->B * d->D * 4);
  p->pool_bytes = off;

  const int M = d->max_batch * d->B;
  const int Mlm = d->max_batch * (d->B - 1);
  const int nslot = d->D / 16;
  p->BP = kVTile;  // block V^T padded to one V^T tile
  p->qf = ceil_div((d->Hq / d->Hkv) * d->B, 16);
  if (p->qf == 3) p->qf = 4;
  off = 0;
  p->x_off = off;    off = align_up(off + (size_t)M * d->D * 4);
  p->u_off = off;    off = align_up(off + (size_t)M * d->D * e);
  p->ssq_off = off;  off = align_up(off + (size_t)M * nslot * 4);
  p->q_off = off;    off = align_up(off + (size_t)M * d->Hq * d->hd * e);
  p->kb_off = off;   off = align_up(off + (size_t)M * d->Hkv * d->hd * e);
  p->vbt_off = off;  off = align_up(off + (size_t)d->max_batch * d->Hkv * d->hd * p->BP * e);
  p->o_off = off;    off = align_up(off + (size_t)M * d->Hq * d->hd * e);
  p->h_off = off;    off = align_up(off + (size_t)M * d->I * e);
  const int qr = p->qf * 16;
  p->po_off = off;   off = align_up(off + (size_t)kAttnWorkMax * qr * d->hd * 4);
  p->pml_off = off;  off = align_up(off + (size_t)kAttnWorkMax * qr * 2 * 4);
  size_t lm = 0;
  for (int m = 1; m <= Mlm; ++m)
    lm = std::max(lm, std::max(lm_entries_for(m, d->V, 1), lm_entries_for(m, d->V, 16)));
  p->lm_entries = lm;
  p->lmv_off = off;  off = align_up(off + lm * 4);
  p->lmi_off = off;  off = align_up(off + lm * 4);
  p->hc_off = off;   off = align_up(off + (size_t)kFuseChunk * d->D * e);
  p->hclo_off = off; off = align_up(off + (size_t)kFuseChunk * d->D * e);
  p->fssq_off = off; off = align_up(off + (size_t)kFuseChunk * nslot * 4);
  p->part_off = off; off = align_up(off + kPartFloats * 4);
  p->ctr_off = off;  off = align_up(off + (size_t)kCounters * 4);
  p->relay_rows = d->max_batch * std::max(0, d->B - 2);
  p->rin_off = off;  off = align_up(off + (size_t)p->relay_rows * 3 * d->D * e);
  p->rlnh_off = off; off = align_up(off + (size_t)p->relay_rows * d->D * 4);
  p->rs_off = off;   off = align_up(off + (size_t)p->relay_rows * d->D * e);
  // selector gates [rows][rank <= 256], then pair tables [rows][16][16]
  p->sel_off = off;  off = align_up(off + (size_t)Mlm * 256 * 4 * 2);
  // two-tap convolution: convolved GEMM operand, sub-layer output, tap corrections
  p->cv_off = off;   off = align_up(off + (size_t)M * d->D * e);
  p->ob_off = off;   off = align_up(off + (size_t)M * d->D * e);
  p->zc_off = off;   off = align_up(off + (size_t)M * (d->D / 8) * 4);
  // speculative sampling: per-chunk partials of up to 2B-1 rows per request,
  // row log-sum-exps, accepted counts, row and request tickets
  const int ss_rows = d->max_batch * (2 * d->B - 1);
  p->ss_nchunk = std::max(ceil_div(d->V, kSsThreads * 8), kSsPickParts);  // partial slots per row: 2048-id pieces, block-draw parts
  p->ss_part_off = off; off = align_up(off + (size_t)ss_rows * p->ss_nchunk * 16);
  p->ss_lse_off = off;  off = align_up(off + (size_t)ss_rows * 4);
  p->ss_nacc_off = off; off = align_up(off + (size_t)d->max_batch * 4);
  p->ss_rctr_off = off; off = align_up(off + (size_t)ss_rows * 4);
  p->ss_qctr_off = off; off = align_up(off + (size_t)d->max_batch * 4);
  p->ss_blk_off = off;  off = align_up(off + (size_t)ss_rows * 4);
  p->ws_bytes = off;
}

bool hip_ok(hipError_t e, const char* what, int* rc) {
  if (e == hipSuccess) return true;
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  *rc = DFLASH_EHIP;
  return false;
}

}  // namespace

struct ProfRec {
  int kind;
  hipEvent_t a, b;
};

struct dflash_ctx {
  uint32_t prof_mask = 0;
  std::vector<hipEvent_t> prof_events;  // pool, 2 per launch
  std::vector<ProfRec> prof_recs;
  dflash_dims d;
  dflash_weights w;
  std::vector<dflash_layer_weights> layers;
  Plan p;
  char* pool;
  char* ws;
  std::vector<int> len;
  std::vector<int> relay_n;    // DFlow relay rows stored per slot (offsets 2..1+n)
  std::vector<int> relay_len;  // slot length they were stored at
  int last_draft_n = 0;        // requests of the most recent draft (its final hidden states are in the workspace)
  std::vector<dflash2_conv_layer> conv;  // DFlash 2 two-tap convolution, empty when detached
  template <typename T> T* wsp(size_t off) const { return reinterpret_cast<T*>(ws + off); }
};

namespace {

// Event pair around one launch when its kind is being profiled.
struct ProfScope {
  dflash_ctx* c;
  int kind;
  hipStream_t st;
  bool on;
  ProfScope(dflash_ctx* c_, int k, hipStream_t s)
      : c(c_), kind(k), st(s),
        on(c_ && ((c_->prof_mask >> k) & 1u) && c_->prof_recs.size() * 2 + 2 <= c_->prof_events.size()) {
    if (on) {
      ProfRec r{kind, c->prof_events[c->prof_recs.size() * 2], c->prof_events[c->prof_recs.size() * 2 + 1]};
      (void)hipEventRecord(r.a, st);
      c->prof_recs.push_back(r);
    }
  }
  ~ProfScope() {
    if (on) (void)hipEventRecord(c->prof_recs.back().b, st);
  }
};

// ------------------------------------------------------------------ GEMM dispatch

template <class C, typename T, bool ALO, class Epi>
void launch_tiled(dflash_ctx* c, const WOperand<T>& w, const AOperand<T>& a, const NormIn& nrm, const Epi& epi,
                  hipStream_t st) {
  constexpr int BKE = 128 / sizeof(T);
  const int nst = a.nk * a.kseg / BKE;
  const int MT = ceil_div(a.M, C::BM), NT = ceil_div(w.ngroups, C::BN / 16);
  const int tiles = MT * NT;
  // Split K only when the tiles alone leave CUs idle: at least 8 stages per
  // split, partials and tickets within the workspace.
  int SK = std::max(1, std::min(kTiledSlots / tiles, nst / 8));
  while (SK > 1 && ((size_t)tiles * SK * C::BM * C::BN > kPartFloats || tiles > kCounters - 64)) --SK;
  const int kps = ceil_div(nst, SK);
  SK = ceil_div(nst, kps);
  const SplitK sk{SK, kps, c->wsp<float>(c->p.part_off), c->wsp<int>(c->p.ctr_off), MT <= kStreamMaxShare};
  const int nblocks = tiles * SK;
  const int lds = C::NBUF * ((ALO ? 2 : 1) * C::BM + C::BN) * 128;
  auto kern = gemm_tiled_kernel<T, C::BM, C::BN, C::WM, C::WN, C::NBUF, ALO, Epi>;
  static std::atomic<uint64_t> lds_set{0};
  set_lds_limit(lds_set, reinterpret_cast<const void*>(kern), lds);
  hipLaunchKernelGGL(kern, dim3(round_up(nblocks, 8)), dim3(64 * C::WM * C::WN), lds, st, w, a, nrm, sk, epi,
                     nblocks);
}

// Row-streaming GEMV plan: K ranges and tiles per work-group for about one
// work-group per CU, least time per work-group (ties: fewer K ranges).  A
// tile costs its stages plus a fixed two-stage equivalent (ring fill and
// drain, the split-K ticket): without it, rows of five 1 KB stages (K = 2560)
// were split five ways into one-stage tiles, 1.7x slower than whole rows.
// Returns false where the kernel does not apply (rows not whole 1 KB stages,
// too many stages for the held activations of a row epilogue, tile sums
// beyond LDS, or partials beyond the workspace).
struct RsPlan {
  int nsplit, nst, red2, tpw, nwg, lds;
};
template <typename T, bool ALO, class Epi>
bool plan_rs(const WOperand<T>& w, const AOperand<T>& a, int mt, RsPlan* out) {
  const long row_bytes = (long)a.nk * a.kseg * (long)sizeof(T);
  if (row_bytes % kRsStage != 0 || (Epi::kPaired && w.pair % 8 != 0)) return false;
  const int nst_all = (int)(row_bytes / kRsStage);
  const int ah = gemv_rs_ah(ALO);
  const int ks_min = ceil_div(nst_all, ah);
  const int ks_max = Epi::kRow ? 1 : std::min(nst_all, kRsMaxSplit);
  long best = -1;
  for (int ks = ks_min; ks <= ks_max; ++ks) {
    const int per = std::max(1, kTiledSlots / (ks * mt));
    const int tpw = ceil_div(w.ngroups, per);
    const int nst = ceil_div(nst_all, ks);
    const int red2 = nst < 2 || nst_all - (ceil_div(nst_all, nst) - 1) * nst < 2;
    const int lds = gemv_rs_lds(kRsNbuf, red2, tpw);
    if (lds > kRsLdsMax) continue;
    if (ks > 1 && ((long)mt * w.ngroups > kCounters - 64 || (size_t)mt * w.ngroups * ks * 256 > kPartFloats)) continue;
    const long cost = (long)tpw * (nst + 2) + (long)(ks - 1) * kRsSplitCost;
    if (best < 0 || cost < best) {
      best = cost;
      *out = RsPlan{ceil_div(nst_all, nst), nst, red2, tpw, ceil_div(w.ngroups, tpw), lds};
    }
  }
  return best >= 0;
}

// Work-group tile area per CU slot, summed over whole waves of one work-group
// per CU, for a tile shape with the split-K rule of launch_tiled.
template <class C>
long tiled_cost(int M, int ngroups, int nst) {
  const int tiles = ceil_div(M, C::BM) * ceil_div(ngroups, C::BN / 16);
  const int SK = std::max(1, std::min(kTiledSlots / tiles, nst / 8));
  return (long)ceil_div(tiles * SK, kTiledSlots) * C::BM * C::BN / SK;
}

// The GEMV engines (few rows, or a narrow weight); false where neither applies.
template <typename T, bool ALO = false, class Epi>
bool launch_skinny(dflash_ctx* c, const WOperand<T>& w, const AOperand<T>& a, const NormIn& nrm, const Epi& epi,
                   hipStream_t st) {
  const int K = a.nk * a.kseg;
  {
    const int mt = ceil_div(a.M, 16);
    RsPlan rp;
    if (uses_gemv(a.M, w.ngroups) && mt < kGemvXcds && plan_rs<T, ALO, Epi>(w, a, mt, &rp)) {
      // Row-streaming GEMV (few token blocks against a wide weight).
      auto kern = gemv_rs_kernel<T, kRsNbuf, ALO, Epi::kPaired, Epi>;
      static std::atomic<uint64_t> lds_set{0};
      set_lds_limit(lds_set, reinterpret_cast<const void*>(kern), kRsLdsMax);
      const RsSplit sp{rp.nsplit, rp.nst, rp.red2, c->wsp<float>(c->p.part_off), c->wsp<int>(c->p.ctr_off),
                       mt <= kStreamMaxShare};
      hipLaunchKernelGGL(kern, dim3(rp.nwg, rp.nsplit * mt), dim3(1024), rp.lds, st, w, a, nrm, sp, epi, rp.tpw);
      return true;
    }
    if (uses_gemv(a.M, w.ngroups)) {
      // Activation-stationary GEMV: 16-row tiles, K split across the waves of
      // a work-group (LDS reduction; a cross-work-group split would need
      // device-scope fences, which write back and invalidate the XCD's L2).
      constexpr int KSW = kGemvKSW;
      const int nks = K / Mma<T>::KSTEP;
      const int nw = std::max(1, std::min(16, ceil_div(nks, KSW)));
      const int mt = ceil_div(a.M, 16);
      // tiles per work-group: fill every CU once per 16-token block (even for paired epilogues)
      int tpw = std::max(1, ceil_div(w.ngroups, std::max(1, kGemvWGs / mt)));
      if (Epi::kPaired) tpw += tpw & 1;
      const int nwg = ceil_div(w.ngroups, tpw);
      const int lds = kGemvTB * nw * 64 * 16;
      // row blocks kept on one XCD each once there are enough to go round
      const bool xr = mt >= kGemvXcds;
      auto launch = [&](auto kern, dim3 grid) {
        static std::atomic<uint64_t> lds_set{0};
        set_lds_limit(lds_set, reinterpret_cast<const void*>(kern), kGemvTB * 16 * 64 * 16);
        hipLaunchKernelGGL(kern, grid, dim3(64 * nw), lds, st, w, a, nrm, epi, tpw);
      };
      if (xr)
        launch(gemv_as_kernel<T, KSW, ALO, kGemvTB, true, Epi>,
               dim3(kGemvXcds * nwg * ceil_div(mt, kGemvXcds)));
      else
        launch(gemv_as_kernel<T, KSW, ALO, kGemvTB, false, Epi>, dim3(nwg, mt));
      return true;
    }
  }
  return false;
}

template <typename T, bool ALO = false, class Epi>
void launch_gemm(dflash_ctx* c, const WOperand<T>& w, const AOperand<T>& a, const NormIn& nrm, const Epi& epi,
                 hipStream_t st) {
  if (a.M <= 0 || w.ngroups <= 0) return;
  if (launch_skinny<T, ALO>(c, w, a, nrm, epi, st)) return;
  const int K = a.nk * a.kseg;
  if constexpr (ALO) {
    if ((long)ceil_div(a.M, TileLoWide::BM) * ceil_div(w.ngroups, TileLoWide::BN / 16) >= kTiledSlots)
      launch_tiled<TileLoWide, T, true>(c, w, a, nrm, epi, st);
    else
      launch_tiled<TileLo, T, true>(c, w, a, nrm, epi, st);
  }
  else if (Epi::kRow || (a.M >= 256 && (w.ngroups * 16 >= kWideMinFeatures ||
                                         (long)ceil_div(a.M, 256) * ceil_div(w.ngroups, 16) >= kTiledSlots))) {
    // wide weights, or enough 256 x 256 tiles to fill every CU (many tokens):
    // whole waves of one work-group per CU, times the per-tile cost
    const int mt = ceil_div(a.M, 256);
    const double w256 = ceil_div(mt * ceil_div(w.ngroups, 16), kTiledSlots);
    const double w192 = ceil_div(mt * ceil_div(w.ngroups, 12), kTiledSlots) * kW192TileCost;
    if (!Epi::kRow && w192 < w256)
      launch_tiled<TileW192, T, false>(c, w, a, nrm, epi, st);
    else
      launch_tiled<TileWide, T, false>(c, w, a, nrm, epi, st);
  }
  else {
    const int nst = K * (int)sizeof(T) / 128;
    if (tiled_cost<TileS192>(a.M, w.ngroups, nst) < tiled_cost<TileStd>(a.M, w.ngroups, nst))
      launch_tiled<TileS192, T, false>(c, w, a, nrm, epi, st);
    else
      launch_tiled<TileStd, T, false>(c, w, a, nrm, epi, st);
  }
}

template <typename T>
WOperand<T> wop(std::initializer_list<std::pair<const void*, int>> segs, int pair) {
  WOperand<T> w{};
  int end = 0, n = 0;
  for (auto& s : segs) {
    w.ptr[n] = static_cast<const T*>(s.first);
    end += s.second;
    w.end[n] = end;
    ++n;
  }
  w.nseg = n;
  w.pair = pair;
  w.ngroups = end / 16;
  return w;
}

template <typename T>
AOperand<T> aop(const void* p, int M, int K, int rowmap_b = 0) {
  AOperand<T> a{};
  a.ptr[0] = static_cast<const T*>(p);
  a.nk = 1;
  a.kseg = K;
  a.lda = K;
  a.M = M;
  a.rowmap_b = rowmap_b;
  return a;
}

NormIn norm_in(const float* ssq, int D, float eps) { return NormIn{ssq, D / 16, 1.0f / (float)D, eps}; }

// ------------------------------------------------------------------ fuse

template <typename T>
void run_fuse(dflash_ctx* c, hipStream_t st, const FuseMeta& fm, int total, const void* const* hid) {
  const dflash_dims& d = c->d;
  const Plan& p = c->p;
  T* hc = c->wsp<T>(p.hc_off);
  // bf16: H_c is kept as hi + lo bf16 planes so the context K/V projection
  // sees it at near-fp32 precision (that GEMM is small next to the fusion).
  T* hclo = sizeof(T) == 2 ? c->wsp<T>(p.hclo_off) : nullptr;
  float* fssq = c->wsp<float>(p.fssq_off);
  T* pool = reinterpret_cast<T*>(c->pool + p.kv_off);
  const float2* rope = reinterpret_cast<const float2*>(c->pool + p.rope_off);

  WOperand<T> wc = wop<T>({{c->w.w_c, d.D}}, 0);
  WOperand<T> wkv{};
  {
    int end = 0, n = 0;
    for (int l = 0; l < d.N; ++l) {
      wkv.ptr[n] = static_cast<const T*>(c->layers[l].w_kc);
      end += d.Hkv * d.hd;
      wkv.end[n++] = end;
      wkv.ptr[n] = static_cast<const T*>(c->layers[l].w_vc);
      end += d.Hkv * d.hd;
      wkv.end[n++] = end;
    }
    wkv.nseg = n;
    wkv.pair = d.hd / 2;
    wkv.ngroups = end / 16;
  }
  const NormIn none{nullptr, 0, 0.f, 0.f};
  for (int base = 0; base < total; base += kFuseChunk) {
    const int rows = std::min(kFuseChunk, total - base);
    AOperand<T> a{};
    for (int l = 0; l < d.L; ++l) a.ptr[l] = static_cast<const T*>(hid[l]) + (size_t)base * d.Dt;
    a.nk = d.L;
    a.kseg = d.Dt;
    a.lda = d.Dt;
    a.M = rows;
    {
      ProfScope ps(c, DFLASH_K_FUSE_GEMM, st);
      launch_gemm<T>(c, wc, a, none, EpiNormOut<T>{hc, hclo, static_cast<const T*>(c->w.g_c), fssq, d.D, d.D / 16},
                     st);
    }
    EpiKVAppend<T> epi{};
    epi.pool = pool;
    epi.slot_stride = p.slot_stride;
    epi.layer_stride = p.layer_stride;
    epi.kv_stride = p.kv_stride;
    epi.head_stride = p.head_stride;
    epi.rope = rope;
    epi.Hkv = d.Hkv;
    epi.hd = d.hd;
    epi.use_rope = d.use_rope;
    epi.row_base = base;
    epi.meta = fm;
    ProfScope ps(c, DFLASH_K_CTX_KV_GEMM, st);
    AOperand<T> ah = aop<T>(hc, rows, d.D);
    if (hclo) {
      ah.lo_off = (long)(hclo - hc);
      launch_gemm<T, true>(c, wkv, ah, norm_in(fssq, d.D, d.rms_eps), epi, st);
    } else {
      launch_gemm<T>(c, wkv, ah, norm_in(fssq, d.D, d.rms_eps), epi, st);
    }
  }
}

// ------------------------------------------------------------------ attention

// Split-KV partial kernel (combine = false) or the combine kernel (true).
template <typename T, int HD, int QF>
void launch_attn(const AttnArgs<T>& a, int work, bool combine, hipStream_t st) {
  if (combine) {
    int smax = 1;
    for (int r = 0; r < a.meta.n_req; ++r) smax = std::max(smax, a.meta.nsplit[r]);
    const long outs = (long)a.meta.n_req * a.Hkv * a.G * a.B * (HD / 4);
    auto go = [&](auto kern, int sub) {
      hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div_l(outs * sub, 256)), dim3(256), 0, st, a);
    };
    // lanes per output only when the split loops are long (few outputs, many splits)
    if (smax >= 16) go(attn_combine_kernel<T, HD, QF * 16, 8>, 8);
    else go(attn_combine_kernel<T, HD, QF * 16, 1>, 1);
    return;
  }
  // A ring of NBUF stages of K/V per work-group (fewer where a stage takes
  // many copy instructions per wave); QW query fragments per wave.  The
  // Qwen3-shaped instance (bf16, head dim 128, four query fragments) takes
  // kAttnStg keys per stage on long splits (64: half the barriers of 32-key
  // stages, measured faster at bs 32) and 32 on splits of at most
  // kAttnShortSplit keys (bs 1: more stages in flight per split), with a
  // register cap for kAttnWpe waves per SIMD; the others keep 32-key stages,
  // whose fewer copies per wave keep them out of spills.
  constexpr bool kMain = std::is_same<T, bf16_t>::value && HD == 128 && QF == 4;
  constexpr int QW = QF % kAttnQw == 0 ? kAttnQw : 1;
  constexpr int WPE = kMain ? kAttnWpe : 1;
  auto go = [&](auto stg) {
    constexpr int STG = decltype(stg)::value;
    constexpr int NIW = AttnStage<T, HD, QF / QW, 2, STG>::NIW;
    constexpr int NBUF = std::min(kAttnNbuf, 2 + 63 / NIW);
    const int lds = AttnStage<T, HD, QF / QW, NBUF, STG>::LDS;
    auto kern = attn_kernel<T, HD, QF, QW, NBUF, STG, WPE>;
    static std::atomic<uint64_t> lds_set{0};
    set_lds_limit(lds_set, reinterpret_cast<const void*>(kern), lds);
    hipLaunchKernelGGL(kern, dim3(work), dim3(64 * (QF / QW)), lds, st, a);
  };
  if (kMain && a.chunk > kAttnShortSplit)
    go(std::integral_constant<int, kMain ? kAttnStg : 32>{});
  else
    go(std::integral_constant<int, 32>{});
}

template <typename T>
void attn_dispatch(const AttnArgs<T>& a, int work, int hd, int qf, bool combine, hipStream_t st) {
  if (hd == 128) {
    if (qf == 1) launch_attn<T, 128, 1>(a, work, combine, st);
    else if (qf == 2) launch_attn<T, 128, 2>(a, work, combine, st);
    else launch_attn<T, 128, 4>(a, work, combine, st);
  } else {
    if (qf == 1) launch_attn<T, 64, 1>(a, work, combine, st);
    else if (qf == 2) launch_attn<T, 64, 2>(a, work, combine, st);
    else launch_attn<T, 64, 4>(a, work, combine, st);
  }
}

struct AttnPlan {
  int chunk, work;
  AttnMeta meta;
};

void plan_attention(const dflash_ctx* c, int n_req, const int32_t* slot, AttnPlan* ap) {
  const dflash_dims& d = c->d;
  // Splits of at least kAttnMinChunk keys (partial results stay small next to
  // the K/V they summarise), about kAttnTargetWG work-groups per call.
  long long total = 0;
  for (int r = 0; r < n_req; ++r) total += c->len[slot[r]];
  int chunk = round_up(std::max(1, ceil_div_l(total * d.Hkv, kAttnTargetWG)), kAttnStage);
  chunk = std::max(chunk, kAttnMinChunk);
  for (;;) {
    long long work = 0;
    for (int r = 0; r < n_req; ++r) work += (long long)d.Hkv * std::max(1, ceil_div(c->len[slot[r]], chunk));
    if (work <= kAttnWorkMax) {
      ap->chunk = chunk;
      ap->work = (int)work;
      break;
    }
    chunk *= 2;
  }
  AttnMeta& m = ap->meta;
  memset(&m, 0, sizeof(m));
  m.n_req = n_req;
  int w = 0;
  for (int r = 0; r < n_req; ++r) {
    m.ctx[r] = c->len[slot[r]];
    m.slot[r] = slot[r];
    m.nsplit[r] = std::max(1, ceil_div(m.ctx[r], ap->chunk));
    m.work0[r] = w;
    w += d.Hkv * m.nsplit[r];
  }
  m.work0[n_req] = w;
  // Launch order (see AttnMeta): last splits by descending length in 64-key
  // units (the rest of the context plus one unit for the block), ties by request.
  int last[kMaxReq];
  for (int r = 0; r < n_req; ++r) {
    last[r] = ceil_div(m.ctx[r] - (m.nsplit[r] - 1) * ap->chunk, kAttnStage) + 1;
    m.rorder[r] = r;
  }
  std::stable_sort(m.rorder, m.rorder + n_req, [&](int x, int y) { return last[x] > last[y]; });
  const int full = ap->chunk / kAttnStage;
  m.nbig = 0;
  while (m.nbig < n_req && last[m.rorder[m.nbig]] >= full) ++m.nbig;
}

// ------------------------------------------------------------------ LM head

template <typename T, int KTOP>
void launch_lm_small(const LmArgs<T>& la, int nchunk, int rowblocks, int* tile_ctr, hipStream_t st) {
  // staged rows, reused afterwards for the 16 x 64 x KTOP list merge and its list heads
  const int lds = std::max(16 * (la.a.kseg * (int)sizeof(T) + 16), 16 * 64 * KTOP * 8 + 16 * 64);  // <= kLdsMax (checked)
  auto kern = lmhead_lds_kernel<T, KTOP, kLmFN, kLmU>;
  static std::atomic<uint64_t> lds_set{0};
  set_lds_limit(lds_set, reinterpret_cast<const void*>(kern), 160 * 1024);
  hipLaunchKernelGGL(kern, dim3(nchunk, rowblocks), dim3(1024), lds, st, la, tile_ctr);
}

template <typename T>
void run_lmhead(dflash_ctx* c, hipStream_t st, int n_req, int top_k, int32_t* out_ids, float* out_vals,
                float* out_logits) {
  const dflash_dims& d = c->d;
  const Plan& p = c->p;
  const int Mlm = n_req * (d.B - 1);
  float* pv = c->wsp<float>(p.lmv_off);
  int* pi = c->wsp<int>(p.lmi_off);
  int* tile_ctr = c->wsp<int>(p.ctr_off) + (kCounters - 64);
  const AOperand<T> a = aop<T>(c->wsp<T>(p.u_off), Mlm, d.D, d.B);
  const NormIn nrm = norm_in(c->wsp<float>(p.ssq_off), d.D, d.rms_eps);
  int nchunk;
  {
    ProfScope ps(c, DFLASH_K_LM_HEAD, st);
    if (top_k == 1) {
      nchunk = lm_top1_chunks(Mlm, d.V);
      EpiTop1 epi{pv, pi, out_logits, Mlm, d.V, nchunk};
      launch_gemm<T>(c, wop<T>({{c->w.w_lm, d.V}}, 0), a, nrm, epi, st);
    } else {
      const int rowblocks = ceil_div(Mlm, 16);
      nchunk = lm_chunks_small(rowblocks);
      LmArgs<T> la{a, nrm, static_cast<const T*>(c->w.w_lm), d.V, out_logits, pv, pi};
      launch_lm_small<T, 16>(la, nchunk, rowblocks, tile_ctr, st);
    }
  }
  ProfScope ps(c, DFLASH_K_TOPK_MERGE, st);
  if (top_k == 1)
    hipLaunchKernelGGL(top1_merge_kernel, dim3(Mlm), dim3(1024), 0, st, pv, pi, nchunk, out_ids, out_vals, tile_ctr,
                       64);
  else
    hipLaunchKernelGGL((topk_merge_kernel<16>), dim3(Mlm), dim3(256), 0, st, pv, pi, nchunk, top_k, out_ids,
                       out_vals, tile_ctr, 64);
}

// ------------------------------------------------------------------ draft

template <typename T>
void run_draft(dflash_ctx* c, hipStream_t st, int n_req, const int32_t* slot, const int32_t* anchor,
               int top_k, int32_t* out_ids, float* out_vals, float* out_logits, const AttnPlan& apl,
               const DraftRelay& rl) {
  const dflash_dims& d = c->d;
  const Plan& p = c->p;
  const int M = n_req * d.B;
  float* x = c->wsp<float>(p.x_off);
  T* u = c->wsp<T>(p.u_off);
  float* ssq = c->wsp<float>(p.ssq_off);
  T* q = c->wsp<T>(p.q_off);
  T* kb = c->wsp<T>(p.kb_off);
  T* vbT = c->wsp<T>(p.vbt_off);
  T* o = c->wsp<T>(p.o_off);
  T* h = c->wsp<T>(p.h_off);
  const float2* rope = reinterpret_cast<const float2*>(c->pool + p.rope_off);
  const NormIn nrm = norm_in(ssq, d.D, d.rms_eps);
  const NormIn none{nullptr, 0, 0.f, 0.f};
  const int nslot = d.D / 16;

  DraftMeta dm{};
  dm.n_req = n_req;
  dm.B = d.B;
  for (int r = 0; r < n_req; ++r) dm.ctx[r] = c->len[slot[r]];

  {
    ProfScope ps(c, DFLASH_K_EMBED, st);
    hipLaunchKernelGGL((embed_kernel<T>), dim3(M), dim3(256), 0, st, static_cast<const T*>(c->w.embed),
                       static_cast<const T*>(c->w.e_mask), anchor, static_cast<const T*>(c->layers[0].g_attn), d.B,
                       d.D, d.V, x, u, ssq, rl);
  }

  AttnArgs<T> aa{};
  aa.q = q;
  aa.kb = kb;
  aa.vbT = vbT;
  aa.o = o;
  aa.pool = reinterpret_cast<const T*>(c->pool + p.kv_off);
  aa.slot_stride = p.slot_stride;
  aa.layer_stride = p.layer_stride;
  aa.kv_stride = p.kv_stride;
  aa.head_stride = p.head_stride;
  aa.Hq = d.Hq;
  aa.Hkv = d.Hkv;
  aa.G = d.Hq / d.Hkv;
  aa.B = d.B;
  aa.BP = p.BP;
  aa.chunk = apl.chunk;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.hd));
  aa.part_o = c->wsp<float>(p.po_off);
  aa.part_ml = c->wsp<float>(p.pml_off);
  aa.meta = apl.meta;

  const int qd = d.Hq * d.hd, kd = d.Hkv * d.hd;
  const bool conv = !c->conv.empty();
  T* cv = c->wsp<T>(p.cv_off);
  T* ob = c->wsp<T>(p.ob_off);
  float* zc = c->wsp<float>(p.zc_off);
  // One convolution site.  Few token rows: one launch, the tap corrections
  // [W_0; W_1] x on a GEMV engine (tap rows paired) with the tap mix in its
  // epilogue.  Many rows: the corrections GEMM (K split over 64-token tiles)
  // stores z, then conv_mix_kernel mixes the taps.  Normed sites read the
  // folded RMSNorm operand (u with its row scale) and write the convolved
  // operand cv; residual sites read the sub-layer output ob and update x, u
  // and ssq.
  auto conv_site = [&](const dflash2_conv_site& cs, bool normed, const T* g_next_norm) {
    ProfScope ps(c, DFLASH_K_CONV, st);
    const T* in = normed ? u : ob;
    const AOperand<T> az = aop<T>(in, M, d.D);
    const NormIn& n = normed ? nrm : none;
    if (M <= kSkinnyMaxM) {
      const WOperand<T> wz = wop<T>({{cs.w, d.D / 8}}, d.D / 16);
      bool done;
      if (normed) {
        EpiConvMix<T, false> e{};
        e.in = in;
        e.ssq = ssq;
        e.inv_d = 1.0f / (float)d.D;
        e.eps = d.rms_eps;
        e.kbase = static_cast<const T*>(cs.kbase);
        e.B = d.B;
        e.D = d.D;
        e.y = cv;
        done = launch_skinny<T>(c, wz, az, n, e, st);
      } else {
        EpiConvMix<T, true> e{};
        e.in = in;
        e.kbase = static_cast<const T*>(cs.kbase);
        e.B = d.B;
        e.D = d.D;
        e.h = x;
        e.u = u;
        e.g = g_next_norm;
        e.ssq_out = ssq;
        done = launch_skinny<T>(c, wz, az, n, e, st);
      }
      if (done) return;
    }
    launch_tiled<TileNarrow, T, false>(c, wop<T>({{cs.w, d.D / 8}}, 0), az, n, EpiStore<float>{zc, d.D / 8}, st);
    ConvMixArgs<T> ca{};
    ca.in = in;
    ca.ssq = ssq;
    ca.inv_d = 1.0f / (float)d.D;
    ca.eps = d.rms_eps;
    ca.z = zc;
    ca.kbase = static_cast<const T*>(cs.kbase);
    ca.B = d.B;
    ca.D = d.D;
    ca.y = cv;
    ca.h = x;
    ca.u = u;
    ca.g = g_next_norm;
    ca.ssq_out = ssq;
    const int nt = std::min(1024, round_up(d.D / 4, 64));  // one 4-channel vector per thread (D <= 4096)
    if (normed)
      hipLaunchKernelGGL((conv_mix_kernel<T, false>), dim3(M), dim3(nt), 0, st, ca);
    else
      hipLaunchKernelGGL((conv_mix_kernel<T, true>), dim3(M), dim3(nt), 0, st, ca);
  };
  for (int l = 0; l < d.N; ++l) {
    const dflash_layer_weights& lw = c->layers[l];
    const T* g_next = static_cast<const T*>(l + 1 < d.N ? c->layers[l + 1].g_attn : c->w.g_final);
    if (conv) conv_site(c->conv[l].attn_in, true, nullptr);
    EpiQKV<T> eq{};
    eq.q = q;
    eq.kb = kb;
    eq.vbT = vbT;
    eq.rope = rope;
    eq.Hq = d.Hq;
    eq.Hkv = d.Hkv;
    eq.hd = d.hd;
    eq.BP = p.BP;
    eq.use_rope = d.use_rope;
    eq.meta = dm;
    {
      ProfScope ps(c, DFLASH_K_QKV_GEMM, st);
      launch_gemm<T>(c, wop<T>({{lw.w_q, qd}, {lw.w_kb, kd}, {lw.w_vb, kd}}, d.hd / 2),
                     aop<T>(conv ? cv : u, M, d.D), conv ? none : nrm, eq, st);
    }
    aa.layer = l;
    {
      ProfScope ps(c, DFLASH_K_ATTENTION, st);
      attn_dispatch<T>(aa, apl.work, d.hd, p.qf, false, st);
    }
    {
      ProfScope ps(c, DFLASH_K_ATTN_COMBINE, st);
      attn_dispatch<T>(aa, apl.work, d.hd, p.qf, true, st);
    }
    {
      ProfScope ps(c, DFLASH_K_O_GEMM, st);
      if (conv)
        launch_gemm<T>(c, wop<T>({{lw.w_o, d.D}}, 0), aop<T>(o, M, qd), none, EpiStore<T>{ob, d.D}, st);
      else
        launch_gemm<T>(c, wop<T>({{lw.w_o, d.D}}, 0), aop<T>(o, M, qd), none,
                       EpiResidualNorm<T>{x, u, static_cast<const T*>(lw.g_ffn), ssq, d.D, nslot}, st);
    }
    if (conv) {
      conv_site(c->conv[l].attn_out, false, static_cast<const T*>(lw.g_ffn));
      conv_site(c->conv[l].ffn_in, true, nullptr);
    }
    {
      ProfScope ps(c, DFLASH_K_GATEUP_GEMM, st);
      launch_gemm<T>(c, wop<T>({{lw.w_gate, d.I}, {lw.w_up, d.I}}, d.I), aop<T>(conv ? cv : u, M, d.D),
                     conv ? none : nrm, EpiSwiGLU<T>{h, d.I}, st);
    }
    {
      ProfScope ps(c, DFLASH_K_DOWN_GEMM, st);
      if (conv)
        launch_gemm<T>(c, wop<T>({{lw.w_down, d.D}}, 0), aop<T>(h, M, d.I), none, EpiStore<T>{ob, d.D}, st);
      else
        launch_gemm<T>(c, wop<T>({{lw.w_down, d.D}}, 0), aop<T>(h, M, d.I), none,
                       EpiResidualNorm<T>{x, u, g_next, ssq, d.D, nslot}, st);
    }
    if (conv) conv_site(c->conv[l].ffn_out, false, g_next);
  }
  run_lmhead<T>(c, st, n_req, top_k, out_ids, out_vals, out_logits);
}

}  // namespace

// ====================================================================== C ABI

// ------------------------------------------------------------------ DFlow relay

template <typename T>
void run_relay(dflash_ctx* c, hipStream_t st, const RelayMeta& rm, int total, const void* const* hid,
               const int32_t* cand, int cand_stride, const int32_t* bonus, const dflow_relay_weights* rw) {
  const dflash_dims& d = c->d;
  const Plan& p = c->p;
  T* hc = c->wsp<T>(p.hc_off);
  float* fssq = c->wsp<float>(p.fssq_off);
  T* in = c->wsp<T>(p.rin_off);
  float* lnh = c->wsp<float>(p.rlnh_off);
  T* sbuf = c->wsp<T>(p.rs_off);
  const NormIn none{nullptr, 0, 0.f, 0.f};
  {
    // relay step 1: the shared fusion projection of the suffix states
    ProfScope ps(c, DFLASH_K_FUSE_GEMM, st);
    AOperand<T> a{};
    for (int l = 0; l < d.L; ++l) a.ptr[l] = static_cast<const T*>(hid[l]);
    a.nk = d.L;
    a.kseg = d.Dt;
    a.lda = d.Dt;
    a.M = total;
    launch_gemm<T>(c, wop<T>({{c->w.w_c, d.D}}, 0), a, none,
                   EpiNormOut<T>{hc, nullptr, static_cast<const T*>(c->w.g_c), fssq, d.D, d.D / 16}, st);
  }
  ProfScope ps(c, DFLASH_K_RELAY, st);
  hipLaunchKernelGGL((relay_assemble_kernel<T>), dim3(total), dim3(256), 0, st, hc, fssq, d.D, d.rms_eps,
                     static_cast<const T*>(c->w.embed), d.V, bonus, cand, cand_stride, d.B - 1, rm, in, lnh);
  // relay step 3: [beta; gamma] = w2 SiLU(w1 [E(bonus); E(first rejection); h])
  launch_gemm<T>(c, wop<T>({{rw->w1, d.D}}, 0), aop<T>(in, total, 3 * d.D), none, EpiSiLUOut<T>{sbuf, d.D}, st);
  EpiRelayOut<T> eo{reinterpret_cast<float*>(c->pool + p.relay_off), lnh, static_cast<const T*>(c->w.e_mask),
                    d.B, d.D, rm};
  launch_gemm<T>(c, wop<T>({{rw->w2, 2 * d.D}}, d.D), aop<T>(sbuf, total, d.D), none, eo, st);
}

// ------------------------------------------------------------------ DFlash 2 selector

template <typename T>
void run_select(dflash_ctx* c, hipStream_t st, int n_req, const int32_t* anchor, const int32_t* cand,
                const float* ul, int k, const dflash2_selector_weights* sw, int32_t* out_path, float* out_scores) {
  const dflash_dims& d = c->d;
  const Plan& p = c->p;
  const int Mlm = n_req * (d.B - 1);
  float* gates = c->wsp<float>(p.sel_off);
  ProfScope ps(c, DFLASH_K_SELECT, st);
  // H(h_t) = sigmoid(w_h h_t) over the LM head's operand (the final normed hidden states)
  launch_gemm<T>(c, wop<T>({{sw->w_h, sw->rank}}, 0), aop<T>(c->wsp<T>(p.u_off), Mlm, d.D, d.B),
                 norm_in(c->wsp<float>(p.ssq_off), d.D, d.rms_eps), EpiSigmoidOut{gates, sw->rank}, st);
  float* tables = out_scores ? out_scores : gates + (size_t)Mlm * kSelMaxR;
  hipLaunchKernelGGL((select_tables_kernel<T>), dim3(n_req, d.B - 1), dim3(256), 0, st, anchor, cand, ul, k,
                     d.B - 1, static_cast<const T*>(sw->a), static_cast<const T*>(sw->b), sw->rank, gates, d.V,
                     tables);
  hipLaunchKernelGGL(select_walk_kernel, dim3(n_req), dim3(256), 0, st, cand, tables, k, d.B - 1, out_path);
}

extern "C" {

const char* dflash_strerror(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument";
    case DFLASH_EUNSUPPORTED: return "unsupported configuration";
    case DFLASH_ECAPACITY: return "capacity exceeded";
    case DFLASH_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dflash_last_error(void) { return g_last_error.c_str(); }

int dflash_query_sizes(const dflash_dims* dims, size_t* kv_pool_bytes, size_t* workspace_bytes) {
  g_last_error.clear();
  int rc = validate_dims(dims);
  if (rc) return rc;
  if (!kv_pool_bytes || !workspace_bytes) return fail(DFLASH_EINVAL, "output pointer is NULL");
  Plan p;
  make_plan(dims, &p);
  *kv_pool_bytes = p.pool_bytes;
  *workspace_bytes = p.ws_bytes;
  return DFLASH_OK;
}

int dflash_create(const dflash_dims* dims, const dflash_weights* weights, void* kv_pool,
                  size_t kv_pool_bytes, void* workspace, size_t workspace_bytes, dflash_ctx** out) {
  g_last_error.clear();
  int rc = validate_dims(dims);
  if (rc) return rc;
  if (!weights || !out || !kv_pool || !workspace) return fail(DFLASH_EINVAL, "NULL argument");
  const void* top[] = {weights->w_c, weights->g_c, weights->embed, weights->e_mask, weights->g_final,
                       weights->w_lm};
  for (const void* t : top)
    if (!t) return fail(DFLASH_EINVAL, "a model weight pointer is NULL");
  if (!weights->layers) return fail(DFLASH_EINVAL, "layers array is NULL");
  for (int l = 0; l < dims->N; ++l) {
    const dflash_layer_weights& lw = weights->layers[l];
    const void* lp[] = {lw.g_attn, lw.w_q, lw.w_kb, lw.w_vb, lw.w_kc, lw.w_vc,
                        lw.w_o,    lw.g_ffn, lw.w_gate, lw.w_up, lw.w_down};
    for (const void* t : lp)
      if (!t) return fail(DFLASH_EINVAL, "a layer weight pointer is NULL (layer " + std::to_string(l) + ")");
  }
  if (((uintptr_t)kv_pool % kAlign) || ((uintptr_t)workspace % kAlign))
    return fail(DFLASH_EINVAL, "kv_pool and workspace must be 256-byte aligned");
  Plan p;
  make_plan(dims, &p);
  if (kv_pool_bytes < p.pool_bytes) return fail(DFLASH_ECAPACITY, "kv_pool smaller than required");
  if (workspace_bytes < p.ws_bytes) return fail(DFLASH_ECAPACITY, "workspace smaller than required");

  dflash_ctx* c = new dflash_ctx();
  c->d = *dims;
  c->w = *weights;
  c->layers.assign(weights->layers, weights->layers + dims->N);
  c->w.layers = nullptr;
  c->p = p;
  c->pool = static_cast<char*>(kv_pool);
  c->ws = static_cast<char*>(workspace);
  c->len.assign(dims->max_slots, 0);
  c->relay_n.assign(dims->max_slots, 0);
  c->relay_len.assign(dims->max_slots, -1);

  rc = DFLASH_OK;
  if (!hip_ok(hipMemsetAsync(kv_pool, 0, p.pool_bytes, nullptr), "hipMemsetAsync(pool)", &rc) ||
      !hip_ok(hipMemsetAsync(workspace, 0, p.ws_bytes, nullptr), "hipMemsetAsync(workspace)", &rc)) {
    delete c;
    return rc;
  }
  const int half = dims->hd / 2;
  const int npos = dims->max_ctx + dims->B;
  const int total = npos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3(ceil_div(total, 256)), dim3(256), 0, nullptr,
                     reinterpret_cast<float2*>(c->pool + p.rope_off), npos, half, (double)dims->rope_base,
                     dims->hd);
  if (!hip_ok(hipGetLastError(), "rope table launch", &rc) ||
      !hip_ok(hipStreamSynchronize(nullptr), "hipStreamSynchronize", &rc)) {
    delete c;
    return rc;
  }
  *out = c;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->prof_events) (void)hipEventDestroy(e);
  delete ctx;
}

int dflash_profile_enable(dflash_ctx* ctx, uint32_t kind_mask, int32_t max_launches) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  if (kind_mask >> DFLASH_K_COUNT) return fail(DFLASH_EINVAL, "unknown kernel kind in mask");
  if (max_launches < 0 || max_launches > (1 << 20)) return fail(DFLASH_EINVAL, "max_launches out of range");
  ctx->prof_mask = 0;
  ctx->prof_recs.clear();
  const size_t need = kind_mask ? (size_t)max_launches * 2 : 0;
  int rc = DFLASH_OK;
  while (ctx->prof_events.size() < need) {
    hipEvent_t e;
    if (!hip_ok(hipEventCreate(&e), "hipEventCreate", &rc)) return rc;
    ctx->prof_events.push_back(e);
  }
  ctx->prof_mask = kind_mask;
  return DFLASH_OK;
}

int dflash_profile_read(dflash_ctx* ctx, double* total_ms, int32_t* launches) {
  g_last_error.clear();
  if (!ctx || !total_ms || !launches) return fail(DFLASH_EINVAL, "NULL argument");
  for (int k = 0; k < DFLASH_K_COUNT; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  int rc = DFLASH_OK;
  for (const ProfRec& r : ctx->prof_recs) {
    if (!hip_ok(hipEventSynchronize(r.b), "hipEventSynchronize", &rc)) return rc;
    float ms = 0.f;
    if (!hip_ok(hipEventElapsedTime(&ms, r.a, r.b), "hipEventElapsedTime", &rc)) return rc;
    total_ms[r.kind] += ms;
    launches[r.kind] += 1;
  }
  ctx->prof_recs.clear();
  return DFLASH_OK;
}

int dflash_slot_reset(dflash_ctx* ctx, int32_t slot, int32_t keep_len) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  if (slot < 0 || slot >= ctx->d.max_slots) return fail(DFLASH_ECAPACITY, "slot out of range");
  if (keep_len < 0 || keep_len > ctx->len[slot])
    return fail(DFLASH_EINVAL, "keep_len must be in 0..current length");
  ctx->len[slot] = keep_len;
  ctx->relay_n[slot] = 0;
  return DFLASH_OK;
}

int dflash_slot_len(const dflash_ctx* ctx, int32_t slot, int32_t* len) {
  g_last_error.clear();
  if (!ctx || !len) return fail(DFLASH_EINVAL, "NULL argument");
  if (slot < 0 || slot >= ctx->d.max_slots) return fail(DFLASH_ECAPACITY, "slot out of range");
  *len = ctx->len[slot];
  return DFLASH_OK;
}

static int check_slots(const dflash_ctx* ctx, int32_t n_req, const int32_t* slot) {
  if (n_req < 0) return fail(DFLASH_EINVAL, "n_req must be >= 0");
  if (n_req > ctx->d.max_batch) return fail(DFLASH_ECAPACITY, "n_req exceeds max_batch");
  if (n_req > 0 && !slot) return fail(DFLASH_EINVAL, "slot is NULL");
  for (int r = 0; r < n_req; ++r) {
    if (slot[r] < 0 || slot[r] >= ctx->d.max_slots) return fail(DFLASH_ECAPACITY, "slot out of range");
    for (int q = 0; q < r; ++q)
      if (slot[q] == slot[r]) return fail(DFLASH_EINVAL, "slots in one call must be distinct");
  }
  return DFLASH_OK;
}

int dflash_fuse_ctx(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* slot,
                    const int32_t* n_new, const void* const* tgt_hidden) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  int rc = check_slots(ctx, n_req, slot);
  if (rc) return rc;
  if (n_req > 0 && !n_new) return fail(DFLASH_EINVAL, "n_new is NULL");
  long long total = 0;
  for (int r = 0; r < n_req; ++r) {
    if (n_new[r] < 0) return fail(DFLASH_EINVAL, "n_new must be >= 0");
    if ((long long)ctx->len[slot[r]] + n_new[r] > ctx->d.max_ctx)
      return fail(DFLASH_ECAPACITY, "context would exceed max_ctx for slot " + std::to_string(slot[r]));
    total += n_new[r];
  }
  if (total == 0) return DFLASH_OK;
  if (total > (1LL << 30)) return fail(DFLASH_ECAPACITY, "too many rows in one call");
  if (!tgt_hidden) return fail(DFLASH_EINVAL, "tgt_hidden is NULL");
  for (int l = 0; l < ctx->d.L; ++l)
    if (!tgt_hidden[l]) return fail(DFLASH_EINVAL, "a tgt_hidden layer pointer is NULL");

  FuseMeta fm{};
  fm.n_req = n_req;
  int row = 0;
  for (int r = 0; r < n_req; ++r) {
    fm.row0[r] = row;
    fm.pos0[r] = ctx->len[slot[r]];
    fm.slot[r] = slot[r];
    row += n_new[r];
  }
  fm.row0[n_req] = row;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (ctx->d.dtype == DFLASH_BF16) run_fuse<bf16_t>(ctx, st, fm, (int)total, tgt_hidden);
  else run_fuse<float>(ctx, st, fm, (int)total, tgt_hidden);
  if (!hip_ok(hipGetLastError(), "fuse launch", &rc)) return rc;
  for (int r = 0; r < n_req; ++r) ctx->len[slot[r]] += n_new[r];
  return DFLASH_OK;
}

int dflash_draft_block(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* slot,
                       const int32_t* anchor, int32_t top_k, int32_t* out_ids, float* out_vals,
                       float* out_logits) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  int rc = check_slots(ctx, n_req, slot);
  if (rc) return rc;
  if (top_k < 1 || top_k > 16) return fail(DFLASH_EUNSUPPORTED, "top_k must be in 1..16");
  if (n_req == 0) return DFLASH_OK;
  if (!anchor || !out_ids) return fail(DFLASH_EINVAL, "anchor and out_ids must not be NULL");
  if (top_k > 1 && lm_small_lds(ctx->d) > kLdsMax)
    return fail(DFLASH_EUNSUPPORTED, "top_k > 1 needs 16 rows of D in LDS: D too large for this dtype");
  AttnPlan apl;
  plan_attention(ctx, n_req, slot, &apl);
  const int Mlm = n_req * (ctx->d.B - 1);
  if (lm_entries_for(Mlm, ctx->d.V, top_k) > ctx->p.lm_entries)
    return fail(DFLASH_ECAPACITY, "LM-head partial buffer too small");
  // DFlow relay rows of this round (stored at the slot's current length)
  DraftRelay rl{};
  bool any = false;
  for (int r = 0; r < n_req; ++r) {
    const int s = slot[r];
    rl.slot[r] = s;
    rl.n[r] = (ctx->relay_n[s] > 0 && ctx->relay_len[s] == ctx->len[s]) ? ctx->relay_n[s] : 0;
    any = any || rl.n[r] > 0;
  }
  rl.rows = any ? reinterpret_cast<const float*>(ctx->pool + ctx->p.relay_off) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (ctx->d.dtype == DFLASH_BF16)
    run_draft<bf16_t>(ctx, st, n_req, slot, anchor, top_k, out_ids, out_vals, out_logits, apl, rl);
  else
    run_draft<float>(ctx, st, n_req, slot, anchor, top_k, out_ids, out_vals, out_logits, apl, rl);
  if (!hip_ok(hipGetLastError(), "draft launch", &rc)) return rc;
  for (int r = 0; r < n_req; ++r) ctx->relay_n[slot[r]] = 0;  // a relay lives for one round
  ctx->last_draft_n = n_req;
  return DFLASH_OK;
}

int dflash_accept(void* stream, int32_t n_req, int32_t B, const int32_t* cand, int32_t cand_stride,
                  const int32_t* target, int32_t* tau, int32_t* bonus) {
  g_last_error.clear();
  if (n_req < 0) return fail(DFLASH_EINVAL, "n_req must be >= 0");
  if (B < 1) return fail(DFLASH_EINVAL, "B must be >= 1");
  if (cand_stride < 1) return fail(DFLASH_EINVAL, "cand_stride must be >= 1");
  if (n_req == 0) return DFLASH_OK;
  if (!cand || !target || !tau || !bonus) return fail(DFLASH_EINVAL, "NULL argument");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(accept_kernel, dim3(ceil_div(n_req, 64)), dim3(64), 0, st, n_req, B, cand,
                     cand_stride, target, tau, bonus);
  int rc = DFLASH_OK;
  if (!hip_ok(hipGetLastError(), "accept launch", &rc)) return rc;
  return DFLASH_OK;
}

int dflow_relay(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* slot, const int32_t* n_acc,
                const int32_t* cand, int32_t cand_stride, const int32_t* bonus,
                const void* const* tgt_hidden, const dflow_relay_weights* rw) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  int rc = check_slots(ctx, n_req, slot);
  if (rc) return rc;
  if (n_req == 0) return DFLASH_OK;
  if (!n_acc) return fail(DFLASH_EINVAL, "n_acc is NULL");
  const int B = ctx->d.B;
  long long total = 0;
  for (int r = 0; r < n_req; ++r) {
    if (n_acc[r] < 0 || n_acc[r] > B - 1) return fail(DFLASH_EINVAL, "n_acc must be in 0..B-1");
    total += std::max(0, B - 2 - n_acc[r]);
  }
  RelayMeta rm{};
  rm.n_req = n_req;
  int row = 0;
  for (int r = 0; r < n_req; ++r) {
    rm.row0[r] = row;
    rm.slot[r] = slot[r];
    rm.nacc[r] = n_acc[r];
    row += std::max(0, B - 2 - n_acc[r]);
  }
  rm.row0[n_req] = row;
  if (total > 0) {
    if (ctx->d.D > 4 * 256 * kRelayMaxPass) return fail(DFLASH_EUNSUPPORTED, "the relay needs D <= 16384");
    if (!cand || !bonus) return fail(DFLASH_EINVAL, "cand and bonus must not be NULL");
    if (cand_stride < 1) return fail(DFLASH_EINVAL, "cand_stride must be >= 1");
    if (!rw || !rw->w1 || !rw->w2) return fail(DFLASH_EINVAL, "relay weights must not be NULL");
    if (!tgt_hidden) return fail(DFLASH_EINVAL, "tgt_hidden is NULL");
    for (int l = 0; l < ctx->d.L; ++l)
      if (!tgt_hidden[l]) return fail(DFLASH_EINVAL, "a tgt_hidden layer pointer is NULL");
    if (total > ctx->p.relay_rows) return fail(DFLASH_ECAPACITY, "relay rows exceed max_batch * (B - 2)");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ctx->d.dtype == DFLASH_BF16)
      run_relay<bf16_t>(ctx, st, rm, (int)total, tgt_hidden, cand, cand_stride, bonus, rw);
    else
      run_relay<float>(ctx, st, rm, (int)total, tgt_hidden, cand, cand_stride, bonus, rw);
    if (!hip_ok(hipGetLastError(), "relay launch", &rc)) return rc;
  }
  for (int r = 0; r < n_req; ++r) {
    ctx->relay_n[slot[r]] = std::max(0, B - 2 - n_acc[r]);
    ctx->relay_len[slot[r]] = ctx->len[slot[r]];
  }
  return DFLASH_OK;
}

int dflow_read_relay(dflash_ctx* ctx, void* stream, int32_t slot, float* out, int32_t* count) {
  g_last_error.clear();
  if (!ctx || !out || !count) return fail(DFLASH_EINVAL, "NULL argument");
  if (slot < 0 || slot >= ctx->d.max_slots) return fail(DFLASH_ECAPACITY, "slot out of range");
  const int n = ctx->relay_len[slot] == ctx->len[slot] ? ctx->relay_n[slot] : 0;
  *count = n;
  if (n == 0) return DFLASH_OK;
  const size_t D = ctx->d.D;
  const float* src = reinterpret_cast<const float*>(ctx->pool + ctx->p.relay_off) + ((size_t)slot * ctx->d.B + 2) * D;
  int rc = DFLASH_OK;
  if (!hip_ok(hipMemcpyAsync(out + 2 * D, src, (size_t)n * D * sizeof(float), hipMemcpyDeviceToDevice,
                             static_cast<hipStream_t>(stream)),
              "relay read copy", &rc))
    return rc;
  return DFLASH_OK;
}

int dflash2_select(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* anchor, const int32_t* cand,
                   const float* cand_logits, int32_t k, const dflash2_selector_weights* sw, int32_t* out_path,
                   float* out_scores) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  if (n_req <= 0 || n_req != ctx->last_draft_n)
    return fail(DFLASH_EINVAL, "n_req must equal that of the most recent dflash_draft_block call");
  if (k < 1 || k > kSelMaxK) return fail(DFLASH_EUNSUPPORTED, "k must be in 1..16");
  if (ctx->d.B - 1 > kSelMaxT) return fail(DFLASH_EUNSUPPORTED, "B must be at most 16");
  if (!anchor || !cand || !cand_logits || !out_path) return fail(DFLASH_EINVAL, "NULL argument");
  if (!sw || !sw->a || !sw->b || !sw->w_h) return fail(DFLASH_EINVAL, "selector tables must not be NULL");
  if (sw->rank < 64 || sw->rank > 256 || sw->rank % 64) return fail(DFLASH_EUNSUPPORTED, "rank must be 64, 128, 192 or 256");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (ctx->d.dtype == DFLASH_BF16) run_select<bf16_t>(ctx, st, n_req, anchor, cand, cand_logits, k, sw, out_path, out_scores);
  else run_select<float>(ctx, st, n_req, anchor, cand, cand_logits, k, sw, out_path, out_scores);
  int rc = DFLASH_OK;
  if (!hip_ok(hipGetLastError(), "select launch", &rc)) return rc;
  return DFLASH_OK;
}

int dflash2_conv_attach(dflash_ctx* ctx, const dflash2_conv_layer* layers) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  if (!layers) {
    ctx->conv.clear();
    return DFLASH_OK;
  }
  if (ctx->d.D % 256) return fail(DFLASH_EUNSUPPORTED, "the two-tap convolution needs D % 256 == 0");
  for (int l = 0; l < ctx->d.N; ++l) {
    const dflash2_conv_site* s[4] = {&layers[l].attn_in, &layers[l].attn_out, &layers[l].ffn_in, &layers[l].ffn_out};
    for (const dflash2_conv_site* x : s)
      if (!x->w || !x->kbase) return fail(DFLASH_EINVAL, "convolution tensors must not be NULL");
  }
  ctx->conv.assign(layers, layers + ctx->d.N);
  return DFLASH_OK;
}

namespace {

// Shared checks of the two sampling calls; fills the workspace view and the
// scale factors.
int spec_prep(dflash_ctx* ctx, int32_t n_req, float temperature, const int32_t* req_id, SsWork* w, float* s2) {
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  if (n_req < 0) return fail(DFLASH_EINVAL, "n_req must be >= 0");
  if (n_req > ctx->d.max_batch) return fail(DFLASH_ECAPACITY, "n_req exceeds max_batch");
  if (!(temperature >= 1e-4f && temperature <= 1e4f))
    return fail(DFLASH_EINVAL, "temperature must be in [1e-4, 1e4]");
  if (n_req > 0 && !req_id) return fail(DFLASH_EINVAL, "req_id is NULL");
  if (ceil_div(ctx->d.V, kSsBlock) > kSsMaxBlocks) return fail(DFLASH_EUNSUPPORTED, "sampling needs V <= 1048576");
  const Plan& p = ctx->p;
  w->part = ctx->wsp<float4>(p.ss_part_off);
  w->lse = ctx->wsp<float>(p.ss_lse_off);
  w->nacc = ctx->wsp<int>(p.ss_nacc_off);
  w->row_ctr = ctx->wsp<int>(p.ss_rctr_off);
  w->req_ctr = ctx->wsp<int>(p.ss_qctr_off);
  w->blk = ctx->wsp<int>(p.ss_blk_off);
  *s2 = (float)(1.4426950408889634 / (double)temperature);  // log2(e) / T
  return DFLASH_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Element loads where a row is not 16-byte aligned.
#define SS_LAUNCH(KERNEL, VEC, GRID, ST, ...)                                             \
  do {                                                                                  \
    if (VEC)                                                                            \
      hipLaunchKernelGGL((KERNEL<true>), GRID, dim3(kSsThreads), 0, ST, __VA_ARGS__);   \
    else                                                                                \
      hipLaunchKernelGGL((KERNEL<false>), GRID, dim3(kSsThreads), 0, ST, __VA_ARGS__);  \
  } while (0)

// Piece size of a block-mass pass (entries per thread): the largest piece that
// still gives one work-group per CU over `rows` rows (each work-group holds
// its slot until its ticket returns: fewer, larger pieces waste less).
int ss_mass_per(int V, int rows) {
  for (int per : {64, 16})
    if ((long long)rows * ceil_div(V, kSsThreads * per) >= 256) return per;
  return 8;
}

#define SS_MASS(KERNEL, VEC, PER, ROWS, ST, ...)                                                              \
  do {                                                                                                       \
    const int np_ = ceil_div(V, kSsThreads * (PER));                                                         \
    const dim3 g_(np_, ROWS), b_(kSsThreads);                                                                \
    if ((PER) == 64) {                                                                                       \
      if (VEC) hipLaunchKernelGGL((KERNEL<true, 64>), g_, b_, 0, ST, __VA_ARGS__);                           \
      else hipLaunchKernelGGL((KERNEL<false, 64>), g_, b_, 0, ST, __VA_ARGS__);                              \
    } else if ((PER) == 16) {                                                                                \
      if (VEC) hipLaunchKernelGGL((KERNEL<true, 16>), g_, b_, 0, ST, __VA_ARGS__);                           \
      else hipLaunchKernelGGL((KERNEL<false, 16>), g_, b_, 0, ST, __VA_ARGS__);                              \
    } else {                                                                                                 \
      if (VEC) hipLaunchKernelGGL((KERNEL<true, 8>), g_, b_, 0, ST, __VA_ARGS__);                            \
      else hipLaunchKernelGGL((KERNEL<false, 8>), g_, b_, 0, ST, __VA_ARGS__);                               \
    }                                                                                                        \
  } while (0)

}  // namespace

}  // extern "C"

namespace {

// The two drafting kernels (block masses with the block choice, then the
// Gumbel-max within the chosen block) over n_req * K rows, on scratch `w`
// (part, row_ctr with zero tickets, blk).
void launch_spec_draft(const SsWork& w, hipStream_t st, int n_req, int V, int K, const float* draft_logits,
                       float s2, uint64_t seed, const int32_t* req_id, int32_t* cand, float* draft_lse) {
  const bool vec = V % 4 == 0 && aligned16(draft_logits);
  const int per = ss_mass_per(V, n_req * K);
  const int np = ceil_div(V, kSsThreads * per);
  SS_MASS(ss_draft_mass_kernel, vec, per, n_req * K, st, draft_logits, V, K, np, s2, seed, req_id, w, draft_lse);
  const dim3 g(kSsPickParts, n_req * K), b(kSsThreads);
  if (vec)
    hipLaunchKernelGGL((ss_pick_kernel<true, false>), g, b, 0, st, draft_logits, nullptr, nullptr, V, K, s2, seed,
                       req_id, w, cand, nullptr);
  else
    hipLaunchKernelGGL((ss_pick_kernel<false, false>), g, b, 0, st, draft_logits, nullptr, nullptr, V, K, s2, seed,
                       req_id, w, cand, nullptr);
}

// Scratch of dflash_spec_draft_static, for callers that cannot allocate: the
// per-piece partials of up to kStaticRows drafted rows (pieces of 2048 ids,
// up to kStaticMaxV ids), the row tickets and the chosen blocks.  Each GPU
// holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns on that device.
constexpr int kStaticMaxV = 262144;
constexpr int kStaticRows = kMaxReq * 15;  // n_req <= 64, B <= 16
constexpr int kStaticPieces = kStaticMaxV / (kSsThreads * 8);
constexpr size_t kStaticPartBytes = (size_t)kStaticRows * kStaticPieces * sizeof(float4);
constexpr size_t kStaticBytes = kStaticPartBytes + 2 * (size_t)kStaticRows * sizeof(int);
constexpr int kMaxDevices = 64;
static_assert(kStaticPieces >= kSsPickParts, "block-draw parts fit the per-row partial slots");

std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

static __device__ __align__(256) char scratch[kStaticBytes];

extern "C" {

int dflash_spec_draft(dflash_ctx* ctx, void* stream, int32_t n_req, const float* draft_logits, float temperature,
                      uint64_t seed, const int32_t* req_id, int32_t* cand, float* draft_lse) {
  g_last_error.clear();
  SsWork w;
  float s2;
  int rc = spec_prep(ctx, n_req, temperature, req_id, &w, &s2);
  if (rc) return rc;
  if (n_req == 0) return DFLASH_OK;
  if (!draft_logits || !cand) return fail(DFLASH_EINVAL, "NULL argument");
  hipStream_t st = static_cast<hipStream_t>(stream);
  {
    ProfScope ps(ctx, DFLASH_K_SPEC_DRAFT, st);
    launch_spec_draft(w, st, n_req, ctx->d.V, ctx->d.B - 1, draft_logits, s2, seed, req_id, cand, draft_lse);
  }
  if (!hip_ok(hipGetLastError(), "spec_draft launch", &rc)) return rc;
  return DFLASH_OK;
}

int dflash_spec_draft_static(void* stream, int32_t n_req, int32_t V, int32_t B, const float* draft_logits,
                             float temperature, uint64_t seed, const int32_t* req_id, int32_t* cand,
                             float* draft_lse) {
  g_last_error.clear();
  if (n_req < 0) return fail(DFLASH_EINVAL, "n_req must be >= 0");
  if (n_req > kMaxReq) return fail(DFLASH_ECAPACITY, "n_req exceeds 64 (the static scratch holds 64 x 15 rows)");
  if (B < 2 || B > 16) return fail(DFLASH_EUNSUPPORTED, "block size must be in 2..16");
  if (V < 1) return fail(DFLASH_EINVAL, "V must be >= 1");
  if (V > kStaticMaxV) return fail(DFLASH_ECAPACITY, "V exceeds 262144 (the static scratch limit)");
  if (!(temperature >= 1e-4f && temperature <= 1e4f))
    return fail(DFLASH_EINVAL, "temperature must be in [1e-4, 1e4]");
  if (n_req == 0) return DFLASH_OK;
  if (!draft_logits || !cand || !req_id) return fail(DFLASH_EINVAL, "NULL argument");
  int rc = DFLASH_OK;
  int dev = -1;
  if (!hip_ok(hipGetDevice(&dev), "hipGetDevice", &rc)) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_EUNSUPPORTED, "device index beyond 63");
  char* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
      void* p = nullptr;
      if (!hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)", &rc)) return rc;
      g_scratch_dev[dev] = static_cast<char*>(p);
    }
    base = g_scratch_dev[dev];
  }
  SsWork w{};
  w.part = reinterpret_cast<float4*>(base);
  w.row_ctr = reinterpret_cast<int*>(base + kStaticPartBytes);
  w.blk = w.row_ctr + kStaticRows;
  const int K = B - 1, rows = n_req * K;
  const float s2 = (float)(1.4426950408889634 / (double)temperature);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the array keeps the previous call's contents: the tickets start at zero here
  hipLaunchKernelGGL(zero_ints_kernel, dim3(ceil_div(rows, 256)), dim3(256), 0, st, w.row_ctr, rows);
  launch_spec_draft(w, st, n_req, V, K, draft_logits, s2, seed, req_id, cand, draft_lse);
  if (!hip_ok(hipGetLastError(), "spec_draft_static launch", &rc)) return rc;
  return DFLASH_OK;
}

int dflash_spec_verify(dflash_ctx* ctx, void* stream, int32_t n_req, const float* draft_logits,
                       const float* target_logits, const int32_t* cand, const float* draft_lse, float temperature,
                       uint64_t seed, const int32_t* req_id, int32_t* tokens, int32_t* tau) {
  g_last_error.clear();
  SsWork w;
  float s2;
  int rc = spec_prep(ctx, n_req, temperature, req_id, &w, &s2);
  if (rc) return rc;
  if (n_req == 0) return DFLASH_OK;
  if (!draft_logits || !target_logits || !cand || !tokens || !tau) return fail(DFLASH_EINVAL, "NULL argument");
  const int V = ctx->d.V, K = ctx->d.B - 1;
  const bool vec = V % 4 == 0 && aligned16(draft_logits) && aligned16(target_logits);
  const int rows = n_req * (draft_lse ? K + 1 : 2 * K + 1);
  hipStream_t st = static_cast<hipStream_t>(stream);
  {
    ProfScope ps(ctx, DFLASH_K_SPEC_STATS, st);
    const int nch = ceil_div(V, kSsBlock);
    SS_LAUNCH(ss_stats_kernel, vec, dim3(nch, rows), st, draft_logits, target_logits, cand, draft_lse, V, K, nch, s2,
              seed, req_id, w, tokens);
  }
  if (!hip_ok(hipGetLastError(), "spec_verify stats launch", &rc)) return rc;
  {
    ProfScope ps(ctx, DFLASH_K_SPEC_RESAMPLE, st);
    const int per = ss_mass_per(V, n_req);
    const int np = ceil_div(V, kSsThreads * per);
    SS_MASS(ss_resample_mass_kernel, vec, per, n_req, st, draft_logits, target_logits, draft_lse, V, K, np, s2, seed,
            req_id, w);
    const dim3 g(kSsPickParts, n_req), b(kSsThreads);
    if (vec)
      hipLaunchKernelGGL((ss_pick_kernel<true, true>), g, b, 0, st, draft_logits, target_logits, draft_lse, V, K, s2,
                         seed, req_id, w, tokens, tau);
    else
      hipLaunchKernelGGL((ss_pick_kernel<false, true>), g, b, 0, st, draft_logits, target_logits, draft_lse, V, K, s2,
                         seed, req_id, w, tokens, tau);
  }
  if (!hip_ok(hipGetLastError(), "spec_verify resample launch", &rc)) return rc;
  return DFLASH_OK;
}

int dflash_read_cache(dflash_ctx* ctx, void* stream, int32_t slot, int32_t layer, int32_t pos0, int32_t n,
                      float* k_out, float* v_out) {
  g_last_error.clear();
  if (!ctx || !k_out || !v_out) return fail(DFLASH_EINVAL, "NULL argument");
  if (slot < 0 || slot >= ctx->d.max_slots) return fail(DFLASH_ECAPACITY, "slot out of range");
  if (layer < 0 || layer >= ctx->d.N) return fail(DFLASH_EINVAL, "layer out of range");
  if (pos0 < 0 || n < 0 || pos0 + n > ctx->len[slot]) return fail(DFLASH_EINVAL, "range beyond slot length");
  if (n == 0) return DFLASH_OK;
  const Plan& p = ctx->p;
  const size_t e = elt_size(ctx->d.dtype);
  const char* base = ctx->pool + p.kv_off + (slot * p.slot_stride + layer * p.layer_stride) * e;
  const int total = ctx->d.Hkv * n * ctx->d.hd;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (ctx->d.dtype == DFLASH_BF16)
    hipLaunchKernelGGL(read_cache_kernel<bf16_t>, dim3(ceil_div(total, 256)), dim3(256), 0, st,
                       reinterpret_cast<const bf16_t*>(base),
                       reinterpret_cast<const bf16_t*>(base + p.kv_stride * e), p.head_stride,
                       ctx->d.hd, ctx->d.Hkv, pos0, n, k_out, v_out);
  else
    hipLaunchKernelGGL(read_cache_kernel<float>, dim3(ceil_div(total, 256)), dim3(256), 0, st,
                       reinterpret_cast<const float*>(base),
                       reinterpret_cast<const float*>(base + p.kv_stride * e), p.head_stride,
                       ctx->d.hd, ctx->d.Hkv, pos0, n, k_out, v_out);
  int rc = DFLASH_OK;
  if (!hip_ok(hipGetLastError(), "read_cache launch", &rc)) return rc;
  return DFLASH_OK;
}

}  // extern "C"
