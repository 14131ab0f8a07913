/*
 * dflash_fuse.h -- C ABI of the DFlash block-diffusion draft step on MI355X
 * (gfx950).
 *
 * The draft step has three parts, each one entry point:
 *
 *   dflash_fuse_ctx     target-context fusion H_c = RMSNorm(W_c [H^(l1);...;H^(lL)])
 *                       followed by the per-layer context projections
 *                       K_c = RoPE(W_c^K H_c), V_c = W_c^V H_c, appended to a
 *                       per-request cache ("DFlash 投机解码：块扩散草稿与 KV 注入",
 *                       section 三 fusion equation; section 二 "注意力模式" for
 *                       K_c/V_c; section 四 engineering note: the cache holds
 *                       projected K/V, not raw H_c).
 *   dflash_draft_block  one forward pass of the N drafter layers over the block
 *                       [anchor, mask x (B-1)]: queries from the block only,
 *                       keys/values [K_c; K_b] / [V_c; V_b], no mask, SwiGLU FFN,
 *                       then the shared LM head with per-position top-k over
 *                       block offsets 1..B-1 (same page, section 二 and the
 *                       draft_forward / dflash_cycle pseudocode of section 四).
 *   dflash_accept       greedy verification: longest prefix of candidates that
 *                       match the verifier's argmax tokens, plus the bonus token;
 *                       tau counts the bonus, 1 <= tau <= B (same page, notation
 *                       table and section 四; "DFlow 完全拆解", opening section).
 *
 * Conventions
 *   - Pointers are device pointers unless marked [host].
 *   - Storage dtype is DFLASH_F32 (float) or DFLASH_BF16 (uint16_t bit
 *     patterns, round-to-nearest-even).  Weights, RMSNorm gains and verifier
 *     hidden states use the storage dtype; accumulation is always fp32 and the
 *     residual stream is fp32.
 *   - Every matrix is [out, in] row-major (the input index is contiguous).
 *   - Ownership: all device memory (weights, the KV pool, the workspace,
 *     inputs and outputs) belongs to the caller.  The library borrows the
 *     weight, pool and workspace pointers for the lifetime of a dflash_ctx and
 *     never allocates or frees device memory.
 *   - Calls are asynchronous and ordered on the given stream (a hipStream_t
 *     passed as void*; NULL is the default stream).  Kernel faults surface at
 *     the caller's next synchronisation.
 *   - Errors: every argument is validated before the first launch, so a call
 *     that returns an error has enqueued nothing and changed no state.
 *   - A dflash_ctx is not thread-safe; calls that share a ctx must be ordered
 *     on one stream.
 */
#ifndef DFLASH_FUSE_H
#define DFLASH_FUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dflash_dtype { DFLASH_F32 = 0, DFLASH_BF16 = 1 };

enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1,       /* null pointer, bad dimension or argument */
  DFLASH_EUNSUPPORTED = -2, /* head_dim not 64/128, B > 16, top_k > 16, dtype */
  DFLASH_ECAPACITY = -3,    /* slot out of range, context overflow, batch or buffer too small */
  DFLASH_EHIP = -4          /* a HIP runtime call failed; see dflash_last_error() */
};

/* Model and capacity description. */
typedef struct dflash_dims {
  int32_t dtype;      /* enum dflash_dtype */
  int32_t D;          /* drafter hidden size */
  int32_t L;          /* number of tapped target layers */
  int32_t Dt;         /* target hidden size per tapped layer */
  int32_t N;          /* drafter layers (<= 16) */
  int32_t Hq;         /* query heads */
  int32_t Hkv;        /* key/value heads (Hq % Hkv == 0) */
  int32_t hd;         /* head dim: 64 or 128 */
  int32_t I;          /* SwiGLU intermediate size */
  int32_t V;          /* vocabulary size */
  int32_t B;          /* block size: anchor + (B-1) masks, 2..16 */
  int32_t max_ctx;    /* context capacity per slot (fused tokens) */
  int32_t max_slots;  /* number of request slots in the KV pool */
  int32_t max_batch;  /* requests per call, 1..64 */
  float rope_base;    /* RoPE base (e.g. 10000) */
  float rms_eps;      /* RMSNorm epsilon (e.g. 1e-6) */
  int32_t use_rope;   /* 1: rotate Q and K (rotate-half pairing), 0: no positions */
} dflash_dims;

/* Per-layer weights.  Shapes ([out, in]):
 *   g_attn [D], w_q [Hq*hd, D], w_kb [Hkv*hd, D], w_vb [Hkv*hd, D],
 *   w_kc [Hkv*hd, D], w_vc [Hkv*hd, D], w_o [D, Hq*hd],
 *   g_ffn [D], w_gate [I, D], w_up [I, D], w_down [D, I].
 * w_kc / w_vc project the fused context, w_kb / w_vb the block; they may alias. */
typedef struct dflash_layer_weights {
  const void* g_attn;
  const void* w_q;
  const void* w_kb;
  const void* w_vb;
  const void* w_kc;
  const void* w_vc;
  const void* w_o;
  const void* g_ffn;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} dflash_layer_weights;

/* Model weights.  w_c [D, L*Dt] (fusion projection; the L tapped layers are
 * concatenated along its input axis), g_c [D], embed [V, D] (token
 * embedding), e_mask [D] (shared mask embedding), g_final [D], w_lm [V, D]
 * (shared LM head; may alias embed).  `layers` is a [host] array of N
 * entries, copied at dflash_create. */
typedef struct dflash_weights {
  const void* w_c;
  const void* g_c;
  const void* embed;
  const void* e_mask;
  const void* g_final;
  const void* w_lm;
  const dflash_layer_weights* layers;
} dflash_weights;

typedef struct dflash_ctx dflash_ctx;

/* Byte sizes of the two caller-allocated device buffers for `dims`: the KV
 * pool (projected context K/V of every slot and the RoPE table; persistent)
 * and the workspace (per-call scratch, sized for dims->max_batch requests per
 * call: the batch capacity is part of the dims, so that dflash_create checks
 * the buffers against the same figure).  Pure host computation.  Returns
 * DFLASH_OK or DFLASH_EINVAL / DFLASH_EUNSUPPORTED. */
int dflash_query_sizes(const dflash_dims* dims, size_t* kv_pool_bytes, size_t* workspace_bytes);

/* Create a context over caller-owned buffers.  kv_pool and workspace must be
 * 256-byte aligned and at least the sizes dflash_query_sizes reports.  Clears
 * both buffers and fills the RoPE table on the default stream, then waits.
 * All slots start empty (length 0). */
int dflash_create(const dflash_dims* dims, const dflash_weights* weights, void* kv_pool,
                  size_t kv_pool_bytes, void* workspace, size_t workspace_bytes,
                  dflash_ctx** out);

void dflash_destroy(dflash_ctx* ctx);

/* Context fusion and cache append.
 *   slot [host, n_req]    distinct slot ids in 0..max_slots-1
 *   n_new [host, n_req]   new verifier rows per request (>= 0)
 *   tgt_hidden [host, L]  L device pointers, each [sum(n_new), Dt] in the
 *                         storage dtype; rows grouped by request in `slot` order.
 * Request r's rows are fused and their K/V written at absolute positions
 * len(slot[r]) .. len(slot[r]) + n_new[r] - 1; then len(slot[r]) += n_new[r].
 * ECAPACITY if a slot would exceed max_ctx.  Uses the workspace: calls that
 * share a ctx must not overlap. */
int dflash_fuse_ctx(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* slot,
                    const int32_t* n_new, const void* const* tgt_hidden);

/* Draft one block per request.
 *   slot [host, n_req]     slot ids (distinct); the block of request r sits at
 *                          absolute positions len(slot[r]) .. + B-1
 *   anchor [n_req] int32   anchor token per request (device); the anchors are
 *                          read by a kernel, so an id outside 0..V-1 cannot be
 *                          reported as an error: it is clamped into 0..V-1
 *                          (the caller is responsible for valid ids)
 *   top_k                  1..16; top_k > 1 stages 16 rows of D in one CU's
 *                          LDS (16 * (D * elt + 16) bytes <= 160 KB, so D <= 5056
 *                          for bf16 and D <= 2496 for fp32; EUNSUPPORTED
 *                          beyond)
 *   out_ids [n_req, B-1, top_k] int32: per block offset 1..B-1, ids ordered by
 *                          (logit descending, id ascending)
 *   out_vals  nullable [n_req, B-1, top_k] float: the matching logits
 *   out_logits nullable [n_req, B-1, V] float: all logits (debug)
 * Slot lengths are not changed: the block's own K/V are transient.
 * Relay rows stored for a slot by dflow_relay at the slot's current length
 * replace the mask embedding at their block offsets; every slot of the call
 * then has its relay cleared (the relay lives for one round). */
int dflash_draft_block(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* slot,
                       const int32_t* anchor, int32_t top_k, int32_t* out_ids,
                       float* out_vals, float* out_logits);

/* Greedy acceptance (stateless).
 *   cand [n_req, B-1] int32 with row stride cand_stride (>= 1) between block
 *        offsets (pass top_k to read the top-1 column of out_ids)
 *   target [n_req, B] int32: target[r][j] is the verifier's argmax after block
 *        offset j (j = 0 is the anchor)
 *   tau [n_req] int32 out:  n + 1 where n counts leading j with
 *        cand[r][j] == target[r][j]
 *   bonus [n_req] int32 out: target[r][n], the next anchor */
int dflash_accept(void* stream, int32_t n_req, int32_t B, const int32_t* cand,
                  int32_t cand_stride, const int32_t* target, int32_t* tau, int32_t* bonus);

/* Rewind (or confirm) a slot: set its length to keep_len <= current length
 * ("DFlash 投机解码：块扩散草稿与 KV 注入", section 四: after verification the
 * draft cache is rolled back to the committed prefix, rewind_kv in the
 * dflash_cycle pseudocode).  Host-side bookkeeping only; cached entries past
 * keep_len are ignored and overwritten by later appends; a stored DFlow relay
 * of the slot is dropped. */
int dflash_slot_reset(dflash_ctx* ctx, int32_t slot, int32_t keep_len);

/* Current fused length of a slot. */
int dflash_slot_len(const dflash_ctx* ctx, int32_t slot, int32_t* len);

/* Copy the cached context keys and values of one slot and drafter layer,
 * positions pos0 .. pos0+n-1 (all < the slot's length), into k_out / v_out,
 * each [Hkv, n, hd] float (device).  Keys are stored already rotated at
 * their absolute positions.  For inspection and tests. */
int dflash_read_cache(dflash_ctx* ctx, void* stream, int32_t slot, int32_t layer, int32_t pos0,
                      int32_t n, float* k_out, float* v_out);

/* DFlow relay weights (storage dtype, row-major [out, in]): the two bias-free
 * layers of the relay MLP with a SiLU between them.
 *   w1 [D, 3D]  over the concatenation [E(bonus); E(first rejection); h]
 *   w2 [2D, D]  rows 0..D-1 give beta, rows D..2D-1 give gamma */
typedef struct dflow_relay_weights {
  const void* w1;
  const void* w2;
} dflow_relay_weights;

/* DFlow relay of the rejected suffix ("DFlow 完全拆解", relay steps 1-3 and the
 * inference-loop section).  Call after the round's committed rows have been
 * fused (dflash_fuse_ctx), so that each slot's length is the position of its
 * next anchor (the bonus token).  For request r of the round just verified,
 * with n = n_acc[r] accepted candidates (0..B-1), the reusable suffix is block
 * offsets n+2 .. B-1 (the first rejection, offset n+1, is not reused):
 * k_r = max(0, B-2-n) rows.  For each such row the verifier features h are
 * projected with the shared W_c and RMSNorm (the fusion step), then
 *   [beta; gamma] = w2 SiLU(w1 [E(bonus[r]); E(cand[r][n]); h])
 *   x = e_mask + beta * LN(h) + gamma      (LN: no affine, eps 1e-5)
 * and x is stored for the slot's next block at offset 2 .. B-1-n (the state of
 * offset o serves the prediction of the next position, which is next-block
 * offset o - n).  A request with k_r = 0 only clears its slot's relay.
 *   slot [host, n_req]    distinct slot ids
 *   n_acc [host, n_req]   accepted candidates of the round, 0..B-1
 *   cand [n_req, B-1] int32 (device) with row stride cand_stride: the round's
 *                         candidates (cand[r][n] is the first rejection)
 *   bonus [n_req] int32 (device): the bonus tokens
 *   tgt_hidden [host, L]  L device pointers, each [sum(k_r), Dt] in the storage
 *                         dtype: verifier features of offsets n+2..B-1, grouped
 *                         by request, in offset order (may be NULL if all
 *                         k_r = 0)
 *   rw                    relay MLP weights
 * Stored rows are bound to the slot and its current length: the next
 * dflash_draft_block on the slot at that length uses them; a draft at another
 * length, dflash_slot_reset or the next dflow_relay drops them.  Uses the
 * workspace.  Requires D <= 16384 (EUNSUPPORTED otherwise). */
int dflow_relay(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* slot, const int32_t* n_acc,
                const int32_t* cand, int32_t cand_stride, const int32_t* bonus,
                const void* const* tgt_hidden, const dflow_relay_weights* rw);

/* Copy the relay rows currently stored for a slot into out [B, D] float
 * (device; row j is block offset j, rows without relay are left untouched)
 * and return their count in *count [host] (they occupy offsets 2..count+1).
 * For inspection and tests. */
int dflow_read_relay(dflash_ctx* ctx, void* stream, int32_t slot, float* out, int32_t* count);

/* DFlash 2 path-selector tables (storage dtype, row-major).
 *   a   [V, rank]  compact embedding of the previous token
 *   b   [V, rank]  compact embedding of the next token
 *   w_h [rank, D]  gate projection: H(h) = sigmoid(w_h h)
 *   rank           a multiple of 64, at most 256 */
typedef struct dflash2_selector_weights {
  const void* a;
  const void* b;
  const void* w_h;
  int32_t rank;
} dflash2_selector_weights;

/* DFlash 2 path selector ("DFlash 2：正确 token 已在候选里", the first-insight
 * section).  For request r and drafted position t (block offset t, 1..B-1)
 * with candidates c_t[0..k-1] and their drafter logits U_t, every adjacent
 * pair is scored
 *   S_t(a, b) = U_t(b) + < a_tab[a] * H(h_t), b_tab[b] >,  H(h) = sigmoid(w_h h)
 * where h_t is the final normed hidden state of position t and a runs over
 * c_{t-1} (over the anchor alone for t = 1); then the greedy walk takes
 * y_1 = argmax_b S_1(anchor, b), y_t = argmax_b S_t(y_{t-1}, b) (ties to the
 * lower rank).  h_t comes from the most recent dflash_draft_block call on this
 * ctx, which must have had the same n_req (same request order); later
 * dflash_fuse_ctx / dflow_relay calls do not disturb it.
 *   anchor [n_req] int32 (device)
 *   cand [n_req, B-1, k] int32 (device), k in 1..16, rank order per position
 *   cand_logits [n_req, B-1, k] float (device): U_t of those candidates
 *   out_path [n_req, B-1] int32 (device): the chosen token per position
 *   out_scores nullable [n_req, B-1, k, k] float (device): S_t(c_{t-1}[i], c_t[j])
 *              at [t-1][i][j]; for t = 1 every row i holds S_1(anchor, c_1[j]). */
int dflash2_select(dflash_ctx* ctx, void* stream, int32_t n_req, const int32_t* anchor, const int32_t* cand,
                   const float* cand_logits, int32_t k, const dflash2_selector_weights* sw, int32_t* out_path,
                   float* out_scores);

/* DFlash 2 two-tap dynamic convolution weights of one site (storage dtype,
 * row-major):
 *   w     [2 * D/16, D]  rows 0..D/16-1: W_0 (current-row tap correction),
 *                        rows D/16..2*D/16-1: W_1 (left-row tap correction)
 *   kbase [2, D]         base kernels of the current and the left tap */
typedef struct dflash2_conv_site {
  const void* w;
  const void* kbase;
} dflash2_conv_site;

/* The four sites of one drafter layer: the normed attention input, the
 * attention output (after w_o) before its residual add, the normed FFN input,
 * and the FFN output (after w_down) before its residual add. */
typedef struct dflash2_conv_layer {
  dflash2_conv_site attn_in;
  dflash2_conv_site attn_out;
  dflash2_conv_site ffn_in;
  dflash2_conv_site ffn_out;
} dflash2_conv_layer;

/* DFlash 2 two-tap dynamic depthwise convolution ("DFlash 2：正确 token 已在候选里",
 * the second-insight section).  Attaches (layers != NULL: a [host] array of N
 * entries, copied; the device tensors must outlive the attachment) or detaches
 * (layers == NULL) the convolution.  While attached, every dflash_draft_block
 * applies at each site, along the block offsets t = 0..B-1 of every request,
 *   y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1},
 *   k_{t,j}[c] = kbase[j][c] + (W_j x_t)[c / 16],   x_{-1} = 0,
 * where x is the site's input (the anchor at offset 0 is the last verified
 * token; the first drafted offset reads it).  Requires D % 256 == 0
 * (EUNSUPPORTED otherwise); EINVAL on a NULL tensor.  Host-only call: no
 * device work, takes effect from the next draft. */
int dflash2_conv_attach(dflash_ctx* ctx, const dflash2_conv_layer* layers);

/* Speculative sampling at temperature T > 0 (lossless rejection sampling:
 * "DFlash 2：正确 token 已在候选里", introduction and selector section, where
 * outputs stay lossless because rejection sampling restores the verifier's
 * distribution; "DFlash 投机解码：块扩散草稿与 KV 注入", section 四, where the
 * rejected position is redrawn and the last position yields the bonus token).
 * Both models' distributions are softmax(logits / T), untruncated.  K = B - 1.
 *
 * Every categorical draw below ("draw v ~ w") is exact and taken in two
 * stages: the vocabulary is cut into blocks of 16384 consecutive ids; a block
 * b is chosen by inverse CDF over the block masses with one uniform u
 * (cum_{b-1} <= u S < cum_b), then the id within b that maximises
 * log w_v + G_v, G_v = -log(-log u_v) (ties to the lower id).  So
 * P(v) = w_v / S, with generator output for one block per draw.  V is at
 * most 1048576 (EUNSUPPORTED otherwise).
 *
 * Random numbers come from Philox4x64-10 (Salmon et al., SC 2011) with key
 * (seed, stream) and counter (v / 8, row, req_id[r], 0); entry v takes the top
 * 24 bits k of the high (v even) or low (v odd) 32-bit half of output word
 * (v % 8) / 2, as u = (k + 0.5) 2^-24.  Streams: 0 drafting noise G (row =
 * offset - 1, v = token id), 1 acceptance (row 0, v = offset - 1),
 * 2 replacement / bonus noise G (row 0, v = token id), 3 and 4 the block
 * choice of drafting (row = offset - 1) and of the replacement / bonus (row
 * 0), v = 0.  A caller advances `seed` per block so that blocks draw afresh;
 * req_id tells requests of one call apart.
 *
 * Both calls use the ctx workspace (calls sharing a ctx must be ordered on one
 * stream) and leave slot state untouched.  temperature must lie in
 * [1e-4, 1e4] (EINVAL); n_req <= max_batch (ECAPACITY).  Logit rows must hold
 * at least one finite value.  All pointers are device pointers. */

/* Draft: cand[r][j-1] ~ softmax(draft_logits[r][j-1] / T), drawn as above
 * (block from stream 3, noise from stream 0).
 *   draft_logits [n_req, B-1, V] float (e.g. out_logits of dflash_draft_block)
 *   req_id [n_req] int32 >= 0
 *   cand [n_req, B-1] int32 out
 *   draft_lse nullable [n_req, B-1] float out: log2 sum_v 2^(l_v log2(e) / T)
 *             of each row, for dflash_spec_verify at the same temperature */
int dflash_spec_draft(dflash_ctx* ctx, void* stream, int32_t n_req, const float* draft_logits, float temperature,
                      uint64_t seed, const int32_t* req_id, int32_t* cand, float* draft_lse);

/* Drafting as dflash_spec_draft, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no ctx and no workspace.  The kernels' scratch (per-piece
 * partials, row tickets, chosen blocks) is a fixed array of about 2 MB that
 * each GPU holds for the life of the process; the call allocates nothing.
 * Sizes come as arguments: n_req <= 64 (ECAPACITY beyond), B in 2..16
 * (EUNSUPPORTED), V in 1..262144 (ECAPACITY beyond).  Same draws, same
 * outputs as dflash_spec_draft on a ctx of the same V and B.  The scratch
 * serves the current device, which must be the device of `stream`; every call
 * on one GPU shares it, so calls on one GPU must not overlap (order them on
 * one stream): overlapping calls race.  Each call clears the tickets it uses
 * before its kernels run.
 *   draft_logits [n_req, B-1, V] float, req_id [n_req] int32 >= 0,
 *   cand [n_req, B-1] int32 out, draft_lse nullable [n_req, B-1] float out. */
int dflash_spec_draft_static(void* stream, int32_t n_req, int32_t V, int32_t B, const float* draft_logits,
                             float temperature, uint64_t seed, const int32_t* req_id, int32_t* cand,
                             float* draft_lse);

/* Verify one block per request by the rejection rule of speculative sampling.
 * q_j = softmax(draft_logits[r][j-1] / T) drafted offset j = 1..K;
 * p_j = softmax(target_logits[r][j] / T) is the verifier's distribution of the
 * token after offset j (j = 0: after the anchor).  Walking j = 1..K, x_j =
 * cand[r][j-1] is kept when u_j q_j(x_j) < p_{j-1}(x_j) (u_j from stream 1,
 * the test taken in double from fp32 probabilities); an id outside 0..V-1 is
 * rejected.  At the first rejection j the emitted token is drawn from
 * w = max(0, p_{j-1} - q_j); when all K are kept, from p_K (block from
 * stream 4, noise from stream 2; a residual that rounding leaves empty falls
 * back to the verifier row p_{j-1}).
 *   draft_logits [n_req, B-1, V] float, target_logits [n_req, B, V] float
 *   cand [n_req, B-1] int32, req_id [n_req] int32 >= 0
 *   draft_lse nullable [n_req, B-1] float: the draft_lse of the
 *             dflash_spec_draft call on these drafter rows at this
 *             temperature; saves reading every drafter row once more
 *   tokens [n_req, B] int32 out: the n kept candidates, then the emitted
 *          token at index n, then -1
 *   tau [n_req] int32 out: n + 1 */
int dflash_spec_verify(dflash_ctx* ctx, void* stream, int32_t n_req, const float* draft_logits,
                       const float* target_logits, const int32_t* cand, const float* draft_lse, float temperature,
                       uint64_t seed, const int32_t* req_id, int32_t* tokens, int32_t* tau);

/* Kernel kinds, for per-kernel timing. */
enum dflash_kernel_kind {
  DFLASH_K_FUSE_GEMM = 0,   /* context fusion GEMM W_c [H^(l1);...] */
  DFLASH_K_FUSE_NORM,       /* RMSNorm of the fused context */
  DFLASH_K_CTX_KV_GEMM,     /* per-layer context K/V projection + RoPE + cache append */
  DFLASH_K_EMBED,           /* block assembly */
  DFLASH_K_NORM,            /* pre-attention / pre-FFN / final RMSNorm */
  DFLASH_K_QKV_GEMM,        /* block Q/K_b/V_b projection + RoPE */
  DFLASH_K_ATTENTION,       /* KV-injected block attention, split-KV partials */
  DFLASH_K_ATTN_COMBINE,    /* merge of the attention splits */
  DFLASH_K_O_GEMM,          /* output projection + residual */
  DFLASH_K_GATEUP_GEMM,     /* gate/up projection + SwiGLU */
  DFLASH_K_DOWN_GEMM,       /* down projection + residual */
  DFLASH_K_LM_HEAD,         /* LM head with fused top-k */
  DFLASH_K_TOPK_MERGE,      /* top-k merge */
  DFLASH_K_RELAY,           /* DFlow relay: assembly and the relay MLP GEMMs */
  DFLASH_K_SELECT,          /* DFlash 2 selector: gate GEMM, pair scores and walk */
  DFLASH_K_CONV,            /* DFlash 2 two-tap convolution: tap-correction GEMM and the tap mix */
  DFLASH_K_SPEC_DRAFT,      /* speculative sampling: Gumbel-max drafting */
  DFLASH_K_SPEC_STATS,      /* speculative sampling: row log-sum-exps and the acceptance scan */
  DFLASH_K_SPEC_RESAMPLE,   /* speculative sampling: replacement / bonus draw */
  DFLASH_K_ACCEPT,          /* acceptance scan (stateless call: never timed) */
  DFLASH_K_COUNT
};

/* Diagnostics: time every launch of the kernel kinds in `kind_mask` (bit k =
 * kind k) with a HIP event pair recorded on the launch stream, up to
 * `max_launches` launches in total (events are created here, on the host).
 * Disable with kind_mask = 0.  Not for use under graph capture. */
int dflash_profile_enable(dflash_ctx* ctx, uint32_t kind_mask, int32_t max_launches);

/* Wait for the recorded events and return, per kind, the summed milliseconds
 * and the launch count (arrays of DFLASH_K_COUNT entries, [host]); then
 * clears the records. */
int dflash_profile_read(dflash_ctx* ctx, double* total_ms, int32_t* launches);

/* Static text for a status code. */
const char* dflash_strerror(int status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* dflash_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_FUSE_H */
