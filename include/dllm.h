/*
 * dllm.h -- C ABI of the token-skipping denoising-step library for AMD Instinct MI355X (gfx950).
 *
 * One denoising step of a masked-diffusion LLM (LLaDA / Dream shaped) that recomputes only
 * salient tokens and reuses cached state for the rest, split into five calls:
 *
 *   dllm_saliency               per-token importance score
 *   dllm_select_compact         top-k or threshold selection + stream compaction
 *   (dllm_flags_from_rows       restricts a later selection to the rows of an earlier one)
 *   dllm_gather_qkv_scatter_kv  QKV projection of the selected tokens, K/V scattered into the cache
 *   dllm_partial_attn           selected queries against the whole (updated) K/V cache, no mask
 *   dllm_gather_ffn_scatter     output projection + SwiGLU FFN of the selected tokens, scattered
 *                               back into the cached hidden states
 *
 * and, for a step that keeps the attention context of every token (not only the selected ones):
 *
 *   dllm_gather_kv_rows         copies of the K/V rows a projection call is about to overwrite
 *   dllm_salient_attn           exact rows for the selected tokens, changed-key update for the rest
 *   dllm_gather_rows            compact copies of selected rows (e.g. contexts for the FFN call)
 *
 * and, for a decoding loop that stays on the device (block decoding, graph replay):
 *
 *   dllm_commit                 threshold / top-k commit of the active block, block advance,
 *                               the next step's selection flags
 *   dllm_embed_rows             embedding rows of listed (committed) positions
 *
 * Sources (web pages; section names as printed there):
 *   [ES-dLLM]  "ES-dLLM: Efficient Inference for Diffusion Large Language Models by Early-Skipping",
 *              German summary page §2.A (importance-score equation, alpha = 0.5) and §2.B (top-k
 *              positions proceed; K/V/hidden caches updated in place for selected tokens, old
 *              entries reused for skipped ones; skip at early layers such as 1/8 and 1/4 depth);
 *              Dutch summary page, "Methodologie".
 *   [DyLLM]    "DyLLM: Efficient Diffusion LLM Inference via Saliency-based Token Selection and
 *              Partial Attention", French summary page §1 (bidirectional attention, each step a
 *              prefill-like pass), §2.A (cosine similarity of step t and t-1 vectors, salient below a
 *              threshold tau; FFN skipped for stable tokens), §2.B (attention rows of salient tokens
 *              recomputed exactly), §2.C (response-only steps).
 *   [SlowFast] "Accelerating Diffusion Large Language Models with SlowFast Sampling", German
 *              summary page, "Der SlowFast-Algorithmus" item 2 (threshold commit with a top-k
 *              fallback).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller, 16-byte aligned, row-major and
 *     contiguous with the layouts given below. The library allocates nothing and keeps no mutable
 *     global state (except the static device array of dllm_commit_noalloc); calls are
 *     re-entrant.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously; no
 *     call synchronises the device.
 *   - All arguments are validated on the host before anything is enqueued. DLLM_ERR_INVALID_ARG,
 *     DLLM_ERR_UNSUPPORTED and DLLM_ERR_WORKSPACE mean nothing was enqueued and nothing was
 *     written. DLLM_ERR_HIP means the runtime rejected a kernel launch; a call that makes several
 *     launches (projection, attention and FFN calls, dllm_salient_attn, dllm_commit) may then
 *     have enqueued the launches before the rejected one, so its outputs and any state it
 *     updates in place (caches, softmax state) are undefined until the call succeeds again.
 *     Execution faults surface at the caller's next synchronisation.
 *   - One storage type per call (shape->dtype) covers every tensor except: scores, confidences and
 *     deltas are float32; indices are int32; the force mask is uint8.
 *   - bf16 tensors are multiplied on the matrix cores with float32 accumulation; norms, softmax
 *     and SwiGLU are evaluated in float32.
 *   - Each call is one roctx range named after the call (host part: checks and enqueues), seen
 *     by `rocprofv3 --marker-trace`; the library links librocprofiler-sdk-roctx for it.
 */
#ifndef DLLM_H_
#define DLLM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DLLM_OK = 0,
  DLLM_ERR_INVALID_ARG = 1,   /* NULL required pointer, bad dimension, bad enum, misaligned ptr */
  DLLM_ERR_UNSUPPORTED = 2,   /* valid but outside this build: hd not 64/128, d or F % 64 != 0 ... */
  DLLM_ERR_WORKSPACE = 3,     /* ws_bytes smaller than dllm_workspace_bytes() */
  DLLM_ERR_HIP = 4            /* a kernel launch was rejected by the runtime */
} dllm_status;

typedef enum { DLLM_F32 = 0, DLLM_BF16 = 1 } dllm_dtype;

/* Per-token variation between step t and t-1 (x = current, y = previous vector, length d). */
typedef enum {
  DLLM_DELTA_L1N = 0,  /* ||x - y||_1 / (sqrt(d) ||y||_2)     [ES-dLLM] §2.A equation (default) */
  DLLM_DELTA_COS = 1,  /* 1 - <x,y> / (||x|| ||y||)            [DyLLM] §2.A cosine rule          */
  DLLM_DELTA_L2R = 2   /* ||x - y||_2 / ||y||_2                 relative L2 change                */
} dllm_delta;

typedef enum { DLLM_SEL_THRESHOLD = 0, DLLM_SEL_TOPK = 1 } dllm_sel_mode;

typedef enum {
  DLLM_OP_SALIENCY = 0, DLLM_OP_SELECT = 1, DLLM_OP_QKV = 2, DLLM_OP_ATTN = 3, DLLM_OP_FFN = 4,
  DLLM_OP_COMMIT = 5
} dllm_op;

/* Model / batch shape. 48 bytes, no implicit padding.
 *   B batch rows (sequences), S positions per sequence, d model width, H query heads,
 *   Hkv key/value heads (H % Hkv == 0; query head h reads kv head h / (H / Hkv)), hd head width,
 *   F FFN inner width, dtype a dllm_dtype, V vocabulary size (saliency only), rms_eps RMSNorm
 *   epsilon.
 *   m_plan (>= 0): number of selected rows the layer calls tune their launch plans for (tile
 *   shapes, K and key splits); 0 means m_cap. With threshold selection M is only known on the
 *   device, and m_cap must cover the worst case; m_plan lets a caller that expects far fewer rows
 *   (for example last step's count) get the plan for those. Every M <= m_cap is still computed
 *   in full whatever m_plan says; only the speed and, through the split points of float32
 *   sums, the rounding of the results depend on it. The workspace size depends on it too
 *   (query dllm_workspace_bytes with the same shape). */
typedef struct {
  int32_t B, S, d, H, Hkv, hd, F;
  int32_t dtype;
  int64_t V;
  float rms_eps;
  int32_t m_plan;
} dllm_shape;

#define DLLM_MAX_SELECT_S 8192 /* largest S dllm_select_compact accepts (one row lives in LDS) */
#define DLLM_MAX_SALIENT_S 8192 /* largest S dllm_salient_attn accepts (changed list in LDS) */

/* (1) Saliency [ES-dLLM §2.A equation; DyLLM §2.A].
 *   score[b,s] = alpha * c[b,s] + (1 - alpha) * delta[b,s]
 *   c     = max_v softmax(logits[b,s,:])  (largest probability at temperature 1, previous step)
 *   delta = variation of h_cur[b,s,:] against h_prev[b,s,:] of kind `delta_kind`.
 * h_cur, h_prev : [B,S,d] dtype; may be NULL only when alpha == 1. d % 8 == 0.
 * logits        : [B,S,V] dtype, or NULL: then c is read from conf_out (required when alpha != 0
 *                 without logits, together with h_cur/h_prev), the confidence an earlier call
 *                 wrote from the same logits [ES-dLLM §2.B second skip point: the score of a later
 *                 layer reuses the previous step's confidence].
 * score         : [B,S] float32 (required).
 * conf_out      : [B,S] float32 or NULL: with logits, c is written there; without, see above.
 * delta_out     : [B,S] float32 or NULL (requires h_cur/h_prev).
 * alpha in [0,1]. With alpha == 0 and conf_out == NULL the logits are not read.
 * Workspace: none. */
dllm_status dllm_saliency(const dllm_shape* shape, int32_t delta_kind, float alpha,
                          const void* h_cur, const void* h_prev, const void* logits,
                          float* score, float* conf_out, float* delta_out, void* stream);

/* (2) Selection + stream compaction [ES-dLLM §2.B top-k; DyLLM §2.A threshold; DyLLM §2.C
 * response-only steps leave the prompt out of the candidates].
 * Flag byte force[b,s]: bit 0 set = forced (always selected); else bit 1 set = excluded (never
 * selected); else a candidate. Other bits are ignored. NULL: every position is a candidate.
 * Per sequence b, the selected set is the forced positions plus
 *   TOPK:      the k best candidates by (score descending, position ascending), where
 *              NaN ranks below -inf and -0 equals +0 (fewer than k candidates -> all of them);
 *   THRESHOLD: the candidates with score > tau (float32 compare; NaN never passes).
 * Output: sel_idx[row_ptr[b] .. row_ptr[b+1]) holds the flat ids b*S + s of sequence b in
 * ascending order; row_ptr[0] = 0, row_ptr[B] = total count M. Bit-exact and deterministic.
 * score : [B,S] float32; force : [B,S] uint8 flags or NULL.
 * sel_idx : int32 [B*S] (entries past row_ptr[B] untouched); row_ptr : int32 [B+1].
 * S <= DLLM_MAX_SELECT_S, else DLLM_ERR_UNSUPPORTED. k >= 0; tau not NaN.
 * Workspace: none (ws may be NULL). */
dllm_status dllm_select_compact(const dllm_shape* shape, int32_t mode, float tau, int32_t k,
                                const float* score, const uint8_t* force,
                                int32_t* sel_idx, int32_t* row_ptr,
                                void* ws, size_t ws_bytes, void* stream);

/* Flags that restrict a later selection to listed rows [ES-dLLM §2.B: a second skip point
 * deeper in the model ranks only the tokens still being computed]. flags[p] = 2 (excluded) for
 * every position p = b*S + s, then for j < M = min(row_ptr[B], m_cap), p = sel_idx[j]:
 * flags[p] = force[p] & 1 (forced stays forced; NULL force: 0, a candidate). force and flags
 * are [B,S] uint8 and must not be the same array. Workspace: none. */
dllm_status dllm_flags_from_rows(const dllm_shape* shape, const uint8_t* force,
                                 const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                                 uint8_t* flags, void* stream);

/* (3) Gathered QKV projection + K/V cache scatter [ES-dLLM §2.B partial cache update].
 * For j < M = min(row_ptr[B], m_cap), with (b, s) = (sel_idx[j] / S, sel_idx[j] % S):
 *   xn = h_in[b,s,:] / sqrt(mean(h_in[b,s,:]^2) + rms_eps) * g_attn
 *   [q | k | v] = xn W_qkv^T
 *   q_sel[j,:] = q;  k_cache[b,hk,s,:] = k[hk];  v_cache[b,hk,s,:] = v[hk]
 * h_in    : [B,S,d];  g_attn : [d];  w_qkv : [(H + 2 Hkv) hd, d] rows ordered Q | K | V
 * q_sel   : [m_cap, H hd];  k_cache, v_cache : [B, Hkv, S, hd], entries of unselected positions
 *           are never written.
 * m_cap   : capacity in rows (0 <= m_cap <= B S). M is read on the device, so no host sync.
 * hd in {64,128}; d % 64 == 0. Workspace: dllm_workspace_bytes(DLLM_OP_QKV, shape, m_cap). */
dllm_status dllm_gather_qkv_scatter_kv(const dllm_shape* shape,
                                       const void* h_in, const void* g_attn, const void* w_qkv,
                                       const int32_t* sel_idx, const int32_t* row_ptr,
                                       int32_t m_cap, void* q_sel, void* k_cache, void* v_cache,
                                       void* ws, size_t ws_bytes, void* stream);

/* (4) Partial attention [DyLLM §2.B exact rows for salient queries; §1 bidirectional].
 * For j < M and query head h (kv head hk = h / (H / Hkv)), with b = sel_idx[j] / S:
 *   o_sel[j, h hd : (h+1) hd] = sum_t softmax_t(scale * q . k_cache[b,hk,t,:]) v_cache[b,hk,t,:]
 * over every t in [0, S): no mask, the token itself and masked positions included.
 * q_sel : [m_cap, H hd];  k_cache, v_cache : [B, Hkv, S, hd];  o_sel : [m_cap, H hd].
 * scale finite (usually 1/sqrt(hd)). hd in {64,128}.
 * Workspace: dllm_workspace_bytes(DLLM_OP_ATTN, shape, m_cap) (split-key partials). */
dllm_status dllm_partial_attn(const dllm_shape* shape, float scale,
                              const void* q_sel, const void* k_cache, const void* v_cache,
                              const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                              void* o_sel, void* ws, size_t ws_bytes, void* stream);

/* (5) Gathered output projection + SwiGLU FFN + hidden-state scatter [DyLLM §2.A FFN only for
 * salient tokens; ES-dLLM §2.B hidden-state cache updated in place].
 * For j < M with (b, s) = (sel_idx[j] / S, sel_idx[j] % S):
 *   h  = h_in[b,s,:] + o_sel[j,:] W_o^T
 *   hn = h / sqrt(mean(h^2) + rms_eps) * g_ffn
 *   h_out[b,s,:] = h + (silu(hn W_gate^T) * (hn W_up^T)) W_down^T,  silu(x) = x / (1 + e^-x)
 * h_in : [B,S,d]; o_sel : [m_cap, H hd]; w_o : [d, H hd]; g_ffn : [d]; w_gate, w_up : [F, d];
 * w_down : [d, F]; h_out : [B,S,d], rows of unselected positions are never written. h_out may
 * alias h_in. d % 64 == 0, F % 64 == 0, hd in {64,128}.
 * Workspace: dllm_workspace_bytes(DLLM_OP_FFN, shape, m_cap). */
dllm_status dllm_gather_ffn_scatter(const dllm_shape* shape,
                                    const void* h_in, const void* o_sel, const void* w_o,
                                    const void* g_ffn, const void* w_gate, const void* w_up,
                                    const void* w_down, const int32_t* sel_idx,
                                    const int32_t* row_ptr, int32_t m_cap, void* h_out,
                                    void* ws, size_t ws_bytes, void* stream);

/* Copies of the K/V rows at the selected positions [DyLLM §2.B: the stable-token update takes
 * out the contributions of the changed keys' previous rows, so those rows are copied before
 * dllm_gather_qkv_scatter_kv overwrites them].
 * For j < M = min(row_ptr[B], m_cap), with (b, s) = (sel_idx[j] / S, sel_idx[j] % S):
 *   k_rows[j, hk, :] = k_cache[b, hk, s, :];  v_rows[j, hk, :] = v_cache[b, hk, s, :]
 * k_cache, v_cache : [B, Hkv, S, hd] dtype;  k_rows, v_rows : [m_cap, Hkv, hd] dtype.
 * Bit-exact copies. hd in {64,128}. Workspace: none. */
dllm_status dllm_gather_kv_rows(const dllm_shape* shape, const void* k_cache, const void* v_cache,
                                const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                                void* k_rows, void* v_rows, void* stream);

/* Attention context of every token [DyLLM §2.B: exact rows for salient tokens; for stable
 * tokens the previous step's weights of the unchanged keys are reused and only the contributions
 * of the changed keys are replaced, so the cost is O(S |selected|) instead of O(S^2)].
 * Per-token softmax state, kept by the caller from step to step (positions p = b*S + s):
 *   st_m[p, h]  reference point in base-2 units of the scaled scores,
 *   st_l[p, h]  sum over every key t of 2^(scale log2(e) q.k_t - st_m),
 *   st_o[p, h*hd : (h+1)*hd]  the normalised context (float32);
 *   so ln sum_t exp(scale q.k_t) = ln(2) (st_m + log2 st_l), and q_all[p] is the query the state
 *   belongs to.
 * Given caches already holding this step's K/V rows at the selected positions (after
 * dllm_gather_qkv_scatter_kv) and k_old, v_old from dllm_gather_kv_rows taken before it:
 *   selected token j:  q_all[p] = q_sel[j]; its state and context are recomputed exactly against
 *                      every key (as dllm_partial_attn); o_sel[j] as dllm_partial_attn writes it;
 *   any other token:   its state is updated with the old rows of the changed keys taken out and
 *                      the new rows put in, against its stored query q_all[p];
 *   o_all[p] = st_o[p] rounded to dtype, for every position.
 * The result for every token is the attention of q_all (after the update) against the updated
 * cache, up to rounding, provided the state held that attention for the previous cache. An
 * update that would keep less than a quarter of the token's stored softmax mass (the changed keys
 * held most of its weight, so the rounding of the removed terms would dominate what is left), or
 * would give a sum that is not a positive finite number, is not applied: that (token, head) state
 * is recomputed exactly against every key instead, in a third pass.
 * Initialise the state with a call that selects every position (then nothing is "other").
 * q_first (0 <= q_first <= S) [DyLLM §2.C response-only steps]: unselected positions s < q_first
 * of every sequence are not processed (their query and state are left as they are; o_all there
 * is rewritten from the unchanged state, i.e. the same context as before), so a prompt held at
 * the front of each sequence costs no attention work in such a step. Their state then no longer
 * matches the cache; a later call that selects them (a step that re-injects the prompt)
 * recomputes it exactly. 0 = every position.
 * q_sel : [m_cap, H hd]; q_all : [B, S, H hd] (updated in place); k_cache, v_cache :
 * [B, Hkv, S, hd]; k_old, v_old : [m_cap, Hkv, hd]; st_m, st_l : [B, S, H] float32; st_o :
 * [B, S, H hd] float32 (updated in place); o_sel : [m_cap, H hd]; o_all : [B, S, H hd].
 * bf16 only (DLLM_ERR_UNSUPPORTED for float32); S <= DLLM_MAX_SALIENT_S; hd in {64,128}; scale
 * finite. Workspace: dllm_workspace_bytes(DLLM_OP_ATTN, shape, m_cap). */
dllm_status dllm_salient_attn(const dllm_shape* shape, float scale, const void* q_sel,
                              void* q_all, const void* k_cache, const void* v_cache,
                              const void* k_old, const void* v_old, const int32_t* sel_idx,
                              const int32_t* row_ptr, int32_t m_cap, int32_t q_first,
                              float* st_m, float* st_l, float* st_o, void* o_sel, void* o_all,
                              void* ws, size_t ws_bytes, void* stream);

/* Compact copies of whole rows [DyLLM §2.A: the FFN runs for the tokens whose context changed;
 * this gathers their contexts from the context of every token into the compact rows the FFN call
 * reads]. For j < M = min(row_ptr[B], m_cap): dst[j, :] = src[sel_idx[j], :], rows of `width`
 * elements of shape->dtype (only B, S and dtype of `shape` are used). src : [B*S, width];
 * dst : [m_cap, width]. width * element size must be a multiple of 16 bytes. Bit-exact copies.
 * Workspace: none. */
dllm_status dllm_gather_rows(const dllm_shape* shape, const void* src, int32_t width,
                             const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                             void* dst, void* stream);

#define DLLM_MAX_BLOCK_LEN 256 /* largest block_len dllm_commit accepts */

/* Commit step of semi-autoregressive block decoding [SlowFast §2 "Der SlowFast-Algorithmus"
 * item 2: tokens of the current region above a high confidence threshold are decoded together,
 * with a top-k update when too few are]. Sequence b decodes positions P .. S-1 (P = prompt_len)
 * in blocks of block_len; blk[b] is its active block (blk[b] == number of blocks: done).
 * For the masked positions s (tok[b,s] < 0) of the active block:
 *   conf_s = largest softmax probability of logits[b,s,:] (temperature 1, float32),
 *   arg_s  = index of the largest logit (the lowest one among equal maxima);
 *   the n best by (conf descending, position ascending) commit, tok[b,s] = arg_s, with
 *   n = max(#{conf_s > tau}, min(k_min, #masked)).
 * A block left with no masked position advances blk[b] by one. Outputs: committed_idx
 * [committed_rp[b] .. committed_rp[b+1]) the committed flat ids b*S + s of sequence b, ascending
 * (capacity B * block_len); committed_rp [B+1]; flags [B,S] uint8 = 1 at the positions of the
 * (new) active block, else 0 (the next step's forced selection, dllm_select_compact).
 * logits : [B,S,V] dtype, V % 8 == 0 (else DLLM_ERR_UNSUPPORTED), 16-byte aligned; tok int32
 * [B,S] and blk int32 [B] updated in place; 1 <= block_len <= DLLM_MAX_BLOCK_LEN; k_min >= 0;
 * tau not NaN. The decision is taken on float32 confidences. Everything is read and written on
 * the device: no host synchronisation. Workspace: dllm_workspace_bytes(DLLM_OP_COMMIT, shape,
 * block_len). */
dllm_status dllm_commit(const dllm_shape* shape, const void* logits, int32_t prompt_len,
                        int32_t block_len, float tau, int32_t k_min, int32_t* tok, int32_t* blk,
                        int32_t* committed_idx, int32_t* committed_rp, uint8_t* flags, void* ws,
                        size_t ws_bytes, void* stream);

/* dllm_commit without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * per-position confidences and token ids of the active blocks live in a static device array of
 * the library (DLLM_COMMIT_NOALLOC_MAX_ROWS entries of 8 bytes, one copy per GPU, held until the
 * process ends). Arguments, outputs and errors as dllm_commit, plus DLLM_ERR_WORKSPACE when
 * shape->B * block_len exceeds DLLM_COMMIT_NOALLOC_MAX_ROWS. The call allocates nothing; its
 * first call on a device looks up that device's copy of the array (DLLM_ERR_HIP if the lookup
 * fails). Every call on one GPU shares the array, so calls that overlap on one GPU (on different
 * streams, or from several host threads without ordering) race; calls ordered on one stream do
 * not. Each call writes every array entry it reads before reading it. */
#define DLLM_COMMIT_NOALLOC_MAX_ROWS 65536
dllm_status dllm_commit_noalloc(const dllm_shape* shape, const void* logits, int32_t prompt_len,
                                int32_t block_len, float tau, int32_t k_min, int32_t* tok,
                                int32_t* blk, int32_t* committed_idx, int32_t* committed_rp,
                                uint8_t* flags, void* stream);

/* Embedding rows of listed positions [the next step's input after a commit]. For
 * j < M = min(row_ptr[B], m_cap), with p = sel_idx[j] (flat b*S + s) and t = tok[p]:
 *   x[p, :] = emb[t, :] if 0 <= t < V, else mask_emb (a masked position).
 * emb : [V, d] dtype (V = shape->V); mask_emb : [d]; tok : int32 [B*S]; x : [B,S,d] dtype.
 * d * element size must be a multiple of 16 bytes. Bit-exact copies. Workspace: none. */
dllm_status dllm_embed_rows(const dllm_shape* shape, const void* emb, const void* mask_emb,
                            const int32_t* tok, const int32_t* sel_idx, const int32_t* row_ptr,
                            int32_t m_cap, void* x, void* stream);

/* Bytes of device workspace the call `op` (a dllm_op) needs for this shape and m_cap; 0 when
 * none (for DLLM_OP_COMMIT the third argument is the block length).
 * With shape->m_plan == 0 the size is that of the plan for m_cap rows; with m_plan > 0 it
 * covers every m_plan in [1, m_cap], so a caller may change m_plan from call to call without
 * reallocating. Returns (size_t)-1 for an invalid op or shape. Pure host function. */
size_t dllm_workspace_bytes(int32_t op, const dllm_shape* shape, int32_t m_cap);

/* Static, NUL-terminated name of a dllm_status value. */
const char* dllm_status_string(int32_t status);

/* Library ABI version (major * 100 + minor). */
int32_t dllm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DLLM_H_ */
