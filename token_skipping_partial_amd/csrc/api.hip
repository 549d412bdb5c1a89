// C ABI of the token-skipping step library: host-side validation, workspace sizing, dispatch.
// Every check runs before anything is enqueued; a non-OK status means no launch happened.
#include <math.h>
#include <string.h>

#include <mutex>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "dllm.h"
#include "kernels.h"

using namespace dllm;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool base_shape_ok(const dllm_shape* s) {
  return s && s->B > 0 && s->S > 0 && s->d > 0 && (s->dtype == DLLM_F32 || s->dtype == DLLM_BF16) &&
         s->m_plan >= 0 && (long)s->B * (long)s->S <= 0x7fffffffL;
}

// shape checks shared by the three layer calls; INVALID_ARG before UNSUPPORTED
dllm_status layer_shape_status(const dllm_shape* s, int32_t m_cap) {
  if (!base_shape_ok(s) || s->H <= 0 || s->Hkv <= 0 || s->hd <= 0 || s->F <= 0 ||
      s->H % s->Hkv != 0 || m_cap < 0 || (long)m_cap > (long)s->B * s->S ||
      !(s->rms_eps >= 0.f) || !isfinite(s->rms_eps))
    return DLLM_ERR_INVALID_ARG;
  if ((s->hd != 64 && s->hd != 128) || s->d % 64 != 0 || s->F % 64 != 0)
    return DLLM_ERR_UNSUPPORTED;
  return DLLM_OK;
}

ProjShape proj_shape(const dllm_shape* s, int32_t m_cap) {
  ProjShape p;
  p.B = s->B; p.S = s->S; p.d = s->d; p.H = s->H; p.Hkv = s->Hkv; p.hd = s->hd; p.F = s->F;
  p.eps = s->rms_eps;
  p.m_cap = m_cap;
  p.m_plan = (s->m_plan > 0 && s->m_plan < m_cap) ? s->m_plan : m_cap;
  return p;
}

// One named roctx range per library call (its host part: checks and enqueues; the kernels it
// launched run on the device afterwards). Shown by `rocprofv3 --marker-trace`; without a tool
// attached a push / pop is a call into an empty table slot.
struct CallRange {
  explicit CallRange(const char* name) { roctxRangePushA(name); }
  ~CallRange() { roctxRangePop(); }
  CallRange(const CallRange&) = delete;
  CallRange& operator=(const CallRange&) = delete;
};

dllm_status hip_status(hipError_t e) { return e == hipSuccess ? DLLM_OK : DLLM_ERR_HIP; }

// Static scratch of dllm_commit_noalloc: confidences, then token ids, of up to
// DLLM_COMMIT_NOALLOC_MAX_ROWS (sequence, block row) pairs. Every GPU the library runs on holds
// its own copy at its own address; `scratch` in host code only names the symbol, so the device
// address is looked up once per device (hipGetSymbolAddress) and only that address is used.
static __device__ __align__(256) char scratch[(size_t)DLLM_COMMIT_NOALLOC_MAX_ROWS * 8];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's copy of `scratch` (NULL on a runtime error)
char* commit_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return static_cast<char*>(g_scratch_ptr[dev]);
}

dllm_status ws_status(const void* ws, size_t have, size_t need) {
  if (need == 0) return DLLM_OK;
  if (have < need) return DLLM_ERR_WORKSPACE;
  if (!ws || !aligned16(ws)) return DLLM_ERR_INVALID_ARG;
  return DLLM_OK;
}

}  // namespace

extern "C" {

static_assert(DLLM_MAX_SALIENT_S == kSalientMaxS, "stable-token pass limit");
int32_t dllm_version(void) { return 104; }

const char* dllm_status_string(int32_t status) {
  switch (status) {
    case DLLM_OK: return "DLLM_OK";
    case DLLM_ERR_INVALID_ARG: return "DLLM_ERR_INVALID_ARG";
    case DLLM_ERR_UNSUPPORTED: return "DLLM_ERR_UNSUPPORTED";
    case DLLM_ERR_WORKSPACE: return "DLLM_ERR_WORKSPACE";
    case DLLM_ERR_HIP: return "DLLM_ERR_HIP";
    default: return "DLLM_ERR_UNKNOWN";
  }
}

size_t dllm_workspace_bytes(int32_t op, const dllm_shape* shape, int32_t m_cap) {
  switch (op) {
    case DLLM_OP_COMMIT:  // m_cap is the block length here
      if (!base_shape_ok(shape) || m_cap < 1 || m_cap > kMaxBlockLen) return (size_t)-1;
      return 2 * ((((size_t)shape->B * m_cap * 4) + 255) & ~(size_t)255);
    case DLLM_OP_SALIENCY:
      return base_shape_ok(shape) ? 0 : (size_t)-1;
    case DLLM_OP_SELECT:
      return base_shape_ok(shape) ? 0 : (size_t)-1;
    case DLLM_OP_QKV:
    case DLLM_OP_ATTN:
    case DLLM_OP_FFN: {
      if (layer_shape_status(shape, m_cap) != DLLM_OK) return (size_t)-1;
      const bool bf16 = shape->dtype == DLLM_BF16;
      ProjShape p = proj_shape(shape, m_cap);
      auto bytes = [&](const ProjShape& q) {
        if (op == DLLM_OP_QKV) return qkv_workspace_bytes(bf16, q);
        if (op == DLLM_OP_ATTN) return attn_workspace_bytes(bf16, q);
        return ffn_workspace_bytes(bf16, q);
      };
      if (shape->m_plan == 0) return bytes(p);
      // any m_plan: the weight-streaming plans' K split only shrinks as the planned rows grow,
      // so the first row count of each of their classes bounds it; the larger tiles' plan is the
      // same within each 128-row interval, so one row count per interval covers them; the
      // attention key split is largest at one planned row (its estimate of busy workgroups is
      // smallest there)
      size_t most = bytes(p);
      auto cover = [&](int r) {
        p.m_plan = r;
        const size_t b = bytes(p);
        if (b > most) most = b;
      };
      for (int r : {1, 65, 129}) if (r <= m_cap) cover(r);
      for (long r = kWsMaxRows + 1; r <= m_cap; r = (r + 127) / 128 * 128 + 1) cover((int)r);
      return most;
    }
    default:
      return (size_t)-1;
  }
}

dllm_status dllm_saliency(const dllm_shape* shape, int32_t delta_kind, float alpha,
                          const void* h_cur, const void* h_prev, const void* logits,
                          float* score, float* conf_out, float* delta_out, void* stream) {
  CallRange range_("dllm_saliency");
  if (!base_shape_ok(shape) || !score || !(alpha >= 0.f && alpha <= 1.f) ||
      delta_kind < DLLM_DELTA_L1N || delta_kind > DLLM_DELTA_L2R)
    return DLLM_ERR_INVALID_ARG;
  const bool has_h = h_cur != nullptr || h_prev != nullptr;
  if (has_h && (!h_cur || !h_prev)) return DLLM_ERR_INVALID_ARG;
  if (alpha != 1.f && !has_h) return DLLM_ERR_INVALID_ARG;
  // without logits, `conf_out` is the confidence input of the alpha term (an earlier call's output)
  const bool conf_in = !logits && alpha != 0.f;
  if (conf_in && (!conf_out || !has_h)) return DLLM_ERR_INVALID_ARG;
  if (conf_out && !logits && !conf_in) return DLLM_ERR_INVALID_ARG;
  if (delta_out && !has_h) return DLLM_ERR_INVALID_ARG;
  if (logits && shape->V <= 0) return DLLM_ERR_INVALID_ARG;
  for (const void* p : {h_cur, h_prev, logits, (const void*)score, (const void*)conf_out,
                        (const void*)delta_out})
    if (p && ((uintptr_t)p & 3u)) return DLLM_ERR_INVALID_ARG;
  for (const void* p : {h_cur, h_prev, logits})
    if (p && !aligned16(p)) return DLLM_ERR_INVALID_ARG;
  if (has_h && shape->d % 8 != 0) return DLLM_ERR_UNSUPPORTED;
  if (logits && shape->V % 8 != 0) return DLLM_ERR_UNSUPPORTED;

  SaliencyArgs a;
  a.ntok = shape->B * shape->S;
  a.d = shape->d;
  a.V = (long)shape->V;
  a.kind = delta_kind;
  a.alpha = alpha;
  a.h_cur = h_cur;
  a.h_prev = h_prev;
  // the vocabulary stream is skipped when neither the score nor an output needs it
  a.logits = (alpha != 0.f || conf_out) ? logits : nullptr;
  a.score = score;
  a.conf_out = logits ? conf_out : nullptr;
  a.conf_in = conf_in ? conf_out : nullptr;
  a.delta_out = delta_out;
  return hip_status(launch_saliency(a, shape->dtype == DLLM_BF16, (hipStream_t)stream));
}

dllm_status dllm_select_compact(const dllm_shape* shape, int32_t mode, float tau, int32_t k,
                                const float* score, const uint8_t* force, int32_t* sel_idx,
                                int32_t* row_ptr, void* ws, size_t ws_bytes, void* stream) {
  CallRange range_("dllm_select_compact");
  (void)ws;
  (void)ws_bytes;
  if (!base_shape_ok(shape) || !score || !sel_idx || !row_ptr) return DLLM_ERR_INVALID_ARG;
  if (mode == DLLM_SEL_TOPK) {
    if (k < 0) return DLLM_ERR_INVALID_ARG;
  } else if (mode == DLLM_SEL_THRESHOLD) {
    if (isnan(tau)) return DLLM_ERR_INVALID_ARG;
  } else {
    return DLLM_ERR_INVALID_ARG;
  }
  if (((uintptr_t)score & 3u) || ((uintptr_t)sel_idx & 3u) || ((uintptr_t)row_ptr & 3u))
    return DLLM_ERR_INVALID_ARG;
  if (shape->S > DLLM_MAX_SELECT_S) return DLLM_ERR_UNSUPPORTED;
  SelectArgs a;
  a.B = shape->B;
  a.S = shape->S;
  a.mode = mode;
  a.k = k;
  a.tau = tau;
  a.score = score;
  a.force = force;
  a.sel_idx = sel_idx;
  a.row_ptr = row_ptr;
  return hip_status(launch_select(a, (hipStream_t)stream));
}

dllm_status dllm_gather_qkv_scatter_kv(const dllm_shape* shape, const void* h_in,
                                       const void* g_attn, const void* w_qkv,
                                       const int32_t* sel_idx, const int32_t* row_ptr,
                                       int32_t m_cap, void* q_sel, void* k_cache, void* v_cache,
                                       void* ws, size_t ws_bytes, void* stream) {
  CallRange range_("dllm_gather_qkv_scatter_kv");
  dllm_status st = layer_shape_status(shape, m_cap);
  if (st != DLLM_OK) return st;
  if (!h_in || !g_attn || !w_qkv || !sel_idx || !row_ptr || !q_sel || !k_cache || !v_cache)
    return DLLM_ERR_INVALID_ARG;
  for (const void* p : {h_in, g_attn, w_qkv, (const void*)q_sel, (const void*)k_cache,
                        (const void*)v_cache})
    if (!aligned16(p)) return DLLM_ERR_INVALID_ARG;
  const bool bf16 = shape->dtype == DLLM_BF16;
  const ProjShape p = proj_shape(shape, m_cap);
  if ((st = ws_status(ws, ws_bytes, qkv_workspace_bytes(bf16, p))) != DLLM_OK) return st;
  return hip_status(launch_qkv(bf16, p, h_in, g_attn, w_qkv, sel_idx, row_ptr, q_sel, k_cache,
                               v_cache, ws, (hipStream_t)stream));
}

dllm_status dllm_partial_attn(const dllm_shape* shape, float scale, const void* q_sel,
                              const void* k_cache, const void* v_cache, const int32_t* sel_idx,
                              const int32_t* row_ptr, int32_t m_cap, void* o_sel, void* ws,
                              size_t ws_bytes, void* stream) {
  CallRange range_("dllm_partial_attn");
  dllm_status st = layer_shape_status(shape, m_cap);
  if (st != DLLM_OK) return st;
  if (!q_sel || !k_cache || !v_cache || !sel_idx || !row_ptr || !o_sel || !isfinite(scale))
    return DLLM_ERR_INVALID_ARG;
  for (const void* p : {q_sel, k_cache, v_cache, (const void*)o_sel})
    if (!aligned16(p)) return DLLM_ERR_INVALID_ARG;
  const bool bf16 = shape->dtype == DLLM_BF16;
  const ProjShape p = proj_shape(shape, m_cap);
  if ((st = ws_status(ws, ws_bytes, attn_workspace_bytes(bf16, p))) != DLLM_OK) return st;
  return hip_status(launch_attn(bf16, p, scale, q_sel, k_cache, v_cache, sel_idx, row_ptr, o_sel,
                                ws, (hipStream_t)stream));
}

dllm_status dllm_gather_ffn_scatter(const dllm_shape* shape, const void* h_in, const void* o_sel,
                                    const void* w_o, const void* g_ffn, const void* w_gate,
                                    const void* w_up, const void* w_down,
                                    const int32_t* sel_idx, const int32_t* row_ptr,
                                    int32_t m_cap, void* h_out, void* ws, size_t ws_bytes,
                                    void* stream) {
  CallRange range_("dllm_gather_ffn_scatter");
  dllm_status st = layer_shape_status(shape, m_cap);
  if (st != DLLM_OK) return st;
  if (!h_in || !o_sel || !w_o || !g_ffn || !w_gate || !w_up || !w_down || !sel_idx ||
      !row_ptr || !h_out)
    return DLLM_ERR_INVALID_ARG;
  for (const void* p : {h_in, o_sel, w_o, g_ffn, w_gate, w_up, w_down, (const void*)h_out})
    if (!aligned16(p)) return DLLM_ERR_INVALID_ARG;
  const bool bf16 = shape->dtype == DLLM_BF16;
  const ProjShape p = proj_shape(shape, m_cap);
  if ((st = ws_status(ws, ws_bytes, ffn_workspace_bytes(bf16, p))) != DLLM_OK) return st;
  return hip_status(launch_ffn(bf16, p, h_in, o_sel, w_o, g_ffn, w_gate, w_up, w_down, sel_idx,
                               row_ptr, h_out, ws, (hipStream_t)stream));
}

dllm_status dllm_gather_kv_rows(const dllm_shape* shape, const void* k_cache, const void* v_cache,
                                const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                                void* k_rows, void* v_rows, void* stream) {
  CallRange range_("dllm_gather_kv_rows");
  dllm_status st = layer_shape_status(shape, m_cap);
  if (st != DLLM_OK) return st;
  if (!k_cache || !v_cache || !sel_idx || !row_ptr || !k_rows || !v_rows)
    return DLLM_ERR_INVALID_ARG;
  for (const void* p : {k_cache, v_cache, (const void*)k_rows, (const void*)v_rows})
    if (!aligned16(p)) return DLLM_ERR_INVALID_ARG;
  const size_t elem = shape->dtype == DLLM_BF16 ? 2 : 4;
  return hip_status(launch_gather_kv_rows(proj_shape(shape, m_cap), elem, k_cache, v_cache,
                                          sel_idx, row_ptr, k_rows, v_rows, (hipStream_t)stream));
}

dllm_status dllm_salient_attn(const dllm_shape* shape, float scale, const void* q_sel,
                              void* q_all, const void* k_cache, const void* v_cache,
                              const void* k_old, const void* v_old, const int32_t* sel_idx,
                              const int32_t* row_ptr, int32_t m_cap, int32_t q_first, float* st_m,
                              float* st_l, float* st_o, void* o_sel, void* o_all, void* ws,
                              size_t ws_bytes, void* stream) {
  CallRange range_("dllm_salient_attn");
  dllm_status st = layer_shape_status(shape, m_cap);
  if (st != DLLM_OK) return st;
  if (!q_sel || !q_all || !k_cache || !v_cache || !k_old || !v_old || !sel_idx || !row_ptr ||
      !st_m || !st_l || !st_o || !o_sel || !o_all || !isfinite(scale) || q_first < 0 ||
      q_first > shape->S)
    return DLLM_ERR_INVALID_ARG;
  for (const void* p : {q_sel, (const void*)q_all, k_cache, v_cache, k_old, v_old,
                        (const void*)st_o, (const void*)o_sel, (const void*)o_all})
    if (!aligned16(p)) return DLLM_ERR_INVALID_ARG;
  if (shape->dtype != DLLM_BF16 || shape->S > DLLM_MAX_SALIENT_S) return DLLM_ERR_UNSUPPORTED;
  const ProjShape p = proj_shape(shape, m_cap);
  if ((st = ws_status(ws, ws_bytes, attn_workspace_bytes(true, p))) != DLLM_OK) return st;
  return hip_status(launch_salient_attn(p, scale, q_sel, q_all, k_cache, v_cache, k_old, v_old,
                                        sel_idx, row_ptr, q_first, st_m, st_l, st_o, o_sel, o_all,
                                        ws, (hipStream_t)stream));
}

dllm_status dllm_gather_rows(const dllm_shape* shape, const void* src, int32_t width,
                             const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                             void* dst, void* stream) {
  CallRange range_("dllm_gather_rows");
  if (!base_shape_ok(shape) || width <= 0 || m_cap < 0 || (long)m_cap > (long)shape->B * shape->S)
    return DLLM_ERR_INVALID_ARG;
  if (!src || !sel_idx || !row_ptr || !dst || !aligned16(src) || !aligned16(dst))
    return DLLM_ERR_INVALID_ARG;
  const size_t row_bytes = (size_t)width * (shape->dtype == DLLM_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0) return DLLM_ERR_UNSUPPORTED;
  return hip_status(launch_gather_rows(shape->B, m_cap, row_bytes, src, sel_idx, row_ptr, dst,
                                       (hipStream_t)stream));
}


dllm_status dllm_commit(const dllm_shape* shape, const void* logits, int32_t prompt_len,
                        int32_t block_len, float tau, int32_t k_min, int32_t* tok, int32_t* blk,
                        int32_t* committed_idx, int32_t* committed_rp, uint8_t* flags, void* ws,
                        size_t ws_bytes, void* stream) {
  CallRange range_("dllm_commit");
  if (!base_shape_ok(shape) || !logits || !tok || !blk || !committed_idx || !committed_rp ||
      !flags || shape->V <= 0 || prompt_len < 0 || prompt_len > shape->S || block_len < 1 ||
      k_min < 0 || tau != tau || !aligned16(logits))
    return DLLM_ERR_INVALID_ARG;
  if (block_len > kMaxBlockLen || shape->V % 8 != 0 || shape->V > 0x7fffffffL)
    return DLLM_ERR_UNSUPPORTED;
  dllm_status st = ws_status(ws, ws_bytes, dllm_workspace_bytes(DLLM_OP_COMMIT, shape, block_len));
  if (st != DLLM_OK) return st;
  CommitArgs c;
  c.logits = logits;
  c.B = shape->B; c.S = shape->S; c.V = shape->V;
  c.P = prompt_len; c.L = block_len;
  c.nblk = (shape->S - prompt_len + block_len - 1) / block_len;
  c.tau = tau; c.k_min = k_min;
  c.tok = tok; c.blk = blk; c.cidx = committed_idx; c.crp = committed_rp; c.flags = flags;
  const size_t half = (((size_t)shape->B * block_len * 4) + 255) & ~(size_t)255;
  c.conf = (float*)ws;
  c.arg = (int32_t*)((char*)ws + half);
  return hip_status(launch_commit(shape->dtype == DLLM_BF16, c, (hipStream_t)stream));
}

dllm_status dllm_commit_noalloc(const dllm_shape* shape, const void* logits, int32_t prompt_len,
                                int32_t block_len, float tau, int32_t k_min, int32_t* tok,
                                int32_t* blk, int32_t* committed_idx, int32_t* committed_rp,
                                uint8_t* flags, void* stream) {
  CallRange range_("dllm_commit_noalloc");
  if (!base_shape_ok(shape) || !logits || !tok || !blk || !committed_idx || !committed_rp ||
      !flags || shape->V <= 0 || prompt_len < 0 || prompt_len > shape->S || block_len < 1 ||
      k_min < 0 || tau != tau || !aligned16(logits))
    return DLLM_ERR_INVALID_ARG;
  if (block_len > kMaxBlockLen || shape->V % 8 != 0 || shape->V > 0x7fffffffL)
    return DLLM_ERR_UNSUPPORTED;
  const size_t rows = (size_t)shape->B * block_len;
  if (rows > (size_t)DLLM_COMMIT_NOALLOC_MAX_ROWS) return DLLM_ERR_WORKSPACE;
  char* base = commit_scratch();
  if (!base) return DLLM_ERR_HIP;
  CommitArgs c;
  c.logits = logits;
  c.B = shape->B; c.S = shape->S; c.V = shape->V;
  c.P = prompt_len; c.L = block_len;
  c.nblk = (shape->S - prompt_len + block_len - 1) / block_len;
  c.tau = tau; c.k_min = k_min;
  c.tok = tok; c.blk = blk; c.cidx = committed_idx; c.crp = committed_rp; c.flags = flags;
  // conf at the start of the array, arg after the conf entries of the maximum row count: the
  // row-confidence kernel writes both for every (sequence, block row) before the decision
  // kernel reads them, so no entry needs clearing
  c.conf = (float*)base;
  c.arg = (int32_t*)(base + (size_t)DLLM_COMMIT_NOALLOC_MAX_ROWS * 4);
  return hip_status(launch_commit(shape->dtype == DLLM_BF16, c, (hipStream_t)stream));
}

dllm_status dllm_embed_rows(const dllm_shape* shape, const void* emb, const void* mask_emb,
                            const int32_t* tok, const int32_t* sel_idx, const int32_t* row_ptr,
                            int32_t m_cap, void* x, void* stream) {
  CallRange range_("dllm_embed_rows");
  if (!base_shape_ok(shape) || !emb || !mask_emb || !tok || !sel_idx || !row_ptr || !x ||
      shape->V <= 0 || m_cap < 0 || (long)m_cap > (long)shape->B * shape->S)
    return DLLM_ERR_INVALID_ARG;
  for (const void* p : {emb, mask_emb, (const void*)x})
    if (!aligned16(p)) return DLLM_ERR_INVALID_ARG;
  const size_t row_bytes = (size_t)shape->d * (shape->dtype == DLLM_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0) return DLLM_ERR_UNSUPPORTED;
  return hip_status(launch_embed_rows(shape->B, m_cap, shape->V, row_bytes, emb, mask_emb, tok,
                                      sel_idx, row_ptr, x, (hipStream_t)stream));
}
dllm_status dllm_flags_from_rows(const dllm_shape* shape, const uint8_t* force,
                                 const int32_t* sel_idx, const int32_t* row_ptr, int32_t m_cap,
                                 uint8_t* flags, void* stream) {
  CallRange range_("dllm_flags_from_rows");
  if (!base_shape_ok(shape) || !sel_idx || !row_ptr || !flags || m_cap < 0 ||
      (long)m_cap > (long)shape->B * shape->S || (force && (const void*)force == (void*)flags))
    return DLLM_ERR_INVALID_ARG;
  return hip_status(launch_flags_from_rows(shape->B, shape->S, force, sel_idx, row_ptr, m_cap,
                                           flags, (hipStream_t)stream));
}

}  // extern "C"
