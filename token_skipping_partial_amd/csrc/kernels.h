// Internal launch interface between the C ABI (api.hip) and the kernels. Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dllm {

struct SaliencyArgs {
  int ntok, d;
  long V;
  int kind;
  float alpha;
  const void* h_cur;
  const void* h_prev;
  const void* logits;  // NULL when the confidence term is not needed
  float* score;
  float* conf_out;
  float* delta_out;
  const float* conf_in;  // no logits, alpha != 0: the confidence of an earlier call
};
hipError_t launch_saliency(const SaliencyArgs& a, bool bf16, hipStream_t st);

struct SelectArgs {
  int B, S, mode, k;
  float tau;
  const float* score;
  const uint8_t* force;
  int32_t* sel_idx;
  int32_t* row_ptr;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
hipError_t launch_flags_from_rows(int B, int S, const uint8_t* force, const int32_t* sel,
                                  const int32_t* rp, int m_cap, uint8_t* flags, hipStream_t st);

// ---------------------------------------------------------------- gathered projections
struct ProjShape {
  int B, S, d, H, Hkv, hd, F;
  float eps;
  int m_cap;
  int m_plan;  // rows the launch plans are tuned for (1 <= m_plan <= m_cap, or 0 when m_cap is 0)
};

// GEMM plan classes by planned rows: weight-streaming tiles that hold every row up to
// kWsMaxRows (64 / 128 / 256-row tiles), then 32 x 32 x 16 tiles (256 x 256 or 128 x 256, by an
// estimate of their time).
constexpr int kWsMaxRows = 256;

// launch plan of one GEMM: tile height, number of K splits
struct GemmPlan {
  int bm;      // rows of X per tile (bf16: 64, 128 or 256); the fp32 path uses 64 x 64 tiles
  int bn;      // weight rows per tile (SwiGLU: gate + up rows)
  int bk;      // K columns per LDS ring slot (64 or 128)
  int wm, wn;  // wave grid
  int st;      // ring slots
  int splits;  // K partitions reduced in a second pass (1 = fused epilogue)
  int mfma = 16;  // matrix-core block edge: 16 (16x16x32) or 32 (32x32x16)
  // > 0 (32 x 32 x 16, one K partition): rows [0, rows_big) on 256-row tiles and the rest on
  // 128-row tiles, two launches; bm / bn / ... then describe the 256-row part
  int rows_big = 0;
};
// N = output columns (SwiGLU: F, the tile then holds gate and up rows of the same columns)
GemmPlan plan_gemm(bool bf16, int rows, int N, int K, bool swiglu);
size_t gemm_partials_bytes(const GemmPlan& p, int m_cap, int N);

size_t qkv_workspace_bytes(bool bf16, const ProjShape& s);
size_t ffn_workspace_bytes(bool bf16, const ProjShape& s);

hipError_t launch_qkv(bool bf16, const ProjShape& s, const void* h_in, const void* g_attn,
                      const void* w_qkv, const int32_t* sel_idx, const int32_t* row_ptr,
                      void* q_sel, void* k_cache, void* v_cache, void* ws, hipStream_t st);

hipError_t launch_ffn(bool bf16, const ProjShape& s, const void* h_in, const void* o_sel,
                      const void* w_o, const void* g_ffn, const void* w_gate, const void* w_up,
                      const void* w_down, const int32_t* sel_idx, const int32_t* row_ptr,
                      void* h_out, void* ws, hipStream_t st);

// ---------------------------------------------------------------- partial attention
struct AttnPlan {
  int nsplit;  // key-range partitions merged by log-sum-exp in a second pass
};
AttnPlan plan_attn(bool bf16, const ProjShape& s);
size_t attn_workspace_bytes(bool bf16, const ProjShape& s);

hipError_t launch_attn(bool bf16, const ProjShape& s, float scale, const void* q_sel,
                       const void* k_cache, const void* v_cache, const int32_t* sel_idx,
                       const int32_t* row_ptr, void* o_sel, void* ws, hipStream_t st);

// ---------------------------------------------------------------- context of every token
hipError_t launch_salient_attn(const ProjShape& s, float scale, const void* q_sel, void* q_all,
                               const void* k_cache, const void* v_cache, const void* k_old,
                               const void* v_old, const int32_t* sel_idx, const int32_t* row_ptr,
                               int q_first, float* st_m, float* st_l, float* st_o, void* o_sel,
                               void* o_all, void* ws, hipStream_t st);
hipError_t launch_gather_kv_rows(const ProjShape& s, size_t elem, const void* k_cache,
                                 const void* v_cache, const int32_t* sel_idx,
                                 const int32_t* row_ptr, void* k_rows, void* v_rows,
                                 hipStream_t st);
constexpr int kSalientMaxS = 8192;  // sequence length limit of the stable-token pass
hipError_t launch_gather_rows(int B, int m_cap, size_t row_bytes, const void* src,
                              const int32_t* sel_idx, const int32_t* row_ptr, void* dst,
                              hipStream_t st);

// ---- decode loop (decode.hip)
constexpr int kMaxBlockLen = 256;  // one workgroup of the decision kernel holds a block
struct CommitArgs {
  const void* logits;  // [B, S, V]
  int B, S;
  long V;
  int P, L, nblk;      // prompt length, block length, number of blocks
  float tau;
  int k_min;
  int32_t* tok;        // [B, S], -1 = masked
  int32_t* blk;        // [B] active block (nblk = done)
  int32_t* cidx;       // [B * L] committed positions (flat ids)
  int32_t* crp;        // [B + 1]
  uint8_t* flags;      // [B, S] next step's selection flags (1 = active block)
  float* conf;         // workspace [B, L]
  int32_t* arg;        // workspace [B, L]
};
hipError_t launch_commit(bool bf16, const CommitArgs& c, hipStream_t st);
hipError_t launch_embed_rows(int B, int m_cap, long V, size_t row_bytes, const void* emb,
                             const void* mask_emb, const int32_t* tok, const int32_t* sel,
                             const int32_t* rp, void* x, hipStream_t st);
}  // namespace dllm
