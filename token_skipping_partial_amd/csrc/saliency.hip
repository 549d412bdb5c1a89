// (1) Per-token saliency, gfx950.
//
// ES-dLLM (German summary page) §2.A: importance = alpha * confidence of the previous step +
// (1 - alpha) * normalised variation of the intermediate vector between step t and t-1.
// DyLLM (French summary page) §2.A: cosine similarity of the step-t and step-(t-1) vectors.
//
// The work is a pure HBM stream: 2*d elements of hidden state per token plus, when the
// confidence term is on, V logits per token (126464 at LLaDA shape, the largest stream of the
// step). Each token's sums are fp32 wave/workgroup reductions of coalesced 16-byte loads.
//
//   with logits : one 256-thread workgroup per token (the vocabulary row is 253 KB of bf16)
//   no logits   : one 64-lane wave per token, four tokens per workgroup
#include "common.h"
#include "kernels.h"

namespace dllm {

struct HidSums {
  float s1, s2, sx, sy, sd;  // sum|x-y|, sum(x-y)^2, sum x^2, sum y^2, sum (x-y)(x+y)
};

template <typename T>
__device__ __forceinline__ void load8_stream(const T* p, float v[8]);

__device__ __forceinline__ void hid_add(HidSums& a, const float (&xv)[8], const float (&yv)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float df = xv[e] - yv[e];
    a.s1 += fabsf(df);
    a.s2 = fmaf(df, df, a.s2);
    a.sx = fmaf(xv[e], xv[e], a.sx);
    a.sy = fmaf(yv[e], yv[e], a.sy);
    a.sd = fmaf(df, xv[e] + yv[e], a.sd);
  }
}

// both hidden rows are read once: up to 4 pairs of 16-byte loads in flight per lane
template <typename T>
__device__ __forceinline__ void hid_accumulate(const T* x, const T* y, int d, int lane,
                                               int nlanes, HidSums& a) {
  constexpr int kU = 4;
  const int step = nlanes * 8;
  int i = lane * 8;
  for (; i + (kU - 1) * step + 8 <= d; i += kU * step) {
    float xv[kU][8], yv[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      load8_stream<T>(x + i + u * step, xv[u]);
      load8_stream<T>(y + i + u * step, yv[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) hid_add(a, xv[u], yv[u]);
  }
  for (; i < d; i += step) {
    float xv[8], yv[8];
    load8_stream<T>(x + i, xv);
    load8_stream<T>(y + i, yv);
    hid_add(a, xv, yv);
  }
}

// Variation from the five sums. COS is evaluated through an algebraically identical form that
// avoids cancelling two numbers close to 1:
//   1 - <x,y>/(|x||y|) = (|x-y|^2 - (|x| - |y|)^2) / (2 |x| |y|),  |x| - |y| = sd / (|x| + |y|)
__device__ __forceinline__ float variation(const HidSums& a, int kind, int d) {
  float ny = sqrtf(a.sy);
  if (kind == 0) return a.s1 / (sqrtf((float)d) * ny);
  if (kind == 2) return sqrtf(a.s2) / ny;
  float nx = sqrtf(a.sx);
  float dn = a.sd / (nx + ny);
  return (a.s2 - dn * dn) / (2.0f * nx * ny);
}

// online (max, sum 2^(z*log2e - max)) over a strided part of a logits row, in log2 units
// The logits are read exactly once: non-temporal loads keep them from displacing other data in
// the caches (measured on MI355X at the LLaDA-8B layer, 1024 x 126464 bf16 logits: 57.8 -> 49.3 us,
// 4.8 -> 5.6 TB/s).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ void load8_stream(const T* p, float v[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const f32x4v a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    const f32x4v b = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ void logit_accumulate(const T* z, long V, int lane, int nlanes,
                                                 float& m, float& s) {
  constexpr int kU = 4;  // 16-byte loads in flight per lane
  long i = (long)lane * 8;
  const long step = (long)nlanes * 8;
  for (; i + (kU - 1) * step + 8 <= V; i += kU * step) {
    float v[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) load8_stream<T>(z + i + u * step, v[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float cm = v[u][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cm = fmaxf(cm, v[u][e]);
      cm *= kLog2e;
      if (cm > m) {
        s *= fast_exp2(m - cm);
        m = cm;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s += fast_exp2(fmaf(v[u][e], kLog2e, -m));
    }
  }
  for (; i + 8 <= V; i += step) {
    float v[8];
    load8_stream<T>(z + i, v);
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, v[e]);
    cm *= kLog2e;
    if (cm > m) {
      s *= fast_exp2(m - cm);
      m = cm;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += fast_exp2(fmaf(v[e], kLog2e, -m));
  }
  // ragged tail (V % 8 != 0): the last V % 8 elements, one per lane
  long tail0 = (V / 8) * 8;
  long t = tail0 + lane;
  if (t < V) {
    float c = Elem<T>::load1(z + t) * kLog2e;
    if (c > m) {
      s *= fast_exp2(m - c);
      m = c;
    }
    s += fast_exp2(c - m);
  }
}

__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void wave_merge_ms(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, 64);
    float s2 = __shfl_xor(s, o, 64);
    merge_ms(m, s, m2, s2);
  }
}

__device__ __forceinline__ void wave_sums(HidSums& a) {
  a.s1 = wave_sum(a.s1); a.s2 = wave_sum(a.s2); a.sx = wave_sum(a.sx);
  a.sy = wave_sum(a.sy); a.sd = wave_sum(a.sd);
}

// ------------------------------------------------------------ one workgroup per token (logits)
template <typename T>
__global__ __launch_bounds__(256) void saliency_logits_kernel(SaliencyArgs a) {
  const int tok = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[4][7];

  HidSums hs = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (a.h_cur) {
    const T* x = static_cast<const T*>(a.h_cur) + (size_t)tok * a.d;
    const T* y = static_cast<const T*>(a.h_prev) + (size_t)tok * a.d;
    hid_accumulate<T>(x, y, a.d, tid, 256, hs);
    wave_sums(hs);
  }
  float m = -INFINITY, s = 0.f;
  const T* z = static_cast<const T*>(a.logits) + (size_t)tok * (size_t)a.V;
  logit_accumulate<T>(z, a.V, tid, 256, m, s);
  wave_merge_ms(m, s);
  if (lane == 0) {
    red[wave][0] = hs.s1; red[wave][1] = hs.s2; red[wave][2] = hs.sx;
    red[wave][3] = hs.sy; red[wave][4] = hs.sd; red[wave][5] = m; red[wave][6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    HidSums t = {0.f, 0.f, 0.f, 0.f, 0.f};
    float mm = -INFINITY, ss = 0.f;
    for (int w = 0; w < 4; ++w) {  // fixed order: deterministic
      t.s1 += red[w][0]; t.s2 += red[w][1]; t.sx += red[w][2]; t.sy += red[w][3];
      t.sd += red[w][4];
      merge_ms(mm, ss, red[w][5], red[w][6]);
    }
    float conf = 1.0f / ss;  // the maximum contributes 2^0 = 1 to ss
    float var = a.h_cur ? variation(t, a.kind, a.d) : 0.f;
    a.score[tok] = a.alpha * conf + (1.0f - a.alpha) * var;
    if (a.conf_out) a.conf_out[tok] = conf;
    if (a.delta_out) a.delta_out[tok] = var;
  }
}

// ------------------------------------------------------------ one wave per token (no logits)
template <typename T>
__global__ __launch_bounds__(256) void saliency_hidden_kernel(SaliencyArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.ntok) return;
  const T* x = static_cast<const T*>(a.h_cur) + (size_t)tok * a.d;
  const T* y = static_cast<const T*>(a.h_prev) + (size_t)tok * a.d;
  HidSums hs = {0.f, 0.f, 0.f, 0.f, 0.f};
  hid_accumulate<T>(x, y, a.d, lane, 64, hs);
  wave_sums(hs);
  if (lane == 0) {
    float var = variation(hs, a.kind, a.d);
    // the confidence term comes from an earlier call on the same logits, or is off (alpha == 0)
    a.score[tok] = a.conf_in ? a.alpha * a.conf_in[tok] + (1.0f - a.alpha) * var
                             : (1.0f - a.alpha) * var;
    if (a.delta_out) a.delta_out[tok] = var;
  }
}

hipError_t launch_saliency(const SaliencyArgs& a, bool bf16, hipStream_t st) {
  if (a.ntok == 0) return hipSuccess;
  if (a.logits) {
    if (bf16)
      hipLaunchKernelGGL(saliency_logits_kernel<uint16_t>, dim3(a.ntok), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(saliency_logits_kernel<float>, dim3(a.ntok), dim3(256), 0, st, a);
  } else {
    dim3 grid((a.ntok + 3) / 4);
    if (bf16)
      hipLaunchKernelGGL(saliency_hidden_kernel<uint16_t>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(saliency_hidden_kernel<float>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dllm
