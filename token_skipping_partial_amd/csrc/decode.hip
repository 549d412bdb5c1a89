// Device-side pieces of semi-autoregressive block decoding, gfx950.
//
// SlowFast (German summary page), "Der SlowFast-Algorithmus" item 2: the tokens of the current
// region whose confidence exceeds a high threshold are decoded together; when too few do, a
// top-k update guarantees progress. Here the region is the active block of the sequence; a block
// whose positions are all decoded hands over to the next one. Everything stays on the device
// (token ids, block index, the next step's selection flags), so a whole decoding step can be
// replayed from a HIP graph without a host round trip.
//
// commit: (1) one workgroup per row of the active blocks: largest softmax probability and argmax
// of the row's logits (16-byte loads, one exponential per element, fixed-order merge); (2) one
// workgroup for all sequences: which masked positions commit (rank by confidence, then
// position), token ids, block advance, the compact list of committed positions and the flags.
// embed_rows: the embedding rows of listed positions (the next step's input), 16-byte copies.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kConfThreads = 256;
constexpr int kDecideThreads = 256;

// (max, sum of 2^(z - max), first index of the max) merge; -inf max = empty
__device__ __forceinline__ void merge_msa(float& m, float& s, int& a, float m2, float s2, int a2) {
  const float M = fmaxf(m, m2);
  const float t1 = (m == -INFINITY) ? 0.f : s * fast_exp2(m - M);
  const float t2 = (m2 == -INFINITY) ? 0.f : s2 * fast_exp2(m2 - M);
  a = (m > m2) ? a : ((m2 > m) ? a2 : min(a, a2));
  s = t1 + t2;
  m = M;
}

template <typename T>
__global__ __launch_bounds__(kConfThreads) void row_conf_kernel(CommitArgs c) {
  const int b = blockIdx.y, j = blockIdx.x, tid = threadIdx.x;
  const int bk = c.blk[b];
  const int s = c.P + bk * c.L + j;
  float* conf = c.conf + (size_t)b * c.L + j;
  int32_t* arg = c.arg + (size_t)b * c.L + j;
  if (bk >= c.nblk || s >= c.S || c.tok[(size_t)b * c.S + s] >= 0) {  // not a candidate
    if (tid == 0) {
      *conf = -1.f;
      *arg = -1;
    }
    return;
  }
  const T* row = reinterpret_cast<const T*>(c.logits) + ((size_t)b * c.S + s) * (size_t)c.V;
  float m = -INFINITY, sum = 0.f;
  int am = INT_MAX;
  const long nch = c.V / 8;
  for (long ch = tid; ch < nch; ch += kConfThreads) {
    float v[8];
    Elem<T>::load8(row + 8 * ch, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float z = v[i] * kLog2e;
      if (z > m) {  // strictly greater: the first index of equal maxima stays
        sum = (m == -INFINITY ? 0.f : sum * fast_exp2(m - z)) + 1.f;
        m = z;
        am = (int)(8 * ch + i);
      } else {
        sum += fast_exp2(z - m);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    merge_msa(m, sum, am, __shfl_xor(m, o, 64), __shfl_xor(sum, o, 64), __shfl_xor(am, o, 64));
  __shared__ float wm[kConfThreads / 64], ws[kConfThreads / 64];
  __shared__ int wa[kConfThreads / 64];
  if ((tid & 63) == 0) {
    wm[tid >> 6] = m;
    ws[tid >> 6] = sum;
    wa[tid >> 6] = am;
  }
  __syncthreads();
  if (tid == 0) {
    float M = wm[0], Sm = ws[0];
    int A = wa[0];
    for (int w = 1; w < kConfThreads / 64; ++w) merge_msa(M, Sm, A, wm[w], ws[w], wa[w]);
    *conf = 1.f / Sm;   // the maximum contributes 2^0 = 1
    *arg = A;
  }
}

__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_int(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kDecideThreads / 64; ++w) t += red[w];
  return t;
}

__global__ __launch_bounds__(kDecideThreads) void commit_decide_kernel(CommitArgs c) {
  __shared__ float cf[kMaxBlockLen];
  __shared__ int red[kDecideThreads / 64];
  __shared__ int wcnt[kDecideThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int off = 0;
  if (tid == 0) c.crp[0] = 0;
  for (int b = 0; b < c.B; ++b) {
    const int bk = c.blk[b];
    int new_bk = bk, cnt = 0;
    if (bk < c.nblk) {
      const int lo = c.P + bk * c.L;
      const int nb = min(c.S, lo + c.L) - lo;
      const bool in = tid < nb;
      const float cj = in ? c.conf[(size_t)b * c.L + tid] : -1.f;
      const bool valid = cj >= 0.f;  // a masked position of the block
      const bool was_set = in && !valid;
      __syncthreads();  // cf is rewritten
      if (tid < c.L) cf[tid] = in ? cj : -1.f;
      const int n_above = block_sum(valid && cj > c.tau, red);  // (syncs: cf visible after)
      const int n_valid = block_sum(valid, red);
      const int n = max(n_above, min(c.k_min, n_valid));
      int rank = 0;
      if (valid)
        for (int i = 0; i < nb; ++i) {
          const float ci = cf[i];
          rank += (ci >= 0.f) && (ci > cj || (ci == cj && i < tid));
        }
      const bool ch = valid && rank < n;
      if (ch) c.tok[(size_t)b * c.S + lo + tid] = c.arg[(size_t)b * c.L + tid];
      // ascending compaction of the committed positions
      const uint64_t ball = __ballot(ch);
      if (lane == 0) wcnt[wave] = __popcll(ball);
      __syncthreads();
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w];
      for (int w = 0; w < kDecideThreads / 64; ++w) cnt += wcnt[w];
      if (ch) c.cidx[off + before + lanes_below(ball)] = b * c.S + lo + tid;
      const int open = block_sum(in && !was_set && !ch, red);  // masked positions left
      if (open == 0) new_bk = bk + 1;
      if (tid == 0 && new_bk != bk) c.blk[b] = new_bk;
    }
    const int a0 = c.P + new_bk * c.L, a1 = (new_bk < c.nblk) ? min(c.S, a0 + c.L) : a0;
    for (int s = tid; s < c.S; s += kDecideThreads)
      c.flags[(size_t)b * c.S + s] = (uint8_t)(s >= a0 && s < a1);
    off += cnt;
    if (tid == 0) c.crp[b + 1] = off;
  }
}

hipError_t launch_commit(bool bf16, const CommitArgs& c, hipStream_t st) {
  if (c.B == 0) return hipSuccess;
  const dim3 grid(c.L, c.B);
  if (bf16)
    hipLaunchKernelGGL(row_conf_kernel<uint16_t>, grid, dim3(kConfThreads), 0, st, c);
  else
    hipLaunchKernelGGL(row_conf_kernel<float>, grid, dim3(kConfThreads), 0, st, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_decide_kernel, dim3(1), dim3(kDecideThreads), 0, st, c);
  return hipGetLastError();
}

// x[sel[j]] = emb[tok[sel[j]]] (the mask row for a masked position or an id outside [0, V)),
// 16 bytes per thread
__global__ __launch_bounds__(256) void embed_rows_kernel(const uint4* emb, const uint4* mask,
                                                         const int32_t* tok, const int32_t* sel,
                                                         const int32_t* rp, int B, int m_cap,
                                                         long V, int chunks, uint4* x) {
  const int M = min(rp[B], m_cap);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t j = idx / chunks;
  if (j >= (size_t)M) return;
  const int c = (int)(idx - j * chunks);
  const int flat = sel[j];
  const int t = tok[flat];
  const uint4* src = (t >= 0 && t < V) ? emb + (size_t)t * chunks : mask;
  x[(size_t)flat * chunks + c] = src[c];
}

hipError_t launch_embed_rows(int B, int m_cap, long V, size_t row_bytes, const void* emb,
                             const void* mask_emb, const int32_t* tok, const int32_t* sel,
                             const int32_t* rp, void* x, hipStream_t st) {
  if (m_cap == 0) return hipSuccess;
  const int chunks = (int)(row_bytes / 16);
  const size_t threads = (size_t)m_cap * chunks;
  hipLaunchKernelGGL(embed_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const uint4*)emb, (const uint4*)mask_emb, tok, sel, rp, B, m_cap, V, chunks,
                     (uint4*)x);
  return hipGetLastError();
}

}  // namespace dllm
