// (2) Selection + stream compaction, gfx950.
//
// ES-dLLM (German summary page) §2.B: only the top-k positions by importance go on to the
// next layers. DyLLM (French summary page) §2.A: a token is salient when its similarity falls
// below a threshold, i.e. its dissimilarity score is above it.
//
// One 1024-thread workgroup per sequence; the row's scores live in LDS as order-preserving
// uint32 keys. Top-k finds the k-th largest key with a 4-pass, 8-bit radix select (LDS
// histograms), then takes every key above it plus the lowest-positioned keys equal to it.
// Compaction walks the row in position order in 1024-wide chunks: wave ballots + mbcnt give each
// lane its rank, per-wave totals in LDS give the workgroup offset. No atomics touch global
// memory and no floating-point sum is involved: the result is bit-exact and deterministic.
//
// Each workgroup finds its output offset from the selected counts of the sequences before it, so
// one launch writes sel_idx and row_ptr with no inter-workgroup communication. A top-k count
// depends on the flags only: with no flags it is min(k, S) for every sequence (offset b min(k, S),
// no pass at all); with flags each earlier sequence's flag bytes are counted. In threshold mode
// the counts of all earlier sequences come from one pass over their flags and scores with a
// single reduction.
//
// Flag byte per position: bit 0 forced (always selected), bit 1 excluded (never a candidate, as
// the prompt in DyLLM's response-only steps, French summary page §2.C); forced wins.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// float -> uint32 whose unsigned order is the float order; -0 -> +0; NaN -> 0 (below -inf)
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int block_sum_int(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_int(v);
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) t += scratch[w];
  return t;
}

// 0 candidate, 1 forced, 2 excluded
__device__ __forceinline__ int pos_state(const SelectArgs& a, size_t i) {
  const int fl = a.force ? a.force[i] : 0;
  return (fl & 1) ? 1 : ((fl & 2) ? 2 : 0);
}

// number of positions sequences 0 .. b-1 contribute to the output
__device__ int offset_of(const SelectArgs& a, int b, int* scratch) {
  if (b == 0) return 0;
  if (a.mode == 1) {
    if (!a.force) return b * min(a.k, a.S);
    int base = 0;
    for (int r = 0; r < b; ++r) {  // per sequence: forced + min(k, candidates)
      int nf = 0;                  // forced + 65536 * excluded (S <= 8192)
      for (int s = threadIdx.x; s < a.S; s += kSelThreads) {
        const int st = pos_state(a, (size_t)r * a.S + s);
        nf += st == 1 ? 1 : (st == 2 ? 65536 : 0);
      }
      nf = block_sum_int(nf, scratch);
      base += (nf & 65535) + min(a.k, a.S - (nf & 65535) - (nf >> 16));
    }
    return base;
  }
  // threshold: forced positions plus candidates whose score is above tau, summed over b rows
  int n = 0;
  const size_t end = (size_t)b * a.S;
  for (size_t i = threadIdx.x; i < end; i += kSelThreads) {
    const int st = pos_state(a, i);
    n += st == 1 || (st == 0 && a.score[i] > a.tau);
  }
  return block_sum_int(n, scratch);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                                   // S
  uint8_t* state = reinterpret_cast<uint8_t*>(smem + a.S);  // S: 0 candidate, 1 forced, 2 excluded
  __shared__ int scratch[kSelWaves];
  __shared__ int wtot[2][kSelWaves];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_remaining;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S;

  const int base = offset_of(a, b, scratch);

  int nfx = 0;  // forced + 65536 * excluded
  for (int s = tid; s < S; s += kSelThreads) {
    float v = a.score[(size_t)b * S + s];
    const int st = pos_state(a, (size_t)b * S + s);
    keys[s] = order_key(v);
    state[s] = (uint8_t)st;
    nfx += st == 1 ? 1 : (st == 2 ? 65536 : 0);
  }
  nfx = block_sum_int(nfx, scratch);  // contains __syncthreads: keys/state visible after this

  // ---- top-k: radix select of the kk-th largest candidate key T; `remaining` = how many keys
  // equal to T are taken (the lowest positions among them)
  const bool topk = a.mode == 1;
  const int ncand = S - (nfx & 65535) - (nfx >> 16);
  const int kk = topk ? min(a.k, ncand) : 0;
  uint32_t T = 0xffffffffu;  // no key is above this one, and no key equals it
  uint32_t remaining = 0;
  if (topk && kk > 0) {
    uint32_t prefix = 0, mask = 0, rem = (uint32_t)kk;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int s = tid; s < S; s += kSelThreads) {
        uint32_t key = keys[s];
        if (state[s] == 0 && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 255-4l .. 252-4l (descending); find the bin where the running count
        // from the top first reaches rem
        uint32_t c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; tot += c[j]; }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          uint32_t up = __shfl_up(incl, o, 64);
          if (lane >= o) incl += up;
        }
        uint32_t excl = incl - tot;
        if (excl < rem && rem <= incl) {  // exactly one lane
          uint32_t run = excl;
          for (int j = 0; j < 4; ++j) {
            if (run + c[j] >= rem) {
              uint32_t bin = 255u - 4u * lane - j;
              sh_prefix = prefix | (bin << shift);
              sh_remaining = rem - run;
              break;
            }
            run += c[j];
          }
        }
      }
      __syncthreads();
      prefix = sh_prefix;
      rem = sh_remaining;
      mask |= 255u << shift;
    }
    T = prefix;
    remaining = rem;
  }

  // ---- ordered compaction
  int out = base;          // next output slot of this sequence
  uint32_t eq_seen = 0;    // candidates equal to T already passed, in position order
  for (int c0 = 0; c0 < S; c0 += kSelThreads) {
    const int s = c0 + tid;
    const bool in = s < S;
    const uint32_t key = in ? keys[s] : 0u;
    const int st = in ? state[s] : 2;
    const bool fr = st == 1;
    const bool cand = st == 0;
    const bool eq = topk && cand && key == T;
    const uint64_t eq_ball = __ballot(eq);
    if (lane == 0) wtot[0][wave] = __popcll(eq_ball);
    __syncthreads();
    uint32_t eq_before = eq_seen, eq_chunk = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      uint32_t t = wtot[0][w];
      eq_before += (w < wave) ? t : 0u;
      eq_chunk += t;
    }
    eq_before += lanes_below(eq_ball);
    bool sel;
    if (topk)
      sel = fr || (cand && (key > T || (eq && eq_before < remaining)));
    else
      sel = fr || (cand && a.score[(size_t)b * S + s] > a.tau);
    const uint64_t sel_ball = __ballot(sel);
    if (lane == 0) wtot[1][wave] = __popcll(sel_ball);
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      int t = wtot[1][w];
      before += (w < wave) ? t : 0;
      chunk += t;
    }
    if (sel) a.sel_idx[out + before + lanes_below(sel_ball)] = b * S + s;
    out += chunk;
    eq_seen += eq_chunk;
    __syncthreads();  // wtot is rewritten by the next chunk
  }
  if (tid == 0) {
    a.row_ptr[b + 1] = out;
    if (b == 0) a.row_ptr[0] = 0;
  }
}

// flags restricting a later selection to listed rows: every position excluded (2), then the
// listed ones candidates (0) or forced (1) as bit 0 of `force` says
__global__ __launch_bounds__(256) void flags_fill_kernel(uint8_t* flags, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) flags[i] = 2;
}
__global__ __launch_bounds__(256) void flags_rows_kernel(const uint8_t* force, const int32_t* sel,
                                                         const int32_t* rp, int B, int m_cap,
                                                         uint8_t* flags) {
  const int M = min(rp[B], m_cap);
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= M) return;
  const int p = sel[j];
  flags[p] = force ? (uint8_t)(force[p] & 1) : (uint8_t)0;
}

hipError_t launch_flags_from_rows(int B, int S, const uint8_t* force, const int32_t* sel,
                                  const int32_t* rp, int m_cap, uint8_t* flags, hipStream_t st) {
  const size_t n = (size_t)B * S;
  hipLaunchKernelGGL(flags_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, flags,
                     n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || m_cap == 0) return e;
  hipLaunchKernelGGL(flags_rows_kernel, dim3((unsigned)((m_cap + 255) / 256)), dim3(256), 0, st,
                     force, sel, rp, B, m_cap, flags);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  size_t lds = (size_t)a.S * 4 + (((size_t)a.S + 3) & ~(size_t)3);
  hipLaunchKernelGGL(select_kernel, dim3(a.B), dim3(kSelThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace dllm
