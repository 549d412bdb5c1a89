// (3) + (5) Gathered projections of the selected tokens, gfx950.
//
// ES-dLLM (German summary page) §2.B: only the selected positions are computed; their keys,
// values and hidden states overwrite the cached entries in place, every other entry is reused.
// DyLLM (French summary page) §2.A: the FFN runs only for salient tokens.
//
// Every projection is a dense contraction C[M, N] = X[M, K] W[N, K]^T of the M selected rows
// (compacted to consecutive rows by a gather/RMSNorm pass) with a weight stored [out, in].
// Both operands are K-contiguous, which is the operand layout of the bf16 matrix-core
// instructions: a lane supplies 8 consecutive K values of one row. The kernels multiply W
// (instruction A operand, rows = output columns n) by X (B operand, rows = tokens m), so each
// lane's accumulators are groups of 4 CONSECUTIVE output columns of one token row: every
// epilogue stores 8 or 16 contiguous bytes per lane straight into its target (q rows, K/V cache
// rows of the token's position, residual rows, scattered hidden rows).
//
// Operands reach LDS through a ring of direct-to-LDS loads. Up to 128 selected rows the products
// stream the weights (HBM-bound) with 16 x 16 x 32 blocks and narrow weight slabs, a few K splits
// filling the 256 CUs and reduced in a fixed order by a second pass (deterministic). Above that
// the products are compute-bound and use 32 x 32 x 16 blocks, which sustain about twice the
// matrix-core rate of 16 x 16 x 32 on gfx950, in 256-row tiles.
#include "common.h"
#include "kernels.h"

namespace dllm {

// =========================================================================================
// epilogues: apply to 4 consecutive columns n..n+3 of compact row j (n % 4 == 0)
// =========================================================================================
// Epilogues: row(j) prepares what depends on the compact row j only (called once per row and
// thread), operator() applies to 4 consecutive columns n..n+3 of that row (n % 4 == 0).

// quotient n / d for 0 <= n < 2^31 by multiply-high (round-up method, exact in this range)
struct FastDiv {
  uint32_t m, l, d;
  static FastDiv make(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.l = 0;
    while ((1ull << f.l) < d) ++f.l;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << f.l) - d)) / d + 1);
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const { return (__umulhi(m, n) + n) >> l; }
};

// Epilogues run in two phases per block of rows: pre(row, n) issues the loads a group of 4 output
// columns needs and returns them as loaded (no conversion, so nothing waits for them yet);
// operator()(row, n, v, pre) combines and stores. A kernel issues every pre() of a row block
// before its first store, so the block pays one memory latency instead of one per group.
struct NoPre {};
template <typename T> struct Raw4;  // 4 consecutive elements as loaded
template <> struct Raw4<float> {
  typedef float4 type;
  __device__ __forceinline__ static float4 load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  __device__ __forceinline__ static void cvt(const float4& r, float a[4]) {
    a[0] = r.x; a[1] = r.y; a[2] = r.z; a[3] = r.w;
  }
};
template <> struct Raw4<uint16_t> {  // bf16 bit patterns
  typedef uint2 type;
  __device__ __forceinline__ static uint2 load(const uint16_t* p) {
    return *reinterpret_cast<const uint2*>(p);
  }
  __device__ __forceinline__ static void cvt(const uint2& r, float a[4]) {
    a[0] = __uint_as_float(r.x << 16); a[1] = __uint_as_float(r.x & 0xffff0000u);
    a[2] = __uint_as_float(r.y << 16); a[3] = __uint_as_float(r.y & 0xffff0000u);
  }
};

template <typename T>
struct EpiQKV {  // Q -> q_sel[j]; K/V -> cache[b, hk, s, e] of the token's own position
  T* q_sel;
  T* kc;
  T* vc;
  const int32_t* sel_idx;
  int Nq, Nkv, hd_log2, S, Hkv;
  FastDiv divS;
  struct Row {
    T* q;       // q_sel row j
    size_t kv;  // element offset of cache[b, 0, s, 0]
  };
  __device__ __forceinline__ Row row(int j) const {
    const uint32_t id = (uint32_t)sel_idx[j];
    const uint32_t b = divS.div(id), s = id - b * (uint32_t)S;
    return Row{q_sel + (size_t)j * Nq, ((size_t)b * Hkv * S + s) << hd_log2};
  }
  __device__ __forceinline__ void operator()(const Row& r, int n, const float v[4]) const {
    if (n < Nq) {
      Elem<T>::store4(r.q + n, v);
      return;
    }
    int kv = n - Nq;
    T* cache = kc;
    if (kv >= Nkv) {
      kv -= Nkv;
      cache = vc;
    }
    const int hk = kv >> hd_log2, e = kv & ((1 << hd_log2) - 1);
    Elem<T>::store4(cache + r.kv + (((size_t)hk * S) << hd_log2) + e, v);
  }
  typedef NoPre Pre;
  __device__ __forceinline__ Pre pre(const Row&, int) const { return {}; }
  __device__ __forceinline__ void operator()(const Row& r, int n, const float v[4], Pre) const {
    (*this)(r, n, v);
  }
};

template <typename T>
struct EpiResidF32 {  // h[j] = h_in[sel[j]] + acc  (float32 workspace)
  float* h;
  const T* x;
  const int32_t* sel_idx;
  int d;
  struct Row {
    float* h;
    const T* x;
  };
  __device__ __forceinline__ Row row(int j) const {
    return Row{h + (size_t)j * d, x + (size_t)sel_idx[j] * d};
  }
  typedef typename Raw4<T>::type Pre;
  __device__ __forceinline__ Pre pre(const Row& r, int n) const { return Raw4<T>::load(r.x + n); }
  __device__ __forceinline__ void operator()(const Row& r, int n, const float v[4],
                                             const Pre& p) const {
    float a[4];
    Raw4<T>::cvt(p, a);
    const float o[4] = {v[0] + a[0], v[1] + a[1], v[2] + a[2], v[3] + a[3]};
    Elem<float>::store4(r.h + n, o);
  }
  __device__ __forceinline__ void operator()(const Row& r, int n, const float v[4]) const {
    (*this)(r, n, v, pre(r, n));
  }
};

template <typename T>
struct EpiResidScatter {  // h_out[sel[j]] = h[j] + acc
  T* h_out;
  const float* h;
  const int32_t* sel_idx;
  int d;
  struct Row {
    T* out;
    const float* h;
  };
  __device__ __forceinline__ Row row(int j) const {
    return Row{h_out + (size_t)sel_idx[j] * d, h + (size_t)j * d};
  }
  typedef float4 Pre;
  __device__ __forceinline__ Pre pre(const Row& r, int n) const { return Raw4<float>::load(r.h + n); }
  __device__ __forceinline__ void operator()(const Row& r, int n, const float v[4],
                                             const Pre& p) const {
    float a[4];
    Raw4<float>::cvt(p, a);
    const float o[4] = {v[0] + a[0], v[1] + a[1], v[2] + a[2], v[3] + a[3]};
    Elem<T>::store4(r.out + n, o);
  }
  __device__ __forceinline__ void operator()(const Row& r, int n, const float v[4]) const {
    (*this)(r, n, v, pre(r, n));
  }
};

template <typename T>
struct EpiSwiGLU {  // z[j, n] = silu(gate) * up
  T* z;
  int F;
  typedef T* Row;
  __device__ __forceinline__ Row row(int j) const { return z + (size_t)j * F; }
  __device__ __forceinline__ void operator()(Row r, int n, const float g[4],
                                             const float u[4]) const {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = g[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[i])) * u[i];
    Elem<T>::store4(r + n, o);
  }
  typedef NoPre Pre;
  __device__ __forceinline__ Pre pre(Row, int) const { return {}; }
  __device__ __forceinline__ void operator()(Row r, int n, const float g[4], const float u[4],
                                             Pre) const {
    (*this)(r, n, g, u);
  }
};

__device__ __forceinline__ int live_rows(const int32_t* row_ptr, int B, int m_cap) {
  return min(row_ptr[B], m_cap);
}

// =========================================================================================
// gather + RMSNorm: out[j] = in[row(j)] / sqrt(mean(in^2) + eps) * g, row(j) = sel[j] or j
// =========================================================================================
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const Tin* in, const int32_t* sel_idx,
                                                           const Tout* g, Tout* out, int d,
                                                           float eps, const int32_t* row_ptr,
                                                           int B, int m_cap) {
  const int j = blockIdx.x;
  if (j >= live_rows(row_ptr, B, m_cap)) return;
  const size_t row = sel_idx ? (size_t)sel_idx[j] : (size_t)j;
  const Tin* x = in + row * d;
  __shared__ float red[4];
  float ss = 0.f;
  for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
    float v[8];
    Elem<Tin>::load8(x + i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
    float v[4], gv[4];
    Elem<Tin>::load4(x + i, v);
    Elem<Tout>::load4(g + i, gv);
    const float o[4] = {v[0] * r * gv[0], v[1] * r * gv[1], v[2] * r * gv[2], v[3] * r * gv[3]};
    Elem<Tout>::store4(out + (size_t)j * d + i, o);
  }
}

// Row-resident variant (d <= CH * 2048): thread t owns 8-element chunks t, t + 256, ...; the row
// is loaded once (all loads issued together) and normalised from registers. Same sums in the same
// order as the kernel above.
template <typename Tin, typename Tout, int CH>
__global__ __launch_bounds__(256) void rmsnorm_rows_reg_kernel(const Tin* in, const int32_t* sel_idx,
                                                               const Tout* g, Tout* out, int d,
                                                               float eps, const int32_t* row_ptr,
                                                               int B, int m_cap) {
  const int j = blockIdx.x;
  if (j >= live_rows(row_ptr, B, m_cap)) return;
  const size_t row = sel_idx ? (size_t)sel_idx[j] : (size_t)j;
  const Tin* x = in + row * d;
  __shared__ float red[4];
  float v[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = 8 * (threadIdx.x + 256 * c);
    if (i < d) Elem<Tin>::load8(x + i, v[c]);
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
    if (8 * (threadIdx.x + 256 * c) < d) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[c][e], v[c][e], ss);
    }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = 8 * (threadIdx.x + 256 * c);
    if (i < d) {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        float gv[4];
        Elem<Tout>::load4(g + i + 4 * hlf, gv);
        const float o[4] = {v[c][4 * hlf] * r * gv[0], v[c][4 * hlf + 1] * r * gv[1],
                            v[c][4 * hlf + 2] * r * gv[2], v[c][4 * hlf + 3] * r * gv[3]};
        Elem<Tout>::store4(out + (size_t)j * d + i + 4 * hlf, o);
      }
    }
  }
}

// gather + RMSNorm of the selected rows (row-resident kernel up to d = 8192)
template <typename Tin, typename Tout>
static void launch_rmsnorm_rows(const Tin* in, const int32_t* sel_idx, const Tout* g, Tout* out,
                                int d, float eps, const int32_t* row_ptr, int B, int m_cap,
                                hipStream_t st) {
  const dim3 grid(m_cap), blk(256);
  if (d % 8 == 0 && d <= 2048)
    hipLaunchKernelGGL((rmsnorm_rows_reg_kernel<Tin, Tout, 1>), grid, blk, 0, st, in, sel_idx, g, out, d, eps, row_ptr, B, m_cap);
  else if (d % 8 == 0 && d <= 4096)
    hipLaunchKernelGGL((rmsnorm_rows_reg_kernel<Tin, Tout, 2>), grid, blk, 0, st, in, sel_idx, g, out, d, eps, row_ptr, B, m_cap);
  else if (d % 8 == 0 && d <= 8192)
    hipLaunchKernelGGL((rmsnorm_rows_reg_kernel<Tin, Tout, 4>), grid, blk, 0, st, in, sel_idx, g, out, d, eps, row_ptr, B, m_cap);
  else
    hipLaunchKernelGGL((rmsnorm_rows_kernel<Tin, Tout>), grid, blk, 0, st, in, sel_idx, g, out, d, eps, row_ptr, B, m_cap);
}

// =========================================================================================
// bf16 matrix-core GEMM fed by a direct-to-LDS load ring
// =========================================================================================
// Per K step of 64 a workgroup stages [BM rows of X ; BN rows of W] x 128 bytes in one slot of
// an ST-slot LDS ring. global_load_lds_dwordx4 moves 64 lanes x 16 B (8 rows) per wave
// instruction from global memory straight into 1 KB of LDS, without passing through registers,
// so ST - 1 K steps stay in flight while the matrix cores work on the oldest slot. One
// s_barrier per K step: the slot refilled at step kt is the one every wave finished at kt - 1.
// Inside a 128-byte row the 16-byte chunk c is stored at c ^ g(row), g(r) = (r & 7) ^ (r >> 3 & 1),
// so the 16 lanes that read one MFMA fragment (16 rows, one chunk) hit distinct bank groups.
//
// Tile shapes (host plan): at M <= 128 the products stream weights from HBM, and the plan picks
// BN so that about 256 workgroups each own a disjoint weight slab (QKV: BN = 48 -> 256 slabs of
// the 12288 rows; gate/up: 48 + 48 rows); 4 waves split the M rows, so every X row is read from
// LDS once. Narrow N (4096) uses BN = 64 and a few K splits. At larger M, 128 x 128 tiles with
// 2 x 2 waves.

// Tiles of the 32 x 32 x 16 kernel used when more than kWsMaxRows rows are selected: 256 x 256
// and 128 x 256 (the more tiles, the better they balance over the CUs; plan_g32 chooses), both
// with 8 waves (wave tiles 64 x 128 as 4 x 2, and 64 x 64 as 2 x 4) and 64-wide K slots, so that
// every row a direct-to-LDS load touches is one whole 128-byte line (32-wide slots fetch half
// lines: twice the L1 -> L2 requests for the same bytes, and more time waiting for them). The
// 256 x 256 tile's slots are 64 KB, so it runs a 2-slot ring; the 128 x 256 tile a 3-slot one.
// Measured on the 32-layer batched LLaDA-8B step: 39.8 -> 37.9 ms against 32-wide slots in a
// 4-slot ring (a 4-wave 2 x 2 layout of 128 x 128 wave tiles, half the LDS reads per product,
// was slower: 38.8 ms).
struct G32Shape {
  int bm, bn, bk, wm, wn, st;
};
constexpr G32Shape kG32Big{256, 256, 64, 4, 2, 2};  // bm, bn, bk, wm, wn, ring slots
constexpr G32Shape kG32Mid{128, 256, 64, 2, 4, 3};

// ring slots that fit in the 160 KB of LDS a workgroup may use, capped at `want`
constexpr int ring_slots(int bm, int bn, int bk, int want) {
  return (160 * 1024) / ((bm + bn) * bk * 2) < want ? (160 * 1024) / ((bm + bn) * bk * 2) : want;
}

struct GemmArgs {
  const uint16_t* X;   // [m_cap, K] compact activations
  const uint16_t* W;   // [N, K]  (SwiGLU: gate)
  const uint16_t* W2;  // SwiGLU: up [N, K]; else unused
  int N, K, kchunk;
  int group;           // M-tiles walked together by the 32x32 kernel's tile order
  const int32_t* row_ptr;
  int B, m_cap;
  float* partial;      // [splits, m_cap, N] when split, else NULL
  int row0;            // first row of this launch's tiles (32 x 32 x 16 kernel)
};

// 16-byte chunk swizzle for rows of 128 bytes (8 chunks) or 256 bytes (16 chunks): the 16 rows
// read by one MFMA fragment land on distinct bank groups for either bank width.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return r & 15;
}

// wait until at most N vector-memory operations of this wave are outstanding (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// workgroup barrier without the release/acquire fences of __syncthreads(): the fence would make
// the compiler wait for every load in flight, which defeats the ring
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void;

template <int PB, int A>
__device__ __forceinline__ void wait_batches(int ahead) {  // wait until <= ahead*PB ops pending
  if constexpr (A == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= A)
      wait_vm<A * PB>();
    else
      wait_batches<PB, A - 1>(ahead);
  }
}

// One ring slot = [BM rows of X ; BN rows of W] x BK columns (BK * 2 bytes per row).
template <int BM, int BN, int BK, int NW, bool SWIGLU>
__device__ __forceinline__ void issue_stage(const GemmArgs& g, char* slot, int m0, int n0, int M,
                                            int k0, int wave, int lane) {
  constexpr int RB = BK * 2;         // bytes per row
  constexpr int CPR = RB / 16;       // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;     // rows per wave instruction
  constexpr int I = (BM + BN) / RPI; // wave instructions per slot
  constexpr int PER = (I + NW - 1) / NW;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = wave + NW * i;
    if (j < I) {
      const int row = RPI * j + lane / CPR;
      const int c = (lane % CPR) ^ swz<CPR>(row);
      const uint16_t* src;
      if (row < BM) {
        // rows past M repeat row M-1: their products land in rows that are never stored
        src = g.X + (size_t)min(m0 + row, M - 1) * g.K;
      } else {
        const int r = row - BM;
        if constexpr (SWIGLU) {
          const int n = min(n0 + (r % (BN / 2)), g.N - 1);
          src = ((r < BN / 2) ? g.W : g.W2) + (size_t)n * g.K;
        } else {
          src = g.W + (size_t)min(n0 + r, g.N - 1) * g.K;
        }
      }
      __builtin_amdgcn_global_load_lds(src + k0 + 8 * c, (lds_void*)(slot + j * 1024), 16, 0, 0);
    }
  }
}

// first W row (within the W part of the slot) of the wave's n-block j
template <int BN, int WN, int NB, bool SWIGLU>
__device__ __forceinline__ int wrow(int wn, int j) {
  if constexpr (SWIGLU) {
    constexpr int HW = BN / 2 / WN;  // gate rows per wave
    return (j < NB / 2) ? wn * HW + 16 * j : BN / 2 + wn * HW + 16 * (j - NB / 2);
  } else {
    return wn * (BN / WN) + 16 * j;
  }
}

template <int BK>
__device__ __forceinline__ bf16x8 frag(const char* slot, int row, int chunk) {
  constexpr int RB = BK * 2;
  return *reinterpret_cast<const bf16x8*>(slot + row * RB + ((chunk ^ swz<RB / 16>(row)) << 4));
}

// BM x BN tile, BK columns per ring slot, ST slots, NW waves as WM x WN.
template <int BM, int BN, int BK, int WM, int WN, int ST, bool SWIGLU, class Epi>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmArgs g, Epi epi) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int SLOT = (BM + BN) * BK * 2;
  constexpr int NMIN = (BM + BN) * BK * 2 / 1024 / NW;  // DMA instructions per wave per slot (lower bound)
  static_assert(MB >= 1 && NB >= 1 && (!SWIGLU || NB % 2 == 0), "tile");
  static_assert(ST >= 3 && (ST - 2) * NMIN < 64 && NMIN >= 1, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[ST * SLOT];

  const int M = live_rows(g.row_ptr, g.B, g.m_cap);
  const int m0 = blockIdx.y * BM;
  if (m0 >= M) return;
  const int n0 = blockIdx.x * (SWIGLU ? BN / 2 : BN);
  const int kb = blockIdx.z * g.kchunk;
  const int nk = (min(g.K, kb + g.kchunk) - kb) / BK;  // >= 1 by the plan
  // All workgroups walk K in the same order: tiles that share an X slice then read it at about
  // the same time, so it is fetched into each L2 once instead of being evicted by the weight
  // stream between readers.

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lc = lane >> 4;

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk)
      issue_stage<BM, BN, BK, NW, SWIGLU>(g, ring + s * SLOT, m0, n0, M,
                                          kb + s * BK, wave, lane);

  for (int kt = 0; kt < nk; ++kt) {
    wait_batches<NMIN, ST - 2>(nk - 1 - kt);  // slots issued after slot kt: min(ST-2, nk-1-kt)
    wg_barrier();
    if (kt + ST - 1 < nk)
      issue_stage<BM, BN, BK, NW, SWIGLU>(g, ring + ((kt + ST - 1) % ST) * SLOT, m0, n0, M,
                                          kb + (kt + ST - 1) * BK, wave, lane);
    const char* slot = ring + (kt % ST) * SLOT;
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8 xf[MB], wf[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) xf[i] = frag<BK>(slot, wm * WTM + 16 * i + lr, 4 * kk + lc);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        wf[j] = frag<BK>(slot, BM + wrow<BN, WN, NB, SWIGLU>(wn, j) + lr, 4 * kk + lc);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
    }
  }

  // acc[i][j][r] = C[m = m0 + wm WTM + 16 i + lr][n = n0 + (n-block j) + 4 lc + r]
  // Per 16-row block: the epilogue's loads first, then the masked stores, with the branches
  // outside the store sequences (as in the 32 x 32 x 16 kernel's epilogue).
  constexpr int NJ = SWIGLU ? NB / 2 : NB;
  const bool cols_in = n0 + (SWIGLU ? BN / 2 : BN) <= g.N;
  auto col = [&](int j) __attribute__((always_inline)) {
    return n0 + wrow<BN, WN, NB, SWIGLU>(wn, j) + 4 * lc;
  };
  auto gate = [&](int i, int j, float (&v)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r];
  };
  if (g.partial) {  // K-split partials: [split][row][N] ([split][row][gate 0..N | up N..2N])
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm * WTM + 16 * i + lr;
      if (m >= M) continue;
      float* pr = g.partial + ((size_t)blockIdx.z * g.m_cap + m) * ((SWIGLU ? 2 : 1) * (size_t)g.N);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = col(j);
        if (!cols_in && n >= g.N) continue;
        float v[4];
        gate(i, j, v);
        Elem<float>::store4(pr + n, v);
        if constexpr (SWIGLU) {
          gate(i, j + NB / 2, v);
          Elem<float>::store4(pr + g.N + n, v);
        }
      }
    }
    return;
  }
  decltype(epi.row(0)) ers[MB];  // row addresses of every block before the first store
#pragma unroll
  for (int i = 0; i < MB; ++i) ers[i] = epi.row(min(m0 + wm * WTM + 16 * i + lr, M - 1));
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * WTM + 16 * i + lr;
    const auto& er = ers[i];
    typename Epi::Pre pre[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = col(j);
      pre[j] = epi.pre(er, (cols_in || n < g.N) ? n : 0);
    }
    if (m >= M) continue;
    auto store = [&](int j) __attribute__((always_inline)) {
      const int n = col(j);
      float v[4];
      gate(i, j, v);
      if constexpr (SWIGLU) {
        float u[4];
        gate(i, j + NB / 2, u);
        epi(er, n, v, u, pre[j]);
      } else {
        epi(er, n, v, pre[j]);
      }
    };
    if (cols_in) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) store(j);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (col(j) < g.N) store(j);
    }
  }
}

// Same ring, 32 x 32 x 16 products (about twice the sustained rate of 16 x 16 x 32 on gfx950).
// A lane supplies 8 consecutive K values (k-step half lane/32) of row lane%32 of a 32-row
// fragment; its 16 accumulators of a block are C^T[n = 8 (r/4) + 4 (lane/32) + r%4][m = lane%32],
// i.e. 4 groups of 4 consecutive output columns of one token row. Chunk swizzle for rows of CPR
// 16-byte chunks: the 16 rows read by a quarter-wave (one chunk each) land on 16 distinct bank
// positions of the 256 bank bytes.
template <int CPR>
__device__ __forceinline__ int swz32(int r) {
  if constexpr (CPR == 4) return (r >> 2) & 3;
  else if constexpr (CPR == 8) return (r >> 1) & 7;
  else return r & 15;
}

template <int BM, int BN, int BK, int NW, bool SWIGLU>
__device__ __forceinline__ void issue_stage32(const GemmArgs& g, char* slot, int m0, int n0, int M,
                                              int k0, int wave, int lane) {
  constexpr int RB = BK * 2;         // bytes per row
  constexpr int CPR = RB / 16;       // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;     // rows per wave instruction
  constexpr int I = (BM + BN) / RPI; // wave instructions per slot
  constexpr int PER = (I + NW - 1) / NW;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = wave + NW * i;
    if (I % NW == 0 || j < I) {
      const int row = RPI * j + lane / CPR;
      const int c = (lane % CPR) ^ swz32<CPR>(row);
      const uint16_t* src;
      if (row < BM) {
        src = g.X + (size_t)min(m0 + row, M - 1) * g.K;
      } else {
        const int r = row - BM;
        if constexpr (SWIGLU) {
          const int n = min(n0 + (r % (BN / 2)), g.N - 1);
          src = ((r < BN / 2) ? g.W : g.W2) + (size_t)n * g.K;
        } else {
          src = g.W + (size_t)min(n0 + r, g.N - 1) * g.K;
        }
      }
      __builtin_amdgcn_global_load_lds(src + k0 + 8 * c, (lds_void*)(slot + j * 1024), 16, 0, 0);
    }
  }
}

// first W row (within the W part of the slot) of the wave's 32-row n-block j
template <int BN, int WN, int NB, bool SWIGLU>
__device__ __forceinline__ int wrow32(int wn, int j) {
  if constexpr (SWIGLU) {
    constexpr int HW = BN / 2 / WN;  // gate rows per wave
    return (j < NB / 2) ? wn * HW + 32 * j : BN / 2 + wn * HW + 32 * (j - NB / 2);
  } else {
    return wn * (BN / WN) + 32 * j;
  }
}

template <int BK>
__device__ __forceinline__ bf16x8 frag32(const char* slot, int row, int chunk) {
  constexpr int RB = BK * 2;
  return *reinterpret_cast<const bf16x8*>(slot + row * RB + ((chunk ^ swz32<RB / 16>(row)) << 4));
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile of this workgroup (32 x 32 x 16 kernels). Workgroups are dispatched to the 8 XCDs
// round-robin by linear id, so ids x, x+8, x+16, ... share one L2. They are given one contiguous
// run of the tile sequence, which walks g.group M-tiles at a time across all N-tiles: the tiles
// resident on an XCD together then share few X and W panels.
__device__ __forceinline__ void tile_order(const GemmArgs& g, int& mt, int& nt) {
  const int NT = gridDim.x, MT = gridDim.y, T = NT * MT;
  const int lin = blockIdx.x + blockIdx.y * NT;
  const int tt = (T % 8 == 0) ? (lin % 8) * (T / 8) + lin / 8 : lin;
  const int gm = g.group * NT;
  const int first = (tt / gm) * g.group;
  const int gsize = min(MT - first, g.group);
  mt = first + (tt % gm) % gsize;
  nt = (tt % gm) / gsize;
}

// Epilogue of a 32 x 32 x 16 tile: the wave's accumulators (MB x NB blocks of 32 x 32) go through
// `epi` (or, for a K split, into the float32 partials of split `split`).
template <int BM, int BN, int WM, int WN, bool SWIGLU, class Epi, int MB, int NB>
__device__ __forceinline__ void epilogue32(const GemmArgs& g, const Epi& epi, f32x16 (&acc)[MB][NB],
                                           int m0, int n0, int M, int wm, int wn, int l32, int h,
                                           int split) {
  constexpr int WTM = BM / WM;
  // acc[i][j][4 q + r] = C[m = m0 + wm WTM + 32 i + l32][n = n0 + (n-block j) + 8 q + 4 h + r]
  // Per 32-row block: every load the epilogue needs is issued first (rows past M load row M-1,
  // columns past N column 0), then the stores, masked to the rows below M (and, when the tile
  // reaches past N, to the columns below it). The branches are uniform and sit outside the
  // store sequences, so each store waits only for its own loads (on gfx9 stores count against
  // the same counter as loads: a wait placed at a branch join would wait for every earlier
  // store too).
  constexpr int NJ = SWIGLU ? NB / 2 : NB;
  const bool cols_in = n0 + (SWIGLU ? BN / 2 : BN) <= g.N;
  auto col = [&](int q, int j) __attribute__((always_inline)) {
    return n0 + wrow32<BN, WN, NB, SWIGLU>(wn, j) + 8 * q + 4 * h;
  };
  auto gate = [&](int i, int j, int q, float (&v)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
  };
  if (g.partial) {  // K-split partials: [split][row][N] ([split][row][gate 0..N | up N..2N])
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm * WTM + 32 * i + l32;
      if (m >= M) continue;
      float* pr = g.partial + ((size_t)split * g.m_cap + m) * ((SWIGLU ? 2 : 1) * (size_t)g.N);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = col(q, j);
          if (!cols_in && n >= g.N) continue;
          float v[4];
          gate(i, j, q, v);
          Elem<float>::store4(pr + n, v);
          if constexpr (SWIGLU) {
            gate(i, j + NB / 2, q, v);
            Elem<float>::store4(pr + g.N + n, v);
          }
        }
    }
    return;
  }
  // the rows' addresses (which may load an index) for every block before the first store
  decltype(epi.row(0)) ers[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) ers[i] = epi.row(min(m0 + wm * WTM + 32 * i + l32, M - 1));
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * WTM + 32 * i + l32;
    const auto& er = ers[i];
    typename Epi::Pre pre[4][NJ];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = col(q, j);
        pre[q][j] = epi.pre(er, (cols_in || n < g.N) ? n : 0);
      }
    if (m >= M) continue;
    auto store = [&](int q, int j) __attribute__((always_inline)) {
      const int n = col(q, j);
      float v[4];
      gate(i, j, q, v);
      if constexpr (SWIGLU) {
        float u[4];
        gate(i, j + NB / 2, q, u);
        epi(er, n, v, u, pre[q][j]);
      } else {
        epi(er, n, v, pre[q][j]);
      }
    };
    if (cols_in) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NJ; ++j) store(q, j);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (col(q, j) < g.N) store(q, j);
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, int ST, bool SWIGLU, class Epi>
__global__ __launch_bounds__(64 * WM * WN) void gemm32_bf16_kernel(GemmArgs g, Epi epi) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int SLOT = (BM + BN) * BK * 2;
  constexpr int NMIN = (BM + BN) * BK * 2 / 1024 / NW;  // DMA instructions per wave per slot (lower bound)
  static_assert(MB >= 1 && NB >= 1 && (!SWIGLU || NB % 2 == 0), "tile");
  static_assert(ST >= 2 && (ST < 3 || (ST - 2) * NMIN < 64) && NMIN >= 1 && NMIN < 64, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[ST * SLOT];

  const int M = live_rows(g.row_ptr, g.B, g.m_cap);
  int mt, nt;
  tile_order(g, mt, nt);
  const int m0 = g.row0 + mt * BM;
  if (m0 >= M) return;
  const int n0 = nt * (SWIGLU ? BN / 2 : BN);
  const int kb = blockIdx.z * g.kchunk;
  const int nk = (min(g.K, kb + g.kchunk) - kb) / BK;  // >= 1 by the plan

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, h = lane >> 5;
#define ISSUE32(SLOTP, K0) \
  issue_stage32<BM, BN, BK, NW, SWIGLU>(g, (SLOTP), m0, n0, M, (K0), wave, lane)

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Two register buffers of fragments: A holds the first k-step of slot kt (read at the end of
  // the previous slot), B the remaining ones. The barrier that lets slot kt+1 be read and slot kt-1
  // be refilled sits between the first k-step's products and the rest, so the products of the
  // first k-step cover the barrier and the latency of the next reads.
  constexpr int KS = BK / 16;  // k-steps per slot
  bf16x8 xa[MB], wa[NB];
  auto read_frags = [&](const char* slot, int kk, bf16x8 (&xf)[MB], bf16x8 (&wf)[NB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i) xf[i] = frag32<BK>(slot, wm * WTM + 32 * i + l32, 2 * kk + h);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      wf[j] = frag32<BK>(slot, BM + wrow32<BN, WN, NB, SWIGLU>(wn, j) + l32, 2 * kk + h);
  };
  auto products = [&](const bf16x8 (&xf)[MB], const bf16x8 (&wf)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
  };
  // order of one k-step's region: each fragment read of the next k-step right after one
  // product, then the remaining products, so the reads' latency hides under the products
  // (measured on the 32-layer LLaDA step, 8 x 205 rows: 42.0 -> 40.6 ms per step)
  auto interleave = [&]() __attribute__((always_inline)) {
    constexpr int R = MB + NB, P = MB * NB;
    static_assert(P >= R, "more reads than products");
#pragma unroll
    for (int i = 0; i < R; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (P > R) __builtin_amdgcn_sched_group_barrier(0x008, P - R, 0);
  };

  if constexpr (ST == 2) {
    // Two slots: slot kt+1 loads while slot kt is multiplied. At the last k-step of slot kt
    // every wave has issued its reads of it; once they have returned (lgkmcnt) and slot kt+1 has
    // landed (vmcnt), a barrier lets slot kt+2 refill slot kt and the first fragments of slot
    // kt+1 be read, while the last k-step's products of slot kt run.
    ISSUE32(ring, kb);
    if (nk > 1) ISSUE32(ring + SLOT, kb + BK);
    if (nk > 1) wait_vm<NMIN>(); else wait_vm<0>();
    wg_barrier();
    read_frags(ring, 0, xa, wa);
    for (int kt = 0; kt < nk; ++kt) {
      const char* slot = ring + (kt & 1) * SLOT;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        bf16x8 xn[MB], wn[NB];
        if (kk + 1 < KS) {
          read_frags(slot, kk + 1, xn, wn);
        } else {
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this stage's reads are done
          wait_vm<0>();                       // stage kt+1 landed
          wg_barrier();
          if (kt + 2 < nk) ISSUE32(ring + (kt & 1) * SLOT, kb + (kt + 2) * BK);
          read_frags(ring + ((kt + 1) & 1) * SLOT, 0, xn, wn);  // stale on the last stage, unused
        }
        products(xa, wa);
        interleave();
#pragma unroll
        for (int i = 0; i < MB; ++i) xa[i] = xn[i];
#pragma unroll
        for (int j = 0; j < NB; ++j) wa[j] = wn[j];
      }
    }
  } else {
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk)
      ISSUE32(ring + s * SLOT, kb + s * BK);
  wait_batches<NMIN, (ST >= 2 ? ST - 2 : 0)>(nk - 1);  // slot 0 landed (slots issued after it: min(ST-2, nk-1))
  wg_barrier();
  read_frags(ring, 0, xa, wa);

  for (int kt = 0; kt < nk; ++kt) {
    const char* slot = ring + (kt % ST) * SLOT;
    bf16x8 xb[MB], wb[NB];
    read_frags(slot, 1, xb, wb);
    products(xa, wa);
    interleave();
    if (kt + 1 < nk) {
      // slot kt+1 landed (slots issued after it: min(ST-3, nk-2-kt) + this iteration's none yet)
      wait_batches<NMIN, (ST >= 3 ? ST - 3 : 0)>(nk - 2 - kt);
      wg_barrier();  // every wave finished reading slot kt-1
      if (kt + ST - 1 < nk)
        ISSUE32(ring + ((kt + ST - 1) % ST) * SLOT, kb + (kt + ST - 1) * BK);
    }
#pragma unroll
    for (int kk = 1; kk < KS; ++kk) {
      if (kk + 1 < KS) {
        bf16x8 xc[MB], wc[NB];
        read_frags(slot, kk + 1, xc, wc);
        products(xb, wb);
        interleave();
#pragma unroll
        for (int i = 0; i < MB; ++i) xb[i] = xc[i];
#pragma unroll
        for (int j = 0; j < NB; ++j) wb[j] = wc[j];
      } else {
        // unconditional (the last iteration reads a stale slot and never uses it): a read under a
        // branch would make the wait before these products cover it on both paths
        read_frags(ring + ((kt + 1) % ST) * SLOT, 0, xa, wa);
        products(xb, wb);
        interleave();
      }
    }
  }

  }
#undef ISSUE32
  epilogue32<BM, BN, WM, WN, SWIGLU>(g, epi, acc, m0, n0, M, wm, wn, l32, h, blockIdx.z);
}

// fixed-order sum of the K-split gate and up partials, then SiLU(gate) * up
template <class Epi>
__global__ __launch_bounds__(256) void splitk_swiglu_kernel(const float* partial, int splits,
                                                            int N, const int32_t* row_ptr, int B,
                                                            int m_cap, Epi epi) {
  const int M = live_rows(row_ptr, B, m_cap);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int groups = N / 4;
  const int m = (int)(idx / groups);
  if (m >= M) return;
  const int n = (int)(idx - (size_t)m * groups) * 4;
  float gv[4] = {0.f, 0.f, 0.f, 0.f}, uv[4] = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) {
    const float* pr = partial + ((size_t)z * m_cap + m) * (2 * (size_t)N);
    float a[4], b[4];
    Elem<float>::load4(pr + n, a);
    Elem<float>::load4(pr + N + n, b);
    for (int e = 0; e < 4; ++e) { gv[e] += a[e]; uv[e] += b[e]; }
  }
  epi(epi.row(m), n, gv, uv);
}

// fixed-order sum of the K-split partials, then the epilogue. SPLITS > 0: that many partials,
// all loaded before the sum; SPLITS == 0: `splits` of them, one after the other.
template <class Epi, int SPLITS = 0>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* partial, int splits,
                                                            int N, const int32_t* row_ptr, int B,
                                                            int m_cap, Epi epi) {
  const int M = live_rows(row_ptr, B, m_cap);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;  // one 4-column group
  const int groups = N / 4;
  const int m = (int)(idx / groups);
  if (m >= M) return;
  const int n = (int)(idx - (size_t)m * groups) * 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SPLITS > 0) {
    float p[SPLITS][4];
#pragma unroll
    for (int z = 0; z < SPLITS; ++z) Elem<float>::load4(partial + ((size_t)z * m_cap + m) * N + n, p[z]);
#pragma unroll
    for (int z = 0; z < SPLITS; ++z) {
      v[0] += p[z][0]; v[1] += p[z][1]; v[2] += p[z][2]; v[3] += p[z][3];
    }
  } else {
    for (int z = 0; z < splits; ++z) {
      float p[4];
      Elem<float>::load4(partial + ((size_t)z * m_cap + m) * N + n, p);
      v[0] += p[0]; v[1] += p[1]; v[2] += p[2]; v[3] += p[3];
    }
  }
  epi(epi.row(m), n, v);
}

// =========================================================================================
// float32 path (VALU): 64 x 64 tiles, 16 K per step, 4 x 4 outputs per thread
// =========================================================================================
struct GemmArgsF32 {
  const float* X;
  const float* W;
  const float* W2;
  int N, K;
  const int32_t* row_ptr;
  int B, m_cap;
};

template <bool SWIGLU, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF32 g, Epi epi) {
  constexpr int T = 64, BK = 16;
  __shared__ float sX[BK][T + 4];
  __shared__ float sW[BK][T + 4];
  __shared__ float sU[SWIGLU ? BK : 1][T + 4];
  const int M = live_rows(g.row_ptr, g.B, g.m_cap);
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  if (m0 >= M) return;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    {
      const int r = t >> 2, kc = (t & 3) * 4;
      float4 xv = (m0 + r < M) ? *reinterpret_cast<const float4*>(g.X + (size_t)(m0 + r) * g.K +
                                                                  k0 + kc)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 wv = (n0 + r < g.N) ? *reinterpret_cast<const float4*>(g.W + (size_t)(n0 + r) * g.K +
                                                                    k0 + kc)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
      sX[kc][r] = xv.x; sX[kc + 1][r] = xv.y; sX[kc + 2][r] = xv.z; sX[kc + 3][r] = xv.w;
      sW[kc][r] = wv.x; sW[kc + 1][r] = wv.y; sW[kc + 2][r] = wv.z; sW[kc + 3][r] = wv.w;
      if constexpr (SWIGLU) {
        float4 uv = (n0 + r < g.N) ? *reinterpret_cast<const float4*>(
                                         g.W2 + (size_t)(n0 + r) * g.K + k0 + kc)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        sU[kc][r] = uv.x; sU[kc + 1][r] = uv.y; sU[kc + 2][r] = uv.z; sU[kc + 3][r] = uv.w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sX[k][ty * 4 + i]; b[i] = sW[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      if constexpr (SWIGLU) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = sU[k][tx * 4 + i];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
      }
    }
    __syncthreads();
  }
  const int n = n0 + tx * 4;
  if (n >= g.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    if constexpr (SWIGLU)
      epi(epi.row(m), n, acc[i], accu[i]);
    else
      epi(epi.row(m), n, acc[i]);
  }
}

// =========================================================================================
// host side: plans, workspace and launches
// =========================================================================================
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// Plans of the 32 x 32 x 16 kernel (more than kWsMaxRows rows): the tile (256 x 256 or
// 128 x 256) and K split (1, 2 or 4; the SwiGLU tiles never split) of least estimated time.
// Workgroups run in rounds of one per CU; a round of a tile takes its flops at the tile's
// per-CU rate plus a fixed cost, and a split adds the pass that sums the float32 partials.
// The rates, fixed cost and reduction bandwidth were fitted to the measured times of 8 tile x
// split plans of the four projections of the LLaDA-8B and Dream-7B layers at 320-1640 rows
// (MI355X, kernel traces): the chosen plan is 1.5% slower than the fastest one on average, 23%
// at worst (W_o of Dream-7B at 1632 rows), where the tile chosen before by row count alone was
// up to 1.4x slower. Rows are rounded up to 128, so the plan is the same for every row count
// of one 128-row interval.
static GemmPlan plan_g32(int rows, int N, int K, bool swiglu) {
  constexpr double kRate[2][2] = {{6.35e6, 5.42e6},   // flops per us per CU: {256, 128} rows,
                                  {7.16e6, 5.73e6}};  // without / with SwiGLU
  constexpr double kRoundUs = 9.4, kReduceBytesPerUs = 6.0e6, kReduceUs = 2.0, kSecondLaunchUs = 3.0;
  const double mp = (double)((rows + 127) / 128 * 128);
  const G32Shape cand[2] = {kG32Big, kG32Mid};
  GemmPlan best{};
  double best_t = 0.0;
  for (int c = 0; c < 2; ++c) {
    const G32Shape& t = cand[c];
    const int cols = swiglu ? t.bn / 2 : t.bn;
    const long tiles = (long)((N + cols - 1) / cols) * (long)((mp + t.bm - 1) / t.bm);
    for (int s = 1; s <= (swiglu ? 1 : 4); s *= 2) {
      if (s > 1 && (K + s - 1) / s < 512) break;
      const long wg = tiles * s;
      const long rounds = (wg + 255) / 256;
      const int kc = ((K + s - 1) / s + t.bk - 1) / t.bk * t.bk;
      double us = rounds * (2.0 * t.bm * t.bn * kc / kRate[swiglu][c] + kRoundUs);
      if (s > 1) us += (double)s * mp * N * 4.0 / kReduceBytesPerUs + kReduceUs;
      if (best_t == 0.0 || us < best_t) {
        best_t = us;
        best = GemmPlan{t.bm, t.bn, t.bk, t.wm, t.wn, t.st, s, 32};
      }
    }
  }
  // Two parts: the first rows on 256-row tiles, the remainder on 128-row tiles, in two launches
  // (one round each when that fits), where one tile shape alone leaves a partial last round.
  // Taken only when the estimate is at least 5% below the best single plan (the rate model is
  // off by up to ~20% on single shapes). Measured on MI355X, LLaDA-8B QKV projection at 1640
  // rows: 1024 + 616 rows 200.4 us against 224.6 us on 128-row tiles alone (batched step 37.59 ->
  // 36.95 ms); Dream-7B QKV at 8192 rows 302 vs 325 us, at 656 rows 50.9 vs 56.8 us.
  const int cols = swiglu ? kG32Big.bn / 2 : kG32Big.bn;
  const long nt = (N + cols - 1) / cols;
  for (int r1 = 256; r1 + 128 <= (int)mp; r1 += 256) {
    const long t1 = nt * (r1 / 256), t2 = nt * (long)((mp - r1 + 127) / 128);
    const double us = (double)((t1 + 255) / 256) *
                          (2.0 * 256 * kG32Big.bn * K / kRate[swiglu][0] + kRoundUs) +
                      (double)((t2 + 255) / 256) *
                          (2.0 * 128 * kG32Mid.bn * K / kRate[swiglu][1] + kRoundUs) +
                      kSecondLaunchUs;
    if (us < 0.95 * best_t) {
      best_t = us;
      best = GemmPlan{kG32Big.bm, kG32Big.bn, kG32Big.bk, kG32Big.wm, kG32Big.wn, kG32Big.st, 1, 32, r1};
    }
  }
  return best;
}

// Weight-streaming plans (M <= 128). Every tile covers all selected rows, so each workgroup
// re-reads the K-slice of X it needs next to its weight slab; one workgroup per CU (about 256
// tiles) streams disjoint slabs. Measured on MI355X at the LLaDA-8B layer shape (M = 128), the
// fastest of the tile widths / K splits tried were:
//   wide output (QKV, N = 12288): 48-row slabs (256 tiles), no split;
//   narrow output (W_o, W_down, N = 4096): 64-row slabs, 4 K splits;  gate/up: 48 + 48 rows.
// Wider slabs with more K splits move fewer bytes per CU but pay the partial round trip.
// Up to kWsMaxRows rows the weight-streaming tiles hold every row (256 rows: 8 waves of 32;
// measured at 160-256 rows of the LLaDA-8B layer: QKV 50 vs 56-60 us, FFN 144-148 vs 156-172 us
// for 128 x 256 tiles of the 32 x 32 x 16 kernel).
// `rows`: the number of selected rows the plan is made for (the grid itself always covers
// m_cap rows, so more rows are still computed, by further row tiles).
GemmPlan plan_gemm(bool bf16, int rows, int N, int K, bool swiglu) {
  GemmPlan p{64, 64, 64, 4, 1, 4, 1};
  if (!bf16) return p;
  if (rows > kWsMaxRows) {
    return plan_g32(rows, N, K, swiglu);
  }
  const int bm = rows <= 64 ? 64 : rows <= 128 ? 128 : 256;
  const int wm = bm / 32;  // waves of 32 rows
  if (swiglu) {
    p = GemmPlan{bm, 96, 64, wm, 1, 0, 1};
  } else if (cdiv(N, 48) >= 224) {
    p = GemmPlan{bm, 48, 64, wm, 1, 0, 1};
  } else {
    p = GemmPlan{bm, 64, 64, wm, 1, 0, 1};
    const long tiles = cdiv(N, 64);
    while (tiles * p.splits < 224 && K % (p.splits * 2 * 64) == 0 && K / (p.splits * 2) >= 512 &&
           p.splits < 8)
      p.splits *= 2;
  }
  p.st = ring_slots(p.bm, p.bn, p.bk, 4);
  return p;
}

size_t gemm_partials_bytes(const GemmPlan& p, int m_cap, int N) {
  return p.splits > 1 ? (size_t)p.splits * m_cap * N * sizeof(float) : 0;
}

static int kchunk_of(const GemmPlan& p, int K) { return cdiv(cdiv(K, p.splits), p.bk) * p.bk; }

size_t qkv_workspace_bytes(bool bf16, const ProjShape& s) {
  const int N = (s.H + 2 * s.Hkv) * s.hd;
  const size_t es = bf16 ? 2 : 4;
  GemmPlan p = plan_gemm(bf16, s.m_plan, N, s.d, false);
  return align256((size_t)s.m_cap * s.d * es) + align256(gemm_partials_bytes(p, s.m_cap, N));
}

size_t ffn_workspace_bytes(bool bf16, const ProjShape& s) {
  const size_t es = bf16 ? 2 : 4;
  const int Nq = s.H * s.hd;
  GemmPlan po = plan_gemm(bf16, s.m_plan, s.d, Nq, false);
  GemmPlan pg = plan_gemm(bf16, s.m_plan, s.F, s.d, true);
  GemmPlan pd = plan_gemm(bf16, s.m_plan, s.d, s.F, false);
  size_t part = gemm_partials_bytes(po, s.m_cap, s.d);
  const size_t part_g = gemm_partials_bytes(pg, s.m_cap, 2 * s.F);
  const size_t part_d = gemm_partials_bytes(pd, s.m_cap, s.d);
  if (part_g > part) part = part_g;
  if (part_d > part) part = part_d;
  return align256((size_t)s.m_cap * s.d * 4) + align256((size_t)s.m_cap * s.d * es) +
         align256((size_t)s.m_cap * s.F * es) + align256(part);
}

template <int BM, int BN, int BK, int WM, int WN, int ST, bool SWIGLU, class Epi>
static bool launch_if(const GemmPlan& p, const GemmArgs& g, dim3 grid, Epi epi, hipStream_t st) {
  if constexpr (ST < 3) {  // shape does not fit a 3-slot ring in LDS; never planned
    return false;
  } else {
    if (p.bm != BM || p.bn != BN || p.bk != BK || p.wm != WM || p.wn != WN || p.st != ST)
      return false;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, ST, SWIGLU, Epi>), grid,
                       dim3(64 * WM * WN), 0, st, g, epi);
    return true;
  }
}

template <int BM, int BN, int BK, int WM, int WN, int ST, bool SWIGLU, class Epi>
static bool launch32_if(const GemmPlan& p, const GemmArgs& g, dim3 grid, Epi epi, hipStream_t st) {
  if (p.mfma != 32 || p.bm != BM || p.bn != BN || p.bk != BK || p.wm != WM || p.wn != WN ||
      p.st != ST)
    return false;
  hipLaunchKernelGGL((gemm32_bf16_kernel<BM, BN, BK, WM, WN, ST, SWIGLU, Epi>), grid,
                     dim3(64 * WM * WN), 0, st, g, epi);
  return true;
}

template <bool SWIGLU, class Epi>
static hipError_t run_gemm_bf16(const GemmPlan& p, const uint16_t* X, const uint16_t* W,
                                const uint16_t* W2, int N, int K, const int32_t* row_ptr, int B,
                                int m_cap, float* partial, Epi epi, hipStream_t st,
                                bool reduce = true, int row0 = 0);

// two-part plan: rows [0, rows_big) on the 256-row tiles, the rest on the 128-row tiles
template <bool SWIGLU, class Epi>
static hipError_t run_gemm_two_part(const GemmPlan& p, const uint16_t* X, const uint16_t* W,
                                    const uint16_t* W2, int N, int K, const int32_t* row_ptr,
                                    int B, int m_cap, Epi epi, hipStream_t st) {
  GemmPlan big = p, mid = p;
  big.rows_big = mid.rows_big = 0;
  mid.bm = kG32Mid.bm; mid.bn = kG32Mid.bn; mid.bk = kG32Mid.bk;
  mid.wm = kG32Mid.wm; mid.wn = kG32Mid.wn; mid.st = kG32Mid.st;
  const int r1 = p.rows_big < m_cap ? p.rows_big : m_cap;
  hipError_t e = run_gemm_bf16<SWIGLU>(big, X, W, W2, N, K, row_ptr, B, r1, nullptr, epi, st);
  if (e != hipSuccess || r1 >= m_cap) return e;
  return run_gemm_bf16<SWIGLU>(mid, X, W, W2, N, K, row_ptr, B, m_cap, nullptr, epi, st, true, r1);
}

// row0: the launch covers rows [row0, m_cap) (its tiles start at row0)
template <bool SWIGLU, class Epi>
static hipError_t run_gemm_bf16(const GemmPlan& p, const uint16_t* X, const uint16_t* W,
                                const uint16_t* W2, int N, int K, const int32_t* row_ptr, int B,
                                int m_cap, float* partial, Epi epi, hipStream_t st,
                                bool reduce, int row0) {
  if (p.rows_big > 0) return run_gemm_two_part<SWIGLU>(p, X, W, W2, N, K, row_ptr, B, m_cap, epi, st);
  GemmArgs g;
  g.X = X; g.W = W; g.W2 = W2; g.N = N; g.K = K;
  g.kchunk = kchunk_of(p, K);
  // measured at the LLaDA shapes: all row tiles together up to 8 of them, else 4
  const int mtiles = cdiv(m_cap - row0, p.bm);
  g.group = mtiles <= 8 ? mtiles : 4;
  g.row_ptr = row_ptr; g.B = B; g.m_cap = m_cap;
  g.partial = (p.splits > 1) ? partial : nullptr;
  g.row0 = row0;
  const int cols = SWIGLU ? p.bn / 2 : p.bn;
  dim3 grid(cdiv(N, cols), mtiles, p.splits);
#define RS(bm, bn) ring_slots(bm, bn, 64, 4)
  bool ok;
  if constexpr (SWIGLU) {
    ok = launch32_if<kG32Big.bm, kG32Big.bn, kG32Big.bk, kG32Big.wm, kG32Big.wn, kG32Big.st, true>(
             p, g, grid, epi, st) ||
         launch32_if<kG32Mid.bm, kG32Mid.bn, kG32Mid.bk, kG32Mid.wm, kG32Mid.wn, kG32Mid.st, true>(
             p, g, grid, epi, st) ||
         launch_if<256, 96, 64, 8, 1, RS(256, 96), true>(p, g, grid, epi, st) ||
         launch_if<128, 96, 64, 4, 1, RS(128, 96), true>(p, g, grid, epi, st) ||
         launch_if<64, 96, 64, 2, 1, RS(64, 96), true>(p, g, grid, epi, st);
  } else {
    ok = launch32_if<kG32Big.bm, kG32Big.bn, kG32Big.bk, kG32Big.wm, kG32Big.wn, kG32Big.st, false>(
             p, g, grid, epi, st) ||
         launch32_if<kG32Mid.bm, kG32Mid.bn, kG32Mid.bk, kG32Mid.wm, kG32Mid.wn, kG32Mid.st, false>(
             p, g, grid, epi, st) ||
         launch_if<256, 48, 64, 8, 1, RS(256, 48), false>(p, g, grid, epi, st) ||
         launch_if<256, 64, 64, 8, 1, RS(256, 64), false>(p, g, grid, epi, st) ||
         launch_if<128, 48, 64, 4, 1, RS(128, 48), false>(p, g, grid, epi, st) ||
         launch_if<128, 64, 64, 4, 1, RS(128, 64), false>(p, g, grid, epi, st) ||
         launch_if<64, 48, 64, 2, 1, RS(64, 48), false>(p, g, grid, epi, st) ||
         launch_if<64, 64, 64, 2, 1, RS(64, 64), false>(p, g, grid, epi, st);
  }
#undef RS
  if (!ok) return hipErrorInvalidConfiguration;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1 || !reduce) return e;
  const size_t groups = (size_t)m_cap * (N / 4);
  if constexpr (SWIGLU)
    hipLaunchKernelGGL((splitk_swiglu_kernel<Epi>), dim3((unsigned)((groups + 255) / 256)),
                       dim3(256), 0, st, partial, p.splits, N, row_ptr, B, m_cap, epi);
  else {
    const dim3 rg((unsigned)((groups + 255) / 256)), rb(256);
    if (p.splits == 2)
      hipLaunchKernelGGL((splitk_reduce_kernel<Epi, 2>), rg, rb, 0, st, partial, 2, N, row_ptr, B, m_cap, epi);
    else if (p.splits == 4)
      hipLaunchKernelGGL((splitk_reduce_kernel<Epi, 4>), rg, rb, 0, st, partial, 4, N, row_ptr, B, m_cap, epi);
    else if (p.splits == 8)
      hipLaunchKernelGGL((splitk_reduce_kernel<Epi, 8>), rg, rb, 0, st, partial, 8, N, row_ptr, B, m_cap, epi);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<Epi>), rg, rb, 0, st, partial, p.splits, N, row_ptr, B, m_cap, epi);
  }
  return hipGetLastError();
}

template <bool SWIGLU, class Epi>
static hipError_t run_gemm_f32(const float* X, const float* W, const float* W2, int N, int K,
                               const int32_t* row_ptr, int B, int m_cap, Epi epi,
                               hipStream_t st) {
  GemmArgsF32 g{X, W, W2, N, K, row_ptr, B, m_cap};
  dim3 grid(cdiv(N, 64), cdiv(m_cap, 64));
  hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, Epi>), grid, dim3(256), 0, st, g, epi);
  return hipGetLastError();
}

template <typename T>
static hipError_t qkv_impl(const ProjShape& s, const T* h_in, const T* g_attn, const T* w_qkv,
                           const int32_t* sel_idx, const int32_t* row_ptr, T* q_sel, T* kc,
                           T* vc, char* ws, hipStream_t st) {
  constexpr bool kBf16 = sizeof(T) == 2;
  const int Nq = s.H * s.hd, Nkv = s.Hkv * s.hd, N = Nq + 2 * Nkv;
  T* xn = reinterpret_cast<T*>(ws);
  float* partial = reinterpret_cast<float*>(ws + align256((size_t)s.m_cap * s.d * sizeof(T)));
  launch_rmsnorm_rows<T, T>(h_in, sel_idx, g_attn, xn, s.d, s.eps, row_ptr, s.B, s.m_cap, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int hd_log2 = 0;
  while ((1 << hd_log2) < s.hd) ++hd_log2;  // hd is 64 or 128
  EpiQKV<T> epi{q_sel, kc, vc, sel_idx, Nq, Nkv, hd_log2, s.S, s.Hkv, FastDiv::make((uint32_t)s.S)};
  if constexpr (kBf16) {
    GemmPlan p = plan_gemm(true, s.m_plan, N, s.d, false);
    return run_gemm_bf16<false>(p, xn, w_qkv, nullptr, N, s.d, row_ptr, s.B, s.m_cap, partial,
                                epi, st);
  } else {
    return run_gemm_f32<false>(xn, w_qkv, nullptr, N, s.d, row_ptr, s.B, s.m_cap, epi, st);
  }
}

// h[j] = h_in[sel[j]] + sum_z partial[z][j] (fixed order); hn[j] = RMSNorm(h[j]) * g.
// Finishes a K-split output projection and normalises its rows in one pass.
template <typename T>
__global__ __launch_bounds__(256) void resid_rmsnorm_kernel(const T* x, const int32_t* sel_idx,
                                                            const float* partial, int splits,
                                                            const T* g, float* h, T* hn, int d,
                                                            float eps, const int32_t* row_ptr,
                                                            int B, int m_cap) {
  const int j = blockIdx.x;
  if (j >= live_rows(row_ptr, B, m_cap)) return;
  const T* xr = x + (size_t)sel_idx[j] * d;
  __shared__ float red[4];
  float ss = 0.f;
  for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
    float v[4];
    Elem<T>::load4(xr + i, v);
    for (int z = 0; z < splits; ++z) {
      float p[4];
      Elem<float>::load4(partial + ((size_t)z * m_cap + j) * d + i, p);
      v[0] += p[0]; v[1] += p[1]; v[2] += p[2]; v[3] += p[3];
    }
    Elem<float>::store4(h + (size_t)j * d + i, v);
    ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], ss))));
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
  // each thread re-reads only the h entries it wrote itself
  for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
    float v[4], gv[4];
    Elem<float>::load4(h + (size_t)j * d + i, v);
    Elem<T>::load4(g + i, gv);
    const float o[4] = {v[0] * r * gv[0], v[1] * r * gv[1], v[2] * r * gv[2], v[3] * r * gv[3]};
    Elem<T>::store4(hn + (size_t)j * d + i, o);
  }
}

// Row-resident variant for d <= 8192: thread t owns 4-element chunks t, t + 256, ... (CH of
// them) of the row, issues every load of the row (x and each split's partial) before using any,
// keeps the sums in registers, and writes h and hn from them (no second pass over memory).
template <typename T, int CH, int SPLITS>
__global__ __launch_bounds__(256) void resid_rmsnorm_reg_kernel(const T* x, const int32_t* sel_idx,
                                                                const float* partial,
                                                                const T* g, float* h, T* hn, int d,
                                                                float eps, const int32_t* row_ptr,
                                                                int B, int m_cap) {
  const int j = blockIdx.x;
  if (j >= live_rows(row_ptr, B, m_cap)) return;
  const T* xr = x + (size_t)sel_idx[j] * d;
  const int nch = d / 4;
  float v[CH][4], p[SPLITS][CH][4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = 4 * (threadIdx.x + 256 * c);
    if (i < d) {
      Elem<T>::load4(xr + i, v[c]);
#pragma unroll
      for (int z = 0; z < SPLITS; ++z)
        Elem<float>::load4(partial + ((size_t)z * m_cap + j) * d + i, p[z][c]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (threadIdx.x + 256 * c < nch) {
#pragma unroll
      for (int z = 0; z < SPLITS; ++z)  // fixed order, as the generic kernel
        for (int e = 0; e < 4; ++e) v[c][e] += p[z][c][e];
      Elem<float>::store4(h + (size_t)j * d + 4 * (threadIdx.x + 256 * c), v[c]);
      ss = fmaf(v[c][0], v[c][0], fmaf(v[c][1], v[c][1], fmaf(v[c][2], v[c][2], fmaf(v[c][3], v[c][3], ss))));
    }
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = 4 * (threadIdx.x + 256 * c);
    if (i < d) {
      float gv[4];
      Elem<T>::load4(g + i, gv);
      const float o[4] = {v[c][0] * r * gv[0], v[c][1] * r * gv[1], v[c][2] * r * gv[2],
                          v[c][3] * r * gv[3]};
      Elem<T>::store4(hn + (size_t)j * d + i, o);
    }
  }
}

template <typename T, int CH>
static bool launch_resid_rmsnorm_reg(int splits, dim3 grid, hipStream_t st, const T* x,
                                     const int32_t* sel, const float* partial, const T* g,
                                     float* h, T* hn, int d, float eps, const int32_t* rp, int B,
                                     int m_cap) {
  switch (splits) {
    case 2: hipLaunchKernelGGL((resid_rmsnorm_reg_kernel<T, CH, 2>), grid, dim3(256), 0, st, x, sel, partial, g, h, hn, d, eps, rp, B, m_cap); return true;
    case 4: hipLaunchKernelGGL((resid_rmsnorm_reg_kernel<T, CH, 4>), grid, dim3(256), 0, st, x, sel, partial, g, h, hn, d, eps, rp, B, m_cap); return true;
    case 8: hipLaunchKernelGGL((resid_rmsnorm_reg_kernel<T, CH, 8>), grid, dim3(256), 0, st, x, sel, partial, g, h, hn, d, eps, rp, B, m_cap); return true;
    default: return false;
  }
}

// h = h_in[sel] + sum of the K-split partials, hn = RMSNorm(h) * g: the row-resident kernel when
// the width and split count allow, else the generic one
template <typename T>
static void launch_resid_rmsnorm(const ProjShape& s, int splits, const T* h_in,
                                 const int32_t* sel_idx, const float* partial, const T* g,
                                 float* h, T* hn, const int32_t* row_ptr, hipStream_t st) {
  const dim3 grid(s.m_cap);
  const int ch = (s.d + 1023) / 1024;
  bool done = false;
  if (s.d % 4 == 0) {
    if (ch <= 1) done = launch_resid_rmsnorm_reg<T, 1>(splits, grid, st, h_in, sel_idx, partial, g, h, hn, s.d, s.eps, row_ptr, s.B, s.m_cap);
    else if (ch <= 2) done = launch_resid_rmsnorm_reg<T, 2>(splits, grid, st, h_in, sel_idx, partial, g, h, hn, s.d, s.eps, row_ptr, s.B, s.m_cap);
    else if (ch <= 4) done = launch_resid_rmsnorm_reg<T, 4>(splits, grid, st, h_in, sel_idx, partial, g, h, hn, s.d, s.eps, row_ptr, s.B, s.m_cap);
  }
  if (!done)
    hipLaunchKernelGGL((resid_rmsnorm_kernel<T>), grid, dim3(256), 0, st, h_in, sel_idx, partial,
                       splits, g, h, hn, s.d, s.eps, row_ptr, s.B, s.m_cap);
}

template <typename T>
static hipError_t ffn_impl(const ProjShape& s, const T* h_in, const T* o_sel, const T* w_o,
                           const T* g_ffn, const T* w_gate, const T* w_up, const T* w_down,
                           const int32_t* sel_idx, const int32_t* row_ptr, T* h_out, char* ws,
                           hipStream_t st) {
  constexpr bool kBf16 = sizeof(T) == 2;
  const int Nq = s.H * s.hd;
  char* p = ws;
  float* hbuf = reinterpret_cast<float*>(p);
  p += align256((size_t)s.m_cap * s.d * 4);
  T* hn = reinterpret_cast<T*>(p);
  p += align256((size_t)s.m_cap * s.d * sizeof(T));
  T* z = reinterpret_cast<T*>(p);
  p += align256((size_t)s.m_cap * s.F * sizeof(T));
  float* partial = reinterpret_cast<float*>(p);
  hipError_t e;

  // h = h_in[sel] + o_sel W_o^T ; hn = RMSNorm(h) * g_ffn
  EpiResidF32<T> e1{hbuf, h_in, sel_idx, s.d};
  if constexpr (kBf16) {
    const GemmPlan po = plan_gemm(true, s.m_plan, s.d, Nq, false);
    e = run_gemm_bf16<false>(po, o_sel, w_o, nullptr, s.d, Nq, row_ptr, s.B, s.m_cap, partial,
                             e1, st, /*reduce=*/false);
    if (e != hipSuccess) return e;
    if (po.splits > 1)
      launch_resid_rmsnorm<T>(s, po.splits, h_in, sel_idx, partial, g_ffn, hbuf, hn, row_ptr, st);
    else
      launch_rmsnorm_rows<float, T>(hbuf, nullptr, g_ffn, hn, s.d, s.eps, row_ptr, s.B, s.m_cap,
                                    st);
  } else {
    e = run_gemm_f32<false>(o_sel, w_o, nullptr, s.d, Nq, row_ptr, s.B, s.m_cap, e1, st);
    if (e != hipSuccess) return e;
    launch_rmsnorm_rows<float, T>(hbuf, nullptr, g_ffn, hn, s.d, s.eps, row_ptr, s.B, s.m_cap, st);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // z = silu(hn W_gate^T) * (hn W_up^T)
  EpiSwiGLU<T> e2{z, s.F};
  if constexpr (kBf16)
    e = run_gemm_bf16<true>(plan_gemm(true, s.m_plan, s.F, s.d, true), hn, w_gate, w_up, s.F, s.d,
                            row_ptr, s.B, s.m_cap, partial, e2, st);
  else
    e = run_gemm_f32<true>(hn, w_gate, w_up, s.F, s.d, row_ptr, s.B, s.m_cap, e2, st);
  if (e != hipSuccess) return e;

  // h_out[sel] = h + z W_down^T
  EpiResidScatter<T> e3{h_out, hbuf, sel_idx, s.d};
  if constexpr (kBf16)
    e = run_gemm_bf16<false>(plan_gemm(true, s.m_plan, s.d, s.F, false), z, w_down, nullptr, s.d,
                             s.F, row_ptr, s.B, s.m_cap, partial, e3, st);
  else
    e = run_gemm_f32<false>(z, w_down, nullptr, s.d, s.F, row_ptr, s.B, s.m_cap, e3, st);
  return e;
}

hipError_t launch_qkv(bool bf16, const ProjShape& s, const void* h_in, const void* g_attn,
                      const void* w_qkv, const int32_t* sel_idx, const int32_t* row_ptr,
                      void* q_sel, void* k_cache, void* v_cache, void* ws, hipStream_t st) {
  if (s.m_cap == 0) return hipSuccess;
  if (bf16)
    return qkv_impl<uint16_t>(s, (const uint16_t*)h_in, (const uint16_t*)g_attn,
                              (const uint16_t*)w_qkv, sel_idx, row_ptr, (uint16_t*)q_sel,
                              (uint16_t*)k_cache, (uint16_t*)v_cache, (char*)ws, st);
  return qkv_impl<float>(s, (const float*)h_in, (const float*)g_attn, (const float*)w_qkv,
                         sel_idx, row_ptr, (float*)q_sel, (float*)k_cache, (float*)v_cache,
                         (char*)ws, st);
}

hipError_t launch_ffn(bool bf16, const ProjShape& s, const void* h_in, const void* o_sel,
                      const void* w_o, const void* g_ffn, const void* w_gate, const void* w_up,
                      const void* w_down, const int32_t* sel_idx, const int32_t* row_ptr,
                      void* h_out, void* ws, hipStream_t st) {
  if (s.m_cap == 0) return hipSuccess;
  if (bf16)
    return ffn_impl<uint16_t>(s, (const uint16_t*)h_in, (const uint16_t*)o_sel,
                              (const uint16_t*)w_o, (const uint16_t*)g_ffn,
                              (const uint16_t*)w_gate, (const uint16_t*)w_up,
                              (const uint16_t*)w_down, sel_idx, row_ptr, (uint16_t*)h_out,
                              (char*)ws, st);
  return ffn_impl<float>(s, (const float*)h_in, (const float*)o_sel, (const float*)w_o,
                         (const float*)g_ffn, (const float*)w_gate, (const float*)w_up,
                         (const float*)w_down, sel_idx, row_ptr, (float*)h_out, (char*)ws, st);
}

}  // namespace dllm
