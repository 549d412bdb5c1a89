// (3) + (5) Gathered projections of the selected tokens, gfx950.
//
// ES-dLLM (German summary page) §2.B: only the selected positions are computed; their keys,
// values and hidden states overwrite the cached entries in place, every other entry is reused.
// DyLLM (French summary page) §2.A: the FFN runs only for salient tokens.
//
// Every projection is a dense contraction C[M, N] = X[M, K] W[N, K]^T of the M selected rows
// (compacted to consecutive rows by a gather/RMSNorm pass) with a weight stored [out, in].
// Both operands are K-contiguous, which is the operand layout of the bf16 matrix-core
// instruction v_mfma_f32_16x16x32_bf16: a lane supplies 8 consecutive K values of one row.
// The kernel multiplies W (instruction A operand, rows = output columns n) by X (B operand,
// rows = tokens m), so each lane's 4 accumulators are 4 CONSECUTIVE output columns of one
// token row: every epilogue stores 8 or 16 contiguous bytes per lane straight into its target
// (q rows, K/V cache rows of the token's position, residual rows, scattered hidden rows).
//
// Tiles: BM (64|128) tokens x 128 weight rows x 64 K per step, 256 threads = 2 x 2 waves.
// Global -> register prefetch of the next K step overlaps the MFMAs of the current one; LDS rows
// are padded to 144 bytes so the 16 lanes reading one 16-row fragment hit distinct banks.
// At small M the GEMMs stream weights (HBM-bound); a few K splits fill the 256 CUs and are
// reduced in a fixed order by a second pass (deterministic).
#include "common.h"
#include "kernels.h"

namespace dllm {

// =========================================================================================
// epilogues: apply to 4 consecutive columns n..n+3 of compact row j (n % 4 == 0)
// =========================================================================================
template <typename T>
struct EpiQKV {  // Q -> q_sel[j]; K/V -> cache[b, hk, s, e] of the token's own position
  T* q_sel;
  T* kc;
  T* vc;
  const int32_t* sel_idx;
  int Nq, Nkv, hd, S, Hkv;
  __device__ __forceinline__ void operator()(int j, int n, const float v[4]) const {
    if (n < Nq) {
      Elem<T>::store4(q_sel + (size_t)j * Nq + n, v);
      return;
    }
    const int id = sel_idx[j];
    const int b = id / S, s = id - (id / S) * S;
    int kv = n - Nq;
    T* cache = kc;
    if (kv >= Nkv) {
      kv -= Nkv;
      cache = vc;
    }
    const int hk = kv / hd, e = kv - hk * hd;
    Elem<T>::store4(cache + (((size_t)b * Hkv + hk) * S + s) * hd + e, v);
  }
};

template <typename T>
struct EpiResidF32 {  // h[j] = h_in[sel[j]] + acc  (float32 workspace)
  float* h;
  const T* x;
  const int32_t* sel_idx;
  int d;
  __device__ __forceinline__ void operator()(int j, int n, const float v[4]) const {
    float r[4];
    Elem<T>::load4(x + (size_t)sel_idx[j] * d + n, r);
    const float o[4] = {v[0] + r[0], v[1] + r[1], v[2] + r[2], v[3] + r[3]};
    Elem<float>::store4(h + (size_t)j * d + n, o);
  }
};

template <typename T>
struct EpiResidScatter {  // h_out[sel[j]] = h[j] + acc
  T* h_out;
  const float* h;
  const int32_t* sel_idx;
  int d;
  __device__ __forceinline__ void operator()(int j, int n, const float v[4]) const {
    float r[4];
    Elem<float>::load4(h + (size_t)j * d + n, r);
    const float o[4] = {v[0] + r[0], v[1] + r[1], v[2] + r[2], v[3] + r[3]};
    Elem<T>::store4(h_out + (size_t)sel_idx[j] * d + n, o);
  }
};

template <typename T>
struct EpiSwiGLU {  // z[j, n] = silu(gate) * up
  T* z;
  int F;
  __device__ __forceinline__ void operator()(int j, int n, const float g[4],
                                             const float u[4]) const {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = g[i] / (1.0f + __expf(-g[i])) * u[i];
    Elem<T>::store4(z + (size_t)j * F + n, o);
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

// =========================================================================================
// bf16 matrix-core GEMM
// =========================================================================================
constexpr int kBN = 128;      // weight rows per tile (SwiGLU: 64 gate + 64 up rows)
constexpr int kBK = 64;       // K per step
constexpr int kPitch = 72;    // LDS row pitch in bf16 (64 + 8 pad = 144 bytes)

struct GemmArgs {
  const uint16_t* X;   // [m_cap, K] compact activations
  const uint16_t* W;   // [N, K]  (SwiGLU: gate)
  const uint16_t* W2;  // SwiGLU: up [N, K]; else unused
  int N, K, kchunk;
  const int32_t* row_ptr;
  int B, m_cap;
  float* partial;      // [splits, m_cap, N] when split, else NULL
};

template <int BM>
struct TileRegs {
  uint4 a[BM / 32];
  uint4 w[4];
};

template <int BM, bool SWIGLU>
__device__ __forceinline__ void load_tile(const GemmArgs& g, int m0, int n0, int M, int k0,
                                          TileRegs<BM>& r) {
  const int t = threadIdx.x;
  const int col = (t & 7) * 8;
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int row = (t >> 3) + 32 * i;
    const int m = m0 + row;
    r.a[i] = (m < M) ? *reinterpret_cast<const uint4*>(g.X + (size_t)m * g.K + k0 + col)
                     : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (t >> 3) + 32 * i;
    const uint16_t* src;
    int n;
    if (SWIGLU) {
      n = n0 + (row & 63);
      src = (row < 64) ? g.W : g.W2;
    } else {
      n = n0 + row;
      src = g.W;
    }
    r.w[i] = (n < g.N) ? *reinterpret_cast<const uint4*>(src + (size_t)n * g.K + k0 + col)
                       : make_uint4(0, 0, 0, 0);
  }
}

template <int BM>
__device__ __forceinline__ void store_tile(uint16_t* sA, uint16_t* sW, const TileRegs<BM>& r) {
  const int t = threadIdx.x;
  const int col = (t & 7) * 8;
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
    *reinterpret_cast<uint4*>(sA + ((t >> 3) + 32 * i) * kPitch + col) = r.a[i];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(sW + ((t >> 3) + 32 * i) * kPitch + col) = r.w[i];
}

// LDS row of the wave's n-block nb (0..3). SwiGLU pairs gate block nb with up block nb + 2.
template <bool SWIGLU>
__device__ __forceinline__ int wrow_base(int wn, int nb) {
  if (SWIGLU) return (nb < 2) ? (32 * wn + 16 * nb) : (64 + 32 * wn + 16 * (nb - 2));
  return 64 * wn + 16 * nb;
}

template <int BM, bool SWIGLU, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g, Epi epi) {
  constexpr int MB = BM / 32;  // 16-row m-blocks per wave (2 waves along m)
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sW[kBN * kPitch];

  const int M = live_rows(g.row_ptr, g.B, g.m_cap);
  const int m0 = blockIdx.y * BM;
  if (m0 >= M) return;
  const int n0 = blockIdx.x * (SWIGLU ? kBN / 2 : kBN);
  const int kb = blockIdx.z * g.kchunk;
  const int ke = min(g.K, kb + g.kchunk);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  f32x4 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  TileRegs<BM> regs;
  if (kb < ke) {  // a K split never starts past K (see plan_gemm), kept as a bound check
    load_tile<BM, SWIGLU>(g, m0, n0, M, kb, regs);
    store_tile<BM>(sA, sW, regs);
  }
  __syncthreads();

  for (int k0 = kb; k0 < ke; k0 += kBK) {
    const bool more = k0 + kBK < ke;
    if (more) load_tile<BM, SWIGLU>(g, m0, n0, M, k0 + kBK, regs);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 bx[MB], aw[4];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        bx[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * (BM / 2) + 16 * i + lr) * kPitch +
                                                 kk + lk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        aw[j] = *reinterpret_cast<const bf16x8*>(sW + (wrow_base<SWIGLU>(wn, j) + lr) * kPitch +
                                                 kk + lk);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[j], bx[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      __syncthreads();
      store_tile<BM>(sA, sW, regs);
      __syncthreads();
    }
  }

  // acc[i][j][r] = C[m = wm*BM/2 + 16 i + lr][n = (n-block j row base) + 4*(lane/16) + r]
  const int nq = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * (BM / 2) + 16 * i + lr;
    if (m >= M) continue;
    if constexpr (SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + 32 * wn + 16 * j + nq;
        const float gv[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        const float uv[4] = {acc[i][j + 2][0], acc[i][j + 2][1], acc[i][j + 2][2],
                             acc[i][j + 2][3]};
        epi(m, n, gv, uv);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 64 * wn + 16 * j + nq;
        if (n >= g.N) continue;
        const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        if (g.partial) {
          Elem<float>::store4(g.partial + ((size_t)blockIdx.z * g.m_cap + m) * g.N + n, v);
        } else {
          epi(m, n, v);
        }
      }
    }
  }
}

// fixed-order sum of the K-split partials, then the epilogue
template <class Epi>
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
  for (int z = 0; z < splits; ++z) {
    float p[4];
    Elem<float>::load4(partial + ((size_t)z * m_cap + m) * N + n, p);
    v[0] += p[0]; v[1] += p[1]; v[2] += p[2]; v[3] += p[3];
  }
  epi(m, n, v);
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
      epi(m, n, acc[i], accu[i]);
    else
      epi(m, n, acc[i]);
  }
}

// =========================================================================================
// host side: plans, workspace and launches
// =========================================================================================
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

GemmPlan plan_gemm(bool bf16, int m_cap, int N, int K, bool splittable) {
  GemmPlan p{64, 1};
  if (!bf16) return p;
  p.bm = m_cap <= 64 ? 64 : 128;
  const long tiles = (long)cdiv(N, kBN) * cdiv(m_cap, p.bm);
  if (splittable) {
    // fill the 256 compute units (about two tiles each) while every split keeps >= 8 K steps
    while (tiles * p.splits < 512 && K / (p.splits * 2) >= 8 * kBK && p.splits < 8) p.splits *= 2;
  }
  return p;
}

size_t gemm_partials_bytes(const GemmPlan& p, int m_cap, int N) {
  return p.splits > 1 ? (size_t)p.splits * m_cap * N * sizeof(float) : 0;
}

static int kchunk_of(const GemmPlan& p, int K) {
  return cdiv(cdiv(K, p.splits), kBK) * kBK;
}

size_t qkv_workspace_bytes(bool bf16, const ProjShape& s) {
  const int N = (s.H + 2 * s.Hkv) * s.hd;
  const size_t es = bf16 ? 2 : 4;
  GemmPlan p = plan_gemm(bf16, s.m_cap, N, s.d, true);
  return align256((size_t)s.m_cap * s.d * es) + align256(gemm_partials_bytes(p, s.m_cap, N));
}

size_t ffn_workspace_bytes(bool bf16, const ProjShape& s) {
  const size_t es = bf16 ? 2 : 4;
  const int Nq = s.H * s.hd;
  GemmPlan po = plan_gemm(bf16, s.m_cap, s.d, Nq, true);
  GemmPlan pd = plan_gemm(bf16, s.m_cap, s.d, s.F, true);
  size_t part = gemm_partials_bytes(po, s.m_cap, s.d);
  size_t part2 = gemm_partials_bytes(pd, s.m_cap, s.d);
  if (part2 > part) part = part2;
  return align256((size_t)s.m_cap * s.d * 4) + align256((size_t)s.m_cap * s.d * es) +
         align256((size_t)s.m_cap * s.F * es) + align256(part);
}

template <bool SWIGLU, class Epi>
static hipError_t run_gemm_bf16(const GemmPlan& p, const uint16_t* X, const uint16_t* W,
                                const uint16_t* W2, int N, int K, const int32_t* row_ptr, int B,
                                int m_cap, float* partial, Epi epi, hipStream_t st) {
  GemmArgs g;
  g.X = X; g.W = W; g.W2 = W2; g.N = N; g.K = K;
  g.kchunk = kchunk_of(p, K);
  g.row_ptr = row_ptr; g.B = B; g.m_cap = m_cap;
  g.partial = (p.splits > 1) ? partial : nullptr;
  const int ntile = SWIGLU ? cdiv(N, kBN / 2) : cdiv(N, kBN);
  dim3 grid(ntile, cdiv(m_cap, p.bm), p.splits);
  if (p.bm == 64)
    hipLaunchKernelGGL((gemm_bf16_kernel<64, SWIGLU, Epi>), grid, dim3(256), 0, st, g, epi);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<128, SWIGLU, Epi>), grid, dim3(256), 0, st, g, epi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  if constexpr (!SWIGLU) {
    const size_t groups = (size_t)m_cap * (N / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<Epi>), dim3((unsigned)((groups + 255) / 256)),
                       dim3(256), 0, st, partial, p.splits, N, row_ptr, B, m_cap, epi);
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
  hipLaunchKernelGGL((rmsnorm_rows_kernel<T, T>), dim3(s.m_cap), dim3(256), 0, st, h_in, sel_idx,
                     g_attn, xn, s.d, s.eps, row_ptr, s.B, s.m_cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  EpiQKV<T> epi{q_sel, kc, vc, sel_idx, Nq, Nkv, s.hd, s.S, s.Hkv};
  if constexpr (kBf16) {
    GemmPlan p = plan_gemm(true, s.m_cap, N, s.d, true);
    return run_gemm_bf16<false>(p, xn, w_qkv, nullptr, N, s.d, row_ptr, s.B, s.m_cap, partial,
                                epi, st);
  } else {
    return run_gemm_f32<false>(xn, w_qkv, nullptr, N, s.d, row_ptr, s.B, s.m_cap, epi, st);
  }
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

  // h = h_in[sel] + o_sel W_o^T
  EpiResidF32<T> e1{hbuf, h_in, sel_idx, s.d};
  if constexpr (kBf16)
    e = run_gemm_bf16<false>(plan_gemm(true, s.m_cap, s.d, Nq, true), o_sel, w_o, nullptr, s.d,
                             Nq, row_ptr, s.B, s.m_cap, partial, e1, st);
  else
    e = run_gemm_f32<false>(o_sel, w_o, nullptr, s.d, Nq, row_ptr, s.B, s.m_cap, e1, st);
  if (e != hipSuccess) return e;

  // hn = RMSNorm(h) * g_ffn
  hipLaunchKernelGGL((rmsnorm_rows_kernel<float, T>), dim3(s.m_cap), dim3(256), 0, st, hbuf,
                     nullptr, g_ffn, hn, s.d, s.eps, row_ptr, s.B, s.m_cap);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // z = silu(hn W_gate^T) * (hn W_up^T)
  EpiSwiGLU<T> e2{z, s.F};
  if constexpr (kBf16)
    e = run_gemm_bf16<true>(plan_gemm(true, s.m_cap, 2 * s.F, s.d, false), hn, w_gate, w_up, s.F,
                            s.d, row_ptr, s.B, s.m_cap, nullptr, e2, st);
  else
    e = run_gemm_f32<true>(hn, w_gate, w_up, s.F, s.d, row_ptr, s.B, s.m_cap, e2, st);
  if (e != hipSuccess) return e;

  // h_out[sel] = h + z W_down^T
  EpiResidScatter<T> e3{h_out, hbuf, sel_idx, s.d};
  if constexpr (kBf16)
    e = run_gemm_bf16<false>(plan_gemm(true, s.m_cap, s.d, s.F, true), z, w_down, nullptr, s.d,
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
