// (4) Partial attention, gfx950.
//
// DyLLM (French summary page) §2.B: for salient tokens the row of the attention-score matrix
// is recomputed exactly; §1: attention is bidirectional, so a selected query attends to every
// cached position (no mask), including masked tokens and itself, with the K/V entries that the
// projection call of this step has just overwritten.
//
// Work decomposition: one workgroup = 128 query rows (4 waves x two 16-row blocks) of one
// (sequence b, kv head hk) against a key range. A "query row" is a (selected token, query head of
// hk's group) pair, so grouped heads share every K/V tile that is loaded (GQA packing), and each
// K/V fragment read from LDS feeds the MFMAs of both query blocks of a wave. Per 64-key tile:
//   * K rows -> LDS; V rows -> LDS transposed ([hd][key]); the next tile's K/V loads are issued
//     into registers before this tile is multiplied, so their latency hides behind the MFMAs;
//   * S^T = K Q^T on the bf16 matrix cores (16x16x32): the lane's accumulator column is ONE
//     query, so the online-softmax max/sum over keys is a 2-step cross-lane shuffle;
//   * within each 32-key group the keys feeding the two 16-row S^T blocks are interleaved
//     (block 0: keys 8g+0..3, block 1: keys 8g+4..7 for lane group g) so that the exponentiated
//     scores already sit in registers in the B-operand layout of the next product;
//   * O^T += V^T P^T on the matrix cores, fp32 accumulation, rescaled by the running max.
// When the selected rows alone cannot fill the 256 compute units (batch 1, M = 128), the key
// range is split and the fp32 partials (o, max, sum) are merged in a fixed order by a second
// pass, so results stay deterministic.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kQB = 2;             // 16-row query blocks per wave
constexpr int kTQ = 64 * kQB;      // query rows per workgroup (4 waves x 2 blocks x 16)
constexpr int kTK = 64;            // keys per tile
constexpr int kVtPitch = kTK + 8;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* row_ptr;
  uint16_t* o;
  float* part_o;   // [nsplit, m_cap, H, hd]   (nsplit > 1)
  float* part_ml;  // [nsplit, m_cap, H, 2]
  int B, S, H, Hkv, m_cap, nsplit, kps;
  float scale_log2;  // scale * log2(e): scores are kept in base-2 units
};

// grid.x enumerates (sequence, kv head, key split) and grid.y the query tiles, so the tiles that
// share one K/V panel have ids grid.x apart: with grid.x a multiple of 8 they run on the same XCD
// and read the panel through one L2.
template <int HD>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KB = HD / 32;         // 32-wide k-steps of q.k over hd
  constexpr int HB = HD / 16;         // 16-wide output blocks of hd
  constexpr int KCH = HD / 8;         // 16-byte chunks per K/V row
  constexpr int KPT = HD / 32;        // keys per thread in the transposing V load
  constexpr int KPitch = HD + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kTK * KPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[HD * kVtPitch];

  const int G = a.H / a.Hkv;
  const int Nq = a.H * HD;
  const int per_b = a.Hkv * a.nsplit;
  const int b = blockIdx.x / per_b;
  const int hk = (blockIdx.x - b * per_b) / a.nsplit;
  const int split = blockIdx.x - b * per_b - hk * a.nsplit;
  const int M = min(a.row_ptr[a.B], a.m_cap);
  const int r0 = min(a.row_ptr[b], M), r1 = min(a.row_ptr[b + 1], M);
  const int nrows = (r1 - r0) * G;
  const int tile0 = blockIdx.y * kTQ;
  if (tile0 >= nrows) return;
  const int t0 = split * a.kps;
  const int t1 = min(a.S, t0 + a.kps);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  // ---- this lane's query rows: column lr of each of the wave's S^T blocks
  bool qvalid[kQB];
  int qj[kQB], qh[kQB];
  bf16x8 qf[kQB][KB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qr = tile0 + wave * (16 * kQB) + qb * 16 + lr;
    qvalid[qb] = qr < nrows;
    qj[qb] = qvalid[qb] ? r0 + qr / G : 0;
    qh[qb] = qvalid[qb] ? hk * G + qr % G : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qf[qb][kb] = qvalid[qb] ? *reinterpret_cast<const bf16x8*>(a.q + (size_t)qj[qb] * Nq +
                                                                 qh[qb] * HD + kb * 32 + lg * 8)
                              : bf16x8{};
  }

  f32x4 oacc[kQB][HB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int i = 0; i < HB; ++i) oacc[qb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[kQB], l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; }

  const size_t head_off = ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
  const uint16_t* kbase = a.kc + head_off;
  const uint16_t* vbase = a.vc + head_off;

  // K load: chunks tid + 256 i -> (row, 8-col); V load: KPT consecutive keys x 8 hd columns
  const int vkg = tid / KCH, vcol = (tid % KCH) * 8;
  uint4 kreg[KPT], vreg[KPT];
  auto load_tile = [&](int tk) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i;
      const int key = tk + c / KCH;
      kreg[i] = (key < t1) ? *reinterpret_cast<const uint4*>(kbase + (size_t)key * HD +
                                                              (c % KCH) * 8)
                           : make_uint4(0, 0, 0, 0);
      const int vkey = tk + vkg * KPT + i;
      vreg[i] = (vkey < t1) ? *reinterpret_cast<const uint4*>(vbase + (size_t)vkey * HD + vcol)
                            : make_uint4(0, 0, 0, 0);
    }
  };

  load_tile(t0);
  for (int tk = t0; tk < t1; tk += kTK) {
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(sK + (c / KCH) * KPitch + (c % KCH) * 8) = kreg[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t vals[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t w = (e < 2) ? vreg[i].x : (e < 4) ? vreg[i].y : (e < 6) ? vreg[i].z
                                                                             : vreg[i].w;
        vals[i] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
      }
      uint16_t* dst = sVt + (vcol + e) * kVtPitch + vkg * KPT;
      if constexpr (KPT == 4) {
        uint2 pk;
        pk.x = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
        pk.y = (uint32_t)vals[2] | ((uint32_t)vals[3] << 16);
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
      }
    }
    __syncthreads();
    // the next tile's loads fly while this one is multiplied
    if (tk + kTK < t1) load_tile(tk + kTK);

    // ---- S^T blocks: blk = 2 ks + half, row m <-> key 32 ks + 8 (m/4) + 4 half + m%4
    f32x4 sacc[kQB][4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int ks = blk >> 1, half = blk & 1;
      const int kr = 32 * ks + 8 * (lr >> 2) + 4 * half + (lr & 3);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) sacc[qb][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + kr * KPitch + kb * 32 + lg * 8);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sacc[qb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][kb], sacc[qb][blk],
                                                                   0, 0, 0);
      }
    }
    // sacc[qb][blk][i] = score of query (qb, lr) with key tk + 32 ks + 8 lg + 4 half + i
    bf16x8 pf[kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float sv[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = tk + 32 * (blk >> 1) + 8 * lg + 4 * (blk & 1) + i;
          sv[blk][i] = (key < t1) ? sacc[qb][blk][i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[blk][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qb], mx);
      const float alpha = fast_exp2(m_run[qb] - m_new);  // 0 on the first tile
      float psum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(sv[blk][i] - m_new);
          psum += p;
          pf[qb][blk >> 1][4 * (blk & 1) + i] = (__bf16)p;
        }
      l_run[qb] = l_run[qb] * alpha + psum;
      m_run[qb] = m_new;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        oacc[qb][hb][0] *= alpha; oacc[qb][hb][1] *= alpha;
        oacc[qb][hb][2] *= alpha; oacc[qb][hb][3] *= alpha;
      }
    }
    // ---- O^T += V^T P^T; the k-slot s of lane group lg is key 32 ks + 8 lg + s
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sVt + (hb * 16 + lr) * kVtPitch +
                                                           32 * ks + 8 * lg);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          oacc[qb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][ks], oacc[qb][hb],
                                                                  0, 0, 0);
      }
  }

  // oacc[qb][hb][i] = unnormalised o[query (qb, lr)][hd = 16 hb + 4 lg + i]; this lane's sum
  // covers a quarter of the keys
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!qvalid[qb]) continue;
    const int j = qj[qb], h = qh[qb];
    if (a.nsplit == 1) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float v[4] = {oacc[qb][hb][0] * inv, oacc[qb][hb][1] * inv, oacc[qb][hb][2] * inv,
                            oacc[qb][hb][3] * inv};
        Elem<uint16_t>::store4(a.o + (size_t)j * Nq + h * HD + hb * 16 + 4 * lg, v);
      }
    } else {
      const size_t base = ((size_t)split * a.m_cap + j) * a.H + h;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float v[4] = {oacc[qb][hb][0], oacc[qb][hb][1], oacc[qb][hb][2], oacc[qb][hb][3]};
        Elem<float>::store4(a.part_o + base * HD + hb * 16 + 4 * lg, v);
      }
      if (lg == 0) {
        a.part_ml[base * 2] = m_run[qb];
        a.part_ml[base * 2 + 1] = l_tot;
      }
    }
  }
}

// fixed-order log-sum-exp merge of the key-split partials; one thread per 4 output columns
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int M = min(a.row_ptr[a.B], a.m_cap);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  constexpr int QG = HD / 4;
  const size_t jh = idx / QG;
  const int j = (int)(jh / a.H);
  if (j >= M) return;
  const int h = (int)(jh - (size_t)j * a.H);
  const int c = (int)(idx - jh * QG) * 4;
  float mmax = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s)
    mmax = fmaxf(mmax, a.part_ml[(((size_t)s * a.m_cap + j) * a.H + h) * 2]);
  float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.nsplit; ++s) {
    const size_t base = ((size_t)s * a.m_cap + j) * a.H + h;
    const float w = fast_exp2(a.part_ml[base * 2] - mmax);
    L += w * a.part_ml[base * 2 + 1];
    float p[4];
    Elem<float>::load4(a.part_o + base * HD + c, p);
    o[0] += w * p[0]; o[1] += w * p[1]; o[2] += w * p[2]; o[3] += w * p[3];
  }
  const float inv = 1.0f / L;
  const float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  Elem<uint16_t>::store4(a.o + (size_t)j * a.H * HD + h * HD + c, v);
}

// ---------------------------------------------------------------- float32 path (VALU)
// one wave per (selected token, query head); lanes over hd; online softmax over every key
struct AttnArgsF32 {
  const float* q;
  const float* kc;
  const float* vc;
  const int32_t* sel_idx;
  const int32_t* row_ptr;
  float* o;
  int B, S, H, Hkv, hd, m_cap;
  float scale;
};

template <int HD>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgsF32 a) {
  constexpr int E = HD / 64;
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int M = min(a.row_ptr[a.B], a.m_cap);
  const int j = wid / a.H, h = wid - (wid / a.H) * a.H;
  if (j >= M) return;
  const int b = a.sel_idx[j] / a.S;
  const int hk = h / (a.H / a.Hkv);
  const float* q = a.q + (size_t)j * a.H * HD + h * HD;
  const float* kb = a.kc + ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
  const float* vb = a.vc + ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
  float qv[E], ov[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { qv[e] = q[lane + 64 * e]; ov[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < a.S; ++t) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) d = fmaf(qv[e], kb[(size_t)t * HD + lane + 64 * e], d);
    const float s = wave_sum(d) * a.scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
#pragma unroll
    for (int e = 0; e < E; ++e) ov[e] = fmaf(p, vb[(size_t)t * HD + lane + 64 * e], ov[e] * al);
    m = mn;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) a.o[(size_t)j * a.H * HD + h * HD + lane + 64 * e] = ov[e] / l;
}

// ---------------------------------------------------------------- host side
static inline int cdiv(long x, long y) { return (int)((x + y - 1) / y); }

static void split_keys(bool bf16, const ProjShape& s, int& nsplit, int& kps) {
  nsplit = 1;
  if (bf16) {
    const int G = s.H / s.Hkv;
    const long est = (long)(cdiv((long)s.m_cap * G, kTQ) > 0 ? cdiv((long)s.m_cap * G, kTQ) : 1) *
                     s.Hkv;
    while (est * nsplit < 512 && s.S / (nsplit * 2) >= 128) nsplit *= 2;
  }
  kps = cdiv(cdiv(s.S, nsplit), kTK) * kTK;
  nsplit = cdiv(s.S, kps);  // every split owns at least one key
}

AttnPlan plan_attn(bool bf16, const ProjShape& s) {
  int n, k;
  split_keys(bf16, s, n, k);
  return AttnPlan{n};
}

size_t attn_workspace_bytes(bool bf16, const ProjShape& s) {
  int nsplit, kps;
  split_keys(bf16, s, nsplit, kps);
  if (nsplit <= 1) return 0;
  const size_t rows = (size_t)nsplit * s.m_cap * s.H;
  return ((rows * s.hd * 4 + 255) & ~(size_t)255) + rows * 2 * 4;
}

hipError_t launch_attn(bool bf16, const ProjShape& s, float scale, const void* q_sel,
                       const void* k_cache, const void* v_cache, const int32_t* sel_idx,
                       const int32_t* row_ptr, void* o_sel, void* ws, hipStream_t st) {
  if (s.m_cap == 0) return hipSuccess;
  if (!bf16) {
    AttnArgsF32 f{(const float*)q_sel, (const float*)k_cache, (const float*)v_cache, sel_idx,
                  row_ptr, (float*)o_sel, s.B, s.S, s.H, s.Hkv, s.hd, s.m_cap, scale};
    dim3 grid(cdiv((long)s.m_cap * s.H, 4));
    if (s.hd == 64)
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, st, f);
    else
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, st, f);
    return hipGetLastError();
  }
  AttnArgs a;
  a.q = (const uint16_t*)q_sel; a.kc = (const uint16_t*)k_cache; a.vc = (const uint16_t*)v_cache;
  a.row_ptr = row_ptr; a.o = (uint16_t*)o_sel;
  a.B = s.B; a.S = s.S; a.H = s.H; a.Hkv = s.Hkv; a.m_cap = s.m_cap;
  split_keys(true, s, a.nsplit, a.kps);
  a.scale_log2 = scale * kLog2e;
  a.part_o = nullptr; a.part_ml = nullptr;
  if (a.nsplit > 1) {
    const size_t rows = (size_t)a.nsplit * s.m_cap * s.H;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + ((rows * s.hd * 4 + 255) & ~(size_t)255));
  }
  const int G = s.H / s.Hkv;
  const int rows_max = (s.m_cap < s.S ? s.m_cap : s.S) * G;
  dim3 grid(s.B * s.Hkv * a.nsplit, cdiv(rows_max, kTQ));
  if (s.hd == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const size_t threads = (size_t)s.m_cap * s.H * (s.hd / 4);
  dim3 mg((unsigned)((threads + 255) / 256));
  if (s.hd == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, mg, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_merge_kernel<128>, mg, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dllm
