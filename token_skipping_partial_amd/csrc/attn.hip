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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kQB = 2;             // 16-row query blocks per wave
constexpr int kTQ = 64 * kQB;      // query rows per workgroup (4 waves x 2 blocks x 16)
constexpr int kTK = 64;            // keys per tile
constexpr float kLazy = 8.f;       // running-max slack before the accumulators are rescaled
#ifndef DLLM_ATTN_ST
#define DLLM_ATTN_ST 2
#endif
constexpr int kAttnST = DLLM_ATTN_ST;  // LDS ring slots (tiles in flight + the one being used)

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

typedef __attribute__((address_space(3))) void lds_void_a;
typedef short __attribute__((ext_vector_type(4))) s16x4;

template <int N>
__device__ __forceinline__ void attn_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// 16-byte chunk swizzle of a K or V row of 8 or 16 chunks, a function of row bits 0, 1, 3, 4. A K
// fragment read touches, per 16-lane group, the 16 rows in which those bits vary: they land on 16
// distinct chunk positions (256-byte rows) or on distinct (row parity, chunk) positions (128-byte
// rows). A transposing V read touches, per 32 lanes, 8 rows in which bits 0, 1, 3 vary, 32 bytes
// (one aligned chunk pair) each: the pair index depends on exactly those bits, so the 8 rows cover
// all banks once.
template <int CPR>
__device__ __forceinline__ int aswz(int r) {
  if constexpr (CPR == 8) return ((r >> 4) & 1) | (r & 2) | ((r >> 1) & 4);
  else return ((r >> 4) & 1) | ((r & 3) << 1) | (r & 8);
}

// V^T fragments of one 32-key group KS for every 16-wide hd block, read from V rows in their
// natural [key][hd] layout by the transposing LDS read (lane i of a 16-lane group receives, for each
// of the 4 keys addressed by lanes 4k .. 4k+3, the value at hd column i of the block). addr[hb] is
// the LDS byte address of the lane's first row (key 8 lg + q/4) for block hb; the second read of
// each block covers the keys 4 rows further, and group KS sits 32 rows further. The reads wait for
// their own completion inside the asm statement, so no result register is live while a read is
// still in flight. Written as asm because the compiler otherwise drains every outstanding
// direct-to-LDS K/V load before each transposing read.
template <int HD>
struct VtFrag;
template <>
struct VtFrag<128> {
  template <int KS>
  static __device__ __forceinline__ void read(const uint32_t (&addr)[8], s16x4 (&lo)[8],
                                              s16x4 (&hi)[8]) {
    if constexpr (KS == 0)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:0\n"
        "ds_read_b64_tr_b16 %1, %16 offset:1024\n"
        "ds_read_b64_tr_b16 %2, %17 offset:0\n"
        "ds_read_b64_tr_b16 %3, %17 offset:1024\n"
        "ds_read_b64_tr_b16 %4, %18 offset:0\n"
        "ds_read_b64_tr_b16 %5, %18 offset:1024\n"
        "ds_read_b64_tr_b16 %6, %19 offset:0\n"
        "ds_read_b64_tr_b16 %7, %19 offset:1024\n"
        "ds_read_b64_tr_b16 %8, %20 offset:0\n"
        "ds_read_b64_tr_b16 %9, %20 offset:1024\n"
        "ds_read_b64_tr_b16 %10, %21 offset:0\n"
        "ds_read_b64_tr_b16 %11, %21 offset:1024\n"
        "ds_read_b64_tr_b16 %12, %22 offset:0\n"
        "ds_read_b64_tr_b16 %13, %22 offset:1024\n"
        "ds_read_b64_tr_b16 %14, %23 offset:0\n"
        "ds_read_b64_tr_b16 %15, %23 offset:1024\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]), "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]), "v"(addr[7]));
    else
      asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:8192\n"
        "ds_read_b64_tr_b16 %1, %16 offset:9216\n"
        "ds_read_b64_tr_b16 %2, %17 offset:8192\n"
        "ds_read_b64_tr_b16 %3, %17 offset:9216\n"
        "ds_read_b64_tr_b16 %4, %18 offset:8192\n"
        "ds_read_b64_tr_b16 %5, %18 offset:9216\n"
        "ds_read_b64_tr_b16 %6, %19 offset:8192\n"
        "ds_read_b64_tr_b16 %7, %19 offset:9216\n"
        "ds_read_b64_tr_b16 %8, %20 offset:8192\n"
        "ds_read_b64_tr_b16 %9, %20 offset:9216\n"
        "ds_read_b64_tr_b16 %10, %21 offset:8192\n"
        "ds_read_b64_tr_b16 %11, %21 offset:9216\n"
        "ds_read_b64_tr_b16 %12, %22 offset:8192\n"
        "ds_read_b64_tr_b16 %13, %22 offset:9216\n"
        "ds_read_b64_tr_b16 %14, %23 offset:8192\n"
        "ds_read_b64_tr_b16 %15, %23 offset:9216\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]), "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]), "v"(addr[7]));
  }
};
template <>
struct VtFrag<64> {
  template <int KS>
  static __device__ __forceinline__ void read(const uint32_t (&addr)[4], s16x4 (&lo)[4],
                                              s16x4 (&hi)[4]) {
    if constexpr (KS == 0)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:0\n"
        "ds_read_b64_tr_b16 %1, %8 offset:512\n"
        "ds_read_b64_tr_b16 %2, %9 offset:0\n"
        "ds_read_b64_tr_b16 %3, %9 offset:512\n"
        "ds_read_b64_tr_b16 %4, %10 offset:0\n"
        "ds_read_b64_tr_b16 %5, %10 offset:512\n"
        "ds_read_b64_tr_b16 %6, %11 offset:0\n"
        "ds_read_b64_tr_b16 %7, %11 offset:512\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]));
    else
      asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:4096\n"
        "ds_read_b64_tr_b16 %1, %8 offset:4608\n"
        "ds_read_b64_tr_b16 %2, %9 offset:4096\n"
        "ds_read_b64_tr_b16 %3, %9 offset:4608\n"
        "ds_read_b64_tr_b16 %4, %10 offset:4096\n"
        "ds_read_b64_tr_b16 %5, %10 offset:4608\n"
        "ds_read_b64_tr_b16 %6, %11 offset:4096\n"
        "ds_read_b64_tr_b16 %7, %11 offset:4608\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]));
  }
};

// grid.x enumerates (sequence, kv head, key split) and grid.y the query tiles, so the tiles that
// share one K/V panel have ids grid.x apart: with grid.x a multiple of 8 they run on the same XCD
// and read the panel through one L2.
#ifndef DLLM_ATTN_WAVES
#define DLLM_ATTN_WAVES 2
#endif
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DLLM_ATTN_WAVES, DLLM_ATTN_WAVES)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int KB = HD / 32;          // 32-wide k-steps of q.k over hd
  constexpr int HB = HD / 16;          // 16-wide output blocks of hd
  constexpr int RB = HD * 2;           // bytes per K or V row
  constexpr int CPR = RB / 16;         // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;       // rows per DMA wave instruction
  constexpr int HALF = kTK * RB;       // bytes of the K (or V) rows of one tile
  constexpr int SLOT = 2 * HALF;       // K rows, then V rows
  constexpr int PER = SLOT / 1024 / 4;  // DMA instructions per wave per tile (K half, then V half)
  constexpr int ST = kAttnST;
  static_assert(ST >= 2 && (ST - 2) * PER < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char ring[ST * SLOT];

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
  const int ntile = (t1 - t0 + kTK - 1) / kTK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // m_run: reference point of the exponentials (base-2 units), identical in the 4 lanes that hold
  // one query; lacc: the sum of the exponentials (all 4 entries, in all 4 lanes of the query)
  float m_run[kQB];
  f32x4 lacc[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) { m_run[qb] = -INFINITY; lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  const size_t head_off = ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
  const uint16_t* kbase = a.kc + head_off;
  const uint16_t* vbase = a.vc + head_off;

  // ---- direct-to-LDS loads of one tile. DMA instruction p of a wave fills 1 KB = RPI rows of the
  // K half (p < PER/2) or V half: row = RPI (wave + 4 pp) + lane / CPR, pp = p mod PER/2, chunk
  // swizzled by the row. The swizzle repeats every 8 RPI rows, so two per-lane byte offsets cover
  // every pp; the rest of the address is wave-uniform.
  uint32_t doff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int rw = RPI * wave + lane / CPR;
    doff[e] = (uint32_t)(rw * RB + 16 * ((lane % CPR) ^ aswz<CPR>(rw + 4 * RPI * e)));
  }
  auto issue = [&](int it, char* slot) {
    const int tk = t0 + it * kTK;
    if (tk + kTK <= t1) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const bool isk = p < PER / 2;
        const int pp = isk ? p : p - PER / 2;
        const char* gb = (const char*)((isk ? kbase : vbase) + (size_t)(tk + 4 * RPI * pp) * HD);
        __builtin_amdgcn_global_load_lds(gb + doff[pp & 1],
                                         (lds_void_a*)(slot + (isk ? 0 : HALF) + (wave + 4 * pp) * 1024),
                                         16, 0, 0);
      }
    } else {  // last tile of a ragged range: rows past it repeat the last key (masked below)
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const bool isk = p < PER / 2;
        const int pp = isk ? p : p - PER / 2;
        const int row = RPI * (wave + 4 * pp) + lane / CPR;
        const int key = min(tk + row, t1 - 1);
        const int c = (lane % CPR) ^ aswz<CPR>(row);
        const uint16_t* src = (isk ? kbase : vbase) + (size_t)key * HD + 8 * c;
        __builtin_amdgcn_global_load_lds(src, (lds_void_a*)(slot + (isk ? 0 : HALF) + (wave + 4 * pp) * 1024),
                                         16, 0, 0);
      }
    }
  };

  // V^T fragment addresses relative to the slot: lane q of a 16-lane group reads 4 values of key
  // row 8 lg + q/4 at hd column 16 hb + 4 (q%4)
  const int trow = 8 * lg + (lr >> 2);
  uint32_t voff[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int col = 16 * hb + 4 * (lr & 3);
    voff[hb] = (uint32_t)(HALF + trow * RB + (((col >> 3) ^ aswz<CPR>(trow)) << 4) + (col & 7) * 2);
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
  // a zero scale (uniform attention) runs as a tiny positive one: every exponential is then exactly
  // 1 and masked keys still map to -inf rather than 0 * inf
  const float c = a.scale_log2 != 0.f ? a.scale_log2 : 1e-30f;
  const bool c_pos = c > 0.f;

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < ntile) issue(s, ring + s * SLOT);

  for (int it = 0; it < ntile; ++it) {
    const int ahead = min(ST - 2, ntile - 1 - it);  // tiles issued after tile it
    if (ST > 3 && ahead >= 2) attn_wait_vm<(ST > 3 ? 2 : 0) * PER>();
    else if (ST > 2 && ahead == 1) attn_wait_vm<PER>();
    else attn_wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");  // tile it landed everywhere; slot of it-1 is free
    if (it + ST - 1 < ntile) issue(it + ST - 1, ring + ((it + ST - 1) % ST) * SLOT);
    const int slot = it % ST;
    const char* sK = ring + slot * SLOT;
    const int tk = t0 + it * kTK;

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
        const int ch = (kb * 4 + lg) ^ aswz<CPR>(kr);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + kr * RB + (ch << 4));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sacc[qb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][kb], sacc[qb][blk],
                                                                   0, 0, 0);
      }
    }
    // sacc[qb][blk][i] = raw score q.k of query (qb, lr) with key tk + 32 ks + 8 lg + 4 half + i,
    // i.e. key offset 32 ks + 4 half + i from tk + 8 lg. On the last tile of a ragged range, keys
    // past it get the raw score whose scaled value is -inf: they drop out of the maximum and their
    // exponential is 0.
    if (tk + kTK > t1) {
      const int rem = t1 - tk - 8 * lg;
      const float excl = c_pos ? -INFINITY : INFINITY;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            if (32 * (blk >> 1) + 4 * (blk & 1) + i >= rem) sacc[qb][blk][i] = excl;
    }
    // ---- this lane's maximum of the scaled scores (the scale may be negative). The reference
    // point moves only when a tile maximum exceeds it by more than kLazy (base-2 units), so the
    // exponentials stay below 2^kLazy (exact in fp32 and bf16) and the final division by the sum of
    // the same exponentials cancels the reference. Whether any query of the wave needs a move is
    // decided from the lanes' own maxima; only then are they reduced across the 4 lanes of a query
    // and the accumulators rescaled.
    float lmax[kQB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float m;
      if (c_pos) {
        m = fmaxf(fmaxf(sacc[qb][0][0], sacc[qb][0][1]), fmaxf(sacc[qb][0][2], sacc[qb][0][3]));
#pragma unroll
        for (int blk = 1; blk < 4; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, sacc[qb][blk][i]);
      } else {
        m = fminf(fminf(sacc[qb][0][0], sacc[qb][0][1]), fminf(sacc[qb][0][2], sacc[qb][0][3]));
#pragma unroll
        for (int blk = 1; blk < 4; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fminf(m, sacc[qb][blk][i]);
      }
      lmax[qb] = m * c;
      need |= lmax[qb] > m_run[qb] + kLazy;
    }
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        float mx = lmax[qb];
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = (mx > m_run[qb] + kLazy) ? mx : m_run[qb];
        const float alpha = fast_exp2(m_run[qb] - m_new);  // 1 if kept; 0 on the first tile
        m_run[qb] = m_new;
        lacc[qb][0] *= alpha; lacc[qb][1] *= alpha; lacc[qb][2] *= alpha; lacc[qb][3] *= alpha;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          oacc[qb][hb][0] *= alpha; oacc[qb][hb][1] *= alpha;
          oacc[qb][hb][2] *= alpha; oacc[qb][hb][3] *= alpha;
        }
      }
    }
    bf16x8 pf[kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float mneg = -m_run[qb];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pf[qb][blk >> 1][4 * (blk & 1) + i] = (__bf16)fast_exp2(fmaf(sacc[qb][blk][i], c, mneg));
    }
    // ---- O^T += V^T P^T: A operand row = hd column, k-slot s = key 32 ks + 8 lg + s
    const uint32_t vslot = ring_lds + slot * SLOT;
    uint32_t addr[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) addr[hb] = vslot + voff[hb];
    auto pv = [&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      s16x4 lo[HB], hi[HB];
      VtFrag<HD>::template read<ks>(addr, lo, hi);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        typedef short __attribute__((ext_vector_type(8))) s16x8;
        const s16x8 both = {lo[hb][0], lo[hb][1], lo[hb][2], lo[hb][3],
                            hi[hb][0], hi[hb][1], hi[hb][2], hi[hb][3]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, both);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          oacc[qb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][ks], oacc[qb][hb],
                                                                  0, 0, 0);
      }
    };
    pv(std::integral_constant<int, 0>{});
    pv(std::integral_constant<int, 1>{});
    // sums of the same (bf16) probabilities: an all-ones A operand makes every row of the product
    // the column sum, so each lane receives its query's complete sum
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb][0], lacc[qb], 0, 0, 0);
      lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb][1], lacc[qb], 0, 0, 0);
    }
  }

  // oacc[qb][hb][i] = unnormalised o[query (qb, lr)][hd = 16 hb + 4 lg + i]; lacc holds the
  // query's complete sum
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l_tot = lacc[qb][0];
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
