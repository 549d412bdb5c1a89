// (4) Partial attention, gfx950.
//
// DyLLM (French summary page) §2.B: for salient tokens the row of the attention-score matrix
// is recomputed exactly; §1: attention is bidirectional, so a selected query attends to every
// cached position (no mask), including masked tokens and itself, with the K/V entries that the
// projection call of this step has just overwritten.
//
// Work decomposition: one workgroup = NW waves x 32 query rows of one (sequence b, kv head hk)
// against a key range. A "query row" is a (selected token, query head of hk's group) pair, so
// grouped heads share every K/V tile that is loaded (GQA packing). Per 64-key tile:
//   * K and V rows go straight from global memory into an LDS ring (direct-to-LDS loads issued
//     several tiles ahead), in their natural [key][hd] layout with a 16-byte-chunk swizzle;
//   * S^T = K Q^T on the bf16 matrix cores in 32x32x16 blocks (two per tile): the lane's
//     accumulator column is one query, so the lane owns 32 of its 64 scores;
//   * the 32 keys of an S^T block are permuted so that the exponentiated scores already sit in
//     the B-operand layout of the next product (4 chunks of 16 keys, 8 per lane);
//   * O^T += V^T P^T in 32x32x16 blocks; the V^T fragments come from the natural-layout V rows
//     through the transposing LDS read, fp32 accumulation.
// The exponentials use a lazily moved reference point: it moves (and the accumulators are
// rescaled) only when a tile's maximum exceeds it by more than 2^kLazy, so the common tile needs
// no cross-lane traffic. When the selected rows alone cannot fill the 256 compute units, the key
// range is split and the fp32 partials (o, reference, sum) are merged in a fixed order by a
// second pass, so results stay deterministic.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kTK = 64;         // keys per tile
constexpr float kLazy = 8.f;    // reference-point slack (base-2 units) before rescaling
constexpr float kKeepMass = 0.25f;  // stable-token update: smallest kept share of the stored mass

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
  // context of every token (NULL in the selected-rows-only call): per-token softmax state
  // (reference m in base-2 units, sum l of 2^(score - m), normalised context o in fp32), the
  // bf16 context and query of every token, and the compact copies of the overwritten K/V rows
  const int32_t* sel_idx;
  float* st_m;        // [B*S, H]
  float* st_l;        // [B*S, H]
  float* st_o;        // [B*S, H*hd]
  uint16_t* o_all;    // [B*S, H*hd]
  uint16_t* q_all;    // [B*S, H*hd]
  const uint16_t* k_old;  // [m_cap, Hkv, hd]
  const uint16_t* v_old;
  int q_first;            // stable-token pass: positions q_first .. S-1 of every sequence
  int qtiles;             // > 0: 1-D grid of groups x qtiles query tiles, XCD-grouped (FULL only)
};
constexpr int kDeltaMaxS = kSalientMaxS;  // the changed-position list of a sequence lives in LDS

typedef __attribute__((address_space(3))) void lds_void_a;
typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int N>
__device__ __forceinline__ void attn_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16-byte chunk swizzles of the K and V rows (CPR chunks per row).
// K: a fragment read touches, per 16-lane group, 16 key rows whose bits 0-3 vary; they land on
// 16 distinct chunk positions (256-byte rows) or distinct (row parity, chunk) positions (128-byte
// rows). V: a transposing read touches, per 32 lanes, 4 rows whose bits 0-1 vary, 64 bytes each;
// those bits select distinct 64-byte groups of the 256 bank bytes. The V swizzle ignores row
// bits 2, 4 and 5, so the reads 4 and 16 rows further are plain byte offsets.
template <int CPR>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (CPR == 8) return (r >> 1) & 7;
  else return r & 15;
}
template <int CPR>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (CPR == 8) return (r & 2) << 1;
  else return (r & 3) << 2;
}

// V^T fragments of one 16-key chunk CC for every 32-wide hd block, read from V rows in their
// natural [key][hd] layout by the transposing LDS read (per 16-lane group, lane i receives for each
// of the 4 rows addressed by lanes 4k .. 4k+3 the value at column i of the 16 columns they cover).
// addr[hb] is the LDS byte address of the lane's row (8 (lane/32) + q/4 of chunk 0); the second
// read of each block covers the rows 4 further, chunk CC sits 16 CC rows further. The reads wait
// for their own completion inside the asm statement, so no result register is live while a read is
// still in flight. Written as asm because the compiler otherwise drains every outstanding
// direct-to-LDS K/V load before each transposing read.
template <int HD>
struct VtFrag;
template <>
struct VtFrag<128> {
  template <int CC>
  static __device__ __forceinline__ void read(const uint32_t (&addr)[4], s16x4 (&lo)[4],
                                              s16x4 (&hi)[4]) {
    if constexpr (CC == 0)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:0\n"
        "ds_read_b64_tr_b16 %1, %8 offset:1024\n"
        "ds_read_b64_tr_b16 %2, %9 offset:0\n"
        "ds_read_b64_tr_b16 %3, %9 offset:1024\n"
        "ds_read_b64_tr_b16 %4, %10 offset:0\n"
        "ds_read_b64_tr_b16 %5, %10 offset:1024\n"
        "ds_read_b64_tr_b16 %6, %11 offset:0\n"
        "ds_read_b64_tr_b16 %7, %11 offset:1024\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]));
    else if constexpr (CC == 1)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:4096\n"
        "ds_read_b64_tr_b16 %1, %8 offset:5120\n"
        "ds_read_b64_tr_b16 %2, %9 offset:4096\n"
        "ds_read_b64_tr_b16 %3, %9 offset:5120\n"
        "ds_read_b64_tr_b16 %4, %10 offset:4096\n"
        "ds_read_b64_tr_b16 %5, %10 offset:5120\n"
        "ds_read_b64_tr_b16 %6, %11 offset:4096\n"
        "ds_read_b64_tr_b16 %7, %11 offset:5120\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]));
    else if constexpr (CC == 2)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:8192\n"
        "ds_read_b64_tr_b16 %1, %8 offset:9216\n"
        "ds_read_b64_tr_b16 %2, %9 offset:8192\n"
        "ds_read_b64_tr_b16 %3, %9 offset:9216\n"
        "ds_read_b64_tr_b16 %4, %10 offset:8192\n"
        "ds_read_b64_tr_b16 %5, %10 offset:9216\n"
        "ds_read_b64_tr_b16 %6, %11 offset:8192\n"
        "ds_read_b64_tr_b16 %7, %11 offset:9216\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]));
    else
      asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:12288\n"
        "ds_read_b64_tr_b16 %1, %8 offset:13312\n"
        "ds_read_b64_tr_b16 %2, %9 offset:12288\n"
        "ds_read_b64_tr_b16 %3, %9 offset:13312\n"
        "ds_read_b64_tr_b16 %4, %10 offset:12288\n"
        "ds_read_b64_tr_b16 %5, %10 offset:13312\n"
        "ds_read_b64_tr_b16 %6, %11 offset:12288\n"
        "ds_read_b64_tr_b16 %7, %11 offset:13312\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]));
  }
};

template <>
struct VtFrag<64> {
  template <int CC>
  static __device__ __forceinline__ void read(const uint32_t (&addr)[2], s16x4 (&lo)[2],
                                              s16x4 (&hi)[2]) {
    if constexpr (CC == 0)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:0\n"
        "ds_read_b64_tr_b16 %1, %4 offset:512\n"
        "ds_read_b64_tr_b16 %2, %5 offset:0\n"
        "ds_read_b64_tr_b16 %3, %5 offset:512\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(addr[0]), "v"(addr[1]));
    else if constexpr (CC == 1)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:2048\n"
        "ds_read_b64_tr_b16 %1, %4 offset:2560\n"
        "ds_read_b64_tr_b16 %2, %5 offset:2048\n"
        "ds_read_b64_tr_b16 %3, %5 offset:2560\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(addr[0]), "v"(addr[1]));
    else if constexpr (CC == 2)
      asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:4096\n"
        "ds_read_b64_tr_b16 %1, %4 offset:4608\n"
        "ds_read_b64_tr_b16 %2, %5 offset:4096\n"
        "ds_read_b64_tr_b16 %3, %5 offset:4608\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(addr[0]), "v"(addr[1]));
    else
      asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:6144\n"
        "ds_read_b64_tr_b16 %1, %4 offset:6656\n"
        "ds_read_b64_tr_b16 %2, %5 offset:6144\n"
        "ds_read_b64_tr_b16 %3, %5 offset:6656\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(addr[0]), "v"(addr[1]));
  }
};

// grid.x enumerates (sequence, kv head, key split) and grid.y the query tiles, so the tiles that
// share one K/V panel have ids grid.x apart: with grid.x a multiple of 8 they run on the same XCD
// and read the panel through one L2.
//
// DELTA: the stable-token pass of DyLLM (French summary page) §2.B. The queries are every
// position of the sequence (their cached query vectors), and the keys are the changed rows only:
// tile t holds the new K/V rows of selected entries 32t .. 32t+31 (rows 0-31, gathered from the
// cache) and their old rows (rows 32-63, from the copies taken before the projection call). The
// old rows' exponentials enter with a negative sign, so the tile loop accumulates the change of
// the softmax numerator and denominator relative to the token's stored reference point; the
// epilogue adds it to the stored state. Rows of selected positions are computed too and are
// overwritten by the exact pass that runs next.
//
// FULL: the call is planned for every position of every sequence as a query row (m_plan >= B S:
// the dense layers), so every query tile of a (sequence, kv head) has rows. With a.qtiles > 0 the
// grid is 1-D and the query tiles of one K/V panel are dispatched together on one XCD: workgroup
// ids x, x+8, x+16, ... share an L2, and the panel's a.qtiles tiles take consecutive ones of
// them, so the panel is fetched from HBM once rather than once per round of workgroups. (The
// selected-row launches keep the 2-D grid: there most tiles past the first are empty. A call with
// room for every position but planned for fewer rows, as in the layer-adaptive step, is one of
// them: on the 1-D grid its few live tiles sat behind empty ones, 9.0 vs 8.5 ms per 32-layer step.)
template <int HD, int NW, int ST, bool DELTA, bool FULL = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int KK = HD / 16;              // 16-wide k-steps of q.k over hd
  constexpr int NB = HD / 32;              // 32-wide hd blocks of the output
  constexpr int RB = HD * 2;               // bytes per K or V row
  constexpr int CPR = RB / 16;             // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;           // rows per DMA wave instruction
  constexpr int HALF = kTK * RB;           // bytes of the K (or V) rows of one tile
  constexpr int SLOT = 2 * HALF;           // K rows, then V rows
  constexpr int PER = SLOT / 1024 / NW;    // DMA instructions per wave per tile (K half, V half)
  constexpr int TQ = 32 * NW;              // query rows per workgroup
  static_assert(PER % 2 == 0 && ST >= 2 && (ST - 2) * PER < 64, "tile shape");
  // DELTA: the ring is followed by the list of changed positions of the sequence
  __shared__ __attribute__((aligned(1024))) char ring[ST * SLOT + (DELTA ? kDeltaMaxS * 4 : 0)];

  const int G = a.H / a.Hkv;
  const int Nq = a.H * HD;
  const int per_b = a.Hkv * a.nsplit;
  int bx = blockIdx.x, by = blockIdx.y;
  if constexpr (FULL) {
    if (a.qtiles > 0) {  // id l on XCD l % 8; that XCD's (l / 8)-th workgroup
      const int slot = (int)blockIdx.x >> 3;
      by = slot % a.qtiles;
      bx = (slot / a.qtiles) * 8 + ((int)blockIdx.x & 7);
    }
  }
  const int b = bx / per_b;
  const int hk = (bx - b * per_b) / a.nsplit;
  const int split = bx - b * per_b - hk * a.nsplit;
  const int M = min(a.row_ptr[a.B], a.m_cap);
  const int r0 = min(a.row_ptr[b], M), r1 = min(a.row_ptr[b + 1], M);
  const int nA = r1 - r0;  // selected (changed) positions of the sequence
  const int nrows = DELTA ? (a.S - a.q_first) * G : nA * G;
  const int tile0 = by * TQ;
  if (tile0 >= nrows) return;
  // key range [t0, t1) of this split; DELTA: entries [0, nA) of the changed list, 32 per tile
  const int t0 = DELTA ? 0 : split * a.kps;
  const int t1 = DELTA ? nA : min(a.S, t0 + a.kps);
  const int ntile = DELTA ? (nA + 31) / 32 : (t1 - t0 + kTK - 1) / kTK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5, g = lane >> 4, q16 = lane & 15;

  // ---- this lane's query: column n of the wave's 32-query block. qj: compact row of a selected
  // token, or (DELTA) the flat position b*S + s
  const int qr = tile0 + 32 * wave + n;
  const bool qvalid = qr < nrows;
  const int qj = qvalid ? (DELTA ? b * a.S + a.q_first + qr / G : r0 + qr / G) : 0;
  const int qh = qvalid ? hk * G + qr % G : 0;
  const uint16_t* qsrc = DELTA ? a.q_all : a.q;
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = qvalid ? *reinterpret_cast<const bf16x8*>(qsrc + (size_t)qj * Nq + qh * HD + 16 * kk + 8 * h)
                    : bf16x8{};

  f32x16 oacc[NB];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[hb][i] = 0.f;
  // m_run: reference point of the exponentials (base-2 units), the same in the two lanes of a
  // query; l_run: this lane's share (its 32 keys of every tile) of the sum of exponentials.
  // DELTA starts from the token's stored reference point.
  const float m_state = (DELTA && qvalid) ? a.st_m[(size_t)qj * a.H + qh] : 0.f;
  float m_run = DELTA ? m_state : -INFINITY, l_run = 0.f;
  const int* apos = reinterpret_cast<const int*>(ring + ST * SLOT);
  if constexpr (DELTA) {
    int* wpos = reinterpret_cast<int*>(ring + ST * SLOT);
    for (int i = tid; i < nA; i += 64 * NW) wpos[i] = a.sel_idx[r0 + i] - b * a.S;
    __syncthreads();
  }

  const size_t head_off = ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
  const uint16_t* kbase = a.kc + head_off;
  const uint16_t* vbase = a.vc + head_off;

  // ---- direct-to-LDS loads of one tile. DMA instruction p of a wave fills 1 KB block
  // j = wave + NW pp (pp = p mod PER/2) of the K half (p < PER/2) or of the V half: rows
  // RPI j + lane/CPR, chunk swizzled by the row. The swizzles do not see the row bits that pp
  // changes, so one per-lane byte offset per half covers every pp; the rest is wave-uniform.
  const int rw = RPI * wave + lane / CPR;
  const uint32_t doff_k = (uint32_t)(rw * RB + 16 * ((lane % CPR) ^ swz_k<CPR>(rw)));
  const uint32_t doff_v = (uint32_t)(rw * RB + 16 * ((lane % CPR) ^ swz_v<CPR>(rw)));
  auto issue = [&](int it, char* slot) {
    if constexpr (DELTA) {  // rows 0-31: new rows of changed entries 32 it + r; rows 32-63: old
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const bool isk = p < PER / 2;
        const int pp = isk ? p : p - PER / 2;
        const int row = RPI * (wave + NW * pp) + lane / CPR;
        const int j = min(32 * it + (row & 31), nA - 1);  // past the list: repeat its last entry
        const int cch = (lane % CPR) ^ (isk ? swz_k<CPR>(row) : swz_v<CPR>(row));
        const uint16_t* src = row < 32 ? (isk ? kbase : vbase) + (size_t)apos[j] * HD
                                       : (isk ? a.k_old : a.v_old) + ((size_t)(r0 + j) * a.Hkv + hk) * HD;
        __builtin_amdgcn_global_load_lds(src + 8 * cch,
                                         (lds_void_a*)(slot + (isk ? 0 : HALF) + (wave + NW * pp) * 1024),
                                         16, 0, 0);
      }
      return;
    }
    const int tk = t0 + it * kTK;
    if (tk + kTK <= t1) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const bool isk = p < PER / 2;
        const int pp = isk ? p : p - PER / 2;
        const char* gb = (const char*)((isk ? kbase : vbase) + (size_t)(tk + RPI * NW * pp) * HD);
        __builtin_amdgcn_global_load_lds(gb + (isk ? doff_k : doff_v),
                                         (lds_void_a*)(slot + (isk ? 0 : HALF) + (wave + NW * pp) * 1024),
                                         16, 0, 0);
      }
    } else {  // last tile of a ragged range: rows past it repeat the last key (masked below)
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const bool isk = p < PER / 2;
        const int pp = isk ? p : p - PER / 2;
        const int row = RPI * (wave + NW * pp) + lane / CPR;
        const int key = min(tk + row, t1 - 1);
        const int c = (lane % CPR) ^ (isk ? swz_k<CPR>(row) : swz_v<CPR>(row));
        const uint16_t* src = (isk ? kbase : vbase) + (size_t)key * HD + 8 * c;
        __builtin_amdgcn_global_load_lds(src, (lds_void_a*)(slot + (isk ? 0 : HALF) + (wave + NW * pp) * 1024),
                                         16, 0, 0);
      }
    }
  };

  // K fragment rows: S^T row n of key block kb2 holds key 32 kb2 + 16 (n/16) + 8 ((n/4)%2) +
  // 4 ((n/8)%2) + n%4, which puts the scores of chunk cc (16 keys) at accumulator entries
  // 8 (cc%2) .. 8 (cc%2) + 7 of block cc/2, in k-slot order 8 (lane/32) + i
  const int kr = 16 * (n >> 4) + 8 * ((n >> 2) & 1) + 4 * ((n >> 3) & 1) + (n & 3);
  // V^T fragment addresses (relative to the slot): lane q16 of 16-lane group g reads row
  // 8 (g/2) + q16/4 at hd column 32 hb + 16 (g%2) + 4 (q16%4)
  const int vr = 8 * (g >> 1) + (q16 >> 2);
  uint32_t voff[NB];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    const int col = 32 * hb + 16 * (g & 1) + 4 * (q16 & 3);
    voff[hb] = (uint32_t)(HALF + vr * RB + (((col >> 3) ^ swz_v<CPR>(vr)) << 4) + (col & 7) * 2);
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
  // a zero scale (uniform attention) runs as a tiny positive one: every exponential is then exactly
  // 1 and masked keys still map to -inf rather than 0 * inf
  const float c = a.scale_log2 != 0.f ? a.scale_log2 : 1e-30f;
  const bool c_pos = c > 0.f;

  static_assert(ST == 4, "the pipelined loop below assumes a 4-slot ring");
  // ---- S^T blocks (32 keys x 32 queries) of the tile in slot `sK`
  auto scores = [&](const char* sK, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb2][i] = 0.f;
      const int key = 32 * kb2 + kr;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int ch = (2 * kk + h) ^ swz_k<CPR>(key);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + key * RB + (ch << 4));
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb2], 0, 0, 0);
      }
    }
  };
  // sacc[kb2][rr] = raw score of query n with key tk + 8 h + koff(kb2, rr),
  // koff = 32 kb2 + 16 (rr/8) + 4 ((rr/4)%2) + rr%4. On the last tile of a ragged range, keys
  // past it get the raw score whose scaled value is -inf: they drop out of the maximum and their
  // exponential is 0. DELTA: both halves (new and old rows) hold entries 32 it + 8 h + koff % 32.
  auto mask_tail = [&](f32x16 (&sacc)[2], int it) __attribute__((always_inline)) {
    const int span = DELTA ? 32 : kTK;
    const int tk = t0 + it * span;
    if (tk + span > t1) {
      const int rem = t1 - tk - 8 * h;
      const float excl = c_pos ? -INFINITY : INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if ((DELTA ? 0 : 32 * kb2) + 16 * (rr >> 3) + 4 * ((rr >> 2) & 1) + (rr & 3) >= rem)
            sacc[kb2][rr] = excl;
    }
  };
  // DELTA: the old rows (block 1, chunks 2 and 3) enter with a negative sign
  auto sgn = [](int kb2) constexpr { return (DELTA && kb2 == 1) ? -1.f : 1.f; };
  // ---- lazily moved reference point: it moves only when a tile maximum exceeds it by more than
  // kLazy, so the exponentials stay below 2^kLazy (exact in fp32 and bf16) and the final division
  // by the sum of the same exponentials cancels it. Whether any query of the wave needs a move is
  // decided from the lanes' own maxima; only then are they combined across the two lanes of a
  // query and the accumulators rescaled (after the previous tile's products, before this tile's).
  auto reference = [&](const f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    float lmax;
    if (c_pos) {
      lmax = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) lmax = fmaxf(lmax, sacc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) lmax = fmaxf(lmax, sacc[1][i]);
    } else {
      lmax = fminf(sacc[0][0], sacc[0][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) lmax = fminf(lmax, sacc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) lmax = fminf(lmax, sacc[1][i]);
    }
    lmax *= c;
    if (__any(lmax > m_run + kLazy)) {
      const float mx = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
      const float m_new = (mx > m_run + kLazy) ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);  // 1 if kept; 0 on the first tile
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int hb = 0; hb < NB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[hb][i] *= alpha;
    }
  };
  // exponentials of one tile in the B-operand layout of the next product: chunk cc holds keys
  // 16 cc + 8 h + i8
  auto expo = [&](const f32x16 (&sacc)[2], bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    const float mneg = -m_run;
    float psum = 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8) {
        const float p = sgn(cc >> 1) * fast_exp2(fmaf(sacc[cc >> 1][8 * (cc & 1) + i8], c, mneg));
        psum += p;
        pf[cc][i8] = (__bf16)p;
      }
    l_run += psum;
  };
  // Scores of the next tile on the matrix cores interleaved, in a fixed instruction order, with
  // the exponentials of the current tile on the vector units: group t issues product t (block
  // t%2, k-step t/2; its K fragment was read two groups earlier), the read for product t+2 and the
  // exponentials of entries 2t, 2t+1 of the current tile. The scheduling barriers keep the
  // compiler from regrouping the products and the vector work.
  auto scores_expo = [&](const char* sK, f32x16 (&sacc)[2], const f32x16 (&cur)[2],
                         bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    constexpr int NG = 2 * KK > 16 ? 2 * KK : 16;  // groups: products and pairs of exponentials
    bf16x8 kf[2 * KK];
    auto kread = [&](int t) __attribute__((always_inline)) {
      const int key = 32 * (t & 1) + kr;
      const int ch = (2 * (t >> 1) + h) ^ swz_k<CPR>(key);
      kf[t] = *reinterpret_cast<const bf16x8*>(sK + key * RB + (ch << 4));
    };
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb2][i] = 0.f;
    kread(0);
    kread(1);
    const float mneg = -m_run;
    float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      if (t < 2 * KK)
        sacc[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[t >> 1], sacc[t & 1], 0, 0, 0);
      if (t + 2 < 2 * KK) kread(t + 2);
      if (t < 16) {
        const int v = 2 * t, kb2 = v >> 4, rr = v & 15;
        const float p0 = sgn(kb2) * fast_exp2(fmaf(cur[kb2][rr], c, mneg));
        const float p1 = sgn(kb2) * fast_exp2(fmaf(cur[kb2][rr + 1], c, mneg));
        psum0 += p0;
        psum1 += p1;
        pf[2 * kb2 + (rr >> 3)][rr & 7] = (__bf16)p0;
        pf[2 * kb2 + (rr >> 3)][(rr & 7) + 1] = (__bf16)p1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += psum0 + psum1;
  };
  // ---- O^T += V^T P^T for the tile in ring slot `slot`, 16 keys per product
  auto pv = [&](int slot, const bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    const uint32_t vslot = ring_lds + slot * SLOT;
    uint32_t addr[NB];
#pragma unroll
    for (int hb = 0; hb < NB; ++hb) addr[hb] = vslot + voff[hb];
    auto block = [&](auto cc_c) __attribute__((always_inline)) {
      constexpr int cc = decltype(cc_c)::value;
      s16x4 lo[NB], hi[NB];
      VtFrag<HD>::template read<cc>(addr, lo, hi);
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
        typedef short __attribute__((ext_vector_type(8))) s16x8;
        const s16x8 both = {lo[hb][0], lo[hb][1], lo[hb][2], lo[hb][3],
                            hi[hb][0], hi[hb][1], hi[hb][2], hi[hb][3]};
        oacc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[cc],
                                                            oacc[hb], 0, 0, 0);
      }
    };
    block(std::integral_constant<int, 0>{});
    block(std::integral_constant<int, 1>{});
    block(std::integral_constant<int, 2>{});
    block(std::integral_constant<int, 3>{});
  };

  // Software pipeline over the 4-slot ring: while the exponentials of tile it are computed on the
  // vector units, the matrix cores already form the scores of tile it+1; then tile it's products
  // with V. Tile t is loaded 3 tiles ahead into the slot that tile t-4 used.
  // A wave whose 32 query rows all lie past the last one (the tail of the last query tile) still
  // loads its share of every tile and meets every barrier, but forms no scores or products: the
  // matrix cores of its SIMD are left to the other wave there.
  const bool live = tile0 + 32 * wave < nrows;
  if (!DELTA || ntile > 0) {  // (a stable-token pass over a sequence with no change has no tile)
#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
      if (s < ntile) issue(s, ring + s * SLOT);
    if (ntile > 2) attn_wait_vm<2 * PER>();  // tile 0 landed
    else if (ntile > 1) attn_wait_vm<PER>();
    else attn_wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");
    f32x16 sa[2], sb[2];
    if (live) {
      scores(ring, sa);
      mask_tail(sa, 0);
    }
    bf16x8 pf[4];

    for (int it = 0; it + 1 < ntile; ++it) {
      // tile it+1 landed (the only later tile in flight is it+2); every wave finished tile it-1
      if (it + 2 < ntile) attn_wait_vm<PER>();
      else attn_wait_vm<0>();
      asm volatile("s_barrier" ::: "memory");
      if (it + 3 < ntile) issue(it + 3, ring + ((it + 3) % ST) * SLOT);
      if (live) {
        reference(sa);
        scores_expo(ring + ((it + 1) % ST) * SLOT, sb, sa, pf);
        pv(it % ST, pf);
        mask_tail(sb, it + 1);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) sa[kb2] = sb[kb2];
      }
    }
    if (live) {
      reference(sa);
      expo(sa, pf);
      pv((ntile - 1) % ST, pf);
    }
  }

  // oacc[hb][rr] = unnormalised o[query n][hd 32 hb + 8 (rr/4) + 4 h + rr%4]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  if constexpr (DELTA) {
    // stored state scaled to this pass's reference point, plus the change of numerator and sum
    const size_t sh = (size_t)qj * a.H + qh;
    const float lf = a.st_l[sh] * fast_exp2(m_state - m_run);
    const float l_new = lf + l_tot;
    // Cancellation guard. The old rows' exponentials are taken out of the numerator in bf16, so
    // its error is about 2^-9 of the removed mass, which is at most lf; relative to the result
    // that is 2^-9 lf / l_new. Where less than a quarter of the stored mass is left (a changed key
    // held most of the token's weight), or the sum is not a positive finite number, the update
    // is not used: the state is marked (st_l = -1) and the recompute pass that runs after the
    // exact pass rebuilds it against every key. Both lanes of a query hold the same sums.
    if (!(l_new > 0.f && l_new >= kKeepMass * lf && l_new < INFINITY)) {
      if (h == 0) a.st_l[sh] = -1.f;
      return;
    }
    const float inv = 1.0f / l_new;
    float* so = a.st_o + (size_t)qj * Nq + qh * HD;
#pragma unroll
    for (int hb = 0; hb < NB; ++hb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int e = 32 * hb + 8 * jj + 4 * h;
        float o0[4];
        Elem<float>::load4(so + e, o0);
        const float v[4] = {(o0[0] * lf + oacc[hb][4 * jj]) * inv, (o0[1] * lf + oacc[hb][4 * jj + 1]) * inv,
                            (o0[2] * lf + oacc[hb][4 * jj + 2]) * inv, (o0[3] * lf + oacc[hb][4 * jj + 3]) * inv};
        Elem<float>::store4(so + e, v);
        Elem<uint16_t>::store4(a.o_all + (size_t)qj * Nq + qh * HD + e, v);
      }
    if (h == 0) {
      a.st_m[sh] = m_run;
      a.st_l[sh] = l_new;
    }
    return;
  }
  // exact pass with the context of every token: the token's position, query and state
  const int pos = a.st_o ? a.sel_idx[qj] : 0;
  if (a.q_all && split == 0) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      *reinterpret_cast<bf16x8*>(a.q_all + (size_t)pos * Nq + qh * HD + 16 * kk + 8 * h) = qf[kk];
  }
  if (a.nsplit == 1) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int hb = 0; hb < NB; ++hb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float v[4] = {oacc[hb][4 * jj] * inv, oacc[hb][4 * jj + 1] * inv,
                            oacc[hb][4 * jj + 2] * inv, oacc[hb][4 * jj + 3] * inv};
        Elem<uint16_t>::store4(a.o + (size_t)qj * Nq + qh * HD + 32 * hb + 8 * jj + 4 * h, v);
        if (a.st_o) {
          Elem<float>::store4(a.st_o + (size_t)pos * Nq + qh * HD + 32 * hb + 8 * jj + 4 * h, v);
          Elem<uint16_t>::store4(a.o_all + (size_t)pos * Nq + qh * HD + 32 * hb + 8 * jj + 4 * h, v);
        }
      }
    if (a.st_o && h == 0) {
      a.st_m[(size_t)pos * a.H + qh] = m_run;
      a.st_l[(size_t)pos * a.H + qh] = l_tot;
    }
  } else {
    const size_t base = ((size_t)split * a.m_cap + qj) * a.H + qh;
#pragma unroll
    for (int hb = 0; hb < NB; ++hb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float v[4] = {oacc[hb][4 * jj], oacc[hb][4 * jj + 1], oacc[hb][4 * jj + 2],
                            oacc[hb][4 * jj + 3]};
        Elem<float>::store4(a.part_o + base * HD + 32 * hb + 8 * jj + 4 * h, v);
      }
    if (h == 0) {
      a.part_ml[base * 2] = m_run;
      a.part_ml[base * 2 + 1] = l_tot;
    }
  }
}

// fixed-order log-sum-exp merge of the key-split partials; one thread per 4 output columns.
// NS > 0: exactly NS splits, every partial loaded before the merge; NS == 0: a.nsplit of them.
template <int HD, int NS = 0>
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
  float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (NS > 0) {
    float2 ml[NS];
    float p[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const size_t base = ((size_t)s * a.m_cap + j) * a.H + h;
      ml[s] = *reinterpret_cast<const float2*>(a.part_ml + base * 2);
      Elem<float>::load4(a.part_o + base * HD + c, p[s]);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) mmax = fmaxf(mmax, ml[s].x);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float w = fast_exp2(ml[s].x - mmax);
      L += w * ml[s].y;
      o[0] += w * p[s][0]; o[1] += w * p[s][1]; o[2] += w * p[s][2]; o[3] += w * p[s][3];
    }
  } else {
    for (int s = 0; s < a.nsplit; ++s)
      mmax = fmaxf(mmax, a.part_ml[(((size_t)s * a.m_cap + j) * a.H + h) * 2]);
    for (int s = 0; s < a.nsplit; ++s) {
      const size_t base = ((size_t)s * a.m_cap + j) * a.H + h;
      const float w = fast_exp2(a.part_ml[base * 2] - mmax);
      L += w * a.part_ml[base * 2 + 1];
      float p[4];
      Elem<float>::load4(a.part_o + base * HD + c, p);
      o[0] += w * p[0]; o[1] += w * p[1]; o[2] += w * p[2]; o[3] += w * p[3];
    }
  }
  const float inv = 1.0f / L;
  const float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  Elem<uint16_t>::store4(a.o + (size_t)j * a.H * HD + h * HD + c, v);
  if (a.st_o) {  // context of every token: state and context at the token's position
    const size_t pos = (size_t)a.sel_idx[j];
    Elem<float>::store4(a.st_o + pos * a.H * HD + h * HD + c, v);
    Elem<uint16_t>::store4(a.o_all + pos * a.H * HD + h * HD + c, v);
    if (c == 0) {
      a.st_m[pos * a.H + h] = mmax;
      a.st_l[pos * a.H + h] = L;
    }
  }
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

// bf16 launch plan: waves per workgroup (32 query rows each) and the key split. Eight waves
// (256 rows; at hd 128 one workgroup per CU with a 4-slot ring of 128 KB); at hd 64 four waves
// (two workgroups per CU) when a (sequence, kv head) has at most 160 query rows on average. The
// key range is split until the workgroups fill every CU slot, keeping at least 256 keys (four
// tiles) per split: with two tiles most of a split's time is the ring's start-up. Measured on
// MI355X at 128 query rows of one sequence (S = 1024, 32 heads of 128), us per call: eight waves
// with at least two / four tiles per split 18.8 / 16.2; four waves (one 128-row tile per
// sequence and kv head) 19.7 / 17.8.
struct AttnCfg {
  int nw, st, nsplit, kps;
};
static AttnCfg plan_bf16(const ProjShape& s) {
  AttnCfg c;
  const int G = s.H / s.Hkv;
  const long rows_avg = (long)cdiv((long)s.m_plan * G, s.B);
  c.nw = (s.hd == 128 || rows_avg > 160) ? 8 : 4;
  c.st = 4;
  const long slots = 256L * (s.hd == 128 ? 1 : 2);
  const long est = (long)s.B * s.Hkv * (rows_avg > 0 ? cdiv(rows_avg, 32 * c.nw) : 1);
  c.nsplit = 1;
  while (est * c.nsplit < slots && s.S / (c.nsplit * 2) >= 256) c.nsplit *= 2;
  c.kps = cdiv(cdiv(s.S, c.nsplit), kTK) * kTK;
  c.nsplit = cdiv(s.S, c.kps);  // every split owns at least one key
  return c;
}

AttnPlan plan_attn(bool bf16, const ProjShape& s) {
  return AttnPlan{bf16 ? plan_bf16(s).nsplit : 1};
}

size_t attn_workspace_bytes(bool bf16, const ProjShape& s) {
  if (!bf16) return 0;
  const AttnCfg c = plan_bf16(s);
  if (c.nsplit <= 1) return 0;
  const size_t rows = (size_t)c.nsplit * s.m_cap * s.H;
  return ((rows * s.hd * 4 + 255) & ~(size_t)255) + rows * 2 * 4;
}

template <int HD, bool FULL>
static void launch_bf16(const AttnCfg& c, dim3 grid, const AttnArgs& a, hipStream_t st) {
  if constexpr (HD == 64) {
    if (c.nw == 4) {
      hipLaunchKernelGGL((attn_bf16_kernel<HD, 4, 4, false, FULL>), grid, dim3(256), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((attn_bf16_kernel<HD, 8, 4, false, FULL>), grid, dim3(512), 0, st, a);
}

template <int HD>
static void launch_merge(int nsplit, dim3 grid, const AttnArgs& a, hipStream_t st) {
  switch (nsplit) {
    case 2: hipLaunchKernelGGL((attn_merge_kernel<HD, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_merge_kernel<HD, 4>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_merge_kernel<HD, 8>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((attn_merge_kernel<HD>), grid, dim3(256), 0, st, a); break;
  }
}

// exact pass over the selected rows (plus, when `ctx` carries them, the state outputs)
static hipError_t launch_exact_bf16(const ProjShape& s, float scale, const void* q_sel,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* row_ptr, void* o_sel, void* ws,
                                    const AttnArgs& ctx, hipStream_t st);

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
  AttnArgs none{};
  return launch_exact_bf16(s, scale, q_sel, k_cache, v_cache, row_ptr, o_sel, ws, none, st);
}

static hipError_t launch_exact_bf16(const ProjShape& s, float scale, const void* q_sel,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* row_ptr, void* o_sel, void* ws,
                                    const AttnArgs& ctx, hipStream_t st) {
  const AttnCfg c = plan_bf16(s);
  AttnArgs a = ctx;
  a.q = (const uint16_t*)q_sel; a.kc = (const uint16_t*)k_cache; a.vc = (const uint16_t*)v_cache;
  a.row_ptr = row_ptr; a.o = (uint16_t*)o_sel;
  a.B = s.B; a.S = s.S; a.H = s.H; a.Hkv = s.Hkv; a.m_cap = s.m_cap;
  a.nsplit = c.nsplit; a.kps = c.kps;
  a.scale_log2 = scale * kLog2e;
  a.part_o = nullptr; a.part_ml = nullptr;
  if (a.nsplit > 1) {
    const size_t rows = (size_t)a.nsplit * s.m_cap * s.H;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + ((rows * s.hd * 4 + 255) & ~(size_t)255));
  }
  const int G = s.H / s.Hkv;
  const int rows_max = (s.m_cap < s.S ? s.m_cap : s.S) * G;
  const int groups = s.B * s.Hkv * a.nsplit, qtiles = cdiv(rows_max, 32 * c.nw);
  dim3 grid(groups, qtiles);
  const bool full = (long)s.m_plan >= (long)s.B * s.S;
  a.qtiles = 0;
  if (full && groups % 8 == 0 && qtiles > 1) {
    a.qtiles = qtiles;
    grid = dim3((unsigned)(groups * qtiles));
  }
  if (s.hd == 64)
    full ? launch_bf16<64, true>(c, grid, a, st) : launch_bf16<64, false>(c, grid, a, st);
  else
    full ? launch_bf16<128, true>(c, grid, a, st) : launch_bf16<128, false>(c, grid, a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const size_t threads = (size_t)s.m_cap * s.H * (s.hd / 4);
  dim3 mg((unsigned)((threads + 255) / 256));
  if (s.hd == 64) launch_merge<64>(a.nsplit, mg, a, st);
  else launch_merge<128>(a.nsplit, mg, a, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- context of every token
// Positions before q_first (a prompt left out of a response-only step, DyLLM French summary page
// §2.C): their state is not touched; the bf16 context is re-emitted from it, so o_all holds every
// token's context after each call. One thread per 4 columns of a row.
__global__ __launch_bounds__(256) void state_context_kernel(const float* st_o, uint16_t* o_all,
                                                            int S, int q_first, int Nq,
                                                            size_t total) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c4 = Nq / 4;
  const size_t row = idx / c4;             // b * q_first + s
  const int c = (int)(idx - row * c4) * 4;
  const size_t b = row / q_first, si = row - b * q_first;
  const size_t off = (b * S + si) * Nq + c;
  float v[4];
  Elem<float>::load4(st_o + off, v);
  Elem<uint16_t>::store4(o_all + off, v);
}

// Exact state of the (token, head) pairs the stable-token update marked (st_l < 0, or not a
// number: a state that no update may build on), against every key of the updated cache with the
// token's stored query: the definition of the state written out, in float32 with exact
// exponentials. One workgroup per 256 pairs; it lists its marked pairs in LDS and works through
// them one at a time with all its threads: scores (a thread per key), maximum and sum, then the
// context (a thread per (column, key residue) with a fixed-order sum of the residues). Positions
// before q_first are never touched. A workgroup with no marked pair only reads its 256 sums.
template <int HD>
__global__ __launch_bounds__(256) void stable_recompute_kernel(AttnArgs a) {
  constexpr int KG = 256 / HD;  // key residues of the context sums
  __shared__ float sc[kSalientMaxS];
  __shared__ float qs[HD];
  __shared__ float part[KG][HD];
  __shared__ float red[4];
  __shared__ int list[256];
  __shared__ int nlist;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Nq = a.H * HD, G = a.H / a.Hkv;
  const size_t total = (size_t)a.B * a.S * a.H;
  const size_t pair = (size_t)blockIdx.x * 256 + tid;
  if (tid == 0) nlist = 0;
  __syncthreads();
  if (pair < total) {
    const int s = (int)((pair / a.H) % a.S);
    if (s >= a.q_first && !(a.st_l[pair] >= 0.f)) list[atomicAdd(&nlist, 1)] = tid;
  }
  __syncthreads();
  const int n = nlist;
  for (int f = 0; f < n; ++f) {
    const size_t pr = (size_t)blockIdx.x * 256 + list[f];
    const size_t pos = pr / a.H;
    const int h = (int)(pr - pos * a.H), b = (int)(pos / a.S), hk = h / G;
    const uint16_t* kb = a.kc + ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
    const uint16_t* vb = a.vc + ((size_t)b * a.Hkv + hk) * (size_t)a.S * HD;
    if (tid < HD) qs[tid] = bf2f(a.q_all[pos * Nq + (size_t)h * HD + tid]);
    __syncthreads();
    float mx = -INFINITY;
    for (int t = tid; t < a.S; t += 256) {
      float d = 0.f;
      for (int e = 0; e < HD; ++e) d = fmaf(qs[e], bf2f(kb[(size_t)t * HD + e]), d);
      sc[t] = d * a.scale_log2;
      mx = fmaxf(mx, sc[t]);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float ls = 0.f;
    for (int t = tid; t < a.S; t += 256) {
      const float pt = exp2f(sc[t] - m);
      sc[t] = pt;
      ls += pt;
    }
    ls = wave_sum(ls);
    if (lane == 0) red[wave] = ls;
    __syncthreads();
    const float l = (red[0] + red[1]) + (red[2] + red[3]);
    const int e = tid % HD, g = tid / HD;
    float acc = 0.f;
    for (int t = g; t < a.S; t += KG) acc = fmaf(sc[t], bf2f(vb[(size_t)t * HD + e]), acc);
    part[g][e] = acc;
    __syncthreads();
    if (tid < HD) {
      float o = 0.f;
      for (int k = 0; k < KG; ++k) o += part[k][tid];
      o /= l;
      a.st_o[pos * Nq + (size_t)h * HD + tid] = o;
      a.o_all[pos * Nq + (size_t)h * HD + tid] = f2bf(o);
    }
    if (tid == 0) {
      a.st_m[pr] = m;
      a.st_l[pr] = l;
    }
    __syncthreads();  // qs, sc and part are rewritten for the next pair
  }
}

// DyLLM (French summary page) §2.B: stable tokens reuse their previous attention weights and take
// in only the changed keys (pass 1, every position), salient tokens are recomputed exactly against
// the updated cache (pass 2, the selected rows; it overwrites what pass 1 wrote at their positions);
// the stable tokens whose update pass 1 declined are recomputed exactly (pass 3).
hipError_t launch_salient_attn(const ProjShape& s, float scale, const void* q_sel, void* q_all,
                               const void* k_cache, const void* v_cache, const void* k_old,
                               const void* v_old, const int32_t* sel_idx, const int32_t* row_ptr,
                               int q_first, float* st_m, float* st_l, float* st_o, void* o_sel,
                               void* o_all, void* ws, hipStream_t st) {
  AttnArgs d{};
  d.kc = (const uint16_t*)k_cache; d.vc = (const uint16_t*)v_cache;
  d.row_ptr = row_ptr;
  d.B = s.B; d.S = s.S; d.H = s.H; d.Hkv = s.Hkv; d.m_cap = s.m_cap;
  d.nsplit = 1; d.kps = s.S;
  d.scale_log2 = scale * kLog2e;
  d.sel_idx = sel_idx; d.st_m = st_m; d.st_l = st_l; d.st_o = st_o;
  d.o_all = (uint16_t*)o_all; d.q_all = (uint16_t*)q_all;
  d.k_old = (const uint16_t*)k_old; d.v_old = (const uint16_t*)v_old;
  d.q_first = q_first;
  if (q_first > 0) {
    const size_t total = (size_t)s.B * q_first * (s.H * s.hd / 4);
    hipLaunchKernelGGL(state_context_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, st_o, (uint16_t*)o_all, s.S, q_first, s.H * s.hd, total);
  }
  const int G = s.H / s.Hkv;
  const long rows = (long)(s.S - q_first) * G;
  // eight waves (256 query rows) when that still gives a workgroup per CU, else four
  const int nw = (long)s.B * s.Hkv * cdiv(rows, 256) >= 256 ? 8 : 4;
  dim3 grid(s.B * s.Hkv, cdiv(rows, 32 * nw));
  if (rows == 0) {
    // every position before q_first: no stable-token pass
  } else if (s.hd == 64) {
    if (nw == 8) hipLaunchKernelGGL((attn_bf16_kernel<64, 8, 4, true>), grid, dim3(512), 0, st, d);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, 4, 4, true>), grid, dim3(256), 0, st, d);
  } else {
    if (nw == 8) hipLaunchKernelGGL((attn_bf16_kernel<128, 8, 4, true>), grid, dim3(512), 0, st, d);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, 4, 4, true>), grid, dim3(256), 0, st, d);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.m_cap > 0) {
    e = launch_exact_bf16(s, scale, q_sel, k_cache, v_cache, row_ptr, o_sel, ws, d, st);
    if (e != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  const dim3 rg(cdiv((long)s.B * s.S * s.H, 256));
  if (s.hd == 64)
    hipLaunchKernelGGL(stable_recompute_kernel<64>, rg, dim3(256), 0, st, d);
  else
    hipLaunchKernelGGL(stable_recompute_kernel<128>, rg, dim3(256), 0, st, d);
  return hipGetLastError();
}

// copies of the K/V rows at the selected positions: rows[j, hk, :] = cache[b, hk, s, :]
__global__ __launch_bounds__(256) void gather_kv_rows_kernel(const uint4* kc, const uint4* vc,
                                                             const int32_t* sel_idx,
                                                             const int32_t* row_ptr, uint4* kr,
                                                             uint4* vr, int B, int S, int Hkv,
                                                             int m_cap, int chunks) {
  const int M = min(row_ptr[B], m_cap);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;  // one 16-byte chunk of K and of V
  const size_t per_row = (size_t)Hkv * chunks;
  const int j = (int)(idx / per_row);
  if (j >= M) return;
  const int rest = (int)(idx - (size_t)j * per_row);
  const int hk = rest / chunks, c = rest - hk * chunks;
  const int id = sel_idx[j];
  const int b = id / S, sp = id - b * S;
  const size_t src = (((size_t)b * Hkv + hk) * S + sp) * chunks + c;
  kr[idx] = kc[src];
  vr[idx] = vc[src];
}

hipError_t launch_gather_kv_rows(const ProjShape& s, size_t elem, const void* k_cache,
                                 const void* v_cache, const int32_t* sel_idx,
                                 const int32_t* row_ptr, void* k_rows, void* v_rows,
                                 hipStream_t st) {
  if (s.m_cap == 0) return hipSuccess;
  const int chunks = (int)(s.hd * elem / 16);
  const size_t threads = (size_t)s.m_cap * s.Hkv * chunks;
  hipLaunchKernelGGL(gather_kv_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, (const uint4*)k_cache, (const uint4*)v_cache, sel_idx, row_ptr,
                     (uint4*)k_rows, (uint4*)v_rows, s.B, s.S, s.Hkv, s.m_cap, chunks);
  return hipGetLastError();
}

// compact copies of whole rows: dst[j, :] = src[sel_idx[j], :] (16-byte chunks per row)
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* src, const int32_t* sel_idx,
                                                          const int32_t* row_ptr, uint4* dst,
                                                          int B, int m_cap, int chunks) {
  const int M = min(row_ptr[B], m_cap);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int j = (int)(idx / chunks);
  if (j >= M) return;
  const int c = (int)(idx - (size_t)j * chunks);
  dst[idx] = src[(size_t)sel_idx[j] * chunks + c];
}

hipError_t launch_gather_rows(int B, int m_cap, size_t row_bytes, const void* src,
                              const int32_t* sel_idx, const int32_t* row_ptr, void* dst,
                              hipStream_t st) {
  if (m_cap == 0) return hipSuccess;
  const int chunks = (int)(row_bytes / 16);
  const size_t threads = (size_t)m_cap * chunks;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, (const uint4*)src, sel_idx, row_ptr, (uint4*)dst, B, m_cap, chunks);
  return hipGetLastError();
}

}  // namespace dllm
