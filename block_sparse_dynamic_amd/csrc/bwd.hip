// Backward kernels of dynamic-mask attention for gfx950.
//
// Gradients for query, key, value and bias (Flash-DMA README: complete
// gradient path including the bias gradient, computed inside the backward
// kernels; the backward reuses the forward's block decisions).  With
// P = softmax of the valid scores (recomputed from the saved log-sum-exp),
//   D_i = sum_c dO_ic O_ic,   dP = dO V^T,   dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
//   dBias[g] = sum over the query heads of group g of dS.
//
// Kernels:
//   bwd_pre_kernel    row terms -D = -rowsum(dO * O) and -lse log2(e).
//   kt_kernel         K transposed ([b, g, d, keys]), the A operand of the dQ products.
//   pair_base_kernel  offsets of each query block's dS tiles (live 128-key pairs before it).
//   bwd_main_kernel   one workgroup per (batch, kv head g, 128 keys = two
//                     classification blocks); four wavefronts own 32 keys each.
//                     Work items are (query block, 32-row half, two heads; one
//                     head when the group size is odd), heads innermost: the
//                     item's loads, its barrier and its control run once for
//                     both heads.
//                     K and V of the keys sit in registers for the whole kernel
//                     and dK/dV accumulate in registers over every non-SKIP query
//                     block and every head of the group, so they are written
//                     once, without atomics.  Per query block and 32-row half the
//                     initial S values (bias / scale where valid, -inf elsewhere)
//                     are formed once and serve all G heads; dBias of the rows is
//                     summed over the heads in registers and stored once.  SKIP
//                     blocks get zeros and no loads.  The Q/dO tiles (and the
//                     bias/mask rows of a new query block) of the next item are
//                     loaded straight into LDS while the current item computes.
//                     Each item's dS (bf16) goes to the workspace in the order the
//                     dQ kernel consumes it, nonzero 16-byte chunks only.
//   dq_kernel         dQ = scale dS K: one workgroup per (batch, g, 64-row query block,
//                     heads), summing over the live key pairs in registers and
//                     writing bf16 dQ once.
//
// Why dQ is not accumulated with atomics: on this device every fp32 atomic add to global
// memory is performed at the memory side, at about 3.4e11 adds/s whatever the access
// pattern.  Adding each item's dS K into a dQ accumulator costs one add per (query, d,
// 128-key pair): 4.3e9 adds, ~12.7 ms, at L = 16384 with causal top-k, more than all the
// matrix work of the backward.  Writing dS (one bf16 per query, key and head) and reading
// it back once is plain traffic and no atomics, and dQ becomes deterministic.  Only the
// nonzero 16-byte chunks (8 keys of one query row) travel: with sparse masks most are zero
// (at top-k 1024 of 16384 keys, 60% of them), which cuts the round trip from ~17 GB to ~7 GB
// at L = 16384.
//
// MFMA: v_mfma_f32_32x32x16_bf16 for all five products.  S = Q K^T puts one key
// per lane (lane l%32) and 16 query rows per lane, which is the A-operand layout
// of the key-major products dV = P^T dO and dK = dS^T Q (the query order inside
// a k-step only has to agree between A and B); their B operands (dO, Q with the
// query index as the contraction) come from the row-major tiles through
// ds_read_b64_tr_b16.  dQ^T = K^T dS^T takes K^T rows from LDS and the stored dS
// chunks as B, so a result lane holds one query row.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace dma {

constexpr float kLog2eB = 1.4426950408889634f;
constexpr uint16_t kNegInfB = 0xFF80u;

// ---------------------------------------------------------------------------
// Row terms of the backward, in the [b, hq, lq] order the main kernel loads them:
// nd = -rowsum(dO * O) (so the dP accumulator starts at -D) and nl2 = -lse * log2(e).
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                      const float* __restrict__ lse, float* __restrict__ nd,
                                                      float* __restrict__ nl2, int64_t rows, int64_t lq, int64_t hq,
                                                      int d) {
  // rows = b * lq * hq (row index = (b*lq + i)*hq + h); d/8 lanes per row.
  const int lpr = d / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = gid / lpr;
  const int c = (int)(gid % lpr);
  float acc = 0.f;
  if (r < rows) {
    const u32x4 ow = *reinterpret_cast<const u32x4*>(o + r * d + c * 8);
    const u32x4 gw = *reinterpret_cast<const u32x4*>(dout + r * d + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(ow[e]) * bf16_lo(gw[e]) + bf16_hi(ow[e]) * bf16_hi(gw[e]);
  }
  for (int off = lpr / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, lpr);
  if (r < rows && c == 0) {
    const int64_t h = r % hq, bi = r / hq;  // bi = b*lq + i
    const int64_t bb = bi / lq, i = bi % lq;
    const int64_t dst = (bb * hq + h) * lq + i;
    nd[dst] = -acc;
    nl2[dst] = -lse[dst] * kLog2eB;
  }
}

// ---------------------------------------------------------------------------
// K^T for the dQ products: kt[(b*hkv + g)*d + c][j] = K[b, j, g, c] for j < lk, 0 up to the
// next multiple of 128 keys.  One workgroup per (b, g, 64 keys), through an LDS tile.
__global__ __launch_bounds__(256) void kt_kernel(const uint16_t* __restrict__ k, uint16_t* __restrict__ kt, int64_t lk,
                                                 int64_t hkv, int64_t ktrow, int nkb64, int d) {
  __shared__ uint16_t tile[64 * (128 + 2)];  // [key][d], odd-word row pad
  const int tr = d + 2;
  const int64_t plane = blockIdx.x / nkb64;
  const int kb = blockIdx.x % nkb64;
  const int64_t bb = plane / hkv, g = plane % hkv;
  for (int t = threadIdx.x; t < 64 * (d / 8); t += 256) {
    const int r = t / (d / 8), c = t % (d / 8);
    const int64_t key = (int64_t)kb * 64 + r;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < lk) w = *reinterpret_cast<const u32x4*>(k + ((bb * lk + key) * hkv + g) * d + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r * tr + c * 8 + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      tile[r * tr + c * 8 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < d * 8; t += 256) {  // row c of K^T: 64 keys = 8 chunks
    const int c = t / 8, j8 = t % 8;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[(j8 * 8 + 2 * e) * tr + c] | ((uint32_t)tile[(j8 * 8 + 2 * e + 1) * tr + c] << 16);
    *reinterpret_cast<u32x4*>(kt + (plane * d + c) * ktrow + (int64_t)kb * 64 + j8 * 8) = w;
  }
}

// pair_base[qb] = live key-block pairs of the query blocks before qb (the same for every
// plane); pair_base[nqb] = all of them.  One workgroup.
__global__ __launch_bounds__(1024) void pair_base_kernel(int64_t* __restrict__ pair_base, int64_t nqb, int64_t lq,
                                                         int64_t lk, int causal) {
  __shared__ int64_t wave_sum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per = (nqb + 1023) / 1024;
  const int64_t lo = min(nqb, (int64_t)tid * per), hi = min(nqb, lo + per);
  int64_t sum = 0;
  for (int64_t qb = lo; qb < hi; ++qb) sum += live_pairs(qb, lq, lk, causal);
  // exclusive scan of the 1024 thread sums: inside each wave, then over the 16 wave totals
  int64_t incl = sum;
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int64_t run = incl - sum;
  for (int w2 = 0; w2 < wave; ++w2) run += wave_sum[w2];
  if (tid == 1023) pair_base[nqb] = run + sum;
  for (int64_t qb = lo; qb < hi; ++qb) {
    pair_base[qb] = run;
    run += live_pairs(qb, lq, lk, causal);
  }
}

// Query blocks [q_lo, q_hi] that the workgroup of key pair KB and segment seg walks inside the
// launch's range [band_lo, band_hi]: all of them, or (splits = 2) one half of the pair's live
// blocks there (the first live one is the smallest qb with KB < live_pairs(qb), which only grows
// with qb).  Shared by the main kernel and the count of each workgroup's work.
__device__ inline void walk_range(int KB, int seg, int splits, int nqb, int64_t lq, int64_t lk, int causal,
                                  int band_lo, int band_hi, int& q_lo, int& q_hi) {
  q_lo = band_lo;
  q_hi = band_hi;
  if (splits > 1) {
    int lo = 0, hi = nqb;  // first live query block, found by bisection
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (KB < live_pairs(mid, lq, lk, causal)) hi = mid;
      else lo = mid + 1;
    }
    lo = max(lo, band_lo);
    const int upper = lo + (band_hi + 1 - lo) / 2;  // segment 0: [upper, band_hi], segment 1: [lo, upper)
    q_lo = seg == 0 ? upper : lo;
    q_hi = seg == 0 ? band_hi : upper - 1;
  }
}

// Work of each main-kernel workgroup of a one-pass backward: the query blocks its walk visits
// (those where one of its pair's two key blocks is not SKIP and causality leaves the pair live),
// written to counts[(plane * nkb2 + KB) * splits + seg].  One wave per (plane, pair): lanes take 64
// query blocks at a time, a ballot and its population count per segment.
__global__ __launch_bounds__(256) void pair_count_kernel(const uint8_t* __restrict__ state, int32_t* __restrict__ counts,
                                                         int64_t planes, int nqb, int nkb, int nkb2, int splits,
                                                         int64_t lq, int64_t lk, int causal) {
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wv >= planes * nkb2) return;  // whole waves
  const int KB = (int)(wv % nkb2);
  const int64_t plane = wv / nkb2;
  int q_lo = 0, q_hi = nqb - 1;
  if (splits > 1) walk_range(KB, 0, splits, nqb, lq, lk, causal, 0, nqb - 1, q_lo, q_hi);  // segment 0: [q_lo, nqb)
  int n0 = 0, n1 = 0;
  for (int base = 0; base < nqb; base += 64) {
    const int qb = base + lane;
    bool live = false;
    if (qb < nqb && KB < live_pairs(qb, lq, lk, causal)) {
      const uint8_t* row = state + (plane * nqb + qb) * nkb + 2 * KB;
      live = row[0] != kSkip || (2 * KB + 1 < nkb && row[1] != kSkip);
    }
    const uint64_t b = __ballot(live);
    const uint64_t upper = __ballot(live && qb >= q_lo);
    n0 += __popcll(upper);
    n1 += __popcll(b) - __popcll(upper);
  }
  if (lane == 0) {
    counts[(plane * nkb2 + KB) * splits] = n0;
    if (splits > 1) counts[(plane * nkb2 + KB) * splits + 1] = n1;
  }
}

// The main kernel's workgroup order: order[w] = the task (plane * nkb2 + KB) * splits + seg that
// workgroup w runs.  Workgroup w runs on XCD w % 8 as the w / 8-th of that XCD, and each CU holds
// one main-kernel workgroup at a time.  Where every plane's work falls with the key pair (the
// causal triangle with a uniform mask) the XCD-aware contiguous order (xcd_task) already pairs
// long and short walks and keeps a plane's rows in one XCD's L2.  Otherwise (document masks and
// other irregular ones) the tasks are sorted longest first and dealt to the XCDs in serpentine
// order (ranks 8k .. 8k+7 to XCDs 0..7 for even k, 7..0 for odd k), so that each CU starts the
// longest task left when it frees: a long walk no longer waits behind another on the same CU.
// One workgroup; a bitonic sort of up to kMaxOrder tasks in LDS (more tasks keep xcd_task).
constexpr int kMaxOrder = 16384;
__global__ __launch_bounds__(1024) void pair_order_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ order,
                                                          int T, int planes, int nkb2, int splits) {
  __shared__ uint32_t keys[kMaxOrder];
  const int tid = threadIdx.x;
  const int per_plane = nkb2 * splits;
  // does each plane's work fall (weakly) with the pair?
  int rising = 0;
  for (int i = tid; i < T; i += 1024) {
    const int KB = (i % per_plane) / splits, seg = i % splits;
    if (seg == 0 && KB + 1 < nkb2) {
      int a = 0, b = 0;
      for (int s2 = 0; s2 < splits; ++s2) {
        a += counts[i + s2];
        b += counts[i + splits + s2];
      }
      rising |= b > a;
    }
  }
  const bool irregular = __syncthreads_or(rising) != 0;
  if (!irregular || T > kMaxOrder) {
    for (int w = tid; w < T; w += 1024) order[w] = xcd_task(w, T, planes);
    return;
  }
  int n2 = 1;
  while (n2 < T) n2 *= 2;
  // key: (most work first) then the task index; counts are at most 2^18 query blocks
  for (int i = tid; i < n2; i += 1024)
    keys[i] = i < T ? (((uint32_t)((1 << 18) - 1 - counts[i]) << 14) | (uint32_t)i) : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= n2; k *= 2) {
    for (int j = k / 2; j > 0; j /= 2) {
      for (int i = tid; i < n2; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t x = keys[i], y = keys[l];
          const bool up = (i & k) == 0;
          if (up ? x > y : x < y) {
            keys[i] = y;
            keys[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < T; r += 1024) {
    const int k = r / 8, j = r % 8;
    const bool full_group = 8 * k + 8 <= T;
    const int x = (full_group && (k & 1)) ? 7 - j : j;  // a last, partial group keeps its order
    order[8 * k + x] = (int32_t)(keys[r] & 0x3FFFu);
  }
}

// ---------------------------------------------------------------------------
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* mask;
  const int32_t* rstart;  // column ranges (instead of the mask): key j attends rows rstart[j] <= i < rend[j]
  const int32_t* rend;
  const uint8_t* mbits;  // bit-packed PARTIAL blocks (instead of the mask)
  const uint16_t* bias;
  const uint8_t* state;
  const uint16_t* dout;
  const float* nl2;  // -lse * log2(e), fp32 [b, hq, lq]
  const float* nd;   // -D, fp32 [b, hq, lq]
  const int64_t* pair_base;
  uint16_t* ds;
  uint64_t* dsmap;
  int64_t npairs;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dbias;
  float* dkv_acc;  // fp32 dK, dV sums when the pairs are split (splits > 1) or the query blocks banded
  const int32_t* order;  // workgroup w runs task order[w] (pair_order_kernel), or null: xcd_task
  int64_t lq, lk, hq, hkv;
  // This launch covers query blocks [band_lo, band_hi] (all of them unless the backward runs in
  // bands); the dS slots hold that range's pairs only, the first of which is pair_base[band_lo] = pb_lo.
  int64_t pb_lo;
  int band_lo, band_hi;
  int G, nqb, nkb, nkb2, splits, total_wg;
  int wg_pairs;  // key pairs per plane in the grid: those live for some query block of the range
  float scale;
  int causal;
};

constexpr int kKeys = 128;  // keys per workgroup: two classification blocks
constexpr int kRows = 32;   // query rows per item (half a classification block)
constexpr int kStateChunk = 1024;  // query blocks whose states are cached in LDS at a time

constexpr int kLeadA = 2;  // S/dP operand steps read ahead of their products
constexpr int kLeadB = 3;  // dV/dK operand steps read ahead of their products
constexpr int kLeadQ = 4;  // dQ kernel: K^T operand reads ahead of their products
// An empty statement that LDS reads and writes cannot be moved across (MFMAs and other
// arithmetic still can): it fixes how far operand reads run ahead of their use.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }
constexpr int kWaves = 8;                 // waves of a backward workgroup: 16 keys each
constexpr int kThreads = kWaves * 64;
constexpr int kWKeys = kKeys / kWaves;    // keys per wave

// LDS layouts of the backward tiles.  A Q or dO tile [32 rows][D] and a raw bias or mask tile
// [32 rows][128 keys] keep the 16-byte chunk c of row r at chunk c ^ bx<chunks per row>(r),
// rows unpadded; bx depends on r % 16 only, so 16-row offsets add to a per-lane base.  The
// operand reads of this kernel are: per wave, 16 rows x one chunk per 16-lane group with the
// four groups on four chunks of the same rows (128-bit reads of the S and dP A operands), and
// 8 rows x two adjacent chunks per 32 lanes (transposing 64-bit reads).  Each XOR below is a
// linear map of the row bits chosen by timing these exact patterns on the hardware: both run at
// the rate of a contiguous read (about 4.1 and 2.9 cycles per wave instruction per CU), where the
// plain row-interleaved XORs halve the 128-bit rate.  In the timings, the 128-bit pattern was
// conflict-free exactly when the row step that flips chunk bit 0 has row bit 2 set.  Any XOR
// suits the DMA loads, which write whole rows in lane order.
template <int CPR>
__device__ __forceinline__ int bx(int r) {
  const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
  if constexpr (CPR == 16) {  // 256-byte rows (D = 128, or 128 keys)
    return (b1 ^ b2) | ((b0 ^ b2) << 1) | (b1 << 2) | ((b2 ^ b3) << 3);
  } else {  // 128-byte rows (D = 64)
    return b2 | ((b0 ^ b1 ^ b2) << 1) | ((b0 ^ b1 ^ b3) << 2);
  }
}
template <int W>  // W bf16 a row
__device__ __forceinline__ int bt_off(int row, int col) {
  return row * W + ((((col >> 3) ^ bx<W / 8>(row)) << 3) | (col & 7));
}
// The dS^T tile [128 keys][32 queries] keeps the 8-byte unit u of row r at unit u ^ 2 ((r/4)%4):
// the dS writes (16 aligned rows x units {u, u+1} per 32 lanes) and the export's transposing
// reads (4 aligned rows x all 8 units per 32 lanes) both touch 64 distinct banks.
__device__ __forceinline__ int st_off(int row, int col) {
  return (row << 5) | ((((col >> 2) ^ (((row >> 2) & 3) << 1)) << 2) | (col & 3));
}

template <int D, int HPI>
struct alignas(16) BwdSmem {  // 16-byte aligned so tile reads and writes stay single 16-byte LDS accesses
  static constexpr int kTile = kRows * D;       // Q or dO tile [row][d], bt_off<D> layout
  static constexpr int kBTile = kRows * kKeys;  // raw bias or mask tile [row][key], bt_off<128> layout
  static constexpr int kSTile = kKeys * kRows;  // dS^T [key][query], st_off layout
  // Two buffers each: the current item's and the next item's, which loads meanwhile; an item
  // covers HPI consecutive heads of the group.
  uint16_t q[2][HPI][kTile];
  uint16_t g[2][HPI][kTile];
  uint16_t b[2][kBTile];
  uint16_t m[2][kBTile];  // raw mask tile, or (bit input) the item's rows of the two blocks' bits
  uint16_t s[2][HPI][kSTile];
  float nl2[2][HPI][64];  // -lse * log2(e) of the item's rows (rows 32..63 take the out-of-range lanes of the load)
  float nd[2][HPI][64];   // -D = -rowsum(dO * O)
  // Initial values of the S accumulators in the S layout, one slot per lane: bias / scale on
  // valid pairs, -inf (signed so that scale * it is -inf) elsewhere.  Written when a query
  // block starts, read by the same lane for every head of the group.
  f32x4 beff[kWaves][2][64];   // [wave][16-row tile][lane]
  int64_t pb[kStateChunk];     // pair_base of the same query blocks (first dS tile pair of each)
  uint8_t st[2][kStateChunk];  // block states of the two key blocks for a range of query blocks
};

// Words of a raw buffer resource (the layout make_rsrc builds), uniform across the wave.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)LDS_PTR(const void, p));
}
// Loads straight into LDS (buffer_load ... lds): the wave's lane l fetches 16 (or 4) bytes at
// its offset `voff` in buffer `r` and they land at LDS byte address lds + 16 l (or + 4 l).
// Lanes whose offset is out of the buffer's range fetch nothing.  The compiler does not see
// these LDS writes, so it neither waits for them nor orders LDS reads after them: the kernel
// waits for them (vmcnt) and crosses a barrier before any wave reads the data.  Nothing else
// in these kernels uses M0.
__device__ __forceinline__ void dma_x4(u32x4 r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_x1(u32x4 r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
// Barrier after this wave's loads into LDS have landed and its LDS accesses are done.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// dBias zeros of one 64-row query block z = plane * nq + (qb - band_lo) (nq query blocks in the
// launch's range): every 128-key pair that no
// compute workgroup visits for it, i.e. a pair SKIP in both halves or one that causality leaves
// without a valid position, gets 64 rows x 128 keys of zeros (clipped to lq and lk), 16-byte
// stores, 256 bytes per row.  These workgroups follow the compute workgroups in the grid, so the
// streaming writes fill the causal tail of the compute.  `stc` is 2048 bytes of LDS that caches
// the block states of the row.
__device__ void zero_fill_dbias(const BwdParams& p, int z, uint8_t* stc) {
  const int nq = p.band_hi - p.band_lo + 1;
  const int plane = z / nq, qb = p.band_lo + z % nq, tid = threadIdx.x;
  const int64_t i0 = (int64_t)qb * kBlock;
  const uint8_t* st_row = p.state + ((int64_t)plane * p.nqb + qb) * p.nkb;
  uint16_t* base = p.dbias + (int64_t)plane * p.lq * p.lk + i0 * p.lk;
  const int npl = (int)live_pairs(qb, p.lq, p.lk, p.causal);
  const int rows = (int)min((int64_t)kBlock, p.lq - i0);
  constexpr int kChunk = 2048;  // key blocks whose states are cached at a time
  for (int kb_lo = 0; kb_lo < p.nkb; kb_lo += kChunk) {
    __syncthreads();  // every reader of the previous chunk is done
    for (int j = tid; j < kChunk; j += kThreads) stc[j] = kb_lo + j < p.nkb ? st_row[kb_lo + j] : kSkip;
    __syncthreads();
    const int KB_end = min(p.nkb2, (kb_lo + kChunk) / 2);
    for (int KB = kb_lo / 2; KB < KB_end; ++KB) {
      const bool dead = KB >= npl || (stc[2 * KB - kb_lo] == kSkip && stc[2 * KB + 1 - kb_lo] == kSkip);
      if (!dead) continue;
      for (int t2 = tid; t2 < kBlock * (kKeys / 8); t2 += kThreads) {
        const int r = t2 / (kKeys / 8), c = t2 % (kKeys / 8);
        const int64_t j = (int64_t)KB * kKeys + c * 8;
        if (r < rows && j < p.lk)
          *reinterpret_cast<u32x4*>(base + (int64_t)r * p.lk + j) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

// One workgroup per (batch, kv head, 128 keys); eight waves own 16 keys each.  The products are
// v_mfma_f32_16x16x32_bf16 (A: lane l holds row l%16 and k = (l/16)*8..+7; B: column l%16, the
// same k; C: column l%16, rows (l/16)*4..+3).  S = Q K^T and dP = dO V^T, as two 16-row tiles
// with the wave's 16 keys as columns, leave each lane one key and 8 query rows: rows 4g..4g+3 of
// both tiles (g = lane/16).  Taken with that row order as the contraction index, those 8 values
// are the A operand of dV = P^T dO and dK = dS^T Q as they stand, and the B operands (dO, Q: 8
// rows of one d column per lane) come from the row-major tiles by two transposing reads.  With
// 16 keys a wave's K, V, dK and dV take 96 registers, so two waves share a SIMD: one's vector
// and memory work fills the other's idle issue cycles.
template <int D, int MK, int HPI>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdParams p) {
  using Smem = BwdSmem<D, HPI>;
  constexpr int SR = kRows;
  constexpr int RPL = 512 / D;          // tile rows filled by one wave load (1 KB): 4 or 8
  constexpr int NLT = kRows / RPL;      // wave loads per Q (or dO) tile: 8 or 4
  constexpr int CPR = D / 8;            // 16-byte chunks per Q row
  constexpr int KS = D / 32;            // k-steps of the S and dP products
  constexpr int DT = D / 16;            // 16-wide d tiles of dK and dV
  __shared__ Smem sm;

  if ((int)blockIdx.x >= p.total_wg) {  // a zero-fill workgroup: no compute, no barrier shared with others
    zero_fill_dbias(p, (int)blockIdx.x - p.total_wg, &sm.st[0][0]);
    return;
  }
  const int w = blockIdx.x;
  const int per_plane = p.wg_pairs * p.splits;
  const int t = p.order != nullptr ? p.order[w] : xcd_task(w, p.total_wg, p.total_wg / per_plane);  // units: planes
  // low key blocks (most query blocks under causality) first; a split pair's halves next to each other
  const int plane = t / per_plane, KB = (t % per_plane) / p.splits, seg = (t % per_plane) % p.splits;
  const int kb0 = 2 * KB;
  const bool has_kb1 = kb0 + 1 < p.nkb;
  const int64_t bidx = plane / p.hkv, g = plane % p.hkv;
  // query blocks this workgroup walks
  int q_lo, q_hi;
  walk_range(KB, seg, p.splits, p.nqb, p.lq, p.lk, p.causal, p.band_lo, p.band_hi, q_lo, q_hi);
  // wave and the block states below are uniform across a wave; readfirstlane tells the compiler
  // so, which keeps the loop control and the buffer resources in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;  // a lane's key (column) and row group
  const int half = wave >> 2;                 // which 64-key classification block this wave is in
  const int key_loc = wave * kWKeys + l16;    // key of this lane inside the 128
  const int64_t key_abs = (int64_t)kb0 * kBlock + key_loc;
  const int64_t shift = p.lk - p.lq;
  const int64_t plane_off = (int64_t)plane * p.lq * p.lk;
  const bool has_mask = p.mask != nullptr;
  const float scale2 = p.scale * kLog2eB;
  const float inv_scale = 1.f / p.scale;
  const float neg_inf_s = p.scale > 0.f ? -INFINITY : INFINITY;  // scale * neg_inf_s = -inf
  const uint8_t* st_col = p.state + (int64_t)plane * p.nqb * p.nkb + kb0;  // + qb * nkb (+1)

  // Every item buffer starts as zeros, so a lane of a load that fetches nothing (rows past
  // lq, keys past lk, SKIP halves) leaves finite values behind whatever the hardware writes
  // for it: zeros, or the earlier contents of a buffer that only ever held loaded data.
  {
    constexpr int kZero = (int)(sizeof(Smem) / 16);
    u32x4* z = reinterpret_cast<u32x4*>(&sm.q[0][0][0]);
    for (int i = tid; i < kZero; i += kThreads) z[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // Is each of the two key blocks non-SKIP for some query block?  The K and V rows of a key
  // block that is SKIP everywhere are never read: they stay zero here (the dQ product runs
  // over both halves, and 0 * K must not meet whatever such rows hold).
  bool live[2];
  {
    int any0 = 0, any1 = 0;
    for (int qb = tid; qb < p.nqb; qb += kThreads) {
      any0 |= st_col[(int64_t)qb * p.nkb] != kSkip;
      if (has_kb1) any1 |= st_col[(int64_t)qb * p.nkb + 1] != kSkip;
    }
    live[0] = __syncthreads_or(any0) != 0;
    live[1] = __syncthreads_or(any1) != 0;
  }

  // range input: this lane's key attends the rows [krs, kre) (its column range, fixed for the kernel)
  int krs = 0, kre = 0;
  if constexpr (MK == kMaskRanges) {
    const int64_t j = min(key_abs, p.lk - 1);
    krs = p.rstart[(int64_t)plane * p.lk + j];
    kre = p.rend[(int64_t)plane * p.lk + j];
  }

  // this lane's key of K and V, the B operands of S = Q K^T and dP = dO V^T (k-step ks: d =
  // ks*32 + g4*8 ..), held in registers for the whole kernel
  bf16x8 kreg[KS], vreg[KS];
  {
    const int64_t off = ((bidx * p.lk + key_abs) * p.hkv + g) * D + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (key_abs < p.lk && live[half]) {
        kw = *reinterpret_cast<const u32x4*>(p.k + off + ks * 32);
        vw = *reinterpret_cast<const u32x4*>(p.v + off + ks * 32);
      }
      kreg[ks] = __builtin_bit_cast(bf16x8, kw);
      vreg[ks] = __builtin_bit_cast(bf16x8, vw);
    }
  }

  // Query blocks are walked from the last to the first: the workgroups of one XCD start
  // together on the same rows, so their Q/dO reads share the XCD's L2.  The states of
  // this workgroup's two key blocks (and the query blocks' first dS tile pairs) are cached in
  // LDS a chunk of query blocks at a time, so the item loop never waits on a global load.
  int cache_lo = p.nqb;  // cached query blocks: [cache_lo, cache_lo + kStateChunk)
  auto fill_cache = [&](int qb_hi) {
    lds_barrier();  // every reader of the previous chunk is done
    const int lo = max(0, qb_hi - kStateChunk + 1);
    for (int t2 = tid; t2 < 2 * kStateChunk; t2 += kThreads) {
      const int hf = t2 / kStateChunk, j = t2 % kStateChunk, qb = lo + j;
      uint8_t v = kSkip;
      // A pair that causality leaves no valid position for this query block (KB at or past its
      // live pairs) owns no dS slot: it is SKIP whatever the bitmap says, so a bitmap classified
      // without causality cannot send a dS store past the block's slots.
      if (qb <= qb_hi && (hf == 0 || has_kb1) && KB < live_pairs(qb, p.lq, p.lk, p.causal))
        v = st_col[(int64_t)qb * p.nkb + hf];
      sm.st[hf][j] = v;
      if (hf == 0 && qb <= qb_hi) sm.pb[j] = p.pair_base[qb] - p.pb_lo;  // the range's own slot numbering
    }
    lds_barrier();
    cache_lo = lo;
  };
  // next query block with a non-SKIP half at or before `from` (the dBias zeros of the blocks
  // it passes over are written by the zero-fill workgroups)
  auto next_qb = [&](int from, uint8_t& s0, uint8_t& s1) -> int {
    for (int qb = from; qb >= q_lo; --qb) {
      if (qb < cache_lo) fill_cache(qb);
      s0 = (uint8_t)__builtin_amdgcn_readfirstlane(sm.st[0][qb - cache_lo]);
      s1 = (uint8_t)__builtin_amdgcn_readfirstlane(sm.st[1][qb - cache_lo]);
      if (s0 != kSkip || s1 != kSkip) return qb;
    }
    return -1;
  };

  // Per-lane byte offsets of the item loads.  Wave load n fills tile rows n * rows-per-load
  // onwards; lane l lands on physical chunk l % chunks-per-row of row l / chunks-per-row there
  // and fetches the logical chunk the swizzle keeps at that slot.  The item's base and the rows
  // it may read (past lq the range check returns nothing) go into the buffer resource.  Wave w
  // does wave load w of each Q and dO tile (D = 64: the first four waves).
  const bool loads_q = wave < NLT;
  uint32_t qv;
  {
    const int r = (loads_q ? wave : 0) * RPL + lane / CPR;
    const int c = (lane % CPR) ^ bx<CPR>(r);
    qv = (uint32_t)r * (uint32_t)(p.hq * D * 2) + (uint32_t)c * 16u;
  }
  // bias and mask rows: 128 keys = 16 chunks, 4 rows per wave load, one load per wave; a chunk
  // past lk is never fetched, and bh records which key block the chunk is in
  uint32_t bv;
  bool bh;
  {
    const int r = wave * 4 + lane / 16;
    const int c = (lane % 16) ^ bx<16>(r);
    bv = ((int64_t)kb0 * kBlock + c * 8 < p.lk) ? (uint32_t)r * (uint32_t)(p.lk * 2) + (uint32_t)c * 16u : kOutOfRange;
    bh = c >= 8;
  }
  const uint16_t* q_plane = p.q + (bidx * p.lq * p.hq + g * p.G) * D;     // + (i * hq + hh) * D
  const uint16_t* g_plane = p.dout + (bidx * p.lq * p.hq + g * p.G) * D;
  const float* nl2_plane = p.nl2 + (bidx * p.hq + g * p.G) * p.lq;       // + hh * lq + i
  const float* nd_plane = p.nd + (bidx * p.hq + g * p.G) * p.lq;
  const uint16_t* bias_plane = p.bias + plane_off + (int64_t)kb0 * kBlock;  // + i * lk
  const uint16_t* mask_plane = p.mask + plane_off + (int64_t)kb0 * kBlock;
  const uint32_t qrow_bytes = (uint32_t)(p.hq * D * 2);
  const uint32_t krange = (uint32_t)min((int64_t)kKeys, p.lk - (int64_t)kb0 * kBlock) * 2u;
  // bit input: this plane's bits from the workgroup's first key block on (at most 2^31 bytes: the
  // host checks nqb * nkb * 512 per plane)
  u32x4 mb_rsrc = {0u, 0u, 0u, 0u};
  if constexpr (MK == kMaskBits)
    mb_rsrc = rsrc_words(p.mbits + ((int64_t)plane * p.nqb * p.nkb + kb0) * kBitsPerBlock,
                         (uint32_t)(((int64_t)p.nqb * p.nkb - kb0) * kBitsPerBlock));

  // LDS byte addresses of the load destinations (buffer B of a tile is B tiles above buffer 0):
  // plain integers, so no generic-to-LDS pointer conversion is redone on every item
  constexpr uint32_t kTileBytes = Smem::kTile * 2, kBTileBytes = Smem::kBTile * 2;
  const uint32_t lds_q = lds_addr(&sm.q[0][0][0]), lds_g = lds_addr(&sm.g[0][0][0]), lds_b = lds_addr(&sm.b[0][0]),
                 lds_m = lds_addr(&sm.m[0][0]), lds_nl2 = lds_addr(&sm.nl2[0][0][0]), lds_nd = lds_addr(&sm.nd[0][0][0]);
  // Start the loads of an item into buffer B: Q and dO rows, the raw bias and mask rows of a
  // new query block (first head of the group only), and the row terms.
  auto issue = [&](int B, int qb, int rh, int hh, uint8_t s0, uint8_t s1) {
    const int i0 = qb * kBlock + rh * kRows;
    const int rows_left = min(kRows, (int)p.lq - i0);  // >= 1
    const int64_t item = ((int64_t)i0 * p.hq + hh) * D;
    const uint32_t qbytes = (uint32_t)(rows_left - 1) * qrow_bytes + (uint32_t)D * 2u;
    if (loads_q) {
#pragma unroll
      for (int h2 = 0; h2 < HPI; ++h2) {
        const u32x4 rq = rsrc_words(q_plane + item + h2 * D, qbytes), rg = rsrc_words(g_plane + item + h2 * D, qbytes);
        const uint32_t dst = (uint32_t)((B * HPI + h2) * kTileBytes + wave * 1024);
        dma_x4(rq, lds_q + dst, qv);
        dma_x4(rg, lds_g + dst, qv);
      }
    }
    if (hh == 0) {
      const uint32_t bbytes = (uint32_t)(rows_left - 1) * (uint32_t)p.lk * 2u + krange;
      if (p.bias != nullptr) {
        const u32x4 rb = rsrc_words(bias_plane + (int64_t)i0 * p.lk, bbytes);
        dma_x4(rb, lds_b + (uint32_t)B * kBTileBytes + (uint32_t)(wave * 1024), ((bh ? s1 : s0) != kSkip) ? bv : kOutOfRange);
      }
      if (has_mask) {
        const u32x4 rm = rsrc_words(mask_plane + (int64_t)i0 * p.lk, bbytes);
        dma_x4(rm, lds_m + (uint32_t)B * kBTileBytes + (uint32_t)(wave * 1024), ((bh ? s1 : s0) == kPartial) ? bv : kOutOfRange);
      }
      if constexpr (MK == kMaskBits) {
        // rows rh*32 .. +31 of a PARTIAL key block are 256 contiguous bytes of its bits: wave
        // 4 + hf fetches those of block hf, one dword per lane, to bytes hf*256 .. of the tile
        // (one buffer range over the plane's bits, set up once; the item picks its bytes by offset)
        const int hf = wave - 4;
        if (hf >= 0 && hf < 2 && (hf ? s1 : s0) == kPartial) {
          const uint32_t off = ((uint32_t)qb * (uint32_t)p.nkb + (uint32_t)hf) * (uint32_t)kBitsPerBlock +
                               (uint32_t)(rh * (kRows * 8)) + (uint32_t)lane * 4u;
          dma_x1(mb_rsrc, lds_m + (uint32_t)B * kBTileBytes + (uint32_t)hf * 256u, off);
        }
      }
    }
    // row terms of head hh + h2: wave 2 h2 fetches -lse log2 e, wave 2 h2 + 1 fetches -D
#pragma unroll
    for (int h2 = 0; h2 < HPI; ++h2) {
      const int64_t ridx = (int64_t)(hh + h2) * p.lq + i0;
      const uint32_t rdst = (uint32_t)((B * HPI + h2) * 256);
      if (wave == 2 * h2) dma_x1(rsrc_words(nl2_plane + ridx, (uint32_t)rows_left * 4u), lds_nl2 + rdst, (uint32_t)lane * 4u);
      if (wave == 2 * h2 + 1) dma_x1(rsrc_words(nd_plane + ridx, (uint32_t)rows_left * 4u), lds_nd + rdst, (uint32_t)lane * 4u);
    }
  };

  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x4{};
    dv[dt] = f32x4{};
  }
  f32x4 dbacc[2] = {f32x4{}, f32x4{}};

  // Per-lane LDS element offsets.  S / dP A operands: row t*16 + l16, d = ks*32 + g4*8 (chunk
  // 4 ks + g4 of the row).  dV / dK B operands: transposing reads, lane s of a 16-lane group at
  // row 4 g4 + s/4 (+16), columns dt*16 + 4 (s%4): lane l16 receives rows 4 g4 .. +3 of column
  // dt*16 + l16.  Raw bias / mask tiles (init values): transposing reads at row t*16 + 4 g4 +
  // l16/4, key column wave*16 + 4 (l16%4): this lane's key, rows t*16 + 4 g4 .. +3.  dS^T tile
  // writes: the lane's key row, query columns 4 g4 and 16 + 4 g4 (8 bytes each).
  // The swizzles depend on the row modulo 16, so the second 16-row tile is the first's offsets
  // plus 16 rows: a compile-time constant that the LDS instructions take as an immediate.
  int aoff0[KS], troff0[DT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aoff0[ks] = bt_off<D>(l16, ks * 32 + g4 * 8);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) troff0[dt] = bt_off<D>(4 * g4 + (l16 >> 2), dt * 16 + 4 * (l16 & 3));
  const int boff0 = bt_off<kKeys>(4 * g4 + (l16 >> 2), wave * kWKeys + 4 * (l16 & 3));
  const int swoff0 = st_off(key_loc, 4 * g4), swoff1 = st_off(key_loc, 16 + 4 * g4);
  // dS export: wave w exports k-step w of the dQ kernel's B operand (keys w*16 + (l/32)*8 .. +7
  // of query row l%32), read from the dS^T tile by two transposing reads
  const int trow = (lane & 15) >> 2;
  const int tcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const int hi32 = lane >> 5;
  const int sq0 = st_off((wave & 1) * 16 + hi32 * 8 + trow, tcol) + (wave >> 1) * 32 * SR;
  const int sq1 = st_off((wave & 1) * 16 + hi32 * 8 + trow + 4, tcol) + (wave >> 1) * 32 * SR;

  // Item pipeline: the loads of item n+1 go straight into the other buffer while item n
  // computes.  One barrier per item, after the dS^T tile is written: every wave has waited for
  // its own loads of item n+1 before it, and has finished reading item n's buffers, so the
  // loads of item n+2 may start after it.  The dS^T tile alternates as well, so its export
  // after the barrier does not race the next item's writes.
  uint8_t cs0, cs1;  // states of the current item's two key blocks
  // Wait here for every load so far (K, V rows): the compiler then knows they are complete.
  // Otherwise it waits for them (vmcnt) at their first use inside the loop on every item,
  // which would also wait for the item loads issued there.
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();     // buffers zeroed
  int qb = next_qb(q_hi, cs0, cs1);  // -1 when every block of the two key blocks is SKIP
  const bool walked = qb >= 0;       // dK and dV are not all zero
  int rh = 0, hh = 0;
  if (qb >= 0) issue(0, qb, 0, 0, cs0, cs1);
  // first dS tile pair of the current query block, kept as read from LDS (uniform): the next
  // block's value is read when the walk reaches it and taken into scalars one item later
  int64_t pbv = qb >= 0 ? sm.pb[qb - cache_lo] : 0;
  dma_barrier();

  // ---- dS of an item to the workspace: its nonzero chunks only, in dQ-kernel order ----------
  // 16-byte chunk c of a slot holds keys (c/64)*16 + ((c/32)%2)*8 .. +7 of query row c%32.
  // Wave w owns the 64 chunks of k-step w (lane l: chunk w*64 + l) and packs its nonzero ones,
  // in lane order, at the start of the slot's w-th 1 KiB; its 64-bit ballot (which lanes stored
  // one) is the slot's mask w.  dS is zero wherever P is (masked, SKIP or non-causal keys), so
  // with sparse masks most chunks are zero.  A chunk of zeros (either sign) is read back as +0,
  // which leaves every dQ sum unchanged.  One buffer range per item over its heads' slots (head
  // h2 of the item is 2 slots further: the two 32-row halves interleave).  A negative slot (no
  // item yet) gets empty ranges, which drop every store.
  auto export_ds = [&](int Bx, int64_t slot) {
    const bool ok = slot >= 0;
    const int64_t sl = ok ? slot : 0;
    const __amdgpu_buffer_rsrc_t rds =
        make_rsrc(p.ds + sl * (kRows * kKeys), ok ? (uint32_t)((2 * HPI - 1) * kRows * kKeys * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rmp = make_rsrc(p.dsmap + sl * 8, ok ? (uint32_t)((2 * HPI - 1) * 8 * 8) : 0u);
#pragma unroll
    for (int h2 = 0; h2 < HPI; ++h2) {
      const bf16x8 ch = join_bf16x8(lds_read_tr16(&sm.s[Bx][h2][sq0]), lds_read_tr16(&sm.s[Bx][h2][sq1]));
      const u32x4 wv = __builtin_bit_cast(u32x4, ch);
      const bool nz = ((wv[0] | wv[1] | wv[2] | wv[3]) & 0x7FFF7FFFu) != 0u;
      const uint64_t m0 = __ballot(nz);
      const uint32_t r0 = __builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m0, 0u));
      // no branches: a chunk that is not stored, and the mask stores of lanes past 0, take
      // offsets past the buffer range, which drops them
      const uint32_t seg = (uint32_t)(h2 * 2 * kRows * kKeys * 2 + wave * (64 * 16));
      __builtin_amdgcn_raw_buffer_store_b128(wv, rds, nz ? seg + r0 * 16u : kOutOfRange, 0, 0);
      u32x2 mv;
      mv[0] = (uint32_t)m0;
      mv[1] = (uint32_t)(m0 >> 32);
      __builtin_amdgcn_raw_buffer_store_b64(mv, rmp, lane == 0 ? (uint32_t)(h2 * 16 + wave) * 8u : kOutOfRange, 0, 0);
    }
  };
  // ---- dBias of an item's rows, summed over the group (`bytes` = 0 when the item stores none) --
  // Rows at or past the item's last row fall outside the range; a lane whose key is past lk
  // takes an offset beyond it, so its stores are dropped as well.
  auto store_dbias = [&](const f32x4* db, int i0x, uint32_t bytes) {
    const uint32_t rb = (uint32_t)p.lk * 2u;
    // integer address arithmetic: dbias may be null (then bytes is 0 and nothing is stored)
    const uintptr_t base = (uintptr_t)p.dbias + (uintptr_t)((plane_off + (int64_t)i0x * p.lk + (int64_t)kb0 * kBlock) * 2);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(reinterpret_cast<void*>(base), bytes);
    const uint32_t lane_off = (key_abs < p.lk) ? (uint32_t)(4 * g4) * rb + (uint32_t)key_loc * 2u : kOutOfRange;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(db[tt][e]), r, lane_off + (uint32_t)(tt * 16 + e) * rb, 0, 0);
  };
  // the previous item, whose stores run inside the current one
  int64_t prev_slot = -1;
  uint32_t prev_db_bytes = 0;
  int prev_i0 = 0;
  f32x4 dbprev[2] = {f32x4{}, f32x4{}};

  int buf = 0;
  while (qb >= 0) {
    const int B = buf;
    const int i0 = qb * kBlock + rh * kRows;
    const int rows_left = min(kRows, (int)p.lq - i0);
    const uint8_t my_st = half ? cs1 : cs0;
    const int64_t pbc = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)pbv)) |
                                  ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)pbv >> 32)) << 32));

    // ---- start loading the next item ------------------------------------------------
    int nqb = qb, nrh = rh, nhh = hh + HPI;
    uint8_t ns0 = cs0, ns1 = cs1;
    if (nhh == p.G) {
      nhh = 0;
      nrh = rh + 1;
      if (nrh == 2 || i0 + kRows >= p.lq) {
        nrh = 0;
        nqb = next_qb(qb - 1, ns0, ns1);
        if (nqb >= 0) pbv = sm.pb[nqb - cache_lo];  // the walk leaves nqb in the cache
      }
    }
    if (nqb >= 0) issue(B ^ 1, nqb, nrh, nhh, ns0, ns1);

    f32x4 ivr[2];  // the item's initial S values (head 0 takes them from registers)
    if (hh == 0) {
      // S-layout initial values from the raw tiles: this lane's key and rows t*16 + 4 g4 + e of
      // the item.  A pair is valid when it is in range, in causal order, and its block is FULL, or
      // PARTIAL with a non-zero mask (none given: every pair).  Causality is applied on FULL
      // blocks too, as the forward does: a bitmap classified without it may mark a diagonal
      // block FULL.  Tiles that were not loaded read as zeros, and a zero bias is no bias.
      const bool key_ok = my_st != kSkip && key_abs < p.lk;
      const bool partial = my_st == kPartial;
      // causal: row r of the item is valid for this key when r >= key - (lk - lq) - i0
      const int64_t cfirst = p.causal ? key_abs - shift - i0 : (int64_t)INT32_MIN;
      const int first_r = (int)max((int64_t)0, min(cfirst, (int64_t)kRows));
      // rows [lo, up) are in range and causal for this lane's key
      const int lo = first_r, up = key_ok ? rows_left : 0;
      const uint32_t below_up = up >= 32 ? 0xFFFFFFFFu : (1u << up) - 1u;
      const uint32_t below_lo = lo >= 32 ? 0xFFFFFFFFu : (1u << lo) - 1u;
      const uint32_t rv = below_up & ~below_lo;  // bit r: item row r
      // bit input: row r's bits of this lane's key are bit (key % 32) of dword r*2 + key/32 of its block
      const int kbit = (wave & 3) * kWKeys + l16;  // this lane's key inside its 64-key block
      const uint32_t* mrow = reinterpret_cast<const uint32_t*>(&sm.m[B][0]) + half * 64 + (kbit >> 5);
      // the mask is read on PARTIAL blocks only (uniform across the wave)
      auto init = [&](auto use_mask) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const i16x4 xb = lds_read_tr16(&sm.b[B][boff0 + tt * 16 * kKeys]);
          i16x4 xm = {0, 0, 0, 0};
          if constexpr (decltype(use_mask)::value && MK == kMaskDense) xm = lds_read_tr16(&sm.m[B][boff0 + tt * 16 * kKeys]);
          f32x4 iv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = tt * 16 + 4 * g4 + e;
            bool v = ((rv >> r) & 1u) != 0u;
            if constexpr (decltype(use_mask)::value) {
              if constexpr (MK == kMaskDense) {
                v = v && ((uint32_t)(uint16_t)xm[e] & 0x7FFFu) != 0u;
              } else if constexpr (MK == kMaskRanges) {
                v = v && krs <= i0 + r && i0 + r < kre;
              } else {
                v = v && ((mrow[r * 2] >> (kbit & 31)) & 1u) != 0;
              }
            }
            iv[e] = v ? clamp_bias(__uint_as_float((uint32_t)(uint16_t)xb[e] << 16)) * inv_scale : neg_inf_s;
          }
          sm.beff[wave][tt][lane] = iv;  // for the later items of the row half
          ivr[tt] = iv;
        }
      };
      if (partial && (MK != kMaskDense || has_mask)) init(std::true_type{});
      else init(std::false_type{});
      dbacc[0] = f32x4{};
      dbacc[1] = f32x4{};
    } else {
      ivr[0] = sm.beff[wave][0][lane];
      ivr[1] = sm.beff[wave][1][lane];
    }

    // A SKIP half runs the same straight-line code: its initial S values are -inf, so P and
    // dS are exactly zero and it adds nothing.
#pragma unroll
    for (int h2 = 0; h2 < HPI; ++h2) {
      // ---- S + bias/scale = Q K^T + init and dP - D = dO V^T - D: 32 queries x 16 keys -------
      f32x4 sacc[2], pacc[2], nl[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sacc[tt] = h2 == 0 ? ivr[tt] : sm.beff[wave][tt][lane];
        pacc[tt] = *reinterpret_cast<const f32x4*>(&sm.nd[B][h2][tt * 16 + 4 * g4]);
        nl[tt] = *reinterpret_cast<const f32x4*>(&sm.nl2[B][h2][tt * 16 + 4 * g4]);
      }
      // operand reads run kLeadA steps (one step: a Q and a dO read) ahead of their products;
      // the empty asm statements pin where each read issues, so the scheduler cannot pull
      // them back next to their use
      {
        constexpr int NA = 2 * KS;  // steps: (k-step, row tile)
        bf16x8 aq[NA], ag[NA];
        auto read_a = [&](int i) {
          aq[i] = *reinterpret_cast<const bf16x8*>(&sm.q[B][h2][aoff0[i >> 1] + (i & 1) * 16 * D]);
          ag[i] = *reinterpret_cast<const bf16x8*>(&sm.g[B][h2][aoff0[i >> 1] + (i & 1) * 16 * D]);
        };
#pragma unroll
        for (int i = 0; i < kLeadA; ++i) read_a(i);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          if (i + kLeadA < NA) read_a(i + kLeadA);
          lds_order();
          sacc[i & 1] = mfma16(aq[i], kreg[i >> 1], sacc[i & 1]);
          pacc[i & 1] = mfma16(ag[i], vreg[i >> 1], pacc[i & 1]);
        }
      }
      if (h2 == 0) {  // the previous item's stores, while this head's products run
        export_ds(B ^ 1, prev_slot);
        store_dbias(dbprev, prev_i0, prev_db_bytes);
      }
      // ---- P = exp2(scale2 * S' - lse log2 e), dS = P (dP - D) ---------------------------------
      u32x4 pw, sw;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float pv[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[tt][e], scale2, nl[tt][e]));
          ds[e] = pv[e] * pacc[tt][e];
          dbacc[tt][e] += ds[e];
        }
        pw[2 * tt] = pack_bf16x2(pv[0], pv[1]);
        pw[2 * tt + 1] = pack_bf16x2(pv[2], pv[3]);
        sw[2 * tt] = pack_bf16x2(ds[0], ds[1]);
        sw[2 * tt + 1] = pack_bf16x2(ds[2], ds[3]);
      }
      const bf16x8 ap = __builtin_bit_cast(bf16x8, pw), as = __builtin_bit_cast(bf16x8, sw);
      // ---- dV += P^T dO and dK += dS^T Q over the item's 32 rows ------------------------------
      // steps 0 .. DT-1: dV column tiles (dO operand), DT .. 2 DT-1: dK column tiles (Q operand);
      // the transposing reads run kLeadB steps ahead
      {
        bf16x8 bo[2 * DT];
        auto read_b = [&](int j) {
          const uint16_t* t = j < DT ? &sm.g[B][h2][0] : &sm.q[B][h2][0];
          const int dt = j % DT;
          bo[j] = join_bf16x8(lds_read_tr16(t + troff0[dt]), lds_read_tr16(t + troff0[dt] + 16 * D));
        };
#pragma unroll
        for (int j = 0; j < kLeadB; ++j) read_b(j);
#pragma unroll
        for (int j = 0; j < 2 * DT; ++j) {
          if (j + kLeadB < 2 * DT) read_b(j + kLeadB);
          lds_order();
          if (j < DT) dv[j] = mfma16(ap, bo[j], dv[j]);
          else dk[j - DT] = mfma16(as, bo[j], dk[j - DT]);
        }
      }
      // the dS^T tile rows of this lane's key: query columns 4 g4 .. +3 and 16 + 4 g4 .. +3
      u32x2 lo2, hi2;
      lo2[0] = sw[0];
      lo2[1] = sw[1];
      hi2[0] = sw[2];
      hi2[1] = sw[3];
      *reinterpret_cast<u32x2*>(&sm.s[B][h2][swoff0]) = lo2;
      *reinterpret_cast<u32x2*>(&sm.s[B][h2][swoff1]) = hi2;
    }
    dma_barrier();  // dS^T complete; the next item's buffers are loaded; this item's are free

    // the item's dS and (after the group's last head) dBias leave during the next item
    prev_slot = (((int64_t)plane * p.npairs + pbc + KB) * p.G + hh) * 2 + rh;
    prev_db_bytes = (hh + HPI == p.G && p.dbias != nullptr) ? (uint32_t)rows_left * ((uint32_t)p.lk * 2u) : 0u;
    prev_i0 = i0;
    dbprev[0] = dbacc[0];
    dbprev[1] = dbacc[1];
    buf ^= 1;
    qb = nqb;
    rh = nrh;
    hh = nhh;
    cs0 = ns0;
    cs1 = ns1;
  }

  if (prev_slot >= 0) {
    export_ds(buf ^ 1, prev_slot);
    store_dbias(dbprev, prev_i0, prev_db_bytes);
  }

  // ---- dK, dV: lane holds d = dt*16 + l16 for keys wave*16 + 4 g4 + e ------------------------
  // (a split pair's halves, or its parts in the bands of query blocks, add into the fp32 sums,
  // zeroed before and converted by dkv_finalize_kernel after; a workgroup that walked nothing
  // adds nothing.  Within a launch one or two workgroups add to a sum, and launches run in
  // stream order, so the sums come out the same on every run)
  if (p.dkv_acc != nullptr && !walked) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t key = (int64_t)kb0 * kBlock + wave * kWKeys + 4 * g4 + e;
    if (key < p.lk) {
      const int64_t off = ((bidx * p.lk + key) * p.hkv + g) * D + l16;
      if (p.dkv_acc != nullptr) {
        float* acc_k = p.dkv_acc;
        float* acc_v = p.dkv_acc + (p.total_wg / per_plane) / p.hkv * p.lk * p.hkv * D;  // + b lk hkv d
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          atomicAdd(acc_k + off + dt * 16, dk[dt][e] * p.scale);
          atomicAdd(acc_v + off + dt * 16, dv[dt][e]);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          p.dk[off + dt * 16] = f32_to_bf16(dk[dt][e] * p.scale);
          p.dv[off + dt * 16] = f32_to_bf16(dv[dt][e]);
        }
      }
    }
  }
}

// The dK and dV of split key pairs: zero the fp32 sums before the main kernel, convert them to
// bf16 after it (n = b lk hkv d values each; 4 per thread).
__global__ __launch_bounds__(256) void dkv_zero_kernel(float* __restrict__ acc, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) reinterpret_cast<f32x4*>(acc)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}
__global__ __launch_bounds__(256) void dkv_finalize_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dk,
                                                           uint16_t* __restrict__ dv, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const f32x4 x = reinterpret_cast<const f32x4*>(acc)[i];
  uint16_t* out = i < n4 ? dk + 4 * i : dv + 4 * (i - n4);
  u32x2 w;
  w[0] = pack_bf16x2(x[0], x[1]);
  w[1] = pack_bf16x2(x[2], x[3]);
  *reinterpret_cast<u32x2*>(out) = w;
}

// ---------------------------------------------------------------------------
// dQ = scale * sum over the live key-block pairs of dS K, without atomics.  One workgroup per
// (batch, kv head g, 64-row query block, chunk of HC query heads); wave (head, 32-row half)
// accumulates dQ^T = K^T dS^T for its 32 rows in registers:
//   A = K^T rows d (staged once per pair for all heads, swizzled 128-key rows),
//   B = the dS chunks the backward main kernel stored in fragment order (lane l reads
//       chunk ks*64 + l of its tile: query l%32, keys ks*16 + (l/32)*8 .. +7),
// so the result lane holds one query row and 4-element runs of d for the store.  Only the
// nonzero chunks are stored: chunk ks*64 + l was owned by lane l of writer wave ks%4 (half
// ks/4), and sits at that wave's quarter of the slot + its rank among the stored chunks; the
// slot's 8 chunk masks (read before the previous pair's chunks) give presence and rank, and an
// absent chunk takes an offset past the slot, which the buffer load returns as zeros.
struct DqParams {
  const uint8_t* state;
  const int64_t* pair_base;
  const uint16_t* kt;
  const uint16_t* ds;
  const uint64_t* dsmap;
  uint16_t* dq;
  int64_t lq, lk, hq, hkv, npairs, ktrow;
  int64_t pb_lo;      // first pair of the launch's query blocks (its slots are numbered from it)
  int band_lo, nbq;   // the launch's query blocks: [band_lo, band_lo + nbq)
  int G, chunks, nqb, nkb, total_wg;
  float scale;
  int causal;
};

template <int D, int HC>
__global__ __launch_bounds__(HC * 128) void dq_kernel(DqParams p) {
  constexpr int NT = HC * 128;
  constexpr int KT = D * 16 / NT;  // 16-byte chunks of the K^T tile each thread stages
  // two K^T tiles [d][128 keys] (swz128 rows), used by alternate pairs: a pair's tile is written
  // while a slower wave may still read the previous pair's, so one barrier per pair suffices
  __shared__ __attribute__((aligned(16))) uint16_t ktile[2 * D * 128];
  constexpr int kPairChunk = 2048;
  __shared__ uint8_t srow[2 * kPairChunk];  // block states of the query block's row, pairs [cache_lo, + kPairChunk)

  const int w = blockIdx.x;
  const int t = xcd_task(w, p.total_wg, p.total_wg / p.nbq);  // units: (plane, head chunk)
  const int unit = t / p.nbq;
  const int qb = p.band_lo + p.nbq - 1 - (t % p.nbq);
  const int plane = unit / p.chunks, chunk = unit % p.chunks;
  const int64_t bidx = plane / p.hkv, g = plane % p.hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int hh = chunk * HC + (wave >> 1), rh = wave & 1;
  const int64_t head = g * p.G + hh;

  const int64_t npair = live_pairs(qb, p.lq, p.lk, p.causal);
  const int64_t pbase = p.pair_base[qb] - p.pb_lo;
  const uint8_t* st_row = p.state + ((int64_t)plane * p.nqb + qb) * p.nkb;
  const uint16_t* ktp = p.kt + (int64_t)plane * D * p.ktrow;
  // the slot of pair KB for this wave: slot0 + KB * G * 2
  const int64_t slot0 = (((int64_t)plane * p.npairs + pbase) * p.G + hh) * 2 + rh;
  const int64_t slot_stride = (int64_t)p.G * 2;

  // The block states of this query block's row are cached in LDS a chunk of pairs at a time:
  // the pair walk then waits on LDS only, never on a global load that would also wait for the
  // prefetches.  The chunk always holds the pair the walk last returned.
  int64_t cache_lo = -kPairChunk;
  auto fill = [&](int64_t lo) {
    lds_barrier();  // every reader of the previous chunk is done
    for (int j = tid; j < 2 * kPairChunk; j += NT) {
      const int64_t kb = 2 * lo + j;
      srow[j] = kb < p.nkb ? st_row[kb] : kSkip;
    }
    lds_barrier();
    cache_lo = lo;
  };
  auto state = [&](int64_t kb2, int hf) -> uint8_t { return srow[2 * (kb2 - cache_lo) + hf]; };
  auto next_pair = [&](int64_t from) -> int64_t {
    for (int64_t kb2 = from; kb2 < npair; ++kb2) {
      if (kb2 >= cache_lo + kPairChunk) fill(kb2);
      if (state(kb2, 0) != kSkip || state(kb2, 1) != kSkip) return kb2;
    }
    return npair;
  };

  // The pair walk runs three pairs ahead of the products: the K^T chunks of a pair load one pair
  // before it is staged into LDS, this wave's dS chunks two pairs before their products, and the
  // pair's chunk masks three pairs before (ahead of the chunk loads of the pair before it, so
  // that waiting for them never waits for chunk loads).  The SKIP halves of a pair are taken
  // when the walk finds it.  A pair past the last is replaced by the current one: every load
  // stays unconditional and in bounds.
  struct Pair {
    int kb;
    bool d0, d1;  // halves that are SKIP
  };
  auto walk = [&](int from) -> Pair {
    Pair r;
    r.kb = from < npair ? (int)next_pair(from) : (int)npair;
    r.kb = __builtin_amdgcn_readfirstlane(r.kb);
    r.d0 = r.kb < npair && state(r.kb, 0) == kSkip;
    r.d1 = r.kb < npair && state(r.kb, 1) == kSkip;
    return r;
  };
  // a pair's 8 masks arrive as 16 words in lanes 0..15 of one register (a vector load, counted
  // in order with the chunk loads) and are taken into scalars where the chunk offsets need them
  auto load_maps = [&](int kb) -> uint32_t {
    const uint32_t* mp = reinterpret_cast<const uint32_t*>(p.dsmap + (slot0 + (int64_t)kb * slot_stride) * 8);
    return mp[lane & 15];
  };
  u32x4 pkt[KT];
  auto load_kt = [&](int kb) {
#pragma unroll
    for (int n = 0; n < KT; ++n) {
      const int task = tid + n * NT;
      const int r = task >> 4, c = task & 15;
      pkt[n] = *reinterpret_cast<const u32x4*>(ktp + (int64_t)r * p.ktrow + (int64_t)kb * 128 + c * 8);
    }
  };
  auto load_chunks = [&](int kb, uint32_t mv, bf16x8* dst) {
    uint64_t mk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      mk[i] = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mv, 2 * i) |
              ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mv, 2 * i + 1) << 32);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(const_cast<uint16_t*>(p.ds + (slot0 + (int64_t)kb * slot_stride) * (kRows * kKeys)), kRows * kKeys * 2);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint64_t m = mk[ks];
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t off = ((m >> lane) & 1u) ? ((uint32_t)ks * 64u + rank) * 16u : kOutOfRange;
      dst[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  int aoff[D / 32];  // A operand rows dt*32 + l32, keys hi*8 (+ ks*16: the XOR term is per row, so per-lane)
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) aoff[dt] = swz128(dt * 32 + l32, hi * 8);

  // Pair n's dS chunks sit in B[n % 3] and its masks in M[n % 3]; the loop is unrolled three
  // times so that the stages rotate by name: a register copy between stages would wait for the
  // loads in flight.
  bf16x8 B[3][8];
  uint32_t M[3] = {0u, 0u, 0u};
  Pair p0 = walk(0);
  Pair p1 = walk(p0.kb + 1);
  Pair p2 = walk(p1.kb + 1);
  if (p0.kb < npair) {  // the loads in the loop's order: K^T of a pair, then masks, then chunks
    M[0] = load_maps(p0.kb);
    M[1] = load_maps(p1.kb < npair ? p1.kb : p0.kb);
    load_chunks(p0.kb, M[0], B[0]);
    load_kt(p0.kb);
    M[2] = load_maps(p2.kb < npair ? p2.kb : p0.kb);
    asm volatile("" ::: "memory");
    load_chunks(p1.kb < npair ? p1.kb : p0.kb, M[1], B[1]);
    asm volatile("" ::: "memory");
  }
  int kbo = 0;  // element offset of this pair's K^T tile: 0 or D * 128, alternating
  auto step = [&](auto rc) -> bool {
    constexpr int r = decltype(rc)::value;  // n % 3
    if (p0.kb >= npair) return false;
    // a key block that is SKIP for this query block has dS = 0 and may hold any K rows (they
    // are never loaded elsewhere): its half of the tile is staged as zeros.  The tile written
    // here was last read two pairs ago, and every wave has passed the barrier of the pair
    // between after those reads.
#pragma unroll
    for (int n = 0; n < KT; ++n) {
      const int task = tid + n * NT;
      const int rr = task >> 4, c = task & 15;
      const bool dead = (c < 8) ? p0.d0 : p0.d1;
      *reinterpret_cast<u32x4*>(&ktile[kbo + swz128(rr, c * 8)]) = dead ? u32x4{0u, 0u, 0u, 0u} : pkt[n];
    }
    lds_barrier();
    const Pair p3 = walk(p2.kb + 1);
    load_kt(p1.kb < npair ? p1.kb : p0.kb);
    M[r] = load_maps(p3.kb < npair ? p3.kb : p0.kb);  // pair n + 3
    asm volatile("" ::: "memory");  // the masks of pair n + 3 load before the chunks of pair n + 2
    load_chunks(p2.kb < npair ? p2.kb : p0.kb, M[(r + 2) % 3], B[(r + 2) % 3]);
    asm volatile("" ::: "memory");  // keep the loads here: the compiler would sink them below the products
    // steps i = ks * (D/32) + dt; the K^T operand reads run kLeadQ steps ahead of their products
    // (keys ks*16 + hi*8 are 16-byte chunk 2*ks + hi; swz128 XORs the chunk index, so the k-step
    // flips bits 4..6 of the per-lane offset)
    {
      constexpr int NS = 8 * (D / 32);
      bf16x8 av[NS];
      auto read_k = [&](int i) {
        av[i] = *reinterpret_cast<const bf16x8*>(&ktile[kbo + (aoff[i % (D / 32)] ^ ((i / (D / 32)) << 4))]);
      };
#pragma unroll
      for (int i = 0; i < kLeadQ; ++i) read_k(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + kLeadQ < NS) read_k(i + kLeadQ);
        // the product's accumulator passes through the fence, so the product stays after the
        // read just issued (otherwise the scheduler moves it up next to its own read)
        asm volatile("" : "+v"(acc[i % (D / 32)])::"memory");
        acc[i % (D / 32)] = mfma32(av[i], B[r][i / (D / 32)], acc[i % (D / 32)]);
      }
    }
    p0 = p1;
    p1 = p2;
    p2 = p3;
    kbo ^= D * 128;
    return true;
  };
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{}) &&
         step(std::integral_constant<int, 2>{})) {
  }

  // ---- dQ rows qb*64 + rh*32 + l32, d = dt*32 + gi*8 + hi*4 .. +3 ------------------------
  const int64_t row = (int64_t)qb * kBlock + rh * kRows + l32;
  if (row < p.lq) {
    uint16_t* op = p.dq + ((bidx * p.lq + row) * p.hq + head) * D + hi * 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 w2;
        w2[0] = pack_bf16x2(acc[dt][gi * 4 + 0] * p.scale, acc[dt][gi * 4 + 1] * p.scale);
        w2[1] = pack_bf16x2(acc[dt][gi * 4 + 2] * p.scale, acc[dt][gi * 4 + 3] * p.scale);
        *reinterpret_cast<u32x2*>(op + dt * 32 + gi * 8) = w2;
      }
  }
}

template <int D, int HC>
static hipError_t launch_dq_t(const DqParams& q, hipStream_t stream) {
  hipLaunchKernelGGL((dq_kernel<D, HC>), dim3(q.total_wg), dim3(HC * 128), 0, stream, q);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
hipError_t launch_bwd(const AttnArgs& a, hipStream_t stream, int parts) {
  const int64_t rows = a.b * a.lq * a.hq;
  const int nqb = (int)((a.lq + kBlock - 1) / kBlock), nkb = (int)((a.lk + kBlock - 1) / kBlock);
  const int nkb2 = (nkb + 1) / 2;
  const int64_t ktrow = (int64_t)nkb2 * 128;
  if (parts & kBwdPrepare) {
    const int64_t threads = rows * (a.d / 8);
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.o, a.dout,
                       a.lse_in, a.nd, a.nl2, rows, a.lq, a.hq, (int)a.d);
    hipLaunchKernelGGL(kt_kernel, dim3((unsigned)(a.b * a.hkv * nkb2 * 2)), dim3(256), 0, stream, a.k, a.kt, a.lk,
                       a.hkv, ktrow, nkb2 * 2, (int)a.d);
    hipLaunchKernelGGL(pair_base_kernel, dim3(1), dim3(1024), 0, stream, a.pair_base, (int64_t)nqb, a.lq, a.lk,
                       a.causal);
    if (a.dkv_acc != nullptr) {
      const int64_t n4 = 2 * a.b * a.lk * a.hkv * a.d / 4;
      hipLaunchKernelGGL(dkv_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a.dkv_acc, n4);
    }
    if (a.order != nullptr) {  // one pass: the main kernel's workgroup order from the bitmap
      const int splits = a.dkv_acc != nullptr ? bwd_splits(a.b, a.hkv, a.lq, a.lk, a.causal) : 1;
      const int64_t T = a.b * a.hkv * nkb2 * splits;
      const int64_t waves = a.b * a.hkv * nkb2;  // one per (plane, pair)
      hipLaunchKernelGGL(pair_count_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a.state,
                         a.pair_counts, a.b * a.hkv, nqb, nkb, nkb2, splits, a.lq, a.lk, a.causal);
      hipLaunchKernelGGL(pair_order_kernel, dim3(1), dim3(1024), 0, stream, a.pair_counts, a.order, (int)T,
                         (int)(a.b * a.hkv), nkb2, splits);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.mask = a.mask;
  p.mbits = a.mbits;
  p.rstart = a.rstart;
  p.rend = a.rend;
  p.bias = a.bias;
  p.state = a.state;
  p.dout = a.dout;
  p.nl2 = a.nl2;
  p.nd = a.nd;
  p.pair_base = a.pair_base;
  p.ds = a.ds;
  p.dsmap = a.dsmap;
  p.npairs = a.npairs;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dbias = a.dbias;
  p.dkv_acc = a.dkv_acc;
  p.order = a.band_pairs > 0 ? nullptr : a.order;
  p.lq = a.lq;
  p.lk = a.lk;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = (int)(a.hq / a.hkv);
  p.nqb = nqb;
  p.nkb = nkb;
  p.nkb2 = nkb2;
  const bool banded = a.band_pairs > 0;
  p.splits = a.dkv_acc != nullptr && !banded ? bwd_splits(a.b, a.hkv, a.lq, a.lk, a.causal) : 1;  // banded: per band below
  p.scale = a.scale;
  p.causal = a.causal;
  const int MK = a.rstart != nullptr ? kMaskRanges : a.mbits != nullptr ? kMaskBits : kMaskDense;
  const int G = p.G;
  const int HC = G >= 4 ? 4 : G;

  // The main kernel over query blocks [lo, hi] whose dS slots start at pair pb_lo and hold
  // npairs pairs per plane: the compute workgroups (the key pairs live for some block of the
  // range), then (with a dBias output) one zero-fill workgroup per query block of the range.
  auto run_main = [&](int lo, int hi, int64_t pb_lo, int64_t npairs) -> hipError_t {
    p.band_lo = lo;
    p.band_hi = hi;
    p.pb_lo = pb_lo;
    p.npairs = npairs;
    p.wg_pairs = (int)live_pairs(hi, a.lq, a.lk, a.causal);
    // bands: the first band's dK/dV sums start at zero, so its pairs may split as the one pass's
    // do (two partial sums onto zero, the same bits in either order); later bands add onto
    // earlier sums and keep one workgroup per pair
    if (banded) p.splits = (lo == 0 && a.causal && a.b * a.hkv * p.wg_pairs <= 256 && hi + 1 >= 8) ? 2 : 1;
    p.total_wg = (int)(a.b * a.hkv * p.wg_pairs * p.splits);
    const int64_t grid = p.total_wg + (a.dbias != nullptr ? a.b * a.hkv * (int64_t)(hi - lo + 1) : 0);
    if (grid == 0) return hipSuccess;
    auto launch_main = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p); };
    // an item covers two heads when the group size is even
    auto launch_d = [&](auto dconst) {
      constexpr int D = decltype(dconst)::value;
      if (p.G % 2 == 0) {
        if (MK == kMaskRanges) launch_main(bwd_main_kernel<D, kMaskRanges, 2>);
        else if (MK == kMaskBits) launch_main(bwd_main_kernel<D, kMaskBits, 2>);
        else launch_main(bwd_main_kernel<D, kMaskDense, 2>);
      } else {
        if (MK == kMaskRanges) launch_main(bwd_main_kernel<D, kMaskRanges, 1>);
        else if (MK == kMaskBits) launch_main(bwd_main_kernel<D, kMaskBits, 1>);
        else launch_main(bwd_main_kernel<D, kMaskDense, 1>);
      }
    };
    if (a.d == 64) launch_d(std::integral_constant<int, 64>{});
    else launch_d(std::integral_constant<int, 128>{});
    return hipGetLastError();
  };
  auto run_finalize = [&]() -> hipError_t {
    if (a.dkv_acc == nullptr) return hipSuccess;
    const int64_t n4 = a.b * a.lk * a.hkv * a.d / 4;
    hipLaunchKernelGGL(dkv_finalize_kernel, dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0, stream,
                       a.dkv_acc, a.dk, a.dv, n4);
    return hipGetLastError();
  };

  DqParams q;
  q.state = a.state;
  q.pair_base = a.pair_base;
  q.kt = a.kt;
  q.ds = a.ds;
  q.dsmap = a.dsmap;
  q.dq = a.dq;
  q.lq = a.lq;
  q.lk = a.lk;
  q.hq = a.hq;
  q.hkv = a.hkv;
  q.ktrow = ktrow;
  q.G = G;
  q.chunks = G / HC;
  q.nqb = nqb;
  q.nkb = nkb;
  q.scale = a.scale;
  q.causal = a.causal;
  // The dQ kernel over query blocks [lo, hi] (slots as for run_main).
  auto run_dq = [&](int lo, int hi, int64_t pb_lo, int64_t npairs) -> hipError_t {
    q.band_lo = lo;
    q.nbq = hi - lo + 1;
    q.pb_lo = pb_lo;
    q.npairs = npairs;
    q.total_wg = (int)(a.b * a.hkv * q.chunks * q.nbq);
    if (a.d == 64) {
      if (HC == 1) return launch_dq_t<64, 1>(q, stream);
      if (HC == 2) return launch_dq_t<64, 2>(q, stream);
      return launch_dq_t<64, 4>(q, stream);
    }
    if (HC == 1) return launch_dq_t<128, 1>(q, stream);
    if (HC == 2) return launch_dq_t<128, 2>(q, stream);
    return launch_dq_t<128, 4>(q, stream);
  };

  hipError_t e = hipSuccess;
  if (!banded) {
    if (parts & kBwdMain) {
      if ((e = run_main(0, nqb - 1, 0, a.npairs)) != hipSuccess) return e;
      if ((e = run_finalize()) != hipSuccess) return e;
    }
    if (parts & kBwdDq) return run_dq(0, nqb - 1, 0, a.npairs);
    return hipSuccess;
  }
  // Bands of consecutive query blocks whose live pairs fit the dS slots (a.band_pairs per plane),
  // each taken by the main kernel and then the dQ kernel; dK and dV gather in the fp32 sums.
  int64_t pb_lo = 0;
  for (int lo = 0; lo < nqb;) {
    const int hi = (int)bwd_band_end(lo, nqb, a.lq, a.lk, a.causal, a.band_pairs) - 1;
    int64_t np = 0;
    for (int qb = lo; qb <= hi; ++qb) np += live_pairs(qb, a.lq, a.lk, a.causal);
    if ((e = run_main(lo, hi, pb_lo, np)) != hipSuccess) return e;
    if ((e = run_dq(lo, hi, pb_lo, np)) != hipSuccess) return e;
    pb_lo += np;
    lo = hi + 1;
  }
  return run_finalize();
}

}  // namespace dma
