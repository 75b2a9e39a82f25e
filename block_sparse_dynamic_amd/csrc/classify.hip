// Block classification pass (Flash-DMA README, key design: OR-reduction of each
// mask block, one decision for forward and backward; FlashMask README, Key
// Features: fully masked / partially masked / unmasked blocks).
//
// One wavefront classifies one 64 x 64 block: each lane streams 8 rows x 16
// bytes of the block (row it*8 + lane/8, columns (lane%8)*8 .. +7), so a wave
// instruction covers 8 whole 128-byte rows.  any/all over the wave come from
// ballots, so no LDS and no barrier is needed.  Blocks wholly above the causal
// diagonal are written SKIP without reading the mask; without a mask the class
// follows from geometry alone.
#include "common.h"

namespace dma {

__global__ __launch_bounds__(256) void classify_kernel(const uint16_t* __restrict__ mask, int64_t lq, int64_t lk,
                                                        int nqb, int nkb, int causal, uint8_t* __restrict__ state,
                                                        uint8_t* __restrict__ mbits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = blockIdx.x * 4 + wave;
  const int qb = blockIdx.y;
  const int64_t plane = blockIdx.z;
  if (kb >= nkb) return;
  const int64_t i0 = (int64_t)qb * kBlock, j0 = (int64_t)kb * kBlock;
  const int64_t i_end = min(i0 + kBlock, lq), j_end = min(j0 + kBlock, lk);
  const int64_t shift = lk - lq;  // key j is visible from query i iff j <= i + shift
  uint8_t* out = state + ((plane * nqb + qb) * (int64_t)nkb + kb);
  const bool ragged = (i0 + kBlock > lq) || (j0 + kBlock > lk);
  if (causal && j0 > i_end - 1 + shift) {  // every element excluded by causality
    if (lane == 0) *out = kSkip;
    return;
  }
  const bool diag = causal && (j_end - 1 > i0 + shift);  // some element excluded by causality
  if (mask == nullptr) {
    if (lane == 0) *out = (ragged || diag) ? kPartial : kFull;
    return;
  }
  bool any = false, all = true;
  const int64_t j = j0 + (lane & 7) * 8;
  uint32_t bytes[2] = {0u, 0u};  // the mask bits of this lane's 8 columns in its 8 rows, one byte per row
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int64_t i = i0 + it * 8 + (lane >> 3);
    if (i < lq && j < lk) {  // lk % 8 == 0: the 8 columns are all inside the row
      const u32x4 w = *reinterpret_cast<const u32x4*>(mask + ((plane * lq + i) * lk + j));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool a0 = attends_lo(w[e]), a1 = attends_hi(w[e]);
        bytes[it >> 2] |= ((uint32_t)a0 << (2 * e) | (uint32_t)a1 << (2 * e + 1)) << (8 * (it & 3));
        if (diag) {
          a0 = a0 && (j + 2 * e <= i + shift);
          a1 = a1 && (j + 2 * e + 1 <= i + shift);
        }
        any = any || a0 || a1;
        all = all && a0 && a1;
      }
    } else {
      all = false;
    }
  }
  const bool block_any = __any(any);
  const bool block_all = __all(all);
  if (lane == 0) *out = block_any ? (block_all ? kFull : kPartial) : kSkip;
  // Bit-packed PARTIAL blocks (the only ones whose mask the attention kernels read): row r of
  // the block is the 64-bit word at bytes 8r .. 8r+7, bit c = mask of column c (causality not
  // applied); this lane owns byte lane%8 of rows it*8 + lane/8.
  if (mbits != nullptr && block_any && !block_all) {
    uint8_t* dst = mbits + ((plane * nqb + qb) * (int64_t)nkb + kb) * kBitsPerBlock + (lane >> 3) * 8 + (lane & 7);
#pragma unroll
    for (int it = 0; it < 8; ++it) dst[it * 64] = (uint8_t)(bytes[it >> 2] >> (8 * (it & 3)));
  }
}

// The same classes from column ranges (FlashMask README, column-wise sparse representation):
// key column j attends rows start_row[j] <= i < end_row[j].  One wavefront per block, lane c
// on column j0 + c: the rows of its column that are valid inside the block form one interval,
// so "any" and "all" of the block follow from 64 intervals and two ballots, without reading
// any mask.
__global__ __launch_bounds__(256) void classify_ranges_kernel(const int32_t* __restrict__ rstart,
                                                               const int32_t* __restrict__ rend, int64_t lq,
                                                               int64_t lk, int nqb, int nkb, int causal,
                                                               uint8_t* __restrict__ state) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = blockIdx.x * 4 + wave;
  const int qb = blockIdx.y;
  const int64_t plane = blockIdx.z;
  if (kb >= nkb) return;
  const int64_t i0 = (int64_t)qb * kBlock, j0 = (int64_t)kb * kBlock;
  const int64_t i_end = min(i0 + kBlock, lq);
  const int64_t shift = lk - lq;
  uint8_t* out = state + ((plane * nqb + qb) * (int64_t)nkb + kb);
  if (causal && j0 > i_end - 1 + shift) {
    if (lane == 0) *out = kSkip;
    return;
  }
  const int64_t j = j0 + lane;
  bool any = false, all = false;
  if (j < lk) {
    int64_t lo = max((int64_t)rstart[plane * lk + j], i0);
    const int64_t hi = min((int64_t)rend[plane * lk + j], i_end);
    if (causal) lo = max(lo, j - shift);
    any = lo < hi;
    all = lo == i0 && hi == i0 + kBlock;  // every one of the block's 64 rows exists and is valid
  }
  const bool block_any = __any(any);
  const bool block_all = __all(all);
  if (lane == 0) *out = block_any ? (block_all ? kFull : kPartial) : kSkip;
}

hipError_t launch_classify_ranges(const int32_t* rstart, const int32_t* rend, int64_t b, int64_t hkv, int64_t lq,
                                  int64_t lk, int causal, uint8_t* state, hipStream_t stream) {
  const int nqb = (int)((lq + kBlock - 1) / kBlock), nkb = (int)((lk + kBlock - 1) / kBlock);
  dim3 grid((nkb + 3) / 4, nqb, (unsigned)(b * hkv));
  hipLaunchKernelGGL(classify_ranges_kernel, grid, dim3(256), 0, stream, rstart, rend, lq, lk, nqb, nkb, causal, state);
  return hipGetLastError();
}

hipError_t launch_classify(const uint16_t* mask, int64_t b, int64_t hkv, int64_t lq, int64_t lk, int causal,
                           uint8_t* state, uint8_t* mbits, hipStream_t stream) {
  const int nqb = (int)((lq + kBlock - 1) / kBlock), nkb = (int)((lk + kBlock - 1) / kBlock);
  dim3 grid((nkb + 3) / 4, nqb, (unsigned)(b * hkv));
  hipLaunchKernelGGL(classify_kernel, grid, dim3(256), 0, stream, mask, lq, lk, nqb, nkb, causal, state, mbits);
  return hipGetLastError();
}

}  // namespace dma
