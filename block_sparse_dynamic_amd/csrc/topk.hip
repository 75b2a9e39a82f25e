// Top-k mask construction on the GPU (Flash-DMA README, usage example: the dynamic mask keeps
// the keep_window_size largest bias values of each query row, and the bias at every other
// position is overwritten with the smallest bf16 value).
//
// One workgroup per row.  The row's bf16 bits are read once into LDS; the k-th largest value
// is found by a two-level radix select over 16-bit order-preserving keys (top 12 bits, then
// the low 4), ties at that value go to the lowest key indices (a per-thread count over contiguous
// chunks and a workgroup scan fix which tied elements are kept), and the mask and the new bias
// are written in one coalesced pass.  HBM traffic: one read of the bias, two writes.
//
// Order of values: the bf16 numbers in their numeric order, +0 and -0 equal, every NaN below
// every number (NaN never outranks a number; NaNs tie among themselves).
#include "common.h"

namespace dma {

constexpr int kTopkThreads = 256;
constexpr uint16_t kBf16Lowest = 0xFF7Fu;  // -3.3895e38, the most negative finite bf16
constexpr uint16_t kBf16One = 0x3F80u;

// Order-preserving 16-bit key of a bf16 value: larger value -> larger key.
__device__ __forceinline__ uint32_t topk_key(uint32_t x) {
  x &= 0xFFFFu;
  if ((x & 0x7FFFu) > 0x7F80u) return 0u;  // NaN: below everything
  if (x == 0x8000u) x = 0u;                // -0 ties with +0
  return (x & 0x8000u) ? (~x & 0xFFFFu) : (x | 0x8000u);
}

// Exclusive prefix sum of v over the workgroup's 256 threads (4 waves).
__device__ int block_exclusive_scan(int v, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  __syncthreads();  // wave_tot is reused by the next call
  return base + incl - v;
}

// The k-th largest key of the row, by a two-level radix select: a 4096-bin histogram of the
// top 12 key bits (the bins of bf16 values of one magnitude stay apart, so LDS atomics rarely
// collide), then a 16-bin histogram of the low 4 bits among the keys of the selected bin.
// Returns the key and sets *count_above to the number of keys above it.  Every thread calls this.
__device__ uint32_t topk_select(const uint16_t* row, int lk, int64_t k, int* hist, int* small, int* wave_tot,
                                int64_t* count_above) {
  const int tid = threadIdx.x;
  for (int j = tid; j < 4096; j += kTopkThreads) hist[j] = 0;
  if (tid < 16) small[tid] = 0;
  __syncthreads();
  for (int c = tid; c < lk / 8; c += kTopkThreads) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicAdd(&hist[topk_key(w[e >> 1] >> (16 * (e & 1))) >> 4], 1);
  }
  __syncthreads();
  // thread t owns bins 16t .. 16t+15; keys in higher bins = total - inclusive prefix
  int s16 = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) s16 += hist[tid * 16 + j];
  const int excl = block_exclusive_scan(s16, wave_tot);
  __shared__ int total, bin_sel;
  __shared__ int64_t above_sel;
  if (tid == kTopkThreads - 1) total = excl + s16;
  __syncthreads();
  int64_t run = total - (excl + s16);  // keys in bins above this thread's
  for (int j = 15; j >= 0; --j) {
    const int64_t ge = run + hist[tid * 16 + j];
    if (run < k && k <= ge) {
      bin_sel = tid * 16 + j;
      above_sel = run;
    }
    run = ge;
  }
  __syncthreads();
  const int bin = bin_sel;
  const int64_t above = above_sel;
  for (int c = tid; c < lk / 8; c += kTopkThreads) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t key = topk_key(w[e >> 1] >> (16 * (e & 1)));
      if ((int)(key >> 4) == bin) atomicAdd(&small[key & 15u], 1);
    }
  }
  __syncthreads();
  __shared__ uint32_t key_sel;
  __shared__ int64_t above_key;
  if (tid == 0) {
    int64_t r = above;
    for (int j = 15; j >= 0; --j) {
      const int64_t ge = r + small[j];
      if (r < k && k <= ge) {
        key_sel = (uint32_t)(bin * 16 + j);
        above_key = r;
      }
      r = ge;
    }
  }
  __syncthreads();
  *count_above = above_key;
  const uint32_t key = key_sel;
  __syncthreads();  // the shared results are rewritten by the next call
  return key;
}

__global__ __launch_bounds__(kTopkThreads) void topk_mask_kernel(const uint16_t* bias, int64_t rows,
                                                                   int lk, int64_t k, uint16_t* __restrict__ mask_out,
                                                                   uint16_t* bias_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t topk_smem[];
  const int lk16 = (lk + 7) / 8 * 8;
  uint16_t* row = reinterpret_cast<uint16_t*>(topk_smem);                       // lk16 bf16 bits
  uint32_t* keep_tied = reinterpret_cast<uint32_t*>(topk_smem + (size_t)lk16 * 2);  // ceil(lk/32) words
  const int nwords = (lk + 31) / 32;
  __shared__ int hist[4096], small[16], wave_tot[4];

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const uint16_t* src = bias + r * lk;

  // ---- the row into LDS (16-byte loads; lk is a multiple of 8) ---------------------------
  for (int c = tid; c < lk / 8; c += kTopkThreads)
    *reinterpret_cast<u32x4*>(row + c * 8) = *reinterpret_cast<const u32x4*>(src + c * 8);
  for (int wd = tid; wd < nwords; wd += kTopkThreads) keep_tied[wd] = 0u;
  __syncthreads();

  uint32_t thr = 0;     // key of the k-th largest value
  int64_t need = 0;     // how many keys equal to thr are kept (the lowest-indexed ones)
  const bool all = k >= (int64_t)lk;
  if (!all) {
    int64_t above = 0;
    thr = topk_select(row, lk, k, hist, small, wave_tot, &above);
    need = k - above;  // >= 1

    // ---- ties: thread t owns keys [t*C, (t+1)*C), C a multiple of 8; count, scan, keep the
    // first `need` in key order.  The count reads its chunk 16 bytes at a time starting at a
    // per-thread rotation, which spreads a wave's reads over the LDS banks.
    const int C = ((lk + kTopkThreads - 1) / kTopkThreads + 7) / 8 * 8;
    const int lo = min(lk, tid * C), hi = min(lk, lo + C);
    const int nv = (hi - lo) / 8;
    int eq = 0;
    for (int j = 0; j < nv; ++j) {
      const int v = (j + tid) % nv;
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + lo + v * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) eq += (topk_key(w[e]) == thr) + (topk_key(w[e] >> 16) == thr);
    }
    int64_t rank = block_exclusive_scan(eq, wave_tot);
    // walk the chunk in key order, 8 keys (one 16-byte read, one byte of keep_tied) at a time
    for (int v = 0; v < nv && rank < need; ++v) {
      const int i = lo + v * 8;
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + i);
      uint32_t m = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) m |= (uint32_t)(topk_key(w[e >> 1] >> (16 * (e & 1))) == thr) << e;
      uint32_t take = 0u;
      for (int e = 0; e < 8 && rank < need; ++e) {
        if ((m >> e) & 1u) {
          take |= 1u << e;
          ++rank;
        }
      }
      if (take) atomicOr(&keep_tied[i >> 5], take << (i & 31));
    }
    __syncthreads();
  }

  // ---- mask and bias out, 8 keys per thread per step -------------------------------------
  uint16_t* mdst = mask_out + r * lk;
  uint16_t* bdst = bias_out + r * lk;
  for (int c = tid; c < lk / 8; c += kTopkThreads) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + c * 8);
    const uint32_t kbits = keep_tied[c >> 2] >> ((c & 3) * 8);  // the 8 tie bits of keys c*8 ..
    u32x4 mo, bo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t m2 = 0u, b2 = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = (w[e] >> (16 * h)) & 0xFFFFu;
        const uint32_t key = topk_key(x);
        const bool kept = all || key > thr || (key == thr && ((kbits >> (2 * e + h)) & 1u));
        const bool one = all || (kept && x != kBf16Lowest);
        m2 |= (one ? (uint32_t)kBf16One : 0u) << (16 * h);
        b2 |= (one ? x : (all ? x : (uint32_t)kBf16Lowest)) << (16 * h);
      }
      mo[e] = m2;
      bo[e] = b2;
    }
    *reinterpret_cast<u32x4*>(mdst + c * 8) = mo;
    *reinterpret_cast<u32x4*>(bdst + c * 8) = bo;
  }
}

size_t topk_smem_bytes(int64_t lk) { return (size_t)(lk + 7) / 8 * 8 * 2 + (size_t)(lk + 31) / 32 * 4; }

hipError_t launch_topk(const uint16_t* bias, int64_t rows, int64_t lk, int64_t k, uint16_t* mask_out,
                       uint16_t* bias_out, hipStream_t stream) {
  const size_t smem = topk_smem_bytes(lk);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_mask_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_mask_kernel, dim3((unsigned)rows), dim3(kTopkThreads), smem, stream, bias, rows, (int)lk, k,
                     mask_out, bias_out);
  return hipGetLastError();
}

}  // namespace dma
