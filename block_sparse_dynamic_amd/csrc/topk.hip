// Top-k mask construction on the GPU (Flash-DMA README, usage example: the dynamic mask keeps
// the keep_window_size largest bias values of each query row, and the bias at every other
// position is overwritten with the smallest bf16 value).
//
// One workgroup per row.  The row's bf16 bits are read once into registers (thread t holds the
// 16-byte chunks t, t + 256, ...); the k-th largest value is found by a two-level radix select
// over 16-bit order-preserving keys (top 12 bits, then the low 4).  Ties at that value go to the
// lowest key indices: the second level also counts the keys of each low-4 value per row of 256
// chunks, which names the chunk row holding the last kept tie; a scan over that row's chunks
// finds its index P, and a tied key is kept when its index is below P.  The mask and the new
// bias are written in one coalesced pass that compares fp32 values with the threshold.  HBM
// traffic: one read of the bias, two writes.  LDS holds only the histograms, so many rows are
// in flight on a CU and their selection overlaps the others' loads and stores.
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

// The row as registers: thread t holds chunks t + 256 m (m < CH) of 8 keys each; a chunk past
// the row's end (c >= nch) takes part in nothing.  "Row" m of chunks is chunks 256 m .. 256 m + 255,
// the m-th chunk of every thread, so index order within it is thread order.
template <int CH>
struct TopkRow {
  u32x4 v[CH];
};

// The k-th largest key of the row, by a two-level radix select: a 4096-bin histogram of the
// top 12 key bits (LDS atomics), then a 16-bin histogram of the low 4 bits among the keys of the
// selected bin.  The second level also counts, for each chunk row m and low-4 value j, the keys
// of the selected bin in that row: rowcnt[m * 16 + j].  Returns the key and sets *count_above to
// the number of keys above it.  Every thread calls this.
template <int CH>
__device__ uint32_t topk_select(const TopkRow<CH>& rw, int nch, int64_t k, int* hist, int* small, int* rowcnt,
                                int* wave_tot, int64_t* count_above) {
  const int tid = threadIdx.x;
  for (int j = tid; j < 4096; j += kTopkThreads) hist[j] = 0;
  if (tid < 16) small[tid] = 0;
  for (int j = tid; j < CH * 16; j += kTopkThreads) rowcnt[j] = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < CH; ++m) {
    if (tid + m * kTopkThreads < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) atomicAdd(&hist[topk_key(rw.v[m][e >> 1] >> (16 * (e & 1))) >> 4], 1);
    }
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
#pragma unroll
  for (int m = 0; m < CH; ++m) {
    if (tid + m * kTopkThreads < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t key = topk_key(rw.v[m][e >> 1] >> (16 * (e & 1)));
        if ((int)(key >> 4) == bin) {
          atomicAdd(&small[key & 15u], 1);
          atomicAdd(&rowcnt[m * 16 + (int)(key & 15u)], 1);
        }
      }
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
  return key_sel;
}

template <int CH>
__global__ __launch_bounds__(kTopkThreads) void topk_mask_kernel(const uint16_t* bias, int lk, int64_t k,
                                                                   uint16_t* __restrict__ mask_out, uint16_t* bias_out) {
  __shared__ int hist[4096], small[16], rowcnt[CH * 16], wave_tot[4];
  __shared__ int cut_sh;

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const uint16_t* src = bias + r * lk;
  const int nch = lk / 8;  // 16-byte chunks of the row (lk is a multiple of 8)

  // ---- the row into registers (16-byte loads, consecutive threads on consecutive chunks) ----
  TopkRow<CH> rw;
#pragma unroll
  for (int m = 0; m < CH; ++m) {
    const int c = tid + m * kTopkThreads;
    rw.v[m] = c < nch ? *reinterpret_cast<const u32x4*>(src + c * 8) : u32x4{0u, 0u, 0u, 0u};
  }

  uint16_t* mdst = mask_out + r * lk;
  uint16_t* bdst = bias_out + r * lk;
  if (k >= (int64_t)lk) {  // everything kept: mask 1, bias unchanged
#pragma unroll
    for (int m = 0; m < CH; ++m) {
      const int c = tid + m * kTopkThreads;
      if (c < nch) {
        *reinterpret_cast<u32x4*>(mdst + c * 8) = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        *reinterpret_cast<u32x4*>(bdst + c * 8) = rw.v[m];
      }
    }
    return;
  }

  int64_t above = 0;
  const uint32_t thr = topk_select<CH>(rw, nch, k, hist, small, rowcnt, wave_tot, &above);  // the k-th largest key
  const int64_t need = k - above;  // keys equal to thr that are kept (the lowest-indexed ones), >= 1

  // ---- the cut P: a key equal to thr is kept iff its index is below P ---------------------
  // The chunk row holding the need-th tie, from the per-row counts; then a scan of the ties in
  // that row's chunks (one chunk per thread, in index order) finds the chunk and the key.
  int m_cut = 0;
  int64_t left = need;  // the row counts of thr add up to at least need
  for (; m_cut + 1 < CH; ++m_cut) {
    const int cnt = rowcnt[m_cut * 16 + (int)(thr & 15u)];
    if (left <= cnt) break;
    left -= cnt;
  }
  {
    const int c = m_cut * kTopkThreads + tid;
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < CH; ++m)
      if (m == m_cut) w = rw.v[m];
    uint32_t tie = 0u;  // bit e: key c*8 + e equals thr
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) tie |= (uint32_t)(topk_key(w[e >> 1] >> (16 * (e & 1))) == thr) << e;
    }
    const int n = __builtin_popcount(tie);
    const int rank = block_exclusive_scan(n, wave_tot);
    if (rank < left && left <= rank + n) {
      int seen = rank;
      for (int e = 0; e < 8; ++e) {
        if ((tie >> e) & 1u) {
          if (++seen == left) cut_sh = c * 8 + e + 1;
        }
      }
    }
    __syncthreads();
  }
  const int cut = cut_sh;

  // ---- mask and bias out -------------------------------------------------------------------
  // A key is kept when it is above thr, or equal to it with an index below the cut; a kept key
  // whose value is the smallest bf16 still gets mask 0 (its bias is that value either way).
  // fp32 comparisons give the key order exactly when the threshold t is a number: +0 equals -0
  // and a NaN compares false.  Below the cut the test is f >= t, as f > t_lo with t_lo the fp32
  // value just below t (no bf16 value lies between them).  t is taken with a nonzero exponent
  // (normal or infinite), so the outcome is the same whether or not subnormal operands are
  // flushed to zero.  A NaN, zero or subnormal threshold, or one at or below the smallest bf16,
  // takes the key comparison.
  const uint32_t tbits = thr >= 0x8000u ? (thr & 0x7FFFu) : (~thr & 0xFFFFu);
  const float t = __uint_as_float(tbits << 16);
  const float t_lo = __uint_as_float((tbits & 0x8000u) ? (tbits << 16) + 1u : (tbits << 16) - 1u);
  const bool fast = thr != 0u && (tbits & 0x7F80u) != 0u && t > __uint_as_float((uint32_t)kBf16Lowest << 16);
  if (fast) {
#pragma unroll
    for (int m = 0; m < CH; ++m) {
      const int c = tid + m * kTopkThreads;
      if (c >= nch) continue;
      const u32x4 w = rw.v[m];
      const int below = cut - c * 8;  // keys c*8 + e with e < below are before the cut
      u32x4 mo, bo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = __uint_as_float(w[e] << 16), f1 = __uint_as_float(w[e] & 0xFFFF0000u);
        const bool k0 = f0 > (2 * e < below ? t_lo : t);
        const bool k1 = f1 > (2 * e + 1 < below ? t_lo : t);
        const uint32_t mk = (k0 ? 0x0000FFFFu : 0u) | (k1 ? 0xFFFF0000u : 0u);
        mo[e] = mk & 0x3F803F80u;
        bo[e] = (w[e] & mk) | (0xFF7FFF7Fu & ~mk);
      }
      *reinterpret_cast<u32x4*>(mdst + c * 8) = mo;
      *reinterpret_cast<u32x4*>(bdst + c * 8) = bo;
    }
  } else {
#pragma unroll
    for (int m = 0; m < CH; ++m) {
      const int c = tid + m * kTopkThreads;
      if (c >= nch) continue;
      const u32x4 w = rw.v[m];
      u32x4 mo, bo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t m2 = 0u, b2 = 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t x = (w[e] >> (16 * h)) & 0xFFFFu;
          const uint32_t key = topk_key(x);
          const bool kept = key > thr || (key == thr && c * 8 + 2 * e + h < cut);
          const bool one = kept && x != kBf16Lowest;
          m2 |= (one ? (uint32_t)kBf16One : 0u) << (16 * h);
          b2 |= (one ? x : (uint32_t)kBf16Lowest) << (16 * h);
        }
        mo[e] = m2;
        bo[e] = b2;
      }
      *reinterpret_cast<u32x4*>(mdst + c * 8) = mo;
      *reinterpret_cast<u32x4*>(bdst + c * 8) = bo;
    }
  }
}

template <int CH>
static void launch_topk_ch(const uint16_t* bias, int64_t rows, int64_t lk, int64_t k, uint16_t* mask_out,
                           uint16_t* bias_out, hipStream_t stream) {
  hipLaunchKernelGGL(topk_mask_kernel<CH>, dim3((unsigned)rows), dim3(kTopkThreads), 0, stream, bias, (int)lk, k,
                     mask_out, bias_out);
}

// Chunks per thread: the power of two that holds the row (lk <= 65536: at most 32).
hipError_t launch_topk(const uint16_t* bias, int64_t rows, int64_t lk, int64_t k, uint16_t* mask_out,
                       uint16_t* bias_out, hipStream_t stream) {
  const int64_t per = (lk / 8 + kTopkThreads - 1) / kTopkThreads;
  if (per <= 1) launch_topk_ch<1>(bias, rows, lk, k, mask_out, bias_out, stream);
  else if (per <= 2) launch_topk_ch<2>(bias, rows, lk, k, mask_out, bias_out, stream);
  else if (per <= 4) launch_topk_ch<4>(bias, rows, lk, k, mask_out, bias_out, stream);
  else if (per <= 8) launch_topk_ch<8>(bias, rows, lk, k, mask_out, bias_out, stream);
  else if (per <= 16) launch_topk_ch<16>(bias, rows, lk, k, mask_out, bias_out, stream);
  else if (per <= 32) launch_topk_ch<32>(bias, rows, lk, k, mask_out, bias_out, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dma
