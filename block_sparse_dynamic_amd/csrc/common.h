// Device-side helpers shared by the gfx950 kernels of libdma.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dma {

constexpr int kBlock = 64;  // classification block: 64 query rows x 64 key columns
constexpr uint8_t kSkip = 0, kPartial = 1, kFull = 2;
// How the attention kernels learn which (query, key) pairs attend: a dense bf16 mask (or none),
// per-key row intervals, or the bit-packed PARTIAL blocks written by the classification.
constexpr int kMaskDense = 0, kMaskRanges = 1, kMaskBits = 2;
// The forward with a dense mask that also classifies the blocks it visits (no input bitmap).
constexpr int kMaskDenseClassify = 3;
constexpr int kBitsPerBlock = kBlock * kBlock / 8;  // bytes of one block's bits: row r at bytes 8r .. 8r+7

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over [base, base + bytes).  A buffer access whose per-lane offset (plus
// its immediate offset) is at or past `bytes` is dropped by the hardware: stores and atomics
// write nothing.  Word 3 is the data-format word of the gfx9 family.  The per-lane offset
// must carry every part of the address that needs the check; the scalar offset is not checked.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past any range these kernels make

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ bool attends_lo(uint32_t w) { return (w & 0x7FFFu) != 0; }
__device__ __forceinline__ bool attends_hi(uint32_t w) { return (w & 0x7FFF0000u) != 0; }

// Bias values at valid positions are clamped to [-kBiasClamp, kBiasClamp] before use, in the
// forward and the backward alike.  Scores are fp32, so a score of magnitude M carries a rounding
// of about M 2^-24 (M 2^-24 / |scale| in the units the kernels carry it in), and the fp32
// log-sum-exp handed from the forward to the backward has a spacing of M 2^-23.  At 2^12 these
// cost O at most about 1e-3 of the output tolerance and the backward's P = exp(S - lse) about
// 1e-3 relative; at the smallest bf16 that the pages' recipe writes into masked bias entries
// (-3.39e38, which a caller may pass without the mask) nothing of the q.k term or of the
// normaliser would be left.  A clamped entry still weighs exp(-2^12) = 0 against every
// unclamped score of its row, and equal entries stay equal, so only a row whose valid keys all
// carry distinct biases beyond the clamp is changed (its weights no longer favour the larger).
// Task of workgroup w of `total`, which the hardware dispatches to XCD w % 8 (the k-th of them
// on an XCD being w / 8).  The tasks form `units` independent ranges of equal length (a (batch,
// KV head) plane, or a plane's head chunk), each ordered longest first under causality.  With
// the units a multiple of 8, XCD x gets the contiguous tasks of whole units: every XCD the same
// work, and one XCD's L2 serves a unit's shared rows.  With 1, 2 or 4 units, each unit gets 8 /
// units XCDs of its own, its range is cut into twice as many contiguous segments, and the j-th
// of its XCDs takes segments j and (last - j), the earlier one first: under a causal mask a
// segment of long tasks and one of short ones (equal sums for a linear decline), still
// contiguous rows or keys of one unit for the L2.  A plain contiguous split would give one XCD
// the longest tasks of a range and another its shortest.  Other counts keep the dispatch order.
__device__ __forceinline__ int xcd_task(int w, int total, int units) {
  if (total % 8 == 0 && units % 8 == 0) return (w % 8) * (total / 8) + w / 8;
  if ((units != 1 && units != 2 && units != 4) || total % 16 != 0) return w;
  const int per = total / units, xpu = 8 / units, nseg = 2 * xpu, seg = per / nseg;
  const int x = w % 8, k = w / 8, unit = x / xpu, j = x % xpu;
  return unit * per + (k < seg ? j * seg + k : (nseg - 1 - j) * seg + (k - seg));
}

constexpr float kBiasClamp = 4096.f;
__device__ __forceinline__ float clamp_bias(float b) { return __builtin_amdgcn_fmed3f(b, -kBiasClamp, kBiasClamp); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// Two fp32 values -> bf16 pair, as one v_cvt_pk_bf16_f32 (the same rounding as f32_to_bf16);
// converting the halves one by one costs a shift and a merge on top of two conversions.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// LDS tile layouts.  A [rows][D] bf16 tile stores the 16-byte chunk c of row r at chunk
// c ^ tile_xor<D>(r), rows unpadded.  For D = 128 the XOR is 4*(r%4) + (r/4)%4: a 128-bit
// operand read (16 lanes on 16 consecutive rows, one chunk each) and a transposing 64-bit
// read (4 consecutive rows x 32 bytes per 16-lane group) both touch every bank once per
// cycle.  For D = 64 it is (r/2)%8.  Every row offset that is a multiple of 16 leaves the
// XOR unchanged, so such offsets add to a per-lane base.  Whole 16-byte chunks stay
// together, which lets a buffer load write a tile straight into LDS (each lane fetches the
// global chunk that belongs at its slot).
template <int D>
__device__ __forceinline__ int tile_xor(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (row >> 1) & 7;
  }
}
__device__ __forceinline__ int swz128(int row, int col) {
  return (row << 7) | ((((col >> 3) ^ tile_xor<128>(row)) << 3) | (col & 7));
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ tile_xor<D>(row)) << 3) | (col & 7));
}
template <int D>
constexpr int tile_row() {
  return D;
}
// A [rows][32] bf16 tile stores the 8-byte unit u of row r at unit u ^ ((r/4)%8): conflict
// free for 8-byte writes of 32 consecutive rows and for transposing reads of 4-row groups.
__device__ __forceinline__ int swz32(int row, int col) {
  return (row << 5) | ((((col >> 2) ^ ((row >> 2) & 7)) << 2) | (col & 3));
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also waits for
// every outstanding global load, store and atomic of the wave (vmcnt(0)), which
// would stall on the loads a kernel issues early to overlap them with compute.
// Global results loaded into registers are still waited for by the compiler
// before their first use.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// x of the partner lane l ^ 32 combined with x by max / sum (v_permlane32_swap).
__device__ __forceinline__ float max_with_half_swap(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_half_swap(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s supplies the address of 4 consecutive 16-bit elements in[s][0..3];
// lane j receives out[j][e] = in[4e + j/4][j%4].  With lane s pointing at row
// r0 + s/4, columns c0 + 4(s%4) .. +3 of a row-major tile, lane j gets rows
// r0 .. r0+3 of column c0 + j: a column read of 4 elements.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, const_cast<void*>(p)));
}

__device__ __forceinline__ bf16x8 join_bf16x8(i16x4 a, i16x4 b) {
  bf16x8 r;
  u32x4 u;
  u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  u[0] = ua[0];
  u[1] = ua[1];
  u[2] = ub[0];
  u[3] = ub[1];
  r = __builtin_bit_cast(bf16x8, u);
  return r;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// Two fp32 values -> fp16 pair, round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace dma

// Host-side launchers (one per kernel file).
namespace dma {
hipError_t launch_classify(const uint16_t* mask, int64_t b, int64_t hkv, int64_t lq, int64_t lk, int causal,
                           uint8_t* state, uint8_t* mbits, hipStream_t stream);
hipError_t launch_classify_ranges(const int32_t* rstart, const int32_t* rend, int64_t b, int64_t hkv, int64_t lq,
                                  int64_t lk, int causal, uint8_t* state, hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* mask;
  const int32_t* rstart;  // column ranges instead of the mask: key j attends rows rstart[j] <= i < rend[j]
  const int32_t* rend;
  const uint8_t* mbits;  // bit-packed PARTIAL blocks instead of the mask, see launch_classify
  const uint16_t* bias;
  const uint8_t* state;
  uint8_t* state_out;  // the forward's classification output (dense mask, no input bitmap)
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse_in;
  uint16_t* o_out;
  float* lse_out;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dbias;
  float* nd;          // fp32 [b, hq, lq]: -rowsum(dO * O)
  float* nl2;         // fp32 [b, hq, lq]: -lse * log2(e)
  int64_t* pair_base; // [nqb + 1]: index of query block qb's first dS tile pair (live pairs before it)
  uint16_t* kt;       // bf16 [b, hkv, d, nkb2 * 128]: K transposed, zero past lk
  uint16_t* ds;       // bf16 dS tiles: per (plane, live pair, head, 32-row half) a slot of 32 x 128 values
                      // holding only the tile's nonzero 16-byte chunks, packed per writing wave
  uint64_t* dsmap;    // per slot 8 masks: which chunks of each (wave, half) of the writer are stored
  int64_t npairs;     // live key-block pairs of one plane (pair_base[nqb])
  float* dkv_acc;     // fp32 [2][b, lk, hkv, d]: dK, dV sums of split pairs (bwd_splits > 1) or of
                      // a backward in bands, else null
  int32_t* order;       // one-pass backward: main-kernel workgroup order [b * hkv * nkb2 * splits]
  int32_t* pair_counts; // its work counts, same size (null with bands)
  int64_t band_pairs; // backward in bands of query blocks whose live pairs fit this many dS slot
                      // pairs per plane (bwd_band_end); 0: one pass over all query blocks
  int64_t b, lq, lk, hq, hkv, d;
  float scale;
  int causal;
};

// Workgroups per 128-key pair in the backward.  Under causality a pair's walk over query blocks
// runs from all of them (the first pair) down to one or two (the last), and one workgroup per
// pair leaves the longest walk setting the kernel's time when the pairs are few (up to 256,
// about one per CU): there each pair's walk is cut in two halves run by two workgroups, which
// add their dK and dV into an fp32 accumulator.  Shared by the workspace sizing and the launch.
__host__ __device__ inline int bwd_splits(int64_t b, int64_t hkv, int64_t lq, int64_t lk, int causal) {
  const int64_t nqb = (lq + 63) / 64, nkb2 = ((lk + 63) / 64 + 1) / 2;
  return (causal && b * hkv * nkb2 <= 256 && nqb >= 8) ? 2 : 1;
}

// Key-block pairs (128 keys) that can hold a valid position for query block qb: all of them
// without causality, else those whose first key is at most the block's last row + lk - lq.
// Shared by the workspace sizing on the host and the kernels that index the dS tiles.
__host__ __device__ inline int64_t live_pairs(int64_t qb, int64_t lq, int64_t lk, int causal) {
  const int64_t nkb2 = ((lk + 63) / 64 + 1) / 2;
  if (!causal) return nkb2;
  const int64_t last = qb * 64 + 63 + (lk - lq);  // largest key a row of the block may attend
  if (last < 0) return 0;
  const int64_t n = last / 128 + 1;
  return n < nkb2 ? n : nkb2;
}

// The backward in bands: the band that starts at query block lo ends (exclusive) where adding
// the next block's live pairs would pass max_pairs; it holds at least one block.
inline int64_t bwd_band_end(int64_t lo, int64_t nqb, int64_t lq, int64_t lk, int causal, int64_t max_pairs) {
  int64_t hi = lo, n = 0;
  while (hi < nqb) {
    const int64_t lp = live_pairs(hi, lq, lk, causal);
    if (hi > lo && n + lp > max_pairs) break;
    n += lp;
    ++hi;
  }
  return hi;
}

hipError_t launch_fwd(const AttnArgs& a, hipStream_t stream);
hipError_t launch_topk(const uint16_t* bias, int64_t rows, int64_t lk, int64_t k, uint16_t* mask_out,
                       uint16_t* bias_out, hipStream_t stream);
// The backward's three phases (a bit set of them): the row terms, K^T and dS tile offsets; the
// main kernel (dK, dV, dBias and the dS chunks); dQ from the dS chunks.
constexpr int kBwdPrepare = 1, kBwdMain = 2, kBwdDq = 4, kBwdAll = 7;
hipError_t launch_bwd(const AttnArgs& a, hipStream_t stream, int parts = kBwdAll);
}  // namespace dma
