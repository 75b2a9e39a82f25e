// C ABI of libdma.so: argument validation and dispatch to the gfx950 kernels.
// Declarations, layouts and error behaviour are documented in include/dma.h.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/dma.h"

#include "common.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_or_null(const void* p) { return p == nullptr || aligned16(p); }

// Element counts must stay below 2^62 so that every offset fits in int64.
bool sizes_ok(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv) {
  if (b < 1 || lq < 1 || lk < 1 || hq < 1 || hkv < 1) return false;
  const double plane = (double)b * (double)hkv * (double)lq * (double)lk;
  return plane < 4.0e18;
}

int check_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const uint16_t* bias,
               const uint8_t* state, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
               int is_causal) {
  if (!q || !k || !v || !state) return DMA_ERR_INVALID_ARGUMENT;
  if (!sizes_ok(b, lq, lk, hq, hkv) || d < 1) return DMA_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return DMA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned_or_null(mask) || !aligned_or_null(bias))
    return DMA_ERR_INVALID_ARGUMENT;
  if ((mask || bias) && lk % 8 != 0) return DMA_ERR_INVALID_ARGUMENT;
  if (hq % hkv != 0) return DMA_ERR_INVALID_ARGUMENT;
  const int64_t G = hq / hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return DMA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return DMA_ERR_UNSUPPORTED;
  const int64_t nqb = (lq + 63) / 64, nkb = (lk + 63) / 64;
  if (b * hkv * nqb * (G >= 4 ? G / 4 : 1) > 0x7FFFFFFF || b * hkv * nkb > 0x7FFFFFFF) return DMA_ERR_UNSUPPORTED;
  return DMA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DMA_OK : DMA_ERR_HIP; }

// Longest query or key length the attention kernels take: their per-thread offsets inside a
// tile row range (64 rows of lk bf16 values) are 32-bit.
constexpr int64_t kMaxLen = int64_t(1) << 24;

// |scale| in [2^-100, 2^100]: the kernels carry scores as q.k + bias / |scale| with the bias
// clamped to +-2^12 and fold |scale| log2(e) into one product, all of which stay finite there.
bool scale_in_range(float scale) {
  const float a = std::fabs(scale);
  return a >= 0x1p-100f && a <= 0x1p100f;
}

}  // namespace

extern "C" {

// The block of the skip decisions (Flash-DMA README, key design: a block's mask is OR-reduced
// to decide whether it is computed; FlashMask README, Key Features: fully / partially /
// unmasked blocks).  The pages leave its size to the kernel; this library fixes 64 x 64.
int dma_block_size(void) { return dma::kBlock; }

// Text of the status codes of this C ABI (the pages define no error interface; the Python
// binding raises with this text).
const char* dma_status_string(int status) {
  switch (status) {
    case DMA_OK:
      return "ok";
    case DMA_ERR_INVALID_ARGUMENT:
      return "invalid argument";
    case DMA_ERR_UNSUPPORTED:
      return "unsupported configuration (d must be 64 or 128, hq/hkv in {1,2,4,8,16}, lq and lk at most 2^24, "
             "|scale| in [2^-100, 2^100])";
    case DMA_ERR_WORKSPACE_TOO_SMALL:
      return "workspace too small";
    case DMA_ERR_HIP:
      return "HIP runtime error";
    default:
      return "unknown status";
  }
}

int dma_block_classify(const uint16_t* mask, int64_t b, int64_t hkv, int64_t lq, int64_t lk, int is_causal,
                       uint8_t* block_state, void* stream) {
  if (!block_state || !sizes_ok(b, lq, lk, 1, hkv)) return DMA_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return DMA_ERR_INVALID_ARGUMENT;
  if (mask && (lk % 8 != 0 || !aligned16(mask))) return DMA_ERR_INVALID_ARGUMENT;
  if (b * hkv > 65535 || (lq + 63) / 64 > 65535) return DMA_ERR_UNSUPPORTED;
  return hip_status(dma::launch_classify(mask, b, hkv, lq, lk, is_causal, block_state, nullptr, (hipStream_t)stream));
}

size_t dma_mask_bits_size(int64_t b, int64_t hkv, int64_t lq, int64_t lk) {
  if (!sizes_ok(b, lq, lk, 1, hkv)) return 0;
  return (size_t)b * hkv * ((lq + 63) / 64) * ((lk + 63) / 64) * dma::kBitsPerBlock;
}

int dma_block_classify_bits(const uint16_t* mask, int64_t b, int64_t hkv, int64_t lq, int64_t lk, int is_causal,
                            uint8_t* block_state, uint8_t* mask_bits, void* stream) {
  if (!mask || !mask_bits) return DMA_ERR_INVALID_ARGUMENT;
  if (!aligned16(mask_bits)) return DMA_ERR_INVALID_ARGUMENT;
  if (!block_state || !sizes_ok(b, lq, lk, 1, hkv)) return DMA_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return DMA_ERR_INVALID_ARGUMENT;
  if (lk % 8 != 0 || !aligned16(mask)) return DMA_ERR_INVALID_ARGUMENT;
  if (b * hkv > 65535 || (lq + 63) / 64 > 65535) return DMA_ERR_UNSUPPORTED;
  return hip_status(
      dma::launch_classify(mask, b, hkv, lq, lk, is_causal, block_state, mask_bits, (hipStream_t)stream));
}

}  // extern "C"

namespace {
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shared by the dense-mask and the column-range entry points (at most one of mask and
// rstart / rend is given).
int attn_fwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const int32_t* rstart,
                  const int32_t* rend, const uint8_t* mbits, const uint16_t* bias, const uint8_t* block_state,
                  int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d, float scale, int is_causal,
                  uint16_t* o, float* lse, void* stream, uint8_t* state_out = nullptr) {
  int st = check_attn(q, k, v, mask, bias, block_state, b, lq, lk, hq, hkv, d, is_causal);
  if (st != DMA_OK) return st;
  if (!o || !lse || !aligned16(o) || !aligned16(lse)) return DMA_ERR_INVALID_ARGUMENT;
  // the scores are carried as q.k + bias / |scale|: scale must be finite and nonzero
  if (!(scale != 0.f) || !std::isfinite(scale)) return DMA_ERR_INVALID_ARGUMENT;
  if (!scale_in_range(scale)) return DMA_ERR_UNSUPPORTED;
  // per-thread byte offsets of the bias and mask tiles inside a 64 x 64 block are 32-bit
  if (lk > kMaxLen || lq > kMaxLen) return DMA_ERR_UNSUPPORTED;
  dma::AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.mask = mask;
  a.rstart = rstart;
  a.rend = rend;
  a.mbits = mbits;
  a.bias = bias;
  a.state = state_out ? nullptr : block_state;  // the fused classification writes the bitmap instead
  a.state_out = state_out;
  a.o_out = o;
  a.lse_out = lse;
  a.b = b;
  a.lq = lq;
  a.lk = lk;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.scale = scale;
  a.causal = is_causal;
  return hip_status(dma::launch_fwd(a, (hipStream_t)stream));
}
}  // namespace

extern "C" {

int dma_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const uint16_t* bias,
                 const uint8_t* block_state, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                 float scale, int is_causal, uint16_t* o, float* lse, void* stream) {
  return attn_fwd_impl(q, k, v, mask, nullptr, nullptr, nullptr, bias, block_state, b, lq, lk, hq, hkv, d, scale,
                       is_causal, o, lse, stream);
}

int dma_attn_fwd_classify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask,
                          const uint16_t* bias, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                          float scale, int is_causal, uint8_t* block_state, uint16_t* o, float* lse, void* stream) {
  if (o == nullptr || (void*)o == (void*)block_state || (void*)lse == (void*)block_state) return DMA_ERR_INVALID_ARGUMENT;
  return attn_fwd_impl(q, k, v, mask, nullptr, nullptr, nullptr, bias, block_state, b, lq, lk, hq, hkv, d, scale,
                       is_causal, o, lse, stream, block_state);
}

int dma_block_classify_ranges(const int32_t* start_row, const int32_t* end_row, int64_t b, int64_t hkv, int64_t lq,
                              int64_t lk, int is_causal, uint8_t* block_state, void* stream) {
  if (!start_row || !end_row || !block_state || !sizes_ok(b, lq, lk, 1, hkv)) return DMA_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return DMA_ERR_INVALID_ARGUMENT;
  if (!aligned4(start_row) || !aligned4(end_row)) return DMA_ERR_INVALID_ARGUMENT;
  if (b * hkv > 65535 || (lq + 63) / 64 > 65535) return DMA_ERR_UNSUPPORTED;
  return hip_status(
      dma::launch_classify_ranges(start_row, end_row, b, hkv, lq, lk, is_causal, block_state, (hipStream_t)stream));
}

int dma_attn_fwd_bits(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint8_t* mask_bits,
                      const uint16_t* bias, const uint8_t* block_state, int64_t b, int64_t lq, int64_t lk, int64_t hq,
                      int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* o, float* lse, void* stream) {
  if (!mask_bits || !aligned16(mask_bits)) return DMA_ERR_INVALID_ARGUMENT;
  return attn_fwd_impl(q, k, v, nullptr, nullptr, nullptr, mask_bits, bias, block_state, b, lq, lk, hq, hkv, d, scale,
                       is_causal, o, lse, stream);
}

int dma_attn_fwd_ranges(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* start_row,
                        const int32_t* end_row, const uint16_t* bias, const uint8_t* block_state, int64_t b, int64_t lq,
                        int64_t lk, int64_t hq, int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* o,
                        float* lse, void* stream) {
  if (!start_row || !end_row || !aligned4(start_row) || !aligned4(end_row)) return DMA_ERR_INVALID_ARGUMENT;
  return attn_fwd_impl(q, k, v, nullptr, start_row, end_row, nullptr, bias, block_state, b, lq, lk, hq, hkv, d, scale,
                       is_causal, o, lse, stream);
}

}  // extern "C"

namespace {
// Byte offsets of the backward's workspace regions, each 256-byte aligned:
//   rows       fp32 2 x [b, hq, lq]                -rowsum(dO * O), then -lse * log2(e)
//   pair_base  int64 [nqb + 1]                     first dS tile pair of each query block
//   kt         bf16 [b, hkv, d, nkb2 * 128]        K transposed
//   ds         bf16 [b, hkv, np, G, 2, 32*128]     dS tile slots of np (query block, key pair) pairs
//                                                  per plane: every live one, or those of a band
//   dsmap      u64  [b, hkv, np, G, 2, 8]          which 16-byte chunks of each slot are stored
//   dkv        fp32 2 x [b, lk, hkv, d]            dK, dV sums of split key pairs or of a banded
//                                                  backward (only then)
//   order      int32 2 x [b * hkv * nkb2 * splits] the main kernel's workgroup order and the work
//                                                  counts it is sorted by (one pass only)
struct WsLayout {
  size_t rows, pair_base, kt, ds, dsmap, dkv, order, total;
  int64_t npairs;
};
size_t up256(size_t x) { return (x + 255) / 256 * 256; }
constexpr size_t kSlotPairBytes = 2 * 32 * 128 * sizeof(uint16_t) + 2 * 8 * sizeof(uint64_t);  // per head
int64_t all_live_pairs(int64_t lq, int64_t lk, int causal) {
  int64_t np = 0;
  for (int64_t qb = 0, nqb = (lq + 63) / 64; qb < nqb; ++qb) np += dma::live_pairs(qb, lq, lk, causal);
  return np;
}
// Slots for np pairs per plane; the fp32 dK/dV sums when acc; order_tasks entries of workgroup order.
WsLayout ws_layout_n(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d, int64_t np, bool acc,
                     int64_t order_tasks = 0) {
  WsLayout w = {};
  const int64_t nqb = (lq + 63) / 64, nkb2 = ((lk + 63) / 64 + 1) / 2;
  w.npairs = np;
  w.rows = 0;
  w.pair_base = w.rows + up256((size_t)2 * b * hq * lq * sizeof(float));
  w.kt = w.pair_base + up256((size_t)(nqb + 1) * sizeof(int64_t));
  w.ds = w.kt + up256((size_t)b * hkv * d * nkb2 * 128 * sizeof(uint16_t));
  w.dsmap = w.ds + up256((size_t)b * hq * np * 2 * 32 * 128 * sizeof(uint16_t));
  w.dkv = w.dsmap + up256((size_t)b * hq * np * 2 * 8 * sizeof(uint64_t));
  w.order = w.dkv + up256(acc ? (size_t)2 * b * lk * hkv * d * sizeof(float) : 0);
  w.total = w.order + up256((size_t)2 * order_tasks * sizeof(int32_t));
  return w;
}
// One pass over all query blocks (the fastest backward).
WsLayout ws_layout(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d, int causal) {
  const int splits = dma::bwd_splits(b, hkv, lq, lk, causal);
  const int64_t nkb2 = ((lk + 63) / 64 + 1) / 2;
  return ws_layout_n(b, lq, lk, hq, hkv, d, all_live_pairs(lq, lk, causal), splits > 1, b * hkv * nkb2 * splits);
}
// Bands of single query blocks: the smallest workspace the backward runs in.
WsLayout ws_layout_min(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d, int causal) {
  const int64_t nqb = (lq + 63) / 64;
  return ws_layout_n(b, lq, lk, hq, hkv, d, dma::live_pairs(nqb - 1, lq, lk, causal), true);
}
}  // namespace

extern "C" {

size_t dma_attn_bwd_workspace_size(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                                   int is_causal) {
  if (!sizes_ok(b, lq, lk, hq, hkv) || d < 1 || hq % hkv != 0 || (is_causal != 0 && is_causal != 1)) return 0;
  return ws_layout(b, lq, lk, hq, hkv, d, is_causal).total;
}

size_t dma_attn_bwd_workspace_size_min(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                                       int is_causal) {
  if (!sizes_ok(b, lq, lk, hq, hkv) || d < 1 || hq % hkv != 0 || (is_causal != 0 && is_causal != 1)) return 0;
  return ws_layout_min(b, lq, lk, hq, hkv, d, is_causal).total;
}

}  // extern "C"

namespace {
int attn_bwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const int32_t* rstart,
                  const int32_t* rend, const uint8_t* mbits, const uint16_t* bias, const uint8_t* block_state,
                  const uint16_t* o, const uint16_t* dout, const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv,
                  int64_t d, float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                  void* workspace, size_t workspace_bytes, void* stream, bool validate_only = false,
                  int parts = dma::kBwdAll, bool allow_bands = false) {
  int st = check_attn(q, k, v, mask, bias, block_state, b, lq, lk, hq, hkv, d, is_causal);
  if (st != DMA_OK) return st;
  if (!o || !dout || !lse || !dq || !dk || !dv || !workspace) return DMA_ERR_INVALID_ARGUMENT;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned_or_null(dbias) || !aligned16(workspace))
    return DMA_ERR_INVALID_ARGUMENT;
  if (dbias && lk % 8 != 0) return DMA_ERR_INVALID_ARGUMENT;
  // the scores are carried as S + bias / scale: scale must be finite and nonzero
  if (!(scale != 0.f) || !std::isfinite(scale)) return DMA_ERR_INVALID_ARGUMENT;
  if (!scale_in_range(scale)) return DMA_ERR_UNSUPPORTED;
  // per-row byte ranges of dbias and row indices must stay within 32-bit offsets
  if (lk > kMaxLen || lq > kMaxLen) return DMA_ERR_UNSUPPORTED;
  WsLayout wl = ws_layout(b, lq, lk, hq, hkv, d, is_causal);
  int64_t band_pairs = 0;
  if (workspace_bytes < wl.total) {
    // a smaller workspace: bands of query blocks, each with as many slot pairs as fit
    if (!allow_bands) return DMA_ERR_WORKSPACE_TOO_SMALL;
    const WsLayout fixed = ws_layout_n(b, lq, lk, hq, hkv, d, 0, true);
    if (workspace_bytes < fixed.total) return DMA_ERR_WORKSPACE_TOO_SMALL;
    // an upper bound (the slot regions' 256-byte rounding only adds), then down to what fits
    int64_t np = (int64_t)((workspace_bytes - fixed.total) / ((size_t)b * hq * kSlotPairBytes));
    np = std::min(np, wl.npairs);
    while (np > 0 && ws_layout_n(b, lq, lk, hq, hkv, d, np, true).total > workspace_bytes) --np;
    if (np < dma::live_pairs((lq + 63) / 64 - 1, lq, lk, is_causal)) return DMA_ERR_WORKSPACE_TOO_SMALL;
    wl = ws_layout_n(b, lq, lk, hq, hkv, d, np, true);
    band_pairs = np;
  }
  if (validate_only) return DMA_OK;
  dma::AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.mask = mask;
  a.rstart = rstart;
  a.rend = rend;
  a.mbits = mbits;
  a.bias = bias;
  a.state = block_state;
  a.o = o;
  a.dout = dout;
  a.lse_in = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dbias = dbias;
  char* ws = static_cast<char*>(workspace);
  a.nd = reinterpret_cast<float*>(ws + wl.rows);
  a.nl2 = a.nd + b * hq * lq;
  a.pair_base = reinterpret_cast<int64_t*>(ws + wl.pair_base);
  a.kt = reinterpret_cast<uint16_t*>(ws + wl.kt);
  a.ds = reinterpret_cast<uint16_t*>(ws + wl.ds);
  a.dsmap = reinterpret_cast<uint64_t*>(ws + wl.dsmap);
  a.npairs = wl.npairs;
  a.band_pairs = band_pairs;
  if (band_pairs == 0) {  // one pass: the workgroup order and its counts, T entries each
    const int64_t tasks = b * hkv * (((lk + 63) / 64 + 1) / 2) * dma::bwd_splits(b, hkv, lq, lk, is_causal);
    a.order = reinterpret_cast<int32_t*>(ws + wl.order);
    a.pair_counts = a.order + tasks;
  }
  a.dkv_acc = (band_pairs > 0 || dma::bwd_splits(b, hkv, lq, lk, is_causal) > 1) ? reinterpret_cast<float*>(ws + wl.dkv)
                                                                                  : nullptr;
  a.b = b;
  a.lq = lq;
  a.lk = lk;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.scale = scale;
  a.causal = is_causal;
  return hip_status(dma::launch_bwd(a, (hipStream_t)stream, parts));
}
}  // namespace

extern "C" {

int dma_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const uint16_t* bias,
                 const uint8_t* block_state, const uint16_t* o, const uint16_t* dout, const float* lse, int64_t b,
                 int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* dq,
                 uint16_t* dk, uint16_t* dv, uint16_t* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_impl(q, k, v, mask, nullptr, nullptr, nullptr, bias, block_state, o, dout, lse, b, lq, lk, hq, hkv, d,
                       scale, is_causal, dq, dk, dv, dbias, workspace, workspace_bytes, stream, false, dma::kBwdAll,
                       /*allow_bands=*/true);
}

int dma_attn_bwd_part(int part, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask,
                      const uint16_t* bias, const uint8_t* block_state, const uint16_t* o, const uint16_t* dout,
                      const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                      float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int parts = 0;
  if (part == DMA_BWD_PREPARE) parts = dma::kBwdPrepare;
  else if (part == DMA_BWD_MAIN) parts = dma::kBwdMain;
  else if (part == DMA_BWD_DQ) parts = dma::kBwdDq;
  else return DMA_ERR_INVALID_ARGUMENT;
  return attn_bwd_impl(q, k, v, mask, nullptr, nullptr, nullptr, bias, block_state, o, dout, lse, b, lq, lk, hq, hkv, d,
                       scale, is_causal, dq, dk, dv, dbias, workspace, workspace_bytes, stream, false, parts);
}

int dma_attn_bwd_bits(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint8_t* mask_bits,
                      const uint16_t* bias, const uint8_t* block_state, const uint16_t* o, const uint16_t* dout,
                      const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                      float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!mask_bits || !aligned16(mask_bits)) return DMA_ERR_INVALID_ARGUMENT;
  // the main kernel addresses one plane's bits through a single buffer range
  if (lq > 0 && lk > 0 && ((lq + dma::kBlock - 1) / dma::kBlock) * ((lk + dma::kBlock - 1) / dma::kBlock) * 512 > (int64_t)1 << 31)
    return DMA_ERR_UNSUPPORTED;
  return attn_bwd_impl(q, k, v, nullptr, nullptr, nullptr, mask_bits, bias, block_state, o, dout, lse, b, lq, lk, hq,
                       hkv, d, scale, is_causal, dq, dk, dv, dbias, workspace, workspace_bytes, stream, false,
                       dma::kBwdAll, /*allow_bands=*/true);
}

int dma_attn_bwd_ranges(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* start_row,
                        const int32_t* end_row, const uint16_t* bias, const uint8_t* block_state, const uint16_t* o,
                        const uint16_t* dout, const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq,
                        int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                        uint16_t* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  if (!start_row || !end_row || !aligned4(start_row) || !aligned4(end_row)) return DMA_ERR_INVALID_ARGUMENT;
  return attn_bwd_impl(q, k, v, nullptr, start_row, end_row, nullptr, bias, block_state, o, dout, lse, b, lq, lk, hq,
                       hkv, d, scale, is_causal, dq, dk, dv, dbias, workspace, workspace_bytes, stream, false,
                       dma::kBwdAll, /*allow_bands=*/true);
}

int dma_topk_mask(const uint16_t* bias, int64_t rows, int64_t lk, int64_t k, uint16_t* mask_out, uint16_t* bias_out,
                  void* stream) {
  if (!bias || !mask_out || !bias_out) return DMA_ERR_INVALID_ARGUMENT;
  if (!aligned16(bias) || !aligned16(mask_out) || !aligned16(bias_out)) return DMA_ERR_INVALID_ARGUMENT;
  if (rows < 1 || lk < 1 || k < 1 || lk % 8 != 0) return DMA_ERR_INVALID_ARGUMENT;
  if (mask_out == bias || mask_out == bias_out) return DMA_ERR_INVALID_ARGUMENT;
  if (lk > 65536 || rows > 0x7FFFFFFF) return DMA_ERR_UNSUPPORTED;
  return dma::launch_topk(bias, rows, lk, k, mask_out, bias_out, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DMA_OK
             : DMA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Backward without allocation: the workspace is this file-scope device array.  In host code
// `scratch` names a host-side stand-in, not device memory; the device address of each GPU's
// copy comes from hipGetSymbolAddress, taken once per device with that device current and
// kept in scratch_ptr.  Every call on a GPU shares that GPU's copy.
static __device__ __align__(256) unsigned char scratch[DMA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, or nullptr if it cannot be had.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}
}  // namespace

extern "C" {

int dma_attn_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask,
                         const uint16_t* bias, const uint8_t* block_state, const uint16_t* o, const uint16_t* dout,
                         const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                         float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                         void* stream) {
  // every argument first, against a stand-in workspace of the array's size: sizes past the
  // array get the status of a caller's workspace that is too small
  const int st = attn_bwd_impl(q, k, v, mask, nullptr, nullptr, nullptr, bias, block_state, o, dout, lse, b, lq, lk, hq,
                               hkv, d, scale, is_causal, dq, dk, dv, dbias, reinterpret_cast<void*>(uintptr_t(256)),
                               (size_t)DMA_NOALLOC_SCRATCH_BYTES, stream, /*validate_only=*/true);
  if (st != DMA_OK) return st;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return DMA_ERR_HIP;
  // every workspace region the kernels read is written earlier in the same call (row terms,
  // pair offsets, K^T, and the dS chunks and chunk masks of every item the dQ kernel visits),
  // so nothing has to start at zero
  return attn_bwd_impl(q, k, v, mask, nullptr, nullptr, nullptr, bias, block_state, o, dout, lse, b, lq, lk, hq, hkv,
                       d, scale, is_causal, dq, dk, dv, dbias, ws, (size_t)DMA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
