// Forward kernel of dynamic-mask attention for gfx950.
//
// Computes O = softmax(scale * Q K^T + B, invalid positions -> -inf) V and the
// row log-sum-exp (Flash-DMA issue "Project Progress"; FlashMask README,
// Formulation), visiting only the key blocks the classification marked
// non-SKIP (Flash-DMA README, key design: K/V are loaded only for blocks whose
// mask OR-reduces to true).
//
// Work decomposition.  One workgroup owns one (batch, kv head g, 64-row query
// block, chunk of HC query heads of g's group).  All HC heads read one staged
// copy of the block's K, V, mask and bias, so the dense mask/bias planes are
// streamed from HBM once per group instead of once per query head.  Each
// wavefront owns 32 query rows of one head.
//
// Per key block (64 keys):
//   1. the workgroup copies K and V (row-major, [key][d], bf16 as loaded) and
//      the *effective* bias into LDS.  The effective bias is bias / |scale| in
//      fp32 where the position is valid and -inf elsewhere: mask, causality and
//      the ragged matrix edge are folded in once here for all HC heads.  The
//      bias is first clamped to [-2^12, 2^12] (see kBiasClamp).  The tiles of
//      the next non-SKIP block are loaded into registers meanwhile, by buffer
//      loads whose per-thread offsets are fixed for the kernel (the block's
//      corner and its valid extent go into the buffer resource, so keys past
//      lk and rows past lq read as zeros).
//   2. y = S^T / |scale| + bias / |scale| = K Q^T + the staged tile, on
//      v_mfma_f32_32x32x16_bf16: the accumulators start from the effective
//      bias, A = K rows from LDS, B = the wave's Q rows held in registers for
//      the whole kernel (negated for a negative scale, which is exact).  The
//      result's lane l holds query l%32 and 16 keys of each 32-key half, so a
//      row's 64 scores live in lanes l and l^32.  The score is x = |scale| y.
//   3. online softmax in fp32: row max over the lane pair (v_permlane32_swap),
//      exp2 with |scale| log2(e) folded into one fma per element; the reference
//      maximum (and with it the running output) moves only when a row maximum
//      exceeds it by more than 2^8 in weight, so weights stay in [0, 256] and
//      the rescale runs rarely (the wave skips it when no row needs it).
//   4. O^T += V^T P^T on v_mfma_f32_32x32x16_f16, one product per k-step.  V
//      is staged as fp16 scaled by a power of two per 8-key group (a multiple
//      of 8 that puts its largest magnitude in [2^7, 2^15), so the bf16 values
//      are exact in fp16), and the weights as P * 2^(group exponent - e_ref)
//      rounded to fp16 (relative 2^-11; no scaling when the groups share
//      e_ref; P carries a constant 2^7 that cancels in O and keeps weights
//      scaled down for small groups out of fp16's subnormals), e_ref being
//      the largest group exponent met so far: the output
//      accumulators stay in units of 2^e_ref and are rescaled exactly when it
//      rises; O takes the factor 2^e_ref at the end.  P^T goes from the
//      accumulator registers straight into the B operand (the key order inside
//      a k-step only has to agree between A and B); V^T comes out of the
//      row-major V tile by ds_read_b64_tr_b16.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace dma {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* mask;
  const int32_t* rstart;  // column ranges (instead of the mask): key j attends rows rstart[j] <= i < rend[j]
  const int32_t* rend;
  const uint8_t* mbits;   // bit-packed PARTIAL blocks (instead of the mask)
  const uint16_t* bias;
  const uint8_t* state;
  uint8_t* state_out;  // classification output of the fused mode
  uint16_t* o;
  float* lse;
  int64_t lq, lk, hq, hkv;
  int G, chunks, nqb, nkb, total_wg;
  float scale;
  int causal;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStateChunkF = 1024;                    // key blocks whose states are cached in LDS at a time
constexpr float kRescaleMargin = 8.f * 0.69314718f;  // natural-log units
// The weights are computed as exp(x - m_ref) * 2^kPShift: under the rescale margin they stay below
// 2^15, inside fp16, and weights scaled down to a smaller V group's units keep 7 more bits before
// they reach fp16's subnormals.  The factor cancels in O = sum(P V) / sum(P); the log-sum-exp
// takes it out.
constexpr float kPShift = 7.f;
constexpr uint16_t kBf16NegInf = 0xFF80u;

template <int D>
struct alignas(16) FwdSmem {  // 16-byte aligned so tile reads and writes stay single 16-byte LDS accesses
  static constexpr int kRow = tile_row<D>();  // row (elements) of the K and V tiles (tile_off layout)
  static constexpr int kBRow = kBlock + 4;  // fp32 row: 272 bytes, so 8 consecutive rows hit distinct banks
  // Two buffers of the K and effective-bias tiles and three of V: iteration i reads K, bias and V
  // of its block and (the waves that defer their P V) the V of the block before, while it
  // stages K, bias and V of the next block.
  uint16_t k[2][kBlock * kRow];
  uint16_t v[3][kBlock * kRow];
  float b[2][kBlock * kBRow];  // effective bias / |scale| (-inf where invalid): the S accumulators' start
  uint8_t st[kStateChunkF];    // block states of this query block's row, a chunk at a time
  int32_t rs[2][kBlock];       // column ranges of the blocks staged in alternate iterations (range input)
  int32_t re[2][kBlock];
  int32_t cls[2][2][8];        // per-wave any / all of a staged block's validity (fused classification)
  int32_t ve[3][8];            // exponent of each 8-key group of the V buffers: V = V_tile * 2^ve
};

// Operand reads issued this many products ahead (K for S, two V reads per step for P V).  Each
// product's accumulator passes through an empty asm statement after the read issued for a later
// product, which keeps the product behind that read: the scheduler would otherwise place every
// product right after its own read and wait out the LDS round trip.
constexpr int kLeadQK = 2, kLeadPV = 2;

template <int D, int HC, int MK>
__global__ __launch_bounds__(HC * 128) void fwd_kernel(FwdParams p) {
  constexpr int NT = HC * 128;
  constexpr int KR = FwdSmem<D>::kRow, BR = FwdSmem<D>::kBRow;
  __shared__ FwdSmem<D> sm;

  // XCD-aware order (xcd_task): units of (plane, head chunk), query blocks from the last
  // (longest under causality) to the first.
  const int w = blockIdx.x;
  const int t = xcd_task(w, p.total_wg, p.total_wg / p.nqb);
  const int unit = t / p.nqb;
  const int qb = p.nqb - 1 - (t % p.nqb);
  const int plane = unit / p.chunks, chunk = unit % p.chunks;
  const int64_t bidx = plane / p.hkv, g = plane % p.hkv;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int head = (int)g * p.G + chunk * HC + (wave >> 1);
  const int rloc = (wave & 1) * 32 + (lane & 31);  // query row inside the block
  const int64_t row = (int64_t)qb * kBlock + rloc;
  const int64_t shift = p.lk - p.lq;
  const int hi = lane >> 5;  // which half of the key quartets this lane holds

  // Q rows in registers: B operand of S^T = K Q^T, d = s*16 + hi*8 .. +7.
  bf16x8 qreg[D / 16];
  {
    const uint16_t* qp = p.q + ((bidx * p.lq + row) * p.hq + head) * D + hi * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 w4 = {0u, 0u, 0u, 0u};
      if (row < p.lq) w4 = *reinterpret_cast<const u32x4*>(qp + s * 16);
      if (p.scale < 0.f) w4 ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};  // exact
      qreg[s] = __builtin_bit_cast(bf16x8, w4);
    }
  }
  // Wait for Q here: the compiler then knows it is loaded, instead of waiting for it (vmcnt) at
  // its first use inside the loop on every block, which would also wait for the prefetch.
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  float m_ref = -INFINITY, l_part = 0.f;

  const uint8_t* st_row = MK == kMaskDenseClassify ? nullptr : p.state + ((int64_t)plane * p.nqb + qb) * p.nkb;
  const uint16_t* kbase = p.k + (bidx * p.lk * p.hkv + g) * D;
  const uint16_t* vbase = p.v + (bidx * p.lk * p.hkv + g) * D;
  const int64_t plane_off = (int64_t)plane * p.lq * p.lk;
  const bool has_bias = p.bias != nullptr, has_mask = p.mask != nullptr;
  // scores are carried as y = x / |scale| (Q negated above for a negative scale)
  const float as = fabsf(p.scale), inv_as = 1.f / as, as_l2e = as * kLog2e;

  // Block states of this row are cached in LDS a chunk at a time, so skipping a SKIP block
  // costs an LDS read instead of a dependent global load.
  int cache_lo = -kStateChunkF;  // cached key blocks: [cache_lo, cache_lo + kStateChunkF)
  // fused classification: the blocks not wholly excluded by causality are [0, kb_end)
  constexpr bool kCls = MK == kMaskDenseClassify;
  int kb_end = p.nkb;
  if (kCls && p.causal) {
    const int64_t last = min((int64_t)qb * kBlock + kBlock - 1, p.lq - 1) + shift;  // largest visible key
    kb_end = last < 0 ? 0 : (int)min((int64_t)p.nkb, last / kBlock + 1);
  }
  auto next_kb = [&](int from) -> int {
    if constexpr (kCls) return from < kb_end ? from : p.nkb;
    for (int kb = from; kb < p.nkb; ++kb) {
      if (kb >= cache_lo + kStateChunkF) {
        lds_barrier();  // every reader of the previous chunk is done
        for (int t = tid; t < kStateChunkF; t += NT) sm.st[t] = (kb + t < p.nkb) ? st_row[kb + t] : kSkip;
        lds_barrier();
        cache_lo = kb;
      }
      if (sm.st[kb - cache_lo] != kSkip) return kb;
    }
    return p.nkb;
  };

  // Registers that carry the next non-SKIP block's K, V, bias and mask while the current
  // block computes.  Every load is unconditional: lanes whose data is not needed (keys past
  // lk, rows past lq, no bias, no mask or a FULL block's mask) load an in-bounds stand-in
  // address and the value is discarded at staging, so no branch around a load makes the
  // compiler wait for the whole prefetch.
  constexpr int KN = kBlock * (D / 8) / NT, BN = kBlock * 8 / NT;
  u32x4 pk[KN], pv[KN], pb[BN], pm[BN];
  int32_t prs = 0, pre = 0;  // column range of key kb*64 + tid (range input, tid < 64)
  uint32_t pmb[BN];          // mask bits of this thread's 8 keys of its row (bit input)
  const uint8_t* mb_row = MK == kMaskBits ? p.mbits + ((int64_t)plane * p.nqb + qb) * p.nkb * kBitsPerBlock : nullptr;
  const int32_t* rs_plane = MK == kMaskRanges ? p.rstart + (int64_t)plane * p.lk : nullptr;
  const int32_t* re_plane = MK == kMaskRanges ? p.rend + (int64_t)plane * p.lk : nullptr;
  // Per-thread byte offsets of the tile loads inside a block (the same for every block); the
  // block's corner and the bytes it may read go into buffer resources, whose range checks
  // return zeros for keys past lk and rows past lq.
  // K and V: wave w loads and stages rows w*RPW .. +RPW-1 of a block (whole 8-key groups, each
  // of which gets one V exponent), 16-byte chunk kc[n] of row kr[n].
  constexpr int RPW = kBlock / (NT / 64);
  uint32_t kvo[KN], bo[BN];
  int kr[KN], kc[KN];
#pragma unroll
  for (int n = 0; n < KN; ++n) {
    const int li = lane + n * 64;
    kr[n] = wave * RPW + li / (D / 8);
    kc[n] = li % (D / 8);
    kvo[n] = (uint32_t)(kr[n] * p.hkv * D + kc[n] * 8) * 2u;
  }
#pragma unroll
  for (int n = 0; n < BN; ++n) {
    const int task = tid + n * NT;
    bo[n] = (uint32_t)(task >> 3) * (uint32_t)(p.lk * 2) + (uint32_t)(task & 7) * 16u;
  }
  const int q_rows = (int)min((int64_t)kBlock, p.lq - (int64_t)qb * kBlock);
  // Loads of a block's K rows, bias and mask (or its column ranges / mask bits), and of a block's
  // V rows: the software pipeline below stages K and bias one block ahead of V.
  auto load_ranges = [&](int kb) {
    if constexpr (MK == kMaskRanges) {
      const int64_t j = min((int64_t)kb * kBlock + (tid & 63), p.lk - 1);
      prs = rs_plane[j];
      pre = re_plane[j];
    }
  };
  auto load_kbm = [&](int kb, uint8_t st) {
    const int k_rows = (int)min((int64_t)kBlock, p.lk - (int64_t)kb * kBlock);  // >= 1
    const int64_t kv0 = (int64_t)kb * kBlock * p.hkv * D;
    const uint32_t kvbytes = (uint32_t)k_rows * (uint32_t)(p.hkv * D * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(const_cast<uint16_t*>(kbase + kv0), kvbytes);
#pragma unroll
    for (int n = 0; n < KN; ++n)
      pk[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)kvo[n], 0, 0));
    // rows past lq and, in the last row, keys past lk fall outside the range (zeros); keys past
    // lk in earlier rows read the next row's values, which the staging replaces
    const int64_t corner = plane_off + (int64_t)qb * kBlock * p.lk + (int64_t)kb * kBlock;
    const uint32_t bbytes = (uint32_t)(q_rows - 1) * (uint32_t)(p.lk * 2) + (uint32_t)k_rows * 2u;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(const_cast<uint16_t*>(has_bias ? p.bias + corner : p.q), has_bias ? bbytes : 0u);
    const __amdgpu_buffer_rsrc_t rm =
        make_rsrc(const_cast<uint16_t*>(has_mask ? p.mask + corner : p.q), (has_mask && st != kFull) ? bbytes : 0u);
#pragma unroll
    for (int n = 0; n < BN; ++n) {
      pb[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)bo[n], 0, 0));
      if constexpr (MK == kMaskDense || MK == kMaskDenseClassify)
        pm[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rm, (int)bo[n], 0, 0));
      if constexpr (MK == kMaskBits) {
        const int task = tid + n * NT;
        pmb[n] = mb_row[(int64_t)kb * kBitsPerBlock + (task >> 3) * 8 + (task & 7)];
      }
    }
  };
  auto load_v = [&](int kb) {
    const int k_rows = (int)min((int64_t)kBlock, p.lk - (int64_t)kb * kBlock);
    const int64_t kv0 = (int64_t)kb * kBlock * p.hkv * D;
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(const_cast<uint16_t*>(vbase + kv0), (uint32_t)k_rows * (uint32_t)(p.hkv * D * 2));
#pragma unroll
    for (int n = 0; n < KN; ++n)
      pv[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)kvo[n], 0, 0));
  };

  // Stage block kb's K rows and effective bias into buffer `buf` (its column ranges, for the
  // range input, are in sm.rs[buf]); in the classifying mode also each wave's any / all.
  auto stage_kb = [&](int buf, int kb, uint8_t st) {
#pragma unroll
    for (int n = 0; n < KN; ++n)
      *reinterpret_cast<u32x4*>(&sm.k[buf][tile_off<D>(kr[n], kc[n] * 8)]) = pk[n];  // rows past lk are zeros
    const bool full = (st == kFull);
    bool any_v = false, all_v = true;  // fused classification: this thread's positions of the block
    // a block inside the matrix whose every key is causal for its first row: no position is cut
    // by the ragged edge or by causality (uniform across the workgroup)
    const int64_t kend = (int64_t)kb * kBlock + kBlock;
    const bool inner = q_rows == kBlock && kend <= p.lk && (!p.causal || kend - 1 <= (int64_t)qb * kBlock + shift);
    auto stage_bias = [&](auto inner_c) {
#pragma unroll
    for (int n = 0; n < BN; ++n) {
      const int task = tid + n * NT;
      const int r = task >> 3, c = task & 7;
      const int64_t i = (int64_t)qb * kBlock + r, j0 = (int64_t)kb * kBlock + c * 8;
      // columns j0 + e of this chunk are inside the matrix and causal for e <= emax
      int emax = 7;
      if constexpr (!decltype(inner_c)::value) {
        int64_t lim = p.lk - 1 - j0;
        if (p.causal) lim = min(lim, i + shift - j0);
        emax = (i < p.lq) ? (int)max((int64_t)-1, min(lim, (int64_t)7)) : -1;
      }
      const u32x4 bw = pb[n];  // zeros without a bias
      u32x4 mw = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
      if (!full) {
        if constexpr (MK == kMaskRanges) {  // attends iff start <= i < end of the key's column
          const int4 s0 = *reinterpret_cast<const int4*>(&sm.rs[buf][c * 8]);
          const int4 s1 = *reinterpret_cast<const int4*>(&sm.rs[buf][c * 8 + 4]);
          const int4 e0 = *reinterpret_cast<const int4*>(&sm.re[buf][c * 8]);
          const int4 e1 = *reinterpret_cast<const int4*>(&sm.re[buf][c * 8 + 4]);
          const int rs8[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          const int re8[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool a0 = rs8[2 * e] <= i && i < re8[2 * e];
            const bool a1 = rs8[2 * e + 1] <= i && i < re8[2 * e + 1];
            mw[e] = (a0 ? 0x3F80u : 0u) | (a1 ? 0x3F800000u : 0u);
          }
        } else if constexpr (MK == kMaskBits) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mw[e] = (((pmb[n] >> (2 * e)) & 1u) ? 0x3F80u : 0u) | (((pmb[n] >> (2 * e + 1)) & 1u) ? 0x3F800000u : 0u);
        } else {
          if (has_mask) mw = pm[n];
        }
      }
      f32x4 y0, y1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v0 = 2 * e <= emax && attends_lo(mw[e]);
        const bool v1 = 2 * e + 1 <= emax && attends_hi(mw[e]);
        if constexpr (kCls) {
          any_v = any_v || v0 || v1;
          all_v = all_v && v0 && v1;
        }
        const float lo = v0 ? clamp_bias(bf16_lo(bw[e])) * inv_as : -INFINITY;
        const float hi16 = v1 ? clamp_bias(bf16_hi(bw[e])) * inv_as : -INFINITY;
        if (e < 2) {
          y0[2 * e] = lo;
          y0[2 * e + 1] = hi16;
        } else {
          y1[2 * e - 4] = lo;
          y1[2 * e - 3] = hi16;
        }
      }
      *reinterpret_cast<f32x4*>(&sm.b[buf][r * BR + c * 8]) = y0;
      *reinterpret_cast<f32x4*>(&sm.b[buf][r * BR + c * 8 + 4]) = y1;
    }
    };
    if (inner) stage_bias(std::true_type{});
    else stage_bias(std::false_type{});
    if constexpr (kCls) {
      // the block is SKIP without a valid position, FULL when all 4096 are valid (rows past lq
      // and keys past lk count as invalid), PARTIAL otherwise; every thread holds 8 positions
      const bool wany = __any(any_v), wall = __all(all_v);
      if (lane == 0) {
        sm.cls[buf][0][wave] = wany;
        sm.cls[buf][1][wave] = wall;
      }
    }
  };
  // V goes to LDS as fp16 scaled by a power of two per wave's rows (so per 8-key group).  The
  // exponent e with V = tile * 2^e is the smallest multiple of 8 that puts the rows' largest
  // magnitude below 2^15: it lands in [2^7, 2^15), where every bf16 value within 2^22 of it is
  // exact in fp16 (smaller ones move by at most 2^-32 of it).  Groups whose largest magnitudes
  // lie within the same factor-256 band share e, so the weights of a block usually need no
  // scaling.  e goes to sm.ve for the P V products.
  auto stage_v = [&](int buf, bool keep) {
    uint32_t mx = 0u;  // largest |V| bits (bf16 magnitudes order as integers)
#pragma unroll
    for (int n = 0; n < KN; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(pv[n][e] & 0x7FFFu, (pv[n][e] >> 16) & 0x7FFFu));
    // wave maximum by DPP (no LDS round trips): prefix maxima within each row of 16 lanes, then
    // across rows; lane 63 ends with the wave's maximum (lanes shifted in from outside a row
    // contribute 0, the identity)
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x111, 0xf, 0xf, false));  // row_shr:1
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x112, 0xf, 0xf, false));  // row_shr:2
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x114, 0xf, 0xf, false));  // row_shr:4
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x118, 0xf, 0xf, false));  // row_shr:8
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x142, 0xa, 0xf, false));  // row_bcast:15
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x143, 0xc, 0xf, false));  // row_bcast:31
    mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
    const int ef = keep ? (int)(mx >> 7) : 0;  // biased exponent of the largest value (0: zero or denormal)
    const int sh = -((ef - 134) & ~7);         // -e: ef - 141 (largest value in [2^14, 2^15)) rounded up to a multiple of 8
#pragma unroll
    for (int n = 0; n < KN; ++n) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_f16x2(__builtin_amdgcn_ldexpf(bf16_lo(pv[n][e]), sh), __builtin_amdgcn_ldexpf(bf16_hi(pv[n][e]), sh));
      *reinterpret_cast<u32x4*>(&sm.v[buf][tile_off<D>(kr[n], kc[n] * 8)]) = keep ? w : u32x4{0u, 0u, 0u, 0u};
    }
    if (lane < RPW / 8) sm.ve[buf][wave * (RPW / 8) + lane] = -sh;
  };

  // Per-lane LDS element offsets of the K operand reads and the transposing V reads; the
  // loop adds compile-time row offsets only.  With the swizzled 128-wide layout the XOR of
  // the chunk index factors into these per-lane terms (equal to tile_off<D> element for element).
  const int l32 = lane & 31;
  const int trow = (lane & 15) >> 2;                           // row offset inside a 4-row tr group
  const int tcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;    // column inside a 32-wide tile
  int koff[D / 16], voff0[D / 32], voff1[D / 32];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) koff[s] = tile_off<D>(l32, s * 16 + hi * 8);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    voff0[dt] = tile_off<D>(hi * 4 + trow, dt * 32 + tcol);
    voff1[dt] = tile_off<D>(hi * 4 + trow + 8, dt * 32 + tcol);
  }

  // O^T += V^T P^T for the block whose V sits in buffer vb, both in fp16: V scaled per 8-key
  // group (sm.ve), and P scaled to match, P * 2^(ve - e_ref), so that the output accumulators
  // stay in units of 2^e_ref (e_ref: the largest group exponent met so far; the accumulators are
  // rescaled, exactly, when it rises).  P * 2^(ve - e_ref) <= P < 2^15 (P carries 2^kPShift)
  // fits fp16, whose rounding (2^-11 relative) keeps O well inside the 1e-2 its bf16 storage
  // leaves.
  u32x4 pf[2][2];  // the weights, fp16 [32-key half][16-key step]
  int e_ref = -1000;
  auto pv_products = [&](int vb) {
    constexpr int NJ = 4 * (D / 32);  // steps: (16-key step, d tile)
    f16x8 av[NJ];
    auto read_v = [&](int j) {
      const int ks = j / (D / 32), dt = j % (D / 32);
      const int rbase = ks * 16 * KR;
      av[j] = __builtin_bit_cast(f16x8, join_bf16x8(lds_read_tr16(&sm.v[vb][voff0[dt] + rbase]),
                                                     lds_read_tr16(&sm.v[vb][voff1[dt] + rbase])));
    };
#pragma unroll
    for (int j = 0; j < kLeadPV; ++j) read_v(j);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + kLeadPV < NJ) read_v(j + kLeadPV);
      const int ks = j / (D / 32), dt = j % (D / 32);
      asm volatile("" : "+v"(oacc[dt])::"memory");
      oacc[dt] = mfma32_f16(av[j], __builtin_bit_cast(f16x8, pf[ks >> 1][ks & 1]), oacc[dt]);
    }
  };

  // ---- the key-block loop, with the two waves of each SIMD in opposite phases ----------------
  // Waves of the first half (one per SIMD) take a block as S products -> softmax -> P V; the
  // other waves as S products -> P V of the block before -> softmax, keeping the weights for one
  // block.  After the S products, which both waves of a SIMD issue together, one wave's softmax
  // (vector work) runs while the other wave's P V products occupy the matrix core, and the other
  // way round: the two waves keep each other's idle units busy.  Per block (iteration i, one
  // barrier): K, bias from buffer i % 2, V of the block from buffer i % 3 and of the block before
  // from (i - 1) % 3; K, bias and V of the next block are staged into the other buffers.
  const bool defer = wave >= NT / 128;  // waves 0 .. n/2-1 do not defer, the others do
  int kbc = next_kb(0);
  uint8_t stc = kbc < p.nkb ? (kCls ? kPartial : sm.st[kbc - cache_lo]) : kSkip;
  int kbn = p.nkb;
  uint8_t stn = kSkip;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) pf[kt][hh] = u32x4{0u, 0u, 0u, 0u};
  // the deferring waves' first P V reads buffer 2 with zero weights: clear it
  for (int t2 = tid; t2 < kBlock * KR / 8; t2 += NT) reinterpret_cast<u32x4*>(&sm.v[2][0])[t2] = u32x4{0u, 0u, 0u, 0u};
  if (kbc < p.nkb) {
    load_ranges(kbc);
    load_kbm(kbc, stc);
    load_v(kbc);
    if constexpr (MK == kMaskRanges) {
      if (tid < kBlock) {
        sm.rs[0][tid] = prs;
        sm.re[0][tid] = pre;
      }
      lds_barrier();
    }
    stage_kb(0, kbc, stc);
    stage_v(0, true);
    kbn = next_kb(kbc + 1);
    stn = kbn < p.nkb ? (kCls ? kPartial : sm.st[kbn - cache_lo]) : kSkip;
    if (kbn < p.nkb) {
      load_ranges(kbn);
      load_kbm(kbn, stn);
      load_v(kbn);
    }
  }
  int vcur = 0;       // V buffer of the current block; the block before's is (vcur + 2) % 3
  bool prev_ok = false;  // the block before computed (its V and weights are valid)
  auto iteration = [&](auto parity) {
    constexpr int buf = decltype(parity)::value;
    lds_barrier();  // the tiles staged in the iteration before are visible, the buffers it read are free
    if constexpr (MK == kMaskRanges) {  // the next block's ranges, staged below
      if (kbn < p.nkb && tid < kBlock) {
        sm.rs[buf ^ 1][tid] = prs;
        sm.re[buf ^ 1][tid] = pre;
      }
    }
    bool compute = true;  // a block with no valid position (fused classification) adds nothing
    if constexpr (kCls) {
      bool a = false, f = true;
#pragma unroll
      for (int w2 = 0; w2 < NT / 64; ++w2) {
        a = a || sm.cls[buf][0][w2] != 0;
        f = f && sm.cls[buf][1][w2] != 0;
      }
      const uint8_t bst = a ? (f ? kFull : kPartial) : kSkip;
      if (chunk == 0 && tid == 0) p.state_out[((int64_t)plane * p.nqb + qb) * p.nkb + kbc] = bst;
      compute = bst != kSkip;
    }
    const int vprev = vcur == 0 ? 2 : vcur - 1;
    if (defer && prev_ok) pv_products(vprev);  // the block before's P V (oacc still in its reference)
    if (compute) {
      // ---- y = S^T / |scale| + effective bias / |scale| = K Q^T + the staged tile ----------
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.b[buf][rloc * BR + kt * 32 + gi * 8 + hi * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[kt][gi * 4 + e] = y[e];
        }
      {  // steps i = k-step * 2 + key half; the K reads run kLeadQK steps ahead
        constexpr int NI = 2 * (D / 16);
        bf16x8 ak[NI];
        auto read_k = [&](int i) { ak[i] = *reinterpret_cast<const bf16x8*>(&sm.k[buf][koff[i >> 1] + (i & 1) * 32 * KR]); };
#pragma unroll
        for (int i = 0; i < kLeadQK; ++i) read_k(i);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i + kLeadQK < NI) read_k(i + kLeadQK);
          asm volatile("" : "+v"(sacc[i & 1])::"memory");
          sacc[i & 1] = mfma32(ak[i], qreg[i >> 1], sacc[i & 1]);
        }
      }
      // ---- online softmax ----------------------------------------------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
      mx = max_with_half_swap(mx) * as;
      // The reference maximum moves only when a row's maximum exceeds it by more than
      // kRescaleMargin (8 in log2 units): below that the weights exp(x - m_ref) stay under 256
      // (2^15 with the 2^kPShift factor), which fp32 sums and fp16 weights hold, and the rescale of the
      // output accumulators (64 multiplies per lane) runs a few times per row instead of on most
      // key blocks.  It follows every P V of the old reference, whichever order the wave runs.
      if (__any(mx > m_ref + kRescaleMargin)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f((m_ref - m_new) * kLog2e);
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      }
      const float mb = ((m_ref == -INFINITY) ? 0.f : m_ref * kLog2e) - kPShift;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pw = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], as_l2e, -mb));
          sacc[kt][i] = pw;
        }
      // the block's V exponents (uniform): the reference moves up to the largest, the output
      // accumulators follow exactly; then the weights in units of 2^e_ref.  A lane's 8 weights
      // of k-step (kt, hh) are keys kt*32 + hh*16 + 4 hi + {0..3} (group kt*4 + hh*2) and
      // kt*32 + hh*16 + 8 + 4 hi + {0..3} (group kt*4 + hh*2 + 1): the accumulator layout, which
      // the transposing V reads follow.
      int ve[8];
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) ve[g8] = __builtin_amdgcn_readfirstlane(sm.ve[vcur][g8]);
      int eb = ve[0];
#pragma unroll
      for (int g8 = 1; g8 < 8; ++g8) eb = max(eb, ve[g8]);
      if (eb > e_ref) {
        const float f = __builtin_amdgcn_ldexpf(1.f, max(e_ref - eb, -200));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= f;
        e_ref = eb;
      }
      bool uniform = true;  // every group at e_ref: the weights go to fp16 unscaled
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) uniform = uniform && ve[g8] == e_ref;
      if (uniform) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // the row sum takes the fp16 weights the P V products take, two per dot instruction
              // (from the pair as built: a bit cast of an element of pf compiled to element 0)
              const f16x2 h = {(_Float16)sacc[kt][hh * 8 + 2 * e], (_Float16)sacc[kt][hh * 8 + 2 * e + 1]};
              pf[kt][hh][e] = __builtin_bit_cast(uint32_t, h);
              rs = __builtin_amdgcn_fdot2(h, f16x2{(_Float16)1.f, (_Float16)1.f}, rs, false);
            }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) rs += sacc[kt][i];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float sa = __builtin_amdgcn_ldexpf(1.f, max(ve[kt * 4 + hh * 2] - e_ref, -200));
          const float sb = __builtin_amdgcn_ldexpf(1.f, max(ve[kt * 4 + hh * 2 + 1] - e_ref, -200));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sc = e < 2 ? sa : sb;
            pf[kt][hh][e] = pack_f16x2(sacc[kt][hh * 8 + 2 * e] * sc, sacc[kt][hh * 8 + 2 * e + 1] * sc);
          }
        }
      }
      l_part += rs;
      if (!defer) pv_products(vcur);
    }
    prev_ok = compute;
    // ---- stage the next block's K, bias and V; load the one after -----------------------------
    // (range input: the next block's column ranges were written after this iteration's barrier by
    // the first wave; one more barrier orders them before the staging reads them)
    if constexpr (MK == kMaskRanges) lds_barrier();
    if (kbn < p.nkb) {
      const int vnext = vcur == 2 ? 0 : vcur + 1;  // the buffer of the block two back, read by no one now
      stage_kb(buf ^ 1, kbn, stn);
      stage_v(vnext, true);
      kbc = kbn;
      stc = stn;
      kbn = next_kb(kbn + 1);
      stn = kbn < p.nkb ? (kCls ? kPartial : sm.st[kbn - cache_lo]) : kSkip;
      if (kbn < p.nkb) {
        load_ranges(kbn);
        load_kbm(kbn, stn);
        load_v(kbn);
      }
      vcur = vnext;
    } else {
      kbc = p.nkb;
    }
  };
  // The loop is unrolled twice, so the K / bias buffer of every LDS access is a compile-time
  // constant (an immediate offset instead of an address add per access).
  while (kbc < p.nkb) {
    iteration(std::integral_constant<int, 0>{});
    if (kbc >= p.nkb) break;
    iteration(std::integral_constant<int, 1>{});
  }
  lds_barrier();  // the same barrier count in every wave
  if (defer && prev_ok) pv_products(vcur);  // the last block's P V

  if constexpr (kCls) {  // blocks wholly excluded by causality are SKIP without a read
    if (chunk == 0)
      for (int kbd = kb_end + tid; kbd < p.nkb; kbd += NT) p.state_out[((int64_t)plane * p.nqb + qb) * p.nkb + kbd] = kSkip;
  }

  // ---- epilogue -----------------------------------------------------------------
  const float l_tot = sum_with_half_swap(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row < p.lq) {
    uint16_t* op = p.o + ((bidx * p.lq + row) * p.hq + head) * D + hi * 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 w2;
        // O = accumulator * 2^e_ref / l, the power of two applied exactly last
        w2[0] = pack_bf16x2(__builtin_amdgcn_ldexpf(oacc[dt][gi * 4 + 0] * inv, e_ref),
                            __builtin_amdgcn_ldexpf(oacc[dt][gi * 4 + 1] * inv, e_ref));
        w2[1] = pack_bf16x2(__builtin_amdgcn_ldexpf(oacc[dt][gi * 4 + 2] * inv, e_ref),
                            __builtin_amdgcn_ldexpf(oacc[dt][gi * 4 + 3] * inv, e_ref));
        *reinterpret_cast<u32x2*>(op + dt * 32 + gi * 8) = w2;
      }
    // l_tot carries the weights' 2^kPShift
    if (hi == 0) p.lse[(bidx * p.hq + head) * p.lq + row] = l_tot > 0.f ? m_ref + logf(l_tot) - kPShift * 0.69314718f : INFINITY;
  }
}

template <int D, int HC>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  if (p.rstart != nullptr)
    hipLaunchKernelGGL((fwd_kernel<D, HC, kMaskRanges>), dim3(p.total_wg), dim3(HC * 128), 0, stream, p);
  else if (p.mbits != nullptr)
    hipLaunchKernelGGL((fwd_kernel<D, HC, kMaskBits>), dim3(p.total_wg), dim3(HC * 128), 0, stream, p);
  else if (p.state_out != nullptr)
    hipLaunchKernelGGL((fwd_kernel<D, HC, kMaskDenseClassify>), dim3(p.total_wg), dim3(HC * 128), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<D, HC, kMaskDense>), dim3(p.total_wg), dim3(HC * 128), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.mask = a.mask;
  p.rstart = a.rstart;
  p.rend = a.rend;
  p.mbits = a.mbits;
  p.bias = a.bias;
  p.state = a.state;
  p.state_out = a.state_out;
  p.o = a.o_out;
  p.lse = a.lse_out;
  p.lq = a.lq;
  p.lk = a.lk;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = (int)(a.hq / a.hkv);
  const int HC = p.G >= 4 ? 4 : p.G;
  p.chunks = p.G / HC;
  p.nqb = (int)((a.lq + kBlock - 1) / kBlock);
  p.nkb = (int)((a.lk + kBlock - 1) / kBlock);
  p.total_wg = (int)(a.b * a.hkv * p.chunks * p.nqb);
  p.scale = a.scale;
  p.causal = a.causal;
  if (a.d == 64) {
    if (HC == 1) return launch_fwd_t<64, 1>(p, stream);
    if (HC == 2) return launch_fwd_t<64, 2>(p, stream);
    return launch_fwd_t<64, 4>(p, stream);
  }
  if (HC == 1) return launch_fwd_t<128, 1>(p, stream);
  if (HC == 2) return launch_fwd_t<128, 2>(p, stream);
  return launch_fwd_t<128, 4>(p, stream);
}

}  // namespace dma
