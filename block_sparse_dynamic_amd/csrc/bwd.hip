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
//   bwd_pre_kernel    D = rowsum(dO * O) and a zeroed fp32 dQ accumulator.
//   bwd_main_kernel   one workgroup per (batch, kv head g, 64-key block); four
//                     wavefronts own 16 keys each.  K and V of the block sit in
//                     registers for the whole kernel and dK/dV accumulate in
//                     registers over every non-SKIP query block and every head
//                     of the group, so they are written once, without atomics.
//                     Per query block the effective bias (bias where valid,
//                     -inf elsewhere) is staged once and serves all G heads;
//                     dBias for the block is summed over the heads in
//                     registers and stored once.  SKIP blocks get zeros.
//                     dQ: dS^T goes to LDS and each wave multiplies 16 query
//                     rows by the block's K, adding into the fp32 accumulator
//                     with atomics (query rows are shared by all key blocks).
//   dq_convert_kernel fp32 accumulator -> bf16 dQ.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  S = Q K^T puts one key per lane (lane l%16)
// and 4 query rows per lane group, which is the A-operand layout of the
// key-major products dV = P^T dO and dK = dS^T Q; their B operands (dO, Q with
// the query index as the contraction) come from the row-major tiles through
// ds_read_b64_tr_b16.
#include <math.h>

#include "common.h"

namespace dma {

constexpr float kLog2eB = 1.4426950408889634f;
constexpr uint16_t kNegInfB = 0xFF80u;

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                      float* __restrict__ drow, float* __restrict__ dq_acc,
                                                      int64_t rows, int64_t lq, int64_t hq, int d) {
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
    float4* z = reinterpret_cast<float4*>(dq_acc + r * d + c * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int off = lpr / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, lpr);
  if (r < rows && c == 0) {
    const int64_t h = r % hq, bi = r / hq;  // bi = b*lq + i
    const int64_t bb = bi / lq, i = bi % lq;
    drow[(bb * hq + h) * lq + i] = acc;
  }
}

// ---------------------------------------------------------------------------
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* mask;
  const uint16_t* bias;
  const uint8_t* state;
  const uint16_t* dout;
  const float* lse;
  const float* drow;
  float* dq_acc;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dbias;
  int64_t lq, lk, hq, hkv;
  int G, nqb, nkb, total_wg;
  float scale;
  int causal;
};

template <int D>
struct BwdSmem {
  static constexpr int kRow = D + 8;
  static constexpr int kSRow = kBlock + 8;
  uint16_t k[kBlock * kRow];   // K tile [key][d]
  uint16_t q[kBlock * kRow];   // Q tile of one head [query][d]
  uint16_t g[kBlock * kRow];   // dO tile of one head [query][d]
  uint16_t s[kBlock * kSRow];  // dS^T [key][query] (bf16)
  uint16_t b[kBlock * kSRow];  // effective bias [query][key] (bf16)
  float lse2[kBlock];          // lse * log2(e), +inf outside the matrix
  float dr[kBlock];            // D = rowsum(dO * O)
};

template <int D>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdParams p) {
  constexpr int KR = BwdSmem<D>::kRow, SR = BwdSmem<D>::kSRow;
  __shared__ BwdSmem<D> sm;

  const int w = blockIdx.x;
  const int t = (p.total_wg % 8 == 0) ? (w % 8) * (p.total_wg / 8) + w / 8 : w;
  const int plane = t / p.nkb, kb = t % p.nkb;  // low kb (most query blocks under causality) first
  const int64_t bidx = plane / p.hkv, g = plane % p.hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kl = lane & 15, qg = lane >> 4;
  const int key_loc = wave * 16 + kl;
  const int64_t key_abs = (int64_t)kb * kBlock + key_loc;
  const int64_t shift = p.lk - p.lq;
  const int64_t plane_off = (int64_t)plane * p.lq * p.lk;
  const bool has_bias = p.bias != nullptr, has_mask = p.mask != nullptr;
  const float scale2 = p.scale * kLog2eB;

  // K, V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kreg[D / 32], vreg[D / 32];
  {
    const int64_t off = ((bidx * p.lk + key_abs) * p.hkv + g) * D + qg * 8;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (key_abs < p.lk) {
        kw = *reinterpret_cast<const u32x4*>(p.k + off + s * 32);
        vw = *reinterpret_cast<const u32x4*>(p.v + off + s * 32);
      }
      kreg[s] = __builtin_bit_cast(bf16x8, kw);
      vreg[s] = __builtin_bit_cast(bf16x8, vw);
    }
  }
  // K tile for dQ.
  for (int task = tid; task < kBlock * (D / 8); task += 256) {
    const int r = task / (D / 8), c = task % (D / 8);
    const int64_t key = (int64_t)kb * kBlock + r;
    u32x4 kw = {0u, 0u, 0u, 0u};
    if (key < p.lk) kw = *reinterpret_cast<const u32x4*>(p.k + ((bidx * p.lk + key) * p.hkv + g) * D + c * 8);
    *reinterpret_cast<u32x4*>(&sm.k[r * KR + c * 8]) = kw;
  }

  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    dk[dt] = f32x4{};
    dv[dt] = f32x4{};
  }

  const int trow = kl >> 2, tcol = (kl & 3) * 4;  // ds_read_b64_tr_b16 addressing inside a lane group

  for (int qb = 0; qb < p.nqb; ++qb) {
    const uint8_t st = p.state[((int64_t)plane * p.nqb + qb) * p.nkb + kb];
    const int64_t i0 = (int64_t)qb * kBlock;
    if (st == kSkip) {
      if (p.dbias != nullptr) {  // dense contract: zeros on skipped blocks
        for (int task = tid; task < kBlock * 8; task += 256) {
          const int r = task >> 3, c = task & 7;
          const int64_t i = i0 + r, j = (int64_t)kb * kBlock + c * 8;
          if (i < p.lq && j < p.lk)
            *reinterpret_cast<u32x4*>(p.dbias + plane_off + i * p.lk + j) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      continue;
    }
    const bool full = (st == kFull);
    const bool use_b = has_bias || !full;
    __syncthreads();  // previous block's readers of the staged tiles are done
    if (use_b) {
      for (int task = tid; task < kBlock * 8; task += 256) {
        const int r = task >> 3, c = task & 7;
        const int64_t i = i0 + r, j0 = (int64_t)kb * kBlock + c * 8;
        const bool inside = i < p.lq && j0 < p.lk;
        u32x4 bw = {0u, 0u, 0u, 0u};
        if (has_bias && inside) bw = *reinterpret_cast<const u32x4*>(p.bias + plane_off + i * p.lk + j0);
        if (!full) {
          u32x4 mw = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
          if (has_mask && inside) mw = *reinterpret_cast<const u32x4*>(p.mask + plane_off + i * p.lk + j0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t j = j0 + 2 * e;
            const bool v0 = inside && attends_lo(mw[e]) && (!p.causal || j <= i + shift);
            const bool v1 = inside && attends_hi(mw[e]) && (!p.causal || j + 1 <= i + shift);
            const uint32_t lo = v0 ? (bw[e] & 0xFFFFu) : kNegInfB;
            const uint32_t hi16 = v1 ? (bw[e] >> 16) : kNegInfB;
            bw[e] = lo | (hi16 << 16);
          }
        }
        *reinterpret_cast<u32x4*>(&sm.b[r * SR + c * 8]) = bw;
      }
    }
    __syncthreads();
    // effective bias of this lane's 16 (query, key) pairs, in log2 units
    f32x4 beff[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bv = 0.f;
        if (use_b) bv = __uint_as_float((uint32_t)sm.b[(tt * 16 + qg * 4 + i) * SR + key_loc] << 16) * kLog2eB;
        beff[tt][i] = bv;
      }
    f32x4 dbacc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};

    for (int hh = 0; hh < p.G; ++hh) {
      const int64_t h = g * p.G + hh;
      // ---- stage Q, dO, lse, D of head h -------------------------------------
      for (int task = tid; task < kBlock * (D / 8); task += 256) {
        const int r = task / (D / 8), c = task % (D / 8);
        const int64_t i = i0 + r;
        u32x4 qw = {0u, 0u, 0u, 0u}, gw = {0u, 0u, 0u, 0u};
        if (i < p.lq) {
          const int64_t off = ((bidx * p.lq + i) * p.hq + h) * D + c * 8;
          qw = *reinterpret_cast<const u32x4*>(p.q + off);
          gw = *reinterpret_cast<const u32x4*>(p.dout + off);
        }
        *reinterpret_cast<u32x4*>(&sm.q[r * KR + c * 8]) = qw;
        *reinterpret_cast<u32x4*>(&sm.g[r * KR + c * 8]) = gw;
      }
      if (tid < kBlock) {
        const int64_t i = i0 + tid;
        float l2 = INFINITY, dd = 0.f;
        if (i < p.lq) {
          l2 = p.lse[(bidx * p.hq + h) * p.lq + i] * kLog2eB;
          dd = p.drow[(bidx * p.hq + h) * p.lq + i];
        }
        sm.lse2[tid] = l2;
        sm.dr[tid] = dd;
      }
      __syncthreads();
      // ---- S = Q K^T and dP = dO V^T (query tiles tt, key = this lane) -------
      f32x4 sacc[4], pacc[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        sacc[tt] = f32x4{};
        pacc[tt] = f32x4{};
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.q[(tt * 16 + kl) * KR + s * 32 + qg * 8]);
          const bf16x8 ag = *reinterpret_cast<const bf16x8*>(&sm.g[(tt * 16 + kl) * KR + s * 32 + qg * 8]);
          sacc[tt] = mfma16(aq, kreg[s], sacc[tt]);
          pacc[tt] = mfma16(ag, vreg[s], pacc[tt]);
        }
      }
      // ---- P, dS -------------------------------------------------------------
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sm.lse2[tt * 16 + qg * 4]);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&sm.dr[tt * 16 + qg * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[tt][i], scale2, beff[tt][i] - l2[i]));
          const float ds = pv * (pacc[tt][i] - dd[i]);
          sacc[tt][i] = pv;
          pacc[tt][i] = ds;
          dbacc[tt][i] += ds;
        }
      }
      // ---- dV += P^T dO, dK += dS^T Q ------------------------------------------
#pragma unroll
      for (int t0 = 0; t0 < 4; t0 += 2) {
        u32x4 pw, sw;
        pw[0] = pack_bf16x2(sacc[t0][0], sacc[t0][1]);
        pw[1] = pack_bf16x2(sacc[t0][2], sacc[t0][3]);
        pw[2] = pack_bf16x2(sacc[t0 + 1][0], sacc[t0 + 1][1]);
        pw[3] = pack_bf16x2(sacc[t0 + 1][2], sacc[t0 + 1][3]);
        sw[0] = pack_bf16x2(pacc[t0][0], pacc[t0][1]);
        sw[1] = pack_bf16x2(pacc[t0][2], pacc[t0][3]);
        sw[2] = pack_bf16x2(pacc[t0 + 1][0], pacc[t0 + 1][1]);
        sw[3] = pack_bf16x2(pacc[t0 + 1][2], pacc[t0 + 1][3]);
        const bf16x8 ap = __builtin_bit_cast(bf16x8, pw), as = __builtin_bit_cast(bf16x8, sw);
        const int r0 = t0 * 16 + qg * 4 + trow;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const i16x4 g0 = lds_read_tr16(&sm.g[r0 * KR + dt * 16 + tcol]);
          const i16x4 g1 = lds_read_tr16(&sm.g[(r0 + 16) * KR + dt * 16 + tcol]);
          dv[dt] = mfma16(ap, join_bf16x8(g0, g1), dv[dt]);
          const i16x4 q0 = lds_read_tr16(&sm.q[r0 * KR + dt * 16 + tcol]);
          const i16x4 q1 = lds_read_tr16(&sm.q[(r0 + 16) * KR + dt * 16 + tcol]);
          dk[dt] = mfma16(as, join_bf16x8(q0, q1), dk[dt]);
        }
        // dS^T rows of this lane's key: 4 consecutive queries per tile
#pragma unroll
        for (int tt = t0; tt < t0 + 2; ++tt) {
          u32x2 w2;
          w2[0] = pack_bf16x2(pacc[tt][0], pacc[tt][1]);
          w2[1] = pack_bf16x2(pacc[tt][2], pacc[tt][3]);
          *reinterpret_cast<u32x2*>(&sm.s[key_loc * SR + tt * 16 + qg * 4]) = w2;
        }
      }
      __syncthreads();
      // ---- dQ rows wave*16 .. +15 += scale * dS K  (fp32 atomics) -----------
      {
        bf16x8 aS[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = ks * 32 + qg * 8 + trow;
          const i16x4 s0 = lds_read_tr16(&sm.s[r0 * SR + wave * 16 + tcol]);
          const i16x4 s1 = lds_read_tr16(&sm.s[(r0 + 4) * SR + wave * 16 + tcol]);
          aS[ks] = join_bf16x8(s0, s1);
        }
        const int64_t qrow0 = i0 + wave * 16 + qg * 4;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          f32x4 c = f32x4{};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int r0 = ks * 32 + qg * 8 + trow;
            const i16x4 k0 = lds_read_tr16(&sm.k[r0 * KR + dt * 16 + tcol]);
            const i16x4 k1 = lds_read_tr16(&sm.k[(r0 + 4) * KR + dt * 16 + tcol]);
            c = mfma16(aS[ks], join_bf16x8(k0, k1), c);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t qi = qrow0 + i;
            if (qi < p.lq) atomicAdd(p.dq_acc + ((bidx * p.lq + qi) * p.hq + h) * D + dt * 16 + kl, c[i] * p.scale);
          }
        }
      }
    }
    // ---- dBias of the block, summed over the group, from registers ----------
    if (p.dbias != nullptr && key_abs < p.lk) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t qi = i0 + tt * 16 + qg * 4 + i;
          if (qi < p.lq) p.dbias[plane_off + qi * p.lk + key_abs] = f32_to_bf16(dbacc[tt][i]);
        }
    }
  }

  // ---- dK, dV -----------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t key = (int64_t)kb * kBlock + wave * 16 + qg * 4 + i;
    if (key < p.lk) {
      const int64_t off = ((bidx * p.lk + key) * p.hkv + g) * D + kl;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        p.dk[off + dt * 16] = f32_to_bf16(dk[dt][i] * p.scale);
        p.dv[off + dt * 16] = f32_to_bf16(dv[dt][i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                         int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  u32x4 w;
  w[0] = pack_bf16x2(a.x, a.y);
  w[1] = pack_bf16x2(a.z, a.w);
  w[2] = pack_bf16x2(b.x, b.y);
  w[3] = pack_bf16x2(b.z, b.w);
  reinterpret_cast<u32x4*>(dq)[i] = w;
}

// ---------------------------------------------------------------------------
hipError_t launch_bwd(const AttnArgs& a, hipStream_t stream) {
  const int64_t rows = a.b * a.lq * a.hq;
  {
    const int64_t threads = rows * (a.d / 8);
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.o, a.dout,
                       a.drow, a.dq_acc, rows, a.lq, a.hq, (int)a.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.mask = a.mask;
  p.bias = a.bias;
  p.state = a.state;
  p.dout = a.dout;
  p.lse = a.lse_in;
  p.drow = a.drow;
  p.dq_acc = a.dq_acc;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dbias = a.dbias;
  p.lq = a.lq;
  p.lk = a.lk;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = (int)(a.hq / a.hkv);
  p.nqb = (int)((a.lq + kBlock - 1) / kBlock);
  p.nkb = (int)((a.lk + kBlock - 1) / kBlock);
  p.total_wg = (int)(a.b * a.hkv * p.nkb);
  p.scale = a.scale;
  p.causal = a.causal;
  if (a.d == 64)
    hipLaunchKernelGGL(bwd_main_kernel<64>, dim3(p.total_wg), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_main_kernel<128>, dim3(p.total_wg), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n8 = rows * a.d / 8;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, a.dq_acc, a.dq, n8);
  return hipGetLastError();
}

}  // namespace dma
