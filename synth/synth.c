/*
 * Seeded synthetic inputs for dynamic-mask attention workloads.
 *
 * This module only draws inputs.  It holds none of the attention arithmetic
 * and is shared, unchanged, by the oracle side and the device side of every
 * test and benchmark.
 *
 * Random numbers: counter-based SplitMix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014): the n-th output of
 * the stream with seed s is mix(s + (n + 1) * 0x9E3779B97F4A7C15).  Every
 * element is a pure function of (stream key, element index), so any row can be
 * regenerated alone and rows can be filled in parallel in any order.
 * Normals: Box-Muller on two 53-bit uniforms.  Values are rounded to bf16
 * with round-to-nearest-even directly from fp64 (no double rounding).
 *
 * Mask recipes (bf16 0.0 / 1.0 values):
 *   topk   the usage example on the Flash-DMA README: per query row keep the k
 *          largest bias values (ties: lowest key index first), drop selected
 *          values equal to the bf16 minimum, mask = 0 elsewhere, and set the
 *          bias at masked positions to the bf16 minimum.  Rows with lk <= k
 *          keep an all-ones mask and the bias unchanged.
 *   doc    FlashMask's column-wise row ranges (FlashMask README, Overview):
 *          key column j of a document [s, e) covers rows [j, e), i.e. causal
 *          attention inside each document, expanded to a dense mask.
 *   blocks per 64x64 block: empty, full, or per-element Bernoulli(1/2), so
 *          that all three block classes occur.
 *   ones   all-ones mask.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL
#define BF16_LOWEST 0xFF7Fu
#define BF16_ONE 0x3F80u
#define BF16_QNAN 0x7FC0u

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t ctr) { return mix64(key + GAMMA * (ctr + 1)); }

/* Stream key from a list of integers (seed, workload id, tensor tag, ...). */
uint64_t synth_key(const int64_t* parts, int n) {
  uint64_t h = 0x6A09E667F3BCC909ULL;
  for (int i = 0; i < n; ++i) h = mix64(h + GAMMA + (uint64_t)parts[i]);
  return h;
}

uint64_t synth_draw(uint64_t key, uint64_t ctr) { return draw(key, ctr); }

/* fp64 -> bf16 bits, round to nearest even on the exact value. */
static inline uint16_t bf16_rne(double x) {
  if (isnan(x)) return BF16_QNAN;
  if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
  double ax = fabs(x);
  double y;
  if (ax < 0x1p-126) {
    y = nearbyint(x * 0x1p133) * 0x1p-133; /* bf16 subnormal quantum */
  } else {
    int e;
    double m = frexp(x, &e); /* x = m 2^e, 0.5 <= |m| < 1 */
    y = ldexp(nearbyint(m * 256.0), e - 8);
  }
  if (fabs(y) >= 0x1p128) return signbit(y) ? 0xFF80u : 0x7F80u;
  float f = (float)y; /* exact: y has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

uint16_t synth_bf16_rne(double x) { return bf16_rne(x); }

/* Standard normal number `idx` of stream `key`. */
static inline double normal_at(uint64_t key, uint64_t idx) {
  uint64_t p = idx >> 1;
  double u1 = ((double)(draw(key, 2 * p) >> 11) + 1.0) * 0x1p-53; /* (0, 1] */
  double u2 = (double)(draw(key, 2 * p + 1) >> 11) * 0x1p-53;     /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586 * u2;
  return (idx & 1) ? r * sin(t) : r * cos(t);
}

/* out[i] = bf16(std * N(0,1)[i0 + i]), i in [0, n). */
void synth_normal_bf16(uint64_t key, uint64_t i0, int64_t n, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(std * normal_at(key, i0 + (uint64_t)i));
}

/* Total order on bf16 bit patterns that follows the value; +0 and -0 share a key. */
static inline uint32_t order_key(uint16_t u) {
  if (u == 0x8000u) u = 0;
  return (u & 0x8000u) ? (uint32_t)(~u & 0xFFFFu) : (uint32_t)(u | 0x8000u);
}

/* Select the k largest of row[0..n) (ties: lowest index first) into sel[]. */
static void topk_select(const uint16_t* row, int64_t n, int64_t k, uint8_t* sel) {
  int64_t hist[256];
  memset(hist, 0, sizeof hist);
  for (int64_t j = 0; j < n; ++j) hist[order_key(row[j]) >> 8]++;
  int64_t above = 0;
  int hb = 255;
  for (; hb >= 0; --hb) {
    if (above + hist[hb] >= k) break;
    above += hist[hb];
  }
  memset(hist, 0, sizeof hist);
  for (int64_t j = 0; j < n; ++j) {
    uint32_t key = order_key(row[j]);
    if ((int)(key >> 8) == hb) hist[key & 0xFF]++;
  }
  int lb = 255;
  for (; lb >= 0; --lb) {
    if (above + hist[lb] >= k) break;
    above += hist[lb];
  }
  uint32_t thr = ((uint32_t)hb << 8) | (uint32_t)lb;
  int64_t ties = k - above; /* how many equal to thr to take, lowest index first */
  for (int64_t j = 0; j < n; ++j) {
    uint32_t key = order_key(row[j]);
    uint8_t s = 0;
    if (key > thr) {
      s = 1;
    } else if (key == thr && ties > 0) {
      s = 1;
      --ties;
    }
    sel[j] = s;
  }
}

/* The top-k recipe on caller rows (exposed so that crafted rows with ties can be checked). */
void synth_topk_rows(const uint16_t* bias_in, int64_t nrows, int64_t lk, int64_t k, uint16_t* mask_out,
                     uint16_t* bias_out) {
  uint8_t* sel = (uint8_t*)malloc((size_t)lk);
  for (int64_t r = 0; r < nrows; ++r) {
    const uint16_t* row = bias_in + r * lk;
    if (lk > k) {
      topk_select(row, lk, k, sel);
      for (int64_t j = 0; j < lk; ++j)
        if (sel[j] && row[j] == BF16_LOWEST) sel[j] = 0;
    } else {
      memset(sel, 1, (size_t)lk);
    }
    for (int64_t j = 0; j < lk; ++j) {
      mask_out[r * lk + j] = sel[j] ? BF16_ONE : 0u;
      bias_out[r * lk + j] = sel[j] ? row[j] : BF16_LOWEST;
    }
  }
  free(sel);
}

enum { MASK_TOPK = 0, MASK_DOC = 1, MASK_BLOCKS = 2, MASK_ONES = 3 };
enum { FILL_KEEP = 0, FILL_LOWEST = 1, FILL_NAN = 2 };

/*
 * Rows [row0, row0 + nrows) of one (batch, kv-head) plane of the mask and the
 * bias, each [nrows, lk] bf16 bits.  bias_key / mask_key are the plane's
 * streams; element (i, j) uses counter i * lk + j.
 *   kind       MASK_* above
 *   topk       k for MASK_TOPK
 *   bias_std   standard deviation of the bias
 *   doc_bounds MASK_DOC: ndocs + 1 ascending row offsets, doc t = [b[t], b[t+1])
 *   fill       what masked bias entries hold for DOC/BLOCKS/ONES (TOPK always
 *              stores the bf16 minimum, as its recipe does)
 * mask_out may be NULL (bias only); bias_out may be NULL (mask only).
 */
void synth_rows(uint64_t bias_key, uint64_t mask_key, int kind, int64_t lk, int64_t row0,
                int64_t nrows, int64_t topk, double bias_std, const int64_t* doc_bounds, int ndocs,
                int fill, uint16_t* bias_out, uint16_t* mask_out) {
#pragma omp parallel
  {
    uint16_t* braw = (uint16_t*)malloc((size_t)lk * sizeof(uint16_t));
    uint8_t* sel = (uint8_t*)malloc((size_t)lk);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t i = row0 + r;
      uint64_t base = (uint64_t)i * (uint64_t)lk;
      for (int64_t j = 0; j < lk; ++j) braw[j] = bf16_rne(bias_std * normal_at(bias_key, base + (uint64_t)j));
      /* sel[j] = 1 where the mask attends */
      if (kind == MASK_TOPK) {
        if (lk > topk) {
          topk_select(braw, lk, topk, sel);
          for (int64_t j = 0; j < lk; ++j)
            if (sel[j] && braw[j] == BF16_LOWEST) sel[j] = 0;
        } else {
          memset(sel, 1, (size_t)lk);
        }
      } else if (kind == MASK_DOC) {
        int lo = 0, hi = ndocs; /* find t with b[t] <= i < b[t+1] */
        while (hi - lo > 1) {
          int mid = (lo + hi) / 2;
          if (doc_bounds[mid] <= i) lo = mid; else hi = mid;
        }
        int64_t s = doc_bounds[lo];
        for (int64_t j = 0; j < lk; ++j) sel[j] = (j >= s && j <= i) ? 1 : 0;
      } else if (kind == MASK_BLOCKS) {
        int64_t nkb = (lk + 63) / 64;
        int64_t qb = i / 64;
        for (int64_t kb = 0; kb < nkb; ++kb) {
          int cls = (int)(draw(mask_key, (uint64_t)(qb * nkb + kb)) & 3);
          int64_t j1 = (kb + 1) * 64 < lk ? (kb + 1) * 64 : lk;
          for (int64_t j = kb * 64; j < j1; ++j) {
            uint8_t s;
            if (cls == 0) s = 0;
            else if (cls == 1) s = 1;
            else s = (uint8_t)(draw(mask_key ^ 0x5851F42D4C957F2DULL, base + (uint64_t)j) >> 63);
            sel[j] = s;
          }
        }
      } else {
        memset(sel, 1, (size_t)lk);
      }
      uint16_t fillv = (kind == MASK_TOPK || fill == FILL_LOWEST) ? BF16_LOWEST : BF16_QNAN;
      int do_fill = (kind == MASK_TOPK) || fill != FILL_KEEP;
      if (bias_out) {
        uint16_t* bo = bias_out + r * lk;
        for (int64_t j = 0; j < lk; ++j) bo[j] = (sel[j] || !do_fill) ? braw[j] : fillv;
      }
      if (mask_out) {
        uint16_t* mo = mask_out + r * lk;
        for (int64_t j = 0; j < lk; ++j) mo[j] = sel[j] ? BF16_ONE : 0u;
      }
    }
    free(braw);
    free(sel);
  }
}
