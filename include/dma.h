/*
 * dma.h -- C ABI of the dynamic-mask attention library (libdma.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (Flash-DMA README, features and usage example; Flash-DMA issue
 * "Project Progress"; FlashMask README, Formulation):
 *
 *   valid(b,g,i,j) = mask[b,g,i,j] != 0  AND  (not is_causal OR j <= i + lk - lq)
 *   S[b,h,i,j]     = scale * <q[b,i,h,:], k[b,j,g,:]> + bias[b,g,i,j]   on valid (i,j)
 *                    -inf                                               elsewhere
 *   o[b,i,h,:]     = sum_j softmax_j(S[b,h,i,:]) * v[b,j,g,:]
 *
 * with g = h / (hq / hkv) (grouped-query attention: consecutive query heads
 * share one key/value head).  A mask element attends iff its bf16 value is
 * non-zero (bits & 0x7FFF != 0).  The bias is added after scaling and is not
 * scaled.  A query row with no valid key gets o = 0 and lse = +inf, and
 * contributes nothing to any gradient.
 *
 * Block skipping (Flash-DMA README, key design; FlashMask README, Key
 * Features): the [lq, lk] plane of every (b, g) is cut into 64 x 64 blocks
 * (query rows x key columns).  dma_block_classify() labels each block
 * SKIP (no valid element), FULL (all 4096 positions exist and are valid) or
 * PARTIAL, and forward and backward both read that one bitmap: SKIP blocks
 * load no K/V/mask/bias and do no arithmetic; FULL blocks read the bias only.
 *
 * Conventions shared by every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     row-major in the layouts written below, and 16-byte aligned.
 *   - lk must be a multiple of 8 when a mask or bias is given (16-byte rows).
 *   - Sizes are 64-bit; element offsets are computed in 64 bits (a mask plane
 *     of lq = lk = 65536 holds 2^32 elements).
 *   - stream is a hipStream_t (NULL = the default stream).  Work is enqueued on
 *     it asynchronously; the library never allocates, frees or synchronises
 *     and keeps no mutable global state, so calls on different streams may
 *     run concurrently.
 *   - Every argument is validated before anything is enqueued.  A non-zero
 *     status means nothing was enqueued and the outputs are untouched.  A
 *     launch error reported by the runtime after enqueueing returns DMA_ERR_HIP.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Outputs must not alias inputs.
 */
#ifndef DMA_H_
#define DMA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DMA_OK = 0,
  DMA_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, bad size, misalignment */
  DMA_ERR_UNSUPPORTED = 2,      /* valid but not implemented: d, group size */
  DMA_ERR_WORKSPACE_TOO_SMALL = 3,
  DMA_ERR_HIP = 4 /* the HIP runtime refused a launch */
};

enum { DMA_BLOCK_SKIP = 0, DMA_BLOCK_PARTIAL = 1, DMA_BLOCK_FULL = 2 };

/* Side of the square classification block: 64 (query rows = key columns).  The
 * block is the unit of the skip decision (Flash-DMA README, key design: a
 * block's mask is OR-reduced to decide whether it is computed; FlashMask
 * README, Key Features: fully / partially / unmasked blocks); the pages leave
 * its size to the kernel. */
int dma_block_size(void);

/* Static text for a status code (never NULL).  The pages define no error
 * interface; this is the library's own, and the Python binding raises with it. */
const char* dma_status_string(int status);

/*
 * Block classification (Flash-DMA README, key design: OR-reduction of the mask
 * block, one decision shared by forward and backward; FlashMask README, Key
 * Features: fully masked / partially masked / unmasked blocks).
 *
 *   mask        bf16 [b, hkv, lq, lk], or NULL for "every key attends"
 *   is_causal   0 or 1; blocks wholly above the causal diagonal are SKIP and
 *               their mask bytes are not read
 *   block_state out, uint8 [b, hkv, ceil(lq/64), ceil(lk/64)]:
 *               DMA_BLOCK_SKIP / DMA_BLOCK_PARTIAL / DMA_BLOCK_FULL.
 *               A block that sticks out of the matrix (ragged edge) or
 *               crosses the causal diagonal is never FULL.
 * Errors: DMA_ERR_INVALID_ARGUMENT for sizes < 1, NULL block_state, lk % 8 != 0
 * with a mask, or a misaligned mask pointer.
 */
int dma_block_classify(const uint16_t* mask, int64_t b, int64_t hkv, int64_t lq, int64_t lk, int is_causal,
                       uint8_t* block_state, void* stream);

/*
 * Forward pass (Flash-DMA issue "Project Progress": masked scores to -inf,
 * valid scores scaled, bias added; softmax; times V).
 *
 *   q           bf16 [b, lq, hq, d]
 *   k, v        bf16 [b, lk, hkv, d]; v enters the P V product in fp16,
 *               scaled by a power of two (a multiple of 8) per group of 8 keys
 *               so that the group's largest magnitude lands in [2^7, 2^15):
 *               every finite bf16 value within 2^22 of its group's largest is
 *               taken exactly (smaller ones move by at most 2^-32 of it); the
 *               weights P enter in fp16 too (relative rounding 2^-11)
 *   mask, bias  bf16 [b, hkv, lq, lk]; either may be NULL (no mask: every key
 *               attends; no bias: zero).  bias entries at masked positions
 *               are never read into the result (they may hold NaN or inf).
 *               Bias values at valid positions are clamped to [-4096, 4096]
 *               (fp32 scores and log-sum-exp resolve the softmax only up to
 *               such magnitudes); a clamped entry still weighs exp(-4096) = 0
 *               against any unclamped score of its row, so only a row whose
 *               valid keys all hold distinct biases beyond the clamp differs
 *               from the unclamped formula.  The bf16 minimum that the
 *               Flash-DMA README's recipe writes at masked entries is thus
 *               safe to pass without the mask.
 *   block_state from dma_block_classify with the same mask, sizes and is_causal
 *   scale       multiplies q.k (callers usually pass 1/sqrt(d)); |scale| in
 *               [2^-100, 2^100]
 *   o           out, bf16 [b, lq, hq, d]
 *   lse         out, fp32 [b, hq, lq]: natural log of the softmax denominator
 *               including the row maximum, +inf for rows with no valid key
 * Supported: d in {64, 128}; hq % hkv == 0 with hq / hkv in {1, 2, 4, 8, 16};
 * lq, lk <= 2^24.
 * Errors: DMA_ERR_INVALID_ARGUMENT (NULL q/k/v/o/lse/block_state, sizes < 1,
 * misalignment, lk % 8 != 0 with mask or bias, a scale that is zero or not
 * finite: the kernel carries scores as q.k + bias / |scale|),
 * DMA_ERR_UNSUPPORTED (d, group, lq or lk above 2^24: 32-bit offsets inside a
 * tile row range; |scale| outside [2^-100, 2^100]).
 * The block_state must come from dma_block_classify with the same mask and
 * sizes; one classified without causality may serve a causal call (forward and
 * backward apply causality inside every block, and the backward treats pairs
 * that causality leaves without a valid position as SKIP: only extra work).  A
 * bitmap of another mask gives wrong results (never an access outside the
 * buffers).
 */
int dma_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const uint16_t* bias,
                 const uint8_t* block_state, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                 float scale, int is_causal, uint16_t* o, float* lse, void* stream);

/*
 * Forward pass with the block classification fused in (Flash-DMA README, key
 * design: the mask's block reduction decides which tiles are computed, and the
 * same decisions serve the backward; FlashMask README: fully / partially /
 * unmasked blocks).  Computes o and lse exactly as dma_attn_fwd does after
 * dma_block_classify, and writes the same block_state bitmap, in one pass: each
 * visited block's mask tile is read once, reduced to SKIP / PARTIAL / FULL and
 * applied.  Blocks wholly excluded by causality are written SKIP and never
 * read; a block whose mask tile is all zero is written SKIP and computes
 * nothing, but its K, V and bias rows have been fetched with the mask (the
 * decision needs the tile), so masks with many all-zero blocks are better
 * served by the separate dma_block_classify.
 *
 *   arguments as dma_attn_fwd, except
 *   block_state out, uint8 [b, hkv, ceil(lq/64), ceil(lk/64)], as written by
 *               dma_block_classify for the same mask, sizes and is_causal
 * Errors: as dma_attn_fwd (block_state must not alias o or lse).
 */
int dma_attn_fwd_classify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask,
                          const uint16_t* bias, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                          float scale, int is_causal, uint8_t* block_state, uint16_t* o, float* lse, void* stream);

/* Bytes of device workspace dma_attn_bwd needs for these sizes (0 for invalid
 * sizes): the fp32 row terms -rowsum(dO * O) and -lse log2(e), each
 * [b, hq, lq], K transposed
 * (bf16), and a slot for the bf16 dS tile of every (query head, 64-row query
 * block, 128-key pair of classification blocks) that causality leaves live, from
 * which dQ is formed without atomics (FlashMask README: deterministic backward),
 * with 128 bytes per slot that record which of its 16-byte chunks are nonzero
 * (only those are written and read back).  With is_causal the count of live
 * pairs is about half of all pairs.  When the backward is causal with at most
 * 256 key pairs over all (batch, kv head) planes and at least 8 query blocks,
 * each pair's walk is split over two workgroups and the workspace also holds
 * fp32 dK and dV sums (2 x b x lk x hkv x d floats); two partial sums added
 * onto zero in either order give the same bits, so the results stay
 * deterministic.  This is the workspace of the fastest backward, one pass over
 * all query blocks; dma_attn_bwd also runs in less (down to
 * dma_attn_bwd_workspace_size_min). */
size_t dma_attn_bwd_workspace_size(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                                   int is_causal);

/* The smallest workspace dma_attn_bwd (and its _bits and _ranges variants)
 * accepts for these sizes (0 for invalid sizes): the row terms, K transposed,
 * fp32 dK and dV sums (2 x b x lk x hkv x d floats) and the dS slots of one
 * 64-row query block.  Given less than dma_attn_bwd_workspace_size(), the
 * backward runs in bands of consecutive query blocks, as many per band as the
 * slots that fit hold (Flash-DMA README, features: memory linear in the
 * sequence length); each band runs the main and dQ kernels, and dK and dV gather
 * in the fp32 sums in band order, so the results stay deterministic (they
 * differ from the one-pass results by the rounding of those sums).  Fewer,
 * larger bands run faster: pass as much workspace as can be spared. */
size_t dma_attn_bwd_workspace_size_min(int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                                       int is_causal);

/*
 * Backward pass (Flash-DMA README: gradients for query, key, value and bias,
 * the bias gradient computed inside the backward kernels).
 *
 * Inputs as for dma_attn_fwd plus
 *   o, lse      the forward's outputs for the same inputs
 *   dout        bf16 [b, lq, hq, d], gradient of the loss w.r.t. o
 * Outputs (every element written):
 *   dq          bf16 [b, lq, hq, d]
 *   dk, dv      bf16 [b, lk, hkv, d]
 *   dbias       bf16 [b, hkv, lq, lk] = dS summed over the query heads of each
 *               group; exactly 0 on invalid entries and SKIP blocks.  May be
 *               NULL: then the bias gradient is not produced.
 *   workspace   device scratch of at least dma_attn_bwd_workspace_size() bytes
 *               for the one-pass backward, or of at least
 *               dma_attn_bwd_workspace_size_min() bytes for a backward in bands
 *               of query blocks; 16-byte aligned, owned by the caller, contents
 *               on entry ignored
 * Errors: as dma_attn_fwd, plus DMA_ERR_WORKSPACE_TOO_SMALL (workspace_bytes
 *   below dma_attn_bwd_workspace_size_min()).  A key pair that
 *   the call's causality leaves no valid position for a query block is taken as
 *   SKIP whatever block_state says (such a pair owns no dS slot).
 * dq is deterministic: the same inputs give bit-identical outputs.
 */
int dma_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask, const uint16_t* bias,
                 const uint8_t* block_state, const uint16_t* o, const uint16_t* dout, const float* lse, int64_t b,
                 int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* dq,
                 uint16_t* dk, uint16_t* dv, uint16_t* dbias, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One phase of dma_attn_bwd, for callers that time or schedule the phases
 * separately (the benchmark times the main kernel on its own).  Calling
 * DMA_BWD_PREPARE, DMA_BWD_MAIN and DMA_BWD_DQ in this order on one stream with
 * the same arguments and workspace is dma_attn_bwd, bit for bit:
 *   DMA_BWD_PREPARE  the row terms -rowsum(dout * o) and -lse log2(e), K
 *                    transposed and the dS tile offsets, into the workspace
 *   DMA_BWD_MAIN     dk, dv and dbias, and the nonzero dS chunks into the workspace
 *   DMA_BWD_DQ       dq from the dS chunks
 * Arguments and errors are those of dma_attn_bwd (every call validates all of
 * them), except that the phases run only as one pass: a workspace below
 * dma_attn_bwd_workspace_size() is DMA_ERR_WORKSPACE_TOO_SMALL.  An unknown part
 * is DMA_ERR_INVALID_ARGUMENT.
 */
enum { DMA_BWD_PREPARE = 0, DMA_BWD_MAIN = 1, DMA_BWD_DQ = 2 };
int dma_attn_bwd_part(int part, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask,
                      const uint16_t* bias, const uint8_t* block_state, const uint16_t* o, const uint16_t* dout,
                      const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                      float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, outputs and errors are
 * those of dma_attn_bwd without workspace / workspace_bytes.  Its workspace is
 * one array of DMA_NOALLOC_SCRATCH_BYTES bytes in the library's device memory,
 * one copy per GPU, held until the process ends; sizes whose
 * dma_attn_bwd_workspace_size() exceeds it return DMA_ERR_WORKSPACE_TOO_SMALL
 * before anything is enqueued.  All calls on one GPU share that GPU's copy:
 * calls that overlap on one GPU (on different streams) race and must not be
 * issued; calls in stream order are safe (each call writes every workspace byte
 * it reads, so nothing depends on what an earlier call left there).  The array's
 * device address is looked up once per device (hipGetSymbolAddress) on the
 * first call made with that device current.
 */
#define DMA_NOALLOC_SCRATCH_BYTES (64u << 20)
int dma_attn_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mask,
                         const uint16_t* bias, const uint8_t* block_state, const uint16_t* o, const uint16_t* dout,
                         const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                         float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                         void* stream);

/*
 * Column-range mask input (FlashMask README, column-wise sparse representation:
 * per key column, the rows that may attend form one interval; O(L) memory).
 * Instead of the dense mask, key column j of plane (b, g) attends exactly the
 * rows i with start_row[b,g,j] <= i < end_row[b,g,j]; causality, the bias and
 * everything else are as in the dense entry points, and every result equals the
 * dense entry point's on the expanded mask (mask[b,g,i,j] = 1.0 on those rows,
 * 0 elsewhere).  An empty interval (start >= end) masks the whole column; the
 * bounds may lie outside [0, lq).
 *
 *   start_row, end_row  int32 [b, hkv, lk], device pointers, 4-byte aligned
 *
 * dma_block_classify_ranges writes the same bitmap as dma_block_classify on the
 * expanded mask, reading 8 bytes per key column and block row instead of the
 * mask.  dma_attn_fwd_ranges / dma_attn_bwd_ranges take the ranges where the
 * dense entry points take mask; their other arguments, layouts, workspace and
 * errors are those of dma_attn_fwd / dma_attn_bwd (NULL or misaligned ranges:
 * DMA_ERR_INVALID_ARGUMENT).
 */
int dma_block_classify_ranges(const int32_t* start_row, const int32_t* end_row, int64_t b, int64_t hkv, int64_t lq,
                              int64_t lk, int is_causal, uint8_t* block_state, void* stream);
int dma_attn_fwd_ranges(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* start_row,
                        const int32_t* end_row, const uint16_t* bias, const uint8_t* block_state, int64_t b, int64_t lq,
                        int64_t lk, int64_t hq, int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* o,
                        float* lse, void* stream);
int dma_attn_bwd_ranges(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* start_row,
                        const int32_t* end_row, const uint16_t* bias, const uint8_t* block_state, const uint16_t* o,
                        const uint16_t* dout, const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq,
                        int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                        uint16_t* dbias, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bit-packed mask of the PARTIAL blocks (a variant of the unified skip design
 * of the Flash-DMA README, key design: the classification pass reads the whole
 * mask once anyway, so it can keep what the attention passes need of it, one
 * bit per element of each PARTIAL block, and they read 1/16 of the bf16 mask's
 * bytes).  The pages define no such format; the results equal the dense entry
 * points' bit for bit.
 *
 *   mask_bits  device buffer of dma_mask_bits_size() bytes, 16-byte aligned,
 *              owned by the caller.  Block (b, g, qb, kb) owns the 512 bytes
 *              at ((b*hkv + g)*nqb + qb)*nkb + kb times 512 (nqb, nkb as in
 *              block_state); row r of the block is the little-endian 64-bit
 *              word at byte 8r of them, bit c = 1 iff mask[b,g,qb*64+r,kb*64+c]
 *              attends (bf16 bits & 0x7FFF != 0; 0 past lq or lk; causality
 *              not applied).  Only PARTIAL blocks are written; the bytes of
 *              the other blocks are left as they were and never read.
 *
 * dma_mask_bits_size returns that size (0 for invalid sizes).
 * dma_block_classify_bits writes block_state as dma_block_classify does and, in
 * the same pass, the bits of every PARTIAL block; mask must not be NULL.
 * dma_attn_fwd_bits / dma_attn_bwd_bits take mask_bits where the dense entry
 * points take mask, with the block_state written together with those bits (the
 * bits of any other PARTIAL block are undefined).  Other arguments, layouts,
 * workspace and errors are those of dma_attn_fwd / dma_attn_bwd (NULL or
 * misaligned mask_bits: DMA_ERR_INVALID_ARGUMENT; dma_attn_bwd_bits also
 * returns DMA_ERR_UNSUPPORTED when one plane's bits, nqb * nkb * 512 bytes,
 * exceed 2^31, i.e. above lq * lk = 2^34, L = 131072).
 */
size_t dma_mask_bits_size(int64_t b, int64_t hkv, int64_t lq, int64_t lk);
int dma_block_classify_bits(const uint16_t* mask, int64_t b, int64_t hkv, int64_t lq, int64_t lk, int is_causal,
                            uint8_t* block_state, uint8_t* mask_bits, void* stream);
int dma_attn_fwd_bits(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint8_t* mask_bits,
                      const uint16_t* bias, const uint8_t* block_state, int64_t b, int64_t lq, int64_t lk, int64_t hq,
                      int64_t hkv, int64_t d, float scale, int is_causal, uint16_t* o, float* lse, void* stream);
int dma_attn_bwd_bits(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint8_t* mask_bits,
                      const uint16_t* bias, const uint8_t* block_state, const uint16_t* o, const uint16_t* dout,
                      const float* lse, int64_t b, int64_t lq, int64_t lk, int64_t hq, int64_t hkv, int64_t d,
                      float scale, int is_causal, uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbias,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k mask construction (Flash-DMA README, usage example: keep the
 * keep_window_size largest bias values of every query row; everything else is
 * masked, and its bias is set to the smallest bf16 value).
 *
 *   bias      bf16 [rows, lk] (rows = b * hkv * lq for a [b, hkv, lq, lk] bias)
 *   k         keys kept per row (keep_window_size), >= 1
 *   mask_out  out, bf16 [rows, lk]: 1.0 at the kept positions whose value is not
 *             the smallest bf16 (-3.3895e38), 0 elsewhere
 *   bias_out  out, bf16 [rows, lk]: the bias at positions where mask_out is 1,
 *             the smallest bf16 elsewhere.  May be the same buffer as bias
 *             (in place); mask_out must differ from both.
 * A row with lk <= k keeps everything: mask all 1, bias copied unchanged.
 * Order: numeric order of the bf16 values, +0 equal to -0, NaN below every
 * number; ties at the k-th value go to the lowest key indices (the reading
 * taken for the pages' unsorted top-k), so the result is fully determined.
 * Errors: DMA_ERR_INVALID_ARGUMENT (NULL or misaligned pointers, rows, lk or
 * k < 1, lk % 8 != 0, mask_out aliasing an input), DMA_ERR_UNSUPPORTED
 * (lk > 65536: a row is held in the registers of one workgroup; rows > 2^31 - 1).
 */
int dma_topk_mask(const uint16_t* bias, int64_t rows, int64_t lk, int64_t k, uint16_t* mask_out, uint16_t* bias_out,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DMA_H_ */
