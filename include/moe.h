/*
 * moe.h -- C ABI of one GPU's routed-expert (mixture-of-experts) layer on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "Scalable Training of Mixture-of-Experts Models with Megatron Core"
 * (gist.science technical summaries).  The Spanish summary, section 2.1
 * ("Arquitectura de la capa MoE"), splits the layer into four steps: route
 * each token to its k best experts, dispatch the tokens to their experts,
 * run the experts as grouped GEMMs, combine the results.  On one GPU dispatch
 * and combine are a local permutation and a weighted un-permutation.
 *
 * Conventions for every call
 * --------------------------
 *  - All tensor pointers are DEVICE pointers, owned by the caller, row-major,
 *    16-byte aligned, and not aliased with each other unless stated.  The
 *    library never allocates or frees memory and keeps no state between
 *    calls, apart from the device array of moe_permute_noalloc (a fixed
 *    1 MiB per GPU, see there) and a per-device cache of the compute-unit
 *    count; scratch space is the caller's `ws` buffer of `ws_bytes` bytes
 *    (size from moe_workspace_bytes).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return: no host synchronisation, no copy of
 *    per-expert counts to the host (the German summary, section 2 D, and the
 *    Spanish summary, section 2.3 C: kernels read shape information from GPU
 *    memory, so dropless routing needs no CPU-GPU sync).  Calls are safe to
 *    capture into a HIP graph.
 *  - Return value: a moe_status.  Arguments are validated before anything is
 *    enqueued; MOE_ERR_HIP reports a launch failure.  Faults inside kernels
 *    surface at the caller's next synchronisation.  Nothing aborts or prints.
 *  - Shapes: T tokens, d hidden size, E experts, k experts per token, f
 *    expert FFN width, P = T*k routed rows (dropless: every assignment gets a
 *    row, so permuted buffers always have exactly P rows -- the worst case is
 *    known on the host; cf. the hyper.ai article on Hybrid-EP, which reserves
 *    buffers for the worst case).  Limits: 1 <= k <= E <= 256, T >= 1,
 *    P < 2^31.  The bf16 expert GEMMs need d and f to be multiples of 128,
 *    and P * max(d, 2f) * 2 and d * f * 2 below 2^32 bytes (the shared
 *    expert: T in place of P, f_shared in place of f); outside that they
 *    return MOE_ERR_UNSUPPORTED.
 *  - Expert weights: W1, W3 are [E][d][f], W2 is [E][f][d]; expert e maps a
 *    row x to o = (silu(x W1_e) * (x W3_e)) W2_e with silu(z) = z / (1+e^-z).
 *  - Dtypes: MOE_F32 (every tensor fp32), MOE_BF16 (x, weights, outputs and
 *    saved activations bf16, fp32 accumulation, one round-to-nearest-even per
 *    output element) or MOE_E4M3 (the expert GEMMs take OCP E4M3FN operands
 *    with fp32 block scales -- see "e4m3 expert GEMMs" below -- while x, dY,
 *    y, dX, the saved activations and the weight gradients are bf16) or
 *    MOE_MXFP8 (the same with MXFP8 operands: E4M3FN codes with one
 *    power-of-two E8M0 scale byte per 32 values -- see "MXFP8 expert GEMMs"
 *    below).  Router
 *    logits and probabilities are always fp32 (German summary, section 2 E:
 *    the router stays in high precision).
 */
#ifndef TRE_MOE_H
#define TRE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* null pointer, inconsistent or out-of-range sizes */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside this build's limits (dtype, alignment) */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2, MOE_MXFP8 = 3 } moe_dtype;

typedef struct {
  int64_t T, d, E, k, f;
  int64_t f_shared;  /* width of an always-on shared expert, 0 = none */
  int32_t dtype;     /* moe_dtype of x, weights, activations and outputs */
  int32_t reserved;  /* must be 0 */
} moe_shape;

/* Which call a workspace size is asked for. */
typedef enum {
  MOE_WS_PERMUTE = 0,
  MOE_WS_GEMM_FWD = 1,
  MOE_WS_GEMM_BWD = 2,
  MOE_WS_LAYER_FWD = 3,
  MOE_WS_LAYER_BWD = 4,
  MOE_WS_AUX_LOSS = 5,
  MOE_WS_GEMM_BWD_ROWSCALED = 6,
  MOE_WS_LAYER_BWD_ROWSCALED = 7
} moe_ws_kind;

/*
 * moe_route -- top-k routing (Spanish summary, section 2.1: a router assigns
 * each token to its k best experts).
 *   logits    fp32 [T][E].
 *   topk_idx  out int32 [T][k]: the k largest logits of the token in
 *             descending order; equal logits (IEEE equality, -0 == +0) are
 *             ordered by lower expert index first.  A NaN logit ranks below
 *             every number (-inf included), NaNs among themselves by index,
 *             so every token always gets k distinct experts in [0, E).
 *   topk_prob out fp32 [T][k]: softmax over the k selected logits,
 *             p_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), summed in j order
 *             (NaN for every pick of a token whose picks include a NaN).
 * Errors: MOE_ERR_INVALID for null pointers, T < 1, k < 1 or k > E;
 * MOE_ERR_UNSUPPORTED for E > 256 or T * k >= 2^31.
 */
int moe_route(const float* logits, int64_t T, int64_t E, int64_t k,
              int32_t* topk_idx, float* topk_prob, void* stream);

/*
 * moe_permute -- dispatch on one GPU: copy every token row to one row per
 * assignment, in expert-contiguous order (Spanish summary, section 2.1,
 * dispatch; German summary, section 1: dropless routing).
 *   build_map = 1: from topk_idx [T][k] computes
 *       counts   out int32 [E]   rows per expert;
 *       offsets  out int32 [E+1] exclusive prefix sum, offsets[E] = P;
 *       row_of   out int32 [T][k] destination row of assignment (t, j);
 *       token_of out int32 [P]   source token of each row;
 *     rows of one expert ascend by token index (a stable counting sort), so
 *     the map is unique.  An index outside [0, E) gets no row: its row_of
 *     entry is -1 and it is not counted (offsets[E] is then below P and the
 *     rows from offsets[E] on are not written).  Needs ws_bytes >=
 *     moe_workspace_bytes(sh, MOE_WS_PERMUTE).
 *   build_map = 0: uses the caller's row_of; counts, offsets, token_of, ws
 *     may be NULL.
 *   dst NULL (build_map = 1 only): the map alone, no rows moved (src may be
 *     NULL); the experts then read x through token_of (the *_gather calls).
 *   src [T][d] and dst [P][d] are in sh->dtype.  Assignments whose row_of
 *   entry lies outside [0, P) are skipped (here and in every call that reads
 *   row_of).  row_scale NULL: dst rows are bit copies of src rows.  row_scale fp32 [T][k] non-NULL: dst[row_of[t][j]]
 *   = round(row_scale[t][j] * src[t]) computed in fp32 (the backward of the
 *   weighted combine, dO = p * dY).
 */
int moe_permute(const moe_shape* sh, const void* src, const int32_t* topk_idx,
                const float* row_scale, int build_map, int32_t* counts, int32_t* offsets,
                int32_t* row_of, int32_t* token_of, void* dst, void* ws, size_t ws_bytes,
                void* stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  With build_map = 1
 * the map's per-(expert, 256-token block) counts, E * ceil(T / 256) int32
 * (aligned up to 256 bytes), go to a 1 MiB array that the library keeps in
 * device memory, one per GPU, for the life of the process (e.g. E = 256
 * experts allow T <= 262144 tokens); larger maps return MOE_ERR_WORKSPACE
 * before anything is enqueued.  All calls on one GPU share that array: calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Nothing in it needs to start at zero.  The first
 * call on a device looks up the array's device address (MOE_ERR_HIP if the
 * runtime cannot); no call allocates or frees memory.  Arguments, results
 * and errors otherwise as moe_permute.
 */
int moe_permute_noalloc(const moe_shape* sh, const void* src, const int32_t* topk_idx,
                        const float* row_scale, int build_map, int32_t* counts,
                        int32_t* offsets, int32_t* row_of, int32_t* token_of, void* dst,
                        void* stream);

/*
 * moe_unpermute -- combine on one GPU (Spanish summary, section 2.1):
 *   dst[t] = round( sum_{j=0..k-1} w[t][j] * src[row_of[t][j]] + add[t] )
 * with the sum in fp32 in j order, w = topk_prob (fp32 [T][k]) or 1 when
 * topk_prob is NULL (the backward of moe_permute), add [T][d] optional
 * (NULL = none; used for the shared expert).  src [P][d], dst [T][d] in
 * sh->dtype.  dst must not alias src.
 */
int moe_unpermute(const moe_shape* sh, const void* src, const int32_t* row_of,
                  const float* topk_prob, const void* add, void* dst, void* stream);

/*
 * moe_grouped_gemm_fwd -- the experts' forward as grouped GEMMs over the
 * expert-contiguous rows (German summary, section 2 D, and Spanish summary,
 * section 2.3 C: one grouped GEMM bundles the many small expert GEMMs).
 * For expert e and its rows r in [offsets[e], offsets[e+1]):
 *   a = xp_r W1_e, b = xp_r W3_e           saved: ab [P][2f] = [a | b]
 *   h = silu(a) * b                        saved: h  [P][f]
 *   o = h W2_e                             out:   o  [P][d]
 * offsets int32 [E+1] lives on the device (typically from moe_permute); the
 * kernels read it there.  Rows of experts with no tokens are not touched.
 * ws may be NULL (current kernels need no workspace).
 */
int moe_grouped_gemm_fwd(const moe_shape* sh, const int32_t* offsets, const void* xp,
                         const void* W1, const void* W3, const void* W2, void* ab, void* h,
                         void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_bwd -- data and weight gradients of moe_grouped_gemm_fwd,
 * as separate products (German summary, section 2 C: W/D split).  Inputs are
 * the forward's xp, ab, h and the upstream gradient dO [P][d]; outputs:
 *   dab [P][2f] = [da | db],  dH = dO W2_e^T, s = sigmoid(a),
 *                 da = dH * b * s * (1 + a (1 - s)), db = dH * silu(a)
 *   dXp [P][d]  = da W1_e^T + db W3_e^T
 *   dW2 [E][f][d] = h_e^T dO_e, dW1 = xp_e^T da_e, dW3 = xp_e^T db_e
 * (each accumulated in fp32 over all of the expert's rows, rounded once).
 * Experts with no rows get all-zero dW1, dW3, dW2.
 */
int moe_grouped_gemm_bwd(const moe_shape* sh, const int32_t* offsets, const void* xp,
                         const void* ab, const void* h, const void* dO, const void* W1,
                         const void* W3, const void* W2, void* dab, void* dXp, void* dW1,
                         void* dW3, void* dW2, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_fwd_gather / moe_grouped_gemm_bwd_gather -- the same
 * products with the permutation fused into the expert GEMMs' operand loads
 * (the pages' dispatchers eliminate permutation steps: German technical
 * summary, section 2 C, and the hyper.ai article on Hybrid-EP): row r of the
 * permuted input is row token_of[r] of x [T][d] (token_of from moe_permute's
 * map), read by fc1 forward and by the fc1 weight gradient, so no permuted
 * copy xp is written or read.  Results equal moe_grouped_gemm_fwd / _bwd on
 * xp = x[token_of] bit for bit.  bf16 and fp32; MOE_ERR_UNSUPPORTED when
 * T * d * element bytes >= 2^31 - 4096.
 */
int moe_grouped_gemm_fwd_gather(const moe_shape* sh, const int32_t* offsets,
                                const int32_t* token_of, const void* x, const void* W1,
                                const void* W3, const void* W2, void* ab, void* h, void* o,
                                void* ws, size_t ws_bytes, void* stream);
int moe_grouped_gemm_bwd_gather(const moe_shape* sh, const int32_t* offsets,
                                const int32_t* token_of, const void* x, const void* ab,
                                const void* h, const void* dO, const void* W1, const void* W3,
                                const void* W2, void* dab, void* dXp, void* dW1, void* dW3,
                                void* dW2, void* ws, size_t ws_bytes, void* stream);

/*
 * Buffers of a whole layer.  Inputs are read-only; "saved" buffers are
 * written by moe_layer_fwd and read by moe_layer_bwd; the rest are outputs.
 * Shared-expert pointers are ignored when f_shared == 0.
 */
typedef struct {
  /* inputs */
  const float* logits;                    /* fp32 [T][E] */
  const void* x;                          /* [T][d] */
  const void *W1, *W3, *W2;               /* [E][d][f], [E][d][f], [E][f][d] */
  const void *Ws1, *Ws3, *Ws2;            /* shared expert [d][fs], [d][fs], [fs][d] */
  const void* dY;                         /* [T][d], backward only */
  /* routing (written by fwd) */
  int32_t* topk_idx;                      /* [T][k] */
  float* topk_prob;                       /* [T][k] */
  int32_t *counts, *offsets;              /* [E], [E+1] */
  int32_t *row_of, *token_of;             /* [T][k], [P] */
  /* saved activations (written by fwd) */
  void *xp, *ab, *h, *o;                  /* [P][d], [P][2f], [P][f], [P][d] */
  void *s_ab, *s_h, *ys;                  /* shared expert: [T][2fs], [T][fs], [T][d] */
  /* forward output */
  void* y;                                /* [T][d] */
  /* backward scratch and outputs */
  void *dO, *dab, *dXp;                   /* [P][d], [P][2f], [P][d] */
  void *s_dab, *dXs;                      /* shared expert: [T][2fs], [T][d] */
  void* dX;                               /* [T][d] */
  void *dW1, *dW3, *dW2;                  /* like W1, W3, W2 */
  void *dWs1, *dWs3, *dWs2;               /* like Ws1, Ws3, Ws2 */
  /* e4m3 layers only (sh->dtype == MOE_E4M3; ignored otherwise): the
     quantised weights replace W1, W3, W2, which may be NULL; xp is not
     used (the backward reads x and token_of instead) */
  const struct moe_e4m3_weights* wq;
  uint8_t* xq;                            /* [T][d] codes of x */
  float* xs;                              /* [T][d/128] scales of x */
  uint8_t* xpq;                           /* [P][d] permuted codes */
  float* xps;                             /* [P][d/128] permuted scales */
  /* router gradient (optional; NULL = not computed): the forward writes the
     load-balancing loss when aux_loss is set, the backward writes dprob and
     dlogits when dlogits is set (dprob is then required) */
  float* aux_loss;                        /* device scalar */
  float* dprob;                           /* [T][k] */
  float* dlogits;                         /* [T][E] */
  float aux_alpha;                        /* coefficient alpha of the loss; 0 = none */
  /* memory-efficient permutation (bf16, e4m3, MXFP8): when memory_efficient != 0
     the probabilities are applied before W2 (h and o hold p-scaled values),
     the backward reads neither o nor a scaled dO, and row_prob [P] (written
     by the forward, read by the backward) holds each permuted row's
     probability; memory_efficient == 2 also recomputes h in the backward
     (the forward's h need not be kept, io->h is then overwritten) */
  float* row_prob;
  int32_t memory_efficient;
  /* MXFP8 layers (sh->dtype == MOE_MXFP8): the quantised weights (W1, W3, W2
     may be NULL); xq, xpq hold codes as for e4m3 and xs, xps hold E8M0 scale
     bytes, [T][d/32] and [P][d/32] (the same byte count as the e4m3 scales) */
  const struct moe_mx_weights* wmx;
  /* fused permutation (bf16 and fp32 layers): when fused_permute != 0 the
     forward builds the map alone and the experts' fc1 forward and fc1 weight
     gradient read row token_of[r] of x directly (moe_grouped_gemm_fwd_gather
     / moe_grouped_gemm_bwd_gather), so xp is neither written nor read and
     may be NULL; needs T * d * element bytes below 2^31 - 4096 */
  int32_t fused_permute;
} moe_layer_io;

/*
 * moe_layer_fwd -- route, permute, expert forward (+ shared expert applied to
 * every token with weight 1), weighted combine into y.  Same as calling
 * moe_route, moe_permute(build_map=1), moe_grouped_gemm_fwd and
 * moe_unpermute in sequence on one stream.  For MOE_E4M3: moe_route,
 * moe_quantize_rows of x into xq/xs, moe_permute_e4m3 into xpq/xps,
 * moe_grouped_gemm_fwd_e4m3, moe_unpermute (MOE_MXFP8: the _mx calls, weights
 * io->wmx).  With io->aux_loss set, the routing is moe_route_aux and
 * moe_aux_loss_final (alpha = io->aux_alpha) follows the permutation;
 * ws_bytes then needs MOE_WS_AUX_LOSS more bytes.  With io->memory_efficient:
 * moe_row_probs into io->row_prob, the row-scaled expert forward (bf16:
 * moe_grouped_gemm_fwd_rowscaled; e4m3 / MXFP8: fc1's epilogue scales h by p
 * before h is quantised) and an unweighted moe_unpermute.
 */
int moe_layer_fwd(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * moe_layer_bwd -- backward of moe_layer_fwd for upstream gradient dY:
 * dO = p * dY permuted, expert backward, dX = un-permuted sum of dXp (+ the
 * shared expert's dXs), and all weight gradients.  No gradient flows to the
 * logits unless io->dlogits is set: then dO comes from moe_combine_bwd
 * (writing io->dprob) and moe_route_bwd adds the router gradient, with the
 * load-balancing term (coefficient io->aux_alpha, upstream gradient 1).  For
 * MOE_E4M3 the expert backward is moe_grouped_gemm_bwd_e4m3.  With
 * io->memory_efficient: dO = dY permuted without scaling, then
 * moe_grouped_gemm_bwd_rowscaled (io->o is not read; dprob comes from its
 * partials; e4m3 and MXFP8 layers run the same steps with their products);
 * ws_bytes >= moe_workspace_bytes(sh, MOE_WS_LAYER_BWD_ROWSCALED).
 */
int moe_layer_bwd(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * e4m3 expert GEMMs
 * -----------------
 * The pages train the experts in FP8 with blockwise scaling on Hopper and
 * quantise weights straight from fp32 masters, keeping the router in high
 * precision (German technical summary, section 2 E; French summary, section
 * 2 E).  The quantiser used for every block B of values:
 *   amax = max |v| over B; scale = 1 if amax == 0 else fp32(amax / 448);
 *   code = OCP E4M3FN(fp32(v / scale)) rounded to nearest even, saturating
 *   at +-448, subnormals kept, -0 and tiny negatives -> 0x80; an all-zero
 *   block has every code +0.  A code stands for code * scale.
 * Block shapes: 1 x 128 along the contraction for activations and
 * gradients (xp, h, dO, da|db), 128 x 128 tiles for expert weights, and for
 * the weight-gradient products (contraction over an expert's rows) 128
 * consecutive rows of one expert per column, the expert's last block short.
 * The GEMMs accumulate in fp32: each 128-long block product is added times
 * the product of its two scales.  Outputs are bf16.  d and f must be
 * multiples of 128; e4m3 layers have no shared expert.
 */

/* Quantised expert weights as written by moe_quantize_weights. */
typedef struct moe_e4m3_weights {
  const uint8_t *W1, *W3, *W2;    /* codes [E][d][f], [E][d][f], [E][f][d] */
  const uint8_t *W1t, *W3t, *W2t; /* not read (may be NULL): the products take every weight in the
                                     orientation above, the forward ones MN-contiguous */
  const float *W1s, *W3s, *W2s;   /* tile scales [E][d/128][f/128] (W1, W3), [E][f/128][d/128] (W2) */
} moe_e4m3_weights;

/*
 * moe_quantize_rows -- 1 x 128 blocks along each row of src [rows][cols]
 * (src_dtype MOE_BF16 or MOE_F32, cols a multiple of 128):
 *   codes  out uint8 [rows][cols];  scales out fp32 [rows][cols/128].
 */
int moe_quantize_rows(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                      uint8_t* codes, float* scales, void* stream);

/*
 * moe_quantize_weights -- 128 x 128 tiles of E fp32 matrices W [E][R][C]
 * (R, C multiples of 128):
 *   codes   out uint8 [E][R][C];
 *   codes_t out uint8 [E][C][R], the same codes transposed (may be NULL);
 *   scales  out fp32 [E][R/128][C/128].
 * For a layer: W1 and W3 with (R, C) = (d, f), W2 with (f, d).
 */
int moe_quantize_weights(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                         uint8_t* codes_t, float* scales, void* stream);

/* Number of 128-row blocks that P rows over E experts can need at most
 * (P/128 + E); the token-block buffers below are sized with it. */
int64_t moe_token_block_capacity(int64_t P, int64_t E);

/*
 * moe_quantize_token_blocks -- the weight-gradient operand blocks: for every
 * expert e (rows offsets[e] .. offsets[e+1]-1 of a [P][C] matrix) and each
 * of its 128-row blocks b (the last one short), one block per column.
 * Row r of the matrix is row src_row[r] of src (src_row NULL: row r), src
 * bf16 [.][C], C a multiple of 128.  With cap = moe_token_block_capacity:
 *   blk     out int32 [E+1]: first block of each expert, blk[E] = blocks used;
 *   codes   out uint8 [P][C]: the codes of row r in row r (row-major, the
 *           matrix's own layout; the weight-gradient GEMMs read them
 *           MN-contiguous);
 *   scales  out fp32 [cap][C]: scale of the expert's block j (rows
 *           offsets[e] + 128 j ..) and column c at row blk[e] + j; rows from
 *           blk[E] on are not written.
 */
int moe_quantize_token_blocks(const int32_t* offsets, int64_t E, int64_t P, const void* src,
                              const int32_t* src_row, int64_t C, int32_t* blk, uint8_t* codes,
                              float* scales, void* stream);

/*
 * moe_quantize_token_blocks_with_rows -- moe_quantize_token_blocks and, in
 * the same pass over the matrix, moe_quantize_rows of its rows: row_codes
 * uint8 [P][C] and row_scales fp32 [P][C/128], bit-identical to
 * moe_quantize_rows (the backward's dO and [da db] feed both a data gradient
 * and a weight gradient, German §2 E / French §2 E).  Arguments and errors as
 * moe_quantize_token_blocks; row_codes and row_scales must not be NULL.
 */
int moe_quantize_token_blocks_with_rows(const int32_t* offsets, int64_t E, int64_t P,
                                        const void* src, const int32_t* src_row, int64_t C,
                                        int32_t* blk, uint8_t* codes, float* scales,
                                        uint8_t* row_codes, float* row_scales, void* stream);

/*
 * moe_permute_e4m3 -- moe_permute for rows of e4m3 codes: codes [T][d] and
 * their scales [T][d/128] (from moe_quantize_rows of x) are copied bit for
 * bit to dst_codes [P][d] and dst_scales [P][d/128] at row row_of[t][j];
 * build_map and the map arguments as in moe_permute (quantising before the
 * permutation gives the same rows as after it, as scales are per row).
 */
int moe_permute_e4m3(const moe_shape* sh, const uint8_t* codes, const float* scales,
                     const int32_t* topk_idx, int build_map, int32_t* counts, int32_t* offsets,
                     int32_t* row_of, int32_t* token_of, uint8_t* dst_codes, float* dst_scales,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_fwd_e4m3 -- moe_grouped_gemm_fwd with e4m3 operands:
 * [a|b] = xp W{1,3} from xpq [P][d] / xps [P][d/128] and the weight codes;
 * ab and h = silu(a) * b are stored bf16; h is quantised (1 x 128 along f)
 * into the workspace and o = h W2 is stored bf16.  sh->dtype == MOE_E4M3;
 * ws_bytes >= moe_workspace_bytes(sh, MOE_WS_GEMM_FWD).
 */
int moe_grouped_gemm_fwd_e4m3(const moe_shape* sh, const int32_t* offsets, const uint8_t* xpq,
                              const float* xps, const moe_e4m3_weights* w, void* ab, void* h,
                              void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_bwd_e4m3 -- moe_grouped_gemm_bwd with e4m3 operands.
 * dO (bf16 [P][d]) is quantised 1 x 128 along d; dab = [da|db] is stored
 * bf16 and quantised 1 x 128 along 2f for dXp = da W1^T + db W3^T; the
 * weight gradients take token blocks of h, dO, dab and of the permuted x
 * (row r is x[token_of[r]], x bf16 [T][d]).  All outputs bf16.
 * ws_bytes >= moe_workspace_bytes(sh, MOE_WS_GEMM_BWD).
 */
int moe_grouped_gemm_bwd_e4m3(const moe_shape* sh, const int32_t* offsets,
                              const int32_t* token_of, const void* x, const void* ab,
                              const void* h, const void* dO, const moe_e4m3_weights* w, void* dab,
                              void* dXp, void* dW1, void* dW3, void* dW2, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Router gradient and load-balancing loss
 * ----------------------------------------
 * The pages fuse routing, permutation and auxiliary-loss computations into
 * few kernels (German technical summary, section 2 D "Kernel Fusion";
 * Spanish summary, section 2.3 C) without stating a formula.  Readings:
 *  - y[t] = sum_j p[t][j] o[row_of[t][j]] with p the softmax over the k
 *    selected logits, so dp[t][j] = <dY[t], o[row_of[t][j]]> and
 *    dlogits[t][topk_idx[t][j]] = p_j (dp_j - sum_i p_i dp_i), 0 for the
 *    experts not selected;
 *  - L = alpha E sum_e f_e P_e, f_e = counts[e] / (T k), P_e = mean over
 *    tokens of the softmax over all E logits; counts are held constant:
 *    dL/dlogits[t] = s[t] (g - <g, s[t]>), g_e = alpha E f_e / T.
 */

/*
 * moe_aux_loss -- *loss (device fp32 scalar) = L above, from the router
 * logits [T][E] and counts [E] (from moe_permute).  ws_bytes >=
 * moe_workspace_bytes(sh with this T and E, MOE_WS_AUX_LOSS).  Deterministic.
 */
int moe_aux_loss(const float* logits, int64_t T, int64_t E, int64_t k, const int32_t* counts,
                 float alpha, float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_aux / moe_aux_loss_final -- moe_route fused with the first half
 * of moe_aux_loss (the pages fuse routing with the auxiliary-loss
 * computation: German technical summary, section 2 D).  moe_route_aux writes
 * topk_idx and topk_prob bit-identical to moe_route and, into ws (ws_bytes >=
 * moe_workspace_bytes(sh with this T and E, MOE_WS_AUX_LOSS)), the softmax
 * column sums of each 32-token block; once the permutation has produced the
 * counts, moe_aux_loss_final (the same ws, T, E, k) writes *loss, bit-
 * identical to moe_aux_loss on the same logits and counts.  One kernel fewer
 * than moe_route followed by moe_aux_loss.  Errors as moe_aux_loss.
 */
int moe_route_aux(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* topk_idx,
                  float* topk_prob, void* ws, size_t ws_bytes, void* stream);
int moe_aux_loss_final(const void* ws, int64_t T, int64_t E, int64_t k, const int32_t* counts,
                       float alpha, float* loss, void* stream);

/*
 * moe_combine_bwd -- the backward of the weighted combine with the
 * probability gradient: dO[row_of[t][j]] = round(p[t][j] dY[t]) (exactly
 * moe_permute's scaled form) and dprob [T][k] fp32 = <dY[t], o[row_of[t][j]]>
 * with o [P][d] the expert outputs of the forward (sh->dtype; bf16 for
 * e4m3 layers).  d * element bytes must be at most 32768.
 */
int moe_combine_bwd(const moe_shape* sh, const void* dY, const void* o, const int32_t* row_of,
                    const float* topk_prob, void* dO, float* dprob, void* stream);

/*
 * moe_route_bwd -- dlogits [T][E] fp32: the top-k softmax Jacobian applied to
 * dprob, plus aux_scale * dL/dlogits of the load-balancing loss (skipped when
 * counts is NULL or alpha or aux_scale is 0).  logits, topk_idx, topk_prob
 * as in moe_route.  The Jacobian term is evaluated as
 * p_j sum_i p_i (dp_j - dp_i), which keeps its relative accuracy when one
 * probability is close to 1.
 */
int moe_route_bwd(const float* logits, int64_t T, int64_t E, int64_t k, const int32_t* topk_idx,
                  const float* topk_prob, const float* dprob, const int32_t* counts, float alpha,
                  float aux_scale, float* dlogits, void* stream);

/*
 * Memory-efficient permutation
 * -----------------------------
 * The pages reorder the routing weights algebraically so that the
 * permutation keeps no redundant intermediates ("Scalable Training of
 * Mixture-of-Experts Models with Megatron Core", German technical summary,
 * section 2 B, memory; Spanish summary, section 2.3 A).  Reading: W2 is
 * linear, so p (h W2) = (p h) W2; the probability is applied to h in the fc1
 * epilogue, the combine is an unweighted sum, and the backward needs neither
 * the expert outputs o nor a scaled dO: with dh' = dY[t] W2^T (unscaled
 * rows), dh = p dh' and dp = <h, dh'>, taken in the fc2 dgrad epilogue.
 * Results equal the plain layer's up to rounding.  The stand-alone row-scaled
 * GEMM calls below are bf16; e4m3 and MXFP8 layers take the same form through
 * moe_layer_fwd / moe_layer_bwd (io->memory_efficient).
 */

/*
 * moe_row_probs -- row_prob[row_of[t][j]] = topk_prob[t][j]: each permuted
 * row's routing probability ([P] fp32).
 */
int moe_row_probs(const moe_shape* sh, const int32_t* row_of, const float* topk_prob,
                  float* row_prob, void* stream);

/*
 * moe_grouped_gemm_fwd_rowscaled -- as moe_grouped_gemm_fwd, but h =
 * row_prob[r] * silu(a) * b, so o = h W2 is already weighted (combine with
 * moe_unpermute and topk_prob = NULL).  bf16 only (MOE_ERR_UNSUPPORTED else).
 */
int moe_grouped_gemm_fwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const void* xp,
                                   const void* W1, const void* W3, const void* W2,
                                   const float* row_prob, void* ab, void* h, void* o,
                                   void* stream);

/*
 * moe_grouped_gemm_bwd_rowscaled -- backward of the row-scaled forward: dO
 * [P][d] is the UNSCALED permuted upstream gradient (moe_permute without
 * row_scale), h the p-scaled h of the forward, or, when recompute_h != 0, a
 * [P][f] buffer that the call first fills with p * silu(a) * b recomputed
 * from ab (so the forward's h need not be kept).  Writes dab, dXp, dW1, dW3,
 * dW2 as moe_grouped_gemm_bwd, and, when dprob is not NULL, the probability
 * gradient <silu(a_r) b_r, dO_r W2^T> of each permuted row r: dprob [P] in
 * row order when row_of is NULL, else dprob [T][k] with
 * dprob[t][j] = that of row row_of[t][j].  ws_bytes >= moe_workspace_bytes(sh,
 * MOE_WS_GEMM_BWD_ROWSCALED) (per-row partials of the dot product).
 */
int moe_grouped_gemm_bwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const void* xp,
                                   const void* ab, void* h, int32_t recompute_h, const void* dO,
                                   const void* W1, const void* W3, const void* W2,
                                   const float* row_prob, void* dab, void* dXp, void* dW1,
                                   void* dW3, void* dW2, const int32_t* row_of, float* dprob,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP8 expert GEMMs
 * ------------------
 * The pages run the Blackwell results in MXFP8 (French summary, section 2 E;
 * Spanish summary, section 2.4) and name it without a definition; the
 * storage is the OCP Microscaling one.  Every block of 32 consecutive values
 * along a product's contraction axis has one scale 2^s, stored as the E8M0
 * byte s + 127, with s the smallest integer such that max|v| <= 448 * 2^s
 * (the scale rounded up, so nothing saturates; s clamped to [-127, 127]; an
 * all-zero block has s = 0 and +0 codes); codes are E4M3FN(v * 2^-s), round
 * to nearest even.  This scale rule departs from the OCP MX v1.0 reference
 * conversion (s = floor(log2 max|v|) - 8 with elements above 448 clamped),
 * which can clip a block's largest element by up to 12.5 %.  gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes one E8M0
 * scale per lane, which is one 32-value block of one row, so the scales go
 * straight into the matrix instruction.  Scale bytes are stored row-major next
 * to the codes they scale:
 *  - activation rows [rows][K] -> bytes [rows][K/32];
 *  - each weight matrix in both orientations (the blocks of the two differ):
 *    codes [E][R][C] with row-block bytes [E][R][C/32] (read by the
 *    data-gradient products), and transposed codes [E][C][R] with
 *    column-block bytes [E][C][R/32] (read by the forward products);
 *  - weight-gradient operands as moe_quantize_token_blocks lays them out
 *    (codes [P][C]), with bytes [cap][C][4] (byte g of word (b, c): rows
 *    32 g.. of 128-row block b; 32-row blocks restart at each expert).
 * Shapes: d, f multiples of 128, no shared expert.
 */

/* Quantised expert weights as written by moe_quantize_weights_mx. */
typedef struct moe_mx_weights {
  const uint8_t *W1, *W3, *W2;       /* codes [E][d][f], [E][d][f], [E][f][d] */
  const uint8_t *W1t, *W3t, *W2t;    /* transposed codes [E][f][d], [E][f][d], [E][d][f] */
  const uint8_t *W1s, *W3s, *W2s;    /* row-block bytes [E][d][f/32], .., [E][f][d/32] */
  const uint8_t *W1ts, *W3ts, *W2ts; /* column-block bytes [E][f][d/32], .., [E][d][f/32] */
} moe_mx_weights;

/* moe_quantize_rows_mx -- 1 x 32 blocks along each row of src [rows][cols]
 * (MOE_BF16 or MOE_F32, cols a multiple of 32): codes [rows][cols], scale
 * bytes [rows][cols/32]. */
int moe_quantize_rows_mx(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                         uint8_t* codes, uint8_t* scales, void* stream);

/* moe_quantize_weights_mx -- both orientations of E fp32 matrices W [E][R][C]
 * (R, C multiples of 128): codes [E][R][C] + bytes [E][R][C/32], codes_t
 * [E][C][R] + bytes [E][C][R/32]; one pass over W. */
int moe_quantize_weights_mx(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                            uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, void* stream);

/* moe_quantize_token_blocks_mx -- as moe_quantize_token_blocks, with 32-row
 * scale blocks: codes [P][C], scale bytes [capacity][C][4] (the four 32-row
 * blocks of each 128-row block and column in one word); 32-row blocks with
 * no rows have s = 0. */
int moe_quantize_token_blocks_mx(const int32_t* offsets, int64_t E, int64_t P, const void* src,
                                 const int32_t* src_row, int64_t C, int32_t* blk,
                                 uint8_t* codes, uint8_t* scales, void* stream);

/* moe_quantize_token_blocks_with_rows_mx -- moe_quantize_token_blocks_mx and,
 * in the same pass, moe_quantize_rows_mx of its rows: row_codes uint8 [P][C],
 * row_scales E8M0 bytes [P][C/32], bit-identical to moe_quantize_rows_mx. */
int moe_quantize_token_blocks_with_rows_mx(const int32_t* offsets, int64_t E, int64_t P,
                                           const void* src, const int32_t* src_row, int64_t C,
                                           int32_t* blk, uint8_t* codes, uint8_t* scales,
                                           uint8_t* row_codes, uint8_t* row_scales, void* stream);

/* moe_permute_mx -- moe_permute_e4m3 for MXFP8 rows: codes [T][d] and scale
 * bytes [T][d/32] moved to the permuted order (bit copies). */
int moe_permute_mx(const moe_shape* sh, const uint8_t* codes, const uint8_t* scales,
                   const int32_t* topk_idx, int build_map, int32_t* counts, int32_t* offsets,
                   int32_t* row_of, int32_t* token_of, uint8_t* dst_codes, uint8_t* dst_scales,
                   void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_gemm_fwd_mx / moe_grouped_gemm_bwd_mx -- the e4m3 calls' MXFP8
 * counterparts (sh->dtype == MOE_MXFP8; xps are scale bytes [P][d/32]); the
 * same workspace sizes (MOE_WS_GEMM_FWD / MOE_WS_GEMM_BWD). */
int moe_grouped_gemm_fwd_mx(const moe_shape* sh, const int32_t* offsets, const uint8_t* xpq,
                            const uint8_t* xps, const moe_mx_weights* w, void* ab, void* h,
                            void* o, void* ws, size_t ws_bytes, void* stream);
int moe_grouped_gemm_bwd_mx(const moe_shape* sh, const int32_t* offsets, const int32_t* token_of,
                            const void* x, const void* ab, const void* h, const void* dO,
                            const moe_mx_weights* w, void* dab, void* dXp, void* dW1, void* dW3,
                            void* dW2, void* ws, size_t ws_bytes, void* stream);

/* moe_probe_mfma -- measurement helper, not a step of the layer: the dense
 * matrix-core rate and the shader clock this GPU sustains under MFMAs alone,
 * the ceiling against which the grouped GEMMs' rates can be read (published
 * peaks assume the peak clock; the chip clocks lower under a sustained
 * matrix-core load).  Launches, on `stream`, 8 blocks of 256 threads per
 * compute unit; every wavefront runs `iters` (1 .. 2^24) rounds of 8
 * independent MFMAs on register operands, v_mfma_f32_16x16x32_bf16 for
 * dtype = MOE_BF16 or v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 codes for
 * MOE_E4M3 (other dtypes: MOE_ERR_UNSUPPORTED).
 *   ticks    device, 2 x uint64, written by the kernel: the shader-clock
 *            cycles and the wall-clock ticks one wavefront's loop took;
 *   sink     device, 1 float, written only in the unlikely case that the
 *            folded results equal a sentinel (keeps the MFMAs alive);
 *   flops    host: the launch's MFMA flop count (2 per multiply-add);
 *   wall_khz host: the wall-clock tick rate, so clock = ticks[0] /
 *            (ticks[1] / (wall_khz * 1e3)).
 * The rate is flops / the launch's duration measured by the caller on
 * `stream`.  Returns MOE_ERR_INVALID for null pointers or iters outside the
 * range, MOE_ERR_HIP if the device cannot be queried or the launch fails. */
int moe_probe_mfma(int dtype, int64_t iters, unsigned long long* ticks, float* sink,
                   int64_t* flops, int64_t* wall_khz, void* stream);

/* Bytes of workspace the call `kind` needs for shape sh (0 if none). */
size_t moe_workspace_bytes(const moe_shape* sh, int kind);

/* Static, NUL-terminated name of a moe_status value. */
const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TRE_MOE_H */
