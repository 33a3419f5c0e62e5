// Internal launchers shared between the library's translation units.  Every
// launcher assumes its arguments were validated by the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tre {

// route.hip
int route_launch(const float* logits, int T, int E, int k, int32_t* idx, float* prob,
                 hipStream_t s);
// routing plus the load-balancing loss's per-32-token softmax column sums
// (partial [ceil(T/32)][E], the layout aux_final_launch reads)
int route_aux_launch(const float* logits, int T, int E, int k, int32_t* idx, float* prob,
                     float* partial, hipStream_t s);

// permute.hip
size_t permute_ws_bytes(int64_t T, int64_t E);
// the file-scope scratch of the allocation-free map: its size, and its device
// address on the current device (looked up once per device)
size_t permute_scratch_bytes();
int permute_scratch(void** ptr);
int permute_map_launch(const int32_t* idx, int T, int E, int k, int32_t* counts,
                       int32_t* offsets, int32_t* row_of, int32_t* token_of, void* ws,
                       hipStream_t s);
// elem_bytes: 4 (fp32) or 2 (bf16); row_scale may be NULL (bit copy)
int permute_rows_launch(const void* src, const int32_t* row_of, const float* row_scale, int T,
                        int k, int d, int elem_bytes, void* dst, hipStream_t s);
int unpermute_launch(const void* src, const int32_t* row_of, const float* prob, const void* add,
                     int T, int k, int d, int elem_bytes, void* dst, hipStream_t s);

// router_grad.hip: router backward and load-balancing loss
int combine_bwd_launch(const void* dY, const void* o, const int32_t* row_of, const float* prob,
                       int T, int k, int d, int elem_bytes, void* dO, float* dprob, hipStream_t s);
int route_bwd_launch(const float* logits, int T, int E, int k, const int32_t* idx,
                     const float* prob, const float* dprob, const int32_t* counts, float alpha,
                     float aux_scale, float* dlogits, hipStream_t s);
size_t aux_ws_bytes(int64_t T, int64_t E);
// row-scaled products: row_prob[row_of[i]] = prob[i] (i < n = T*k); and
// out[i] = sum over the N-tiles of part[r][.] with r = row_of[i] (or i)
int row_probs_launch(const int32_t* row_of, const float* prob, int n, float* row_prob,
                     hipStream_t s);
int dp_rows_launch(const float* part, int NT, const int32_t* row_of, int n, float* out,
                   hipStream_t s);
int aux_loss_launch(const float* logits, int T, int E, int k, const int32_t* counts, float alpha,
                    float* loss, void* ws, hipStream_t s);
// the loss from the column-sum partials and the counts
int aux_final_launch(const float* partial, int T, int E, int k, const int32_t* counts,
                     float alpha, float* loss, hipStream_t s);

// Grouped-GEMM problem: which of the six expert products to run.
enum GemmOp {
  OP_FC1_FWD = 0,    // [a|b] = xp W{1,3}; saves ab, h = silu(a) b     (M ragged, K = d)
  OP_FC2_FWD = 1,    // o = h W2                                       (M ragged, K = f)
  OP_FC2_DGRAD = 2,  // dH = dO W2^T, epilogue -> dab                  (M ragged, K = d)
  OP_FC1_DGRAD = 3,  // dXp = [da|db] [W1|W3]^T                        (M ragged, K = 2f)
  OP_FC2_WGRAD = 4,  // dW2 = h^T dO                                   (K ragged = rows)
  OP_FC1_WGRAD = 5,  // [dW1|dW3] = xp^T [da|db]                       (K ragged = rows)
};

struct GemmArgs {
  const int32_t* offsets;  // [E+1], device
  int E, d, f, P;          // P = rows of the permuted buffers
  const void* xp;
  const void* h;
  const void* dO;
  const void* ab;          // forward pre-activations [P][2f]
  const void* dab;         // backward [P][2f] (input of dgrad fc1 / wgrad fc1)
  const void* W1;
  const void* W3;
  const void* W2;
  void* ab_out;
  void* h_out;
  void* o_out;
  void* dab_out;
  void* dXp_out;
  void* dW1;
  void* dW3;
  void* dW2;
  // e4m3 products only (gemm_fp8.hip).  Every operand is K-contiguous codes:
  //   ragged-M ops: A = a_q [P][K] with scales a_s [P][K/128]; B = weight
  //     codes laid out [n][k] (b_q, and b_q2 for the W3 half of fc1 products)
  //     with 128x128 block scales b_s, b_s2 as stored by the weight quantiser;
  //   wgrad ops: A = a_q [P][M], B = b_q [P][N], row-major codes of the
  //     permuted rows (MN-contiguous), with one scale per 128-row token block
  //     of an expert and column: a_s [NB][M], b_s [NB][N], the expert's blocks
  //     from row blk[e] on.
  const uint8_t* a_q;
  const float* a_s;
  const uint8_t* b_q;
  const uint8_t* b_q2;
  const float* b_s;
  const float* b_s2;
  const int32_t* blk;  // [E+1] token-block table (wgrad)
  // row-scaled products (probabilities applied before W2), bf16 only: the
  // routing probability of every permuted row, and the fc2 dgrad's partial
  // probability gradients [P][ceil(f/256)]
  const float* row_prob;
  float* dp_part;
  // MXFP8 products (gemm_fp8.hip with E8M0 scales): the same code operands as
  // e4m3, with one scale byte per 32 contraction values, stored row-major per
  // operand row: A rows [.][K/32]; B: the byte array of each weight matrix in
  // the orientation read ([E][n][K/32]; fc1 forward and fc1 dgrad use b_sx2
  // for W3).  Weight gradients: words [NB][M] and [NB][N], the four
  // 32-row scales of each 128-row token block and column.
  const uint8_t* a_sx;
  const uint8_t* b_sx;
  const uint8_t* b_sx2;
  // fused permutation (bf16 and fp32 fc1 forward and fc1 weight gradient):
  // when `gather` (token_of [P]) is set, row r of the permuted input is row
  // gather[r] of gx [gT][d], and xp is not read
  const int32_t* gather;
  const void* gx;
  int gT;
};

// gemm_bf16.hip: MFMA kernels, bf16 in/out, fp32 accumulation
int gemm_bf16_launch(GemmOp op, const GemmArgs& a, hipStream_t s);
// gemm_f32.hip: fp32 kernels
int gemm_f32_launch(GemmOp op, const GemmArgs& a, hipStream_t s);
// gemm_fp8.hip: e4m3 x e4m3 MFMA with fp32 block scales, bf16 outputs
int gemm_fp8_launch(GemmOp op, const GemmArgs& a, hipStream_t s);
// the same products with MXFP8 operands (hardware block-scaled MFMA)
int gemm_mx_launch(GemmOp op, const GemmArgs& a, hipStream_t s);
// Compute units of the current device rounded down to a multiple of 8 (the
// grid of the persistent grouped-GEMM launches), or -1.
int gemm_persistent_blocks();

// quant.hip: e4m3 block quantisers
int quant_rows_launch(const void* src, bool src_f32, int64_t rows, int64_t cols, uint8_t* codes,
                      float* scales, hipStream_t s);
int quant_tiles_launch(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                       uint8_t* codes_t, float* scales, hipStream_t s);
int64_t tokblk_max_blocks(int64_t P, int64_t E);
// MXFP8 quantisers (E8M0 byte scales per 32 values): rows [rows][cols] ->
// codes + bytes [rows][cols/32]; both orientations of expert weights; token
// blocks (32-row scale blocks inside the 128-row blocks of quant_tokblk)
int quant_rows_mx_launch(const void* src, bool src_f32, int64_t rows, int64_t cols,
                         uint8_t* codes, uint8_t* sb, hipStream_t s);
int quant_weights_mx_launch(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                            uint8_t* sb, uint8_t* codes_t, uint8_t* sbt, hipStream_t s);
// (rcodes != NULL: the same pass also writes the rows' 1 x 32 blocks, rcodes
// [P][C] and bytes rsb [P][C/32], as quant_rows_mx_launch would)
int quant_tokblk_mx_launch(const void* src, const int32_t* src_row, const int32_t* offsets,
                           const int32_t* blk, int E, int64_t P, int64_t C, uint8_t* codes,
                           uint8_t* sbt, hipStream_t s, uint8_t* rcodes = nullptr,
                           uint8_t* rsb = nullptr);  // bound on sum_e ceil(m_e / 128)
int tokblk_table_launch(const int32_t* offsets, int E, int32_t* blk, hipStream_t s);
// (rcodes != NULL: the same pass also writes the rows' 1 x 128 blocks, rcodes
// [P][C] and rscales [P][C/128], as quant_rows_launch would)
int quant_tokblk_launch(const void* src, const int32_t* src_row, const int32_t* offsets,
                        const int32_t* blk, int E, int64_t P, int64_t C, uint8_t* codes,
                        float* scales, hipStream_t s, uint8_t* rcodes = nullptr,
                        float* rscales = nullptr);
// permute.hip: rows of e4m3 codes [T][d] and their scales [T][d/128]
int permute_e4m3_launch(const uint8_t* codes, const float* scales, const int32_t* row_of, int T,
                        int k, int d, uint8_t* dst_codes, float* dst_scales, hipStream_t s);

}  // namespace tre
