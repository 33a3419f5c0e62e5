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

// permute.hip
size_t permute_ws_bytes(int64_t T, int64_t E);
int permute_map_launch(const int32_t* idx, int T, int E, int k, int32_t* counts,
                       int32_t* offsets, int32_t* row_of, int32_t* token_of, void* ws,
                       hipStream_t s);
// elem_bytes: 4 (fp32) or 2 (bf16); row_scale may be NULL (bit copy)
int permute_rows_launch(const void* src, const int32_t* row_of, const float* row_scale, int T,
                        int k, int d, int elem_bytes, void* dst, hipStream_t s);
int unpermute_launch(const void* src, const int32_t* row_of, const float* prob, const void* add,
                     int T, int k, int d, int elem_bytes, void* dst, hipStream_t s);

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
};

// gemm_bf16.hip: MFMA kernels, bf16 in/out, fp32 accumulation
int gemm_bf16_launch(GemmOp op, const GemmArgs& a, hipStream_t s);
// gemm_f32.hip: fp32 kernels
int gemm_f32_launch(GemmOp op, const GemmArgs& a, hipStream_t s);

}  // namespace tre
