// C entry points: argument validation, workspace carving and launch sequences.
// Every call validates its arguments before enqueuing anything, enqueues on
// the caller's stream only, and never synchronises, allocates or prints.
#include "common.h"
#include "internal.h"

using namespace tre;

namespace {

constexpr int64_t kMaxE = 256;

__global__ void fill_offsets_kernel(int32_t* off, int32_t T) {
  if (threadIdx.x == 0) { off[0] = 0; off[1] = T; }
}

int elem_bytes(const moe_shape* sh) { return sh->dtype == MOE_F32 ? 4 : 2; }

// Shape checks shared by every call.  Returns MOE_OK or an error code.
int check_shape(const moe_shape* sh) {
  if (!sh) return MOE_ERR_INVALID;
  if (sh->T < 1 || sh->d < 1 || sh->E < 1 || sh->k < 1 || sh->f < 1 || sh->f_shared < 0)
    return MOE_ERR_INVALID;
  if (sh->k > sh->E || sh->reserved != 0) return MOE_ERR_INVALID;
  if (sh->dtype != MOE_F32 && sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (sh->E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (sh->T * sh->k >= ((int64_t)1 << 31) || sh->d >= (1 << 30) || sh->f >= (1 << 30) ||
      sh->f_shared >= (1 << 30))
    return MOE_ERR_UNSUPPORTED;
  // 16-byte row moves
  if ((sh->d * elem_bytes(sh)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_gemm_dims(const moe_shape* sh, int64_t f) {
  if (sh->dtype == MOE_BF16 && (sh->d % 128 != 0 || f % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int run_gemm(const moe_shape* sh, GemmOp op, const GemmArgs& a, hipStream_t s) {
  return sh->dtype == MOE_F32 ? gemm_f32_launch(op, a, s) : gemm_bf16_launch(op, a, s);
}

GemmArgs expert_args(const moe_shape* sh, const int32_t* offsets) {
  GemmArgs a = {};
  a.offsets = offsets;
  a.E = (int)sh->E;
  a.d = (int)sh->d;
  a.f = (int)sh->f;
  a.P = (int)(sh->T * sh->k);
  return a;
}

// The shared expert is a one-group grouped GEMM over all T token rows.
GemmArgs shared_args(const moe_shape* sh, const int32_t* offsets2) {
  GemmArgs a = {};
  a.offsets = offsets2;
  a.E = 1;
  a.d = (int)sh->d;
  a.f = (int)sh->f_shared;
  a.P = (int)sh->T;
  return a;
}

int fwd_sequence(const moe_shape* sh, GemmArgs a, hipStream_t s) {
  int st = run_gemm(sh, OP_FC1_FWD, a, s);
  if (st) return st;
  return run_gemm(sh, OP_FC2_FWD, a, s);
}

int bwd_sequence(const moe_shape* sh, GemmArgs a, hipStream_t s) {
  int st;
  if ((st = run_gemm(sh, OP_FC2_DGRAD, a, s))) return st;
  a.dab = a.dab_out;
  if ((st = run_gemm(sh, OP_FC1_DGRAD, a, s))) return st;
  if ((st = run_gemm(sh, OP_FC2_WGRAD, a, s))) return st;
  return run_gemm(sh, OP_FC1_WGRAD, a, s);
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(const moe_shape* sh, int kind) {
  if (check_shape(sh) != MOE_OK) return 0;
  switch (kind) {
    case MOE_WS_PERMUTE: return permute_ws_bytes(sh->T, sh->E);
    case MOE_WS_GEMM_FWD:
    case MOE_WS_GEMM_BWD: return 0;
    case MOE_WS_LAYER_FWD: return permute_ws_bytes(sh->T, sh->E) + 256;
    case MOE_WS_LAYER_BWD: return 256;
  }
  return 0;
}

int moe_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* topk_idx,
              float* topk_prob, void* stream) {
  if (!logits || !topk_idx || !topk_prob) return MOE_ERR_INVALID;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T * k >= ((int64_t)1 << 31) || T * E >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  return route_launch(logits, (int)T, (int)E, (int)k, topk_idx, topk_prob, (hipStream_t)stream);
}

int moe_permute(const moe_shape* sh, const void* src, const int32_t* topk_idx,
                const float* row_scale, int build_map, int32_t* counts, int32_t* offsets,
                int32_t* row_of, int32_t* token_of, void* dst, void* ws, size_t ws_bytes,
                void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (!src || !dst || !row_of) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  if (build_map) {
    if (!topk_idx || !counts || !offsets || !token_of) return MOE_ERR_INVALID;
    if (!ws || ws_bytes < permute_ws_bytes(sh->T, sh->E)) return MOE_ERR_WORKSPACE;
    st = permute_map_launch(topk_idx, (int)sh->T, (int)sh->E, (int)sh->k, counts, offsets, row_of,
                            token_of, ws, s);
    if (st) return st;
  }
  return permute_rows_launch(src, row_of, row_scale, (int)sh->T, (int)sh->k, (int)sh->d,
                             elem_bytes(sh), dst, s);
}

int moe_unpermute(const moe_shape* sh, const void* src, const int32_t* row_of,
                  const float* topk_prob, const void* add, void* dst, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (!src || !row_of || !dst) return MOE_ERR_INVALID;
  return unpermute_launch(src, row_of, topk_prob, add, (int)sh->T, (int)sh->k, (int)sh->d,
                          elem_bytes(sh), dst, (hipStream_t)stream);
}

int moe_grouped_gemm_fwd(const moe_shape* sh, const int32_t* offsets, const void* xp,
                         const void* W1, const void* W3, const void* W2, void* ab, void* h,
                         void* o, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->f))) return st;
  if (!offsets || !xp || !W1 || !W3 || !W2 || !ab || !h || !o) return MOE_ERR_INVALID;
  GemmArgs a = expert_args(sh, offsets);
  a.xp = xp; a.W1 = W1; a.W3 = W3; a.W2 = W2;
  a.ab_out = ab; a.h_out = h; a.h = h; a.o_out = o;
  return fwd_sequence(sh, a, (hipStream_t)stream);
}

int moe_grouped_gemm_bwd(const moe_shape* sh, const int32_t* offsets, const void* xp,
                         const void* ab, const void* h, const void* dO, const void* W1,
                         const void* W3, const void* W2, void* dab, void* dXp, void* dW1,
                         void* dW3, void* dW2, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->f))) return st;
  if (!offsets || !xp || !ab || !h || !dO || !W1 || !W3 || !W2 || !dab || !dXp || !dW1 || !dW3 ||
      !dW2)
    return MOE_ERR_INVALID;
  GemmArgs a = expert_args(sh, offsets);
  a.xp = xp; a.ab = ab; a.h = h; a.dO = dO; a.W1 = W1; a.W3 = W3; a.W2 = W2;
  a.dab_out = dab; a.dXp_out = dXp; a.dW1 = dW1; a.dW3 = dW3; a.dW2 = dW2;
  return bwd_sequence(sh, a, (hipStream_t)stream);
}

int moe_layer_fwd(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                  void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->f))) return st;
  if (sh->f_shared && (st = check_gemm_dims(sh, sh->f_shared))) return st;
  if (!io || !io->logits || !io->x || !io->W1 || !io->W3 || !io->W2 || !io->topk_idx ||
      !io->topk_prob || !io->counts || !io->offsets || !io->row_of || !io->token_of || !io->xp ||
      !io->ab || !io->h || !io->o || !io->y)
    return MOE_ERR_INVALID;
  if (sh->f_shared &&
      (!io->Ws1 || !io->Ws3 || !io->Ws2 || !io->s_ab || !io->s_h || !io->ys))
    return MOE_ERR_INVALID;
  const size_t pws = permute_ws_bytes(sh->T, sh->E);
  if (!ws || ws_bytes < pws + 256) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;

  if ((st = moe_route(io->logits, sh->T, sh->E, sh->k, io->topk_idx, io->topk_prob, stream)))
    return st;
  if ((st = moe_permute(sh, io->x, io->topk_idx, nullptr, 1, io->counts, io->offsets, io->row_of,
                        io->token_of, io->xp, ws, pws, stream)))
    return st;
  if ((st = moe_grouped_gemm_fwd(sh, io->offsets, io->xp, io->W1, io->W3, io->W2, io->ab, io->h,
                                 io->o, nullptr, 0, stream)))
    return st;
  const void* add = nullptr;
  if (sh->f_shared) {
    int32_t* off2 = (int32_t*)((char*)ws + pws);
    fill_offsets_kernel<<<1, 64, 0, s>>>(off2, (int32_t)sh->T);
    TRE_LAUNCH_CHECK();
    GemmArgs a = shared_args(sh, off2);
    a.xp = io->x; a.W1 = io->Ws1; a.W3 = io->Ws3; a.W2 = io->Ws2;
    a.ab_out = io->s_ab; a.h_out = io->s_h; a.h = io->s_h; a.o_out = io->ys;
    if ((st = fwd_sequence(sh, a, s))) return st;
    add = io->ys;
  }
  return moe_unpermute(sh, io->o, io->row_of, io->topk_prob, add, io->y, stream);
}

int moe_layer_bwd(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                  void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->f))) return st;
  if (sh->f_shared && (st = check_gemm_dims(sh, sh->f_shared))) return st;
  if (!io || !io->dY || !io->W1 || !io->W3 || !io->W2 || !io->topk_prob || !io->offsets ||
      !io->row_of || !io->xp || !io->ab || !io->h || !io->dO || !io->dab || !io->dXp || !io->dX ||
      !io->dW1 || !io->dW3 || !io->dW2)
    return MOE_ERR_INVALID;
  if (sh->f_shared && (!io->x || !io->Ws1 || !io->Ws3 || !io->Ws2 || !io->s_ab || !io->s_h ||
                       !io->s_dab || !io->dXs || !io->dWs1 || !io->dWs3 || !io->dWs2))
    return MOE_ERR_INVALID;
  if (!ws || ws_bytes < 256) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;

  // dO[row_of[t][j]] = p[t][j] * dY[t]
  if ((st = moe_permute(sh, io->dY, nullptr, io->topk_prob, 0, nullptr, nullptr, io->row_of,
                        nullptr, io->dO, nullptr, 0, stream)))
    return st;
  if ((st = moe_grouped_gemm_bwd(sh, io->offsets, io->xp, io->ab, io->h, io->dO, io->W1, io->W3,
                                 io->W2, io->dab, io->dXp, io->dW1, io->dW3, io->dW2, nullptr, 0,
                                 stream)))
    return st;
  const void* add = nullptr;
  if (sh->f_shared) {
    int32_t* off2 = (int32_t*)ws;
    fill_offsets_kernel<<<1, 64, 0, s>>>(off2, (int32_t)sh->T);
    TRE_LAUNCH_CHECK();
    GemmArgs a = shared_args(sh, off2);
    a.xp = io->x; a.ab = io->s_ab; a.h = io->s_h; a.dO = io->dY;
    a.W1 = io->Ws1; a.W3 = io->Ws3; a.W2 = io->Ws2;
    a.dab_out = io->s_dab; a.dXp_out = io->dXs;
    a.dW1 = io->dWs1; a.dW3 = io->dWs3; a.dW2 = io->dWs2;
    if ((st = bwd_sequence(sh, a, s))) return st;
    add = io->dXs;
  }
  return moe_unpermute(sh, io->dXp, io->row_of, nullptr, add, io->dX, stream);
}

}  // extern "C"
