// C entry points: argument validation, workspace carving and launch sequences.
// Every call validates its arguments before enqueuing anything, enqueues on
// the caller's stream only, and never synchronises, allocates or prints.
#include "common.h"
#include "internal.h"

#include <algorithm>

using namespace tre;

namespace {

constexpr int64_t kMaxE = 256;

__global__ void fill_offsets_kernel(int32_t* off, int32_t T) {
  if (threadIdx.x == 0) { off[0] = 0; off[1] = T; }
}

int elem_bytes(const moe_shape* sh) { return sh->dtype == MOE_F32 ? 4 : 2; }
// e4m3 or MXFP8 expert GEMMs (bf16 activations)
bool is_fp8(const moe_shape* sh) { return sh->dtype == MOE_E4M3 || sh->dtype == MOE_MXFP8; }

// Shape checks shared by every call.  Returns MOE_OK or an error code.
int check_shape(const moe_shape* sh) {
  if (!sh) return MOE_ERR_INVALID;
  if (sh->T < 1 || sh->d < 1 || sh->E < 1 || sh->k < 1 || sh->f < 1 || sh->f_shared < 0)
    return MOE_ERR_INVALID;
  if (sh->k > sh->E || sh->reserved != 0) return MOE_ERR_INVALID;
  if (sh->dtype != MOE_F32 && sh->dtype != MOE_BF16 && sh->dtype != MOE_E4M3 &&
      sh->dtype != MOE_MXFP8)
    return MOE_ERR_UNSUPPORTED;
  if (is_fp8(sh) && sh->f_shared != 0) return MOE_ERR_UNSUPPORTED;
  if (sh->E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (sh->T * sh->k >= ((int64_t)1 << 31) || sh->d >= (1 << 30) || sh->f >= (1 << 30) ||
      sh->f_shared >= (1 << 30))
    return MOE_ERR_UNSUPPORTED;
  // 16-byte row moves
  if ((sh->d * elem_bytes(sh)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Expert GEMM dimensions for `rows` permuted rows (P, or T for the shared
// expert) and FFN width f.  The bf16 kernels address their operands through
// 32-bit buffer ranges and offsets: a weight-gradient tile spans all rows of
// one expert (up to `rows`) of xp / dO ([.][d]) or dab ([.][2f]), and a
// forward or data-gradient tile one expert's d x f weight matrix.  Shapes
// where those byte counts reach 2^32 are refused rather than read wrapped.
int check_gemm_dims(const moe_shape* sh, int64_t rows, int64_t f) {
  if (sh->dtype != MOE_F32 && (sh->d % 128 != 0 || f % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  if (sh->dtype == MOE_BF16) {
    const int64_t lim = (int64_t)1 << 32;
    if (rows * std::max(sh->d, 2 * f) * 2 >= lim || sh->d * f * 2 >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// ---- e4m3 workspaces: consecutive 256-byte aligned regions
struct Carver {
  char* p;
  size_t used = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* r = (T*)(p ? p + used : nullptr);
    used += align_up(bytes, 256);
    return r;
  }
};

struct Fwd8Ws {
  uint8_t* hq;
  float* hs;
};
Fwd8Ws carve_fwd8(const moe_shape* sh, void* ws, size_t* bytes) {
  const size_t P = (size_t)(sh->T * sh->k), f = (size_t)sh->f;
  Carver c{(char*)ws};
  Fwd8Ws w;
  w.hq = c.take<uint8_t>(P * f);
  w.hs = c.take<float>(P * (f / 128) * 4);
  *bytes = c.used;
  return w;
}

struct Bwd8Ws {
  uint8_t *dOq, *dabq, *tokA, *tokB;
  float *dOs, *dabs, *sA, *sB;
  int32_t* blk;
  int64_t cap;
};
Bwd8Ws carve_bwd8(const moe_shape* sh, void* ws, size_t* bytes) {
  const size_t P = (size_t)(sh->T * sh->k), d = (size_t)sh->d, f = (size_t)sh->f;
  const int64_t cap = tokblk_max_blocks((int64_t)P, sh->E);
  const size_t ma = f > d ? f : d, mb = d > 2 * f ? d : 2 * f;
  Carver c{(char*)ws};
  Bwd8Ws w;
  w.cap = cap;
  w.dOq = c.take<uint8_t>(P * d);
  w.dOs = c.take<float>(P * (d / 128) * 4);
  w.dabq = c.take<uint8_t>(P * 2 * f);
  w.dabs = c.take<float>(P * (2 * f / 128) * 4);
  w.blk = c.take<int32_t>((size_t)(sh->E + 1) * 4);
  w.tokA = c.take<uint8_t>(P * ma);
  w.tokB = c.take<uint8_t>(P * mb);
  w.sA = c.take<float>((size_t)cap * ma * 4);
  w.sB = c.take<float>((size_t)cap * mb * 4);
  *bytes = c.used;
  return w;
}

size_t fwd8_ws_bytes(const moe_shape* sh) {
  size_t b;
  carve_fwd8(sh, nullptr, &b);
  return b;
}
size_t bwd8_ws_bytes(const moe_shape* sh) {
  size_t b;
  carve_bwd8(sh, nullptr, &b);
  return b;
}

bool weights_ok(const moe_e4m3_weights* w) {
  // (the transposed codes W1t, W3t, W2t are not read: the forward products take
  // B in the weights' own orientation)
  return w && w->W1 && w->W3 && w->W2 && w->W1s && w->W3s && w->W2s;
}
bool weights_ok(const moe_mx_weights* w) {
  return w && w->W1 && w->W3 && w->W2 && w->W1t && w->W3t && w->W2t && w->W1s && w->W3s &&
         w->W2s && w->W1ts && w->W3ts && w->W2ts;
}

// The weight operands of the fp8 products: codes in both orientations and
// the scales read with each (e4m3: one tile-scale array serves both; MXFP8:
// row-block bytes with W1/W3/W2, column-block bytes with the transposed codes).
struct Wq8 {
  const uint8_t *W1, *W3, *W2, *W1t, *W3t, *W2t;
  const void *s1, *s3, *s2, *s1t, *s3t, *s2t;
};
Wq8 wq8_of(const moe_e4m3_weights* w) {
  return Wq8{w->W1, w->W3, w->W2, w->W1t, w->W3t, w->W2t,
             w->W1s, w->W3s, w->W2s, w->W1s, w->W3s, w->W2s};
}
Wq8 wq8_of(const moe_mx_weights* w) {
  return Wq8{w->W1, w->W3, w->W2, w->W1t, w->W3t, w->W2t,
             w->W1s, w->W3s, w->W2s, w->W1ts, w->W3ts, w->W2ts};
}
void set_a_scales(GemmArgs& a, const void* sc, bool mx) {
  if (mx) a.a_sx = (const uint8_t*)sc; else a.a_s = (const float*)sc;
}
void set_b_scales(GemmArgs& a, const void* sc, const void* sc2, bool mx) {
  if (mx) { a.b_sx = (const uint8_t*)sc; a.b_sx2 = (const uint8_t*)sc2; }
  else { a.b_s = (const float*)sc; a.b_s2 = (const float*)sc2; }
}
int gemm8(GemmOp op, const GemmArgs& a, hipStream_t s, bool mx) {
  return mx ? gemm_mx_launch(op, a, s) : gemm_fp8_launch(op, a, s);
}
int qrows8(const void* src, int64_t rows, int64_t cols, uint8_t* codes, void* sc, hipStream_t s,
           bool mx) {
  return mx ? quant_rows_mx_launch(src, false, rows, cols, codes, (uint8_t*)sc, s)
            : quant_rows_launch(src, false, rows, cols, codes, (float*)sc, s);
}
// token blocks of src (rcodes != NULL: and its row blocks, in the same pass)
int qtok8(const void* src, const int32_t* src_row, const int32_t* offsets, const int32_t* blk,
          int E, int64_t P, int64_t C, uint8_t* codes, void* sc, hipStream_t s, bool mx,
          uint8_t* rcodes = nullptr, void* rsc = nullptr) {
  return mx ? quant_tokblk_mx_launch(src, src_row, offsets, blk, E, P, C, codes, (uint8_t*)sc, s,
                                     rcodes, (uint8_t*)rsc)
            : quant_tokblk_launch(src, src_row, offsets, blk, E, P, C, codes, (float*)sc, s, rcodes,
                                  (float*)rsc);
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

// Where the experts' input rows come from: the permuted copy xp, or (fused
// permutation) row token_of[r] of x, read by fc1 forward and fc1 wgrad.
struct RowSrc {
  const void* xp;
  const int32_t* token_of;
  const void* x;
};
void set_rows(GemmArgs& a, const moe_shape* sh, const RowSrc& r) {
  a.xp = r.xp;
  a.gather = r.token_of;
  a.gx = r.x;
  a.gT = (int)sh->T;
}
RowSrc rows_of(const moe_layer_io* io) {
  return io->fused_permute ? RowSrc{nullptr, io->token_of, io->x} : RowSrc{io->xp, nullptr, nullptr};
}
// Gathered rows: bf16 or fp32, and x's byte range below 2^31 (the bf16
// kernels give rows past an expert's end an offset past that range).
int check_gather(const moe_shape* sh) {
  if (sh->dtype != MOE_F32 && sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (sh->T * sh->d * elem_bytes(sh) >= ((int64_t)1 << 31) - 4096) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
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

int layer_fwd_e4m3(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                   void* stream);
int layer_bwd_e4m3(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                   void* stream);
int layer_aux_loss(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                   void* stream);
int layer_route(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                void* stream);
bool aux_ws_ok(const moe_shape* sh, const moe_layer_io* io, size_t ws_bytes);
int layer_fwd_rowscaled(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                        void* stream);
int layer_bwd_rowscaled(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                        void* stream);
// per-row partials of the row-scaled fc2 dgrad: [P][ceil(f/256)] fp32
size_t dp_part_bytes(const moe_shape* sh) {
  return align_up((size_t)(sh->T * sh->k) * (size_t)((sh->f + 255) / 256) * sizeof(float), 256);
}
int layer_combine_bwd(const moe_shape* sh, const moe_layer_io* io, void* stream);
int fwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const RowSrc& rows, const void* W1,
                  const void* W3, const void* W2, const float* row_prob, void* ab, void* h, void* o,
                  void* stream);
int bwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const RowSrc& rows, const void* ab,
                  void* h, int32_t recompute_h, const void* dO, const void* W1, const void* W3,
                  const void* W2, const float* row_prob, void* dab, void* dXp, void* dW1,
                  void* dW3, void* dW2, const int32_t* row_of, float* dprob, void* ws,
                  void* stream);

// Expert forward of the fp8 products (e4m3 or MXFP8); arguments checked by the caller.
// row_prob != NULL: the memory-efficient form, h = p silu(a) b.
int gemm_fwd8(const moe_shape* sh, const int32_t* offsets, const uint8_t* xpq, const void* xps,
              const Wq8& w, void* ab, void* h, void* o, void* ws, size_t ws_bytes, void* stream,
              bool mx, const float* row_prob = nullptr) {
  int st;
  size_t need;
  Fwd8Ws W = carve_fwd8(sh, ws, &need);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int64_t P = sh->T * sh->k;
  GemmArgs a = expert_args(sh, offsets);
  a.a_q = xpq; set_a_scales(a, xps, mx);
  // B: MXFP8 the transposed codes (its scale blocks run along the contraction);
  // e4m3 the codes in their own orientation, read MN-contiguous
  a.b_q = mx ? w.W1t : w.W1; a.b_q2 = mx ? w.W3t : w.W3; set_b_scales(a, w.s1t, w.s3t, mx);
  a.ab_out = ab; a.h_out = h;
  a.row_prob = row_prob;
  if ((st = gemm8(OP_FC1_FWD, a, s, mx))) return st;
  a.row_prob = nullptr;
  if ((st = qrows8(h, P, sh->f, W.hq, W.hs, s, mx))) return st;
  a.a_q = W.hq; set_a_scales(a, W.hs, mx);
  a.b_q = mx ? w.W2t : w.W2; a.b_q2 = nullptr; set_b_scales(a, w.s2t, nullptr, mx);
  a.o_out = o;
  return gemm8(OP_FC2_FWD, a, s, mx);
}


// Expert backward of the fp8 products (e4m3 or MXFP8); arguments checked by the caller.
// row_prob != NULL: the memory-efficient form (dO unscaled; fc2 dgrad scales
// dh by p and writes its <h, dh'> partials to dp_part; with recompute_h it
// also refills h = p silu(a) b for the fc2 weight gradient).
int gemm_bwd8(const moe_shape* sh, const int32_t* offsets, const int32_t* token_of, const void* x,
              const void* ab, const void* h, const void* dO, const Wq8& w, void* dab, void* dXp,
              void* dW1, void* dW3, void* dW2, void* ws, size_t ws_bytes, void* stream, bool mx,
              const float* row_prob = nullptr, float* dp_part = nullptr, bool recompute_h = false) {
  int st;
  size_t need;
  Bwd8Ws W = carve_bwd8(sh, ws, &need);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const int64_t P = sh->T * sh->k, d = sh->d, f = sh->f, E = sh->E;
  if ((std::max(d, 2 * f) + 256) * 128 * W.cap >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs a = expert_args(sh, offsets);
  // dO and [da db] feed a data gradient (1 x 128 or 1 x 32 row blocks) and a
  // weight gradient (128-row token blocks).  MXFP8: one pass over each writes
  // both (measured: 758 against 816 us of quantisers a step on the skewed
  // shape); e4m3: separate passes (the fused e4m3 pass, with two scale
  // divisions per value and 103 VGPRs, took 310 us where the two took 232).
  // Order: dH = dO W2^T (+ SwiGLU backward -> dab); dW2 = h^T dO; dXp = dab
  // [W1|W3]^T; [dW1|dW3] = xp^T dab (the token-block buffers are reused).
  if ((st = tokblk_table_launch(offsets, (int)E, W.blk, s))) return st;
  a.blk = W.blk;
  auto rows_and_blocks = [&](const void* src, int64_t C, uint8_t* rq, void* rs) -> int {
    if (mx) return qtok8(src, nullptr, offsets, W.blk, (int)E, P, C, W.tokB, W.sB, s, mx, rq, rs);
    int r = qrows8(src, P, C, rq, rs, s, mx);
    return r ? r : qtok8(src, nullptr, offsets, W.blk, (int)E, P, C, W.tokB, W.sB, s, mx);
  };
  if ((st = rows_and_blocks(dO, d, W.dOq, W.dOs))) return st;
  a.a_q = W.dOq; set_a_scales(a, W.dOs, mx); a.b_q = w.W2; set_b_scales(a, w.s2, nullptr, mx);
  a.ab = ab; a.dab_out = dab;
  a.row_prob = row_prob;
  a.dp_part = dp_part;
  a.h_out = row_prob && recompute_h ? (void*)h : nullptr;
  if ((st = gemm8(OP_FC2_DGRAD, a, s, mx))) return st;
  a.row_prob = nullptr;
  a.h_out = nullptr;
  // (h after fc2 dgrad, which refills it in the recompute form)
  if ((st = qtok8(h, nullptr, offsets, W.blk, (int)E, P, f, W.tokA, W.sA, s, mx))) return st;
  a.a_q = W.tokA; set_a_scales(a, W.sA, mx);
  a.b_q = W.tokB; a.b_q2 = nullptr; set_b_scales(a, W.sB, nullptr, mx);
  a.dW2 = dW2;
  if ((st = gemm8(OP_FC2_WGRAD, a, s, mx))) return st;
  if ((st = rows_and_blocks(dab, 2 * f, W.dabq, W.dabs))) return st;
  a.a_q = W.dabq; set_a_scales(a, W.dabs, mx);
  a.b_q = w.W1; a.b_q2 = w.W3; set_b_scales(a, w.s1, w.s3, mx);
  a.dXp_out = dXp;
  if ((st = gemm8(OP_FC1_DGRAD, a, s, mx))) return st;
  if ((st = qtok8(x, token_of, offsets, W.blk, (int)E, P, d, W.tokA, W.sA, s, mx))) return st;
  a.a_q = W.tokA; set_a_scales(a, W.sA, mx);
  a.b_q = W.tokB; a.b_q2 = nullptr; set_b_scales(a, W.sB, nullptr, mx);
  a.dW1 = dW1; a.dW3 = dW3;
  return gemm8(OP_FC1_WGRAD, a, s, mx);
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
  if (is_fp8(sh)) {
    switch (kind) {
      case MOE_WS_AUX_LOSS: return aux_ws_bytes(sh->T, sh->E);
      case MOE_WS_PERMUTE: return permute_ws_bytes(sh->T, sh->E);
      case MOE_WS_GEMM_FWD: return fwd8_ws_bytes(sh);
      case MOE_WS_GEMM_BWD: return bwd8_ws_bytes(sh);
      case MOE_WS_LAYER_FWD: return permute_ws_bytes(sh->T, sh->E) + fwd8_ws_bytes(sh);
      case MOE_WS_LAYER_BWD: return bwd8_ws_bytes(sh);
      case MOE_WS_LAYER_BWD_ROWSCALED: return bwd8_ws_bytes(sh) + dp_part_bytes(sh);
    }
    return 0;
  }
  switch (kind) {
    case MOE_WS_AUX_LOSS: return aux_ws_bytes(sh->T, sh->E);
    case MOE_WS_PERMUTE: return permute_ws_bytes(sh->T, sh->E);
    case MOE_WS_GEMM_BWD_ROWSCALED: return sh->dtype == MOE_BF16 ? dp_part_bytes(sh) : 0;
    case MOE_WS_LAYER_BWD_ROWSCALED: return sh->dtype == MOE_BF16 ? 256 + dp_part_bytes(sh) : 0;
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
  // dst NULL with build_map: the map alone (the fused permutation's experts
  // read x through token_of)
  if (!row_of || (!dst && !build_map) || (dst && !src)) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  if (build_map) {
    if (!topk_idx || !counts || !offsets || !token_of) return MOE_ERR_INVALID;
    if (!ws || ws_bytes < permute_ws_bytes(sh->T, sh->E)) return MOE_ERR_WORKSPACE;
    st = permute_map_launch(topk_idx, (int)sh->T, (int)sh->E, (int)sh->k, counts, offsets, row_of,
                            token_of, ws, s);
    if (st) return st;
  }
  if (!dst) return MOE_OK;
  return permute_rows_launch(src, row_of, row_scale, (int)sh->T, (int)sh->k, (int)sh->d,
                             elem_bytes(sh), dst, s);
}

int moe_permute_noalloc(const moe_shape* sh, const void* src, const int32_t* topk_idx,
                        const float* row_scale, int build_map, int32_t* counts, int32_t* offsets,
                        int32_t* row_of, int32_t* token_of, void* dst, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (!row_of || (!dst && !build_map) || (dst && !src)) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  if (build_map) {
    if (!topk_idx || !counts || !offsets || !token_of) return MOE_ERR_INVALID;
    if (permute_ws_bytes(sh->T, sh->E) > permute_scratch_bytes()) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = permute_scratch(&ws))) return st;
    st = permute_map_launch(topk_idx, (int)sh->T, (int)sh->E, (int)sh->k, counts, offsets, row_of,
                            token_of, ws, s);
    if (st) return st;
  }
  if (!dst) return MOE_OK;
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
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (is_fp8(sh)) return MOE_ERR_UNSUPPORTED;  // moe_grouped_gemm_fwd_e4m3 / _mx
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
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (is_fp8(sh)) return MOE_ERR_UNSUPPORTED;  // moe_grouped_gemm_bwd_e4m3 / _mx
  if (!offsets || !xp || !ab || !h || !dO || !W1 || !W3 || !W2 || !dab || !dXp || !dW1 || !dW3 ||
      !dW2)
    return MOE_ERR_INVALID;
  GemmArgs a = expert_args(sh, offsets);
  a.xp = xp; a.ab = ab; a.h = h; a.dO = dO; a.W1 = W1; a.W3 = W3; a.W2 = W2;
  a.dab_out = dab; a.dXp_out = dXp; a.dW1 = dW1; a.dW3 = dW3; a.dW2 = dW2;
  return bwd_sequence(sh, a, (hipStream_t)stream);
}

int moe_grouped_gemm_fwd_gather(const moe_shape* sh, const int32_t* offsets,
                                const int32_t* token_of, const void* x, const void* W1,
                                const void* W3, const void* W2, void* ab, void* h, void* o,
                                void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f)) || (st = check_gather(sh))) return st;
  if (!offsets || !token_of || !x || !W1 || !W3 || !W2 || !ab || !h || !o) return MOE_ERR_INVALID;
  GemmArgs a = expert_args(sh, offsets);
  set_rows(a, sh, RowSrc{nullptr, token_of, x});
  a.W1 = W1; a.W3 = W3; a.W2 = W2;
  a.ab_out = ab; a.h_out = h; a.h = h; a.o_out = o;
  return fwd_sequence(sh, a, (hipStream_t)stream);
}

int moe_grouped_gemm_bwd_gather(const moe_shape* sh, const int32_t* offsets,
                                const int32_t* token_of, const void* x, const void* ab,
                                const void* h, const void* dO, const void* W1, const void* W3,
                                const void* W2, void* dab, void* dXp, void* dW1, void* dW3,
                                void* dW2, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f)) || (st = check_gather(sh))) return st;
  if (!offsets || !token_of || !x || !ab || !h || !dO || !W1 || !W3 || !W2 || !dab || !dXp ||
      !dW1 || !dW3 || !dW2)
    return MOE_ERR_INVALID;
  GemmArgs a = expert_args(sh, offsets);
  set_rows(a, sh, RowSrc{nullptr, token_of, x});
  a.ab = ab; a.h = h; a.dO = dO; a.W1 = W1; a.W3 = W3; a.W2 = W2;
  a.dab_out = dab; a.dXp_out = dXp; a.dW1 = dW1; a.dW3 = dW3; a.dW2 = dW2;
  return bwd_sequence(sh, a, (hipStream_t)stream);
}

int moe_row_probs(const moe_shape* sh, const int32_t* row_of, const float* topk_prob,
                  float* row_prob, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (!row_of || !topk_prob || !row_prob) return MOE_ERR_INVALID;
  return row_probs_launch(row_of, topk_prob, (int)(sh->T * sh->k), row_prob, (hipStream_t)stream);
}

int moe_grouped_gemm_fwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const void* xp,
                                   const void* W1, const void* W3, const void* W2,
                                   const float* row_prob, void* ab, void* h, void* o,
                                   void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !xp || !W1 || !W3 || !W2 || !row_prob || !ab || !h || !o) return MOE_ERR_INVALID;
  return fwd_rowscaled(sh, offsets, RowSrc{xp, nullptr, nullptr}, W1, W3, W2, row_prob, ab, h, o,
                       stream);
}

int moe_grouped_gemm_bwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const void* xp,
                                   const void* ab, void* h, int32_t recompute_h, const void* dO,
                                   const void* W1, const void* W3, const void* W2,
                                   const float* row_prob, void* dab, void* dXp, void* dW1,
                                   void* dW3, void* dW2, const int32_t* row_of, float* dprob,
                                   void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !xp || !ab || !h || !dO || !W1 || !W3 || !W2 || !row_prob || !dab || !dXp ||
      !dW1 || !dW3 || !dW2)
    return MOE_ERR_INVALID;
  if (!ws || ws_bytes < dp_part_bytes(sh)) return MOE_ERR_WORKSPACE;
  return bwd_rowscaled(sh, offsets, RowSrc{xp, nullptr, nullptr}, ab, h, recompute_h, dO, W1, W3,
                       W2, row_prob, dab, dXp, dW1, dW3, dW2, row_of, dprob, ws, stream);
}

}  // extern "C"

namespace {

// Row-scaled expert forward and backward (bf16; arguments checked by the caller).
int fwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const RowSrc& rows, const void* W1,
                  const void* W3, const void* W2, const float* row_prob, void* ab, void* h, void* o,
                  void* stream) {
  GemmArgs a = expert_args(sh, offsets);
  set_rows(a, sh, rows);
  a.W1 = W1; a.W3 = W3; a.W2 = W2; a.row_prob = row_prob;
  a.ab_out = ab; a.h_out = h; a.h = h; a.o_out = o;
  return fwd_sequence(sh, a, (hipStream_t)stream);
}

int bwd_rowscaled(const moe_shape* sh, const int32_t* offsets, const RowSrc& rows, const void* ab,
                  void* h, int32_t recompute_h, const void* dO, const void* W1, const void* W3,
                  const void* W2, const float* row_prob, void* dab, void* dXp, void* dW1,
                  void* dW3, void* dW2, const int32_t* row_of, float* dprob, void* ws,
                  void* stream) {
  int st;
  GemmArgs a = expert_args(sh, offsets);
  set_rows(a, sh, rows);
  a.ab = ab; a.h = h; a.dO = dO; a.W1 = W1; a.W3 = W3; a.W2 = W2;
  a.dab_out = dab; a.dXp_out = dXp; a.dW1 = dW1; a.dW3 = dW3; a.dW2 = dW2;
  a.row_prob = row_prob;
  a.dp_part = (float*)ws;
  a.h_out = recompute_h ? h : nullptr;  // fc2 dgrad's epilogue refills h for fc2 wgrad
  hipStream_t s = (hipStream_t)stream;
  // fc2 dgrad alone is row-scaled; the other products take the plain path
  if ((st = gemm_bf16_launch(OP_FC2_DGRAD, a, s))) return st;
  a.row_prob = nullptr;
  a.h_out = nullptr;
  a.dab = a.dab_out;
  if ((st = gemm_bf16_launch(OP_FC1_DGRAD, a, s))) return st;
  if ((st = gemm_bf16_launch(OP_FC2_WGRAD, a, s))) return st;
  if ((st = gemm_bf16_launch(OP_FC1_WGRAD, a, s))) return st;
  if (!dprob) return MOE_OK;
  return dp_rows_launch((const float*)ws, (int)((sh->f + 255) / 256), row_of,
                        (int)(sh->T * sh->k), dprob, s);
}

}  // namespace

extern "C" {

int moe_aux_loss(const float* logits, int64_t T, int64_t E, int64_t k, const int32_t* counts,
                 float alpha, float* loss, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !counts || !loss) return MOE_ERR_INVALID;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T >= (1 << 30)) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < aux_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  return aux_loss_launch(logits, (int)T, (int)E, (int)k, counts, alpha, loss, ws,
                         (hipStream_t)stream);
}

int moe_route_aux(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* topk_idx,
                  float* topk_prob, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !topk_idx || !topk_prob) return MOE_ERR_INVALID;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T >= (1 << 30)) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < aux_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  return route_aux_launch(logits, (int)T, (int)E, (int)k, topk_idx, topk_prob, (float*)ws,
                          (hipStream_t)stream);
}

int moe_aux_loss_final(const void* ws, int64_t T, int64_t E, int64_t k, const int32_t* counts,
                       float alpha, float* loss, void* stream) {
  if (!ws || !counts || !loss) return MOE_ERR_INVALID;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T >= (1 << 30)) return MOE_ERR_UNSUPPORTED;
  return aux_final_launch((const float*)ws, (int)T, (int)E, (int)k, counts, alpha, loss,
                          (hipStream_t)stream);
}

int moe_combine_bwd(const moe_shape* sh, const void* dY, const void* o, const int32_t* row_of,
                    const float* topk_prob, void* dO, float* dprob, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (!dY || !o || !row_of || !topk_prob || !dO || !dprob) return MOE_ERR_INVALID;
  if (sh->d * elem_bytes(sh) > 32768) return MOE_ERR_UNSUPPORTED;
  return combine_bwd_launch(dY, o, row_of, topk_prob, (int)sh->T, (int)sh->k, (int)sh->d,
                            elem_bytes(sh), dO, dprob, (hipStream_t)stream);
}

int moe_route_bwd(const float* logits, int64_t T, int64_t E, int64_t k, const int32_t* topk_idx,
                  const float* topk_prob, const float* dprob, const int32_t* counts, float alpha,
                  float aux_scale, float* dlogits, void* stream) {
  if (!logits || !topk_idx || !topk_prob || !dprob || !dlogits) return MOE_ERR_INVALID;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T * k >= ((int64_t)1 << 31) || T * E >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  return route_bwd_launch(logits, (int)T, (int)E, (int)k, topk_idx, topk_prob, dprob, counts,
                          alpha, aux_scale, dlogits, (hipStream_t)stream);
}

int moe_quantize_rows(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                      uint8_t* codes, float* scales, void* stream) {
  if (!src || !codes || !scales || rows < 0 || cols < 0) return MOE_ERR_INVALID;
  if (src_dtype != MOE_BF16 && src_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (cols % 128 != 0 || rows * (cols / 128) >= ((int64_t)1 << 35)) return MOE_ERR_UNSUPPORTED;
  return quant_rows_launch(src, src_dtype == MOE_F32, rows, cols, codes, scales,
                           (hipStream_t)stream);
}

int moe_quantize_weights(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                         uint8_t* codes_t, float* scales, void* stream) {
  if (!W || !codes || !scales || E < 0 || R < 0 || C < 0) return MOE_ERR_INVALID;
  if (R % 128 != 0 || C % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (R >= (1 << 30) || C >= (1 << 30) || E > 65535 || C / 128 > 65535 || R / 128 > 65535)
    return MOE_ERR_UNSUPPORTED;
  return quant_tiles_launch(W, E, R, C, codes, codes_t, scales, (hipStream_t)stream);
}

int64_t moe_token_block_capacity(int64_t P, int64_t E) {
  if (P < 0 || E < 0) return 0;
  return tokblk_max_blocks(P, E);
}

int moe_quantize_token_blocks(const int32_t* offsets, int64_t E, int64_t P, const void* src,
                              const int32_t* src_row, int64_t C, int32_t* blk, uint8_t* codes,
                              float* scales, void* stream) {
  if (!offsets || !src || !blk || !codes || !scales) return MOE_ERR_INVALID;
  if (E < 1 || P < 0 || C < 0) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (C % 128 != 0 || C >= (1 << 30) || P >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  // the GEMMs address an expert's rows and scale blocks with 32-bit offsets
  if ((C + 256) * 128 * tokblk_max_blocks(P, E) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  int st = tokblk_table_launch(offsets, (int)E, blk, s);
  if (st) return st;
  return quant_tokblk_launch(src, src_row, offsets, blk, (int)E, P, C, codes, scales, s);
}

int moe_quantize_token_blocks_with_rows(const int32_t* offsets, int64_t E, int64_t P,
                                        const void* src, const int32_t* src_row, int64_t C,
                                        int32_t* blk, uint8_t* codes, float* scales,
                                        uint8_t* row_codes, float* row_scales, void* stream) {
  if (!offsets || !src || !blk || !codes || !scales || !row_codes || !row_scales) return MOE_ERR_INVALID;
  if (E < 1 || P < 0 || C < 0) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (C % 128 != 0 || C >= (1 << 30) || P >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if ((C + 256) * 128 * tokblk_max_blocks(P, E) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  int st = tokblk_table_launch(offsets, (int)E, blk, s);
  if (st) return st;
  return quant_tokblk_launch(src, src_row, offsets, blk, (int)E, P, C, codes, scales, s, row_codes,
                             row_scales);
}

int moe_permute_e4m3(const moe_shape* sh, const uint8_t* codes, const float* scales,
                     const int32_t* topk_idx, int build_map, int32_t* counts, int32_t* offsets,
                     int32_t* row_of, int32_t* token_of, uint8_t* dst_codes, float* dst_scales,
                     void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (sh->d % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!codes || !scales || !dst_codes || !dst_scales || !row_of) return MOE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  if (build_map) {
    if (!topk_idx || !counts || !offsets || !token_of) return MOE_ERR_INVALID;
    if (!ws || ws_bytes < permute_ws_bytes(sh->T, sh->E)) return MOE_ERR_WORKSPACE;
    st = permute_map_launch(topk_idx, (int)sh->T, (int)sh->E, (int)sh->k, counts, offsets, row_of,
                            token_of, ws, s);
    if (st) return st;
  }
  return permute_e4m3_launch(codes, scales, row_of, (int)sh->T, (int)sh->k, (int)sh->d, dst_codes,
                             dst_scales, s);
}

int moe_grouped_gemm_fwd_e4m3(const moe_shape* sh, const int32_t* offsets, const uint8_t* xpq,
                              const float* xps, const moe_e4m3_weights* w, void* ab, void* h,
                              void* o, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (sh->dtype != MOE_E4M3) return MOE_ERR_INVALID;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (!offsets || !xpq || !xps || !weights_ok(w) || !ab || !h || !o) return MOE_ERR_INVALID;
  return gemm_fwd8(sh, offsets, xpq, xps, wq8_of(w), ab, h, o, ws, ws_bytes, stream, false);
}

int moe_grouped_gemm_fwd_mx(const moe_shape* sh, const int32_t* offsets, const uint8_t* xpq,
                            const uint8_t* xps, const moe_mx_weights* w, void* ab, void* h,
                            void* o, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (sh->dtype != MOE_MXFP8) return MOE_ERR_INVALID;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (!offsets || !xpq || !xps || !weights_ok(w) || !ab || !h || !o) return MOE_ERR_INVALID;
  return gemm_fwd8(sh, offsets, xpq, xps, wq8_of(w), ab, h, o, ws, ws_bytes, stream, true);
}

int moe_grouped_gemm_bwd_e4m3(const moe_shape* sh, const int32_t* offsets,
                              const int32_t* token_of, const void* x, const void* ab,
                              const void* h, const void* dO, const moe_e4m3_weights* w, void* dab,
                              void* dXp, void* dW1, void* dW3, void* dW2, void* ws,
                              size_t ws_bytes, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (sh->dtype != MOE_E4M3) return MOE_ERR_INVALID;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (!offsets || !token_of || !x || !ab || !h || !dO || !weights_ok(w) || !dab || !dXp || !dW1 ||
      !dW3 || !dW2)
    return MOE_ERR_INVALID;
  return gemm_bwd8(sh, offsets, token_of, x, ab, h, dO, wq8_of(w), dab, dXp, dW1, dW3, dW2, ws,
                   ws_bytes, stream, false);
}

int moe_grouped_gemm_bwd_mx(const moe_shape* sh, const int32_t* offsets, const int32_t* token_of,
                            const void* x, const void* ab, const void* h, const void* dO,
                            const moe_mx_weights* w, void* dab, void* dXp, void* dW1, void* dW3,
                            void* dW2, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (sh->dtype != MOE_MXFP8) return MOE_ERR_INVALID;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (!offsets || !token_of || !x || !ab || !h || !dO || !weights_ok(w) || !dab || !dXp || !dW1 ||
      !dW3 || !dW2)
    return MOE_ERR_INVALID;
  return gemm_bwd8(sh, offsets, token_of, x, ab, h, dO, wq8_of(w), dab, dXp, dW1, dW3, dW2, ws,
                   ws_bytes, stream, true);
}

int moe_quantize_rows_mx(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                         uint8_t* codes, uint8_t* scales, void* stream) {
  if (!src || !codes || !scales || rows < 0 || cols < 0) return MOE_ERR_INVALID;
  if (src_dtype != MOE_BF16 && src_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (cols % 32 != 0 || rows * (cols / 32) >= ((int64_t)1 << 36)) return MOE_ERR_UNSUPPORTED;
  return quant_rows_mx_launch(src, src_dtype == MOE_F32, rows, cols, codes, scales,
                              (hipStream_t)stream);
}

int moe_quantize_weights_mx(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                            uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, void* stream) {
  if (!W || !codes || !scales || !codes_t || !scales_t || E < 0 || R < 0 || C < 0)
    return MOE_ERR_INVALID;
  if (R % 128 != 0 || C % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (R >= (1 << 30) || C >= (1 << 30) || E > 65535 || C / 128 > 65535 || R / 128 > 65535)
    return MOE_ERR_UNSUPPORTED;
  // the scale bytes are stored as 32-bit words
  if ((((uintptr_t)scales) | ((uintptr_t)scales_t)) & 3) return MOE_ERR_UNSUPPORTED;
  return quant_weights_mx_launch(W, E, R, C, codes, scales, codes_t, scales_t,
                                 (hipStream_t)stream);
}

int moe_quantize_token_blocks_mx(const int32_t* offsets, int64_t E, int64_t P, const void* src,
                                 const int32_t* src_row, int64_t C, int32_t* blk,
                                 uint8_t* codes, uint8_t* scales, void* stream) {
  if (!offsets || !src || !blk || !codes || !scales) return MOE_ERR_INVALID;
  if (E < 1 || P < 0 || C < 0) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (C % 128 != 0 || C >= (1 << 30) || P >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if ((C + 256) * 128 * tokblk_max_blocks(P, E) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  int st = tokblk_table_launch(offsets, (int)E, blk, s);
  if (st) return st;
  return quant_tokblk_mx_launch(src, src_row, offsets, blk, (int)E, P, C, codes, scales, s);
}

int moe_quantize_token_blocks_with_rows_mx(const int32_t* offsets, int64_t E, int64_t P,
                                           const void* src, const int32_t* src_row, int64_t C,
                                           int32_t* blk, uint8_t* codes, uint8_t* scales,
                                           uint8_t* row_codes, uint8_t* row_scales, void* stream) {
  if (!offsets || !src || !blk || !codes || !scales || !row_codes || !row_scales) return MOE_ERR_INVALID;
  if (E < 1 || P < 0 || C < 0) return MOE_ERR_INVALID;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (C % 128 != 0 || C >= (1 << 30) || P >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if ((C + 256) * 128 * tokblk_max_blocks(P, E) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  int st = tokblk_table_launch(offsets, (int)E, blk, s);
  if (st) return st;
  return quant_tokblk_mx_launch(src, src_row, offsets, blk, (int)E, P, C, codes, scales, s,
                                row_codes, row_scales);
}

int moe_permute_mx(const moe_shape* sh, const uint8_t* codes, const uint8_t* scales,
                   const int32_t* topk_idx, int build_map, int32_t* counts, int32_t* offsets,
                   int32_t* row_of, int32_t* token_of, uint8_t* dst_codes, uint8_t* dst_scales,
                   void* ws, size_t ws_bytes, void* stream) {
  // d/32 scale bytes per row are the byte count of d/128 fp32 scales: the
  // e4m3 row move copies them bit for bit
  return moe_permute_e4m3(sh, codes, (const float*)scales, topk_idx, build_map, counts, offsets,
                          row_of, token_of, dst_codes, (float*)dst_scales, ws, ws_bytes, stream);
}

int moe_layer_fwd(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                  void* stream) {
  int st = check_shape(sh);
  if (st) return st;
  if (is_fp8(sh)) return layer_fwd_e4m3(sh, io, ws, ws_bytes, stream);
  if (io && io->memory_efficient) return layer_fwd_rowscaled(sh, io, ws, ws_bytes, stream);
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (sh->f_shared && (st = check_gemm_dims(sh, sh->T, sh->f_shared))) return st;
  if (!io || !io->logits || !io->x || !io->W1 || !io->W3 || !io->W2 || !io->topk_idx ||
      !io->topk_prob || !io->counts || !io->offsets || !io->row_of || !io->token_of ||
      (!io->xp && !io->fused_permute) || !io->ab || !io->h || !io->o || !io->y)
    return MOE_ERR_INVALID;
  if (io->fused_permute && (st = check_gather(sh))) return st;
  if (sh->f_shared &&
      (!io->Ws1 || !io->Ws3 || !io->Ws2 || !io->s_ab || !io->s_h || !io->ys))
    return MOE_ERR_INVALID;
  const size_t pws = permute_ws_bytes(sh->T, sh->E);
  if (!ws || ws_bytes < pws + 256 || !aux_ws_ok(sh, io, ws_bytes)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;

  if ((st = layer_route(sh, io, ws, ws_bytes, stream))) return st;
  // fused permutation: the map alone; fc1 reads x through token_of
  if ((st = moe_permute(sh, io->x, io->topk_idx, nullptr, 1, io->counts, io->offsets, io->row_of,
                        io->token_of, io->fused_permute ? nullptr : io->xp, ws, pws, stream)))
    return st;
  if ((st = layer_aux_loss(sh, io, ws, ws_bytes, stream))) return st;
  {
    GemmArgs a = expert_args(sh, io->offsets);
    set_rows(a, sh, rows_of(io));
    a.W1 = io->W1; a.W3 = io->W3; a.W2 = io->W2;
    a.ab_out = io->ab; a.h_out = io->h; a.h = io->h; a.o_out = io->o;
    if ((st = fwd_sequence(sh, a, s))) return st;
  }
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
  if (is_fp8(sh)) return layer_bwd_e4m3(sh, io, ws, ws_bytes, stream);
  if (io && io->memory_efficient) return layer_bwd_rowscaled(sh, io, ws, ws_bytes, stream);
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (sh->f_shared && (st = check_gemm_dims(sh, sh->T, sh->f_shared))) return st;
  if (!io || !io->dY || !io->W1 || !io->W3 || !io->W2 || !io->topk_prob || !io->offsets ||
      !io->row_of || !io->ab || !io->h || !io->dO || !io->dab || !io->dXp || !io->dX ||
      !io->dW1 || !io->dW3 || !io->dW2)
    return MOE_ERR_INVALID;
  if (io->fused_permute ? (!io->token_of || !io->x) : !io->xp) return MOE_ERR_INVALID;
  if (io->fused_permute && (st = check_gather(sh))) return st;
  if (sh->f_shared && (!io->x || !io->Ws1 || !io->Ws3 || !io->Ws2 || !io->s_ab || !io->s_h ||
                       !io->s_dab || !io->dXs || !io->dWs1 || !io->dWs3 || !io->dWs2))
    return MOE_ERR_INVALID;
  if (!ws || ws_bytes < 256) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;

  // dO[row_of[t][j]] = p[t][j] * dY[t] (+ dprob and the router gradient when asked for)
  if ((st = layer_combine_bwd(sh, io, stream))) return st;
  {
    GemmArgs a = expert_args(sh, io->offsets);
    set_rows(a, sh, rows_of(io));
    a.ab = io->ab; a.h = io->h; a.dO = io->dO; a.W1 = io->W1; a.W3 = io->W3; a.W2 = io->W2;
    a.dab_out = io->dab; a.dXp_out = io->dXp; a.dW1 = io->dW1; a.dW3 = io->dW3; a.dW2 = io->dW2;
    if ((st = bwd_sequence(sh, a, s))) return st;
  }
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

namespace {

// e4m3 and MXFP8 layers
int layer_fwd_e4m3(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                   void* stream) {
  int st;
  const bool mx = sh->dtype == MOE_MXFP8;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (!io || !(mx ? weights_ok(io->wmx) : weights_ok(io->wq))) return MOE_ERR_INVALID;
  if (!io->logits || !io->x || !io->topk_idx || !io->topk_prob ||
      !io->counts || !io->offsets || !io->row_of || !io->token_of || !io->xq || !io->xs ||
      !io->xpq || !io->xps || !io->ab || !io->h || !io->o || !io->y)
    return MOE_ERR_INVALID;
  const bool me = io->memory_efficient != 0;  // probabilities applied before W2
  if (me && !io->row_prob) return MOE_ERR_INVALID;
  const size_t pws = permute_ws_bytes(sh->T, sh->E);
  const size_t gws = fwd8_ws_bytes(sh);
  if (!ws || ws_bytes < pws + gws || !aux_ws_ok(sh, io, ws_bytes)) return MOE_ERR_WORKSPACE;
  if ((st = layer_route(sh, io, ws, ws_bytes, stream))) return st;
  if ((st = (mx ? moe_quantize_rows_mx(io->x, MOE_BF16, sh->T, sh->d, io->xq,
                                       (uint8_t*)io->xs, stream)
                 : moe_quantize_rows(io->x, MOE_BF16, sh->T, sh->d, io->xq, io->xs, stream))))
    return st;
  if ((st = moe_permute_e4m3(sh, io->xq, io->xs, io->topk_idx, 1, io->counts, io->offsets,
                             io->row_of, io->token_of, io->xpq, io->xps, ws, pws, stream)))
    return st;
  if ((st = layer_aux_loss(sh, io, ws, ws_bytes, stream))) return st;
  if (me && (st = moe_row_probs(sh, io->row_of, io->topk_prob, io->row_prob, stream))) return st;
  if ((st = gemm_fwd8(sh, io->offsets, io->xpq, io->xps, mx ? wq8_of(io->wmx) : wq8_of(io->wq),
                      io->ab, io->h, io->o, (char*)ws + pws, gws, stream, mx,
                      me ? io->row_prob : nullptr)))
    return st;
  // memory-efficient: o rows already carry their probability
  return moe_unpermute(sh, io->o, io->row_of, me ? nullptr : io->topk_prob, nullptr, io->y,
                       stream);
}

int layer_bwd_e4m3(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                   void* stream) {
  int st;
  const bool mx = sh->dtype == MOE_MXFP8;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (!io || !(mx ? weights_ok(io->wmx) : weights_ok(io->wq))) return MOE_ERR_INVALID;
  if (!io->dY || !io->x || !io->topk_prob || !io->offsets ||
      !io->row_of || !io->token_of || !io->ab || !io->h || !io->dO || !io->dab || !io->dXp ||
      !io->dX || !io->dW1 || !io->dW3 || !io->dW2)
    return MOE_ERR_INVALID;
  const bool me = io->memory_efficient != 0;  // probabilities applied before W2
  const size_t gws = bwd8_ws_bytes(sh);
  if (!me) {
    if (!ws || ws_bytes < gws) return MOE_ERR_WORKSPACE;
    if ((st = layer_combine_bwd(sh, io, stream))) return st;
    if ((st = gemm_bwd8(sh, io->offsets, io->token_of, io->x, io->ab, io->h, io->dO,
                        mx ? wq8_of(io->wmx) : wq8_of(io->wq), io->dab, io->dXp, io->dW1, io->dW3,
                        io->dW2, ws, ws_bytes, stream, mx)))
      return st;
    return moe_unpermute(sh, io->dXp, io->row_of, nullptr, nullptr, io->dX, stream);
  }
  if (!io->row_prob) return MOE_ERR_INVALID;
  if (io->dlogits && (!io->dprob || !io->logits || !io->topk_idx || !io->counts))
    return MOE_ERR_INVALID;
  if (!ws || ws_bytes < gws + dp_part_bytes(sh)) return MOE_ERR_WORKSPACE;
  float* dp_part = (float*)((char*)ws + gws);
  // dO = dY permuted, unscaled; the fc2 dgrad epilogue yields the dprob partials
  if ((st = moe_permute(sh, io->dY, nullptr, nullptr, 0, nullptr, nullptr, io->row_of, nullptr,
                        io->dO, nullptr, 0, stream)))
    return st;
  if ((st = gemm_bwd8(sh, io->offsets, io->token_of, io->x, io->ab, io->h, io->dO,
                      mx ? wq8_of(io->wmx) : wq8_of(io->wq), io->dab, io->dXp, io->dW1, io->dW3,
                      io->dW2, ws, gws, stream, mx, io->row_prob, dp_part,
                      io->memory_efficient == 2)))
    return st;
  if ((st = moe_unpermute(sh, io->dXp, io->row_of, nullptr, nullptr, io->dX, stream))) return st;
  if (!io->dlogits) return MOE_OK;
  if ((st = dp_rows_launch(dp_part, (int)((sh->f + 255) / 256), io->row_of,
                           (int)(sh->T * sh->k), io->dprob, (hipStream_t)stream)))
    return st;
  return moe_route_bwd(io->logits, sh->T, sh->E, sh->k, io->topk_idx, io->topk_prob, io->dprob,
                       io->counts, io->aux_alpha, 1.0f, io->dlogits, stream);
}

}  // namespace

namespace {

// the aux loss's workspace follows the layer's forward workspace
bool aux_ws_ok(const moe_shape* sh, const moe_layer_io* io, size_t ws_bytes) {
  return !io->aux_loss ||
         ws_bytes >= moe_workspace_bytes(sh, MOE_WS_LAYER_FWD) + aux_ws_bytes(sh->T, sh->E);
}

// Routing of a layer; when io->aux_loss is set, fused with the loss's
// softmax column sums, which go to the aux region of the forward workspace
// (after the MOE_WS_LAYER_FWD bytes, untouched by the permutation).
int layer_route(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                void* stream) {
  if (!io->aux_loss)
    return moe_route(io->logits, sh->T, sh->E, sh->k, io->topk_idx, io->topk_prob, stream);
  const size_t base = moe_workspace_bytes(sh, MOE_WS_LAYER_FWD);
  const size_t need = aux_ws_bytes(sh->T, sh->E);
  if (ws_bytes < base + need) return MOE_ERR_WORKSPACE;
  return moe_route_aux(io->logits, sh->T, sh->E, sh->k, io->topk_idx, io->topk_prob,
                       (char*)ws + base, need, stream);
}

// aux loss from those column sums and the permutation's counts
int layer_aux_loss(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                   void* stream) {
  if (!io->aux_loss) return MOE_OK;
  const size_t base = moe_workspace_bytes(sh, MOE_WS_LAYER_FWD);
  if (ws_bytes < base + aux_ws_bytes(sh->T, sh->E)) return MOE_ERR_WORKSPACE;
  return moe_aux_loss_final((char*)ws + base, sh->T, sh->E, sh->k, io->counts, io->aux_alpha,
                            io->aux_loss, stream);
}

// Memory-efficient layer (probabilities applied before W2), bf16 only.
int layer_fwd_rowscaled(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                        void* stream) {
  int st;
  if (sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (sh->f_shared && (st = check_gemm_dims(sh, sh->T, sh->f_shared))) return st;
  if (!io->logits || !io->x || !io->W1 || !io->W3 || !io->W2 || !io->topk_idx ||
      !io->topk_prob || !io->counts || !io->offsets || !io->row_of || !io->token_of ||
      (!io->xp && !io->fused_permute) || !io->ab || !io->h || !io->o || !io->y || !io->row_prob)
    return MOE_ERR_INVALID;
  if (io->fused_permute && (st = check_gather(sh))) return st;
  if (sh->f_shared &&
      (!io->Ws1 || !io->Ws3 || !io->Ws2 || !io->s_ab || !io->s_h || !io->ys))
    return MOE_ERR_INVALID;
  const size_t pws = permute_ws_bytes(sh->T, sh->E);
  if (!ws || ws_bytes < pws + 256 || !aux_ws_ok(sh, io, ws_bytes)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if ((st = layer_route(sh, io, ws, ws_bytes, stream))) return st;
  if ((st = moe_permute(sh, io->x, io->topk_idx, nullptr, 1, io->counts, io->offsets, io->row_of,
                        io->token_of, io->fused_permute ? nullptr : io->xp, ws, pws, stream)))
    return st;
  if ((st = layer_aux_loss(sh, io, ws, ws_bytes, stream))) return st;
  if ((st = moe_row_probs(sh, io->row_of, io->topk_prob, io->row_prob, stream))) return st;
  if ((st = fwd_rowscaled(sh, io->offsets, rows_of(io), io->W1, io->W3, io->W2, io->row_prob,
                          io->ab, io->h, io->o, stream)))
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
  // o rows already carry their probability: unweighted combine
  return moe_unpermute(sh, io->o, io->row_of, nullptr, add, io->y, stream);
}

int layer_bwd_rowscaled(const moe_shape* sh, const moe_layer_io* io, void* ws, size_t ws_bytes,
                        void* stream) {
  int st;
  if (sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((st = check_gemm_dims(sh, sh->T * sh->k, sh->f))) return st;
  if (sh->f_shared && (st = check_gemm_dims(sh, sh->T, sh->f_shared))) return st;
  if (!io->dY || !io->W1 || !io->W3 || !io->W2 || !io->offsets || !io->row_of ||
      !io->ab || !io->h || !io->dO || !io->dab || !io->dXp || !io->dX || !io->dW1 || !io->dW3 ||
      !io->dW2 || !io->row_prob)
    return MOE_ERR_INVALID;
  if (io->fused_permute ? (!io->token_of || !io->x) : !io->xp) return MOE_ERR_INVALID;
  if (io->fused_permute && (st = check_gather(sh))) return st;
  if (sh->f_shared && (!io->x || !io->Ws1 || !io->Ws3 || !io->Ws2 || !io->s_ab || !io->s_h ||
                       !io->s_dab || !io->dXs || !io->dWs1 || !io->dWs3 || !io->dWs2))
    return MOE_ERR_INVALID;
  if (io->dlogits && (!io->dprob || !io->logits || !io->topk_idx || !io->topk_prob || !io->counts))
    return MOE_ERR_INVALID;
  const size_t part = dp_part_bytes(sh);
  if (!ws || ws_bytes < 256 + part) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  float* dp_part = (float*)((char*)ws + 256);
  // dO = dY permuted, unscaled
  if ((st = moe_permute(sh, io->dY, nullptr, nullptr, 0, nullptr, nullptr, io->row_of, nullptr,
                        io->dO, nullptr, 0, stream)))
    return st;
  // dprob[t][j] too when the router gradient is asked for
  if ((st = bwd_rowscaled(sh, io->offsets, rows_of(io), io->ab, io->h, io->memory_efficient == 2,
                          io->dO, io->W1, io->W3, io->W2, io->row_prob, io->dab, io->dXp,
                          io->dW1, io->dW3, io->dW2, io->row_of,
                          io->dlogits ? io->dprob : nullptr, dp_part, stream)))
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
  if ((st = moe_unpermute(sh, io->dXp, io->row_of, nullptr, add, io->dX, stream))) return st;
  if (!io->dlogits) return MOE_OK;
  return moe_route_bwd(io->logits, sh->T, sh->E, sh->k, io->topk_idx, io->topk_prob, io->dprob,
                       io->counts, io->aux_alpha, 1.0f, io->dlogits, stream);
}

// dO for the expert backward, plus dprob and dlogits when io->dlogits is set
int layer_combine_bwd(const moe_shape* sh, const moe_layer_io* io, void* stream) {
  int st;
  if (!io->dlogits)
    return moe_permute(sh, io->dY, nullptr, io->topk_prob, 0, nullptr, nullptr, io->row_of,
                       nullptr, io->dO, nullptr, 0, stream);
  if (!io->dprob || !io->o || !io->logits || !io->topk_idx || !io->counts) return MOE_ERR_INVALID;
  if ((st = moe_combine_bwd(sh, io->dY, io->o, io->row_of, io->topk_prob, io->dO, io->dprob,
                            stream)))
    return st;
  return moe_route_bwd(io->logits, sh->T, sh->E, sh->k, io->topk_idx, io->topk_prob, io->dprob,
                       io->counts, io->aux_alpha, 1.0f, io->dlogits, stream);
}

}  // namespace
