// Router backward and the load-balancing auxiliary loss.
//
// The pages fuse routing, permutation and auxiliary-loss computations into
// few kernels ("Scalable Training of Mixture-of-Experts Models with Megatron
// Core", gist.science German technical summary, section 2 D; Spanish summary,
// section 2.3 C) but state no formula.  Readings:
//  * the combine y[t] = sum_j p[t][j] o[row_of[t][j]] gives the probability
//    gradient dp[t][j] = <dY[t], o[row_of[t][j]]>; p is the softmax over the k
//    selected logits, so dlogits[t][idx[t][j]] = p_j (dp_j - sum_i p_i dp_i)
//    and 0 for the other experts;
//  * switch-style load balancing: L = alpha E sum_e f_e P_e with
//    f_e = counts[e] / (T k) and P_e the mean over tokens of the softmax over
//    all E logits; counts are held constant, so
//    dL/dlogits[t] = s[t] (g - <g, s[t]>), g_e = alpha E f_e / T.
// Every reduction runs in a fixed order: results are deterministic.
#include "common.h"
#include "internal.h"

namespace tre {

namespace {

template <typename T>
__device__ __forceinline__ void vec8(const u32x4_t& v, float* out);
template <>
__device__ __forceinline__ void vec8<float>(const u32x4_t& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}
template <>
__device__ __forceinline__ void vec8<bf16_t>(const u32x4_t& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ u32x4_t pack8(const float* in);
template <>
__device__ __forceinline__ u32x4_t pack8<float>(const float* in) {
  return u32x4_t{__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                 __float_as_uint(in[3])};
}
template <>
__device__ __forceinline__ u32x4_t pack8<bf16_t>(const float* in) {
  return u32x4_t{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]), pack_bf16x2(in[4], in[5]),
                 pack_bf16x2(in[6], in[7])};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- combine backward
// One block (256 threads) per token t; C 16-byte chunks per row, CPT chunks
// per thread at most.  dO[row_of[t][j]] = round(p[t][j] * dY[t]) as the scaled
// permutation does, and dprob[t][j] = <dY[t], o[row_of[t][j]]> in fp32: per
// thread over its chunks in order, then a fixed-order block reduction.  The k
// rows go in groups of KG so that KG * CPT row loads are in flight per thread
// and the group's KG dot products share one block reduction.
constexpr int KG = 8;
template <typename T, int CPT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const u32x4_t* __restrict__ dY,
                                                          const u32x4_t* __restrict__ o,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ prob, int k,
                                                          int C, u32x4_t* __restrict__ dO,
                                                          float* __restrict__ dprob) {
  constexpr int N = 16 / sizeof(T);
  __shared__ float red[4][KG];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float g[CPT][N];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = tid + q * 256;
    if (c < C) vec8<T>(__builtin_nontemporal_load(&dY[(size_t)t * C + c]), g[q]);
  }
  for (int j0 = 0; j0 < k; j0 += KG) {
    const int nj = min(KG, k - j0);
    float dot[KG];
#pragma unroll
    for (int jj = 0; jj < KG; ++jj) {
      dot[jj] = 0.0f;
      if (jj < nj) {
        const int row = row_of[(size_t)t * k + j0 + jj];
        const float p = prob[(size_t)t * k + j0 + jj];
        // an assignment without a row (outside [0, T k)) moves nothing; its dprob is 0
        const bool live = (unsigned)row < (unsigned)(gridDim.x * k);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const int c = tid + q * 256;
          if (live && c < C) {
            float ov[N], y[N];
            vec8<T>(__builtin_nontemporal_load(&o[(size_t)row * C + c]), ov);
#pragma unroll
            for (int i = 0; i < N; ++i) {
              dot[jj] = fmaf(g[q][i], ov[i], dot[jj]);
              y[i] = p * g[q][i];
            }
            __builtin_nontemporal_store(pack8<T>(y), &dO[(size_t)row * C + c]);
          }
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < KG; ++jj) {
      const float v = wave_sum(dot[jj]);
      if (lane == 0) red[w][jj] = v;
    }
    __syncthreads();
    if (tid < nj) dprob[(size_t)t * k + j0 + tid] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- router backward
// One wavefront per token, 4 tokens per block; lane l owns experts l, l+64,
// l+128, l+192 (E <= 256) and the selections l, l+64, ... (k <= E).
// g_e = gscale * counts[e] (gscale = aux_scale * alpha * E / (T * T * k)); the
// auxiliary term is skipped when gscale == 0.  The Jacobian term of selection
// j is computed by the lane that holds j and added into an LDS copy of the
// token's row at expert idx[t][j] (the k experts of a token are distinct).
__global__ __launch_bounds__(256) void route_bwd_kernel(
    const float* __restrict__ logits, int T, int E, int k, const int32_t* __restrict__ idx,
    const float* __restrict__ prob, const float* __restrict__ dprob,
    const int32_t* __restrict__ counts, float gscale, float* __restrict__ dlogits) {
  __shared__ float rowbuf[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  const bool live = t < T;  // no early return: the block synchronises below
  const float* L = logits + (size_t)t * E;
  const float* pt = prob + (size_t)t * k;
  const float* dpt = dprob + (size_t)t * k;
  const int32_t* it = idx + (size_t)t * k;
  float v[4], pj[4], dpj[4];
  int ej[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = live && e < E ? L[e] : -INFINITY;
    const bool sel = live && e < k;
    pj[q] = sel ? pt[e] : 0.0f;
    dpj[q] = sel ? dpt[e] : 0.0f;
    ej[q] = sel ? it[e] : -1;
  }
  float dl[4] = {0.f, 0.f, 0.f, 0.f};
  if (gscale != 0.0f) {
    float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    m = wave_max(m);
    float sum = 0.f, s[4], gs = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      s[q] = e < E ? __expf(v[q] - m) : 0.f;
      sum += s[q];
    }
    sum = wave_sum(sum);
    float gv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      s[q] = s[q] / sum;
      gv[q] = live && e < E ? gscale * (float)counts[e] : 0.f;
      gs = fmaf(gv[q], s[q], gs);
    }
    gs = wave_sum(gs);
#pragma unroll
    for (int q = 0; q < 4; ++q) dl[q] = s[q] * (gv[q] - gs);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) rowbuf[w][lane + 64 * q] = dl[q];
  // top-k softmax Jacobian p_j (dp_j - sum_i p_i dp_i), evaluated as
  // p_j sum_i p_i (dp_j - dp_i) (equal, as the p sum to one): the plain form
  // cancels catastrophically when one p_j is close to 1 and the others tiny.
  // Selection i's p and dp are read from the lane that holds it, in order.
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < k; ++i) {
    const int src = i & 63, q = i >> 6;
    const float p_i = __shfl(q == 0 ? pj[0] : q == 1 ? pj[1] : q == 2 ? pj[2] : pj[3], src, 64);
    const float dp_i = __shfl(q == 0 ? dpj[0] : q == 1 ? dpj[1] : q == 2 ? dpj[2] : dpj[3], src, 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(p_i, dpj[r] - dp_i, acc[r]);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (ej[r] >= 0) rowbuf[w][ej[r]] += pj[r] * acc[r];
  __syncthreads();
  if (live) {
    float* D = dlogits + (size_t)t * E;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E) D[e] = rowbuf[w][e];
    }
  }
}

// ---------------------------------------------------------------- auxiliary loss
// Block b (4 wavefronts) sums the softmax of tokens [AUX_TOK b, AUX_TOK b +
// AUX_TOK) per expert: wavefront w takes AUX_TOK / 4 consecutive tokens, 4 at a
// time with their loads issued together, accumulating in token order; the four
// wavefront sums are added in order into partial[b][e].
constexpr int AUX_TOK = 32;
constexpr int AUX_U = 4;
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int T,
                                                          int E, float* __restrict__ partial) {
  __shared__ float red[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int t0 = blockIdx.x * AUX_TOK + w * (AUX_TOK / 4);
  for (int i0 = 0; i0 < AUX_TOK / 4; i0 += AUX_U) {
    float v[AUX_U][4];
#pragma unroll
    for (int u = 0; u < AUX_U; ++u) {
      const int t = t0 + i0 + u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        v[u][q] = t < T && e < E ? logits[(size_t)t * E + e] : -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < AUX_U; ++u) {
      if (t0 + i0 + u >= T) break;  // uniform across the wavefront
      float m = fmaxf(fmaxf(v[u][0], v[u][1]), fmaxf(v[u][2], v[u][3]));
      m = wave_max(m);
      float s[4], sum = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        s[q] = e < E ? __expf(v[u][q] - m) : 0.f;
        sum += s[q];
      }
      sum = wave_sum(sum);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += s[q] / sum;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) red[w][lane + 64 * q] = acc[q];
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) partial[(size_t)blockIdx.x * E + e] = (red[0][e] + red[1][e]) + (red[2][e] + red[3][e]);
}

// One block of 1024 threads: thread (r, e) with r = tid / 256 sums the partials
// b = r, r + 4, r + 8, ... of expert e in order (8 loads issued together), the
// four sums are added in order, then loss = scale * sum_e counts[e] colsum[e]
// (scale = alpha E / (T T k)) by a fixed-order block reduction.
constexpr int AUX_FIN_U = 8;
__global__ __launch_bounds__(1024) void aux_final_kernel(const float* __restrict__ partial, int NB,
                                                         int E, const int32_t* __restrict__ counts,
                                                         float scale, float* __restrict__ loss) {
  __shared__ float cols[4][256];
  __shared__ float red[4];
  const int e = threadIdx.x & 255, r = threadIdx.x >> 8;
  float col = 0.f;
  if (e < E) {
    for (int b0 = r; b0 < NB; b0 += 4 * AUX_FIN_U) {
      float pv[AUX_FIN_U];
#pragma unroll
      for (int u = 0; u < AUX_FIN_U; ++u) {
        const int b = b0 + 4 * u;
        pv[u] = b < NB ? partial[(size_t)b * E + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < AUX_FIN_U; ++u) col += pv[u];
    }
  }
  cols[r][e] = col;
  __syncthreads();
  if (r == 0) {
    const int lane = e & 63, w = e >> 6;
    float v = e < E ? (float)counts[e] * ((cols[0][e] + cols[1][e]) + (cols[2][e] + cols[3][e])) : 0.f;
    v = wave_sum(v);
    if (lane == 0) red[w] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) *loss = scale * ((red[0] + red[1]) + (red[2] + red[3]));
}

// ---------------------------------------------------------------- row-scaled products
// Probabilities applied before W2: each permuted row's probability, and the
// sum of the fc2 dgrad's per-N-tile partials of <h, dh'> in N-tile order.
__global__ __launch_bounds__(256) void row_probs_kernel(const int32_t* __restrict__ row_of,
                                                        const float* __restrict__ prob, int n,
                                                        float* __restrict__ row_prob) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n && (unsigned)row_of[i] < (unsigned)n) row_prob[row_of[i]] = prob[i];
}

// out[i] = sum_nt part[r * NT + nt] with r = row_of[i] (or r = i without a map)
__global__ __launch_bounds__(256) void dp_rows_kernel(const float* __restrict__ part, int NT,
                                                      const int32_t* __restrict__ row_of, int n,
                                                      float* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = row_of ? row_of[i] : i;
  float s = 0.0f;
  if ((unsigned)r < (unsigned)n)  // an assignment without a row gets 0
    for (int nt = 0; nt < NT; ++nt) s += part[(size_t)r * NT + nt];
  out[i] = s;
}

template <typename T, int CPT>
void combine_bwd_typed(const void* dY, const void* o, const int32_t* row_of, const float* prob,
                       int T_, int k, int C, void* dO, float* dprob, hipStream_t s) {
  combine_bwd_kernel<T, CPT><<<T_, 256, 0, s>>>((const u32x4_t*)dY, (const u32x4_t*)o, row_of,
                                                 prob, k, C, (u32x4_t*)dO, dprob);
}

}  // namespace

int combine_bwd_launch(const void* dY, const void* o, const int32_t* row_of, const float* prob,
                       int T, int k, int d, int elem_bytes, void* dO, float* dprob,
                       hipStream_t s) {
  const int C = d * elem_bytes / 16;
  const int cpt = (C + 255) / 256;
  if (cpt > 8) return MOE_ERR_UNSUPPORTED;
  if (elem_bytes == 4) {
    if (cpt <= 2) combine_bwd_typed<float, 2>(dY, o, row_of, prob, T, k, C, dO, dprob, s);
    else if (cpt <= 4) combine_bwd_typed<float, 4>(dY, o, row_of, prob, T, k, C, dO, dprob, s);
    else combine_bwd_typed<float, 8>(dY, o, row_of, prob, T, k, C, dO, dprob, s);
  } else {
    if (cpt <= 2) combine_bwd_typed<bf16_t, 2>(dY, o, row_of, prob, T, k, C, dO, dprob, s);
    else if (cpt <= 4) combine_bwd_typed<bf16_t, 4>(dY, o, row_of, prob, T, k, C, dO, dprob, s);
    else combine_bwd_typed<bf16_t, 8>(dY, o, row_of, prob, T, k, C, dO, dprob, s);
  }
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int route_bwd_launch(const float* logits, int T, int E, int k, const int32_t* idx,
                     const float* prob, const float* dprob, const int32_t* counts, float alpha,
                     float aux_scale, float* dlogits, hipStream_t s) {
  const float gscale =
      (counts && alpha != 0.0f && aux_scale != 0.0f)
          ? (float)((double)aux_scale * alpha * E / ((double)T * T * k))
          : 0.0f;
  route_bwd_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, idx, prob, dprob, counts, gscale,
                                              dlogits);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int row_probs_launch(const int32_t* row_of, const float* prob, int n, float* row_prob,
                     hipStream_t s) {
  if (n <= 0) return MOE_OK;
  row_probs_kernel<<<(n + 255) / 256, 256, 0, s>>>(row_of, prob, n, row_prob);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int dp_rows_launch(const float* part, int NT, const int32_t* row_of, int n, float* out,
                   hipStream_t s) {
  if (n <= 0) return MOE_OK;
  dp_rows_kernel<<<(n + 255) / 256, 256, 0, s>>>(part, NT, row_of, n, out);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

size_t aux_ws_bytes(int64_t T, int64_t E) {
  return align_up((size_t)((T + AUX_TOK - 1) / AUX_TOK) * (size_t)E * sizeof(float), 256);
}

int aux_final_launch(const float* partial, int T, int E, int k, const int32_t* counts,
                     float alpha, float* loss, hipStream_t s) {
  const int NB = (T + AUX_TOK - 1) / AUX_TOK;
  const float scale = (float)((double)alpha * E / ((double)T * T * k));
  aux_final_kernel<<<1, 1024, 0, s>>>(partial, NB, E, counts, scale, loss);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int aux_loss_launch(const float* logits, int T, int E, int k, const int32_t* counts, float alpha,
                    float* loss, void* ws, hipStream_t s) {
  const int NB = (T + AUX_TOK - 1) / AUX_TOK;
  float* partial = (float*)ws;
  aux_partial_kernel<<<NB, 256, 0, s>>>(logits, T, E, partial);
  TRE_LAUNCH_CHECK();
  return aux_final_launch(partial, T, E, k, counts, alpha, loss, s);
}

}  // namespace tre
