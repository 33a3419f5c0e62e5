// Top-k routing from router logits (Spanish summary of "Scalable Training of
// Mixture-of-Experts Models with Megatron Core", section 2.1: each token goes
// to its k best experts), with a softmax over the k selected logits.
//
// Layout: a group of L lanes (L = next power of two >= E, at most 64) owns one
// token; a 64-lane wavefront therefore routes 64/L tokens at once.  Lane i of
// a group holds logits e = i, i+L, i+2L, ... (V = ceil(E/L) <= 4 values for
// E <= 256), so a row is read with coalesced loads.  Each of the k rounds takes
// a lane-local best, then a reduction inside the group (DPP inside 16-lane
// rows, shuffles across them); the winner's owner marks it taken.  The order key is (logit desc,
// expert asc), so equal logits go to the lower expert index; +0 and -0 are
// equal under the float comparison.  A NaN logit ranks below every number
// (-inf included), NaNs among themselves by index, so every token always gets
// k distinct experts in [0, E) whatever its logits hold.  The result is the
// same as a full stable sort of the row, independent of lane order.
#include "common.h"
#include "internal.h"

namespace tre {

namespace {

// (v, e) ranks before (bv, be): larger logit, then lower index; NaN last.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  if (v != v) return bv != bv && e < be;  // NaN only beats a NaN of higher index
  if (bv != bv) return true;              // any number beats NaN
  return v > bv || (v == bv && e < be);
}

// One level of the group-wide best-of reduction: every lane takes its
// partner's (value, index) and keeps the better.  Levels 1 and 2 pair lanes
// inside a quad, 4 and 8 mirror them inside 8- and 16-lane rows (DPP: no LDS
// round trip), 16 and 32 swap across rows.  The key is a total order, so
// after the levels up to L/2 every lane of an L-lane group holds its best.
template <int LEVEL>
__device__ __forceinline__ void best_level(float& bv, int& be) {
  float ov;
  int oe;
  if constexpr (LEVEL <= 8) {
    constexpr int ctrl = LEVEL == 1 ? 0xB1 : LEVEL == 2 ? 0x4E : LEVEL == 4 ? 0x141 : 0x140;
    ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), ctrl, 0xF, 0xF, false));
    oe = __builtin_amdgcn_update_dpp(0, be, ctrl, 0xF, 0xF, false);
  } else {
    ov = __shfl_xor(bv, LEVEL, 64);
    oe = __shfl_xor(be, LEVEL, 64);
  }
  if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
}
template <int L>
__device__ __forceinline__ void best_of_group(float& bv, int& be) {
  if constexpr (L >= 2) best_level<1>(bv, be);
  if constexpr (L >= 4) best_level<2>(bv, be);
  if constexpr (L >= 8) best_level<4>(bv, be);
  if constexpr (L >= 16) best_level<8>(bv, be);
  if constexpr (L >= 32) best_level<16>(bv, be);
  if constexpr (L >= 64) best_level<32>(bv, be);
}

template <int L, int V>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ idx,
                                                    float* __restrict__ prob) {
  constexpr int GROUPS_PER_WAVE = 64 / L;
  const int lane = threadIdx.x & 63;
  const int gl = lane & (L - 1);           // lane inside the token group
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int t = wave * GROUPS_PER_WAVE + lane / L;
  const bool active = t < T;

  float val[V];
  int ex[V];
  bool taken[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    ex[v] = gl + v * L;
    const bool ok = active && ex[v] < E;
    val[v] = ok ? logits[(size_t)t * E + ex[v]] : -INFINITY;
    taken[v] = !ok;                        // padding slots never win
  }

  float sel_v = 0.f;                       // lane j of the group keeps pick j
  int sel_e = 0;
  float first = 0.f;
  for (int j = 0; j < k; ++j) {
    // the sentinel (NaN, INT_MAX) loses to every candidate, NaN logits included
    float bv = __builtin_nanf("");
    int be = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (!taken[v] && better(val[v], ex[v], bv, be)) { bv = val[v]; be = ex[v]; }
    best_of_group<L>(bv, be);
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (ex[v] == be) taken[v] = true;
    if (gl == j) { sel_v = bv; sel_e = be; }
    if (j == 0) first = bv;
  }
  // softmax over the k picks, max = the first pick; sum in j order
  const float w = (gl < k) ? __expf(sel_v - first) : 0.f;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += __shfl(w, (lane & ~(L - 1)) + j, 64);
  if (active && gl < k) {
    idx[(size_t)t * k + gl] = sel_e;
    prob[(size_t)t * k + gl] = w / s;
  }
}

// Routing fused with the first half of the load-balancing loss (the pages
// fuse routing and the auxiliary-loss computation into one kernel: German
// technical summary, section 2 D).  Block b (16 wavefronts) takes the RA_TOK
// = 32 tokens from 32 b, wavefront w tokens 32 b + 2 w and 32 b + 2 w + 1
// (their loads issued together), lane l holding logits l, l+64, .. (V per
// lane).  Per token: the k picks and their probabilities are those of
// route_kernel (the same key; the same exp and j-order sum), and the token's
// softmax over all E logits (wave max, exp, wave sum) goes to LDS.  Then
// thread e adds the 32 tokens' values for expert e in the order of
// aux_partial_kernel (four runs of eight tokens from 0, then the four run sums
// pairwise), so partial[b][e] is bit-identical to its.
constexpr int RA_TOK = 32;

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int V>
__global__ __launch_bounds__(1024) void route_aux_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ prob,
                                                         float* __restrict__ partial) {
  __shared__ float contrib[RA_TOK][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int U = 2;  // tokens per wavefront
  const int t0 = blockIdx.x * RA_TOK + w * U;
  float val[U][V];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = lane + 64 * v;
      val[u][v] = t < T && e < E ? logits[(size_t)t * E + e] : -INFINITY;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u;
    const int tl = w * U + u;  // token within the block
    if (t >= T) {              // uniform across the wavefront: no contribution
#pragma unroll
      for (int v = 0; v < V; ++v) contrib[tl][lane + 64 * v] = 0.f;
      continue;
    }
    // the token's softmax over all E logits
    float m = val[u][0];
#pragma unroll
    for (int v = 1; v < V; ++v) m = fmaxf(m, val[u][v]);
    m = wave_max64(m);
    float sx[V], sum = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      sx[v] = lane + 64 * v < E ? __expf(val[u][v] - m) : 0.f;
      sum += sx[v];
    }
    sum = wave_sum64(sum);
#pragma unroll
    for (int v = 0; v < V; ++v) contrib[tl][lane + 64 * v] = sx[v] / sum;
    // the k picks (key: logit desc, index asc, NaN last) and their softmax
    bool taken[V];
#pragma unroll
    for (int v = 0; v < V; ++v) taken[v] = lane + 64 * v >= E;
    float sel_v = 0.f, first = 0.f;
    int sel_e = 0;
    for (int j = 0; j < k; ++j) {
      float bv = __builtin_nanf("");
      int be = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (!taken[v] && better(val[u][v], lane + 64 * v, bv, be)) { bv = val[u][v]; be = lane + 64 * v; }
      best_of_group<64>(bv, be);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (lane + 64 * v == be) taken[v] = true;
      if (lane == j) { sel_v = bv; sel_e = be; }
      if (j == 0) first = bv;
    }
    const float wt = lane < k ? __expf(sel_v - first) : 0.f;
    float ps = 0.f;
    for (int j = 0; j < k; ++j) ps += __shfl(wt, j, 64);
    if (lane < k) {
      idx[(size_t)t * k + lane] = sel_e;
      prob[(size_t)t * k + lane] = wt / ps;
    }
  }
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) {
    float run[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      run[r] = 0.f;
#pragma unroll
      for (int i = 0; i < RA_TOK / 4; ++i) run[r] += contrib[r * (RA_TOK / 4) + i][e];
    }
    partial[(size_t)blockIdx.x * E + e] = (run[0] + run[1]) + (run[2] + run[3]);
  }
}

template <int L, int V>
int launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* prob,
                 hipStream_t s) {
  constexpr int tokens_per_block = 256 / L;
  const int blocks = (T + tokens_per_block - 1) / tokens_per_block;
  route_kernel<L, V><<<blocks, 256, 0, s>>>(logits, T, E, k, idx, prob);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

int route_launch(const float* logits, int T, int E, int k, int32_t* idx, float* prob,
                 hipStream_t s) {
  if (E <= 1) return launch_route<1, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 2) return launch_route<2, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 4) return launch_route<4, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 8) return launch_route<8, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 16) return launch_route<16, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 32) return launch_route<32, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 64) return launch_route<64, 1>(logits, T, E, k, idx, prob, s);
  if (E <= 128) return launch_route<64, 2>(logits, T, E, k, idx, prob, s);
  return launch_route<64, 4>(logits, T, E, k, idx, prob, s);
}

int route_aux_launch(const float* logits, int T, int E, int k, int32_t* idx, float* prob,
                     float* partial, hipStream_t s) {
  const int blocks = (T + RA_TOK - 1) / RA_TOK;
  if (E <= 64) route_aux_kernel<1><<<blocks, 1024, 0, s>>>(logits, T, E, k, idx, prob, partial);
  else if (E <= 128) route_aux_kernel<2><<<blocks, 1024, 0, s>>>(logits, T, E, k, idx, prob, partial);
  else route_aux_kernel<4><<<blocks, 1024, 0, s>>>(logits, T, E, k, idx, prob, partial);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace tre
