// Top-k routing from router logits (Spanish summary of "Scalable Training of
// Mixture-of-Experts Models with Megatron Core", section 2.1: each token goes
// to its k best experts), with a softmax over the k selected logits.
//
// Layout: a group of L lanes (L = next power of two >= E, at most 64) owns one
// token; a 64-lane wavefront therefore routes 64/L tokens at once.  Lane i of
// a group holds logits e = i, i+L, i+2L, ... (V = ceil(E/L) <= 4 values for
// E <= 256), so a row is read with coalesced loads.  Each of the k rounds takes
// a lane-local best, then a butterfly (xor-shuffle) reduction inside the
// group; the winner's owner marks it taken.  The order key is (logit desc,
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
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
    }
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

}  // namespace tre
