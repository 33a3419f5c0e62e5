// Device-side tile schedule of the grouped GEMMs: no host synchronisation.
//
// The per-expert row counts exist only in device memory (offsets, produced by
// the permutation); every block derives its own tile from them, as the
// sync-free, device-initiated kernels of "Scalable Training of
// Mixture-of-Experts Models with Megatron Core" do (Spanish summary, section
// 2.3 C; German summary, section 2 D).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tre {

// Bijection on [0, n): block ids with the same value mod 8 (dispatched to the
// same XCD, each XCD with its own L2) get consecutive logical tile ids.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int x = i & 7, j = i >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + j;
}

struct TileInfo {
  int e;     // expert
  int row0;  // first permuted row of the tile (ragged M) or of the expert (wgrad)
  int rows;  // valid rows of the tile (ragged M) or rows of the expert (wgrad: K)
  int m0;    // M offset of the tile (wgrad)
  int n0;    // N-tile index (scaled to columns by the caller)
};

// Ragged-M decode for a 256-thread block and E <= 256 experts: expert e owns
// ceil(m_e / BM) M-tiles; tiles are numbered expert-major, N fastest.
// `scratch` is >= 8 ints of shared memory.  Returns false (uniformly for the
// block) when the block id is past the device-side tile count.
template <int BM>
__device__ __forceinline__ bool decode_ragged_m(const int32_t* __restrict__ offsets, int E, int NT, int* scratch,
                                TileInfo& ti) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int c = 0, o0 = 0, o1 = 0;
  if (tid < E) {
    o0 = offsets[tid];
    o1 = offsets[tid + 1];
    c = (o1 - o0 + BM - 1) / BM;
  }
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += scratch[i];
  const int total = (scratch[0] + scratch[1] + scratch[2] + scratch[3]) * NT;
  if ((int)blockIdx.x >= total) return false;
  const int logical = xcd_remap(blockIdx.x, total);
  const int g = logical / NT;
  const int excl = before + incl - c;
  if (c > 0 && g >= excl && g < excl + c) {
    scratch[4] = tid;
    scratch[5] = o0 + (g - excl) * BM;
    scratch[6] = min(BM, o1 - (o0 + (g - excl) * BM));
  }
  __syncthreads();
  ti.e = scratch[4];
  ti.row0 = scratch[5];
  ti.rows = scratch[6];
  ti.m0 = 0;
  ti.n0 = logical % NT;
  return true;
}

}  // namespace tre
