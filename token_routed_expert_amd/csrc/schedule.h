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

// Ragged-M decode for a block of NWAVES wavefronts and E <= 64 * NWAVES
// experts: expert e owns ceil(m_e / BM) M-tiles; tiles are numbered
// expert-major.  `scratch` is >= NWAVES + 4 ints of shared memory.
// Returns false (uniformly for the block) when the block id is past the
// device-side tile count.
template <int BM, int NWAVES = 4>
__device__ __forceinline__ bool decode_ragged_m(const int32_t* __restrict__ offsets, int E, int NT,
                                                int* scratch, TileInfo& ti) {
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
  int before = 0, total_m = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    if (i < w) before += scratch[i];
    total_m += scratch[i];
  }
  const int total = total_m * NT;
  if ((int)blockIdx.x >= total) return false;
  const int logical = xcd_remap(blockIdx.x, total);
  // expert e owns logical tiles [excl * NT, (excl + c) * NT), N-tile-major
  // with the M-tile fastest: tiles that share an expert's weight strip run
  // side by side, and a split across dispatch rounds re-reads the (smaller)
  // activation rows rather than the weights
  const int excl = before + incl - c;
  if (c > 0 && logical >= excl * NT && logical < (excl + c) * NT) {
    const int local = logical - excl * NT;
    const int mt = local % c;
    scratch[NWAVES] = tid;
    scratch[NWAVES + 1] = o0 + mt * BM;
    scratch[NWAVES + 2] = min(BM, o1 - (o0 + mt * BM));
    scratch[NWAVES + 3] = local / c;
  }
  __syncthreads();
  ti.e = scratch[NWAVES];
  ti.row0 = scratch[NWAVES + 1];
  ti.rows = scratch[NWAVES + 2];
  ti.m0 = 0;
  ti.n0 = scratch[NWAVES + 3];
  return true;
}


// Persistent blocks: every block walks the tile list with a stride of the
// grid size, so the ragged-M decode is split into a block-wide prefix sum of
// the experts' M-tile counts, computed once per block, and a per-tile lookup.
// incl[e] = sum over e' <= e of ceil(m_e' / BM), written to shared memory
// (E <= 64 * NWAVES); `scratch` is >= NWAVES ints of shared memory.  Returns
// the total number of M-tiles (uniform for the block).
template <int BM, int NWAVES>
__device__ __forceinline__ int mtile_prefix(const int32_t* __restrict__ offsets, int E, int* incl,
                                            int* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int c = 0;
  if (tid < E) c = (offsets[tid + 1] - offsets[tid] + BM - 1) / BM;
  int v = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) scratch[w] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    if (i < w) before += scratch[i];
    total += scratch[i];
  }
  if (tid < E) incl[tid] = before + v;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(total);
}

// Tile `logical` of the ragged-M numbering (expert-major; inside an expert
// N-tile-major with the M-tile fastest, as decode_ragged_m) from the prefix
// of mtile_prefix.  Expert e owns logical tiles [excl_e * NT, incl_e * NT),
// so it is the smallest e with incl[e] > logical / NT; one wavefront finds it
// with a ballot over 64 experts at a time.  The caller guarantees
// logical < incl[E-1] * NT.  ti.n0 is the N-tile index.
__device__ __forceinline__ void ragged_tile(const int32_t* __restrict__ offsets, const int* incl,
                                            int E, int NT, int BM, int logical, TileInfo& ti) {
  const int lane = threadIdx.x & 63;
  const int G = logical / NT;
  int e = E - 1;
  for (int base = 0; base < E; base += 64) {
    const int x = base + lane;
    const uint64_t m = __ballot(x < E && incl[x] > G);
    if (m) {
      e = base + (int)__builtin_ctzll(m);
      break;
    }
  }
  e = __builtin_amdgcn_readfirstlane(e);
  const int excl = __builtin_amdgcn_readfirstlane(e > 0 ? incl[e - 1] : 0);
  const int c = __builtin_amdgcn_readfirstlane(incl[e]) - excl;
  const int local = logical - excl * NT;
  const int mt = local % c;
  const int o0 = offsets[e], o1 = offsets[e + 1];
  ti.e = e;
  ti.row0 = o0 + mt * BM;
  ti.rows = min(BM, o1 - ti.row0);
  ti.m0 = 0;
  ti.n0 = local / c;
}

}  // namespace tre
