// Dispatch and combine on one GPU: the dropless token -> expert-contiguous row
// map, the row scatter, and the weighted gather (Spanish summary of "Scalable
// Training of Mixture-of-Experts Models with Megatron Core", section 2.1:
// dispatch and combine; German summary, section 1: dropless routing with
// dynamic per-expert sizes, and section 2 D: shapes stay on the device).
//
// Map construction is a stable counting sort without atomics on the result:
//   1. count: a block of 256 tokens (4 wavefronts) builds, per wavefront and
//      expert, a 64-bit mask of the lanes whose token picked that expert (LDS
//      OR is order-independent), and writes its per-expert totals to
//      blk[e][b];
//   2. scan: one block turns blk (expert-major) into exclusive prefix sums,
//      which are the first row of each (expert, block) pair, and writes
//      counts and offsets;
//   3. rank: each block rebuilds its masks; the row of (t, j) with expert e
//      is blk[e][b] + popcounts of lower wavefronts + popcount of the lower
//      lanes of its own wavefront.  Within an expert rows therefore ascend by
//      token, which is the one canonical order.
// Row moves are separate, fully parallel kernels with 16-byte accesses: the
// scatter reads each token row once and writes it k times; the combine
// gathers k rows and writes one.
#include "common.h"
#include "internal.h"

#include <atomic>

// Scratch of the allocation-free permutation map (moe_permute_noalloc): the
// per-(expert, token block) counts live here instead of in a caller
// workspace.  Every GPU holds its own copy until the process ends; calls on
// one GPU share it, so calls that overlap on one GPU race.  The map kernels
// overwrite every count they read, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[1 << 20];

namespace tre {

namespace {

constexpr int TOK_PER_BLOCK = 256;
constexpr int MAX_E = 256;

__device__ __forceinline__ void build_masks(unsigned long long (*mask)[MAX_E],
                                            const int32_t* __restrict__ idx, int T, int E, int k,
                                            int t, int w, int lane) {
  for (int i = threadIdx.x; i < 4 * MAX_E; i += blockDim.x) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[w][e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T, int E,
                                                    int k, int NB, int32_t* __restrict__ blk) {
  __shared__ unsigned long long mask[4][MAX_E];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * TOK_PER_BLOCK + threadIdx.x;
  build_masks(mask, idx, T, E, k, t, w, lane);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = __popcll(mask[0][e]) + __popcll(mask[1][e]) + __popcll(mask[2][e]) +
                  __popcll(mask[3][e]);
    blk[(size_t)e * NB + blockIdx.x] = c;
  }
}

// Single block of 1024 threads: exclusive scan of blk[E*NB] in place.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int E, int NB,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[16];
  __shared__ int total_s;
  const int N = E * NB;
  const int nt = blockDim.x;
  const int chunk = (N + nt - 1) / nt;
  const int i0 = min(N, (int)threadIdx.x * chunk), i1 = min(N, i0 + chunk);
  int local = 0;
  for (int i = i0; i < i1; ++i) local += blk[i];
  // inclusive scan across the wavefront
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wave_tot[i];
  if (threadIdx.x == nt - 1) total_s = before + incl;
  int run = before + incl - local;
  for (int i = i0; i < i1; ++i) {
    const int v = blk[i];
    blk[i] = run;
    run += v;
  }
  __syncthreads();
  const int total = total_s;
  for (int e = threadIdx.x; e < E; e += nt) {
    const int o0 = blk[(size_t)e * NB];
    const int o1 = (e + 1 < E) ? blk[(size_t)(e + 1) * NB] : total;
    offsets[e] = o0;
    counts[e] = o1 - o0;
  }
  if (threadIdx.x == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ idx, int T, int E,
                                                   int k, int NB, const int32_t* __restrict__ blk,
                                                   int32_t* __restrict__ row_of,
                                                   int32_t* __restrict__ token_of) {
  __shared__ unsigned long long mask[4][MAX_E];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * TOK_PER_BLOCK + threadIdx.x;
  build_masks(mask, idx, T, E, k, t, w, lane);
  if (t >= T) return;
  const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    if ((unsigned)e >= (unsigned)E) {  // no row for an index outside [0, E)
      row_of[(size_t)t * k + j] = -1;
      continue;
    }
    int before = __popcll(mask[w][e] & lower);
    for (int ww = 0; ww < w; ++ww) before += __popcll(mask[ww][e]);
    const int row = blk[(size_t)e * NB + blockIdx.x] + before;
    row_of[(size_t)t * k + j] = row;
    token_of[row] = t;
  }
}

// ---------------------------------------------------------------- row moves
template <typename T>
__device__ __forceinline__ void load_vec(const u32x4_t& v, float* out);
template <>
__device__ __forceinline__ void load_vec<float>(const u32x4_t& v, float* out) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void load_vec<bf16_t>(const u32x4_t& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ u32x4_t store_vec(const float* in);
template <>
__device__ __forceinline__ u32x4_t store_vec<float>(const float* in) {
  return u32x4_t{__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                    __float_as_uint(in[3])};
}
template <>
__device__ __forceinline__ u32x4_t store_vec<bf16_t>(const float* in) {
  return u32x4_t{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                    pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7])};
}

// Rows outside [0, P) (P = T * k, the grid's token count times k; the map
// marks an assignment without a row with -1) are skipped by every row move.
__device__ __forceinline__ bool row_ok(int row, int k) {
  return (unsigned)row < (unsigned)(gridDim.x * k);
}

// One block per token; C = 16-byte chunks per row.
template <typename T, bool SCALED>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4_t* __restrict__ src,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ scale,
                                                           int k, int C, u32x4_t* __restrict__ dst) {
  constexpr int N = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int32_t* rows = row_of + (size_t)t * k;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    const u32x4_t v = __builtin_nontemporal_load(&src[(size_t)t * C + c]);
    if (!SCALED) {
      for (int j = 0; j < k; ++j)
        if (row_ok(rows[j], k)) __builtin_nontemporal_store(v, &dst[(size_t)rows[j] * C + c]);
    } else {
      float x[N], y[N];
      load_vec<T>(v, x);
      for (int j = 0; j < k; ++j) {
        if (!row_ok(rows[j], k)) continue;
        const float p = scale[(size_t)t * k + j];
#pragma unroll
        for (int i = 0; i < N; ++i) y[i] = p * x[i];
        __builtin_nontemporal_store(store_vec<T>(y), &dst[(size_t)rows[j] * C + c]);
      }
    }
  }
}

template <typename T, bool WEIGHTED, bool ADD>
__global__ __launch_bounds__(512) void gather_rows_kernel(const u32x4_t* __restrict__ src,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ prob,
                                                          const u32x4_t* __restrict__ add, int k,
                                                          int C, u32x4_t* __restrict__ dst) {
  constexpr int N = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int32_t* rows = row_of + (size_t)t * k;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      if (!row_ok(rows[j], k)) continue;
      float v[N];
      load_vec<T>(__builtin_nontemporal_load(&src[(size_t)rows[j] * C + c]), v);
      if (WEIGHTED) {
        const float p = prob[(size_t)t * k + j];
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = fmaf(p, v[i], acc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] += v[i];
      }
    }
    if (ADD) {
      float a[N];
      load_vec<T>(add[(size_t)t * C + c], a);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += a[i];
    }
    __builtin_nontemporal_store(store_vec<T>(acc), &dst[(size_t)t * C + c]);
  }
}

// e4m3 dispatch: one block per token; C = 16-byte chunks of codes per row,
// KB = scales per row (one per 128 codes).  Codes and scales are bit copies.
__global__ __launch_bounds__(256) void scatter_e4m3_kernel(const u32x4_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           const int32_t* __restrict__ row_of,
                                                           int k, int C, int KB,
                                                           u32x4_t* __restrict__ dst_codes,
                                                           float* __restrict__ dst_scales) {
  const int t = blockIdx.x;
  const int32_t* rows = row_of + (size_t)t * k;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    const u32x4_t v = __builtin_nontemporal_load(&codes[(size_t)t * C + c]);
    for (int j = 0; j < k; ++j)
      if (row_ok(rows[j], k)) __builtin_nontemporal_store(v, &dst_codes[(size_t)rows[j] * C + c]);
  }
  for (int c = threadIdx.x; c < KB; c += blockDim.x) {
    const float v = scales[(size_t)t * KB + c];
    for (int j = 0; j < k; ++j)
      if (row_ok(rows[j], k)) dst_scales[(size_t)rows[j] * KB + c] = v;
  }
}

// Threads per block for a row of C 16-byte chunks: one wavefront per 64
// chunks, at most `cap` (measured on the Qwen3-shaped rows: 512 for the
// gathers of the combine, 256 for the scatter).
int block_for_chunks(int C, int cap) {
  int b = ((C + 63) / 64) * 64;
  return b > cap ? cap : b;
}

template <typename T>
int scatter_typed(const void* src, const int32_t* row_of, const float* scale, int T_, int k, int d,
                  void* dst, hipStream_t s) {
  const int C = d * (int)sizeof(T) / 16;
  const int bs = block_for_chunks(C, 256);
  if (scale)
    scatter_rows_kernel<T, true><<<T_, bs, 0, s>>>((const u32x4_t*)src, row_of, scale, k, C,
                                                   (u32x4_t*)dst);
  else
    scatter_rows_kernel<T, false><<<T_, bs, 0, s>>>((const u32x4_t*)src, row_of, scale, k, C,
                                                    (u32x4_t*)dst);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

template <typename T>
int gather_typed(const void* src, const int32_t* row_of, const float* prob, const void* add,
                 int T_, int k, int d, void* dst, hipStream_t s) {
  const int C = d * (int)sizeof(T) / 16;
  const int bs = block_for_chunks(C, 512);
  const u32x4_t* S = (const u32x4_t*)src;
  const u32x4_t* A = (const u32x4_t*)add;
  u32x4_t* D = (u32x4_t*)dst;
  if (prob && add)
    gather_rows_kernel<T, true, true><<<T_, bs, 0, s>>>(S, row_of, prob, A, k, C, D);
  else if (prob)
    gather_rows_kernel<T, true, false><<<T_, bs, 0, s>>>(S, row_of, prob, A, k, C, D);
  else if (add)
    gather_rows_kernel<T, false, true><<<T_, bs, 0, s>>>(S, row_of, prob, A, k, C, D);
  else
    gather_rows_kernel<T, false, false><<<T_, bs, 0, s>>>(S, row_of, prob, A, k, C, D);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

size_t permute_scratch_bytes() { return sizeof(scratch); }

// Device address of `scratch` on the current device: hipGetSymbolAddress once
// per device (with that device current), kept per device; host code passes
// this address to the kernels, never the array's host-side name.
int permute_scratch(void** ptr) {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    addr[dev].store(p, std::memory_order_release);  // concurrent first calls store the same value
  }
  *ptr = p;
  return MOE_OK;
}

size_t permute_ws_bytes(int64_t T, int64_t E) {
  const int64_t NB = (T + TOK_PER_BLOCK - 1) / TOK_PER_BLOCK;
  return align_up((size_t)(E * NB) * sizeof(int32_t), 256);
}

int permute_map_launch(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                       int32_t* row_of, int32_t* token_of, void* ws, hipStream_t s) {
  const int NB = (T + TOK_PER_BLOCK - 1) / TOK_PER_BLOCK;
  int32_t* blk = (int32_t*)ws;
  count_kernel<<<NB, 256, 0, s>>>(idx, T, E, k, NB, blk);
  TRE_LAUNCH_CHECK();
  scan_kernel<<<1, 1024, 0, s>>>(blk, E, NB, counts, offsets);
  TRE_LAUNCH_CHECK();
  rank_kernel<<<NB, 256, 0, s>>>(idx, T, E, k, NB, blk, row_of, token_of);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int permute_rows_launch(const void* src, const int32_t* row_of, const float* row_scale, int T,
                        int k, int d, int elem_bytes, void* dst, hipStream_t s) {
  if (elem_bytes == 4) return scatter_typed<float>(src, row_of, row_scale, T, k, d, dst, s);
  return scatter_typed<bf16_t>(src, row_of, row_scale, T, k, d, dst, s);
}

int unpermute_launch(const void* src, const int32_t* row_of, const float* prob, const void* add,
                     int T, int k, int d, int elem_bytes, void* dst, hipStream_t s) {
  if (elem_bytes == 4) return gather_typed<float>(src, row_of, prob, add, T, k, d, dst, s);
  return gather_typed<bf16_t>(src, row_of, prob, add, T, k, d, dst, s);
}

int permute_e4m3_launch(const uint8_t* codes, const float* scales, const int32_t* row_of, int T,
                        int k, int d, uint8_t* dst_codes, float* dst_scales, hipStream_t s) {
  const int C = d / 16, KB = d / 128;
  scatter_e4m3_kernel<<<T, block_for_chunks(C, 256), 0, s>>>((const u32x4_t*)codes, scales, row_of, k,
                                                         C, KB, (u32x4_t*)dst_codes, dst_scales);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace tre
