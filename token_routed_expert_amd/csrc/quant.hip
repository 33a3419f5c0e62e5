// e4m3 block quantisers: OCP E4M3FN codes with one fp32 scale per block.
//
// The pages run the expert GEMMs in FP8 with a blockwise recipe while the
// router stays in high precision, and quantise weights straight from the
// fp32 masters (German technical summary of "Scalable Training of
// Mixture-of-Experts Models with Megatron Core", section 2 E; French summary,
// section 2 E).  They give no formula; the one used here, for a block B of
// values v:
//   amax = max |v| over B;  scale = 1 if amax == 0, else fp32(amax / 448);
//   code(v) = E4M3FN(fp32(v / scale)), round to nearest even, |x| >= 448
//   saturates to 448, subnormals kept, sign kept (-0 -> 0x80); an all-zero
//   block gets code +0 everywhere.
// Both divisions are IEEE fp32 divisions, so codes and scales are one
// well-defined function of the stored input values.
//
// Three block shapes, one kernel each:
//  * rows (1 x 128 along a row): activation operands of the forward and
//    data-gradient GEMMs, whose contraction runs along the row;
//  * tiles (128 x 128): expert weights, from fp32 masters; one copy serves
//    both orientations (the forward GEMMs read it MN-contiguous), and the
//    kernel can also write the transposed codes;
//  * token blocks (128 consecutive rows of one expert, per column): operands
//    of the weight-gradient GEMMs, whose contraction runs over the expert's
//    rows; written row-major [P][C] like the source (the GEMMs read them
//    MN-contiguous), optionally with the rows' 1 x 128 blocks in the same
//    pass.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace tre {

namespace {

constexpr float kE4M3Max = 448.0f;

// E4M3FN code of a finite fp32 value, from the format: sign bit, 4 exponent
// bits with bias 7, 3 mantissa bits; normals from 2^-6 to 448, subnormals
// m * 2^-9.  Round to nearest, ties to even; |v| >= 448 gives 448 (0x7e).
// gfx950's v_cvt_pk_fp8_f32 produces exactly these codes for |v| < 464 (a
// comparison over every fp32 value of magnitude below 2^9, both signs,
// subnormals and ties included) and NaN above, so the value is clamped to
// +-448 first (the sign of -0 is kept).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float c = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xffu;
}

__device__ __forceinline__ float block_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;
}

// Code of v in a block with scale `scale` (zero_block: the block's amax is 0).
__device__ __forceinline__ uint32_t quant1(float v, float scale, bool zero_block) {
  return zero_block ? 0u : e4m3_code(v / scale);
}

// The quotient v / s without a division per value.  With y = fp32(1 / s),
// the product q0 = fp32(v y) is corrected once by the remainder v - s q0,
// which one FMA gives exactly (the correction step of Markstein's division
// method).  For s >= kFastDivMin this equals the IEEE quotient fp32(v / s)
// whenever that quotient is at least 2^-14 in magnitude -- checked on the CPU
// over every bf16 pair |v| <= 448 s and over 1.3e9 fp32 pairs, among them
// values placed on and next to the midpoints between e4m3 codes.  Smaller
// quotients may differ in their last bits but give code +0 or -0 either way,
// and the sign is taken from v (the FMAs turn -0 into +0).
constexpr float kFastDivMin = 0x1p-90f;
__device__ __forceinline__ float div_by_scale(float v, float s, float y) {
  const float q0 = v * y;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, v), y, q0), v);
}
// quant1 through div_by_scale (FAST) or the IEEE division.
template <bool FAST>
__device__ __forceinline__ uint32_t quant1s(float v, float s, float y, bool zero_block) {
  return zero_block ? 0u : e4m3_code(FAST ? div_by_scale(v, s, y) : v / s);
}

// Value q (0..7) of eight bf16 packed in four 32-bit words.
__device__ __forceinline__ float bf16_at(const u32x4_t& w, int q) {
  return __uint_as_float((q & 1) ? (w[q >> 1] & 0xffff0000u) : (w[q >> 1] << 16));
}

// Eight consecutive values as fp32 (non-temporal loads: every source value is
// read once).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  const u32x4_t w = __builtin_nontemporal_load((const u32x4_t*)p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const f32x4_t a = __builtin_nontemporal_load((const f32x4_t*)p);
  const f32x4_t b = __builtin_nontemporal_load((const f32x4_t*)(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// ---------------------------------------------------------------- rows
// 16 lanes per 128-value block (8 values each); block g covers values
// [128 g, 128 g + 128) of the row-major matrix (nblk = rows * cols / 128) and
// its scale is scales[g] (= [row][col / 128]).  A wavefront takes 16
// consecutive blocks: lane group k = lane / 16 takes blocks 4 j + k (j < 4),
// so each load instruction reads four neighbouring blocks in one piece and
// every lane has four loads in flight.  Blocks past nblk load as +0 and store
// nothing.
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ src, int64_t nblk,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16 + (lane >> 4);
  float v[4][8], sc[4], y[4];
  bool z[4], fast = true;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (g0 + 4 * j < nblk) {
      load8<T>(src + (g0 + 4 * j) * 128 + sub * 8, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    sc[j] = block_scale(m);
    y[j] = 1.0f / sc[j];
    z[j] = m == 0.0f;
    fast = fast && sc[j] >= kFastDivMin;
  }
  auto emit = [&](auto fst) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = g0 + 4 * j;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= quant1s<decltype(fst)::value>(v[j][i], sc[j], y[j], z[j]) << (8 * i);
        hi |= quant1s<decltype(fst)::value>(v[j][4 + i], sc[j], y[j], z[j]) << (8 * i);
      }
      if (g < nblk) {
        *(uint2*)(codes + g * 128 + sub * 8) = make_uint2(lo, hi);
        if (sub == 0) scales[g] = sc[j];
      }
    }
  };
  if (__all(fast))
    emit(std::true_type{});
  else
    emit(std::false_type{});
}

// ---------------------------------------------------------------- tiles
// One block per 128 x 128 tile of matrix e (grid: C/128, R/128, E).
// codes [E][R][C], codes_t [E][C][R] (may be NULL), scales [E][R/128][C/128].
// Thread (rg, cl) = (tid / 32, tid % 32) holds rows 16 rg .. 16 rg + 15 and
// columns 4 cl .. 4 cl + 3: float4 loads (a wavefront reads 2 rows of 512
// bytes), 4-byte row-major code stores, and per column 16 consecutive row
// codes -- one 16-byte LDS write into the transposed tile, which is then
// stored row by row.
__global__ __launch_bounds__(256) void quant_tiles_kernel(const float* __restrict__ W, int R, int C,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ codes_t,
                                                          float* __restrict__ scales) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tt[128][144];  // [col][row], padded rows
  const int cb = blockIdx.x, rb = blockIdx.y, e = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int rg = tid >> 5, col = (tid & 31) * 4;
  const size_t mat = (size_t)e * R * C;
  const float* Wt = W + mat + (size_t)rb * 128 * C + (size_t)cb * 128;
  f32x4_t v[16];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = __builtin_nontemporal_load((const f32x4_t*)(Wt + (size_t)(16 * rg + i) * C + col));
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fabsf(v[i][q]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = block_scale(m);
  const float y = 1.0f / sc;
  const bool z = m == 0.0f;
  uint8_t* Ct = codes + mat + (size_t)rb * 128 * C + (size_t)cb * 128;
  uint32_t colw[4][4] = {};  // [column q][word w]: rows 16 rg + 4 w .. + 3 of column col + q
  const bool fast = sc >= kFastDivMin;  // the same in every lane
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c[4];
    if (fast) {
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = quant1s<true>(v[i][q], sc, y, z);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = quant1(v[i][q], sc, z);
    }
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w |= c[q] << (8 * q);
      colw[q][i >> 2] |= c[q] << (8 * (i & 3));
    }
    *(uint32_t*)(Ct + (size_t)(16 * rg + i) * C + col) = w;
  }
  if (tid == 0) scales[((size_t)e * (R / 128) + rb) * (C / 128) + cb] = sc;
  if (codes_t == nullptr) return;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(u32x4_t*)&tt[col + q][16 * rg] = u32x4_t{colw[q][0], colw[q][1], colw[q][2], colw[q][3]};
  __syncthreads();
  // transposed tile: row c of codes_t holds column c of the tile (128 bytes)
  uint8_t* Tt = codes_t + mat + (size_t)cb * 128 * R + (size_t)rb * 128;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int id = pass * 256 + tid;
    const int c = id >> 3, r16 = (id & 7) * 16;
    *(u32x4_t*)(Tt + (size_t)c * R + r16) = *(const u32x4_t*)&tt[c][r16];
  }
}

// ---------------------------------------------------------------- token blocks
// blk[e] = sum_{e' < e} ceil(m_e' / 128), blk[E] = number of blocks.
__global__ __launch_bounds__(256) void tokblk_table_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int32_t* __restrict__ blk) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int c = 0;
  if (tid < E) c = (offsets[tid + 1] - offsets[tid] + 127) / 128;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  if (tid < E) blk[tid] = before + incl - c;
  if (tid == E - 1) blk[E] = before + incl;
}

// One block per (token block b, 128 columns cb): rows r0 .. r0 + nr - 1 of the
// expert that owns block b (source row src_row[r] if src_row is given, else
// r), columns cb*128 .. +127 of a bf16 [.][C] matrix.  Writes
//   codes[r][c] for the block's rows r (row-major [P][C], as the source);
//   scales[b][c].
// Blocks with b >= blk[E] leave at once.  The grid is one-dimensional with cb
// varying fastest: workgroups launched together read neighbouring 256-byte
// pieces of the same source rows (b fastest, where concurrent workgroups read
// rows far apart, measured 10 % slower).
//
// Thread (rq, cg) = (tid / 16, tid % 16) holds rows 8 rq .. 8 rq + 7 and
// columns 8 cg .. 8 cg + 7: a load instruction reads four 256-byte row
// pieces, wavefront w holds rows 32 w .. 32 w + 31, and each row's eight
// codes leave the thread as one 8-byte store (a wavefront's store covers four
// 128-byte row pieces).

// Owner expert of token block b: the last e with blk[e] <= b, which (blk being
// non-decreasing with blk[0] = 0 <= b) is the number of e < E with
// blk[e] <= b, less one -- counted with ballots over independent loads rather
// than found by a binary search whose loads depend on each other.
__device__ __forceinline__ int tokblk_owner(const int32_t* __restrict__ blk, int E, int b) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    int x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 64 * j + lane;
      x[j] = e < E ? blk[e] : INT32_MAX;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) n += __popcll(__ballot(x[j] <= b));
  }
  return n - 1;
}

// Rows 8 rq .. 8 rq + 7 as loaded (bf16 pairs; rows past nr are +0) and the
// per-column |max| over the wavefront's 32 rows.  The values stay packed
// until they are quantised (about 64 VGPRs: seven or eight workgroups per CU
// where unpacked values allowed four).
__device__ __forceinline__ void tokblk_load(const bf16_t* __restrict__ src,
                                            const int32_t* __restrict__ src_row, int r0, int nr,
                                            int C, int cb, int rq, int cg, u32x4_t (&raw)[8],
                                            float (&m)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * rq + i;
    if (r < nr) {
      const int s = src_row ? src_row[r0 + r] : r0 + r;
      raw[i] = __builtin_nontemporal_load(
          (const u32x4_t*)(src + (size_t)s * C + (size_t)cb * 128 + 8 * cg));
    } else {
      raw[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // |max| on the bit patterns: for bf16 values other than NaN, the magnitude
  // order is the integer order of the bits without the sign
  uint32_t mb[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) mb[q] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      mb[2 * h] = max(mb[2 * h], raw[i][h] & 0x7fffu);
      mb[2 * h + 1] = max(mb[2 * h + 1], (raw[i][h] >> 16) & 0x7fffu);
    }
  // lanes l, l ^ 16, l ^ 32, l ^ 48 share columns
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mb[q] = max(mb[q], (uint32_t)__shfl_xor((int)mb[q], 16, 64));
    mb[q] = max(mb[q], (uint32_t)__shfl_xor((int)mb[q], 32, 64));
    m[q] = __uint_as_float(mb[q] << 16);
  }
}

// ROWS: the same pass also writes the 1 x 128 row blocks of its rows (the
// blocks of moe_quantize_rows: each row's 128 columns of the workgroup are one
// block), rcodes [P][C] and rscales [P][C/128], bit-identical to
// quant_rows_kernel's.  A row's maximum comes from the 16 lanes that hold it.
template <bool ROWS>
__global__ __launch_bounds__(256) void quant_tokblk_kernel(
    const bf16_t* __restrict__ src, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ blk, int E, int C,
    uint8_t* __restrict__ codes, float* __restrict__ scales, uint8_t* __restrict__ rcodes,
    float* __restrict__ rscales) {
  __shared__ __attribute__((aligned(16))) float red[4][128];
  const int ncb = C >> 7, b = (int)blockIdx.x / ncb, cb = (int)blockIdx.x - b * ncb;
  const int tid = threadIdx.x;
  if (b >= blk[E]) return;
  const int e = tokblk_owner(blk, E, b);
  const int r0 = offsets[e] + (b - blk[e]) * 128;
  const int nr = min(128, offsets[e + 1] - r0);
  const int cg = tid & 15, rq = tid >> 4, w = tid >> 6;
  u32x4_t raw[8];
  float m[8];
  tokblk_load(src, src_row, r0, nr, C, cb, rq, cg, raw, m);
  if ((tid & 63) < 16) {
    *(f32x4_t*)&red[w][8 * cg] = f32x4_t{m[0], m[1], m[2], m[3]};
    *(f32x4_t*)&red[w][8 * cg + 4] = f32x4_t{m[4], m[5], m[6], m[7]};
  }
  __syncthreads();
  float sc[8], y[8];
  bool z[8], fast = true;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4_t a = *(const f32x4_t*)&red[0][8 * cg + 4 * h];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      const f32x4_t t = *(const f32x4_t*)&red[k][8 * cg + 4 * h];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = fmaxf(a[j], t[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * h + j;
      z[q] = a[j] == 0.0f;
      sc[q] = block_scale(a[j]);
      y[q] = 1.0f / sc[q];
      fast = fast && sc[q] >= kFastDivMin;
    }
  }
  if (tid < 16) {
    float* so = scales + (size_t)b * C + (size_t)cb * 128 + 8 * cg;
    *(f32x4_t*)so = f32x4_t{sc[0], sc[1], sc[2], sc[3]};
    *(f32x4_t*)(so + 4) = f32x4_t{sc[4], sc[5], sc[6], sc[7]};
  }
  uint8_t* const dst = codes + (size_t)r0 * C + (size_t)cb * 128 + 8 * cg;
  auto emit = [&](auto fst) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo |= quant1s<decltype(fst)::value>(bf16_at(raw[i], q), sc[q], y[q], z[q]) << (8 * q);
        hi |= quant1s<decltype(fst)::value>(bf16_at(raw[i], 4 + q), sc[4 + q], y[4 + q], z[4 + q])
              << (8 * q);
      }
      const int r = 8 * rq + i;
      if (r < nr) *(uint2*)(dst + (size_t)r * C) = make_uint2(lo, hi);
    }
  };
  if (__all(fast))
    emit(std::true_type{});
  else
    emit(std::false_type{});
  if constexpr (ROWS) {
    float rsc[8], ry[8];
    bool rz[8], rfast = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float mx = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) mx = fmaxf(mx, fabsf(bf16_at(raw[i], q)));
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
      rsc[i] = block_scale(mx);
      ry[i] = 1.0f / rsc[i];
      rz[i] = mx == 0.0f;
      rfast = rfast && rsc[i] >= kFastDivMin;
    }
    uint8_t* const rdst = rcodes + (size_t)r0 * C + (size_t)cb * 128 + 8 * cg;
    float* const rsdst = rscales + (size_t)r0 * (C >> 7) + cb;
    auto emit_rows = [&](auto fst) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lo |= quant1s<decltype(fst)::value>(bf16_at(raw[i], q), rsc[i], ry[i], rz[i]) << (8 * q);
          hi |= quant1s<decltype(fst)::value>(bf16_at(raw[i], 4 + q), rsc[i], ry[i], rz[i]) << (8 * q);
        }
        const int r = 8 * rq + i;
        if (r < nr) {
          *(uint2*)(rdst + (size_t)r * C) = make_uint2(lo, hi);
          if (cg == 0) rsdst[(size_t)r * (C >> 7)] = rsc[i];
        }
      }
    };
    if (__all(rfast))
      emit_rows(std::true_type{});
    else
      emit_rows(std::false_type{});
  }
}

// ================================================================ MXFP8
// OCP microscaling: blocks of 32 values along the contraction axis share a
// power-of-two scale 2^s, stored as the E8M0 byte s + 127; s is the smallest
// integer with amax <= 448 * 2^s (clamped to [-127, 127]; 0 for an all-zero
// block), so the block maximum maps into (224, 448] and nothing saturates.
// Codes are E4M3(v * 2^-s) (exact scaling), all-zero blocks give +0 codes.

// amax = f * 2^E, f in [1, 2): s = E - 8 if f <= 1.75 (448 = 1.75 * 2^8), else E - 7.
__device__ __forceinline__ int mx_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0) return 0;
  const int ef = (int)(u >> 23);
  if (ef == 0) return -127;  // subnormal amax: below any reachable scale
  const int s = ef - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return s < -127 ? -127 : s;
}
// 2^-s as an fp32 (s in [-127, 120])
__device__ __forceinline__ float mx_inv(int s) { return __uint_as_float((uint32_t)(127 - s) << 23); }
__device__ __forceinline__ uint32_t mx_code(float v, float inv, bool zero_block) {
  return zero_block ? 0u : e4m3_code(v * inv);
}

// 1 x 32 blocks along rows: 4 lanes per block (8 values each); block g covers
// values [32 g, 32 g + 32), scale byte sb[g].  A wavefront takes 64
// consecutive blocks: lane group k = lane / 4 takes blocks 16 j + k (j < 4),
// as in quant_rows_kernel.
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_mx_kernel(const T* __restrict__ src, int64_t nblk,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ sb) {
  const int lane = threadIdx.x & 63, sub = lane & 3;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64 + (lane >> 2);
  float v[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (g0 + 16 * j < nblk) {
      load8<T>(src + (g0 + 16 * j) * 32 + sub * 8, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t g = g0 + 16 * j;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
    m = fmaxf(m, __shfl_xor(m, 1, 4));
    m = fmaxf(m, __shfl_xor(m, 2, 4));
    const int s = mx_exp(m);
    const float inv = mx_inv(s);
    const bool z = m == 0.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= mx_code(v[j][i], inv, z) << (8 * i);
      hi |= mx_code(v[j][4 + i], inv, z) << (8 * i);
    }
    if (g < nblk) {
      *(uint2*)(codes + g * 32 + sub * 8) = make_uint2(lo, hi);
      if (sub == 0) sb[g] = (uint8_t)(s + 127);
    }
  }
}

// Both MX orientations of expert weights from the fp32 masters, one block per
// 128 x 128 tile (grid: C/128, R/128, E).  Row blocks (1 x 32 along a row):
// codes [E][R][C], bytes sb [E][R][C/32].  Column blocks (32 x 1 along a
// column): codes_t [E][C][R], bytes sbt [E][C][R/32].  Thread (rg, cl) =
// (tid / 32, tid % 32) holds rows 16 rg .. + 15 and columns 4 cl .. + 3: a row
// block spans the 8 lanes cl / 8 = const (xor shuffles 1, 2, 4), a column
// block the row groups rg = 2 g, 2 g + 1 (lanes l and l + 32, xor 32).  The
// scale bytes leave as aligned 32-bit words (a row's four 32-column blocks,
// gathered by shuffles; a column's four 32-row blocks, through LDS) rather
// than as single bytes.  Held to 128 VGPRs (four workgroups per CU rather
// than three; no spills): 4 % faster.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void quant_weights_mx_kernel(
    const float* __restrict__ W, int R, int C, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ sb, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ sbt) {
  __shared__ __attribute__((aligned(16))) uint8_t tt[128][144];  // [col][row], padded rows
  __shared__ __attribute__((aligned(4))) uint8_t cs[128][4];       // column scales [col][32-row block]
  const int cb = blockIdx.x, rb = blockIdx.y, e = blockIdx.z;
  const int tid = threadIdx.x;
  const int rg = tid >> 5, cl = tid & 31, col = cl * 4;
  const int lane = tid & 63, lbase = lane & 32;  // the row's 32 lanes start at lbase
  const size_t mat = (size_t)e * R * C;
  const float* Wt = W + mat + (size_t)rb * 128 * C + (size_t)cb * 128;
  f32x4_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __builtin_nontemporal_load((const f32x4_t*)(Wt + (size_t)(16 * rg + i) * C + col));
  // row blocks
  uint8_t* Ct = codes + mat + (size_t)rb * 128 * C + (size_t)cb * 128;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    const int s = mx_exp(m);
    const float inv = mx_inv(s);
    const bool z = m == 0.0f;
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) w |= mx_code(v[i][q], inv, z) << (8 * q);
    const int r = rb * 128 + 16 * rg + i;
    *(uint32_t*)(Ct + (size_t)(16 * rg + i) * C + col) = w;
    // the row's four scale bytes (lanes lbase + 0, 8, 16, 24) as one word
    const uint32_t sbyte = (uint32_t)(s + 127);
    uint32_t sw = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) sw |= ((uint32_t)__shfl((int)sbyte, lbase + 8 * k, 64) & 0xffu) << (8 * k);
    if (cl == 0) *(uint32_t*)&sb[((size_t)e * R + r) * (C / 32) + cb * 4] = sw;
  }
  // column blocks: rows 32 g .. 32 g + 31 with g = rg / 2
  uint32_t colw[4][4] = {};  // [column q][word w]: rows 16 rg + 4 w .. + 3
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i][q]));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const int s = mx_exp(m);
    const float inv = mx_inv(s);
    const bool z = m == 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) colw[q][i >> 2] |= mx_code(v[i][q], inv, z) << (8 * (i & 3));
    if ((rg & 1) == 0) cs[col + q][rg >> 1] = (uint8_t)(s + 127);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(u32x4_t*)&tt[col + q][16 * rg] = u32x4_t{colw[q][0], colw[q][1], colw[q][2], colw[q][3]};
  __syncthreads();
  // a column's four 32-row scales of this tile as one word
  if (tid < 128)
    *(uint32_t*)&sbt[((size_t)e * C + (size_t)cb * 128 + tid) * (R / 32) + rb * 4] =
        *(const uint32_t*)&cs[tid][0];
  uint8_t* Tt = codes_t + mat + (size_t)cb * 128 * R + (size_t)rb * 128;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int id = pass * 256 + tid;
    const int c = id >> 3, r16 = (id & 7) * 16;
    *(u32x4_t*)(Tt + (size_t)c * R + r16) = *(const u32x4_t*)&tt[c][r16];
  }
}

// Token blocks in MX form: as quant_tokblk_kernel, with four 32-row scale
// blocks per column in each 128-row block.  codes [P][C] as there; scale
// bytes sbt [NB][C][4]: byte g of word (b, c) for rows 32 g .. 32 g + 31
// of block b (groups past the expert's rows: s = 0) -- one 4-byte word per
// (block, column), block-major like the e4m3 token-block scales, so a GEMM
// stage's words for 256 columns are 1 KB in a row.  With the thread layout of
// quant_tokblk_kernel, wavefront w holds exactly the rows of group w, so each
// group's maxima need only shuffles within the wavefront.
// ROWS: also the 1 x 32 row blocks of its rows, rcodes [P][C] and bytes
// rsb [P][C/32], bit-identical to quant_rows_mx_kernel's (a block is 4 lanes).
template <bool ROWS>
__global__ __launch_bounds__(256) void quant_tokblk_mx_kernel(
    const bf16_t* __restrict__ src, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ blk, int E, int C,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ sbt, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rsb) {
  __shared__ __attribute__((aligned(4))) uint8_t cs[128][4];  // [column][group]
  const int ncb = C >> 7, b = (int)blockIdx.x / ncb, cb = (int)blockIdx.x - b * ncb;
  const int tid = threadIdx.x;
  if (b >= blk[E]) return;
  const int e = tokblk_owner(blk, E, b);
  const int r0 = offsets[e] + (b - blk[e]) * 128;
  const int nr = min(128, offsets[e + 1] - r0);
  const int cg = tid & 15, rq = tid >> 4, g = tid >> 6;
  u32x4_t raw[8];
  float m[8];
  tokblk_load(src, src_row, r0, nr, C, cb, rq, cg, raw, m);
  float inv[8];
  bool z[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int s = mx_exp(m[q]);
    inv[q] = mx_inv(s);
    z[q] = m[q] == 0.0f;
    if ((tid & 63) < 16) cs[8 * cg + q][g] = (uint8_t)(s + 127);
  }
  uint8_t* const dst = codes + (size_t)r0 * C + (size_t)cb * 128 + 8 * cg;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo |= mx_code(bf16_at(raw[i], q), inv[q], z[q]) << (8 * q);
      hi |= mx_code(bf16_at(raw[i], 4 + q), inv[4 + q], z[4 + q]) << (8 * q);
    }
    const int r = 8 * rq + i;
    if (r < nr) *(uint2*)(dst + (size_t)r * C) = make_uint2(lo, hi);
  }
  if constexpr (ROWS) {
    uint8_t* const rdst = rcodes + (size_t)r0 * C + (size_t)cb * 128 + 8 * cg;
    uint8_t* const rsdst = rsb + (size_t)r0 * (C >> 5) + cb * 4 + (cg >> 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float mx = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) mx = fmaxf(mx, fabsf(bf16_at(raw[i], q)));
      mx = fmaxf(mx, __shfl_xor(mx, 1, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 4));
      const int s = mx_exp(mx);
      const float rinv = mx_inv(s);
      const bool rz = mx == 0.0f;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo |= mx_code(bf16_at(raw[i], q), rinv, rz) << (8 * q);
        hi |= mx_code(bf16_at(raw[i], 4 + q), rinv, rz) << (8 * q);
      }
      const int r = 8 * rq + i;
      if (r < nr) {
        *(uint2*)(rdst + (size_t)r * C) = make_uint2(lo, hi);
        if ((cg & 3) == 0) rsdst[(size_t)r * (C >> 5)] = (uint8_t)(s + 127);
      }
    }
  }
  __syncthreads();
  if (tid < 128)
    *(uint32_t*)&sbt[((size_t)b * C + (size_t)cb * 128 + tid) * 4] = *(const uint32_t*)&cs[tid][0];
}

}  // namespace

int quant_rows_mx_launch(const void* src, bool src_f32, int64_t rows, int64_t cols,
                         uint8_t* codes, uint8_t* sb, hipStream_t s) {
  const int64_t nblk = rows * (cols / 32);
  if (nblk == 0) return MOE_OK;
  const int64_t grid = (nblk + 255) / 256;
  if (src_f32)
    quant_rows_mx_kernel<float><<<dim3((unsigned)grid), 256, 0, s>>>((const float*)src, nblk,
                                                                      codes, sb);
  else
    quant_rows_mx_kernel<bf16_t><<<dim3((unsigned)grid), 256, 0, s>>>((const bf16_t*)src, nblk,
                                                                       codes, sb);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int quant_weights_mx_launch(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                            uint8_t* sb, uint8_t* codes_t, uint8_t* sbt, hipStream_t s) {
  if (E == 0) return MOE_OK;
  quant_weights_mx_kernel<<<dim3((unsigned)(C / 128), (unsigned)(R / 128), (unsigned)E), 256, 0,
                            s>>>(W, (int)R, (int)C, codes, sb, codes_t, sbt);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int quant_tokblk_mx_launch(const void* src, const int32_t* src_row, const int32_t* offsets,
                           const int32_t* blk, int E, int64_t P, int64_t C, uint8_t* codes,
                           uint8_t* sbt, hipStream_t s, uint8_t* rcodes, uint8_t* rsb) {
  const int64_t nb = tokblk_max_blocks(P, E);
  if (nb == 0) return MOE_OK;
  if (nb * (C / 128) > INT32_MAX) return MOE_ERR_UNSUPPORTED;  // one block per (b, cb)
  const dim3 grid((unsigned)(nb * (C / 128)));
  if (rcodes)
    quant_tokblk_mx_kernel<true><<<grid, 256, 0, s>>>((const bf16_t*)src, src_row, offsets, blk, E,
                                                      (int)C, codes, sbt, rcodes, rsb);
  else
    quant_tokblk_mx_kernel<false><<<grid, 256, 0, s>>>((const bf16_t*)src, src_row, offsets, blk, E,
                                                       (int)C, codes, sbt, nullptr, nullptr);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int quant_rows_launch(const void* src, bool src_f32, int64_t rows, int64_t cols, uint8_t* codes,
                      float* scales, hipStream_t s) {
  const int64_t nblk = rows * (cols / 128);
  if (nblk == 0) return MOE_OK;
  const int64_t grid = (nblk + 63) / 64;
  if (src_f32)
    quant_rows_kernel<float><<<dim3((unsigned)grid), 256, 0, s>>>((const float*)src, nblk, codes,
                                                                   scales);
  else
    quant_rows_kernel<bf16_t><<<dim3((unsigned)grid), 256, 0, s>>>((const bf16_t*)src, nblk,
                                                                    codes, scales);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int quant_tiles_launch(const float* W, int64_t E, int64_t R, int64_t C, uint8_t* codes,
                       uint8_t* codes_t, float* scales, hipStream_t s) {
  if (E == 0) return MOE_OK;
  quant_tiles_kernel<<<dim3((unsigned)(C / 128), (unsigned)(R / 128), (unsigned)E), 256, 0, s>>>(
      W, (int)R, (int)C, codes, codes_t, scales);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int64_t tokblk_max_blocks(int64_t P, int64_t E) { return P / 128 + E; }

int tokblk_table_launch(const int32_t* offsets, int E, int32_t* blk, hipStream_t s) {
  tokblk_table_kernel<<<1, 256, 0, s>>>(offsets, E, blk);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

int quant_tokblk_launch(const void* src, const int32_t* src_row, const int32_t* offsets,
                        const int32_t* blk, int E, int64_t P, int64_t C, uint8_t* codes,
                        float* scales, hipStream_t s, uint8_t* rcodes, float* rscales) {
  const int64_t nb = tokblk_max_blocks(P, E);
  if (nb == 0) return MOE_OK;
  if (nb * (C / 128) > INT32_MAX) return MOE_ERR_UNSUPPORTED;  // one block per (b, cb)
  const dim3 grid((unsigned)(nb * (C / 128)));
  if (rcodes)
    quant_tokblk_kernel<true><<<grid, 256, 0, s>>>((const bf16_t*)src, src_row, offsets, blk, E,
                                                   (int)C, codes, scales, rcodes, rscales);
  else
    quant_tokblk_kernel<false><<<grid, 256, 0, s>>>((const bf16_t*)src, src_row, offsets, blk, E,
                                                    (int)C, codes, scales, nullptr, nullptr);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace tre
