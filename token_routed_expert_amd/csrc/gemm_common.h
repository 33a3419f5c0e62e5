// Pieces shared by the grouped-GEMM kernels: compile-time loops, buffer
// resources and LDS DMA, barriers and wait counts, and the bf16 epilogue that
// turns a wavefront's fp32 accumulators into stored outputs.
#pragma once

#include "common.h"
#include "internal.h"
#include "schedule.h"

namespace tre {
namespace gemm {

template <int V>
struct IntC {
  static constexpr int value = V;
};
// Compile-time loop: f(IntC<B>), ..., f(IntC<E-1>); indices stay constants.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

typedef int rsrc_t __attribute__((ext_vector_type(4)));  // buffer resource, 4 SGPRs
typedef short i16x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero.  Word 3 selects the 32-bit data format that raw loads need.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// c ? x : y for buffer resources, component by component (uniform c).
__device__ __forceinline__ rsrc_t pick(bool c, rsrc_t x, rsrc_t y) {
  rsrc_t r;
  r[0] = c ? x[0] : y[0];
  r[1] = c ? x[1] : y[1];
  r[2] = c ? x[2] : y[2];
  r[3] = c ? x[3] : y[3];
  return r;
}

// A resource chosen at run time between uniform ones, kept in SGPRs.
__device__ __forceinline__ rsrc_t uniform_rsrc(rsrc_t r) {
  rsrc_t u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

// 16 bytes per lane from `r` at byte offset `voff` into LDS at byte address
// m0 + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the LDS address).
// Issued through inline assembly so that the compiler does not treat it as
// an LDS store it must drain before every LDS read: the kernel orders these
// loads with its own s_waitcnt vmcnt + s_barrier.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0)
               : "memory");
}

// 4 bytes per lane from `r` at byte offset `voff` into LDS at byte address
// m0 + 4 * lane (buffer_load_dword ... lds), ordered like dma16.
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0)
               : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding load); the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt on the vector-memory counter only.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v_permlane16_swap on two registers: x keeps lanes 0-15 and 32-47 and takes
// y's lanes 0-15 / 32-47 into its lanes 16-31 / 48-63; y receives the rest.
__device__ __forceinline__ void swap16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

// Two 16x16 accumulator fragments x (columns 0-15) and y (columns 16-31) with
// lane l holding columns 4(l >> 4)..+3 of row l & 15 -> the lane's 8
// consecutive columns pc..pc+7 (pc = 16((l >> 4) & 1) + 8(l >> 5)) as bf16.
__device__ __forceinline__ u32x4_t pair_bf16(const f32x4_t& x, const f32x4_t& y) {
  uint32_t x0 = pack_bf16x2(x[0], x[1]), x1 = pack_bf16x2(x[2], x[3]);
  uint32_t y0 = pack_bf16x2(y[0], y[1]), y1 = pack_bf16x2(y[2], y[3]);
  swap16(x0, y0);
  swap16(x1, y1);
  return u32x4_t{x0, x1, y0, y1};
}

// The same redistribution in fp32: afterwards x holds columns pc..pc+3 and
// y columns pc+4..pc+7.
__device__ __forceinline__ void pair_f32(f32x4_t& x, f32x4_t& y) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t a = __float_as_uint(x[q]), b = __float_as_uint(y[q]);
    swap16(a, b);
    x[q] = __uint_as_float(a);
    y[q] = __uint_as_float(b);
  }
}


// Writes a wavefront's FM x FN accumulator fragments (16x16 each, the
// wavefront covering rows wm*WM.. and columns wn*WN.. of the block tile) as
// the product's bf16 outputs, with the fused epilogues: SwiGLU for fc1
// forward (a lane holds a in fragment j and b of the same column in j + FN/2),
// the SwiGLU backward for fc2 dgrad (reads the saved a|b), plain stores
// otherwise.  Rows past the tile's valid rows and column pairs past N are
// skipped.
//
// RS (row-scaled products, routing probabilities applied before W2; only
// fc1 forward and fc2 dgrad differ): fc1 forward stores h = p_r silu(a) b;
// fc2 dgrad takes its accumulators as dh' = dO' W2^T for the unscaled dO',
// applies the SwiGLU backward to dh = p_r dh' (and, when args.h_out is set,
// stores the recomputed p_r silu(a) b there), and adds <silu(a) b, dh'> over
// the tile's columns into args.dp_part[r][n-tile] (per lane over its columns
// in order, then xor shuffles over the 4 lanes of a row, then the WAVES_N
// wavefronts of a row in order through `red`, [WAVES_N][256] floats of LDS;
// every wavefront of the block must call store_tile).
//
// LINES (plain-store products, FN == 4: a wavefront covers 64 columns, one
// 128-byte line of a bf16 row): lanes l and l + 8 of each row of 16 lanes
// trade pair halves (one DPP rotate per dword), so that each store
// instruction writes whole lines of 8 rows instead of half lines of 16 rows.
template <int OP, int FM, int FN, int WM, int WN, bool RAGGED, bool RS = false, bool LINES = false>
__device__ __forceinline__ void store_tile(const GemmArgs& args, const f32x4_t (&acc)[FM][FN],
                                           const TileInfo& ti, int M, int N, int wm, int wn,
                                           int lane, float* red = nullptr) {
  constexpr int HB = FN / 2;
  const int d = args.d, f = args.f;
  const size_t e = (size_t)ti.e;
  // lane holds C[m][n + 0..3] with m = wm*WM + i*16 + (lane & 15),
  // n = wn*WN + j*16 + 4*(lane >> 4).  Fragments are taken in pairs (j, j+1):
  // v_permlane16_swap leaves each lane with 8 consecutive columns of the
  // 32-column pair, starting at column pc, so every store is 16 bytes and a
  // row receives 64 contiguous bytes per instruction.
  const int lm = lane & 15;
  const int pc = ((lane >> 4) & 1) * 16 + (lane >> 5) * 8;
  static_for<0, FM>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = I.value;
    const int m = wm * WM + i * 16 + lm;  // row within the tile
    const bool row_ok = RAGGED ? (m < ti.rows) : (ti.m0 + m < M);
    float pr = 1.0f, dp = 0.0f;            // RS: the row's probability, <h, dh'> partial
    if constexpr (RS) pr = row_ok ? args.row_prob[ti.row0 + m] : 0.0f;
    if constexpr (OP == OP_FC1_FWD) {
      // pairs jp < HB/2 hold W1 columns (a), pair jp + HB/2 the same W3 columns (b)
      static_for<0, HB / 2>([&](auto JP) __attribute__((always_inline)) {
        constexpr int j0 = 2 * JP.value;
        const f32x4_t a0 = acc[i][j0], a1 = acc[i][j0 + 1];
        const f32x4_t b0v = acc[i][j0 + HB], b1v = acc[i][j0 + HB + 1];
        f32x4_t h0, h1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h0[q] = silu_f32(a0[q]) * b0v[q];
          h1[q] = silu_f32(a1[q]) * b1v[q];
          if constexpr (RS) {
            h0[q] *= pr;
            h1[q] *= pr;
          }
        }
        const u32x4_t av = pair_bf16(a0, a1), bv = pair_bf16(b0v, b1v), hv = pair_bf16(h0, h1);
        const int fcol = ti.n0 / 2 + (wn * HB + j0) * 16 + pc;
        if (row_ok) {
          const size_t row = (size_t)(ti.row0 + m);
          bf16_t* ab = (bf16_t*)args.ab_out + row * (2 * (size_t)f);
          *(u32x4_t*)(ab + fcol) = av;
          *(u32x4_t*)(ab + f + fcol) = bv;
          *(u32x4_t*)((bf16_t*)args.h_out + row * (size_t)f + fcol) = hv;
        }
      });
    } else if constexpr (LINES) {
      static_assert(FN == 4 && !RS && OP != OP_FC2_DGRAD, "whole-line stores: plain products, 64 columns");
      // lane l < 8 keeps pair 0 (columns 0..31) of row l and receives pair 0
      // of row l + 8; lane l >= 8 keeps pair 1 (columns 32..63) of row l and
      // receives pair 1 of row l - 8.  Instruction H then writes rows 8H..8H+7.
      const bool hi = lm >= 8;
      const u32x4_t v0 = pair_bf16(acc[i][0], acc[i][1]);
      const u32x4_t v1 = pair_bf16(acc[i][2], acc[i][3]);
      u32x4_t w0, w1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t snd = hi ? v0[q] : v1[q];
        // row_ror:8 inside each row of 16 lanes: lane l reads lane l ^ 8
        const uint32_t rcv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd, 0x128, 0xF, 0xF, false);
        w0[q] = hi ? rcv : v0[q];
        w1[q] = hi ? v1[q] : rcv;
      }
      const int colp = ti.n0 + wn * WN + (hi ? 32 : 0);  // first column of the lane's pair
      const int col = colp + pc;
      static_for<0, 2>([&](auto H) __attribute__((always_inline)) {
        const int mh = wm * WM + i * 16 + 8 * H.value + (lm & 7);  // row within the tile
        const bool ok = (RAGGED ? (mh < ti.rows) : (ti.m0 + mh < M)) && colp < N;
        if (ok) {
          bf16_t* out;
          if constexpr (OP == OP_FC2_FWD || OP == OP_FC1_DGRAD) {
            out = (bf16_t*)(OP == OP_FC2_FWD ? args.o_out : args.dXp_out) +
                  (size_t)(ti.row0 + mh) * d + col;
          } else if constexpr (OP == OP_FC2_WGRAD) {
            out = (bf16_t*)args.dW2 + e * (size_t)f * d + (size_t)(ti.m0 + mh) * d + col;
          } else {  // OP_FC1_WGRAD: each 32-column pair lies wholly in dW1 or in dW3
            const bool first = colp < f;
            out = (bf16_t*)(first ? args.dW1 : args.dW3) + e * (size_t)d * f +
                  (size_t)(ti.m0 + mh) * f + (first ? col : col - f);
          }
          *(u32x4_t*)out = H.value == 0 ? w0 : w1;
        }
      });
    } else {
      static_for<0, FN / 2>([&](auto JP) __attribute__((always_inline)) {
        constexpr int j0 = 2 * JP.value;
        const int col0 = ti.n0 + wn * WN + j0 * 16;  // first column of the pair (uniform)
        if (col0 < N) {
          const int col = col0 + pc;
          if constexpr (OP == OP_FC2_DGRAD) {
            f32x4_t x = acc[i][j0], y = acc[i][j0 + 1];
            pair_f32(x, y);  // dh at columns col + 0..3 (x), col + 4..7 (y)
            if (row_ok) {
              const size_t row = (size_t)(ti.row0 + m);
              const bf16_t* abr = (const bf16_t*)args.ab + row * (2 * (size_t)f);
              const u32x4_t av = *(const u32x4_t*)(abr + col);
              const u32x4_t bv = *(const u32x4_t*)(abr + f + col);
              float da[8], db[8], hr[8];
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const uint32_t aw = av[q >> 1], bw = bv[q >> 1];
                const float aq = (q & 1) ? hi_bf16(aw) : lo_bf16(aw);
                const float bq = (q & 1) ? hi_bf16(bw) : lo_bf16(bw);
                float c = q < 4 ? x[q] : y[q - 4];
                const float sg = sigmoid_f32(aq);
                if constexpr (RS) {
                  hr[q] = aq * sg * bq;  // h = silu(a) b from the saved a, b
                  dp = fmaf(hr[q], c, dp);
                  c *= pr;
                }
                da[q] = c * bq * sg * (1.0f + aq * (1.0f - sg));
                db[q] = c * aq * sg;
              }
              bf16_t* dab = (bf16_t*)args.dab_out + row * (2 * (size_t)f);
              *(u32x4_t*)(dab + col) = u32x4_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]),
                                               pack_bf16x2(da[4], da[5]), pack_bf16x2(da[6], da[7])};
              *(u32x4_t*)(dab + f + col) = u32x4_t{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3]),
                                                   pack_bf16x2(db[4], db[5]), pack_bf16x2(db[6], db[7])};
              if constexpr (RS) {
                if (args.h_out) {
#pragma unroll
                  for (int q = 0; q < 8; ++q) hr[q] *= pr;
                  *(u32x4_t*)((bf16_t*)args.h_out + row * (size_t)f + col) =
                      u32x4_t{pack_bf16x2(hr[0], hr[1]), pack_bf16x2(hr[2], hr[3]),
                              pack_bf16x2(hr[4], hr[5]), pack_bf16x2(hr[6], hr[7])};
                }
              }
            }
          } else {
            const u32x4_t v = pair_bf16(acc[i][j0], acc[i][j0 + 1]);
            if (row_ok) {
              bf16_t* out;
              if constexpr (OP == OP_FC2_FWD || OP == OP_FC1_DGRAD) {
                out = (bf16_t*)(OP == OP_FC2_FWD ? args.o_out : args.dXp_out) +
                      (size_t)(ti.row0 + m) * d + col;
              } else if constexpr (OP == OP_FC2_WGRAD) {
                out = (bf16_t*)args.dW2 + e * (size_t)f * d + (size_t)(ti.m0 + m) * d + col;
              } else {  // OP_FC1_WGRAD: the pair lies wholly in dW1 or in dW3 (f % 32 == 0)
                const bool first = col0 < f;
                out = (bf16_t*)(first ? args.dW1 : args.dW3) + e * (size_t)d * f +
                      (size_t)(ti.m0 + m) * f + (first ? col : col - f);
              }
              *(u32x4_t*)out = v;
            }
          }
        }
      });
      if constexpr (RS && OP == OP_FC2_DGRAD) {
        dp += __shfl_xor(dp, 16, 64);
        dp += __shfl_xor(dp, 32, 64);
        if (lane < 16) red[wn * 256 + m] = dp;
      }
    }
  });
  if constexpr (RS && OP == OP_FC2_DGRAD) {
    constexpr int WAVES_N = 256 / WN;
    // the partials were written with plain LDS stores, and other wavefronts
    // read them: they must have completed before the (fence-free) barrier
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    block_barrier();
    const int t = (int)threadIdx.x;
    if (t < 256 && t < ti.rows) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES_N; ++w) s += red[w * 256 + t];
      args.dp_part[(size_t)(ti.row0 + t) * (size_t)((f + 255) / 256) + ti.n0 / 256] = s;
    }
  }
}

}  // namespace gemm
}  // namespace tre
