// Grouped expert GEMMs in bf16 on CDNA4 matrix cores (MFMA), fp32 accumulate.
//
// The pages bundle the many small per-expert GEMMs into grouped GEMMs (German
// summary of "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 2 D; Spanish summary, section 2.3 C) and keep the per-expert
// sizes on the device (same sections: sync-free, device-initiated kernels).
// Here one launch covers all experts of one product:
//
//   op            C (M x N)               A (M x K)        B (K x N)          ragged
//   FC1_FWD   [a|b]  rows x 2f            xp (K-contig)    W1|W3 (N-contig)    M
//   FC2_FWD    o     rows x d             h  (K-contig)    W2    (N-contig)    M
//   FC2_DGRAD  dH    rows x f             dO (K-contig)    W2^T  (K-contig)    M
//   FC1_DGRAD  dXp   rows x d             dab(K-contig)    [W1|W3]^T (K-contig) M
//   FC2_WGRAD  dW2   f x d                h^T (M-contig)   dO    (N-contig)    K
//   FC1_WGRAD  dW13  d x 2f               xp^T(M-contig)   dab   (N-contig)    K
//
// Tile schedule (no host sync): for ragged-M products every block reads the
// device offsets, counts ceil(m_e/BM) M-tiles per expert, scans them, and
// finds its (expert, M-tile, N-tile); blocks past the real tile count exit.
// Block ids are remapped so that the blocks one XCD runs at a time (ids with
// the same value mod 8) take consecutive tiles: they share A rows and expert
// weights in that XCD's L2.  Weight-gradient products have a fixed grid of
// E x (M/BM) x (N/BN) tiles; K is the expert's row count, 0 for an empty
// expert, which then writes zeros.
//
// Block tile BM x BN x 64 with 4 wavefronts in a 2x2 grid, each owning a
// (BM/2) x (BN/2) sub-tile of 16x16 MFMA blocks (v_mfma_f32_16x16x32_bf16).
// Operands are staged through LDS in a K-contiguous layout with a 16-byte row
// pad (144-byte pitch: conflict-free 16-byte fragment reads for any group of
// 16 lanes), double buffered: the global loads of stage k+1 are in flight
// while stage k is multiplied.  Operands that are MN-contiguous in memory are
// loaded as 8x8 element blocks and transposed in registers before the LDS
// store.  The MFMA computes C^T = B^T A^T so that each lane ends with four
// consecutive columns of one row: the epilogue stores 8 bytes per lane.
// The FC1_FWD tile interleaves W1 and W3 columns in groups of 16, so a lane
// holds a and b of the same element and applies SwiGLU in registers.
#include "common.h"
#include "internal.h"
#include "schedule.h"

namespace tre {

namespace {

constexpr int BK = 64;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row
constexpr int NTHREADS = 256;

// 8x8 transpose of bf16: in[j] holds 8 elements along MN at K row j; out[i]
// holds the 8 K elements of MN column i.
__device__ __forceinline__ void transpose8x8(const u32x4_t* in, u32x4_t* out) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int wsel = i >> 1;
    uint32_t r[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = in[2 * p][wsel], hi = in[2 * p + 1][wsel];
      r[p] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    out[i] = u32x4_t{r[0], r[1], r[2], r[3]};
  }
}

template <int OP>
struct OpTraits {
  static constexpr bool ragged_m = OP <= OP_FC2_WGRAD - 1;          // ops 0..3
  static constexpr bool a_kcontig = OP <= OP_FC1_DGRAD;             // ops 0..3
  static constexpr bool b_kcontig = OP == OP_FC2_DGRAD || OP == OP_FC1_DGRAD;
};

template <int OP, int BM, int BN>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmArgs args, int NT, int MT) {
  constexpr int WM = BM / 2, WN = BN / 2;       // wavefront sub-tile
  constexpr int FM = WM / 16, FN = WN / 16;     // 16x16 MFMA blocks per wavefront
  constexpr int STAGE = (BM + BN) * PITCH;
  constexpr int A_KROWS = BM * BK / 8 / NTHREADS;       // 16-byte chunks per thread (K-contig A)
  constexpr int B_KROWS = BN * BK / 8 / NTHREADS;
  constexpr int A_TBLK = (BM / 8) * (BK / 8) / NTHREADS;  // 8x8 blocks per thread (MN-contig A)
  constexpr int B_TBLK = (BN / 8) * (BK / 8) / NTHREADS;
  static_assert(A_KROWS >= 1 && B_KROWS >= 1, "tile too small for 256 threads");
  static_assert(A_TBLK >= 1 && B_TBLK >= 1, "tile too small for transposed loads");
  using TR = OpTraits<OP>;

  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int d = args.d, f = args.f;

  // ---------------------------------------------------------------- tile
  TileInfo ti;
  int K, M, N;
  if constexpr (TR::ragged_m) {
    if (!decode_ragged_m<BM>(args.offsets, args.E, NT, (int*)lds, ti)) return;
    ti.n0 *= BN;
    K = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? d : (OP == OP_FC2_FWD ? f : 2 * f);
    N = (OP == OP_FC1_FWD) ? 2 * f : (OP == OP_FC2_DGRAD ? f : d);
    M = ti.rows;
  } else {
    const int total = args.E * MT * NT;
    if ((int)blockIdx.x >= total) return;
    const int logical = xcd_remap(blockIdx.x, total);
    ti.e = logical / (MT * NT);
    const int rem = logical % (MT * NT);
    ti.m0 = (rem / NT) * BM;
    ti.n0 = (rem % NT) * BN;
    ti.row0 = args.offsets[ti.e];
    ti.rows = args.offsets[ti.e + 1] - ti.row0;
    K = ti.rows;
    M = (OP == OP_FC2_WGRAD) ? f : d;
    N = (OP == OP_FC2_WGRAD) ? d : 2 * f;
  }
  const size_t e = (size_t)ti.e;
  const int KT = (K + BK - 1) / BK;

  // ---------------------------------------------------------------- loaders
  // A K-contig: chunk q = tid + 256*i -> tile row q>>3, 8-element chunk q&7
  const bf16_t* a_src = nullptr;
  int lda = 0;
  if constexpr (TR::a_kcontig) {
    a_src = (const bf16_t*)(OP == OP_FC1_FWD ? args.xp
                            : OP == OP_FC2_FWD ? args.h
                            : OP == OP_FC2_DGRAD ? args.dO : args.dab);
    lda = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? d : (OP == OP_FC2_FWD ? f : 2 * f);
  } else {
    a_src = (const bf16_t*)(OP == OP_FC2_WGRAD ? args.h : args.xp);
    lda = (OP == OP_FC2_WGRAD) ? f : d;
  }

  u32x4_t ra[TR::a_kcontig ? A_KROWS : 8 * A_TBLK];
  u32x4_t rb[TR::b_kcontig ? B_KROWS : 8 * B_TBLK];

  auto load_a = [&](int k0) {
    if constexpr (TR::a_kcontig) {
#pragma unroll
      for (int i = 0; i < A_KROWS; ++i) {
        const int q = tid + NTHREADS * i;
        const int r = min(q >> 3, M - 1);  // clamp rows past the expert's end
        const bf16_t* p = a_src + (size_t)(ti.row0 + r) * lda + k0 + (q & 7) * 8;
        ra[i] = *(const u32x4_t*)p;
      }
    } else {
#pragma unroll
      for (int b = 0; b < A_TBLK; ++b) {
        const int blk = tid + NTHREADS * b;
        const int kb = blk & 7, mb = blk >> 3;
        const int mcol = min(ti.m0 + mb * 8, M - 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kr = k0 + kb * 8 + j;
          if (kr < K) {
            ra[8 * b + j] = *(const u32x4_t*)(a_src + (size_t)(ti.row0 + kr) * lda + mcol);
          } else {
            ra[8 * b + j] = u32x4_t{0u, 0u, 0u, 0u};
          }
        }
      }
    }
  };

  auto load_b = [&](int k0) {
    if constexpr (OP == OP_FC2_DGRAD || OP == OP_FC1_DGRAD) {
      // B[k][n] = W[n][k]: rows of the weight matrix, K contiguous
      const bf16_t* wsrc;
      int ldw, kk;
      if constexpr (OP == OP_FC2_DGRAD) {
        wsrc = (const bf16_t*)args.W2 + e * (size_t)f * d;
        ldw = d;
        kk = k0;
      } else {
        const bool first = k0 < f;
        wsrc = (const bf16_t*)(first ? args.W1 : args.W3) + e * (size_t)d * f;
        ldw = f;
        kk = first ? k0 : k0 - f;
      }
#pragma unroll
      for (int i = 0; i < B_KROWS; ++i) {
        const int q = tid + NTHREADS * i;
        const int n = min(ti.n0 + (q >> 3), N - 1);
        rb[i] = *(const u32x4_t*)(wsrc + (size_t)n * ldw + kk + (q & 7) * 8);
      }
    } else {
#pragma unroll
      for (int b = 0; b < B_TBLK; ++b) {
        const int blk = tid + NTHREADS * b;
        const int kb = blk & 7, nb = blk >> 3;
        const bf16_t* src;
        size_t ld;
        int col;
        bool kmask;
        if constexpr (OP == OP_FC1_FWD) {
          // tile column group of 16: even -> W1, odd -> W3, same f-columns
          const int sub16 = nb >> 1;
          const bf16_t* W = (const bf16_t*)((sub16 & 1) ? args.W3 : args.W1);
          src = W + e * (size_t)d * f;
          ld = f;
          col = ti.n0 / 2 + (sub16 >> 1) * 16 + (nb & 1) * 8;
          kmask = false;
        } else if constexpr (OP == OP_FC2_FWD) {
          src = (const bf16_t*)args.W2 + e * (size_t)f * d;
          ld = d;
          col = min(ti.n0 + nb * 8, N - 8);
          kmask = false;
        } else if constexpr (OP == OP_FC2_WGRAD) {
          src = (const bf16_t*)args.dO + (size_t)ti.row0 * d;
          ld = d;
          col = min(ti.n0 + nb * 8, N - 8);
          kmask = true;
        } else {  // OP_FC1_WGRAD
          src = (const bf16_t*)args.dab + (size_t)ti.row0 * (2 * f);
          ld = 2 * (size_t)f;
          col = min(ti.n0 + nb * 8, N - 8);
          kmask = true;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kr = k0 + kb * 8 + j;
          if (!kmask || kr < K) {
            rb[8 * b + j] = *(const u32x4_t*)(src + (size_t)kr * ld + col);
          } else {
            rb[8 * b + j] = u32x4_t{0u, 0u, 0u, 0u};
          }
        }
      }
    }
  };

  auto store_a = [&](bf16_t* As) {
    if constexpr (TR::a_kcontig) {
#pragma unroll
      for (int i = 0; i < A_KROWS; ++i) {
        const int q = tid + NTHREADS * i;
        *(u32x4_t*)(As + (q >> 3) * PITCH + (q & 7) * 8) = ra[i];
      }
    } else {
#pragma unroll
      for (int b = 0; b < A_TBLK; ++b) {
        const int blk = tid + NTHREADS * b;
        const int kb = blk & 7, mb = blk >> 3;
        u32x4_t t[8];
        transpose8x8(&ra[8 * b], t);
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4_t*)(As + (mb * 8 + i) * PITCH + kb * 8) = t[i];
      }
    }
  };

  auto store_b = [&](bf16_t* Bs) {
    if constexpr (TR::b_kcontig) {
#pragma unroll
      for (int i = 0; i < B_KROWS; ++i) {
        const int q = tid + NTHREADS * i;
        *(u32x4_t*)(Bs + (q >> 3) * PITCH + (q & 7) * 8) = rb[i];
      }
    } else {
#pragma unroll
      for (int b = 0; b < B_TBLK; ++b) {
        const int blk = tid + NTHREADS * b;
        const int kb = blk & 7, nb = blk >> 3;
        u32x4_t t[8];
        transpose8x8(&rb[8 * b], t);
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4_t*)(Bs + (nb * 8 + i) * PITCH + kb * 8) = t[i];
      }
    }
  };

  // ---------------------------------------------------------------- main loop
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // the schedule scratch lived in lds
  if (KT > 0) {
    load_a(0);
    load_b(0);
    store_a(lds);
    store_b(lds + BM * PITCH);
  }
  __syncthreads();

  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const bf16_t* As = lds + (kt & 1) * STAGE;
    const bf16_t* Bs = As + BM * PITCH;
    const bool more = kt + 1 < KT;
    if (more) {
      load_a((kt + 1) * BK);
      load_b((kt + 1) * BK);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8_t*)(As + (wm * WM + i * 16 + frag_row) * PITCH + ks * 32 + frag_k);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const bf16x8_t*)(Bs + (wn * WN + j * 16 + frag_row) * PITCH + ks * 32 + frag_k);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      bf16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
      store_a(nxt);
      store_b(nxt + BM * PITCH);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // lane holds C[m][n + 0..3] with m = wm*WM + i*16 + (lane & 15),
  // n = wn*WN + j*16 + 4*(lane >> 4)
  const int lm = lane & 15, ln = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = wm * WM + i * 16 + lm;
    if constexpr (TR::ragged_m) {
      if (m >= ti.rows) continue;
    } else {
      if (ti.m0 + m >= M) continue;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const f32x4_t c = acc[i][j];
      const int n = wn * WN + j * 16 + ln;
      if constexpr (OP == OP_FC1_FWD) {
        if (j & 1) continue;
        const f32x4_t bb = acc[i][j + 1];
        const int sub16 = (wn * WN) / 16 + j;
        const int fcol = ti.n0 / 2 + (sub16 >> 1) * 16 + ln;
        const size_t row = (size_t)(ti.row0 + m);
        bf16_t* ab = (bf16_t*)args.ab_out + row * (2 * (size_t)f);
        bf16_t* h = (bf16_t*)args.h_out + row * (size_t)f;
        float hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = silu_f32(c[q]) * bb[q];
        *(uint2*)(ab + fcol) = make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
        *(uint2*)(ab + f + fcol) = make_uint2(pack_bf16x2(bb[0], bb[1]), pack_bf16x2(bb[2], bb[3]));
        *(uint2*)(h + fcol) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      } else if constexpr (OP == OP_FC2_FWD || OP == OP_FC1_DGRAD) {
        const int col = ti.n0 + n;
        if (col >= N) continue;
        bf16_t* out = (bf16_t*)(OP == OP_FC2_FWD ? args.o_out : args.dXp_out);
        *(uint2*)(out + (size_t)(ti.row0 + m) * d + col) =
            make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
      } else if constexpr (OP == OP_FC2_DGRAD) {
        const int col = ti.n0 + n;
        if (col >= N) continue;
        const size_t row = (size_t)(ti.row0 + m);
        const bf16_t* abr = (const bf16_t*)args.ab + row * (2 * (size_t)f);
        const uint2 av = *(const uint2*)(abr + col);
        const uint2 bv = *(const uint2*)(abr + f + col);
        const float a4[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                             __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
        const float b4[4] = {__uint_as_float(bv.x << 16), __uint_as_float(bv.x & 0xffff0000u),
                             __uint_as_float(bv.y << 16), __uint_as_float(bv.y & 0xffff0000u)};
        float da[4], db[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float s = sigmoid_f32(a4[q]);
          da[q] = c[q] * b4[q] * s * (1.0f + a4[q] * (1.0f - s));
          db[q] = c[q] * a4[q] * s;
        }
        bf16_t* dab = (bf16_t*)args.dab_out + row * (2 * (size_t)f);
        *(uint2*)(dab + col) = make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
        *(uint2*)(dab + f + col) = make_uint2(pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3]));
      } else if constexpr (OP == OP_FC2_WGRAD) {
        const int col = ti.n0 + n;
        if (col >= N) continue;
        bf16_t* out = (bf16_t*)args.dW2 + e * (size_t)f * d + (size_t)(ti.m0 + m) * d + col;
        *(uint2*)out = make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
      } else {  // OP_FC1_WGRAD
        const int col = ti.n0 + n;
        if (col >= N) continue;
        bf16_t* base = (bf16_t*)(col < f ? args.dW1 : args.dW3);
        const int cc = col < f ? col : col - f;
        bf16_t* out = base + e * (size_t)d * f + (size_t)(ti.m0 + m) * f + cc;
        *(uint2*)out = make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
      }
    }
  }
}

template <int OP, int BM, int BN>
int launch(const GemmArgs& a, hipStream_t s) {
  int NT, MT = 0;
  int64_t grid;
  if (OP <= OP_FC1_DGRAD) {
    const int N = (OP == OP_FC1_FWD) ? 2 * a.f : (OP == OP_FC2_DGRAD ? a.f : a.d);
    NT = (N + BN - 1) / BN;
    // upper bound of sum_e ceil(m_e / BM) given sum_e m_e = P
    const int64_t mt_max = (int64_t)a.P / BM + a.E;
    grid = mt_max * NT;
  } else {
    const int M = (OP == OP_FC2_WGRAD) ? a.f : a.d;
    const int N = (OP == OP_FC2_WGRAD) ? a.d : 2 * a.f;
    MT = (M + BM - 1) / BM;
    NT = (N + BN - 1) / BN;
    grid = (int64_t)a.E * MT * NT;
  }
  if (grid <= 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  gemm_bf16_kernel<OP, BM, BN><<<(unsigned)grid, NTHREADS, 0, s>>>(a, NT, MT);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

int gemm_bf16_launch(GemmOp op, const GemmArgs& a, hipStream_t s) {
  switch (op) {
    case OP_FC1_FWD: return launch<OP_FC1_FWD, 256, 256>(a, s);
    case OP_FC2_FWD: return launch<OP_FC2_FWD, 256, 256>(a, s);
    case OP_FC2_DGRAD: return launch<OP_FC2_DGRAD, 256, 256>(a, s);
    case OP_FC1_DGRAD: return launch<OP_FC1_DGRAD, 256, 256>(a, s);
    case OP_FC2_WGRAD: return launch<OP_FC2_WGRAD, 256, 256>(a, s);
    case OP_FC1_WGRAD: return launch<OP_FC1_WGRAD, 256, 256>(a, s);
  }
  return MOE_ERR_INVALID;
}

}  // namespace tre
