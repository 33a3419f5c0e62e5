// The weight gradients of the 8-bit float expert GEMMs (e4m3 codes with fp32
// token-block scales, or MXFP8 with E8M0 scales), fp32 accumulation, bf16
// outputs:
//
//   op          A (rows x K)                 B (rows x K)               K
//   FC2_WGRAD   h^T token blocks [f][.]      dO^T token blocks [d][.]   128 * blocks
//   FC1_WGRAD   xp^T token blocks [d][.]     dab^T token blocks [2f][.] of the expert
//
// (C[m][n] = sum_k A[m][k] B[n][k]; the token-block quantiser stores both
// operands transposed, every expert starting at column 128 * blk[e], and one
// scale per 128-token block and column, as the pages' blockwise FP8 recipe
// has it: German technical summary of "Scalable Training of Mixture-of-Experts
// Models with Megatron Core", section 2 E; French summary, section 2 E.)
//
// An expert's tile has only its few 128-token blocks of K (about four on the
// Qwen3 shape), so these products take the K = 128 stage of one
// v_mfma_f32_16x16x128_f8f6f4 per scale block: half the stages of the 64-deep
// form of the other products (gemm_fp8.hip), and a promotion per MFMA that
// needs no accumulator rescaling (measured on the skewed shape: e4m3 fc1 /
// fc2 weight gradients 2.35 / 1.21 ms here against 2.52 / 1.30 ms in the
// 64-deep kernel, MXFP8 1.94 / 0.98 against 2.01 / 1.08).
//
// Tiles (256 x 256, 8 wavefronts of 128 x 64) are numbered expert-major and
// XCD-remapped as in the bf16 kernels.  K advances 128 per stage through a
// 2-deep LDS ring (64 KB per stage) filled by buffer_load ... lds; a
// K-contiguous LDS row is 128 bytes (8 chunks of 16) with chunk c of row r
// stored at c ^ ((r >> 1) & 7).  Per stage, the 256 A-row and 256 B-row scale
// words go to LDS with the codes.
#include "gemm_common.h"

namespace tre {

namespace {
using namespace gemm;

constexpr int BM = 256, BN = 256, BK = 128, NSTAGE = 2, NW = 8;
constexpr int OPND_BYTES = 256 * BK;            // 32 KB of codes per operand and stage
constexpr int STAGE_BYTES = 2 * OPND_BYTES;     // A then B
constexpr int DMA_PER_OPND = OPND_BYTES / 1024;  // 32 one-KB DMA instructions
constexpr int DMA_PER_WAVE = DMA_PER_OPND / NW;  // 4 per operand and stage

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// The 16x16x128 MFMA's operand layout (measured): lane group g = lane >> 4
// holds K values [16 g, 16 g + 16) in its bytes 0..15 and [64 + 16 g, 64 +
// 16 g + 16) in bytes 16..31, and the scale of 32-value block g of the row
// comes from lane group g.  So a fragment takes 16-byte chunks g and g + 4 of
// the 128-byte K row (free of LDS bank conflicts with the swizzle above, where
// chunks 2g and 2g + 1 made half of the LDS cycles conflict cycles).
__device__ __forceinline__ i32x8_t lds_frag(const char* row_base, int g, int sw) {
  const i32x4_t lo = *(const __attribute__((address_space(3))) i32x4_t*)(row_base + ((g ^ sw) << 4));
  const i32x4_t hi =
      *(const __attribute__((address_space(3))) i32x4_t*)(row_base + (((g + 4) ^ sw) << 4));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4_t mfma_fp8(const i32x8_t& b, const i32x8_t& a) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, z, 0, 0, 0, 0, 0, 0);
}

// MX = true: MXFP8 operands; the MFMA takes each lane's E8M0 scale (byte
// lane >> 4 of the lane's row word, see lds_frag) and accumulates in place.
// e4m3: each MFMA yields the exact partial product of one scale block, which
// the lane adds to its accumulators times the two block scales.
//
// PER = false: one block per tile.  PER = true (persistent, one block per
// compute unit): a block takes tiles slot = blockIdx.x, blockIdx.x +
// gridDim.x, ... as one stream through the 2-deep ring: the last stage of a
// tile loads the next tile's first stage (codes and scales) into the free
// slot, so a tile starts without waiting for its first loads.  Only buffer
// resources and scalars change from tile to tile: the next tile is kept as its
// decoded indices, and its resources are built where its first stage is
// issued.
template <int OP, bool MX, bool PER>
__global__ __launch_bounds__(NW * 64, 1) void gemm_fp8_wgrad_kernel(GemmArgs args, int NT, int MT) {
  constexpr int WAVES_N = NW / 2;
  constexpr int WM = BM / 2, WN = BN / WAVES_N;  // 128 x 64
  constexpr int FM = WM / 16, FN = WN / 16;      // 8 x 4 MFMA blocks
  static_assert(OP == OP_FC2_WGRAD || OP == OP_FC1_WGRAD, "weight gradients only");

  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE_BYTES];
  // per stage the 256 A-row and 256 B-row scale words
  __shared__ __attribute__((aligned(1024))) float sc_lds[NSTAGE][2][256];
  // persistent: the expert offsets and the token-block table, copied once so
  // that decoding the next tile reads LDS, not global memory (a global read
  // would make the compiler wait for every load in flight, DMAs included)
  __shared__ int offs[PER ? 257 : 1];
  __shared__ int blks[PER ? 257 : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int f = args.f, d = args.d, E = args.E;

  // ---------------------------------------------------------------- tiles
  const int32_t* const offv = PER ? offs : args.offsets;
  const int32_t* const blkv = PER ? blks : args.blk;
  if constexpr (PER) {
    for (int i = tid; i <= E; i += NW * 64) {
      offs[i] = args.offsets[i];
      blks[i] = args.blk[i];
    }
    __syncthreads();
  }
  const int total = uniform(E * MT * NT);
  int slot = blockIdx.x;
  if (slot >= total) return;

  // M, N fixed, K = the expert's token blocks (zero-padded; 0 for an empty
  // expert, which writes zeros)
  const int N = (OP == OP_FC2_WGRAD) ? d : 2 * f;
  const int Mw = (OP == OP_FC2_WGRAD) ? f : d;
  const uint32_t ld = (uint32_t)args.ldt;

  struct FTile {
    TileInfo ti;
    int K, KT, kb0;
    rsrc_t a_src, b_src;
    rsrc_t sca_src, scb_src;  // the stage's scale rows
  };
  auto decode = [&](int s, TileInfo& ti) __attribute__((always_inline)) {
    const int logical = xcd_remap(s, total);
    ti.e = logical / (MT * NT);
    const int rem = logical % (MT * NT);
    ti.m0 = (rem / NT) * BM;
    ti.n0 = (rem % NT) * BN;
    ti.row0 = offv[ti.e];
    ti.rows = offv[ti.e + 1] - ti.row0;
    ti.e = uniform(ti.e);
    ti.row0 = uniform(ti.row0);
    ti.rows = uniform(ti.rows);
    ti.m0 = uniform(ti.m0);
    ti.n0 = uniform(ti.n0);
  };
  auto setup = [&](const TileInfo& ti, FTile& t) __attribute__((always_inline)) {
    t.ti = ti;
    t.kb0 = uniform(blkv[ti.e]);
    t.K = uniform((blkv[ti.e + 1] - t.kb0) * BK);
    t.KT = t.K / BK;
    t.a_src = make_rsrc(args.a_q + (size_t)ti.m0 * args.ldt + (size_t)t.kb0 * BK, (uint32_t)(Mw - ti.m0) * ld);
    t.b_src = make_rsrc(args.b_q + (size_t)ti.n0 * args.ldt + (size_t)t.kb0 * BK, (uint32_t)(N - ti.n0) * ld);
    // the stage's scale rows ([NB][M] and [NB][N], 256 consecutive words
    // each; rows past the matrix read as zero).  MXFP8: the same 4 bytes per
    // block and row, holding the four 32-row E8M0 scales.
    const float* as = MX ? (const float*)args.a_sx : args.a_s;
    const float* bs = MX ? (const float*)args.b_sx : args.b_s;
    t.sca_src = make_rsrc(as + (size_t)t.kb0 * Mw + ti.m0, (uint32_t)(t.KT * Mw - ti.m0) * 4u);
    t.scb_src = make_rsrc(bs + (size_t)t.kb0 * N + ti.n0, (uint32_t)(t.KT * N - ti.n0) * 4u);
  };

  // DMA: instruction tt (0..31) of an operand covers tile rows 8tt..8tt+7;
  // lane -> row 8tt + lane/8, LDS chunk lane%8 holding K chunk (lane%8) ^ swz(row).
  // This wavefront issues tt = wid*4 + t, t < 4, for A and for B.
  uint32_t off[DMA_PER_WAVE];
#pragma unroll
  for (int t = 0; t < DMA_PER_WAVE; ++t) {
    const int tt = wid * DMA_PER_WAVE + t;
    const int row = 8 * tt + (lane >> 3);
    off[t] = (uint32_t)row * ld + (uint32_t)(((lane & 7) ^ swz(row)) << 4);
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const uint32_t sc_base = (uint32_t)(uintptr_t)&sc_lds[0][0][0];
  // DMA instruction p (0 .. 2 DMA_PER_WAVE - 1) of this wavefront for stage
  // kt of tile t into ring slot rs: A instruction p, then B instruction
  // p - DMA_PER_WAVE, with the scale rows (wavefronts 0 and 1) first.
  auto issue_part = [&](const FTile& t, int kt, int rs, int p) __attribute__((always_inline)) {
    const uint32_t st = lds_base + (uint32_t)(rs * STAGE_BYTES);
    const uint32_t ka = (uint32_t)kt * BK;
    if (p == 0) {
      const uint32_t sc = sc_base + (uint32_t)(rs * 2048);
      if (wid == 0) dma16(t.sca_src, (uint32_t)kt * (uint32_t)Mw * 4u + (uint32_t)lane * 16u, sc);
      if (wid == 1) dma16(t.scb_src, (uint32_t)kt * (uint32_t)N * 4u + (uint32_t)lane * 16u, sc + 1024);
    }
    if (p < DMA_PER_WAVE) {
      dma16(t.a_src, off[p] + ka, st + (wid * DMA_PER_WAVE + p) * 1024);
    } else {
      const int q = p - DMA_PER_WAVE;
      dma16(t.b_src, off[q] + ka, st + OPND_BYTES + (wid * DMA_PER_WAVE + q) * 1024);
    }
  };
  auto issue_stage = [&](const FTile& t, int kt, int rs) __attribute__((always_inline)) {
    static_for<0, 2 * DMA_PER_WAVE>([&](auto P) __attribute__((always_inline)) { issue_part(t, kt, rs, P.value); });
  };

  const int lm = lane & 15, lg = lane >> 4;
  auto b_row = [&](int j) __attribute__((always_inline)) -> int { return wn * WN + 16 * j + lm; };

  f32x4_t acc[FM][FN];
  // ---------------------------------------------------------------- one stage
  auto compute = [&](int rs) __attribute__((always_inline)) {
    const char* cur = lds + rs * STAGE_BYTES;
    i32x8_t bf[FN];
    static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
      const int r = b_row(J.value);
      bf[J.value] = lds_frag(cur + OPND_BYTES + r * BK, lg, swz(r));
    });
    if constexpr (MX) {
      const int sh8 = 8 * lg;
      const uint32_t* sct = (const uint32_t*)&sc_lds[rs][0][0];
      uint32_t sa[FM];
      int sbb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) sa[i] = sct[wm * WM + 16 * i + lm];
      static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
        sbb[J.value] = (int)((sct[256 + b_row(J.value)] >> sh8) & 0xffu);
      });
      // the next row's A fragment is read while this row's MFMAs run
      i32x8_t af = lds_frag(cur + (wm * WM + lm) * BK, lg, swz(wm * WM + lm));
      static_for<0, FM>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = I.value;
        i32x8_t af_next;
        if constexpr (i + 1 < FM) {
          const int r = wm * WM + 16 * (i + 1) + lm;
          af_next = lds_frag(cur + r * BK, lg, swz(r));
        }
        const int sab = (int)((sa[i] >> sh8) & 0xffu);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
          constexpr int j = J.value;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0, sbb[j],
                                                                         0, sab);
        });
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i + 1 < FM) af = af_next;
      });
    } else {
      // this stage's A-row scales and the B-row scales of the lane's 4 columns
      // per fragment
      const float* sct = &sc_lds[rs][0][0];
      float sa[FM];
      f32x4_t sb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) sa[i] = sct[wm * WM + 16 * i + lm];
#pragma unroll
      for (int j = 0; j < FN; ++j) sb[j] = *(const f32x4_t*)&sct[256 + wn * WN + 16 * j + 4 * lg];
      // Software pipeline over the FM fragment rows: the FN MFMAs of row i go
      // to their own product registers while the scale FMAs of row i-1 (whose
      // MFMAs have completed meanwhile) and the read of row i+1's A fragment
      // are issued; the sched barriers keep the compiler from pulling each
      // product's FMAs up against its MFMA.
      auto scale_row = [&](int i, const f32x4_t (&p)[FN]) __attribute__((always_inline)) {
        static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
          constexpr int j = J.value;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(p[j][q], sa[i] * sb[j][q], acc[i][j][q]);
        });
      };
      f32x4_t pc[FN], pp[FN];
      i32x8_t af = lds_frag(cur + (wm * WM + lm) * BK, lg, swz(wm * WM + lm));
      static_for<0, FM>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = I.value;
        i32x8_t af_next;
        if constexpr (i + 1 < FM) {
          const int r = wm * WM + 16 * (i + 1) + lm;
          af_next = lds_frag(cur + r * BK, lg, swz(r));
        }
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, FN>([&](auto J) __attribute__((always_inline)) { pc[J.value] = mfma_fp8(bf[J.value], af); });
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i > 0) scale_row(i - 1, pp);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, FN>([&](auto J) __attribute__((always_inline)) { pp[J.value] = pc[J.value]; });
        if constexpr (i + 1 < FM) af = af_next;
      });
      scale_row(FM - 1, pp);
    }
  };

  // ---------------------------------------------------------------- tile loop
  FTile cur;
  TileInfo tn;
  decode(slot, tn);
  setup(tn, cur);
  int base = 0;       // ring slot of the current tile's stage 0
  bool fresh = true;  // the current tile's first stage is not yet loaded
  for (;;) {
    const int nslot = slot + (int)gridDim.x;
    const bool have_next = PER && nslot < total;
    int nKT = 0;
    if (have_next) {
      decode(nslot, tn);
      nKT = uniform(blkv[tn.e + 1] - blkv[tn.e]);
    }
    // the next tile's first stage is loaded during this tile's last one
    const bool chain = have_next && cur.KT > 0 && nKT > 0;
    if (fresh && cur.KT > 0) {
      issue_stage(cur, 0, base);
      wait_vmcnt<0>();
      block_barrier();
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < cur.KT; ++kt) {
      const int rs = (base + kt) & 1;
      if (kt + 1 < cur.KT) {
        issue_stage(cur, kt + 1, rs ^ 1);
      } else if (chain) {
        FTile nxt;
        setup(tn, nxt);
        issue_stage(nxt, 0, rs ^ 1);
      }
      compute(rs);
      wait_vmcnt<0>();
      block_barrier();
    }

    // ---------------------------------------------------------------- epilogue
    store_tile<OP, FM, FN, WM, WN, false>(args, acc, cur.ti, Mw, N, wm, wn, lane);
    if (!have_next) break;
    base = (base + cur.KT) & 1;
    fresh = !chain;
    slot = nslot;
    setup(tn, cur);
  }
}

// Persistent launches where they measured faster: fc1 (both forms) and the
// MXFP8 fc2 (on the skewed shape MXFP8 fc1 / fc2 4 % / 3 % faster, e4m3 fc1
// 3 %; the persistent e4m3 fc2 spills and was 13 % slower, so it keeps one
// block per tile).
template <int OP, bool MX>
constexpr bool kPersistent = OP == OP_FC1_WGRAD || (MX && OP == OP_FC2_WGRAD);

template <int OP, bool MX>
int launch(const GemmArgs& a, hipStream_t s) {
  const int M = (OP == OP_FC2_WGRAD) ? a.f : a.d;
  const int N = (OP == OP_FC2_WGRAD) ? a.d : 2 * a.f;
  const int MT = (M + BM - 1) / BM, NT = (N + BN - 1) / BN;
  int64_t grid = (int64_t)a.E * MT * NT;
  if (grid == 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  constexpr bool PER = kPersistent<OP, MX>;
  if (PER) {
    const int ncu = gemm_persistent_blocks();
    if (ncu <= 0) return MOE_ERR_HIP;
    if (grid > ncu) grid = ncu;
  }
  gemm_fp8_wgrad_kernel<OP, MX, PER><<<dim3((unsigned)grid), NW * 64, 0, s>>>(a, NT, MT);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

int gemm_fp8_wgrad_launch(GemmOp op, bool mx, const GemmArgs& a, hipStream_t s) {
  if (op == OP_FC2_WGRAD) return mx ? launch<OP_FC2_WGRAD, true>(a, s) : launch<OP_FC2_WGRAD, false>(a, s);
  if (op == OP_FC1_WGRAD) return mx ? launch<OP_FC1_WGRAD, true>(a, s) : launch<OP_FC1_WGRAD, false>(a, s);
  return MOE_ERR_INVALID;
}

}  // namespace tre
