// Grouped expert GEMMs with e4m3 operands and fp32 block scales on CDNA4
// matrix cores, fp32 accumulation, bf16 outputs.
//
// The pages run the expert GEMMs in FP8 with blockwise scaling (German
// technical summary of "Scalable Training of Mixture-of-Experts Models with
// Megatron Core", section 2 E; French summary, section 2 E); the block shapes
// are 1 x 128 along the contraction for activations, 128 x 128 for weights,
// and 128 tokens per column for the operands of the weight gradients.  Every
// scale block spans exactly 128 values of the contraction axis, which is the
// K of one v_mfma_f32_16x16x128_f8f6f4: each MFMA yields the exact partial
// product of one scale block, and the lane adds it to its fp32 accumulator
// times the two block scales (scale promotion per 128-K block).
//
// All six products read both operands with the contraction axis contiguous
// (C[m][n] = sum_k A[m][k] B[n][k]): the weight quantiser stores transposed
// codes for the forward products and the token-block quantiser stores the
// weight-gradient operands transposed, so one LDS layout serves every op:
//
//   op          A (rows x K)                 B (rows x K)               K
//   FC1_FWD     xp codes [P][d]              W1^T, W3^T codes [f][d]    d
//   FC2_FWD     h codes  [P][f]              W2^T codes [d][f]          f
//   FC2_DGRAD   dO codes [P][d]              W2 codes [f][d]            d
//   FC1_DGRAD   dab codes [P][2f]            W1 | W3 codes [d][f]       2f
//   FC2_WGRAD   h^T token blocks [f][.]      dO^T token blocks [d][.]   128 * blocks
//   FC1_WGRAD   xp^T token blocks [d][.]     dab^T token blocks [2f][.] of the expert
//
// Tiles, schedule and epilogues are those of the bf16 kernels (256 x 256
// block tile, 8 wavefronts of 128 x 64, device-side ragged-M schedule, fused
// SwiGLU forward / backward epilogues, bf16 stores).  K advances 128 per
// stage through a 2-deep LDS ring (64 KB per stage) filled by buffer_load ...
// lds; a K-contiguous LDS row is 128 bytes (8 chunks of 16) with chunk c of
// row r stored at c ^ ((r >> 1) & 7).  A fragment (32 K bytes of one row per
// lane: chunks g and g + 4 for lane group g) is two ds_read_b128, free of
// bank conflicts (measured).
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

// The scaled MFMA's operand layout (measured): lane group g = lane >> 4 holds
// K values [16 g, 16 g + 16) in its bytes 0..15 and [64 + 16 g, 64 + 16 g + 16)
// in bytes 16..31, and the scale of 32-value block g of the row comes from
// lane group g.  So a fragment takes 16-byte chunks g and g + 4 of the
// 128-byte K row.  The e4m3 path (one 128-value scale block per MFMA) could
// take any K order that A and B share; it takes the same one, which is free
// of LDS bank conflicts, where chunks 2g and 2g + 1 made half of the LDS
// cycles conflict cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = 0.5).
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

__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// A value loaded a stage ahead is complete once the stage's explicit
// s_waitcnt vmcnt(0) has passed, but the compiler's wait insertion merges the
// loop's entry and back edge and still counts it as pending: it then puts a
// vmcnt(0) in front of the first use -- in the middle of the next stage's
// MFMAs, where it also waits for that stage's freshly issued DMA loads.  Passing
// the value through an empty asm at the top of the stage, while nothing is
// outstanding, ends that chain.
template <typename T>
__device__ __forceinline__ void settle(T& v) {
  asm volatile("" : "+v"(v));
}

// MX = true: MXFP8 operands.  v_mfma_scale_f32_16x16x128_f8f6f4 takes one
// E8M0 scale per lane and operand -- that of 32-value block (lane >> 4) of the
// lane's row (see lds_frag for the matching fragment layout) -- so the
// scales go straight into the MFMA, which accumulates in place: no promotion.
// A lane's scale byte for fragment row r and stage kt is byte (lane >> 4) of
// the word at r * ld + 4 kt.
// RS: row-scaled epilogues (probabilities applied before W2; fc1 forward and
// fc2 dgrad only), as in the bf16 kernels.
//
// Tiles are numbered and XCD-remapped as in the bf16 kernels.  PER = false:
// one block per tile.  PER = true (persistent, one block per compute unit):
// a block takes tiles slot = blockIdx.x, blockIdx.x + gridDim.x, ... as one
// stream through the 2-deep ring: the last stage of a tile loads the next
// tile's first stage (codes and scales) into the free slot, so a tile starts
// without waiting for its first loads.
// Only buffer resources and scalars change from tile to tile (every DMA lane
// offset is relative to the tile): the next tile is kept as its decoded
// indices, and its resources are built where its first stage is issued.
template <int OP, bool MX, bool RS, bool PER>
__global__ __launch_bounds__(NW * 64, 1) void gemm_fp8_kernel(GemmArgs args, int NT, int MT) {
  constexpr int WAVES_N = NW / 2;
  constexpr int WM = BM / 2, WN = BN / WAVES_N;  // 128 x 64
  constexpr int FM = WM / 16, FN = WN / 16;      // 8 x 4 MFMA blocks
  constexpr bool RAGGED = OP <= OP_FC1_DGRAD;
  constexpr bool WGRAD = !RAGGED;

  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE_BYTES];
  // weight-gradient products: per stage the 256 A-row and 256 B-column scales
  __shared__ __attribute__((aligned(1024))) float sc_lds[NSTAGE][2][256];
  // persistent: the expert offsets (weight gradients: and the token-block
  // table), copied once so that decoding the next tile reads LDS, not global
  // memory (a global read would make the compiler wait for every load in
  // flight, DMAs included)
  __shared__ int offs[PER ? 257 : 1];
  __shared__ int blks[PER && WGRAD ? 257 : 1];
  __shared__ int mt_incl[PER && RAGGED ? 256 : 1];  // ragged: inclusive prefix of the experts' M-tiles
  __shared__ int sched[NW + 4];
  __shared__ float dp_red[RS ? (NW / 2) * 256 : 1];  // row-scaled fc2 dgrad: <h, dh'> partials
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int d = args.d, f = args.f, E = args.E;

  // ---------------------------------------------------------------- tiles
  const int32_t* const offv = PER ? offs : args.offsets;
  const int32_t* const blkv = PER ? blks : args.blk;
  int total = 0;
  if constexpr (PER) {
    for (int i = tid; i <= E; i += NW * 64) {
      offs[i] = args.offsets[i];
      if constexpr (WGRAD) blks[i] = args.blk[i];
    }
    __syncthreads();
    if constexpr (RAGGED) total = mtile_prefix<BM, NW>(offs, E, mt_incl, sched) * NT;
    else total = E * MT * NT;
  } else if constexpr (WGRAD) {
    total = E * MT * NT;
  }
  total = uniform(total);
  int slot = blockIdx.x;
  if ((PER || WGRAD) && slot >= total) return;

  // ragged: K fixed, M = the tile's rows; weight gradients: M, N fixed, K =
  // the expert's token blocks (zero-padded; 0 for an empty expert)
  const int Kr = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? d : (OP == OP_FC2_FWD ? f : 2 * f);
  const int N = RAGGED ? ((OP == OP_FC1_FWD) ? 2 * f : (OP == OP_FC2_DGRAD ? f : d))
                       : ((OP == OP_FC2_WGRAD) ? d : 2 * f);
  const int Mw = (OP == OP_FC2_WGRAD) ? f : d;
  const uint32_t a_ld = RAGGED ? (uint32_t)Kr : (uint32_t)args.ldt;
  uint32_t b_ld;
  if constexpr (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) b_ld = (uint32_t)d;
  else if constexpr (OP == OP_FC2_FWD || OP == OP_FC1_DGRAD) b_ld = (uint32_t)f;
  else b_ld = (uint32_t)args.ldt;
  // MXFP8 ragged products: words of scale bytes per row
  const uint32_t xa_ld = (uint32_t)(Kr / 32);
  const uint32_t xb_ld = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? (uint32_t)(d / 32) : (uint32_t)(f / 32);

  struct FTile {
    TileInfo ti;
    int K, KT, M, kb0;
    rsrc_t a_src, b_src, b_src2;
    rsrc_t sca_src, scb_src;              // weight gradients: the stage's scale rows
    __amdgpu_buffer_rsrc_t sa_src;        // e4m3 ragged: the A rows' block scales
    __amdgpu_buffer_rsrc_t xa, xb, xb2;   // MXFP8 ragged: scale words of A rows and B rows
  };
  // (one block per tile, ragged: the whole decode in one pass over the
  // offsets; a block past the device-side tile count returns)
  auto decode = [&](int s, TileInfo& ti) __attribute__((always_inline)) -> bool {
    if constexpr (RAGGED && !PER) {
      if (!decode_ragged_m<BM, NW>(args.offsets, E, NT, sched, ti)) return false;
      ti.n0 *= BN;
    } else if constexpr (RAGGED) {
      ragged_tile(offs, mt_incl, E, NT, BM, xcd_remap(s, total), ti);
      ti.n0 *= BN;
    } else {
      const int logical = xcd_remap(s, total);
      ti.e = logical / (MT * NT);
      const int rem = logical % (MT * NT);
      ti.m0 = (rem / NT) * BM;
      ti.n0 = (rem % NT) * BN;
      ti.row0 = offv[ti.e];
      ti.rows = offv[ti.e + 1] - ti.row0;
    }
    ti.e = uniform(ti.e);
    ti.row0 = uniform(ti.row0);
    ti.rows = uniform(ti.rows);
    ti.m0 = uniform(ti.m0);
    ti.n0 = uniform(ti.n0);
    return true;
  };
  auto setup = [&](const TileInfo& ti, FTile& t) __attribute__((always_inline)) {
    t.ti = ti;
    const size_t e = (size_t)ti.e;
    if constexpr (RAGGED) {
      t.K = Kr;
      t.M = ti.rows;
      t.kb0 = 0;
      t.a_src = make_rsrc(args.a_q + (size_t)ti.row0 * Kr, (uint32_t)ti.rows * a_ld);
    } else {
      t.kb0 = uniform(blkv[ti.e]);
      t.K = uniform((blkv[ti.e + 1] - t.kb0) * BK);
      t.M = Mw;
      t.a_src = make_rsrc(args.a_q + (size_t)ti.m0 * args.ldt + (size_t)t.kb0 * BK,
                          (uint32_t)(Mw - ti.m0) * a_ld);
    }
    t.KT = t.K / BK;
    if constexpr (OP == OP_FC1_FWD) {  // W1^T / W3^T rows n0/2 .. +128
      const size_t off = e * (size_t)f * d + (size_t)(ti.n0 / 2) * d;
      t.b_src = make_rsrc(args.b_q + off, 128u * b_ld);
      t.b_src2 = make_rsrc(args.b_q2 + off, 128u * b_ld);
    } else if constexpr (OP == OP_FC2_FWD) {  // W2^T [d][f]
      t.b_src = make_rsrc(args.b_q + e * (size_t)d * f + (size_t)ti.n0 * f, (uint32_t)(d - ti.n0) * b_ld);
      t.b_src2 = t.b_src;
    } else if constexpr (OP == OP_FC2_DGRAD) {  // W2 [f][d]
      t.b_src = make_rsrc(args.b_q + e * (size_t)f * d + (size_t)ti.n0 * d, (uint32_t)(f - ti.n0) * b_ld);
      t.b_src2 = t.b_src;
    } else if constexpr (OP == OP_FC1_DGRAD) {  // W1 | W3 [d][f], K = 2f
      const size_t off = e * (size_t)d * f + (size_t)ti.n0 * f;
      t.b_src = make_rsrc(args.b_q + off, (uint32_t)(d - ti.n0) * b_ld);
      t.b_src2 = make_rsrc(args.b_q2 + off, (uint32_t)(d - ti.n0) * b_ld);
    } else {  // wgrad: token-block operand [N][ldt]
      t.b_src = make_rsrc(args.b_q + (size_t)ti.n0 * args.ldt + (size_t)t.kb0 * BK,
                          (uint32_t)(N - ti.n0) * b_ld);
      t.b_src2 = t.b_src;
    }
    if constexpr (WGRAD) {
      // the stage's scale rows ([NB][M] and [NB][N], 256 consecutive floats
      // each); rows past the matrix read as zero.  (MXFP8: the same 4 bytes
      // per block and row, holding the four 32-row E8M0 scales)
      const float* as = MX ? (const float*)args.a_sx : args.a_s;
      const float* bs = MX ? (const float*)args.b_sx : args.b_s;
      t.sca_src = make_rsrc(as + (size_t)t.kb0 * Mw + ti.m0, (uint32_t)(t.KT * Mw - ti.m0) * 4u);
      t.scb_src = make_rsrc(bs + (size_t)t.kb0 * N + ti.n0, (uint32_t)(t.KT * N - ti.n0) * 4u);
    } else if constexpr (!MX) {
      t.sa_src = __builtin_amdgcn_make_buffer_rsrc((void*)(args.a_s + (size_t)ti.row0 * (Kr / BK)), 0,
                                                   ti.rows * (Kr / BK) * 4, 0x00020000);
    } else {
      t.xa = __builtin_amdgcn_make_buffer_rsrc((void*)(args.a_sx + (size_t)ti.row0 * xa_ld), 0,
                                               ti.rows * (int)xa_ld, 0x00020000);
      size_t b0;
      int brows;
      if constexpr (OP == OP_FC1_FWD) {
        b0 = (e * f + ti.n0 / 2) * xb_ld; brows = 128;
      } else if constexpr (OP == OP_FC2_FWD) {
        b0 = (e * d + ti.n0) * xb_ld; brows = d - ti.n0;
      } else if constexpr (OP == OP_FC2_DGRAD) {
        b0 = (e * f + ti.n0) * xb_ld; brows = f - ti.n0;
      } else {
        b0 = (e * d + ti.n0) * xb_ld; brows = d - ti.n0;
      }
      t.xb = __builtin_amdgcn_make_buffer_rsrc((void*)(args.b_sx + b0), 0, brows * (int)xb_ld, 0x00020000);
      t.xb2 = (OP == OP_FC1_FWD || OP == OP_FC1_DGRAD)
                  ? __builtin_amdgcn_make_buffer_rsrc((void*)(args.b_sx2 + b0), 0, brows * (int)xb_ld,
                                                      0x00020000)
                  : t.xb;
    }
  };

  // DMA: instruction tt (0..31) of an operand covers tile rows 8tt..8tt+7;
  // lane -> row 8tt + lane/8, LDS chunk lane%8 holding K chunk (lane%8) ^ swz(row).
  // This wavefront issues tt = wid*4 + t, t < 4, for A and for B.
  uint32_t a_off[DMA_PER_WAVE], b_off[DMA_PER_WAVE];
#pragma unroll
  for (int t = 0; t < DMA_PER_WAVE; ++t) {
    const int tt = wid * DMA_PER_WAVE + t;
    const int row = 8 * tt + (lane >> 3);
    const uint32_t ch = (uint32_t)(((lane & 7) ^ swz(row)) << 4);
    a_off[t] = (uint32_t)row * a_ld + ch;
    const int brow = (OP == OP_FC1_FWD) ? (row & 127) : row;  // fc1: rows 128.. come from W3
    b_off[t] = (uint32_t)brow * b_ld + ch;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const uint32_t sc_base = (uint32_t)(uintptr_t)&sc_lds[0][0][0];
  // DMA instruction p (0 .. 2 DMA_PER_WAVE - 1) of this wavefront for stage
  // kt of tile t into ring slot rs: A instruction p, then B instruction
  // p - DMA_PER_WAVE (weight gradients: the scale rows with the first).
  auto issue_part = [&](const FTile& t, int kt, int rs, int p) __attribute__((always_inline)) {
    const uint32_t st = lds_base + (uint32_t)(rs * STAGE_BYTES);
    const uint32_t ka = (uint32_t)kt * BK;
    if constexpr (WGRAD) {
      if (p == 0) {
        const uint32_t sc = sc_base + (uint32_t)(rs * 2048);
        if (wid == 0) dma16(t.sca_src, (uint32_t)kt * (uint32_t)Mw * 4u + (uint32_t)lane * 16u, sc);
        if (wid == 1) dma16(t.scb_src, (uint32_t)kt * (uint32_t)N * 4u + (uint32_t)lane * 16u, sc + 1024);
      }
    }
    if (p < DMA_PER_WAVE) {
      const int tt = wid * DMA_PER_WAVE + p;
      dma16(t.a_src, a_off[p] + ka, st + tt * 1024);
    } else {
      const int q = p - DMA_PER_WAVE;
      const int tt = wid * DMA_PER_WAVE + q;
      const uint32_t m0 = st + OPND_BYTES + tt * 1024;
      if constexpr (OP == OP_FC1_FWD) {
        dma16(tt < 16 ? t.b_src : t.b_src2, b_off[q] + ka, m0);
      } else if constexpr (OP == OP_FC1_DGRAD) {
        const bool second = (int)ka >= f;
        dma16(second ? t.b_src2 : t.b_src, b_off[q] + (second ? ka - (uint32_t)f : ka), m0);
      } else {
        dma16(t.b_src, b_off[q] + ka, m0);
      }
    }
  };
  auto issue_stage = [&](const FTile& t, int kt, int rs) __attribute__((always_inline)) {
    static_for<0, 2 * DMA_PER_WAVE>([&](auto P) __attribute__((always_inline)) { issue_part(t, kt, rs, P.value); });
  };

  const int lm = lane & 15, lg = lane >> 4;
  // B rows of fragment j within the B tile (fc1 forward: W1 rows then W3 rows)
  auto b_row = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (OP == OP_FC1_FWD) return (j < FN / 2 ? 0 : 128) + wn * (WN / 2) + 16 * (j % (FN / 2)) + lm;
    else return wn * WN + 16 * j + lm;
  };

  // ---------------------------------------------------------------- scales
  // e4m3 ragged: sa[i], the scale of the A block of fragment row
  // m = wm*WM + 16 i + (lane & 15), a_s[(row0 + m) * K/128 + kt] (0 past the
  // expert's rows); the weight block scale is one value per wavefront and
  // stage (fc1 forward: one for the W1 half, one for the W3 half).  nbw: the
  // wavefront's 128-column block of B rows, clamped for wavefronts past N in
  // a last, half-filled N-tile (their columns are never stored).
  const uint32_t sa_off0 = (uint32_t)(wm * WM + lm) * (uint32_t)(Kr / BK) * 4u;
  const uint32_t sa_istep = 16u * (uint32_t)(Kr / BK) * 4u;  // 16 rows
  auto load_sa = [&](const FTile& t, int kt, float (&sa)[FM]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = buf_f32(t.sa_src, sa_off0 + (uint32_t)i * sa_istep + (uint32_t)kt * 4u);
  };
  auto weight_scale = [&](const FTile& t, int kt, int half) __attribute__((always_inline)) -> float {
    const size_t e = (size_t)t.ti.e;
    const int nbw = min((t.ti.n0 + wn * WN) / 128, (N - 1) / 128);
    if constexpr (OP == OP_FC1_FWD) {  // W1s / W3s [E][d/128][f/128], block (kt, f-block)
      const float* s = half ? args.b_s2 : args.b_s;
      return s[(e * (d / 128) + kt) * (f / 128) + (t.ti.n0 / 2) / 128];
    } else if constexpr (OP == OP_FC2_FWD) {  // W2s [E][f/128][d/128], block (kt, d-block)
      return args.b_s[(e * (f / 128) + kt) * (d / 128) + nbw];
    } else if constexpr (OP == OP_FC2_DGRAD) {  // W2s, block (f-block of n, kt)
      return args.b_s[(e * (f / 128) + nbw) * (d / 128) + kt];
    } else {  // FC1_DGRAD: W1s / W3s [E][d/128][f/128], block (d-block of n, kt mod f/128)
      const int fb = f / 128;
      const float* s = kt < fb ? args.b_s : args.b_s2;
      return s[(e * (d / 128) + nbw) * fb + (kt < fb ? kt : kt - fb)];
    }
  };
  // MXFP8 ragged: buffer loads of the lane's rows' scale words
  auto load_mx = [&](const FTile& t, int kt, uint32_t (&sa)[FM], uint32_t (&sb)[FN])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = buf_u32(t.xa, (uint32_t)(wm * WM + 16 * i + lm) * xa_ld + (uint32_t)kt * 4u);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (OP == OP_FC1_FWD) {
        sb[j] = buf_u32(j < FN / 2 ? t.xb : t.xb2, (uint32_t)(b_row(j) & 127) * xb_ld + (uint32_t)kt * 4u);
      } else if constexpr (OP == OP_FC1_DGRAD) {
        const int fb = f / 128;
        sb[j] = buf_u32(kt < fb ? t.xb : t.xb2,
                        (uint32_t)b_row(j) * xb_ld + (uint32_t)(kt < fb ? kt : kt - fb) * 4u);
      } else {
        sb[j] = buf_u32(t.xb, (uint32_t)b_row(j) * xb_ld + (uint32_t)kt * 4u);
      }
    }
  };

  // Per-lane scale registers of the current stage and of the stage loaded
  // ahead (ragged products; weight gradients read theirs from sc_lds).
  float fsa[FM], fsa_n[FM];  // e4m3: A scales
  float wsc0 = 0.f, wsc1 = 0.f, wsc0_n = 0.f, wsc1_n = 0.f;  // e4m3: weight scales
  uint32_t xsa[FM], xsb[FN], xsa_n[FM], xsb_n[FN];  // MXFP8: scale words
  // the stage-ahead scales of stage kt of tile t
  auto load_ahead = [&](const FTile& t, int kt) __attribute__((always_inline)) {
    if constexpr (RAGGED) {
      if constexpr (MX) {
        load_mx(t, kt, xsa_n, xsb_n);
      } else {
        load_sa(t, kt, fsa_n);
        wsc0_n = weight_scale(t, kt, 0);
        wsc1_n = (OP == OP_FC1_FWD) ? weight_scale(t, kt, 1) : wsc0_n;
      }
    }
  };
  auto rotate = [&]() __attribute__((always_inline)) {
    if constexpr (RAGGED) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < FM; ++i) xsa[i] = xsa_n[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) xsb[j] = xsb_n[j];
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) fsa[i] = fsa_n[i];
        wsc0 = wsc0_n;
        wsc1 = wsc1_n;
      }
    }
  };
  // A value loaded a stage ahead is complete once the stage's explicit
  // vmcnt(0) has passed; the empty asm (settle) tells the compiler so, before
  // this stage's DMAs are issued.
  auto settle_all = [&]() __attribute__((always_inline)) {
    if constexpr (RAGGED) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < FM; ++i) settle(xsa[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j) settle(xsb[j]);
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) settle(fsa[i]);
        settle(wsc0);
        settle(wsc1);
      }
    }
  };

  f32x4_t acc[FM][FN];
  // ---------------------------------------------------------------- one stage
  auto compute = [&](int rs) __attribute__((always_inline)) {
    const char* cur = lds + rs * STAGE_BYTES;
    if constexpr (MX) {
      const int sh8 = 8 * lg;
      uint32_t sa[FM], sb[FN];
      if constexpr (WGRAD) {
        const uint32_t* sct = (const uint32_t*)&sc_lds[rs][0][0];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = sct[wm * WM + 16 * i + lm];
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = sct[256 + b_row(j)];
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = xsa[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = xsb[j];
      }
      i32x8_t bf[FN];
      int sbb[FN];
      static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
        const int r = b_row(J.value);
        bf[J.value] = lds_frag(cur + OPND_BYTES + r * BK, lg, swz(r));
        sbb[J.value] = (int)((sb[J.value] >> sh8) & 0xffu);
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
      float sa[FM];
      f32x4_t sb[FN];  // weight gradients: this stage's B scales (4 columns per fragment)
      if constexpr (WGRAD) {
        const float* sct = &sc_lds[rs][0][0];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = sct[wm * WM + 16 * i + lm];
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = *(const f32x4_t*)&sct[256 + wn * WN + 16 * j + 4 * lg];
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = fsa[i];
      }
      i32x8_t bf[FN];
      static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
        const int r = b_row(J.value);
        bf[J.value] = lds_frag(cur + OPND_BYTES + r * BK, lg, swz(r));
      });
      // Software pipeline over the FM fragment rows: the FN MFMAs of row i go
      // to their own product registers while the scale FMAs of row i-1 (whose
      // MFMAs have completed meanwhile) and the read of row i+1's A fragment
      // are issued; the sched barriers keep the compiler from pulling each
      // product's FMAs up against its MFMA.
      auto scale_row = [&](int i, const f32x4_t (&p)[FN]) __attribute__((always_inline)) {
        static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
          constexpr int j = J.value;
          if constexpr (RAGGED) {
            const float s = sa[i] * (j < FN / 2 ? wsc0 : wsc1);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(p[j][q], s, acc[i][j][q]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(p[j][q], sa[i] * sb[j][q], acc[i][j][q]);
          }
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
  if (!decode(slot, tn)) return;
  setup(tn, cur);
  int base = 0;       // ring slot of the current tile's stage 0
  bool fresh = true;  // the current tile's first stage is not yet loaded
  for (;;) {
    const int nslot = slot + (int)gridDim.x;
    const bool have_next = PER && nslot < total;
    int nKT = 0;
    if (have_next) {
      decode(nslot, tn);
      if constexpr (RAGGED) nKT = Kr / BK;
      else nKT = uniform(blkv[tn.e + 1] - blkv[tn.e]);
    }
    // the next tile's first stage is loaded during this tile's last one
    const bool chain = have_next && cur.KT > 0 && nKT > 0;
    if (fresh && cur.KT > 0) {
      load_ahead(cur, 0);
      issue_stage(cur, 0, base);
      wait_vmcnt<0>();
      block_barrier();
      rotate();
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < cur.KT; ++kt) {
      const int rs = (base + kt) & 1;
      settle_all();
      if (kt + 1 < cur.KT) {
        load_ahead(cur, kt + 1);
        issue_stage(cur, kt + 1, rs ^ 1);
      } else if (chain) {
        FTile nxt;
        setup(tn, nxt);
        load_ahead(nxt, 0);
        issue_stage(nxt, 0, rs ^ 1);
      }
      compute(rs);
      wait_vmcnt<0>();
      block_barrier();
      rotate();
    }

    // ---------------------------------------------------------------- epilogue
    store_tile<OP, FM, FN, WM, WN, RAGGED, RS>(args, acc, cur.ti, cur.M, N, wm, wn, lane, dp_red);
    if (!have_next) break;
    base = (base + cur.KT) & 1;
    fresh = !chain;
    slot = nslot;
    setup(tn, cur);
  }
}

// Products launched persistent: the weight gradients, whose tiles have only
// an expert's few 128-row token blocks of K, so that a first load per tile
// weighs most.  (The ragged-M products, with 12-32 stages per tile, run out
// of scalar registers when persistent: the compiler then spills.)
// (Measured on the skewed shape: MXFP8 fc1 / fc2 wgrad 4 % / 3 % faster, e4m3
// fc1 wgrad 3 % faster; the persistent e4m3 fc2 wgrad spills and was 13 %
// slower, so it keeps one block per tile.)
template <int OP, bool MX>
constexpr bool kPersistent = OP == OP_FC1_WGRAD || (MX && OP == OP_FC2_WGRAD);

template <int OP, bool MX>
int launch(const GemmArgs& a, hipStream_t s) {
  int NT, MT = 0;
  int64_t grid;
  if (OP <= OP_FC1_DGRAD) {
    const int N = (OP == OP_FC1_FWD) ? 2 * a.f : (OP == OP_FC2_DGRAD ? a.f : a.d);
    NT = (N + BN - 1) / BN;
    grid = ((int64_t)a.P / BM + a.E) * NT;  // upper bound of the device-side tile count
  } else {
    const int M = (OP == OP_FC2_WGRAD) ? a.f : a.d;
    const int N = (OP == OP_FC2_WGRAD) ? a.d : 2 * a.f;
    MT = (M + BM - 1) / BM;
    NT = (N + BN - 1) / BN;
    grid = (int64_t)a.E * MT * NT;
  }
  if (grid == 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  constexpr bool PER = kPersistent<OP, MX>;
  if (PER) {
    const int ncu = gemm_persistent_blocks();
    if (ncu <= 0) return MOE_ERR_HIP;
    if (grid > ncu) grid = ncu;
  }
  bool scaled = false;  // row-scaled variant: only fc1 forward and fc2 dgrad change
  if constexpr (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) {
    if (a.row_prob) {
      gemm_fp8_kernel<OP, MX, true, PER><<<dim3((unsigned)grid), NW * 64, 0, s>>>(a, NT, MT);
      scaled = true;
    }
  }
  if (!scaled) gemm_fp8_kernel<OP, MX, false, PER><<<dim3((unsigned)grid), NW * 64, 0, s>>>(a, NT, MT);
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

int gemm_fp8_launch(GemmOp op, const GemmArgs& a, hipStream_t s) {
  switch (op) {
    case OP_FC1_FWD: return launch<OP_FC1_FWD, false>(a, s);
    case OP_FC2_FWD: return launch<OP_FC2_FWD, false>(a, s);
    case OP_FC2_DGRAD: return launch<OP_FC2_DGRAD, false>(a, s);
    case OP_FC1_DGRAD: return launch<OP_FC1_DGRAD, false>(a, s);
    case OP_FC2_WGRAD: return launch<OP_FC2_WGRAD, false>(a, s);
    case OP_FC1_WGRAD: return launch<OP_FC1_WGRAD, false>(a, s);
  }
  return MOE_ERR_INVALID;
}

int gemm_mx_launch(GemmOp op, const GemmArgs& a, hipStream_t s) {
  switch (op) {
    case OP_FC1_FWD: return launch<OP_FC1_FWD, true>(a, s);
    case OP_FC2_FWD: return launch<OP_FC2_FWD, true>(a, s);
    case OP_FC2_DGRAD: return launch<OP_FC2_DGRAD, true>(a, s);
    case OP_FC1_DGRAD: return launch<OP_FC1_DGRAD, true>(a, s);
    case OP_FC2_WGRAD: return launch<OP_FC2_WGRAD, true>(a, s);
    case OP_FC1_WGRAD: return launch<OP_FC1_WGRAD, true>(a, s);
  }
  return MOE_ERR_INVALID;
}

}  // namespace tre
