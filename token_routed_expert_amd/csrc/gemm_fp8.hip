// Grouped expert GEMMs with 8-bit float operands on CDNA4 matrix cores, fp32
// accumulation, bf16 outputs: e4m3 codes with fp32 block scales, and MXFP8
// (e4m3 codes with one power-of-two E8M0 scale per 32 values).
//
// The pages run the expert GEMMs in FP8 with blockwise scaling (German
// technical summary of "Scalable Training of Mixture-of-Experts Models with
// Megatron Core", section 2 E; French summary, section 2 E); the e4m3 block
// shapes are 1 x 128 along the contraction for activations, 128 x 128 for
// weights, and 128 tokens per column for the operands of the weight
// gradients, so every scale block spans 128 values of the contraction axis.
//
// The four products with ragged M (an expert's permuted rows) read A with the
// contraction axis contiguous (C[m][n] = sum_k A[m][k] B[n][k]), and B as
// listed (the MXFP8 weight quantiser stores the transposed codes its forward
// products read):
//
//   op          A (rows x K)                 B (rows x K)               K
//   FC1_FWD     xp codes [P][d]              W1^T, W3^T codes [f][d]    d
//   FC2_FWD     h codes  [P][f]              W2^T codes [d][f]          f
//   FC2_DGRAD   dO codes [P][d]              W2 codes [f][d]            d
//   FC1_DGRAD   dab codes [P][2f]            W1 | W3 codes [d][f]       2f
//
// (e4m3 forward products: B is read in the weights' own orientation instead,
// MN-contiguous -- W1, W3 [d][f] and W2 [f][d] -- as the weight gradients
// read their operands: a 128 x 128 scale block holds for both orientations,
// so the weight quantiser writes one copy.  MXFP8 scales run along the
// contraction, so its forward products keep the transposed codes.)
//
// The weight gradients contract over an expert's rows and read both operands
// in their row-major form, MN-contiguous (C[m][n] = sum_k A[k][m] B[k][n]),
// with one scale per 128-row token block and column:
//
//   FC2_WGRAD   h codes [P][f]   (m: f)      dO codes [P][d]  (n: d)    rows of e
//   FC1_WGRAD   xp codes [P][d]  (m: d)      dab codes [P][2f] (n: 2f)  rows of e
//
// Pipeline: that of the bf16 kernels -- 256 x 256 block tile, 8 wavefronts of
// 128 x 64, persistent blocks walking the XCD-remapped device-side tile list
// with the next tile's first stages streamed under the current one's last,
// fused SwiGLU forward / backward epilogues -- with K advancing 64 codes per
// stage through a 4-deep LDS ring (32 KB of codes per stage: 256 rows of 64
// bytes per operand, or in the weight gradients 64 k-rows of 256 bytes),
// every operand byte moved by buffer_load ... lds issued up to three stages
// ahead.  The products are v_mfma_scale_f32_32x32x64_f8f6f4
// (a wavefront covers its 128 x 64 sub-tile with 4 x 2 blocks of 32 x 32).
// The 64-deep MFMA is what allows the 32 KB stage and so the 4-deep ring: the
// 128-deep 16x16x128 form needs 64 KB per stage, two stages in the LDS.
//
// MFMA operand layout (measured with a probe): lane l supplies row l & 31 of
// its operand; lane group h = l >> 5 holds K values [16 h, 16 h + 16) in bytes
// 0..15 and [32 + 16 h, 32 + 16 h + 16) in bytes 16..31; the E8M0 scale of
// 32-value block b of a row comes from lane group b.  Results: lane l holds
// D[8 q + 4 h + r][l & 31] in accumulator 4 q + r.  The kernel computes
// D = C^T (B rows as the MFMA's rows), so a lane's 16 results are 16 output
// columns of one output row.
//
// Scales.  With each stage's codes come its scale words, 2 KB per stage: one
// 32-bit word per A row and per B row (weight gradients: per A and B column;
// e4m3: the fp32 scale of the row's 128-K block; MXFP8: the four E8M0 bytes
// of that block).  MXFP8 bytes go
// straight into the MFMA.  An e4m3 scale s = 2^e * m (m in [1, 2)) is split:
// the MFMA applies 2^e of the A row and of the B row as E8M0 scales, and the
// accumulators are kept in units of the current block's mantissas,
// u = m_A * m_B (all rows of a 128-row weight block share m_B): at the first
// stage of each 128-K block they are multiplied by u_old / u_new (in
// (1/4, 4)), and at the end of the tile by the last u.  That is one
// multiplication per accumulator per 128-K block, as a promotion of per-block
// partial products would take, without their registers.  In the weight
// gradients m_B varies per output column too, so a lane's factor at a block
// change is r_A(m) * r_B(n) for each of its 16 columns n per 32 x 32 block;
// each lane forms r_B of one of the wavefront's 64 columns, and the wavefront
// trades them through 256 bytes of LDS of its own.
#include "gemm_common.h"

namespace tre {

namespace {
using namespace gemm;

constexpr int BM = 256, BN = 256, BK = 64, NW = 8;
constexpr int OPND_BYTES = 256 * BK;             // 16 KB of codes per operand and stage
constexpr int STAGE_BYTES = 2 * OPND_BYTES;      // A then B
constexpr int SC_BYTES = 2048;                   // per stage: 256 A-row then 256 B-row words
constexpr int DMA_PER_OPND = OPND_BYTES / 1024;  // 16 one-KB DMA instructions
constexpr int DMA_PER_WAVE = DMA_PER_OPND / NW;  // 2 per operand and stage
constexpr int NS = 4;                            // LDS ring depth
constexpr int LOOK = NS - 1;                     // stage kt + LOOK is issued during stage kt
// vector-memory loads a wavefront issues per stage: A, B, one scale DMA
constexpr int LOADS_PER_STAGE = 2 * DMA_PER_WAVE + 1;

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Chunk swizzle of the 64-byte LDS rows: 16-byte chunk c of row r is stored
// at chunk c ^ swz(r).  A fragment read (ds_read_b128) takes chunk h (then
// h + 2) of rows 0..31 of a block in lane group h, so each 16 lanes read 16
// rows of one chunk; with swz(r) = (r >> 2) & 3 those cover the 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ i32x8_t lds_frag(const char* row_base, int h, int sw) {
  const i32x4_t lo = *(const __attribute__((address_space(3))) i32x4_t*)(row_base + ((h ^ sw) << 4));
  const i32x4_t hi =
      *(const __attribute__((address_space(3))) i32x4_t*)(row_base + (((h + 2) ^ sw) << 4));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// MN-contiguous stages of the weight gradients: 64 k-rows of 256 bytes per
// operand; 32-byte unit u of k-row k is stored at unit u ^ (k & 7).  A
// fragment (32 MN indices = one unit, 64 K) is four ds_read_b64_tr_b8: for each
// 8-row group the 16 lanes of a group pass 8-byte pieces (lane i: k-row i / 2,
// bytes 8 (i & 1) .. of the group's 16 columns) and lane i receives the 8
// k-values of column i (measured with a probe).  Lane l takes column l & 31
// and k-rows 16 h .. + 15 and 32 + 16 h .. + 15 (h = l >> 5), the MFMA's
// operand layout.  Each half-wavefront reads 8 k-rows x 32 bytes, which the
// unit swizzle spreads over all 64 banks.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ i32x2_t lds_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
}
__device__ __forceinline__ i32x8_t frag_tr(const char* p) {
  const i32x2_t r0 = lds_tr8(p), r1 = lds_tr8(p + 8 * 256), r2 = lds_tr8(p + 32 * 256),
                r3 = lds_tr8(p + 40 * 256);
  return i32x8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// The same from 128-byte k-rows (fc1 forward's W1 and W3 halves, 64 k-rows
// of 128 bytes each; unit u of k-row k at u ^ ((k >> 1) & 3), which spreads a
// half-wavefront's 8 k-rows x 32 bytes over all 64 banks).
__device__ __forceinline__ i32x8_t frag_tr_half(const char* p) {
  const i32x2_t r0 = lds_tr8(p), r1 = lds_tr8(p + 8 * 128), r2 = lds_tr8(p + 32 * 128),
                r3 = lds_tr8(p + 40 * 128);
  return i32x8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// e4m3 x e4m3 32x32x64 block product into c; sa scales the MFMA's rows (the
// B operand), sb its columns (the A operand), both E8M0.
template <int SEL_A = 0, int SEL_B = 0>
__device__ __forceinline__ f32x16_t mma(const i32x8_t& b, const i32x8_t& a, const f32x16_t& c, int sa,
                                        int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, SEL_A, sa, SEL_B, sb);
}

// fp32 scale -> (E8M0 exponent byte, mantissa): s = m * 2^(e8 - 127) with m in
// [1, 2) for normal s; subnormal s gives e8 = 0 and m = s * 2^127 (< 1); s = 0
// (rows past the data) gives m = 0.
__device__ __forceinline__ int e8_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }
__device__ __forceinline__ float mant_of(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u >> 23) ? __uint_as_float((u & 0x007fffffu) | 0x3f800000u) : s * 0x1p127f;
}

// v_permlane32_swap on two registers: x keeps lanes 0-31 and takes y's lanes
// 0-31 into its lanes 32-63; y receives x's lanes 32-63 into its lanes 0-31.
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16f(float& x, float& y) {
  uint32_t a = __float_as_uint(x), b = __float_as_uint(y);
  swap16(a, b);
  x = __uint_as_float(a);
  y = __uint_as_float(b);
}

// One 32 x 32 block of D = C^T (lane l: C[l & 31][8 q + 4 (l >> 5) + r] in
// c[4 q + r]) -> the four 16 x 16 fragments the bf16 epilogue takes
// (fragment (i, j): lane l holds C[16 i + (l & 15)][16 j + 4 (l >> 4) + r]).
// The value for lane l' = (b5, b4, low) of fragment (i, j) sits in lane
// (b4, i, low), accumulator 4 (2 j + b5) + r: one exchange across lane bit 5
// (accumulator groups 2 j and 2 j + 1), then one across lane bit 4.
__device__ __forceinline__ void to_frags(f32x16_t c, f32x4_t& f00, f32x4_t& f01, f32x4_t& f10,
                                         f32x4_t& f11) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = c[4 * (2 * j) + r], y = c[4 * (2 * j + 1) + r];
      swap32(x, y);  // x: from lane bit 5 = 0, y: from bit 5 = 1
      swap16f(x, y);  // x: fragment row 0, y: fragment row 1
      if (j == 0) {
        f00[r] = x;
        f10[r] = y;
      } else {
        f01[r] = x;
        f11[r] = y;
      }
    }
}

__device__ __forceinline__ int bits_u32(float v) { return (int)__float_as_uint(v); }

// MX = true: MXFP8 operands.  RS: row-scaled epilogues (probabilities applied
// before W2; fc1 forward and fc2 dgrad only), as in the bf16 kernels.
//
// Persistent: a block takes tiles slot = blockIdx.x, blockIdx.x + gridDim.x,
// ... (launched with one block per compute unit, a multiple of 8; fc2 dgrad,
// whose epilogue reads a|b and would wait behind the next tile's loads, is
// launched with one block per tile).  The loads the pipeline issues past a
// tile's last stage fetch the first three stages of the next tile.
//
// Weight gradients (WG): the tiles are E x MT x NT (expert-major), K is the
// expert's rows, ceil(rows / 64) stages (0 for an empty expert, which writes
// zeros).  A 128-row token block spans two stages; its scale words come with
// the first (the second issues a zero-length load) into one of three block
// slots, (block number in the block's stream) mod 3, so that at a block's
// first stage the previous block's words are still there (the words of block
// b + 3, the next to take b's slot, are issued in the second half of b + 1's
// first stage at the earliest, after every read of b's words); the second
// stage's zero-length load lands in a fourth slot that no one reads.
template <int OP, bool MX, bool RS>
__global__ __launch_bounds__(NW * 64, 1) void gemm_fp8_kernel(GemmArgs args, int NT, int MT) {
  constexpr int WAVES_N = NW / 2;
  constexpr int WM = BM / 2, WN = BN / WAVES_N;  // 128 x 64
  constexpr int IB = WM / 32, JB = WN / 32;      // 4 x 2 blocks of 32 x 32
  constexpr bool WG = OP == OP_FC2_WGRAD || OP == OP_FC1_WGRAD;
  // B read MN-contiguous: the weight gradients, and the e4m3 forward products
  // (weights in their own orientation); fc1 forward's B is two 128-column
  // halves (W1 and W3), each stored [64 k][128 bytes]
  constexpr bool BMN = WG || (!MX && (OP == OP_FC1_FWD || OP == OP_FC2_FWD));
  constexpr bool BHALF = BMN && OP == OP_FC1_FWD;
  constexpr int DMA_STEP = 4 / DMA_PER_WAVE;     // MFMA steps per DMA instruction
  static_assert(IB == 4 && JB == 2 && DMA_STEP == 2, "tile shape");
  static_assert(!(WG && RS), "row-scaled epilogues are ragged-M only");

  // the stage ring, the scale ring, then (ragged M) the schedule scratch, the
  // inclusive prefix of the experts' M-tile counts and (row-scaled fc2 dgrad)
  // the per-row <h, dh'> partials, or (weight gradients) 64 floats per
  // wavefront for the column mantissas it trades
  constexpr int EXTRA = WG ? NW * 64 * 4 : (NW + 64 * NW + (RS ? (NW / 2) * 256 : 0)) * 4;
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE_BYTES + NS * SC_BYTES + EXTRA];
  // the expert offsets (and the token-block table), copied once: decoding a
  // tile then reads LDS, whose wait (lgkmcnt) leaves the DMA loads in flight
  __shared__ int offs[257];
  __shared__ int blks[WG ? 257 : 1];
  char* const sc_ring = lds + NS * STAGE_BYTES;
  int* const sched = (int*)(lds + NS * STAGE_BYTES + NS * SC_BYTES);
  int* const mt_incl = sched + NW;
  float* const dp_red = (float*)(mt_incl + 64 * NW);
  float* const nsc = (float*)(lds + NS * STAGE_BYTES + NS * SC_BYTES);  // WG
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int d = args.d, f = args.f, E = args.E;

  // ---------------------------------------------------------------- tiles
  // Ragged M: M = the tile's rows, K and N fixed.  Weight gradients: M and N
  // fixed, K = the expert's rows.
  const int N = WG ? ((OP == OP_FC2_WGRAD) ? d : 2 * f)
                   : ((OP == OP_FC1_FWD) ? 2 * f : (OP == OP_FC2_DGRAD ? f : d));
  const int Kr = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? d : (OP == OP_FC2_FWD ? f : 2 * f);
  const int Mw = (OP == OP_FC2_WGRAD) ? f : d;
  for (int i = tid; i <= E; i += NW * 64) {
    offs[i] = args.offsets[i];
    if constexpr (WG) blks[i] = args.blk[i];
  }
  __syncthreads();
  int total;
  if constexpr (WG) total = E * MT * NT;
  else total = mtile_prefix<BM, NW>(offs, E, mt_incl, sched) * NT;
  total = uniform(total);
  auto decode = [&](int slot, TileInfo& ti) __attribute__((always_inline)) {
    const int logical = xcd_remap(slot, total);
    if constexpr (WG) {
      ti.e = logical / (MT * NT);
      const int rem = logical % (MT * NT);
      ti.m0 = (rem / NT) * BM;
      ti.n0 = (rem % NT) * BN;
      ti.row0 = offs[ti.e];
      ti.rows = offs[ti.e + 1] - ti.row0;
    } else {
      ragged_tile(offs, mt_incl, E, NT, BM, logical, ti);
      ti.n0 *= BN;
    }
    ti.e = uniform(ti.e);
    ti.row0 = uniform(ti.row0);
    ti.rows = uniform(ti.rows);
    ti.m0 = uniform(ti.m0);
    ti.n0 = uniform(ti.n0);
  };

  // ---------------------------------------------------------------- operands
  // row lengths in bytes: ragged M, of the K-contiguous rows; weight
  // gradients, of the MN-contiguous k-rows
  const uint32_t a_ld = WG ? (uint32_t)Mw : (uint32_t)Kr;
  const uint32_t b_ld = WG ? (uint32_t)N
                           : (BMN ? (OP == OP_FC1_FWD ? (uint32_t)f : (uint32_t)d)
                                  : ((OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? (uint32_t)d : (uint32_t)f));
  const int kbr = Kr / 128;  // 128-K blocks per row

  // Per tile: buffer resources over what the tile reads (rows past an
  // expert's end or past the matrix read as zero), the stage count, and this
  // wavefront's scale-word source.  Wavefront w loads scale words 64 (w & 3)
  // .. + 63 of side w >> 2 (0: A rows, 1: B rows); word i of stage kt is at
  // sc_off + (kt / 2) * sc_kstep in sc_src (fc1 dgrad: the W3 source sc_src2
  // from block f / 128 on, at (kt / 2 - f / 128) * sc_kstep).
  struct Opnd {
    rsrc_t a_src, b_src, b_src2, sc_src, sc_src2;
    uint32_t sc_off, sc_kstep;
    int KT;
  };
  const int sside = wid >> 2, sidx = 64 * (wid & 3) + lane;
  auto setup = [&](const TileInfo& ti, Opnd& o) __attribute__((always_inline)) {
    const size_t e = (size_t)ti.e;
    o.sc_src = rsrc_t{0, 0, 0, 0};
    o.sc_src2 = rsrc_t{0, 0, 0, 0};
    o.sc_off = 0;
    o.sc_kstep = 0;
    if constexpr (WG) {
      // codes: the expert's rows from column m0 (n0) on; rows past the
      // expert, and the columns past the matrix in its last row, read zero
      const int64_t rows = ti.rows;
      o.a_src = make_rsrc(args.a_q + (size_t)ti.row0 * Mw + ti.m0,
                          (uint32_t)max(rows * Mw - ti.m0, (int64_t)0));
      o.b_src = make_rsrc(args.b_q + (size_t)ti.row0 * N + ti.n0,
                          (uint32_t)max(rows * N - ti.n0, (int64_t)0));
      o.b_src2 = o.b_src;
      o.KT = (ti.rows + BK - 1) / BK;
      // scale words [blocks][columns] (e4m3 fp32; MXFP8 four E8M0 bytes),
      // the expert's blocks from blks[e] on
      const int nblk = (ti.rows + 127) / 128;
      const int cols = sside == 0 ? Mw : N, c0 = sside == 0 ? ti.m0 : ti.n0;
      const char* sbase = sside == 0 ? (MX ? (const char*)args.a_sx : (const char*)args.a_s)
                                     : (MX ? (const char*)args.b_sx : (const char*)args.b_s);
      o.sc_src = make_rsrc(sbase + ((size_t)blks[ti.e] * cols + c0) * 4,
                           (uint32_t)max(((int64_t)nblk * cols - c0) * 4, (int64_t)0));
      o.sc_off = (uint32_t)sidx * 4u;
      o.sc_kstep = (uint32_t)cols * 4u;
    } else {
      o.a_src = make_rsrc(args.a_q + (size_t)ti.row0 * Kr, (uint32_t)ti.rows * a_ld);
      o.KT = Kr / BK;
      if constexpr (BMN && OP == OP_FC1_FWD) {  // W1 / W3 [d][f] from column n0/2
        const size_t off = e * (size_t)d * f + (size_t)(ti.n0 / 2);
        o.b_src = make_rsrc(args.b_q + off, (uint32_t)d * b_ld - (uint32_t)(ti.n0 / 2));
        o.b_src2 = make_rsrc(args.b_q2 + off, (uint32_t)d * b_ld - (uint32_t)(ti.n0 / 2));
      } else if constexpr (BMN && OP == OP_FC2_FWD) {  // W2 [f][d] from column n0
        o.b_src = make_rsrc(args.b_q + e * (size_t)f * d + (size_t)ti.n0, (uint32_t)f * b_ld - (uint32_t)ti.n0);
        o.b_src2 = o.b_src;
      } else if constexpr (OP == OP_FC1_FWD) {  // W1^T / W3^T rows n0/2 .. +128
        const size_t off = e * (size_t)f * d + (size_t)(ti.n0 / 2) * d;
        o.b_src = make_rsrc(args.b_q + off, 128u * b_ld);
        o.b_src2 = make_rsrc(args.b_q2 + off, 128u * b_ld);
      } else if constexpr (OP == OP_FC2_FWD) {  // W2^T [d][f]
        o.b_src = make_rsrc(args.b_q + e * (size_t)d * f + (size_t)ti.n0 * f, (uint32_t)(d - ti.n0) * b_ld);
        o.b_src2 = o.b_src;
      } else if constexpr (OP == OP_FC2_DGRAD) {  // W2 [f][d]
        o.b_src = make_rsrc(args.b_q + e * (size_t)f * d + (size_t)ti.n0 * d, (uint32_t)(f - ti.n0) * b_ld);
        o.b_src2 = o.b_src;
      } else {  // FC1_DGRAD: W1 | W3 [d][f], K = 2f
        const size_t off = e * (size_t)d * f + (size_t)ti.n0 * f;
        o.b_src = make_rsrc(args.b_q + off, (uint32_t)(d - ti.n0) * b_ld);
        o.b_src2 = make_rsrc(args.b_q2 + off, (uint32_t)(d - ti.n0) * b_ld);
      }
      // ---- scale words (every field set first: a zero-length resource reads nothing)
      if (sside == 0) {
        // A rows: e4m3 a_s [P][K/128] floats; MXFP8 a_sx [P][K/32] bytes
        if constexpr (MX) {
          o.sc_src = make_rsrc(args.a_sx + (size_t)ti.row0 * (Kr / 32), (uint32_t)ti.rows * (uint32_t)(Kr / 32));
          o.sc_off = (uint32_t)sidx * (uint32_t)(Kr / 32);
        } else {
          o.sc_src = make_rsrc(args.a_s + (size_t)ti.row0 * kbr, (uint32_t)ti.rows * (uint32_t)kbr * 4u);
          o.sc_off = (uint32_t)sidx * (uint32_t)kbr * 4u;
        }
        o.sc_kstep = 4u;
      } else if constexpr (MX) {
        // B rows: the E8M0 bytes [E][n][K/32] of the weight in the orientation read
        const int xb = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? d / 32 : f / 32;
        size_t b0;
        int brows;
        if constexpr (OP == OP_FC1_FWD) {
          b0 = (e * f + ti.n0 / 2) * xb; brows = 128;
        } else if constexpr (OP == OP_FC2_FWD) {
          b0 = (e * d + ti.n0) * xb; brows = d - ti.n0;
        } else if constexpr (OP == OP_FC2_DGRAD) {
          b0 = (e * f + ti.n0) * xb; brows = f - ti.n0;
        } else {
          b0 = (e * d + ti.n0) * xb; brows = d - ti.n0;
        }
        const bool w3 = OP == OP_FC1_FWD && sidx >= 128;  // fc1 forward: B rows 128.. are W3's
        o.sc_src = make_rsrc((w3 ? args.b_sx2 : args.b_sx) + b0, (uint32_t)brows * (uint32_t)xb);
        if constexpr (OP == OP_FC1_DGRAD) o.sc_src2 = make_rsrc(args.b_sx2 + b0, (uint32_t)brows * (uint32_t)xb);
        o.sc_off = (uint32_t)((OP == OP_FC1_FWD) ? (sidx & 127) : sidx) * (uint32_t)xb;
        o.sc_kstep = 4u;
      } else {
        // B rows: e4m3 weight block scales, [E][d/128][f/128] (W1, W3) or
        // [E][f/128][d/128] (W2); every B row of a 128-row block reads the same
        // word (rows past N read past the range: zero)
        const int db = d / 128, fb = f / 128;
        const int nb = db * fb;
        const float* s = (OP == OP_FC1_FWD && sidx >= 128) ? args.b_s2 : args.b_s;
        o.sc_src = make_rsrc(s + e * (size_t)nb, (uint32_t)nb * 4u);
        if constexpr (OP == OP_FC1_DGRAD) o.sc_src2 = make_rsrc(args.b_s2 + e * (size_t)nb, (uint32_t)nb * 4u);
        if constexpr (OP == OP_FC1_FWD) {  // block (kb, f-block of the tile's W1 / W3 rows)
          o.sc_off = (uint32_t)((ti.n0 / 2) / 128) * 4u;
          o.sc_kstep = (uint32_t)fb * 4u;
        } else if constexpr (OP == OP_FC2_FWD) {  // W2 block (kb, d-block of the row)
          const int nbk = (ti.n0 + sidx) / 128;
          o.sc_off = nbk < db ? (uint32_t)nbk * 4u : 0x40000000u;
          o.sc_kstep = (uint32_t)db * 4u;
        } else if constexpr (OP == OP_FC2_DGRAD) {  // W2 block (f-block of the row, kb)
          const int nbk = (ti.n0 + sidx) / 128;
          o.sc_off = nbk < fb ? (uint32_t)nbk * (uint32_t)db * 4u : 0x40000000u;
          o.sc_kstep = 4u;
        } else {  // FC1_DGRAD: W1 / W3 block (d-block of the row, kb mod f/128)
          const int nbk = (ti.n0 + sidx) / 128;
          o.sc_off = nbk < db ? (uint32_t)nbk * (uint32_t)fb * 4u : 0x40000000u;
          o.sc_kstep = 4u;
        }
      }
    }
    o.sc_src = uniform_rsrc(o.sc_src);
    o.sc_src2 = uniform_rsrc(o.sc_src2);
    o.sc_kstep = (uint32_t)uniform((int)o.sc_kstep);
    o.KT = uniform(o.KT);
  };

  // ---- DMA lane offsets.  Ragged M: instruction t (0..15) of an operand
  // covers tile rows 16 t .. 16 t + 15; lane -> row 16 t + lane / 4, stored
  // chunk lane % 4 holding logical chunk (lane % 4) ^ swz(row).  Weight
  // gradients: instruction t covers k-rows 4 t .. 4 t + 3 (256 bytes each);
  // lane -> k-row 4 t + lane / 16, stored 16-byte chunk p = lane % 16, i.e.
  // half p & 1 of unit p / 2, holding logical unit (p / 2) ^ (k & 7).  This
  // wavefront issues t = 2 wid + q, q < 2, for A and for B.
  uint32_t a_off[DMA_PER_WAVE], b_off[DMA_PER_WAVE];
#pragma unroll
  for (int q = 0; q < DMA_PER_WAVE; ++q) {
    const int t = wid * DMA_PER_WAVE + q;
    if constexpr (WG) {
      const int k = 4 * t + (lane >> 4), p = lane & 15;
      const uint32_t col = (uint32_t)((((p >> 1) ^ (k & 7)) << 5) | ((p & 1) << 4));
      a_off[q] = (uint32_t)k * a_ld + col;
      b_off[q] = (uint32_t)k * b_ld + col;
    } else {
      const int row = 16 * t + (lane >> 2);
      const uint32_t ch = (uint32_t)(((lane & 3) ^ swz(row)) << 4);
      a_off[q] = (uint32_t)row * a_ld + ch;
      if constexpr (BHALF) {
        // instruction t: half t / 8 (W1, W3), k-rows 8 (t % 8) .. + 7 of 128
        // bytes; lane -> k-row 8 (t % 8) + lane / 8, stored 16-byte chunk
        // p = lane % 8, i.e. half p & 1 of unit p / 2, holding logical unit
        // (p / 2) ^ ((k / 2) & 3)
        const int k = 8 * (t & 7) + (lane >> 3), p = lane & 7;
        b_off[q] = (uint32_t)k * b_ld + (uint32_t)((((p >> 1) ^ ((k >> 1) & 3)) << 5) | ((p & 1) << 4));
      } else if constexpr (BMN) {
        const int k = 4 * t + (lane >> 4), p = lane & 15;
        b_off[q] = (uint32_t)k * b_ld + (uint32_t)((((p >> 1) ^ (k & 7)) << 5) | ((p & 1) << 4));
      } else {
        const int brow = (OP == OP_FC1_FWD) ? (row & 127) : row;  // fc1: rows 128.. come from W3
        b_off[q] = (uint32_t)brow * b_ld + ch;
      }
    }
  }
  const uint32_t lds_base =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(size_t)LDS_PTR(lds));
  const uint32_t sc_base = lds_base + (uint32_t)(NS * STAGE_BYTES) + (uint32_t)(sside * 1024 + (wid & 3) * 256);

  TileInfo ti, tn;
  Opnd cur, nxt;
  int slot = blockIdx.x;
  if (slot >= total) return;
  decode(slot, ti);
  setup(ti, cur);
  tn = ti;
  nxt = cur;
  int phase = 0;       // ring slot of the current tile's stage 0
  int bph = 0;         // weight gradients: block slot of the current tile's first block
  bool cross = false;  // stages past the current tile's last fetch the next tile's first three

  // DMA instruction Q of this wavefront for stage s of the stream, counted
  // from the current tile's stage 0: Q < 2 A, Q == 2 the scale words, Q > 2 B.
  // TAIL = false: the caller knows that s is a stage of the current tile.
  auto issue_one = [&](int s, auto Q, auto TAIL) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
    const uint32_t slot_s = (uint32_t)(phase + s) % NS;
    const uint32_t st_base = lds_base + slot_s * STAGE_BYTES;
    const bool in_cur = !decltype(TAIL)::value || s < cur.KT;
    const int kt = in_cur ? s : s - cur.KT;
    const uint32_t k0 = (uint32_t)kt * BK;
    const bool live = in_cur || cross;
    if constexpr (q < DMA_PER_WAVE) {
      const int t = wid * DMA_PER_WAVE + q;
      rsrc_t r = pick(in_cur, cur.a_src, nxt.a_src);
      r[2] = live ? r[2] : 0;
      dma16(uniform_rsrc(r), a_off[q] + (WG ? k0 * a_ld : k0), st_base + (uint32_t)(t * 1024));
    } else if constexpr (q == DMA_PER_WAVE) {
      // a 128-K block's words serve both of its stages and are loaded with
      // the first; the second stage's DMA reads nothing (a zero-length range:
      // no memory request, and the zeros land in a slot that no one reads),
      // so that every stage issues the same loads for the waits
      const int kb = kt >> 1;
      rsrc_t r;
      uint32_t voff;
      const uint32_t kstep = in_cur ? cur.sc_kstep : nxt.sc_kstep;
      const uint32_t soff = in_cur ? cur.sc_off : nxt.sc_off;
      if constexpr (OP == OP_FC1_DGRAD) {
        // K = [da | db]: blocks from f / 128 on multiply W3
        const int fbk = f / 128;
        const bool second = sside == 1 && kb >= fbk;
        r = pick(in_cur, pick(second, cur.sc_src2, cur.sc_src), pick(second, nxt.sc_src2, nxt.sc_src));
        voff = soff + (uint32_t)(second ? kb - fbk : kb) * kstep;
      } else {
        r = pick(in_cur, cur.sc_src, nxt.sc_src);
        voff = soff + (uint32_t)kb * kstep;
      }
      r[2] = (live && (kt & 1) == 0) ? r[2] : 0;
      // weight gradients: the block's slot, or slot 3 for a block's second
      // stage -- formed without a branch (a branch here splits the stage, and
      // the compiler then sinks the first half's MFMAs below the barrier)
      uint32_t sl;
      if constexpr (WG)
        sl = (uint32_t)((bph + (in_cur ? 0 : (cur.KT + 1) >> 1) + kb) % 3) | (3u * (uint32_t)(kt & 1));
      else sl = slot_s;
      dma4(uniform_rsrc(r), voff, sc_base + sl * SC_BYTES);
    } else {
      const int qq = q - DMA_PER_WAVE - 1;
      const int t = wid * DMA_PER_WAVE + qq;
      const uint32_t dst = st_base + (uint32_t)(OPND_BYTES + t * 1024);
      rsrc_t r;
      uint32_t voff;
      if constexpr (OP == OP_FC1_FWD) {
        const bool second = t >= 8;
        r = pick(in_cur, pick(second, cur.b_src2, cur.b_src), pick(second, nxt.b_src2, nxt.b_src));
        voff = b_off[qq] + (BMN ? k0 * b_ld : k0);
      } else if constexpr (OP == OP_FC1_DGRAD) {
        const bool second = (int)k0 >= f;
        r = pick(in_cur, pick(second, cur.b_src2, cur.b_src), pick(second, nxt.b_src2, nxt.b_src));
        voff = b_off[qq] + (second ? k0 - (uint32_t)f : k0);
      } else {
        r = pick(in_cur, cur.b_src, nxt.b_src);
        voff = b_off[qq] + (BMN ? k0 * b_ld : k0);
      }
      r[2] = live ? r[2] : 0;
      dma16(uniform_rsrc(r), voff, dst);
    }
  };

  // ---- fragments.  Ragged M: block ib of A = rows wm*WM + 32 ib + (lane &
  // 31); block jb of B = rows b_row0(jb) + (lane & 31) (fc1 forward: W1 rows,
  // then the same W3 rows); lane group h reads chunks h and h + 2.  Weight
  // gradients: block ib of A = columns wm*WM + 32 ib .. (LDS unit 4 wm + ib),
  // block jb of B = columns wn*WN + 32 jb .. (unit 2 wn + jb), by frag_tr.
  const int lh = lane >> 5, l31 = lane & 31;
  auto b_row0 = [&](int jb) __attribute__((always_inline)) -> int {
    if constexpr (OP == OP_FC1_FWD) return jb * 128 + wn * (WN / 2);
    else return wn * WN + 32 * jb;
  };
  const int fsw = swz(l31);
  const uint32_t fc0 = (uint32_t)((lh ^ fsw) << 4), fc1 = (uint32_t)(((lh + 2) ^ fsw) << 4);
  auto frag = [&](const char* p) __attribute__((always_inline)) -> i32x8_t {
    const i32x4_t lo = *(const __attribute__((address_space(3))) i32x4_t*)(p + fc0);
    const i32x4_t hi = *(const __attribute__((address_space(3))) i32x4_t*)(p + fc1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // frag_tr lane address: k-row 16 h + (lane & 15) / 2 (of the first group),
  // bytes 16 ((lane >> 4) & 1) + 8 (lane & 1) of the unit, whose stored position
  // is u ^ ((lane & 15) / 2) (the k-row's low three bits)
  const int ih = (lane & 15) >> 1;
  const uint32_t tr_lane = (uint32_t)((16 * lh + ih) * 256 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1));
  auto read_a = [&](const char* st, int ib) __attribute__((always_inline)) -> i32x8_t {
    if constexpr (WG) return frag_tr(st + tr_lane + (((4 * wm + ib) ^ ih) << 5));
    else return frag(st + (wm * WM + 32 * ib + l31) * BK);
  };
  // fc1 forward's halves: k-row 16 h + (lane & 15) / 2 of 128 bytes, unit
  // position wn ^ ((lane & 15) / 4) (the k-row's bits 1..2), the same bytes
  const uint32_t trh_lane = (uint32_t)((16 * lh + ih) * 128 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1));
  auto read_b = [&](const char* st, int jb) __attribute__((always_inline)) -> i32x8_t {
    if constexpr (BHALF) return frag_tr_half(st + OPND_BYTES + jb * 8192 + trh_lane + ((wn ^ (ih >> 1)) << 5));
    else if constexpr (BMN) return frag_tr(st + OPND_BYTES + tr_lane + (((2 * wn + jb) ^ ih) << 5));
    else return frag(st + OPND_BYTES + (b_row0(jb) + l31) * BK);
  };
  auto stage_ptr = [&](int s) __attribute__((always_inline)) -> const char* {
    return lds + ((uint32_t)(phase + s) % NS) * STAGE_BYTES;
  };
  // the scale words of stage s: in the slot of its block's first stage
  // (weight gradients: its block's slot; b_back = 1: the block before)
  auto scale_ptr = [&](int s, int b_back = 0) __attribute__((always_inline)) -> const char* {
    if constexpr (WG) return sc_ring + ((bph + (s >> 1) + 3 - b_back) % 3) * SC_BYTES;
    else return sc_ring + ((uint32_t)(phase + (s & ~1)) % NS) * SC_BYTES;
  };

  // ---------------------------------------------------------------- scales
  // MXFP8: ea[ib], the E8M0 byte of the lane's A row in block ib (the MFMA's
  // column scale), eb[jb] that of its B row (the row scale).  e4m3: the same
  // bytes packed into ea_pk (byte ib) and eb_pk (byte jb), taken by the MFMA's
  // byte select, and ma / mb, the mantissas the accumulators are in units of;
  // in the ragged products every B row of a 128-row weight block has the same
  // scale, so eb_pk and mb are uniform (the weight gradients keep the B-side
  // mantissas in LDS instead, see nsc_ratio).
  i32x8_t af[IB], b0, b1;
  int ea[IB], eb[JB];
  int ea_pk = 0, eb_pk = 0;
  float ma[IB], mb[JB];
  f32x16_t acc[IB][JB];
  // weight gradients, e4m3: the wavefront's 64 B-column values v (lane l:
  // column wn*WN + l) traded through LDS and applied with the lane's A-side
  // factors: acc[ib][jb][4 q + r] *= fa[ib] * v(32 jb + 8 q + 4 h + r)
  auto apply_cols = [&](float v, const float (&fa)[IB]) __attribute__((always_inline)) {
    nsc[wid * 64 + lane] = v;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wavefront's writes before its reads
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t vn = *(const f32x4_t*)&nsc[wid * 64 + 32 * jb + 8 * q + 4 * lh];
#pragma unroll
        for (int ib = 0; ib < IB; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ib][jb][4 * q + r] *= fa[ib] * vn[r];
      }
  };
  // The scales of stage kt; e4m3, at the first stage of a 128-K block: the
  // new exponents and mantissas, and the accumulators times u_old / u_new
  // (not at a tile's first stage, where they are zero).  Measured faster than
  // multiplying each block right before its first MFMA, which keeps the
  // factors in registers through the stage.
  auto stage_scales = [&](int kt) __attribute__((always_inline)) {
    const char* sc = scale_ptr(kt);
    const uint32_t* wa = (const uint32_t*)sc;
    const uint32_t* wb = (const uint32_t*)(sc + 1024);
    if constexpr (MX) {
      const int sh = 8 * (2 * (kt & 1) + lh);
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) ea[ib] = (int)((wa[wm * WM + 32 * ib + l31] >> sh) & 0xffu);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) eb[jb] = (int)((wb[b_row0(jb) + l31] >> sh) & 0xffu);
    } else if ((kt & 1) == 0) {
      float ra[IB], rb[JB];
      ea_pk = 0;
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        const float s = __uint_as_float(wa[wm * WM + 32 * ib + l31]);
        ea_pk |= e8_of(s) << (8 * ib);
        const float m = mant_of(s);
        ra[ib] = ma[ib] * __builtin_amdgcn_rcpf(m);
        ma[ib] = m;
      }
      eb_pk = 0;
      if constexpr (WG) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) eb_pk |= e8_of(__uint_as_float(wb[b_row0(jb) + l31])) << (8 * jb);
        if (kt > 0) {
          const uint32_t* wo = (const uint32_t*)(scale_ptr(kt, 1) + 1024);
          const int n = wn * WN + lane;
          apply_cols(mant_of(__uint_as_float(wo[n])) * __builtin_amdgcn_rcpf(mant_of(__uint_as_float(wb[n]))),
                     ra);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float s = __uint_as_float((uint32_t)uniform((int)wb[b_row0(jb)]));
          eb_pk |= e8_of(s) << (8 * jb);
          const float m = mant_of(s);
          rb[jb] = mb[jb] * __builtin_amdgcn_rcpf(m);
          mb[jb] = m;
        }
        eb_pk = uniform(eb_pk);
        if (kt > 0) {
#pragma unroll
          for (int ib = 0; ib < IB; ++ib)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
              const float g = ra[ib] * rb[jb];
#pragma unroll
              for (int x = 0; x < 16; ++x) acc[ib][jb][x] *= g;
            }
        }
      }
    }
  };
  // block product (ib, jb) of this stage
  auto product = [&](auto IBc, auto JBc, const i32x8_t& b) __attribute__((always_inline)) {
    constexpr int ib = decltype(IBc)::value, jb = decltype(JBc)::value;
    if constexpr (MX) acc[ib][jb] = mma(b, af[ib], acc[ib][jb], eb[jb], ea[ib]);
    else acc[ib][jb] = mma<jb, ib>(b, af[ib], acc[ib][jb], eb_pk, ea_pk);
  };

  // ---------------------------------------------------------------- main loop
  // Per stage the first half multiplies the four A blocks by B block 0 (read
  // during the previous stage), the second half by B block 1 (read at the
  // start of this one).  The wait + barrier that releases the next stage (and
  // frees the oldest buffer for stage kt+3) sits between the halves; right
  // after it B block 0 of the next stage is read, and each A block is
  // replaced by the next stage's as soon as its second MFMA is issued.  The
  // refill of a freed buffer is spread over the stage: B operand of stage kt+2
  // in the first half, A operand and scale words of stage kt+3 in the second.
  // (Rows past a ragged tile's end are multiplied like the others: a second
  // copy of the loop that skips their blocks, as the bf16 fc1 products have,
  // pushes the fc1 products here past the register budget -- they spill, and
  // the reloads before the loop make every stage wait for all loads.)
  auto stage_body = [&](int kt, const char* __restrict__ st, const char* __restrict__ nst, auto TAIL)
      __attribute__((always_inline)) {
    stage_scales(kt);
    b1 = read_b(st, 1);
    static_for<0, IB>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = U.value;
      __builtin_amdgcn_sched_barrier(0);
      product(IntC<u>{}, IntC<0>{}, b0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (u % DMA_STEP == DMA_STEP - 1)
        issue_one(kt + LOOK - 1, IntC<DMA_PER_WAVE + 1 + u / DMA_STEP>{}, TAIL);
    });
    // stage kt+1 has landed for this wavefront; after the barrier it has for
    // all, and every wavefront is done with stage kt-1, whose buffer now
    // takes stage kt+3
    wait_vmcnt<LOADS_PER_STAGE * (LOOK - 2)>();
    block_barrier();
    b0 = read_b(nst, 0);
    static_for<0, IB>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = U.value;
      __builtin_amdgcn_sched_barrier(0);
      product(IntC<u>{}, IntC<1>{}, b1);
      __builtin_amdgcn_sched_barrier(0);
      af[u] = read_a(nst, u);
      if constexpr (u % DMA_STEP == DMA_STEP - 1) issue_one(kt + LOOK, IntC<u / DMA_STEP>{}, TAIL);
      if constexpr (u == IB - 1) issue_one(kt + LOOK, IntC<DMA_PER_WAVE>{}, TAIL);
    });
  };

  bool fresh = true;  // the current tile's first stages are not yet issued
  for (;;) {
    const int nslot = slot + (int)gridDim.x;
    const bool have_next = nslot < total;
    if (have_next) {
      decode(nslot, tn);
      setup(tn, nxt);
    }
    cross = OP != OP_FC2_DGRAD && have_next && cur.KT >= 1 && nxt.KT >= LOOK;
    if (fresh) {
      // stages 0 .. LOOK-2 and stage LOOK-1's A operand and scale words in
      // flight (its B operand follows in stage 0); wait for stage 0
      static_for<0, LOOK - 1>([&](auto S) __attribute__((always_inline)) {
        static_for<0, LOADS_PER_STAGE>([&](auto Q) __attribute__((always_inline)) {
          issue_one(S.value, Q, IntC<1>{});
        });
      });
      static_for<0, DMA_PER_WAVE + 1>([&](auto Q) __attribute__((always_inline)) {
        issue_one(LOOK - 1, Q, IntC<1>{});
      });
      wait_vmcnt<LOADS_PER_STAGE * (LOOK - 2) + DMA_PER_WAVE + 1>();
      block_barrier();
    }
    {
      const char* st0 = stage_ptr(0);
      static_for<0, IB>([&](auto I) __attribute__((always_inline)) { af[I.value] = read_a(st0, I.value); });
      b0 = read_b(st0, 0);
    }
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
      ma[ib] = 1.0f;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) acc[ib][jb] = f32x16_t{};
    }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) mb[jb] = 1.0f;
    // the last LOOK stages issue the loads that may fall past the tile
    const int kt_tail = max(cur.KT - LOOK, 0);
    for (int kt = 0; kt < kt_tail; ++kt) stage_body(kt, stage_ptr(kt), stage_ptr(kt + 1), IntC<0>{});
    for (int kt = kt_tail; kt < cur.KT; ++kt) stage_body(kt, stage_ptr(kt), stage_ptr(kt + 1), IntC<1>{});

    // ---------------------------------------------------------------- epilogue
    // e4m3: back from units of the last block's mantissas
    if constexpr (!MX && WG) {
      if (cur.KT > 0) {
        const uint32_t* wl = (const uint32_t*)(scale_ptr(cur.KT - 1) + 1024);
        apply_cols(mant_of(__uint_as_float(wl[wn * WN + lane])), ma);
      }
    } else if constexpr (!MX) {
#pragma unroll
      for (int ib = 0; ib < IB; ++ib)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float g = ma[ib] * mb[jb];
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[ib][jb][x] *= g;
        }
    }
    {
      f32x4_t frg[2 * IB][2 * JB];
#pragma unroll
      for (int ib = 0; ib < IB; ++ib)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
          to_frags(acc[ib][jb], frg[2 * ib][2 * jb], frg[2 * ib][2 * jb + 1], frg[2 * ib + 1][2 * jb],
                   frg[2 * ib + 1][2 * jb + 1]);
      if constexpr (WG) store_tile<OP, 2 * IB, 2 * JB, WM, WN, false>(args, frg, ti, Mw, N, wm, wn, lane);
      else store_tile<OP, 2 * IB, 2 * JB, WM, WN, true, RS>(args, frg, ti, ti.rows, N, wm, wn, lane, dp_red);
    }
    if (!have_next) break;
    if constexpr (WG) bph = (bph + ((cur.KT + 1) >> 1)) % 3;
    if (cross) {
      phase = (int)((uint32_t)(phase + cur.KT) % NS);
      fresh = false;
    } else {
      // the past-the-end loads read nothing but still write the ring: drain
      // them (and every LDS read) before the next tile's prologue
      wait_vmcnt<0>();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      block_barrier();
      fresh = true;
    }
    slot = nslot;
    ti = tn;
    cur = nxt;
  }
  wait_vmcnt<0>();  // no LDS write may be in flight when the block ends
}

template <int OP, bool MX>
int launch(const GemmArgs& a, hipStream_t s) {
  constexpr bool WG = OP == OP_FC2_WGRAD || OP == OP_FC1_WGRAD;
  int NT, MT = 0;
  int64_t grid;
  if constexpr (WG) {
    const int M = (OP == OP_FC2_WGRAD) ? a.f : a.d;
    const int N = (OP == OP_FC2_WGRAD) ? a.d : 2 * a.f;
    MT = (M + BM - 1) / BM;
    NT = (N + BN - 1) / BN;
    grid = (int64_t)a.E * MT * NT;
  } else {
    const int N = (OP == OP_FC1_FWD) ? 2 * a.f : (OP == OP_FC2_DGRAD ? a.f : a.d);
    NT = (N + BN - 1) / BN;
    grid = ((int64_t)a.P / BM + a.E) * NT;  // upper bound of the device-side tile count
  }
  if (grid <= 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  // persistent blocks, one per compute unit (a multiple of 8), except fc2
  // dgrad (see the kernel)
  if (OP != OP_FC2_DGRAD) {
    const int ncu = gemm_persistent_blocks();
    if (ncu <= 0) return MOE_ERR_HIP;
    if (grid > ncu) grid = ncu;
  }
  const unsigned g = (unsigned)grid;
  bool scaled = false;  // row-scaled variant: only fc1 forward and fc2 dgrad change
  if constexpr (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) {
    if (a.row_prob) {
      gemm_fp8_kernel<OP, MX, true><<<g, NW * 64, 0, s>>>(a, NT, MT);
      scaled = true;
    }
  }
  if (!scaled) gemm_fp8_kernel<OP, MX, false><<<g, NW * 64, 0, s>>>(a, NT, MT);
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
