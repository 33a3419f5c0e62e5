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
// device offsets, counts ceil(m_e/BM) M-tiles per expert and scans them once;
// a tile number then maps to its (expert, M-tile, N-tile) by a search over
// that prefix.  One persistent block per compute unit walks the tile numbers
// with a stride of the grid; numbers past the device-side count end it.
// Block ids are remapped so that the blocks one XCD runs at a time (ids with
// the same value mod 8) take consecutive tiles: they share A rows and expert
// weights in that XCD's L2.  Weight-gradient products have a fixed grid of
// E x (M/BM) x (N/BN) tiles; K is the expert's row count, 0 for an empty
// expert, which then writes zeros.
//
// Block tile 256 x 256, 8 wavefronts in a 2x4 grid, each owning a 128 x 64
// sub-tile of 16x16 MFMA blocks (v_mfma_f32_16x16x32_bf16, fp32 accumulators).  K advances in stages of 32 through a 4-deep LDS ring (32 KB per
// stage): every operand byte is moved by buffer_load ... lds (global -> LDS
// without registers; rows past an expert's end or past K are zero-filled by
// the buffer range check), issued up to three stages ahead.  LDS layouts:
//  * K-contiguous operands: 256 rows of 64 bytes; 16-byte chunk c of row r is
//    stored at chunk c ^ kc_swz(r), so that a fragment read (ds_read_b128,
//    one chunk of 16 consecutive rows) is free of bank conflicts (measured);
//  * MN-contiguous operands (forward weights, both weight-gradient operands):
//    two halves of [32 k][128 mn] (256-byte rows); 32-byte unit u of k-row k
//    is stored at unit u ^ f(k), f(k) = (k & 3) | ((k >> 3) & 1) << 2.  A
//    fragment is two ds_read_b64_tr_b16 (each 16-lane group transposes a
//    4 x 16 block), which turns the MN-contiguous tile into the K-contiguous
//    8-element vectors the MFMA takes.
// For fc1 the two halves of the B tile are the same 128 f-columns of W1 and
// of W3; the first half of a wavefront's B fragments come from W1 and the
// second half from the same columns of W3, so a lane holds a and b of one
// element (accumulators j and j + FN/2) and applies SwiGLU in the epilogue.
// One barrier per stage sits in the middle of the stage's MFMAs, after which
// the next stage's fragments are prefetched; the MFMA computes C^T = B^T A^T
// so that a lane ends with four consecutive columns of one row.
#include "common.h"
#include "internal.h"
#include "gemm_common.h"
#include "schedule.h"

#include <atomic>

namespace tre {

namespace {
using namespace gemm;

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int OPND_BYTES = 256 * BK * 2;         // one operand of one stage (16 KB)
constexpr int STAGE_BYTES = 2 * OPND_BYTES;      // A then B
constexpr int DMA_PER_OPND = OPND_BYTES / 1024;  // 16 one-KB DMA instructions
// a buffer offset past every operand's range: the load returns zeros (the
// gathered operand's range, T * d * 2 bytes, stays below 2^31)
constexpr uint32_t kPastRange = 0x80000000u;

template <int OP>
struct OpTraits {
  static constexpr bool ragged_m = OP <= OP_FC1_DGRAD;             // ops 0..3
  static constexpr bool a_kcontig = OP <= OP_FC1_DGRAD;            // ops 0..3
  static constexpr bool b_kcontig = OP == OP_FC2_DGRAD || OP == OP_FC1_DGRAD;
};

// Chunk swizzle of K-contiguous LDS rows (64 bytes = 4 chunks of 16 bytes).
// A fragment read takes one chunk from 16 consecutive rows; chunk c of row r
// is stored at c ^ kc_swz(r).  With kc_swz(r) = (r >> 1) & 3 every 8
// consecutive rows cover all 64 banks, and rows r and r + 8 use the same
// banks: the LDS bank-conflict counter (SQ_LDS_BANK_CONFLICT) reads zero for
// the fragment reads, where adding bit 3 of r to the swizzle (so that 16 rows
// cover the banks twice over in a different order) made half of the LDS
// cycles conflict cycles.  The swizzle depends on bits 1..2 of r only, so it
// is the same for any 16-row aligned group.
__device__ __forceinline__ int kc_swz(int r) { return (r >> 1) & 3; }

__device__ __forceinline__ bf16x8_t lds_b128(const char* p) {
  return *(const __attribute__((address_space(3))) bf16x8_t*)(p);
}

// Two transposing reads (k rows kr..kr+3 and kr+4..kr+7) -> one fragment.
__device__ __forceinline__ bf16x8_t lds_tr_pair(const char* p) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p + 4 * 256));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// NW wavefronts per block in a 2 x (NW/2) grid: NW = 4 gives 128 x 128
// wavefront tiles (one wavefront per SIMD), NW = 8 gives 128 x 64 (two per
// SIMD, so one wavefront's stalls leave the matrix core to the other).
//
// Persistent: a block takes tiles slot = blockIdx.x, blockIdx.x + gridDim.x,
// ... (launched with one block per compute unit, gridDim.x is a multiple of
// 8, so a block's slots stay on its XCD and the XCD remap of the tile
// numbering holds; launched with a block per tile, as fc2 dgrad is, every
// block takes one).  The K stages of a block's
// tiles form one stream through the LDS ring: the loads the pipeline issues
// past the current tile's last stage fetch the first three stages of the
// next tile (decoded when the current one starts), so the next tile's
// prologue runs under the current tile's last stages and its epilogue
// stores.  When the next tile has fewer than three stages (a weight gradient
// of an expert with under 96 rows) those loads read nothing (a zero-length
// buffer range) and the next tile starts its own prologue after a full wait.
// (LOOK = 3 below: the ring depth minus one.)
//
// GATHER (fc1 forward and fc1 weight gradient): the permuted input xp is not
// read; row r of it is row token_of[r] of x (args.gather, args.gx), fetched by
// the same DMA (the permutation fused into the operand loader).  fc1 forward
// takes the rows' offsets once per tile.  In the fc1 weight gradient the rows
// run along K, so every stage needs new ones: the wavefront's two A DMA
// instructions cover the same four k-rows (both 128-column halves), and five
// stages ahead each wavefront DMAs the token ids of those rows into one of
// eight LDS slots of its own (one more load per stage in the wait counts).  It
// reads the ids of stage kt + 3 at the top of stage kt, where they have
// landed, and turns them into the lane offsets of that stage's A loads after
// the stage's barrier, so the read's latency hides under the MFMAs between.
template <int OP, int NW, bool RS, bool GATHER = false>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_kernel(GemmArgs args, int NT, int MT) {
  constexpr int WAVES_N = NW / 2;
  constexpr int WM = BM / 2, WN = BN / WAVES_N;  // wavefront sub-tile
  constexpr int FM = WM / 16, FN = WN / 16;      // 16x16 MFMA blocks per wavefront
  constexpr int HB = FN / 2;                     // B fragments per half stage
  constexpr int DMA_PER_WAVE = DMA_PER_OPND / NW;  // per operand per stage
  using TR = OpTraits<OP>;
  // ragged-M products (ungathered): the first row of wavefronts (wid < NW/2)
  // issues its own DMA instructions and those of wavefront wid + NW/2, whose
  // rows lie 128 further on (or, fc2 forward's MN-contiguous weights, whose
  // columns do), and the second row issues none.  The second row is the one
  // the first waits for at every barrier (it loses the SIMD's issue
  // arbitration to the older wavefront), so moving its DMA issue to the first
  // row shortens the stage (measured on the Qwen3 shape: fc2 forward and fc2
  // dgrad 6-7 % faster; the weight gradients, whose first row has less slack,
  // 4 % slower, so they keep one share per wavefront).
  constexpr int DW = (TR::ragged_m && !GATHER) ? 2 : 1;
  constexpr int LOADS_PER_STAGE = 2 * DMA_PER_WAVE * DW;  // of an issuing wavefront
  constexpr int DMA_STEP = 4 / DMA_PER_WAVE;       // MFMA steps per DMA instruction
  static_assert(FM == 8 && HB * 2 == FN && DMA_STEP * DMA_PER_WAVE == 4, "tile shape");
  // LDS ring depth (measured on the Qwen3 shape: 3 stages cost 10-30 % on
  // every product, 5 stages, possible for the weight gradients only, made
  // them 5-10 % slower)
  constexpr int NS = 4;
  constexpr int LOOK = NS - 1;  // stage kt + LOOK is issued during stage kt
  // gathered weight gradient: token ids of stage kt + TLOOK are loaded in stage kt
  constexpr bool GW = GATHER && OP == OP_FC1_WGRAD;
  constexpr int TLOOK = LOOK + 2;
  constexpr int VM_STAGE = LOADS_PER_STAGE + (GW ? 1 : 0);  // vector-memory loads per stage

  // the stage ring, then (ragged M) the schedule scratch, the inclusive prefix
  // of the experts' M-tile counts and (row-scaled fc2 dgrad) the wavefronts'
  // per-row <h, dh'> partials
  // (gathered weight gradient: eight 256-byte token slots per wavefront)
  constexpr int TSLOTS = 8;
  constexpr int EXTRA = TR::ragged_m ? (NW + 64 * NW + (RS ? (NW / 2) * 256 : 0)) * 4
                                     : (GW ? NW * TSLOTS * 256 : 0);
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE_BYTES + EXTRA];
  // the expert offsets, copied once: decoding a tile then reads LDS, whose
  // wait (lgkmcnt) leaves the DMA loads in flight, where a global read's
  // vmcnt(0) at the top of every tile drained the prefetched stages and the
  // previous tile's epilogue stores
  __shared__ int offs[257];
  int* const sched = (int*)(lds + NS * STAGE_BYTES);
  int* const mt_incl = sched + NW;
  float* const dp_red = (float*)(mt_incl + 64 * NW);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int d = args.d, f = args.f;

  // ---------------------------------------------------------------- tiles
  // Ragged M: M = the tile's rows, K and N fixed.  Weight gradients: M and N
  // fixed, K = the expert's rows (0 for an empty expert, which writes zeros).
  const int N = TR::ragged_m ? ((OP == OP_FC1_FWD) ? 2 * f : (OP == OP_FC2_DGRAD ? f : d))
                             : ((OP == OP_FC2_WGRAD) ? d : 2 * f);
  const int Kfix = (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD) ? d : (OP == OP_FC2_FWD ? f : 2 * f);
  const int Mfix = (OP == OP_FC2_WGRAD) ? f : d;
  int total;
  for (int i = tid; i <= args.E; i += NW * 64) offs[i] = args.offsets[i];
  __syncthreads();
  if constexpr (TR::ragged_m) total = mtile_prefix<BM, NW>(offs, args.E, mt_incl, sched) * NT;
  else total = args.E * MT * NT;
  total = uniform(total);
  auto decode = [&](int slot, TileInfo& ti) __attribute__((always_inline)) {
    const int logical = xcd_remap(slot, total);
    if constexpr (TR::ragged_m) {
      ragged_tile(offs, mt_incl, args.E, NT, BM, logical, ti);
      ti.n0 *= BN;
    } else {
      ti.e = logical / (MT * NT);
      const int rem = logical % (MT * NT);
      ti.m0 = (rem / NT) * BM;
      ti.n0 = (rem % NT) * BN;
      ti.row0 = offs[ti.e];
      ti.rows = offs[ti.e + 1] - ti.row0;
    }
    ti.e = uniform(ti.e);
    ti.row0 = uniform(ti.row0);
    ti.rows = uniform(ti.rows);
    ti.m0 = uniform(ti.m0);
    ti.n0 = uniform(ti.n0);
  };

  // ---------------------------------------------------------------- operands
  // Per tile: buffer resources over the rows the tile reads (rows past an
  // expert's end or past K read as zero), the wavefront's DMA lane offsets
  // and the stage count.
  struct Opnd {
    rsrc_t a_src, b_src, b_src2;
    uint32_t a_off[DMA_PER_WAVE], b_off[DMA_PER_WAVE];
    uint32_t a_dw, b_dw;  // DW = 2: offset of wavefront wid + NW/2's instruction from this one's
    int KT;
    int row0, rows;  // the tile's permuted rows (gathered operands)
  };
  uint32_t a_ld, b_ld;
  {
    int ld;
    if constexpr (OP == OP_FC1_FWD || OP == OP_FC2_DGRAD || OP == OP_FC1_WGRAD) ld = d;
    else if constexpr (OP == OP_FC2_FWD || OP == OP_FC2_WGRAD) ld = f;
    else ld = 2 * f;
    a_ld = (uint32_t)ld * 2u;
    if constexpr (OP == OP_FC1_FWD || OP == OP_FC1_DGRAD) b_ld = (uint32_t)f * 2u;
    else if constexpr (OP == OP_FC1_WGRAD) b_ld = (uint32_t)f * 4u;
    else b_ld = (uint32_t)d * 2u;
  }
  // ---- DMA lane offsets (bytes, without the stage's k offset) -----------
  // K-contig operand: instruction t (0..15) covers tile rows 16t..16t+15;
  // lane -> row 16t + lane/4, stored chunk lane%4 holds logical chunk
  // (lane%4) ^ kc_swz(row).
  // MN-contig operand: instruction t covers half t>>3, k-rows 4(t&7)..+3;
  // lane -> k-row 4(t&7) + lane/16, stored 16-byte unit lane%16, i.e. 32-byte
  // unit (lane%16)/2 holding logical unit ((lane%16)/2) ^ f(k).
  auto kc_off = [&](int t, int row_base_mn, uint32_t ld) __attribute__((always_inline)) -> uint32_t {
    const int row = 16 * t + (lane >> 2);
    const int c = (lane & 3) ^ kc_swz(row);
    return (uint32_t)(row_base_mn + row) * ld + (uint32_t)c * 16u;
  };
  auto mc_off = [&](int t, int col_base, uint32_t ld) __attribute__((always_inline)) -> uint32_t {
    const int k = 4 * (t & 7) + (lane >> 4);
    const int fk = (k & 3) | (((k >> 3) & 1) << 2);
    const int unit = ((lane & 15) >> 1) ^ fk;
    return (uint32_t)k * ld + (uint32_t)(col_base + unit * 16 + (lane & 1) * 8) * 2u;
  };
  // A DMA instruction q of this wavefront: t = wid * 2 + q, except in the
  // gathered weight gradient, where t = wid + 8 q (half q, k-rows 4 wid..+3)
  auto a_instr = [&](int q) __attribute__((always_inline)) -> int {
    if constexpr (GW) return wid + 8 * q;
    else return wid * DMA_PER_WAVE + q;
  };
  auto setup = [&](const TileInfo& ti, Opnd& o) __attribute__((always_inline)) {
    const size_t e = (size_t)ti.e;
    {
      const bf16_t* base;
      if constexpr (OP == OP_FC1_FWD || OP == OP_FC1_WGRAD) base = (const bf16_t*)args.xp;
      else if constexpr (OP == OP_FC2_FWD || OP == OP_FC2_WGRAD) base = (const bf16_t*)args.h;
      else if constexpr (OP == OP_FC2_DGRAD) base = (const bf16_t*)args.dO;
      else base = (const bf16_t*)args.dab;
      if constexpr (GATHER) o.a_src = make_rsrc(args.gx, (uint32_t)args.gT * a_ld);  // all of x
      else o.a_src = make_rsrc((const char*)base + (size_t)ti.row0 * a_ld, (uint32_t)ti.rows * a_ld);
    }
    o.row0 = ti.row0;
    o.rows = ti.rows;
    if constexpr (OP == OP_FC1_FWD || OP == OP_FC1_DGRAD) {
      o.b_src = make_rsrc((const bf16_t*)args.W1 + e * (size_t)d * f, (uint32_t)d * (uint32_t)f * 2u);
      o.b_src2 = make_rsrc((const bf16_t*)args.W3 + e * (size_t)d * f, (uint32_t)d * (uint32_t)f * 2u);
    } else if constexpr (OP == OP_FC2_FWD || OP == OP_FC2_DGRAD) {
      o.b_src = make_rsrc((const bf16_t*)args.W2 + e * (size_t)f * d, (uint32_t)f * b_ld);
      o.b_src2 = o.b_src;
    } else if constexpr (OP == OP_FC2_WGRAD) {
      o.b_src = make_rsrc((const bf16_t*)args.dO + (size_t)ti.row0 * d, (uint32_t)ti.rows * b_ld);
      o.b_src2 = o.b_src;
    } else {
      o.b_src = make_rsrc((const bf16_t*)args.dab + (size_t)ti.row0 * 2 * f, (uint32_t)ti.rows * b_ld);
      o.b_src2 = o.b_src;
    }
    const int K = TR::ragged_m ? Kfix : ti.rows;
    o.KT = uniform((K + BK - 1) / BK);
    // instruction t + 8 (NW = 8): K-contiguous rows 128 further on (the same
    // chunk swizzle, which depends on row bits 1-2 only); fc1 forward's
    // weights: the same offset in W3; fc2 forward's MN-contiguous weights:
    // the next 128 columns, as clamped for a last, partial N-tile
    o.a_dw = 0;
    o.b_dw = 0;
    if constexpr (DW == 2) {
      static_assert(TR::a_kcontig, "ragged-M A operands are K-contiguous");
      o.a_dw = 128u * a_ld;
      if constexpr (TR::b_kcontig) o.b_dw = 128u * b_ld;
      else if constexpr (OP == OP_FC2_FWD)
        o.b_dw = (uint32_t)(min(ti.n0 + 128, N - 128) - min(ti.n0, N - 128)) * 2u;
      o.a_dw = (uint32_t)uniform((int)o.a_dw);
      o.b_dw = (uint32_t)uniform((int)o.b_dw);
    }
#pragma unroll
    for (int q = 0; q < DMA_PER_WAVE; ++q) {
      const int t = wid * DMA_PER_WAVE + q;
      if constexpr (GATHER && OP == OP_FC1_FWD) {
        // row `row` of the tile is x row token_of[row0 + row]; rows past the
        // expert's end read as zero (an offset past the buffer's range)
        const int row = 16 * t + (lane >> 2);
        const int c = (lane & 3) ^ kc_swz(row);
        o.a_off[q] = row < ti.rows
                         ? (uint32_t)args.gather[ti.row0 + row] * a_ld + (uint32_t)c * 16u
                         : kPastRange;
      } else if constexpr (GW) {
        // the column part only: the k-row's token comes per stage
        const int ta = a_instr(q);
        o.a_off[q] = mc_off(ta, min(ti.m0 + (ta >> 3) * 128, Mfix - 128), 0u);
      } else if constexpr (TR::a_kcontig) o.a_off[q] = kc_off(t, 0, a_ld);
      else o.a_off[q] = mc_off(t, min(ti.m0 + (t >> 3) * 128, Mfix - 128), a_ld);
      if constexpr (TR::b_kcontig) {
        o.b_off[q] = kc_off(t, ti.n0, b_ld);
      } else if constexpr (OP == OP_FC1_FWD) {
        o.b_off[q] = mc_off(t, ti.n0 / 2, b_ld);        // both halves: the tile's f-columns
      } else {
        o.b_off[q] = mc_off(t, min(ti.n0 + (t >> 3) * 128, N - 128), b_ld);
      }
    }
  };

  // LDS byte address of the stage ring (M0 values are this plus constants)
  const uint32_t lds_base =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(size_t)LDS_PTR(lds));

  TileInfo ti, tn;
  Opnd cur, nxt;
  int slot = blockIdx.x;
  if (slot >= total) return;
  decode(slot, ti);
  setup(ti, cur);
  tn = ti;     // nxt always holds valid descriptors (a past-the-end load
  nxt = cur;   // uses them with a zero-length range)
  int phase = 0;        // ring slot of the current tile's stage 0
  bool cross = false;   // stages past the current tile's last fetch the next tile's first three
  // gathered weight gradient: token slot of the current tile's stage 0, the
  // token-id source, the slots' LDS address, and the lane offsets of the A
  // loads of the stage issued next
  int tphase = 0;
  const rsrc_t tok_src = GW ? make_rsrc(args.gather, (uint32_t)args.P * 4u) : rsrc_t{0, 0, 0, 0};
  const uint32_t tok_base = lds_base + (uint32_t)(NS * STAGE_BYTES);
  uint32_t gofs[DMA_PER_WAVE];
#pragma unroll
  for (int q = 0; q < DMA_PER_WAVE; ++q) gofs[q] = kPastRange;
  // token ids of the four k-rows of this wavefront in stage s (lanes 0..3
  // load them; the other lanes' loads land unused) into the stage's slot
  auto issue_tok = [&](int s) __attribute__((always_inline)) {
    const bool in_cur = s < cur.KT;
    const int ks = (in_cur ? s : s - cur.KT) * BK + 4 * wid;
    const int base = (in_cur ? cur.row0 : nxt.row0) + ks;
    const uint32_t idx = (uint32_t)min(max(base + lane, 0), args.P - 1);
    rsrc_t r = tok_src;
    r[2] = (in_cur || cross) ? r[2] : 0;
    dma4(uniform_rsrc(r), idx * 4u,
         tok_base + (uint32_t)((wid * TSLOTS + ((tphase + s) & (TSLOTS - 1))) * 256));
  };
  // A offsets of stage s from its token ids (landed for this wavefront): x row
  // token * d for the lane's k-row, past the range for k-rows past the tile's
  auto read_tok = [&](int s) __attribute__((always_inline)) -> int {
    return *(const __attribute__((address_space(3))) int*)(
        lds + NS * STAGE_BYTES + (wid * TSLOTS + ((tphase + s) & (TSLOTS - 1))) * 256 +
        (lane >> 4) * 4);
  };
  auto gather_offsets = [&](int s, int tok) __attribute__((always_inline)) {
    const bool in_cur = s < cur.KT;
    const int ks = (in_cur ? s : s - cur.KT) * BK + 4 * wid;
    const int lim = (in_cur ? cur.rows : nxt.rows) - ks;  // valid k-rows of the four
#pragma unroll
    for (int q = 0; q < DMA_PER_WAVE; ++q)
      gofs[q] = (lane >> 4) < lim ? (uint32_t)tok * a_ld + (in_cur ? cur.a_off[q] : nxt.a_off[q])
                                  : kPastRange;
  };
  // DMA instruction q of this wavefront (q < DMA_PER_WAVE: A operand, else B)
  // for stage s of the stream, counted from the current tile's stage 0
  // TAIL = false: the caller knows that s is a stage of the current tile.
  auto issue_one = [&](int s, auto Q, auto TAIL) __attribute__((always_inline)) {
    if constexpr (DW == 2) {
      if (wid >= NW / 2) return;
    }
    constexpr int q = decltype(Q)::value;
    const uint32_t st_base = lds_base + (uint32_t)(((uint32_t)(phase + s) % NS) * STAGE_BYTES);
    const bool in_cur = !decltype(TAIL)::value || s < cur.KT;
    const int k0 = (in_cur ? s : s - cur.KT) * BK;
    const bool live = in_cur || cross;
    if constexpr (q < DMA_PER_WAVE) {
      const int t = a_instr(q);
      rsrc_t r = pick(in_cur, cur.a_src, nxt.a_src);
      r[2] = live ? r[2] : 0;
      r = uniform_rsrc(r);
      if constexpr (GW) {
        dma16(r, gofs[q], st_base + (uint32_t)(t * 1024));  // offsets of stage s (gather_offsets)
      } else {
        const uint32_t off = in_cur ? cur.a_off[q] : nxt.a_off[q];
        const uint32_t ka = TR::a_kcontig ? (uint32_t)k0 * 2u : (uint32_t)k0 * a_ld;
        dma16(r, off + ka, st_base + (uint32_t)(t * 1024));
        if constexpr (DW == 2)
          dma16(r, off + ka + (in_cur ? cur.a_dw : nxt.a_dw),
                st_base + (uint32_t)((t + (NW / 2) * DMA_PER_WAVE) * 1024));
      }
    } else {
      const int qq = q - DMA_PER_WAVE;
      const uint32_t off = in_cur ? cur.b_off[qq] : nxt.b_off[qq];
      // instruction t of the B operand (DW = 2: t + 8 with the offset moved by b_dw)
      auto one = [&](int t, uint32_t dw) __attribute__((always_inline)) {
        const uint32_t dst = st_base + (uint32_t)(OPND_BYTES + t * 1024);
        rsrc_t r;
        uint32_t voff;
        if constexpr (OP == OP_FC1_DGRAD) {
          // K = [da | db]: the first f columns multiply W1, the rest W3
          const bool first = k0 < f;
          r = pick(in_cur, pick(first, cur.b_src, cur.b_src2), pick(first, nxt.b_src, nxt.b_src2));
          voff = off + dw + (uint32_t)(first ? k0 : k0 - f) * 2u;
        } else if constexpr (OP == OP_FC1_FWD) {
          const bool second = (t >> 3) != 0;
          r = pick(in_cur, pick(second, cur.b_src2, cur.b_src), pick(second, nxt.b_src2, nxt.b_src));
          voff = off + dw + (uint32_t)k0 * b_ld;
        } else if constexpr (TR::b_kcontig) {
          r = pick(in_cur, cur.b_src, nxt.b_src);
          voff = off + dw + (uint32_t)k0 * 2u;
        } else {
          r = pick(in_cur, cur.b_src, nxt.b_src);
          voff = off + dw + (uint32_t)k0 * b_ld;
        }
        r[2] = live ? r[2] : 0;
        dma16(uniform_rsrc(r), voff, dst);
      };
      one(wid * DMA_PER_WAVE + qq, 0u);
      if constexpr (DW == 2) one((wid + NW / 2) * DMA_PER_WAVE + qq, in_cur ? cur.b_dw : nxt.b_dw);
    }
  };

  // ---- fragment addresses (bytes inside a stage) -------------------------
  // K-contig: row = base + 16*blk + lane%16, chunk lane/16 (swizzled)
  const uint32_t kc_frag = (uint32_t)(lane & 15) * 64u + (uint32_t)((lane >> 4) ^ kc_swz(lane & 15)) * 16u;
  // MN-contig: lane group g = lane/16, s = lane%16: k-row 8g + s/4, 8-byte
  // column piece s%4; unit swizzle f = (s/4) | (g&1) << 2
  const int g = lane >> 4, sl = lane & 15;
  const uint32_t mc_row = (uint32_t)(8 * g + (sl >> 2)) * 256u + (uint32_t)(sl & 3) * 8u;
  const int mc_f = ((sl >> 2) & 3) | ((g & 1) << 2);
  auto a_frag_addr = [&](int i) __attribute__((always_inline)) -> uint32_t {   // A fragment i of this wavefront
    if constexpr (TR::a_kcontig) return (uint32_t)(wm * WM + 16 * i) * 64u + kc_frag;
    else return (uint32_t)wm * 8192u + mc_row + (uint32_t)((i ^ mc_f) * 32);
  };
  auto b_frag_addr = [&](int j) __attribute__((always_inline)) -> uint32_t {   // B fragment j of this wavefront
    if constexpr (TR::b_kcontig) {
      return OPND_BYTES + (uint32_t)(wn * WN + 16 * j) * 64u + kc_frag;
    } else if constexpr (OP == OP_FC1_FWD) {  // j < HB: W1 columns; j + HB: the same columns of W3
      return OPND_BYTES + (uint32_t)(j / HB) * 8192u + mc_row +
             (uint32_t)((((wn * HB) + (j % HB)) ^ mc_f) * 32);
    } else {
      const int col = wn * WN + 16 * j;           // tile column of the fragment
      return OPND_BYTES + (uint32_t)(col >> 7) * 8192u + mc_row +
             (uint32_t)((((col & 127) >> 4) ^ mc_f) * 32);
    }
  };
  uint32_t afa[FM], bfa[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) afa[i] = a_frag_addr(i);
#pragma unroll
  for (int j = 0; j < FN; ++j) bfa[j] = b_frag_addr(j);
  auto read_a = [&](const char* st, int i) __attribute__((always_inline)) -> bf16x8_t {
    if constexpr (TR::a_kcontig) return lds_b128(st + afa[i]);
    else return lds_tr_pair(st + afa[i]);
  };
  auto read_b = [&](const char* st, int j) __attribute__((always_inline)) -> bf16x8_t {
    if constexpr (TR::b_kcontig) return lds_b128(st + bfa[j]);
    else return lds_tr_pair(st + bfa[j]);
  };
  auto stage_ptr = [&](int s) __attribute__((always_inline)) -> const char* {
    return lds + ((uint32_t)(phase + s) % NS) * STAGE_BYTES;
  };

  // ---------------------------------------------------------------- main loop
  f32x4_t acc[FM][FN];

  // Per stage both halves walk the FM = 8 A fragments i-major against HB B
  // fragments held in registers: B fragments 0..HB-1 (b0, read during the
  // previous stage) in the first half, HB..FN-1 (b1, read at the start of
  // the first half) in the second.  The wait + barrier that releases the
  // next stage (and frees the oldest buffer for stage kt+3) sits between the
  // halves; right after it b0 is refilled with the next stage's fragments,
  // and every A fragment is replaced by the next stage's as soon as its
  // MFMAs are issued.  LDS reads return in order, so reads are issued in the
  // order their data is needed.  The refill of a freed buffer (16 one-KB DMA
  // instructions per operand, spread over the wavefronts) is issued evenly
  // over the second half of stage kt (A operand of stage kt+3) and the first
  // half of stage kt+1 (its B operand): issued in a burst they stall the
  // wavefront's instruction issue.
  bf16x8_t af[FM], b0[HB], b1[HB];
  // 16-row fragments of this wavefront that hold valid rows of the tile: the
  // MFMAs and A reads of the others can be skipped (the last M-tile of an
  // expert is often mostly empty: with about 512 +- 21 rows per expert, half
  // the experts need a third 256-row tile for a few dozen rows)
  int nfr = FM;
  // st and nst are distinct stage buffers (restrict lets the compiler keep
  // their reads apart).
  auto stage_body = [&](int kt, const char* __restrict__ st, const char* __restrict__ nst,
                        auto TAIL, auto SKIP) __attribute__((always_inline)) {
    constexpr bool skip = decltype(SKIP)::value;
    // gathered weight gradient: the ids of stage kt + 3 (landed: issued
    // before stage kt's B loads) are read first; those of stage kt + 5 are
    // loaded ahead of this stage's B loads (the wait below counts them)
    int tok = 0;
    if constexpr (GW) {
      tok = read_tok(kt + LOOK);
      issue_tok(kt + TLOOK);
    }
    // B fragments HB..FN-1 for the second half: issued first, needed last
    static_for<0, HB>([&](auto U) __attribute__((always_inline)) { b1[U.value] = read_b(st, HB + U.value); });
    static_for<0, 4>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = U.value;
      __builtin_amdgcn_sched_barrier(0);
      static_for<2 * u, 2 * u + 2>([&](auto I) __attribute__((always_inline)) {
        if (!skip || I.value < nfr) {
          static_for<0, HB>([&](auto J) __attribute__((always_inline)) {
            acc[I.value][J.value] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                b0[J.value], af[I.value], acc[I.value][J.value], 0, 0, 0);
          });
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      // second (B-operand) half of stage kt+2's refill; its buffer was freed
      // by the previous stage's barrier
      if constexpr (u % DMA_STEP == DMA_STEP - 1) issue_one(kt + LOOK - 1, IntC<DMA_PER_WAVE + u / DMA_STEP>{}, TAIL);
    });
    // stage kt+1 has landed for this wavefront; after the barrier it has for
    // all, and every wavefront is done with stage kt-1, whose buffer now
    // takes stage kt+3
    wait_vmcnt<VM_STAGE * (LOOK - 2)>();
    block_barrier();
    // the A offsets of stage kt + 3, issued in the second half
    if constexpr (GW) gather_offsets(kt + LOOK, tok);
    // next stage's B fragments 0..HB-1 first: the next first half starts with them
    static_for<0, HB>([&](auto U) __attribute__((always_inline)) { b0[U.value] = read_b(nst, U.value); });
    static_for<0, 4>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = U.value;
      __builtin_amdgcn_sched_barrier(0);
      static_for<2 * u, 2 * u + 2>([&](auto I) __attribute__((always_inline)) {
        if (!skip || I.value < nfr) {
          static_for<0, HB>([&](auto J) __attribute__((always_inline)) {
            acc[I.value][HB + J.value] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                b1[J.value], af[I.value], acc[I.value][HB + J.value], 0, 0, 0);
          });
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      if (!skip || 2 * u < nfr) af[2 * u] = read_a(nst, 2 * u);
      if (!skip || 2 * u + 1 < nfr) af[2 * u + 1] = read_a(nst, 2 * u + 1);
      // first (A-operand) half of stage kt+3's refill into the buffer stage
      // kt-1 used; one DMA instruction per step keeps the address unit from
      // stalling the issue of the MFMAs
      if constexpr (u % DMA_STEP == DMA_STEP - 1) issue_one(kt + LOOK, IntC<u / DMA_STEP>{}, TAIL);
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
    // fc2 dgrad's epilogue reads a|b from memory and would wait for the next
    // tile's loads in flight: it starts every tile with its own prologue
    cross = OP != OP_FC2_DGRAD && have_next && cur.KT >= 1 && nxt.KT >= LOOK;
    // gathered weight gradient: the next tile's first TLOOK token loads are
    // issued in this tile's last TLOOK stages
    if constexpr (GW) cross = cross && cur.KT >= TLOOK;
    if (fresh) {
      // gathered weight gradient: token ids of stages 0 .. TLOOK-1 first;
      // those of stages 0 .. LOOK-1 land before their A loads are issued
      if constexpr (GW) {
        static_for<0, TLOOK>([&](auto S) __attribute__((always_inline)) { issue_tok(S.value); });
        wait_vmcnt<TLOOK - LOOK>();
      }
      // stages 0 .. LOOK-2 and stage LOOK-1's A half in flight (its B half
      // follows in stage 0); wait for stage 0 and make it visible
      static_for<0, LOOK - 1>([&](auto S) __attribute__((always_inline)) {
        if constexpr (GW) gather_offsets(S.value, read_tok(S.value));
        static_for<0, 2 * DMA_PER_WAVE>([&](auto Q) __attribute__((always_inline)) {
          issue_one(S.value, Q, IntC<1>{});
        });
      });
      if constexpr (GW) gather_offsets(LOOK - 1, read_tok(LOOK - 1));
      static_for<0, DMA_PER_WAVE>([&](auto Q) __attribute__((always_inline)) { issue_one(LOOK - 1, Q, IntC<1>{}); });
      wait_vmcnt<LOADS_PER_STAGE * (LOOK - 2) + DMA_PER_WAVE * DW>();
      block_barrier();
    }
    // (entered from the previous tile's stream, stage 0 has landed and passed
    // that tile's last barrier)
    {
      const char* st0 = stage_ptr(0);
      static_for<0, FM>([&](auto i) __attribute__((always_inline)) { af[i.value] = read_a(st0, i.value); });
      static_for<0, HB>([&](auto j) __attribute__((always_inline)) { b0[j.value] = read_b(st0, j.value); });
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const int valid = (TR::ragged_m ? ti.rows : Mfix - ti.m0) - wm * WM;
      nfr = uniform(min(FM, max(0, (valid + 15) / 16)));
    }
    // the last LOOK stages issue the loads that may fall past the tile
    const int kt_tail = max(cur.KT - LOOK, 0);
    // fc1 forward and dgrad: a tile with rows past its end on some wavefront
    // takes a loop that skips their fragments, full tiles the branch-free one
    // (measured on the Qwen3 shape: 1-2.5 % faster; the branches in every
    // tile's loop cost 1-5 %, and the other products gain nothing)
    constexpr bool kSkipLoop = OP == OP_FC1_FWD || OP == OP_FC1_DGRAD;
    if (!kSkipLoop || nfr == FM) {
      for (int kt = 0; kt < kt_tail; ++kt) stage_body(kt, stage_ptr(kt), stage_ptr(kt + 1), IntC<0>{}, IntC<0>{});
      for (int kt = kt_tail; kt < cur.KT; ++kt) stage_body(kt, stage_ptr(kt), stage_ptr(kt + 1), IntC<1>{}, IntC<0>{});
    } else {
      for (int kt = 0; kt < kt_tail; ++kt) stage_body(kt, stage_ptr(kt), stage_ptr(kt + 1), IntC<0>{}, IntC<1>{});
      for (int kt = kt_tail; kt < cur.KT; ++kt) stage_body(kt, stage_ptr(kt), stage_ptr(kt + 1), IntC<1>{}, IntC<1>{});
    }

    // ---------------------------------------------------------------- epilogue
    // whole-line stores where they do not raise register use past the
    // budget (fc1 dgrad's would spill); measured on the Qwen3 shape: fc1 and
    // fc2 weight gradients 3-4 % faster, fc2 forward 1.6 %
    constexpr bool kLines = FN == 4 && (OP == OP_FC2_FWD || OP == OP_FC2_WGRAD || OP == OP_FC1_WGRAD);
    store_tile<OP, FM, FN, WM, WN, TR::ragged_m, RS, kLines>(args, acc, ti, TR::ragged_m ? ti.rows : Mfix,
                                                               N, wm, wn, lane, dp_red);
    if (!have_next) break;
    if (cross) {
      phase = (int)((uint32_t)(phase + cur.KT) % NS);
      tphase = (tphase + cur.KT) & (TSLOTS - 1);
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

// Compute units of the current device rounded down to a multiple of 8
// (cached per device; concurrent first calls store the same value), or -1
// when the runtime cannot say.
int persistent_blocks() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
    return -1;
  n &= ~7;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int OP, int NW>
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
  // persistent blocks: one per compute unit (the tile takes a whole CU's
  // LDS), a multiple of 8 so that every block's tiles stay on one XCD.
  // fc2 dgrad keeps one block per tile: its blocks, started in tile order as
  // compute units free up, keep the tiles that run together on an XCD
  // adjacent (shared A rows and weights in L2), where a static stride lets
  // them drift apart (measured: 19 % more HBM reads, 2.5 % slower).
  if (OP != OP_FC2_DGRAD) {
    const int ncu = persistent_blocks();
    if (ncu <= 0) return MOE_ERR_HIP;
    if (grid > ncu) grid = ncu;
  }
  // row-scaled variants (only fc1 forward and fc2 dgrad change) and the
  // gathered fc1 operand (fc1 forward and fc1 weight gradient)
  const unsigned g = (unsigned)grid;
  if constexpr (OP == OP_FC1_FWD) {
    if (a.gather && a.row_prob) gemm_bf16_kernel<OP, NW, true, true><<<g, NW * 64, 0, s>>>(a, NT, MT);
    else if (a.gather) gemm_bf16_kernel<OP, NW, false, true><<<g, NW * 64, 0, s>>>(a, NT, MT);
    else if (a.row_prob) gemm_bf16_kernel<OP, NW, true><<<g, NW * 64, 0, s>>>(a, NT, MT);
    else gemm_bf16_kernel<OP, NW, false><<<g, NW * 64, 0, s>>>(a, NT, MT);
  } else if constexpr (OP == OP_FC2_DGRAD) {
    if (a.row_prob) gemm_bf16_kernel<OP, NW, true><<<g, NW * 64, 0, s>>>(a, NT, MT);
    else gemm_bf16_kernel<OP, NW, false><<<g, NW * 64, 0, s>>>(a, NT, MT);
  } else if constexpr (OP == OP_FC1_WGRAD) {
    if (a.gather) gemm_bf16_kernel<OP, NW, false, true><<<g, NW * 64, 0, s>>>(a, NT, MT);
    else gemm_bf16_kernel<OP, NW, false><<<g, NW * 64, 0, s>>>(a, NT, MT);
  } else {
    gemm_bf16_kernel<OP, NW, false><<<g, NW * 64, 0, s>>>(a, NT, MT);
  }
  TRE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace

int gemm_persistent_blocks() { return persistent_blocks(); }

#ifndef GEMM_NW
#define GEMM_NW 8
#endif
int gemm_bf16_launch(GemmOp op, const GemmArgs& a, hipStream_t s) {
  switch (op) {
    case OP_FC1_FWD: return launch<OP_FC1_FWD, GEMM_NW>(a, s);
    case OP_FC2_FWD: return launch<OP_FC2_FWD, GEMM_NW>(a, s);
    case OP_FC2_DGRAD: return launch<OP_FC2_DGRAD, GEMM_NW>(a, s);
    case OP_FC1_DGRAD: return launch<OP_FC1_DGRAD, GEMM_NW>(a, s);
    case OP_FC2_WGRAD: return launch<OP_FC2_WGRAD, GEMM_NW>(a, s);
    case OP_FC1_WGRAD: return launch<OP_FC1_WGRAD, GEMM_NW>(a, s);
  }
  return MOE_ERR_INVALID;
}

}  // namespace tre
