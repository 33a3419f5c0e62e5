// Matrix-core probe: the dense MFMA rate and the shader clock this GPU
// sustains under a load of MFMAs alone (no memory traffic, no LDS), the
// ceiling against which the grouped GEMMs' rates are read: the published
// peaks assume the 2.4 GHz peak clock, and the chip clocks lower under a
// sustained matrix-core load.
#include "common.h"
#include "internal.h"

namespace tre {
namespace {

constexpr int CHAINS = 8;             // independent accumulators per wavefront
constexpr int BLOCKS_PER_CU = 8;      // 32 wavefronts per CU, 8 per SIMD
constexpr int THREADS = 256;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Every wavefront runs `iters` rounds of CHAINS independent MFMAs on operands
// held in registers.  Wavefront 0 of block 0 records the shader-clock and
// wall-clock ticks its loop took (ticks[0], ticks[1]).  The accumulators are
// folded into one value that is stored only if it equals a sentinel, which
// keeps the MFMAs from being removed without a store in practice.
template <bool FP8>
__global__ __launch_bounds__(THREADS) void mfma_probe_kernel(int64_t iters,
                                                            unsigned long long* ticks,
                                                            float* sink) {
  const int lane = threadIdx.x & 63;
  f32x4_t acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  if constexpr (!FP8) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (float)(lane + i));
      b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
  } else {
    i32x8_t a, b;  // e4m3 codes (0x38 = 1.0) with lane-dependent low bits
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 ^ ((lane + i) & 7);
      b[i] = 0x30303030 ^ ((lane * 3 + i) & 7);
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1234567.0f) sink[0] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ticks[0] = c1 - c0;
    ticks[1] = w1 - w0;
  }
}

}  // namespace
}  // namespace tre

extern "C" int moe_probe_mfma(int dtype, int64_t iters, unsigned long long* ticks, float* sink,
                              int64_t* flops, int64_t* wall_khz, void* stream) {
  using namespace tre;
  if (!ticks || !sink || !flops || !wall_khz) return MOE_ERR_INVALID;
  if (iters < 1 || iters > ((int64_t)1 << 24)) return MOE_ERR_INVALID;
  if (dtype != MOE_BF16 && dtype != MOE_E4M3) return MOE_ERR_UNSUPPORTED;
  int dev = 0, ncu = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || ncu < 1)
    return MOE_ERR_HIP;
  const int grid = ncu * BLOCKS_PER_CU;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MOE_BF16) mfma_probe_kernel<false><<<grid, THREADS, 0, s>>>(iters, ticks, sink);
  else mfma_probe_kernel<true><<<grid, THREADS, 0, s>>>(iters, ticks, sink);
  TRE_LAUNCH_CHECK();
  const int64_t per_mfma = dtype == MOE_BF16 ? 16LL * 16 * 32 * 2 : 16LL * 16 * 128 * 2;
  *flops = (int64_t)grid * (THREADS / 64) * iters * CHAINS * per_mfma;
  *wall_khz = khz;
  return MOE_OK;
}
