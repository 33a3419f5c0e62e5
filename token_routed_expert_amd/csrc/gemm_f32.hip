// Grouped expert GEMMs in fp32 (every tensor fp32): the same six products as
// the bf16 MFMA kernels (see gemm_bf16.hip for the table), computed with fp32
// FMAs on the vector ALUs.  This path serves the all-fp32 layer configuration,
// whose shapes are small; it shares the device-side tile schedule.
//
// Block tile 64 x 64 x 16, 256 threads; thread (ty, tx) owns the 4 x 4 outputs
// (ty + 16 i, tx + 16 j).  Operands are loaded element-wise with bounds checks
// (any d, f), staged K-major in LDS.  FC1_FWD writes [a|b]; the SwiGLU product
// h = silu(a) * b is a separate element-wise kernel.
#include "common.h"
#include "internal.h"
#include "schedule.h"

namespace tre {

namespace {

constexpr int BM = 64, BN = 64, BKF = 16;

template <int OP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs args, int NT, int MT) {
  __shared__ float As[BKF][BM + 1];
  __shared__ float Bs[BKF][BN + 1];
  __shared__ int scratch[8];  // >= 4 wavefronts + 4
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int d = args.d, f = args.f;
  constexpr bool ragged = OP <= OP_FC1_DGRAD;

  TileInfo ti;
  int K, M, N;
  if constexpr (ragged) {
    if (!decode_ragged_m<BM>(args.offsets, args.E, NT, scratch, ti)) return;
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
  const float* xp = (const float*)args.xp;
  const float* h = (const float*)args.h;
  const float* dO = (const float*)args.dO;
  const float* dab = (const float*)args.dab;
  const float* W1 = (const float*)args.W1 + e * (size_t)d * f;
  const float* W3 = (const float*)args.W3 + e * (size_t)d * f;
  const float* W2 = (const float*)args.W2 + e * (size_t)f * d;

  // A[m][k] of the tile (m, k local to the tile's origin; 0 outside)
  auto a_at = [&](int m, int k) -> float {
    if (k >= K) return 0.f;
    if constexpr (ragged) {
      if (m >= M) return 0.f;
      const size_t r = (size_t)(ti.row0 + m);
      if constexpr (OP == OP_FC1_FWD) {
        if (args.gather) return ((const float*)args.gx)[(size_t)args.gather[r] * d + k];
        return xp[r * d + k];
      }
      if constexpr (OP == OP_FC2_FWD) return h[r * f + k];
      if constexpr (OP == OP_FC2_DGRAD) return dO[r * d + k];
      return dab[r * 2 * f + k];
    } else {
      const int mm = ti.m0 + m;
      if (mm >= M) return 0.f;
      const size_t r = (size_t)(ti.row0 + k);
      if constexpr (OP == OP_FC2_WGRAD) return h[r * f + mm];
      if (args.gather) return ((const float*)args.gx)[(size_t)args.gather[r] * d + mm];
      return xp[r * d + mm];
    }
  };
  auto b_at = [&](int k, int n) -> float {
    const int nn = ti.n0 + n;
    if (k >= K || nn >= N) return 0.f;
    if constexpr (OP == OP_FC1_FWD) return nn < f ? W1[(size_t)k * f + nn] : W3[(size_t)k * f + nn - f];
    if constexpr (OP == OP_FC2_FWD) return W2[(size_t)k * d + nn];
    if constexpr (OP == OP_FC2_DGRAD) return W2[(size_t)nn * d + k];
    if constexpr (OP == OP_FC1_DGRAD) return k < f ? W1[(size_t)nn * f + k] : W3[(size_t)nn * f + k - f];
    if constexpr (OP == OP_FC2_WGRAD) return dO[(size_t)(ti.row0 + k) * d + nn];
    return dab[(size_t)(ti.row0 + k) * 2 * f + nn];
  };

  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BKF) {
    for (int i = tid; i < BKF * BM; i += 256) {
      const int kk = i / BM, mm = i % BM;
      As[kk][mm] = a_at(mm, k0 + kk);
    }
    for (int i = tid; i < BKF * BN; i += 256) {
      const int kk = i / BN, nn = i % BN;
      Bs[kk][nn] = b_at(k0 + kk, nn);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty + 16 * i;
    if (ragged ? m >= M : ti.m0 + m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = ti.n0 + tx + 16 * j;
      if (n >= N) continue;
      const float c = acc[i][j];
      if constexpr (OP == OP_FC1_FWD) {
        ((float*)args.ab_out)[(size_t)(ti.row0 + m) * 2 * f + n] = c;
      } else if constexpr (OP == OP_FC2_FWD) {
        ((float*)args.o_out)[(size_t)(ti.row0 + m) * d + n] = c;
      } else if constexpr (OP == OP_FC1_DGRAD) {
        ((float*)args.dXp_out)[(size_t)(ti.row0 + m) * d + n] = c;
      } else if constexpr (OP == OP_FC2_DGRAD) {
        const size_t r = (size_t)(ti.row0 + m);
        const float a = ((const float*)args.ab)[r * 2 * f + n];
        const float b = ((const float*)args.ab)[r * 2 * f + f + n];
        const float s = sigmoid_f32(a);
        ((float*)args.dab_out)[r * 2 * f + n] = c * b * s * (1.0f + a * (1.0f - s));
        ((float*)args.dab_out)[r * 2 * f + f + n] = c * a * s;
      } else if constexpr (OP == OP_FC2_WGRAD) {
        ((float*)args.dW2)[e * (size_t)f * d + (size_t)(ti.m0 + m) * d + n] = c;
      } else {
        float* base = (float*)(n < f ? args.dW1 : args.dW3);
        base[e * (size_t)d * f + (size_t)(ti.m0 + m) * f + (n < f ? n : n - f)] = c;
      }
    }
  }
}

__global__ __launch_bounds__(256) void swiglu_f32_kernel(const float* __restrict__ ab, int64_t P,
                                                         int f, float* __restrict__ h) {
  const int64_t n = P * f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / f, c = i % f;
    const float a = ab[r * 2 * f + c], b = ab[r * 2 * f + f + c];
    h[i] = silu_f32(a) * b;
  }
}

template <int OP>
int launch(const GemmArgs& a, hipStream_t s) {
  int NT, MT = 0;
  int64_t grid;
  if (OP <= OP_FC1_DGRAD) {
    const int N = (OP == OP_FC1_FWD) ? 2 * a.f : (OP == OP_FC2_DGRAD ? a.f : a.d);
    NT = (N + BN - 1) / BN;
    grid = ((int64_t)a.P / BM + a.E) * NT;
  } else {
    const int M = (OP == OP_FC2_WGRAD) ? a.f : a.d;
    const int N = (OP == OP_FC2_WGRAD) ? a.d : 2 * a.f;
    MT = (M + BM - 1) / BM;
    NT = (N + BN - 1) / BN;
    grid = (int64_t)a.E * MT * NT;
  }
  if (grid <= 0) return MOE_OK;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  gemm_f32_kernel<OP><<<(unsigned)grid, 256, 0, s>>>(a, NT, MT);
  TRE_LAUNCH_CHECK();
  if (OP == OP_FC1_FWD) {
    const int64_t n = (int64_t)a.P * a.f;
    const int64_t blocks = n / 256 + 1 < 65536 ? n / 256 + 1 : 65536;
    swiglu_f32_kernel<<<(unsigned)blocks, 256, 0, s>>>((const float*)a.ab_out, a.P, a.f,
                                                       (float*)a.h_out);
    TRE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace

int gemm_f32_launch(GemmOp op, const GemmArgs& a, hipStream_t s) {
  switch (op) {
    case OP_FC1_FWD: return launch<OP_FC1_FWD>(a, s);
    case OP_FC2_FWD: return launch<OP_FC2_FWD>(a, s);
    case OP_FC2_DGRAD: return launch<OP_FC2_DGRAD>(a, s);
    case OP_FC1_DGRAD: return launch<OP_FC1_DGRAD>(a, s);
    case OP_FC2_WGRAD: return launch<OP_FC2_WGRAD>(a, s);
    case OP_FC1_WGRAD: return launch<OP_FC1_WGRAD>(a, s);
  }
  return MOE_ERR_INVALID;
}

}  // namespace tre
