// INT8 W8A8 GEMM with symmetric or asymmetric per-row operands on the i8
// matrix cores (v_mfma_i32_16x16x64_i8), exact int32 accumulation.
//
// 《推理优化与量化算子深度技术调研》 section 1.2 (symmetric [-127,127] and
// asymmetric [0,255] codes, dequantization fused into the GEMM) and
// 《第 6 课：量化源码走读》 section 3 (the zero-point cross terms must be kept):
//   Y = s_a s_w * sum_k (qa - za)(qw - zw)
//     = s_a s_w * (sum qa qw - zw sum qa - za sum qw + K za zw).
// Asymmetric uint8 codes are moved to signed int8 by flipping bit 7 while
// staging (q - 128), which shifts the zero point to z - 128; the row sums of
// the codes come from extra MFMAs against an all-ones operand.  The integer
// combination is formed in fp64 (exact for the integer terms) and scaled once.
//
// Exactness of the int32 sums: one 128-element k-block adds at most
// 128 * 128^2 = 2^21 in magnitude to a product sum and 2^14 to a row sum, so
// 512 blocks (K = 65536) stay below 2^30.  Longer K (LONGK) folds the int32
// sums into fp64 accumulators every 512 blocks and restarts them at zero;
// fp64 holds every such integer sum exactly (|sum| < 2^53 for K < 2^39).

#include "qg_gemm_common.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int BM = 128, BN = 128, BKB = 128;
constexpr int kFoldBlocks = 512;           // k-blocks per exact int32 run

template <bool AASYM, bool WASYM, bool LONGK>
__global__ __launch_bounds__(256) void gemm_i8_kernel(const uint8_t* __restrict__ A,
                                                      const float* __restrict__ sa,
                                                      const float* __restrict__ za, int M,
                                                      const uint8_t* __restrict__ W,
                                                      const float* __restrict__ sw,
                                                      const float* __restrict__ zw, int N, int K,
                                                      uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * BKB];
  __shared__ __attribute__((aligned(16))) uint8_t sW[BN * BKB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int li = lane & 15, lg = lane >> 4;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (K + BKB - 1) / BKB;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (int64_t)M * K);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (int64_t)N * K);

  uint32_t va[4], vw[4];
  int lds_off[4], ccol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, row = q >> 3, c = q & 7;
    ccol[i] = c * 16;
    lds_off[i] = swz(row, c, BKB);
    va[i] = (m0 + row < M) ? (uint32_t)(m0 + row) * K + c * 16 : kOutOfRange;
    vw[i] = (n0 + row < N) ? (uint32_t)(n0 + row) * K + c * 16 : kOutOfRange;
  }
  // bytes beyond K or beyond the matrix read as 0, which after the bit-7
  // flip of an asymmetric operand would be -128: flip only loaded bytes
  u32x4 ra_reg[4], rw_reg[4];
  bool ka[4];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[i] = kb * BKB + ccol[i] < K;
      ra_reg[i] = buf_load16(ra, ka[i] ? va[i] : kOutOfRange, ka[i] ? kb * BKB : 0);
      rw_reg[i] = buf_load16(rw, ka[i] ? vw[i] : kOutOfRange, ka[i] ? kb * BKB : 0);
    }
  };
  auto lstore = [&]() {
    const u32x4 flip = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 a = ra_reg[i], w = rw_reg[i];
      if (AASYM) a = (ka[i] && va[i] != kOutOfRange) ? (a ^ flip) : zero;
      if (WASYM) w = (ka[i] && vw[i] != kOutOfRange) ? (w ^ flip) : zero;
      *reinterpret_cast<u32x4*>(sA + lds_off[i]) = a;
      *reinterpret_cast<u32x4*>(sW + lds_off[i]) = w;
    }
  };

  i32x4 acc[4][4], rsum_a[4], rsum_w[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    rsum_a[a] = i32x4{0, 0, 0, 0};
    rsum_w[a] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = i32x4{0, 0, 0, 0};
  }
  const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  // fp64 totals of the folded int32 runs (LONGK only)
  double dacc[4][4][4], dsum_a[4], dsum_w[4][4];
  if constexpr (LONGK) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      dsum_a[a] = 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r) dsum_w[a][r] = 0.0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) dacc[a][b][r] = 0.0;
    }
  }
  auto fold = [&]() {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      dsum_a[a] += (double)rsum_a[a][0];
      rsum_a[a] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) dsum_w[a][r] += (double)rsum_w[a][r];
      rsum_w[a] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dacc[a][b][r] += (double)acc[a][b][r];
        acc[a][b] = i32x4{0, 0, 0, 0};
      }
    }
  };

  gload(0);
  lstore();
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    if (kb + 1 < nk) gload(kb + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 af[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = wm * 64 + t * 16 + li;
        af[t] = __builtin_bit_cast(i32x4, *reinterpret_cast<const u32x4*>(sA + swz(r, 4 * h + lg, BKB)));
        if (WASYM) rsum_a[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, af[t], rsum_a[t], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = wn * 64 + u * 16 + li;
        const i32x4 wf =
            __builtin_bit_cast(i32x4, *reinterpret_cast<const u32x4*>(sW + swz(r, 4 * h + lg, BKB)));
        if (AASYM) rsum_w[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf, ones, rsum_w[u], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[u][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf, af[t], acc[u][t], 0, 0, 0);
      }
    }
    __syncthreads();
    if constexpr (LONGK) {
      if (kb % kFoldBlocks == kFoldBlocks - 1 || kb == nk - 1) fold();
    }
    if (kb + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + wm * 64 + t * 16 + li;
    const bool mok = m < M;
    const double sam = mok ? (double)sa[m] : 0.0;
    const double zam = (AASYM && mok) ? (double)za[m] - 128.0 : 0.0;
    // sum_k qa[m][k] (all rows of the MFMA result are equal)
    const double sum_a = LONGK ? dsum_a[t] : (double)rsum_a[t][0];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + wn * 64 + u * 16 + 4 * lg;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool nok = n + r < N;
        const double swn = nok ? (double)sw[n + r] : 0.0;
        const double zwn = (WASYM && nok) ? (double)zw[n + r] - 128.0 : 0.0;
        const double sum_w = LONGK ? dsum_w[u][r] : (double)rsum_w[u][r];   // sum_k qw[n+r][k]
        const double dot = LONGK ? dacc[u][t][r] : (double)acc[u][t][r];
        const double val = dot - zwn * sum_a - zam * sum_w + (double)K * zam * zwn;
        v[r] = (float)(val * sam * swn);
      }
      store_out4(Y, M, N, m, n, v[0], v[1], v[2], v[3]);
    }
  }
}

template <bool AA, bool WA>
void launch_t(const void* a, const void* sa, const void* za, int64_t M, const void* w,
              const void* sw, const void* zw, int64_t N, int64_t K, void* y, hipStream_t s) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  if (K > (int64_t)kFoldBlocks * BKB)
    hipLaunchKernelGGL((gemm_i8_kernel<AA, WA, true>), dim3(tiles), dim3(256), 0, s,
                       (const uint8_t*)a, (const float*)sa, (const float*)za, (int)M,
                       (const uint8_t*)w, (const float*)sw, (const float*)zw, (int)N, (int)K,
                       (uint16_t*)y);
  else
    hipLaunchKernelGGL((gemm_i8_kernel<AA, WA, false>), dim3(tiles), dim3(256), 0, s,
                       (const uint8_t*)a, (const float*)sa, (const float*)za, (int)M,
                       (const uint8_t*)w, (const float*)sw, (const float*)zw, (int)N, (int)K,
                       (uint16_t*)y);
}

}  // namespace

QG_DEBUG_TU_SETTER(debug_set_int8)

hipError_t launch_gemm_int8(bool a_asym, bool w_asym, const void* a, const void* a_scales,
                            const void* a_zeros, int64_t M, const void* w, const void* w_scales,
                            const void* w_zeros, int64_t N, int64_t K, void* y,
                            hipStream_t stream) {
  if (a_asym && w_asym)
    launch_t<true, true>(a, a_scales, a_zeros, M, w, w_scales, w_zeros, N, K, y, stream);
  else if (a_asym)
    launch_t<true, false>(a, a_scales, a_zeros, M, w, w_scales, w_zeros, N, K, y, stream);
  else if (w_asym)
    launch_t<false, true>(a, a_scales, a_zeros, M, w, w_scales, w_zeros, N, K, y, stream);
  else
    launch_t<false, false>(a, a_scales, a_zeros, M, w, w_scales, w_zeros, N, K, y, stream);
  return hipGetLastError();
}

}  // namespace qg
