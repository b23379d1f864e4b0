// FP8 E4M3 W8A8 GEMM and MXFP4 block-scaled GEMM on the gfx950 scaled
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// FP8 (《第 6 课：量化源码走读》 section 2 and figure 6-2): the matrix cores
// multiply the E4M3 codes exactly and accumulate in fp32; the epilogue
// rescales by s_x[m] * s_w[n] (per-token activation scale, per-channel weight
// scale) and rounds once to bf16.  The MFMA's own block scales are set to
// 2^0 (E8M0 byte 127).
//
// MXFP4 (《大模型量化推理引擎全景大复盘》 section 2 eq. 3; 《第 6 课：量化源码走读》
// section 2): each lane of the MFMA holds 32 E2M1 codes of one row that form
// exactly one 32-element block, and passes that block's E8M0 byte as its
// scale, so 2^(ea + eb) is applied inside the matrix core and the epilogue
// only rounds.
//
// Tiling: a 256-thread workgroup owns a 128x128 output tile, its 4 waves a
// 64x64 quarter each (4x4 MFMA tiles).  Each k-step stages 128 bytes per row
// of both operands (128 FP8 codes or 256 FP4 codes) into LDS through
// registers: the next k-step's global loads are issued before the current
// step's matrix math.

#include "qg_gemm_common.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int BM = 128, BN = 128, BKB = 128;   // tile rows and bytes per row per k-step

template <bool MX>
__global__ __launch_bounds__(256) void gemm_f8f4_kernel(const uint8_t* __restrict__ A,
                                                        const void* __restrict__ a_aux, int M,
                                                        const uint8_t* __restrict__ W,
                                                        const void* __restrict__ w_aux, int N,
                                                        int K, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * BKB];
  __shared__ __attribute__((aligned(16))) uint8_t sW[BN * BKB];
  __shared__ __attribute__((aligned(16))) uint8_t sAs[MX ? BM * 8 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sWs[MX ? BN * 8 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int li = lane & 15, lg = lane >> 4;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbytes = MX ? K / 2 : K;           // bytes per operand row
  const int nk = (kbytes + BKB - 1) / BKB;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (int64_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (int64_t)N * kbytes);

  // staging map: 4 chunks of A and 4 of W per thread, chunk q = tid + 256 i
  uint32_t va[4], vw[4];
  int lds_off[4], ccol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, row = q >> 3, c = q & 7;
    ccol[i] = c * 16;
    lds_off[i] = swz(row, c, BKB);
    va[i] = (m0 + row < M) ? (uint32_t)(m0 + row) * kbytes + c * 16 : kOutOfRange;
    vw[i] = (n0 + row < N) ? (uint32_t)(n0 + row) * kbytes + c * 16 : kOutOfRange;
  }
  // MX scales: threads 0..127 stage A's 8 block exponents of row tid, 128..255 W's
  const int kblocks = K / 32;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(a_aux, MX ? (int64_t)M * kblocks : 0);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(w_aux, MX ? (int64_t)N * kblocks : 0);
  const int srow = tid & 127;
  const bool s_is_a = tid < 128;
  const int s_base_row = s_is_a ? m0 + srow : n0 + srow;
  const bool s_row_ok = s_base_row < (s_is_a ? M : N);

  u32x4 ra_reg[4], rw_reg[4];
  uint32_t sc_lo = 0, sc_hi = 0;

  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool kin = kb * BKB + ccol[i] < kbytes;
      ra_reg[i] = buf_load16(ra, kin ? va[i] : kOutOfRange, kin ? kb * BKB : 0);
      rw_reg[i] = buf_load16(rw, kin ? vw[i] : kOutOfRange, kin ? kb * BKB : 0);
    }
    if constexpr (MX) {
      sc_lo = sc_hi = 0;
      const __amdgpu_buffer_rsrc_t rs = s_is_a ? rsa : rsw;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int blk = kb * 8 + j;
        const bool ok = s_row_ok && blk < kblocks;
        const uint32_t off = ok ? (uint32_t)s_base_row * kblocks + blk : kOutOfRange;
        const uint32_t b = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
        if (j < 4) sc_lo |= b << (8 * j); else sc_hi |= b << (8 * (j - 4));
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(sA + lds_off[i]) = ra_reg[i];
      *reinterpret_cast<u32x4*>(sW + lds_off[i]) = rw_reg[i];
    }
    if constexpr (MX) {
      uint8_t* dst = (s_is_a ? sAs : sWs) + srow * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(sc_lo, sc_hi);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore();
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    if (kb + 1 < nk) gload(kb + 1);
    if constexpr (!MX) {
      i32x8 af[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = wm * 64 + t * 16 + li;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + swz(r, 2 * lg, BKB));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + swz(r, 2 * lg + 1, BKB));
        af[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = wn * 64 + u * 16 + li;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sW + swz(r, 2 * lg, BKB));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sW + swz(r, 2 * lg + 1, BKB));
        const i32x8 wf = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[u][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, af[t], acc[u][t], 0, 0,
                                                                       0, 127, 0, 127);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        i32x8 af[4];
        int as[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = wm * 64 + t * 16 + li;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sA + swz(r, 4 * h + lg, BKB));
          af[t] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
          as[t] = sAs[r * 8 + 4 * h + lg];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = wn * 64 + u * 16 + li;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sW + swz(r, 4 * h + lg, BKB));
          const i32x8 wf = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
          const int ws = sWs[r * 8 + 4 * h + lg];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[u][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, af[t], acc[u][t], 4,
                                                                         4, 0, ws, 0, as[t]);
        }
      }
    }
    __syncthreads();
    if (kb + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

  // epilogue: lane holds D[n = 4*lg + r][m = li] of each 16x16 tile
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + wm * 64 + t * 16 + li;
    float sxm = 1.f;
    if constexpr (!MX) sxm = (m < M) ? reinterpret_cast<const float*>(a_aux)[m] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + wn * 64 + u * 16 + 4 * lg;
      float s[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (!MX) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[r] = (n + r < N) ? reinterpret_cast<const float*>(w_aux)[n + r] * sxm : 0.f;
      }
      store_out4(Y, M, N, m, n, acc[u][t][0] * s[0], acc[u][t][1] * s[1], acc[u][t][2] * s[2],
                 acc[u][t][3] * s[3]);
    }
  }
}

template <bool MX>
hipError_t launch(const void* a, const void* a_aux, int64_t M, const void* w, const void* w_aux,
                  int64_t N, int64_t K, void* y, hipStream_t stream) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_f8f4_kernel<MX>), dim3(tiles), dim3(256), 0, stream,
                     (const uint8_t*)a, a_aux, (int)M, (const uint8_t*)w, w_aux, (int)N, (int)K,
                     (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const void* a, const void* a_scales, int64_t M, const void* w,
                           const void* w_scales, int64_t N, int64_t K, void* y,
                           hipStream_t stream) {
  return launch<false>(a, a_scales, M, w, w_scales, N, K, y, stream);
}

hipError_t launch_mx_gemm(const void* a_codes, const void* a_e8m0, int64_t M,
                          const void* b_codes, const void* b_e8m0, int64_t N, int64_t K, void* y,
                          hipStream_t stream) {
  return launch<true>(a_codes, a_e8m0, M, b_codes, b_e8m0, N, K, y, stream);
}

}  // namespace qg
