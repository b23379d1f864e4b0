// W4A16 prefill GEMM: Y[M][N] = X[M][K] (bf16) * dequant(W)^T with INT4
// weights in groups of 128 along K (《推理优化与量化算子深度技术调研》 section
// 1.3; 《第 6 课：量化源码走读》 section 2: the weights are dequantized inside
// the GEMM; section 3: the asymmetric zero-point cross term is kept).
//
// The matrix cores multiply exact integers: nibbles are unpacked in registers
// to the bf16 values 128 + u (one and/or per pair, as in the decode GEMV) and
// fed to v_mfma_f32_16x16x32_bf16 against the bf16 activations, whose pairs
// (x_j, x_{j+4}) are formed once when X is staged into LDS.  Each group of
// 128 has its own fp32 accumulator; at the group's end
//     y += s * (acc_g - c * sum_x),  c = 136 (symmetric) or 128 + z,
// with sum_x from an extra MFMA against 1.0.  Rounding dequantized weights
// to bf16 before the matrix cores is avoided on purpose: it would add an
// error of the same size as the bf16 output rounding itself.
//
// Tiling: 256-thread workgroup, 128 (tokens) x 128 (channels) output tile,
// 4 waves of 64x64; one k-step = one group of 128.  X is staged as bf16
// (32 KiB), the codes as packed nibbles (8 KiB) and the tile's (s, c) pairs
// (1 KiB), through registers so the next group's loads overlap the math.

#include "qg_gemm_common.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int XROW = BK * 2;       // bytes of one staged X row (bf16)
constexpr int WROW = BK / 2;       // bytes of one staged code row

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 pair_activations(const u32x4& d) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return r;
}

// (w >> 4j) & 0x000F000F combined with the bf16 exponent of 128 gives the
// pair (128 + u_j, 128 + u_{j+4}); for symmetric (two's-complement) codes
// flipping bit 3 of each nibble first gives u = q + 8.  Both are one xor
// with a constant after the mask: xor 0x43004300 (asymmetric) or
// 0x43084308 (symmetric; bit 3 of the masked nibble is flipped too).
template <bool ASYM>
__device__ __forceinline__ u32x4 unpack_word(uint32_t w) {
  constexpr uint32_t C = ASYM ? 0x43004300u : 0x43084308u;
  u32x4 r;
  r[0] = (w & 0x000F000Fu) ^ C;
  r[1] = ((w >> 4) & 0x000F000Fu) ^ C;
  r[2] = ((w >> 8) & 0x000F000Fu) ^ C;
  r[3] = ((w >> 12) & 0x000F000Fu) ^ C;
  return r;
}

__device__ __forceinline__ int swz_w(int row, int c) {
  return row * WROW + ((c ^ ((row >> 1) & 3)) << 4);
}

template <bool ASYM>
__global__ __launch_bounds__(256) void gemm_w4a16_kernel(const uint16_t* __restrict__ X, int M,
                                                         const uint32_t* __restrict__ Wc,
                                                         const uint16_t* __restrict__ S,
                                                         const uint16_t* __restrict__ Z, int N,
                                                         int K, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t sX[BM * XROW];
  __shared__ __attribute__((aligned(16))) uint8_t sW[BN * WROW];
  __shared__ __attribute__((aligned(16))) float sSC[BN * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int li = lane & 15, lg = lane >> 4;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int G = K / BK;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rwc = make_rsrc(Wc, (int64_t)N * K / 2);

  // staging map: X 8 chunks of 16 B per thread (row q>>4, chunk q&15), codes 2
  uint32_t vx[8];
  int ox[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + 256 * i, row = q >> 4, c = q & 15;
    ox[i] = row * XROW + ((c ^ (row & 7)) << 4);
    vx[i] = (m0 + row < M) ? (uint32_t)(m0 + row) * (uint32_t)(K * 2) + c * 16 : kOutOfRange;
  }
  uint32_t vw[2];
  int ow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i, row = q >> 2, c = q & 3;
    ow[i] = swz_w(row, c);
    vw[i] = (n0 + row < N) ? (uint32_t)(n0 + row) * (uint32_t)(K / 2) + c * 16 : kOutOfRange;
  }
  const int srow = tid & 127;
  const bool s_ok = tid < 128 && n0 + srow < N;

  u32x4 rxr[8], rwr[2];
  float s_reg = 0.f, c_reg = 0.f;
  auto gload = [&](int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) rxr[i] = buf_load16(rx, vx[i], g * XROW);
#pragma unroll
    for (int i = 0; i < 2; ++i) rwr[i] = buf_load16(rwc, vw[i], g * WROW);
    if (s_ok) {
      const int64_t idx = (int64_t)(n0 + srow) * G + g;
      s_reg = f16_bits_to_f32(S[idx]);
      c_reg = ASYM ? 128.f + f16_bits_to_f32(Z[idx]) : 136.f;
    } else {
      s_reg = 0.f;
      c_reg = 0.f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(sX + ox[i]) = pair_activations(rxr[i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(sW + ow[i]) = rwr[i];
    if (tid < 128) *reinterpret_cast<float2*>(sSC + 2 * srow) = make_float2(s_reg, c_reg);
  };

  f32x4 yacc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) yacc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore();
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    if (g + 1 < G) gload(g + 1);

    // codes of this wave's 4 channel tiles: 16 B = words 4lg..4lg+3 of the group
    u32x4 wf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = wn * 64 + u * 16 + li;
      wf[u] = *reinterpret_cast<const u32x4*>(sW + swz_w(r, lg));
    }
    f32x4 gacc[4][4], sacc[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      bf16x8 bx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = wm * 64 + t * 16 + li;
        const int c = 4 * lg + kc;
        bx[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(sX + r * XROW + ((c ^ (r & 7)) << 4)));
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), bx[t],
                                                          kc ? sacc[t] : zero4, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 a = as_bf16x8(unpack_word<ASYM>(wf[u][kc]));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          gacc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bx[t], kc ? gacc[u][t] : zero4,
                                                               0, 0, 0);
      }
    }
    // flush: rows n = 4lg + r of channel tile u
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4* p = reinterpret_cast<const float4*>(sSC + 2 * (wn * 64 + u * 16 + 4 * lg));
      const float4 p01 = p[0], p23 = p[1];
      const float sv[4] = {p01.x, p01.z, p23.x, p23.z};
      const float cv[4] = {p01.y, p01.w, p23.y, p23.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          yacc[u][t][r] =
              __builtin_fmaf(sv[r], __builtin_fmaf(-cv[r], sacc[t][0], gacc[u][t][r]), yacc[u][t][r]);
    }
    __syncthreads();
    if (g + 1 < G) {
      lstore();
      __syncthreads();
    }
  }

#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + wm * 64 + t * 16 + li;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + wn * 64 + u * 16 + 4 * lg;
      store_out4(Y, M, N, m, n, yacc[u][t][0], yacc[u][t][1], yacc[u][t][2], yacc[u][t][3]);
    }
  }
}

}  // namespace

hipError_t launch_gemm_w4a16(bool asym, const void* x, int64_t M, const void* wcodes,
                             const void* wscales, const void* wzeros, int64_t N, int64_t K,
                             void* y, hipStream_t stream) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  if (asym)
    hipLaunchKernelGGL((gemm_w4a16_kernel<true>), dim3(tiles), dim3(256), 0, stream,
                       (const uint16_t*)x, (int)M, (const uint32_t*)wcodes,
                       (const uint16_t*)wscales, (const uint16_t*)wzeros, (int)N, (int)K,
                       (uint16_t*)y);
  else
    hipLaunchKernelGGL((gemm_w4a16_kernel<false>), dim3(tiles), dim3(256), 0, stream,
                       (const uint16_t*)x, (int)M, (const uint32_t*)wcodes,
                       (const uint16_t*)wscales, (const uint16_t*)wzeros, (int)N, (int)K,
                       (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace qg
