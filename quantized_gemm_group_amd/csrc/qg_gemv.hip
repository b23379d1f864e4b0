// W4A16 decode GEMV: y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] (q[n][k] - z[n][g])
// for 1 <= M <= 16, INT4 weights in groups of 128 along K.
//
// The small-batch W4A16 product is HBM bound (《推理优化与量化算子深度技术调研》
// section 1.3; 《第 1 章：推理加速全景》 roofline: ~1 FLOP per byte), with the
// dequantization done inside the kernel (《第 6 课：量化源码走读》 section 2) and
// the asymmetric zero-point cross term kept (same lesson, section 3).
//
// Design for gfx950 (64-wide waves, bf16 MFMA):
//  * Each workgroup owns a tile of 16*RT output channels and splits K among
//    its KS waves; a wave walks its groups of 128 with 128-bit loads: lane l
//    reads 16 bytes (32 nibbles) of row l%16 at byte offset 16*(l/16) of the
//    group, so one load instruction covers 16 rows x 64 contiguous bytes and
//    the next group completes each 128-byte line.
//  * Nibbles are unpacked in registers with one and/or per pair:
//    (w >> 4j) & 0x000F000F | 0x43004300 is the bf16 pair (128+u_j, 128+u_{j+4}),
//    exact integers, so the matrix cores multiply exact codes and the product
//    needs no rounding of dequantized weights.  The activations are loaded
//    with the same pairing (x_j, x_{j+4}) by a byte permute.
//  * v_mfma_f32_16x16x32_bf16 accumulates, per group, A = codes (rows n) times
//    B = x^T (columns m, zero beyond M), and a second MFMA with A = 1.0 gives
//    the group sums of x.  The fp32 flush per group is
//        y += s * (acc - c * sum_x),  c = 128 + z (asymmetric) or 136
//    (symmetric codes are stored two's complement; xor 0x8 maps q to q + 8).
//  * Group scales and offsets (s, c) of the tile are staged once in LDS as
//    fp32 pairs; at the end the KS partial tiles are summed through LDS and
//    rounded once to bf16 (RNE).

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kGroup = 128;

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Unpack one int32 of 8 nibbles into 4 bf16 pairs (128+u_j, 128+u_{j+4}).
__device__ __forceinline__ u32x4 unpack_word(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

// 8 bf16 activations x0..x7 (dwords d0..d3) -> pairs (x_j, x_{j+4}).
__device__ __forceinline__ u32x4 pair_activations(const u32x4& d) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return r;
}

// Loads of one group: RT x 16 bytes of codes and 4 x 16 bytes of activations.
template <int RT>
__device__ __forceinline__ void load_group(__amdgpu_buffer_rsrc_t wres, __amdgpu_buffer_rsrc_t xres,
                                           const uint32_t (&woff)[RT], uint32_t xoff, int g,
                                           u32x4 (&a)[RT], u32x4 (&b)[4]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    a[rt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rt], g * 64, 0));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, xoff, g * 256 + i * 16, 0));
}

// The math of one group for RT row tiles: MFMA over the 128 codes of each
// row tile, the group sums of x by an MFMA with A = 1.0, then the fp32 flush
// y += s * (acc - c * sum_x) with (s, c) read from LDS.
template <int RT, bool ASYM>
__device__ __forceinline__ void group_step(const u32x4 (&a)[RT], const u32x4 (&b)[4],
                                           const float* lds, int g, int TR, int lg,
                                           float (&yacc)[RT][4]) {
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  bf16x8 bx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bx[i] = as_bf16x8(pair_activations(b[i]));
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), bx[i], sacc, 0, 0, 0);
  const float sx = sacc[0];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t word = a[rt][i];
      if (!ASYM) word ^= 0x88888888u;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(unpack_word(word)), bx[i], acc, 0,
                                                    0, 0);
    }
    const float4* sc = reinterpret_cast<const float4*>(lds + (g * TR + rt * 16 + lg * 4) * 2);
    const float4 p01 = sc[0], p23 = sc[1];
    const float sv[4] = {p01.x, p01.z, p23.x, p23.z};
    const float cv[4] = {p01.y, p01.w, p23.y, p23.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      yacc[rt][r] = __builtin_fmaf(sv[r], __builtin_fmaf(-cv[r], sx, acc[r]), yacc[rt][r]);
  }
}

template <int RT, bool ASYM>
__global__ __launch_bounds__(1024) void qgemv_kernel(const uint16_t* __restrict__ x, int M,
                                                     const uint32_t* __restrict__ w,
                                                     const uint16_t* __restrict__ s16,
                                                     const uint16_t* __restrict__ z16, int N,
                                                     int K, uint16_t* __restrict__ y) {
  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);
  constexpr int TR = 16 * RT;                      // rows per workgroup
  const int G = K / kGroup;
  const int KS = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int n0 = blockIdx.x * TR;

  // ---- stage (s, c) of every (group, row) of the tile: lds[(g*TR + r)*2 + {0,1}]
  for (int idx = threadIdx.x; idx < TR * G; idx += blockDim.x) {
    const int r = idx / G, g = idx - r * G;
    const int n = n0 + r;
    float s = 0.f, c = 0.f;
    if (n < N) {
      s = f16_bits_to_f32(s16[(int64_t)n * G + g]);
      c = ASYM ? 128.f + f16_bits_to_f32(z16[(int64_t)n * G + g]) : 136.f;
    }
    lds[(g * TR + r) * 2] = s;
    lds[(g * TR + r) * 2 + 1] = c;
  }
  __syncthreads();

  const int gb = (int)((int64_t)wave * G / KS);
  const int ge = (int)((int64_t)(wave + 1) * G / KS);

  // Raw buffer loads: bytes past the end of a buffer read as zero, which
  // masks rows n >= N and activation rows m >= M without branches; being
  // intrinsics (not plain loads) they also stay where they are issued, so the
  // next group is in flight while the current one is computed.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)w, (short)0, (int)((int64_t)N * K / 2 > 0x7fffffff ? 0x7fffffff : (int64_t)N * K / 2),
      0x00020000);
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, 0x00020000);
  uint32_t woff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n0 + rt * 16 + li;
    woff[rt] = n < N ? (uint32_t)n * (uint32_t)(K / 2) + lg * 16 : 0x80000000u;
  }
  const uint32_t xoff = li < M ? (uint32_t)li * (uint32_t)(K * 2) + lg * 64 : 0x80000000u;
  float yacc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) yacc[rt][r] = 0.f;

  // Two register sets used in ping-pong (no copies, so the prefetched loads
  // are never waited for before they are needed).
  u32x4 a0[RT], b0[4], a1[RT], b1[4];
  if (gb < ge) load_group<RT>(wres, xres, woff, xoff, gb, a0, b0);
  for (int g = gb; g < ge; g += 2) {
    // unconditional prefetch (clamped: the last group re-reads itself, a
    // cache hit); a branch here would make the compiler wait for it
    load_group<RT>(wres, xres, woff, xoff, g + 1 < ge ? g + 1 : g, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    group_step<RT, ASYM>(a0, b0, lds, g, TR, lg, yacc);
    if (g + 1 >= ge) break;
    load_group<RT>(wres, xres, woff, xoff, g + 2 < ge ? g + 2 : g + 1, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    group_step<RT, ASYM>(a1, b1, lds, g + 1, TR, lg, yacc);
  }

  // ---- sum the KS partial tiles: red[wave][rt][r][lane]
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) lds[((wave * RT + rt) * 4 + r) * 64 + lane] = yacc[rt][r];
  __syncthreads();
  // thread t -> (rt, lg, m): 4 consecutive outputs n = n0 + rt*16 + 4*lg + r
  for (int t = threadIdx.x; t < RT * 64; t += blockDim.x) {
    const int rt = t >> 6, ln = t & 63;
    const int m = ln & 15, lgg = ln >> 4;
    if (m >= M) continue;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float acc = 0.f;
      for (int ww = 0; ww < KS; ++ww) acc += lds[((ww * RT + rt) * 4 + r) * 64 + ln];
      v[r] = acc;
    }
    const int nb = n0 + rt * 16 + lgg * 4;
    uint16_t* yp = y + (int64_t)m * N + nb;
    if (nb + 3 < N && (N & 3) == 0) {
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(yp) = o;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nb + r < N) yp[r] = (uint16_t)f32_to_bf16_bits(v[r]);
    }
  }
}

template <int RT, bool ASYM>
hipError_t launch_rt(const void* x, int M, const void* w, const void* s, const void* z, int N,
                     int K, void* y, hipStream_t stream) {
  constexpr int TR = 16 * RT;
  const int G = K / kGroup;
  const int blocks = (N + TR - 1) / TR;
  int ks = (2048 + blocks - 1) / blocks;
  if (ks > 16) ks = 16;
  if (ks > G) ks = G;
  if (ks < 1) ks = 1;
  const size_t sc_bytes = (size_t)G * TR * 2 * sizeof(float);
  const size_t red_bytes = (size_t)ks * RT * 4 * 64 * sizeof(float);
  const size_t lds = sc_bytes > red_bytes ? sc_bytes : red_bytes;
  hipLaunchKernelGGL((qgemv_kernel<RT, ASYM>), dim3(blocks), dim3(64 * ks), lds, stream,
                     (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,
                     (const uint16_t*)z, N, K, (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

// LDS per workgroup is G * 16*RT * 8 bytes of staged scales; RT = 2 while
// that stays within 64 KiB (K <= 32768), RT = 1 up to K = 65536.
hipError_t launch_qgemv(bool asym, const void* x, int64_t M, const void* wcodes,
                        const void* wscales, const void* wzeros, int64_t N, int64_t K, void* y,
                        hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (K <= 32768) {
    return asym ? launch_rt<2, true>(x, m, wcodes, wscales, wzeros, n, k, y, stream)
                : launch_rt<2, false>(x, m, wcodes, wscales, wzeros, n, k, y, stream);
  }
  return asym ? launch_rt<1, true>(x, m, wcodes, wscales, wzeros, n, k, y, stream)
              : launch_rt<1, false>(x, m, wcodes, wscales, wzeros, n, k, y, stream);
}

}  // namespace qg
