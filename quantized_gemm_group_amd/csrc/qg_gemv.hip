// W4A16 decode GEMV: y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] (q[n][k] - z[n][g])
// for 1 <= M <= 16, INT4 weights in groups of 128 along K.
//
// The small-batch W4A16 product is HBM bound (《推理优化与量化算子深度技术调研》
// section 1.3; 《第 1 章：推理加速全景》 roofline: ~1 FLOP per byte), with the
// dequantization done inside the kernel (《第 6 课：量化源码走读》 section 2) and
// the asymmetric zero-point cross term kept (same lesson, section 3).
//
// Design for gfx950 (64-wide waves, bf16 MFMA):
//  * A wave owns 16 output channels and a slice of the K groups.  Lane l
//    reads 16 bytes (32 nibbles) of row l%16 at byte offset 16*(l/16) of a
//    group: one 128-bit load covers 16 rows x 64 contiguous bytes, the next
//    group completes each 128-byte line.  Loads are raw buffer loads (rows
//    past N read as zero).
//  * Nibbles are unpacked in registers with one and/xor per pair:
//    ((w >> 4j) & 0x000F000F) ^ C is the bf16 pair (128+u_j, 128+u_{j+4}),
//    exact integers (u = q + 8 for two's-complement codes), so the matrix
//    cores multiply exact codes and no dequantized weight is ever rounded.
//  * v_mfma_f32_16x16x32_bf16: A = codes (16 channels), B = x^T (columns m,
//    zero beyond M; pairs (x_j, x_{j+4}) to match the unpack), plus one MFMA
//    with A = 1.0 for the group sums of x.  Per group, in fp32:
//        y += s * (acc - c * sum_x),  c = 136 (symmetric) or 128 + z.
//  * When M*K is small the activations are staged (pair-permuted) in LDS once
//    per workgroup; the only vector-memory loads left in the loop are the
//    weights, kept kRing groups deep in a register ring (vector loads
//    complete in issue order, so a deep ring only works when nothing else
//    shares the queue).  Larger M*K reads x from the cache and prefetches one
//    group ahead.
//  * Group scales and offsets (s, c) of the workgroup's rows are staged once
//    in LDS; the K-slices of a row tile are summed through LDS and rounded
//    once to bf16 (RNE).  No scratch memory.

#include <type_traits>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kGroup = 128;
constexpr int kRing = 4;                    // weight groups in flight per wave
constexpr int kXldsMaxBytes = 48 * 1024;    // x staged in LDS up to this size
constexpr int kXu = 4;                      // x chunks per thread loaded ahead of the ring
constexpr int kSu = 1;                      // 16-byte (s, z) loads per thread issued ahead

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ((w >> 4j) & 0x000F000F) ^ C per pair.  The mask and the constant arrive
// as kernel arguments, so the compiler cannot fold them into literals (gfx950
// VOP3 encodings take no literal operands) and selects one v_bitop3_b32 per
// pair instead of shift, and, or with literals.
template <bool ASYM>
__device__ __forceinline__ u32x4 unpack_word(uint32_t w, uint32_t mask, uint32_t c) {
  u32x4 r;
  r[0] = (w & mask) ^ c;
  r[1] = ((w >> 4) & mask) ^ c;
  r[2] = ((w >> 8) & mask) ^ c;
  r[3] = ((w >> 12) & mask) ^ c;
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

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Where the packed codes of a 16-row tile live.  Canonical layout ([N][K/8]
// int32): row n, group g at n * K/2 + 64 g; one wave-wide 16-byte load covers
// 16 rows x 64 bytes, i.e. half of 16 cache lines.  Tiled layout (written
// once by qg_tile_gemv_weights): tile t, group g is one contiguous 1 KiB block
// [t][g][4 quarters][16 rows][16 bytes], quarter q holding bytes 16 q .. +15
// of each row's group, so the same load reads the block in lane order (lane
// li + 16 lg at 16 (li + 16 lg)): every 4 lanes one 64-byte run, the wave 8
// whole lines.  Those loads carry the non-temporal hint (the codes are read
// once: they stream past the caches instead of displacing the activations and
// scales there).
template <bool TILED>
struct WLayout {
  static constexpr int kGroupStride = TILED ? 1024 : 64;   // bytes between groups of a row
  // byte offset of the lane's 16 bytes (quarter lg) of group 0 of row n
  __device__ static uint32_t row_off(int n, int lg, int N, int K) {
    if (n >= N) return 0x80000000u;                       // past the end: reads zero
    return TILED ? (uint32_t)(n >> 4) * (uint32_t)(K / 128) * 1024u +
                       (uint32_t)(lg * 256 + (n & 15) * 16)
                 : (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)(lg * 16);
  }
  // the same for row li of tile `tile`
  __device__ static uint32_t lane_off(int tile, int li, int lg, int N, int K) {
    return row_off(tile * 16 + li, lg, N, K);
  }
  __device__ static int64_t bytes(int N, int K) {
    return TILED ? (int64_t)((N + 15) / 16) * 16 * K / 2 : (int64_t)N * K / 2;
  }
  __device__ static u32x4 load(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff,
                                                                           TILED ? 2 : 0));
  }
};

// One group of one 16-channel tile: 4 code MFMAs, then the flush
// y += s * (acc - c * sum_x).  sum_x comes precomputed (x staged in LDS) or
// from 4 more MFMAs against 1.0 (x read from the cache).
template <bool ASYM, bool SUMX_GIVEN>
__device__ __forceinline__ void group_math(const u32x4& a, const bf16x8 (&bx)[4], const float* sc,
                                           float sx_given, uint32_t mask, uint32_t cmag,
                                           float (&yacc)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (!SUMX_GIVEN) {
      const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), bx[i], sacc, 0, 0, 0);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(unpack_word<ASYM>(a[i], mask, cmag)),
                                                  bx[i], acc, 0, 0, 0);
  }
  const float4 p01 = reinterpret_cast<const float4*>(sc)[0];
  const float4 p23 = reinterpret_cast<const float4*>(sc)[1];
  const float sx = SUMX_GIVEN ? sx_given : sacc[0];
  yacc[0] = __builtin_fmaf(p01.x, __builtin_fmaf(-p01.y, sx, acc[0]), yacc[0]);
  yacc[1] = __builtin_fmaf(p01.z, __builtin_fmaf(-p01.w, sx, acc[1]), yacc[1]);
  yacc[2] = __builtin_fmaf(p23.x, __builtin_fmaf(-p23.y, sx, acc[2]), yacc[2]);
  yacc[3] = __builtin_fmaf(p23.z, __builtin_fmaf(-p23.w, sx, acc[3]), yacc[3]);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_g(const void* p, int64_t bytes) {
  const int64_t lim = bytes > 0x7ffff000LL ? 0x7ffff000LL : bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)lim, 0x00020000);
}

// Stage the (s, c) pairs of rows [n0, n0 + TR) for all G groups into
// scl[(g * TR + r) * 2 + {0, 1}]; four elements per thread in flight.
template <bool ASYM>
__device__ __forceinline__ void stage_scales(const uint16_t* __restrict__ s16,
                                             const uint16_t* __restrict__ z16, int N, int G,
                                             int n0, int TR, float* scl) {
  const int total = TR * G;
  for (int i0 = threadIdx.x; i0 < total; i0 += 4 * blockDim.x) {
    uint16_t sv[4], zv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = i0 + u * blockDim.x;
      const int r = idx / G, g = idx - r * G;
      const int n = n0 + r;
      sv[u] = 0;
      zv[u] = 0;
      if (idx < total && n < N) {
        sv[u] = s16[(int64_t)n * G + g];
        if (ASYM) zv[u] = z16[(int64_t)n * G + g];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = i0 + u * blockDim.x;
      if (idx >= total) continue;
      const int r = idx / G, g = idx - r * G;
      const bool ok = n0 + r < N;
      scl[(g * TR + r) * 2] = ok ? f16_bits_to_f32(sv[u]) : 0.f;
      scl[(g * TR + r) * 2 + 1] = ok ? (ASYM ? 128.f + f16_bits_to_f32(zv[u]) : 136.f) : 0.f;
    }
  }
}

// Workgroup = RW row tiles x KS K-slices, one wave each (wave = rw*KS + kw).
//   LDS: [x: M*K bf16, pair-permuted (XLDS)] [sum_x: M*G floats (XLDS)]
//        [sc: G * RW*16 float2]; then reused for the partial sums
//        [RW][KS][4][64] floats.
template <bool ASYM, bool XLDS, bool SVEC, bool TILED>
__global__ __launch_bounds__(1024) void qgemv_kernel(const uint16_t* __restrict__ x, int M,
                                                     const uint32_t* __restrict__ w,
                                                     const uint16_t* __restrict__ s16,
                                                     const uint16_t* __restrict__ z16, int N,
                                                     int K, int KS, int RW,
                                                     uint16_t* __restrict__ y, uint32_t mask,
                                                     uint32_t cmag) {
  extern __shared__ float4 lds4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds4);
  const int G = K / kGroup;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int kw = wave % KS, rw = wave / KS;
  const int tile0 = blockIdx.x * RW;                 // first row tile of the workgroup
  const int TR = RW * 16;

  const int gb = (int)((int64_t)kw * G / KS);
  const int ge = (int)((int64_t)(kw + 1) * G / KS);

  using WL = WLayout<TILED>;
  const __amdgpu_buffer_rsrc_t wres = make_rsrc_g(w, WL::bytes(N, K));
  const uint32_t woff = WL::lane_off(tile0 + rw, li, lg, N, K);
  constexpr int kGS = WL::kGroupStride;
  float yacc[4] = {0.f, 0.f, 0.f, 0.f};
  const int xbytes = XLDS ? M * K * 2 : 0;
  const int sxbytes = XLDS ? (M * G * 4 + 15) & ~15 : 0;
  float* sxl = reinterpret_cast<float*>(lds + xbytes);
  float* scl = reinterpret_cast<float*>(lds + xbytes + sxbytes);
  const float* sc_base = scl + (rw * 16 + lg * 4) * 2;

  if constexpr (XLDS) {
    // ---- 1. staging loads first (x: kXu chunks, scales: kSu elements per
    //      thread), then the weight ring: vector loads return in issue order,
    //      so the staging data lands before the ring and the wait below does
    //      not drain the ring.
    const int chunks = M * K / 8;
    const int total_sc = TR * G;
    const int nt = blockDim.x;
    u32x4 xv[kXu];
    // unconditional loads from clamped (always valid) addresses: a
    // predicated load makes the compiler wait for it on the spot; entries
    // past the end are masked when written to LDS
#pragma unroll
    for (int u = 0; u < kXu; ++u) {
      const int q = threadIdx.x + u * nt;
      xv[u] = reinterpret_cast<const u32x4*>(x)[q < chunks ? q : chunks - 1];
    }
    // scales: 8 fp16 per 16-byte load when a row's groups come in whole
    // 16-byte pieces (G % 8 == 0), else one element per load; the first
    // kSu loads per thread are issued ahead of the ring
    constexpr bool svec = SVEC;
    const int total_sv = svec ? total_sc / 8 : total_sc;
    u32x4 svv[kSu], zvv[kSu];
#pragma unroll
    for (int u = 0; u < kSu; ++u) {
      int idx = threadIdx.x + u * nt;
      idx = idx < total_sv ? idx : total_sv - 1;
      if (svec) {
        const int r = idx / (G / 8), gc = idx - r * (G / 8);
        int n = tile0 * 16 + r;
        n = n < N ? n : N - 1;
        svv[u] = reinterpret_cast<const u32x4*>(s16 + (int64_t)n * G)[gc];
        zvv[u] = ASYM ? reinterpret_cast<const u32x4*>(z16 + (int64_t)n * G)[gc] : svv[u];
      } else {
        const int r = idx / G, g = idx - r * G;
        int n = tile0 * 16 + r;
        n = n < N ? n : N - 1;
        svv[u][0] = s16[(int64_t)n * G + g];
        zvv[u][0] = ASYM ? z16[(int64_t)n * G + g] : (uint16_t)0;
      }
    }
    u32x4 ring[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j)
      ring[j] = WL::load(wres, gb + j < ge ? woff : 0x80000000u, (gb + j) * kGS);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. x into LDS pair-permuted, with the group sums of x (16
    //      consecutive chunks of 8 form one group of 128; xor-shuffles sum them).
    //      The preloaded first kXu rounds are handled straight-line so their
    //      loads stay ahead of the ring.
    auto put_x = [&](const u32x4& d, int q) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part += bf16_bits_to_f32(d[e] & 0xffffu) + bf16_bits_to_f32(d[e] >> 16);
      part += shfl_xor(part, 1);
      part += shfl_xor(part, 2);
      part += shfl_xor(part, 4);
      part += shfl_xor(part, 8);
      if (q < chunks) {
        reinterpret_cast<u32x4*>(lds)[q] = pair_activations(d);
        if ((q & 15) == 0) sxl[q >> 4] = part;
      }
    };
#pragma unroll
    for (int u = 0; u < kXu; ++u) put_x(xv[u], threadIdx.x + u * nt);
    for (int u = kXu; u * nt < chunks; ++u) {
      const int q = threadIdx.x + u * nt;
      put_x(reinterpret_cast<const u32x4*>(x)[q < chunks ? q : chunks - 1], q);
    }
    // ---- 3. (s, c) pairs
    auto put_sc = [&](uint32_t sb, uint32_t zb, int r, int g) {
      const bool ok = tile0 * 16 + r < N;
      scl[(g * TR + r) * 2] = ok ? f16_bits_to_f32((uint16_t)sb) : 0.f;
      scl[(g * TR + r) * 2 + 1] =
          ok ? (ASYM ? 128.f + f16_bits_to_f32((uint16_t)zb) : 136.f) : 0.f;
    };
    auto put_sv = [&](const u32x4& sv, const u32x4& zv, int idx) {
      if (idx >= total_sv) return;
      if (svec) {
        const int r = idx / (G / 8), g0 = (idx - r * (G / 8)) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          put_sc(sv[e >> 1] >> (16 * (e & 1)), zv[e >> 1] >> (16 * (e & 1)), r, g0 + e);
      } else {
        const int r = idx / G;
        put_sc(sv[0], zv[0], r, idx - r * G);
      }
    };
#pragma unroll
    for (int u = 0; u < kSu; ++u) put_sv(svv[u], zvv[u], threadIdx.x + u * nt);
    for (int u = kSu; u * nt < total_sv; ++u) {
      const int idx = threadIdx.x + u * nt;
      const int ic = idx < total_sv ? idx : total_sv - 1;
      u32x4 sv = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (svec) {
        const int r = ic / (G / 8), gc = ic - r * (G / 8);
        int n = tile0 * 16 + r;
        n = n < N ? n : N - 1;
        sv = reinterpret_cast<const u32x4*>(s16 + (int64_t)n * G)[gc];
        if (ASYM) zv = reinterpret_cast<const u32x4*>(z16 + (int64_t)n * G)[gc];
      } else {
        const int r = ic / G, g = ic - r * G;
        int n = tile0 * 16 + r;
        n = n < N ? n : N - 1;
        sv[0] = s16[(int64_t)n * G + g];
        if (ASYM) zv[0] = z16[(int64_t)n * G + g];
      }
      put_sv(sv, zv, idx);
    }
    __syncthreads();

    // ---- 4. main loop: group g uses ring slot (g - gb) % kRing.  Columns
    //      m >= M read row 0: their results are never stored.
    const int mrow = li < M ? li : 0;
    const u32x4* xrow = reinterpret_cast<const u32x4*>(lds + (size_t)mrow * K * 2);
    const float* sxrow = sxl + mrow * G;
    for (int g0 = gb; g0 < ge; g0 += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        const int g = g0 + j;
        if (g < ge) {
          bf16x8 bx[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) bx[i] = as_bf16x8(xrow[g * 16 + lg * 4 + i]);
          group_math<ASYM, true>(ring[j], bx, sc_base + g * TR * 2, sxrow[g], mask, cmag, yacc);
        }
        ring[j] = WL::load(wres, g + kRing < ge ? woff : 0x80000000u, (g + kRing) * kGS);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // x from the cache: weights and x of the next group prefetched together
    const bool mvalid = li < M;
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, 0x00020000);
    const uint32_t xoff = mvalid ? (uint32_t)li * (uint32_t)(K * 2) + lg * 64 : 0x80000000u;
    u32x4 a0, a1, b0[4], b1[4];
    auto load_group = [&](int g, u32x4& a, u32x4 (&b)[4]) {
      const bool ok = g < ge;
      a = WL::load(wres, ok ? woff : 0x80000000u, g * kGS);
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = bload(xres, ok ? xoff : 0x80000000u, g * 256 + i * 16);
    };
    stage_scales<ASYM>(s16, z16, N, G, tile0 * 16, TR, scl);
    load_group(gb, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    for (int g = gb; g < ge; g += 2) {
      load_group(g + 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      {
        bf16x8 bx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bx[i] = as_bf16x8(pair_activations(b0[i]));
        group_math<ASYM, false>(a0, bx, sc_base + g * TR * 2, 0.f, mask, cmag, yacc);
      }
      if (g + 1 >= ge) break;
      load_group(g + 2, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      {
        bf16x8 bx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bx[i] = as_bf16x8(pair_activations(b1[i]));
        group_math<ASYM, false>(a1, bx, sc_base + (g + 1) * TR * 2, 0.f, mask, cmag, yacc);
      }
    }
  }

  // ---- 5. sum the K-slices of each row tile: red[rw][kw][r][lane]
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[((rw * KS + kw) * 4 + r) * 64 + lane] = yacc[r];
  __syncthreads();
  // thread t -> (row tile, lane): outputs n = 16*tile + 4*(ln/16) + r, row m = ln%16
  for (int t = threadIdx.x; t < RW * 64; t += blockDim.x) {
    const int rt = t >> 6, ln = t & 63;
    const int m = ln & 15, lgg = ln >> 4;
    const int nb = (tile0 + rt) * 16 + lgg * 4;
    if (m >= M || nb >= N) continue;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float acc = 0.f;
      for (int k2 = 0; k2 < KS; ++k2) acc += red[((rt * KS + k2) * 4 + r) * 64 + ln];
      v[r] = acc;
    }
    uint16_t* yp = y + (int64_t)m * N + nb;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (nb + r < N) QG_DEBUG_STORE((int64_t)m * N + nb + r, v[r]);
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

// Per-wave GEMV for M <= MM (1 or 4) rows of x and G % 8 == 0.  Workgroup =
// one 16-row tile, KS waves; wave kw owns groups [NG kw, NG kw + NG).  Each
// wave issues all of its loads at once and waits only for its own: its slice
// of x (coalesced 1 KiB loads), the fp16 scales / zero points of its rows
// (one lane per row, NG of them per load) and its NG weight groups.  The x
// slice goes through a private LDS region to be pair-permuted; no barrier
// until the K-slices are summed at the end.
// The matrix cores take x as the first operand and the codes as the second,
// so lane (l % 16, l / 16) accumulates D[m = 4 (l / 16) + r][n = l % 16]: its
// outputs, scale and zero point all belong to weight row n0 + l % 16, and a
// second MFMA against 1.0 gives the group sums of x in the same layout.
// With one row of x (MM = 1) every output lane needs the same group sums:
// each lane's 16-byte piece of x lies in one group, so 16-lane shuffles give
// the sums and a lane read puts each in a scalar register, which drops the
// second MFMA (half of the matrix work) and its registers.
// LDS: [x slices: KS * MM * NG * 256 bytes][partials: KS * 1 KiB].
template <bool ASYM, int NG, int MM, bool TILED>
__global__ __launch_bounds__(1024) void qgemv_wave_kernel(const uint16_t* __restrict__ x, int M,
                                                          const uint32_t* __restrict__ w,
                                                          const uint16_t* __restrict__ s16,
                                                          const uint16_t* __restrict__ z16, int N,
                                                          int K, int KS,
                                                          uint16_t* __restrict__ y, uint32_t mask,
                                                          uint32_t cmag) {
  extern __shared__ float4 lds4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds4);
  constexpr int kXBytes = MM * NG * 256;       // one wave's x slice
  constexpr int kXLoads = NG / 4;              // 1 KiB loads per row of x
  const int G = K / kGroup;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int kw = wave;
  const int n0 = blockIdx.x * 16;
  const int gb = kw * NG;

  // ---- 1. loads: x slice, scales / zero points, weights (all in flight)
  const __amdgpu_buffer_rsrc_t xres = make_rsrc_g(x, (int64_t)M * K * 2);
  u32x4 xr[MM * kXLoads];
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int q = 0; q < kXLoads; ++q)
      xr[m * kXLoads + q] = bload(xres, m < M ? (uint32_t)(m * K + gb * 128 + q * 512 + 8 * lane) * 2
                                              : 0x80000000u, 0);
  const int n = n0 + li;
  const __amdgpu_buffer_rsrc_t sres = make_rsrc_g(s16, (int64_t)N * G * 2);
  const __amdgpu_buffer_rsrc_t zres = make_rsrc_g(z16, ASYM ? (int64_t)N * G * 2 : 0);
  const uint32_t soff = n < N ? (uint32_t)(n * G + gb) * 2 : 0x80000000u;
  // NG fp16 scales (zero points) of row n: NG / 2 dwords
  uint32_t sv[NG / 2], zv[NG / 2];
  if constexpr (NG == 4) {
    const uint2 s2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sres, soff, 0, 0));
    sv[0] = s2.x;
    sv[1] = s2.y;
    const uint2 z2 = ASYM ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(zres, soff, 0, 0))
                          : uint2{0u, 0u};
    zv[0] = z2.x;
    zv[1] = z2.y;
  } else {
#pragma unroll
    for (int c = 0; c < NG / 8; ++c) {
      const u32x4 s4 = bload(sres, soff, 16 * c);
      const u32x4 z4 = ASYM ? bload(zres, soff, 16 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[4 * c + e] = s4[e];
        zv[4 * c + e] = z4[e];
      }
    }
  }
  using WL = WLayout<TILED>;
  const __amdgpu_buffer_rsrc_t wres = make_rsrc_g(w, WL::bytes(N, K));
  const uint32_t woff = WL::lane_off(blockIdx.x, li, lg, N, K);
  u32x4 wr[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) wr[j] = WL::load(wres, woff, (gb + j) * WL::kGroupStride);
  __builtin_amdgcn_sched_barrier(0);   // every load issued before any use

  // ---- 2. the x slice, pair-permuted, into this wave's LDS region: row m,
  //      16-byte piece c (covering k = 8 c .. 8 c + 7 of the slice)
  uint8_t* const xw = lds + wave * kXBytes;
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int q = 0; q < kXLoads; ++q)
      reinterpret_cast<u32x4*>(xw)[m * NG * 16 + q * 64 + lane] =
          pair_activations(xr[m * kXLoads + q]);

  // group sums of x for one row: lane l of load q holds elements
  // 512 q + 8 l .. + 7 of the slice, i.e. 8 values of group 4 q + l / 16
  float gsum[MM == 1 ? kXLoads : 1];
  if constexpr (MM == 1) {
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part += __uint_as_float(xr[q][e] << 16);
        part += __uint_as_float(xr[q][e] & 0xffff0000u);
      }
      part += shfl_xor(part, 1);
      part += shfl_xor(part, 2);
      part += shfl_xor(part, 4);
      part += shfl_xor(part, 8);
      gsum[q] = part;
    }
  }

  // ---- 3. groups.  Rows m >= M of the first operand repeat row 0: their
  //      results are never stored.
  const int mrow = li < M ? li : 0;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(xw) + mrow * NG * 16 + lg * 4;
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float yacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    bf16x8 bx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bx[i] = as_bf16x8(xrow[j * 16 + i]);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, sacc = acc0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 cw = as_bf16x8(unpack_word<ASYM>(wr[j][i], mask, cmag));
      if (i & 1)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx[i], cw, acc1, 0, 0, 0);
      else
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx[i], cw, acc0, 0, 0, 0);
      if constexpr (MM != 1)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx[i], as_bf16x8(ones), sacc, 0, 0, 0);
    }
    if constexpr (MM == 1) {
      const float sx = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gsum[j >> 2]), 16 * (j & 3)));
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = sx;
    }
    const uint32_t sb = (sv[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    const float sc = f16_bits_to_f32(sb);
    float cc = 136.f;
    if constexpr (ASYM) cc = 128.f + f16_bits_to_f32((zv[j >> 1] >> (16 * (j & 1))) & 0xffffu);
    static_assert(NG % 4 == 0, "groups per wave: a multiple of 4");
#pragma unroll
    for (int r = 0; r < 4; ++r)
      yacc[r] = __builtin_fmaf(sc, __builtin_fmaf(-cc, sacc[r], acc0[r] + acc1[r]), yacc[r]);
  }

  // ---- 4. sum the K-slices: red[kw][r][lane]; lane (li, lg) of the first
  //      wave writes y[m = 4 lg + r][n0 + li] for m < M
  float* red = reinterpret_cast<float*>(lds + KS * kXBytes);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(kw * 4 + r) * 64 + lane] = yacc[r];
  __syncthreads();
  if (wave == 0 && n < N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lg + r;
      if (m < M) {
        float v = 0.f;
        for (int k2 = 0; k2 < KS; ++k2) v += red[(k2 * 4 + r) * 64 + lane];
        QG_DEBUG_STORE((int64_t)m * N + n, v);
        y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

// SwiGLU decode GEMV for M <= MM (1 or 4) rows of x: h[m][i] = SiLU(g) * u
// with g and u the GEMV outputs of rows i and I + i of the concatenation
// [W_gate; W_up] (《推理优化与量化算子深度技术调研》 section 4.6: the gate and up
// projections as one product over the concatenated weight, SiLU(g) * u
// formed in registers and written once).  Workgroup = one 16-channel tile i
// of h and KS waves over the K-slices, as in qgemv_wave_kernel, but every
// wave streams two weight tiles -- the gate rows of the tile and the same
// channels' up rows -- against one x slice (loaded, permuted and summed
// once).  After the K-slice sum through LDS the first wave holds g and u of
// each output in the same lane and writes bf16(SiLU(g) * u) (fp32, e^-g
// from the hardware exponential).  The codes of either layout (canonical
// or tiled) are addressed per row, so I needs no alignment.
// LDS: [x slices: KS * MM * NG * 256 bytes][partials: KS * 2 KiB].
template <bool ASYM, int NG, int MM, bool TILED>
__global__ __launch_bounds__(1024) void qgemv_swiglu_kernel(const uint16_t* __restrict__ x, int M,
                                                            const uint32_t* __restrict__ w,
                                                            const uint16_t* __restrict__ s16,
                                                            const uint16_t* __restrict__ z16,
                                                            int I, int K, int KS,
                                                            uint16_t* __restrict__ h,
                                                            uint32_t mask, uint32_t cmag) {
  extern __shared__ float4 lds4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds4);
  constexpr int kXBytes = MM * NG * 256;       // one wave's x slice
  constexpr int kXLoads = NG / 4;              // 1 KiB loads per row of x
  const int G = K / kGroup;
  const int N2 = 2 * I;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int kw = wave;
  const int i = blockIdx.x * 16 + li;          // output channel of this lane's rows
  const int gb = kw * NG;
  using WL = WLayout<TILED>;

  // ---- 1. loads: x slice, the (s, z) of both rows, both tiles' codes
  const __amdgpu_buffer_rsrc_t xres = make_rsrc_g(x, (int64_t)M * K * 2);
  u32x4 xr[MM * kXLoads];
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int q = 0; q < kXLoads; ++q)
      xr[m * kXLoads + q] = bload(xres, m < M ? (uint32_t)(m * K + gb * 128 + q * 512 + 8 * lane) * 2
                                              : 0x80000000u, 0);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc_g(s16, (int64_t)N2 * G * 2);
  const __amdgpu_buffer_rsrc_t zres = make_rsrc_g(z16, ASYM ? (int64_t)N2 * G * 2 : 0);
  uint32_t sv[2][NG / 2], zv[2][NG / 2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = t * I + i;                   // gate row i, up row I + i
    const uint32_t soff = i < I ? (uint32_t)(n * G + gb) * 2 : 0x80000000u;
    if constexpr (NG == 4) {
      const uint2 s2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sres, soff, 0, 0));
      const uint2 z2 = ASYM ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(zres, soff, 0, 0))
                            : uint2{0u, 0u};
      sv[t][0] = s2.x;
      sv[t][1] = s2.y;
      zv[t][0] = z2.x;
      zv[t][1] = z2.y;
    } else {
#pragma unroll
      for (int c = 0; c < NG / 8; ++c) {
        const u32x4 s4 = bload(sres, soff, 16 * c);
        const u32x4 z4 = ASYM ? bload(zres, soff, 16 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[t][4 * c + e] = s4[e];
          zv[t][4 * c + e] = z4[e];
        }
      }
    }
  }
  const __amdgpu_buffer_rsrc_t wres = make_rsrc_g(w, WL::bytes(N2, K));
  u32x4 wr[2][NG];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t woff = WL::row_off(i < I ? t * I + i : N2, lg, N2, K);
#pragma unroll
    for (int j = 0; j < NG; ++j) wr[t][j] = WL::load(wres, woff, (gb + j) * WL::kGroupStride);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load issued before any use

  // ---- 2. the x slice, pair-permuted, into this wave's LDS region
  uint8_t* const xw = lds + wave * kXBytes;
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int q = 0; q < kXLoads; ++q)
      reinterpret_cast<u32x4*>(xw)[m * NG * 16 + q * 64 + lane] =
          pair_activations(xr[m * kXLoads + q]);
  float gsum[MM == 1 ? kXLoads : 1];
  if constexpr (MM == 1) {
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part += __uint_as_float(xr[q][e] << 16);
        part += __uint_as_float(xr[q][e] & 0xffff0000u);
      }
      part += shfl_xor(part, 1);
      part += shfl_xor(part, 2);
      part += shfl_xor(part, 4);
      part += shfl_xor(part, 8);
      gsum[q] = part;
    }
  }

  // ---- 3. groups: both tiles against the same x fragments and group sums
  const int mrow = li < M ? li : 0;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(xw) + mrow * NG * 16 + lg * 4;
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float yacc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    bf16x8 bx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bx[q] = as_bf16x8(xrow[j * 16 + q]);
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[t][0] = acc[t][1] = sacc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[t][q & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            bx[q], as_bf16x8(unpack_word<ASYM>(wr[t][j][q], mask, cmag)), acc[t][q & 1], 0, 0, 0);
      if constexpr (MM != 1)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx[q], as_bf16x8(ones), sacc, 0, 0, 0);
    }
    if constexpr (MM == 1) {
      const float sx = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gsum[j >> 2]), 16 * (j & 3)));
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = sx;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float sc = f16_bits_to_f32((sv[t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
      float cc = 136.f;
      if constexpr (ASYM) cc = 128.f + f16_bits_to_f32((zv[t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        yacc[t][r] = __builtin_fmaf(sc, __builtin_fmaf(-cc, sacc[r], acc[t][0][r] + acc[t][1][r]),
                                    yacc[t][r]);
    }
  }

  // ---- 4. sum the K-slices: red[kw][t][r][lane]; lane (li, lg) of the
  //      first wave writes h[m = 4 lg + r][i] for m < M
  float* red = reinterpret_cast<float*>(lds + KS * kXBytes);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((kw * 2 + t) * 4 + r) * 64 + lane] = yacc[t][r];
  __syncthreads();
  if (wave == 0 && i < I) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lg + r;
      if (m < M) {
        float g = 0.f, u = 0.f;
        for (int k2 = 0; k2 < KS; ++k2) {
          g += red[((k2 * 2 + 0) * 4 + r) * 64 + lane];
          u += red[((k2 * 2 + 1) * 4 + r) * 64 + lane];
        }
        const float hv = g / (1.f + __expf(-g)) * u;
        QG_DEBUG_STORE((int64_t)m * I + i, hv);
        h[(int64_t)m * I + i] = (uint16_t)f32_to_bf16_bits(hv);
      }
    }
  }
}

// Codes of one word in natural order: dword d holds the bf16 pair
// (128 + u_{2d}, 128 + u_{2d+1}), so activations read straight from memory
// need no permute.  Byte d of w and of w >> 4 go to the two halves (one
// byte permute), then the same mask / xor as above.
__device__ __forceinline__ u32x4 unpack_word_nat(uint32_t w, uint32_t mask, uint32_t c) {
  const uint32_t t = w >> 4;
  u32x4 r;
  r[0] = (__builtin_amdgcn_perm(t, w, 0x0C040C00u) & mask) ^ c;
  r[1] = (__builtin_amdgcn_perm(t, w, 0x0C050C01u) & mask) ^ c;
  r[2] = (__builtin_amdgcn_perm(t, w, 0x0C060C02u) & mask) ^ c;
  r[3] = (__builtin_amdgcn_perm(t, w, 0x0C070C03u) & mask) ^ c;
  return r;
}

// 4x4 transpose across the four 16-lane rows: row r, register e receives
// row e, register r (two swaps of lane halves, two of odd / even rows).
__device__ __forceinline__ u32x4 transpose_rows(const u32x4& v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  u32x4 r;
  r[0] = c[0];
  r[1] = c[1];
  r[2] = d[0];
  r[3] = d[1];
  return r;
}

// Per-wave GEMV for 5 <= M <= 16.  Workgroup = R tiles of 16 output channels
// and KS waves; wave kw owns groups [NG kw, NG kw + NG).  With all 16 rows
// of the MFMA in use, every matrix instruction takes its activations straight
// from memory (served by the caches: x is shared by every workgroup), no LDS
// staging and no barrier until the K-slices are summed.  Within a group,
// lane (li, lg) and MFMA i cover k = 32 i + 8 lg .. + 7 for both operands.
// The lane's 16-byte code load holds words 4 lg .. 4 lg + 3 of its channel;
// a transpose across the lane rows turns them into words lg, 4 + lg, 8 + lg,
// 12 + lg, the ones its MFMAs need.
// Activations are read in whole 128-byte lines: the lanes of a row pair
// (li = 2p, 2p + 1) load, in load (h, e), all 8 chunks of line h of row
// 2p + e (lane 2p + b takes chunk 4 (b ^ e) + lg of the line).  So each lane
// holds, for line h, one chunk of its own row (k chunk 8 h + lg: MFMA 2 h)
// and one of its partner row (k chunk 8 h + 4 + lg: MFMA 2 h + 1); a select
// on the lane parity picks them.  MFMAs 1 and 3 thus see the rows of each
// pair swapped, which swaps their output rows m, m ^ 1: they accumulate
// apart and are read back with the register index flipped.
// D groups are kept in flight in registers.
// The matrix cores take x as the first operand: lane (li, lg) accumulates
// D[m = 4 lg + r][n = li] of each channel tile, and an MFMA against 1.0
// gives the group sums of x in the same layout.
// LDS: partial sums [KS][R][4][64] floats.
// SWIGLU (R = 2): N is the row count 2I of [W_gate; W_up]; tile 0 of the
// wave is the gate rows of output channels 16 b .. 16 b + 15 and tile 1 the
// same channels' up rows (rows I + ...), and the first wave writes
// h[m][i] = bf16(SiLU(g) * u) into y as [M][I] (《推理优化与量化算子深度技术调研》
// section 4.6).
template <bool ASYM, int NG, int R, bool TILED, bool SWIGLU = false>
__global__ __launch_bounds__(1024) void qgemv_m16_kernel(const uint16_t* __restrict__ x, int M,
                                                         const uint32_t* __restrict__ w,
                                                         const uint16_t* __restrict__ s16,
                                                         const uint16_t* __restrict__ z16, int N,
                                                         int K, int KS,
                                                         uint16_t* __restrict__ y, uint32_t mask,
                                                         uint32_t cmag) {
  extern __shared__ float4 lds4[];
  float* red = reinterpret_cast<float*>(lds4);
  constexpr int D = NG == 2 ? 2 : (NG == 16 ? 2 : (R == 1 ? 4 : 3));   // groups in flight
  static_assert(NG == 2 || NG % 4 == 0, "groups per wave: 2 or a multiple of 4");
  const int G = K / kGroup;
  const int lane = threadIdx.x & 63;
  const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16 * R;
  const int gb = kw * NG;

  // rows m >= M and channels n >= N read as zero (out of the buffer ranges)
  const __amdgpu_buffer_rsrc_t xres = make_rsrc_g(x, (int64_t)M * K * 2);
  const int odd = li & 1;
  uint32_t xoff[2];                              // load (h, e): row (li & ~1) + e
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = (li & ~1) + e;
    xoff[e] = row < M ? (uint32_t)((row * K + gb * kGroup) * 2 + 64 * (odd ^ e) + 16 * lg)
                      : 0x80000000u;
  }
  using WL = WLayout<TILED>;
  const __amdgpu_buffer_rsrc_t wres = make_rsrc_g(w, WL::bytes(N, K));
  const __amdgpu_buffer_rsrc_t sres = make_rsrc_g(s16, (int64_t)N * G * 2);
  const __amdgpu_buffer_rsrc_t zres = make_rsrc_g(z16, ASYM ? (int64_t)N * G * 2 : 0);
  uint32_t woff[R], soffs[R];
  uint32_t sv[R][NG / 2], zv[R][NG / 2];
  static_assert(!SWIGLU || R == 2, "SwiGLU pairs a gate and an up tile");
  const int I = N / 2;
  const int ich = blockIdx.x * 16 + li;          // SwiGLU: output channel of the lane
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int n = SWIGLU ? (ich < I ? t * I + ich : N) : n0 + 16 * t + li;
    woff[t] = SWIGLU ? WL::row_off(n, lg, N, K) : WL::lane_off(blockIdx.x * R + t, li, lg, N, K);
    if (woff[t] != 0x80000000u) woff[t] += (uint32_t)(gb * WL::kGroupStride);
    soffs[t] = n < N ? (uint32_t)(n * G + gb) * 2 : 0x80000000u;
  }
  // Load order: every scale and zero point, then the ring group by group.
  // Vector loads retire in issue order, so a scale load queued behind the
  // ring would hold the first group's arithmetic until the whole ring lands;
  // the scheduling barriers keep the compiler from moving loads across.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const uint32_t soff = soffs[t];
    if constexpr (NG == 2) {
      sv[t][0] = __builtin_amdgcn_raw_buffer_load_b32(sres, soff, 0, 0);
      zv[t][0] = ASYM ? __builtin_amdgcn_raw_buffer_load_b32(zres, soff, 0, 0) : 0u;
    } else if constexpr (NG == 4) {
      const uint2 s2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sres, soff, 0, 0));
      const uint2 z2 = ASYM ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(zres, soff, 0, 0))
                            : uint2{0u, 0u};
      sv[t][0] = s2.x;
      sv[t][1] = s2.y;
      zv[t][0] = z2.x;
      zv[t][1] = z2.y;
    } else {
#pragma unroll
      for (int c = 0; c < NG / 8; ++c) {
        const u32x4 s4 = bload(sres, soff, 16 * c);
        const u32x4 z4 = ASYM ? bload(zres, soff, 16 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[t][4 * c + e] = s4[e];
          zv[t][4 * c + e] = z4[e];
        }
      }
    }
  }

  u32x4 xr[D][4], wr[D][R];                      // xr[slot][2 h + e]
  auto load = [&](int j, int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[slot][i] = bload(xres, xoff[i & 1], j * 256 + (i >> 1) * 128);
#pragma unroll
    for (int t = 0; t < R; ++t) wr[slot][t] = WL::load(wres, woff[t], j * WL::kGroupStride);
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load(j, j);
    __builtin_amdgcn_sched_barrier(0);
  }

  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float yacc[R][4];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) yacc[t][r] = 0.f;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    // one group at a time: nothing of a later group is hoisted into this one
    // (its selects would wait for that group's loads)
    __builtin_amdgcn_sched_barrier(0);
    const int slot = j % D;
    // [0]: MFMAs 0, 2 (own rows); [1]: MFMAs 1, 3 (rows of each pair swapped)
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    u32x4 wt[R];
#pragma unroll
    for (int t = 0; t < R; ++t) wt[t] = transpose_rows(wr[slot][t]);
    f32x4 acc[R][2];
#pragma unroll
    for (int t = 0; t < R; ++t) acc[t][0] = acc[t][1] = sacc[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // MFMA 2 h: own chunk of line h (load (h, odd)); 2 h + 1: the partner's
      const int h = i >> 1, f = i & 1;
      u32x4 xv;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        xv[d] = (odd ^ f) ? xr[slot][2 * h + 1][d] : xr[slot][2 * h][d];
      const bf16x8 a = as_bf16x8(xv);
      sacc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(ones), sacc[f], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < R; ++t)
        acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, as_bf16x8(unpack_word_nat(wt[t][i], mask, cmag)), acc[t][f], 0, 0, 0);
    }
    if (j + D < NG) load(j + D, slot);
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const float sc = f16_bits_to_f32((sv[t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
      float cc = 136.f;
      if constexpr (ASYM) cc = 128.f + f16_bits_to_f32((zv[t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        yacc[t][r] = __builtin_fmaf(
            sc, __builtin_fmaf(-cc, sacc[0][r] + sacc[1][r ^ 1], acc[t][0][r] + acc[t][1][r ^ 1]),
            yacc[t][r]);
    }
  }

  // sum the K-slices: red[kw][t][r][lane]; the first wave writes
  // y[m = 4 lg + r][n0 + 16 t + li] for m < M, n < N
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((kw * R + t) * 4 + r) * 64 + lane] = yacc[t][r];
  __syncthreads();
  if constexpr (SWIGLU) {
    if (kw == 0 && ich < I) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * lg + r;
        if (m < M) {
          float g = 0.f, u = 0.f;
          for (int k2 = 0; k2 < KS; ++k2) {
            g += red[((k2 * 2 + 0) * 4 + r) * 64 + lane];
            u += red[((k2 * 2 + 1) * 4 + r) * 64 + lane];
          }
          const float hv = g / (1.f + __expf(-g)) * u;
          QG_DEBUG_STORE((int64_t)m * I + ich, hv);
          y[(int64_t)m * I + ich] = (uint16_t)f32_to_bf16_bits(hv);
        }
      }
    }
  } else if (kw == 0) {
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int n = n0 + 16 * t + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * lg + r;
        if (m < M && n < N) {
          float v = 0.f;
          for (int k2 = 0; k2 < KS; ++k2) v += red[((k2 * R + t) * 4 + r) * 64 + lane];
          QG_DEBUG_STORE((int64_t)m * N + n, v);
        y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

template <bool ASYM, int NG, int R, bool TILED>
hipError_t launch_m16_t(const void* x, int M, const void* w, const void* s, const void* z, int N,
                        int K, void* y, hipStream_t stream) {
  const int G = K / kGroup;
  const int ks = G / NG;
  const int blocks = (N + 16 * R - 1) / (16 * R);
  const size_t lds = (size_t)ks * R * 4 * 64 * sizeof(float);
  hipLaunchKernelGGL((qgemv_m16_kernel<ASYM, NG, R, TILED>), dim3(blocks), dim3(64 * ks), lds, stream,
                     (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,
                     (const uint16_t*)z, N, K, ks, (uint16_t*)y, 0x000F000Fu,
                     ASYM ? 0x43004300u : 0x43084308u);
  return hipGetLastError();
}

// Groups per wave for the M <= 16 kernel (0: not applicable), measured on
// MI355X for the Llama-3-8B decode shapes at M = 16: 16 for long K (more than
// 64 groups in at most 16 slices: down 14.7 -> 13.9 us against 8), else 4
// (O 6.2 -> 6.0 us against 8), else 8, else 16.
int pick_m16_ng(int K) {
  const int G = K / kGroup;
  if (G % 16 == 0 && G / 16 <= 16 && G > 64) return 16;
  if (G % 4 == 0 && G / 4 <= 16) return 4;
  if (G % 8 == 0 && G / 8 <= 16) return 8;
  if (G % 16 == 0 && G / 16 <= 16) return 16;
  return 0;
}

template <bool TILED>
hipError_t launch_m16(bool asym, int ng, const void* x, int M, const void* w, const void* s,
                      const void* z, int N, int K, void* y, hipStream_t stream) {
  // two channel tiles per wave (4 groups each, to stay within 128 VGPRs)
  // once there are enough tiles for the chip
  const int G = K / kGroup;
  if (N >= 16384 && G % 4 == 0 && G / 4 <= 16)
    return asym ? launch_m16_t<true, 4, 2, TILED>(x, M, w, s, z, N, K, y, stream)
                : launch_m16_t<false, 4, 2, TILED>(x, M, w, s, z, N, K, y, stream);
  if (asym) {
    if (ng == 4) return launch_m16_t<true, 4, 1, TILED>(x, M, w, s, z, N, K, y, stream);
    if (ng == 16) return launch_m16_t<true, 16, 1, TILED>(x, M, w, s, z, N, K, y, stream);
    return launch_m16_t<true, 8, 1, TILED>(x, M, w, s, z, N, K, y, stream);
  }
  if (ng == 4) return launch_m16_t<false, 4, 1, TILED>(x, M, w, s, z, N, K, y, stream);
  if (ng == 16) return launch_m16_t<false, 16, 1, TILED>(x, M, w, s, z, N, K, y, stream);
  return launch_m16_t<false, 8, 1, TILED>(x, M, w, s, z, N, K, y, stream);
}

// x-shared GEMV for 3 <= M <= 16 rows and K <= 4096 (all 16 rows of x fit in
// LDS).  At 16 rows the activations, not the codes, dominate the reads: a
// 16-channel tile's K-slice of codes is a quarter of the bytes of the same
// slice of x, and every tile-wave re-reading x from L2 made those reads the
// bound.  Here a workgroup of TL x KS waves (one per CU) stages x once -- 16
// rows in 1 KiB direct-to-LDS loads, each covering 4 whole rows of a group,
// chunk c of row r stored at 16-byte slot c ^ r so that the 16 rows of a
// fragment read land on distinct banks -- forms the group sums of x once (for
// SwiGLU per group, by an MFMA against 1.0: LDS holds two tiles' partials), and
// then handles T consecutive 16-channel tiles: wave (tl, ks) takes K-slice ks
// (NG groups) of tiles tl, tl + TL, ... (its units), streaming their codes
// through a register ring that runs across unit boundaries, and reading its x
// fragments from LDS.  Since x comes from LDS in any order, lane (li, lg) and
// MFMA i cover chunk 4 lg + i: the lane's 16-byte code load holds exactly the
// words its 4 MFMAs need.  After each unit the KS partial tiles are summed
// through LDS (two barriers) and rounded once to bf16.
// SWIGLU (R = 2): a unit is 16 channels of h, tile 0 their gate rows and
// tile 1 their up rows of [W_gate; W_up] (N = 2I rows); h = bf16(SiLU(g) u)
// (《推理优化与量化算子深度技术调研》 section 4.6).
// LDS: [x: G x 16 x 256 B][sum_x: G x 16 floats, not for SwiGLU][partials: TL KS R x
// 1 KiB].
template <bool ASYM, int NG, int R, bool TILED, bool SWIGLU>
__global__ __launch_bounds__(1024) void qgemv_xs_kernel(const uint16_t* __restrict__ x, int M,
                                                        const uint32_t* __restrict__ w,
                                                        const uint16_t* __restrict__ s16,
                                                        const uint16_t* __restrict__ z16, int N,
                                                        int K, int KS, int TL, int T, int U,
                                                        uint16_t* __restrict__ y, uint32_t mask,
                                                        uint32_t cmag) {
  static_assert(SWIGLU ? R == 2 : R == 1, "one tile per unit, two (gate, up) for SwiGLU");
  static_assert(NG == 2 || NG == 4 || NG % 8 == 0, "groups per unit: 2, 4 or a multiple of 8");
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  extern __shared__ float4 lds4[];
  uint8_t* const xs = reinterpret_cast<uint8_t*>(lds4);
  const int G = K / kGroup;
  // SwiGLU (two tiles a unit) forms the group sums of x with an MFMA against
  // 1.0 instead, which leaves LDS room for both tiles' partial sums
  constexpr bool kSxLds = !SWIGLU;
  float* const sxs = reinterpret_cast<float*>(xs + G * 4096);
  float* const red = sxs + (kSxLds ? G * 16 : 0);
  constexpr int D = NG < 4 / R ? NG : 4 / R;         // ring depth (groups), divides NG
  const int nw = TL * KS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = wave / KS, ks = wave - tl * KS;
  const int li = lane & 15, lg = lane >> 4;
  const int gb = ks * NG;
  const int I = N / 2;
  const int tiles = SWIGLU ? (I + 15) / 16 : (N + 15) / 16;
  using WL = WLayout<TILED>;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc_g(x, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc_g(w, WL::bytes(N, K));
  const __amdgpu_buffer_rsrc_t sres = make_rsrc_g(s16, (int64_t)N * G * 2);
  const __amdgpu_buffer_rsrc_t zres = make_rsrc_g(z16, ASYM ? (int64_t)N * G * 2 : 0);

  // tile of unit u (-1: none) and the weight row of tile t of it for this lane
  auto unit_tile = [&](int u) {
    const int k = tl + u * TL;
    const int tu = blockIdx.x * T + k;
    return (k < T && tu < tiles) ? tu : -1;
  };
  auto unit_row = [&](int tu, int t) {
    if (tu < 0) return N;
    if constexpr (SWIGLU) {
      const int ich = tu * 16 + li;
      return ich < I ? t * I + ich : N;
    }
    return tu * 16 + li;
  };
  uint32_t woff_c[R], woff_n[R];                     // codes of the current / next unit
  auto unit_woff = [&](int u, uint32_t (&wo)[R]) {
    const int tu = u < U ? unit_tile(u) : -1;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const uint32_t o = WL::row_off(unit_row(tu, t), lg, N, K);
      wo[t] = o == 0x80000000u ? o : o + (uint32_t)(gb * WL::kGroupStride);
    }
  };
  uint32_t sv[2][R][NG / 2], zv[2][R][NG / 2];       // by unit parity
  auto load_scales = [&](int u, auto pc) {
    constexpr int P = decltype(pc)::value;
    const int tu = u < U ? unit_tile(u) : -1;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int n = unit_row(tu, t);
      const uint32_t soff = n < N ? (uint32_t)(n * G + gb) * 2 : 0x80000000u;
      if constexpr (NG == 2) {
        sv[P][t][0] = __builtin_amdgcn_raw_buffer_load_b32(sres, soff, 0, 0);
        zv[P][t][0] = ASYM ? __builtin_amdgcn_raw_buffer_load_b32(zres, soff, 0, 0) : 0u;
      } else if constexpr (NG == 4) {
        const uint2 s2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sres, soff, 0, 0));
        const uint2 z2 = ASYM ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(zres, soff, 0, 0))
                              : uint2{0u, 0u};
        sv[P][t][0] = s2.x;
        sv[P][t][1] = s2.y;
        zv[P][t][0] = z2.x;
        zv[P][t][1] = z2.y;
      } else {
#pragma unroll
        for (int c = 0; c < NG / 8; ++c) {
          const u32x4 s4 = bload(sres, soff, 16 * c);
          const u32x4 z4 = ASYM ? bload(zres, soff, 16 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[P][t][4 * c + e] = s4[e];
            zv[P][t][4 * c + e] = z4[e];
          }
        }
      }
    }
  };
  constexpr int kScaleLoads = R * (NG <= 4 ? 1 : NG / 8) * (ASYM ? 2 : 1);

  // ---- 1. x into LDS: load q covers group q / 4, rows 4 (q % 4) .. + 3;
  //      lane l fetches chunk (l % 16) ^ r of row r = 4 (q % 4) + l / 16
  //      (rows >= M read as zero)
  for (int q = wave; q < 4 * G; q += nw) {
    const int r = 4 * (q & 3) + (lane >> 4);
    const int c = (lane & 15) ^ r;
    const uint32_t vo = r < M ? (uint32_t)(r * K * 2 + c * 16) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void*)(xs + q * 1024), 16, vo,
                                             (q >> 2) * 256, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- 2. scales of unit 0, then the first D groups of the code stream
  load_scales(0, std::integral_constant<int, 0>{});
  unit_woff(0, woff_c);
  u32x4 wr[D][R];
#pragma unroll
  for (int j = 0; j < D; ++j)
#pragma unroll
    for (int t = 0; t < R; ++t) wr[j][t] = WL::load(wres, woff_c[t], j * WL::kGroupStride);
  __builtin_amdgcn_sched_barrier(0);
  // this wave's x loads have landed (vector loads retire in order); then
  // every wave's
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kScaleLoads + D * R) : "memory");

  // ---- 3. group sums of x: lane l sums 32 values of row l / 4
  if constexpr (kSxLds) {
    const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    const int r = lane >> 2, part = lane & 3;
    for (int g = wave; g < G; g += nw) {
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int c = 4 * part + h;
        const u32x4 v = *reinterpret_cast<const u32x4*>(xs + g * 4096 + r * 256 + ((c ^ r) << 4));
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t e = v[d];
          ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e), ones2, ps, false);
        }
      }
      ps += shfl_xor(ps, 1);
      ps += shfl_xor(ps, 2);
      if (part == 0) sxs[g * 16 + r] = ps;
    }
  }
  if constexpr (kSxLds) __syncthreads();

  // ---- 4. units.  The lane's 4 fragment addresses in group gb (the group
  //      of the slice then adds an immediate offset)
  const uint8_t* xfa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xfa[i] = xs + gb * 4096 + li * 256 + (((4 * lg + i) ^ li) << 4);
  const float* const sxa = sxs + gb * 16 + 4 * lg;
  auto unit = [&](int u, auto pc) {
    constexpr int P = decltype(pc)::value;
    // (past the last unit these read nothing: the offsets are out of range)
    load_scales(u + 1, std::integral_constant<int, 1 - P>{});
    unit_woff(u + 1, woff_n);
    float yacc[R][4];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[t][r] = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      u32x4 xf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[i] = *reinterpret_cast<const u32x4*>(xfa[i] + j * 4096);
      float4 sx;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kSxLds) sx = *reinterpret_cast<const float4*>(sxa + j * 16);
      f32x4 acc[R][2];
#pragma unroll
      for (int t = 0; t < R; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (!kSxLds) {
          const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xf[i]), as_bf16x8(ones), sacc,
                                                         0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < R; ++t)
          acc[t][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(xf[i]), as_bf16x8(unpack_word_nat(wr[j % D][t][i], mask, cmag)),
              acc[t][i & 1], 0, 0, 0);
      }
      if constexpr (!kSxLds) sx = float4{sacc[0], sacc[1], sacc[2], sacc[3]};
      // the next item of the stream into this slot: group j + D of this unit
      // or group j + D - NG of the next
      if (j + D < NG) {
#pragma unroll
        for (int t = 0; t < R; ++t)
          wr[j % D][t] = WL::load(wres, woff_c[t], (j + D) * WL::kGroupStride);
      } else {
#pragma unroll
        for (int t = 0; t < R; ++t)
          wr[j % D][t] = WL::load(wres, woff_n[t], (j + D - NG) * WL::kGroupStride);
      }
      const float sxr[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const float sc = f16_bits_to_f32((sv[P][t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
        float cc = 136.f;
        if constexpr (ASYM)
          cc = 128.f + f16_bits_to_f32((zv[P][t][j >> 1] >> (16 * (j & 1))) & 0xffffu);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          yacc[t][r] = __builtin_fmaf(sc, __builtin_fmaf(-cc, sxr[r], acc[t][0][r] + acc[t][1][r]),
                                      yacc[t][r]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- partial tiles: red[tl][ks][t][r][lane]; wave (tl, ks) then sums
    //      registers r = ks, ks + KS, ... of its tile-lane's unit and writes
    //      y[m = 4 lg + r][n = 16 tile + li] (m < M, n < N)
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((tl * KS + ks) * R + t) * 4 + r) * 64 + lane] = yacc[t][r];
    __syncthreads();
    const int tu = unit_tile(u);
    if (tu >= 0) {
      for (int r = ks; r < 4; r += KS) {
        const int m = 4 * lg + r;
        float v[R];
#pragma unroll
        for (int t = 0; t < R; ++t) {
          v[t] = 0.f;
          for (int k2 = 0; k2 < KS; ++k2) v[t] += red[(((tl * KS + k2) * R + t) * 4 + r) * 64 + lane];
        }
        if constexpr (SWIGLU) {
          const int ich = tu * 16 + li;
          if (m < M && ich < I) {
            const float hv = v[0] / (1.f + __expf(-v[0])) * v[1];
            QG_DEBUG_STORE((int64_t)m * I + ich, hv);
            y[(int64_t)m * I + ich] = (uint16_t)f32_to_bf16_bits(hv);
          }
        } else {
          const int n = tu * 16 + li;
          if (m < M && n < N) {
            QG_DEBUG_STORE((int64_t)m * N + n, v[0]);
            y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v[0]);
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < R; ++t) woff_c[t] = woff_n[t];
  };
  for (int u = 0; u < U; u += 2) {
    unit(u, std::integral_constant<int, 0>{});
    if (u + 1 < U) unit(u + 1, std::integral_constant<int, 1>{});
  }
}

// Launch shape of the x-shared kernel (measured on MI355X for the Llama-3-8B
// decode shapes): T = ceil(tiles / 256) tiles per workgroup (about one
// workgroup per CU), TL = T tile-lanes up to 8 / R (beyond, the power of two
// up to 4 / R with U = ceil(T / TL) units per wave) and KS K-slices, the
// largest power of two with TL KS <= 16, halved until NG = G / KS is 2, 4, 8
// or 16.  A 4-group ring (2 at R = 2): 8 groups measured slower.  0 when the
// kernel does not apply: M outside 3..16, a single tile per workgroup (it
// measured slower than the per-wave kernel there: nothing is shared), fewer
// than 4 tiles per workgroup at M <= 4, or x and the partial sums beyond 160
// KiB of LDS (K above about 4096).  At M = 4 the Llama-3-8B gate+up (7 tiles
// per workgroup) measured 15.6-15.9 -> 14.8-14.9 us here and the SwiGLU
// gate+up (4) 14.5 -> 14.2 us, while QKV (2 tiles) went 5.7 -> 7.6 us and
// every projection at M = 2 was slower than on the per-wave kernel.
struct XsShape {
  int T, TL, KS, U, NG;
  size_t lds;
};
XsShape xs_shape(int M, int tiles, int K, int R) {
  XsShape sh{0, 0, 0, 0, 0, 0};
  const int G = K / kGroup;
  if (M < 3 || M > 16 || K % kGroup != 0 || G < 2) return sh;
  int T = (tiles + 255) / 256;
  if (T < 2) return sh;                          // one tile a workgroup: nothing to share
  if (M <= 4 && T < 4) return sh;                // few rows: the per-wave kernel is faster
  int TL = 1;
  if (T <= 8 / R) TL = T; else while (TL < T && TL < 4 / R) TL *= 2;
  auto ng_ok = [](int ng) { return ng == 2 || ng == 4 || ng == 8 || ng == 16; };
  int KS = 1;
  while (KS * 2 * TL <= 16) KS *= 2;
  while (KS > 1 && (G % KS != 0 || !ng_ok(G / KS))) KS /= 2;
  const int NG = G / KS;
  if (G % KS != 0 || !ng_ok(NG)) return sh;
  const size_t lds = (size_t)G * 4096 + (R == 1 ? (size_t)G * 64 : 0) + (size_t)TL * KS * R * 1024;
  if (lds > 160 * 1024) return sh;
  sh.T = T;
  sh.TL = TL;
  sh.KS = KS;
  sh.U = (T + TL - 1) / TL;
  sh.NG = NG;
  sh.lds = lds;
  return sh;
}

template <bool ASYM, int NG, int R, bool TILED, bool SWIGLU>
void launch_xs_t(const XsShape& sh, int blocks, const void* x, int M, const void* w, const void* s,
                 const void* z, int N, int K, void* y, hipStream_t stream) {
  hipLaunchKernelGGL((qgemv_xs_kernel<ASYM, NG, R, TILED, SWIGLU>), dim3(blocks),
                     dim3(64 * sh.TL * sh.KS), sh.lds, stream, (const uint16_t*)x, M,
                     (const uint32_t*)w, (const uint16_t*)s, (const uint16_t*)z, N, K, sh.KS, sh.TL,
                     sh.T, sh.U, (uint16_t*)y, 0x000F000Fu, ASYM ? 0x43004300u : 0x43084308u);
}

// The x-shared GEMV (or SwiGLU GEMV over [W_gate; W_up], N = 2I rows) when
// its shape applies; hipErrorNotSupported otherwise.
template <bool TILED, bool SWIGLU>
hipError_t launch_xs(bool asym, const void* x, int M, const void* w, const void* s, const void* z,
                     int N, int K, void* y, hipStream_t stream) {
  constexpr int R = SWIGLU ? 2 : 1;
  const int tiles = SWIGLU ? (N / 2 + 15) / 16 : (N + 15) / 16;
  const XsShape sh = xs_shape(M, tiles, K, R);
  if (!sh.T) return hipErrorNotSupported;
  const int blocks = (tiles + sh.T - 1) / sh.T;
#define QG_XS(A, NGV) launch_xs_t<A, NGV, R, TILED, SWIGLU>(sh, blocks, x, M, w, s, z, N, K, y, stream)
  if (asym) {
    switch (sh.NG) {
      case 2: QG_XS(true, 2); break;
      case 4: QG_XS(true, 4); break;
      case 8: QG_XS(true, 8); break;
      case 16: QG_XS(true, 16); break;
      default: return hipErrorNotSupported;
    }
  } else {
    switch (sh.NG) {
      case 2: QG_XS(false, 2); break;
      case 4: QG_XS(false, 4); break;
      case 8: QG_XS(false, 8); break;
      case 16: QG_XS(false, 16); break;
      default: return hipErrorNotSupported;
    }
  }
#undef QG_XS
  return hipGetLastError();
}

// Launch shape (measured on MI355X for the Llama-3-8B decode shapes): about
// 1024 waves in the grid (4 per CU) with 8-16 groups per wave -- KS K-slices
// per 16-row tile -- and 2 row tiles per workgroup once there are more than
// 1024 tiles.  Deeper rings and more waves measured slower: the kernels are
// bound by the latency of their prologue and epilogue, not by the bytes in
// flight.
template <bool ASYM, bool XLDS, bool SVEC, bool TILED>
hipError_t launch_t(const void* x, int M, const void* w, const void* s, const void* z, int N,
                    int K, void* y, hipStream_t stream) {
  const int G = K / kGroup;
  const int tiles = (N + 15) / 16;
  int ks = (1024 + tiles - 1) / tiles;
  ks = ks < 1 ? 1 : (ks > 16 ? 16 : ks);
  while (ks < 16 && (G + ks - 1) / ks > 16) ++ks;
  if (ks > G) ks = G;
  int rw = tiles > 1024 ? 2 : 1;
  if (rw * ks > 16) rw = 1;
  const size_t x_bytes = XLDS ? (size_t)M * K * 2 + (((size_t)M * G * 4 + 15) & ~(size_t)15) : 0;
  auto lds_for = [&](int r) {
    const size_t sc = (size_t)G * r * 16 * 2 * sizeof(float);
    const size_t red = (size_t)r * ks * 4 * 64 * sizeof(float);
    return (x_bytes + sc) > red ? (x_bytes + sc) : red;
  };
  // keep the staged scales within 32 KiB and the workgroup within 64 KiB of LDS
  while (rw > 1 && ((size_t)G * rw * 16 * 8 > 32 * 1024 || lds_for(rw) > 64 * 1024)) --rw;
  const int blocks = (tiles + rw - 1) / rw;
  hipLaunchKernelGGL((qgemv_kernel<ASYM, XLDS, SVEC, TILED>), dim3(blocks), dim3(64 * rw * ks), lds_for(rw),
                     stream, (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,
                     (const uint16_t*)z, N, K, ks, rw, (uint16_t*)y, 0x000F000Fu,
                     ASYM ? 0x43004300u : 0x43084308u);
  return hipGetLastError();
}

template <bool ASYM, int NG, int MM, bool TILED>
hipError_t launch_wave_t(const void* x, int M, const void* w, const void* s, const void* z, int N,
                         int K, void* y, hipStream_t stream) {
  const int G = K / kGroup;
  const int ks = G / NG;
  const int tiles = (N + 15) / 16;
  const size_t lds = (size_t)ks * (MM * NG * 256 + 1024);
  hipLaunchKernelGGL((qgemv_wave_kernel<ASYM, NG, MM, TILED>), dim3(tiles), dim3(64 * ks), lds, stream,
                     (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,
                     (const uint16_t*)z, N, K, ks, (uint16_t*)y, 0x000F000Fu,
                     ASYM ? 0x43004300u : 0x43084308u);
  return hipGetLastError();
}

// Per-wave kernel for M <= 4 when K splits into slices of NG groups with at
// most 16 slices (G % NG == 0, G / NG <= 16) and the LDS fits.
template <bool TILED>
hipError_t launch_wave(bool asym, int ng, const void* x, int M, const void* w, const void* s,
                       const void* z, int N, int K, void* y, hipStream_t stream) {
  if (M == 1) {
    if (ng == 4) return asym ? launch_wave_t<true, 4, 1, TILED>(x, M, w, s, z, N, K, y, stream)
                             : launch_wave_t<false, 4, 1, TILED>(x, M, w, s, z, N, K, y, stream);
    if (ng == 16) return asym ? launch_wave_t<true, 16, 1, TILED>(x, M, w, s, z, N, K, y, stream)
                              : launch_wave_t<false, 16, 1, TILED>(x, M, w, s, z, N, K, y, stream);
    return asym ? launch_wave_t<true, 8, 1, TILED>(x, M, w, s, z, N, K, y, stream)
                : launch_wave_t<false, 8, 1, TILED>(x, M, w, s, z, N, K, y, stream);
  }
  if (ng == 4) return asym ? launch_wave_t<true, 4, 4, TILED>(x, M, w, s, z, N, K, y, stream)
                           : launch_wave_t<false, 4, 4, TILED>(x, M, w, s, z, N, K, y, stream);
  return asym ? launch_wave_t<true, 8, 4, TILED>(x, M, w, s, z, N, K, y, stream)
              : launch_wave_t<false, 8, 4, TILED>(x, M, w, s, z, N, K, y, stream);
}

// Groups per wave for the per-wave kernel (0: not applicable).  Measured on
// MI355X for the Llama-3-8B decode layer (four projections back to back in
// a graph): 4 groups per wave wherever K fits 16 slices of 4 (more waves in
// flight: at M = 4 the layer 2.81 -> 2.90 TB/s; at M = 1 the 4096 x 4096
// GEMV 4.12 -> 3.91 us, QKV 0.1 - 0.2 us faster, and with the gate+up
// projection on it too the layer 0.2 - 0.3 us faster in six A/B pairs), else
// 8; 16 (M = 1 only: 128 VGPRs) when K is too long for 16 slices of 8.
int pick_wave_ng(int M, int N, int K) {
  const int G = K / kGroup;
  if (M > 4 || G % 4 != 0) return 0;
  const int mm = M == 1 ? 1 : 4;
  auto fits = [&](int ng) {
    const int ks = G / ng;
    return G % ng == 0 && ks <= 16 && (size_t)ks * (mm * ng * 256 + 1024) <= 160 * 1024;
  };
  if (fits(4)) return 4;
  if (fits(8)) return 8;
  if (fits(4)) return 4;
  if (M == 1 && fits(16)) return 16;
  return 0;
}

// W4A16 product for quantization groups other than 128 codes: g = 32, 64 or
// a multiple of 128 dividing K (《第 1 章：推理加速全景》 section 4.1: per-group
// granularity from 32 to 128 elements).  The codes are unpacked in natural k
// order (the 4 x 4 transpose of the 16-row kernel), so MFMA i of a 128-code
// block covers k = 32 i .. 32 i + 31: a group of 32 is one MFMA, a group of
// 64 two, a group of 128 t the 4 t MFMAs of t blocks; each group is flushed
// as y += s (acc - c sum_x) with its own scale and zero point.  Workgroup =
// one 16-channel tile x one block of up to 16 rows of x (blockIdx.y), KS
// waves over K-slices of NB blocks of 128 codes; the x pieces come straight
// from the caches, the weights one block ahead.  Any M (the prefill GEMM's
// fallback for these group sizes as well as the GEMV's).  Either code layout.
template <bool ASYM, int GPB, bool TILED>   // groups per 128-code block: 4, 2 or 1
__global__ __launch_bounds__(1024) void qgemv_groups_kernel(const uint16_t* __restrict__ x, int M,
                                                            const uint32_t* __restrict__ w,
                                                            const uint16_t* __restrict__ s16,
                                                            const uint16_t* __restrict__ z16,
                                                            int N, int K, int gsize, int KS,
                                                            int NB, uint16_t* __restrict__ y,
                                                            uint32_t mask, uint32_t cmag) {
  extern __shared__ float4 lds4[];
  float* red = reinterpret_cast<float*>(lds4);
  const int lane = threadIdx.x & 63;
  const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int n = blockIdx.x * 16 + li;
  const int m0 = blockIdx.y * 16;
  const int G128 = K / kGroup;
  const int Gs = K / gsize;                      // scale groups per row
  const int b0 = kw * NB;
  const int b1 = b0 + NB < G128 ? b0 + NB : G128;
  using WL = WLayout<TILED>;
  // rows m0 + li >= M and channels n >= N read as zero (outside the ranges)
  const int mrows = M - m0 < 16 ? M - m0 : 16;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc_g(x + (int64_t)m0 * K, (int64_t)mrows * K * 2);
  const uint32_t xoff = li < mrows ? (uint32_t)(li * K + 8 * lg) * 2 : 0x80000000u;
  const __amdgpu_buffer_rsrc_t wres = make_rsrc_g(w, WL::bytes(N, K));
  const uint32_t woff = WL::lane_off(blockIdx.x, li, lg, N, K);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc_g(s16, (int64_t)N * Gs * 2);
  const __amdgpu_buffer_rsrc_t zres = make_rsrc_g(z16, ASYM ? (int64_t)N * Gs * 2 : 0);
  const uint32_t srow = n < N ? (uint32_t)n * (uint32_t)Gs * 2u : 0x80000000u;

  struct Block {
    u32x4 wv, xv[4];
    uint32_t sv[GPB], zv[GPB];
  };
  auto load = [&](int b, Block& B) {
    const bool ok = b < b1;
    B.wv = WL::load(wres, ok ? woff : 0x80000000u, b * WL::kGroupStride);
#pragma unroll
    for (int i = 0; i < 4; ++i) B.xv[i] = bload(xres, ok ? xoff : 0x80000000u, b * 256 + i * 64);
#pragma unroll
    for (int h = 0; h < GPB; ++h) {
      const int gi = GPB == 1 ? (int)((int64_t)b * kGroup / gsize) : b * GPB + h;
      const uint32_t so = ok && srow != 0x80000000u ? srow + (uint32_t)gi * 2u : 0x80000000u;
      B.sv[h] = __builtin_amdgcn_raw_buffer_load_b16(sres, so, 0, 0);
      B.zv[h] = ASYM ? __builtin_amdgcn_raw_buffer_load_b16(zres, so, 0, 0) : 0u;
    }
  };
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float yacc[4] = {0.f, 0.f, 0.f, 0.f};
  Block cur, nxt;
  load(b0, cur);
  for (int b = b0; b < b1; ++b) {
    load(b + 1, nxt);
    const u32x4 wt = transpose_rows(cur.wv);
    f32x4 acc[4], sacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 a = as_bf16x8(cur.xv[i]);
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(unpack_word_nat(wt[i], mask, cmag)),
                                                       z4, 0, 0, 0);
      sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(ones), z4, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < GPB; ++h) {
      const float sc = f16_bits_to_f32((uint16_t)cur.sv[h]);
      const float cc = ASYM ? 128.f + f16_bits_to_f32((uint16_t)cur.zv[h]) : 136.f;
      constexpr int kPer = 4 / GPB;              // MFMAs of one group inside the block
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = 0.f, sx = 0.f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          a += acc[h * kPer + i][r];
          sx += sacc[h * kPer + i][r];
        }
        yacc[r] = __builtin_fmaf(sc, __builtin_fmaf(-cc, sx, a), yacc[r]);
      }
    }
    cur = nxt;
  }

  // sum the K-slices: red[kw][r][lane]; lane (li, lg) of the first wave
  // writes y[m0 + 4 lg + r][n]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(kw * 4 + r) * 64 + lane] = yacc[r];
  __syncthreads();
  if (kw == 0 && n < N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 4 * lg + r;
      if (m < M) {
        float v = 0.f;
        for (int k2 = 0; k2 < KS; ++k2) v += red[(k2 * 4 + r) * 64 + lane];
        QG_DEBUG_STORE((int64_t)m * N + n, v);
        y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

template <bool TILED>
hipError_t launch_groups_t(bool asym, const void* x, int M, const void* w, const void* s,
                           const void* z, int N, int K, int gsize, void* y, hipStream_t stream) {
  const int G128 = K / kGroup;
  const int nb = (G128 + 7) / 8;                 // at most 8 K-slices
  const int ks = (G128 + nb - 1) / nb;
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
  const size_t lds = (size_t)ks * 4 * 64 * sizeof(float);
  const int gpb = gsize == 32 ? 4 : (gsize == 64 ? 2 : 1);
  const uint32_t mask = 0x000F000Fu, cmag = asym ? 0x43004300u : 0x43084308u;
#define QG_GROUPS(A, GP)                                                                          \
  hipLaunchKernelGGL((qgemv_groups_kernel<A, GP, TILED>), grid, dim3(64 * ks), lds, stream,         \
                     (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,                  \
                     (const uint16_t*)z, N, K, gsize, ks, nb, (uint16_t*)y, mask, cmag)
  if (asym) {
    if (gpb == 4) QG_GROUPS(true, 4); else if (gpb == 2) QG_GROUPS(true, 2); else QG_GROUPS(true, 1);
  } else {
    if (gpb == 4) QG_GROUPS(false, 4); else if (gpb == 2) QG_GROUPS(false, 2); else QG_GROUPS(false, 1);
  }
#undef QG_GROUPS
  return hipGetLastError();
}

// Groups per wave of the SwiGLU wave kernel (0: not applicable): the
// per-wave GEMV's choice with at most 16 K-slices and the LDS within 160
// KiB; two weight tiles per wave, so 4 groups (8 for M = 1 when K needs
// them; 16 only for M = 1).
int swiglu_wave_ng(int M, int K) {
  const int G = K / kGroup;
  if (G % 4 != 0) return 0;
  const int mm = M == 1 ? 1 : 4;
  auto fits = [&](int ng) {
    const int ks = G / ng;
    return G % ng == 0 && ks <= 16 && (size_t)ks * (mm * ng * 256 + 2048) <= 160 * 1024;
  };
  if (fits(4)) return 4;
  if (fits(8)) return 8;
  if (M == 1 && fits(16)) return 16;
  return 0;
}

// SwiGLU GEMV launch: the x-shared kernel with the gate / up tile pair where
// its shape applies (3 <= M <= 16), else M <= 4 on the per-wave kernel (gate
// and up tiles in every wave, NG groups per wave so that K splits into at
// most 16 slices) and 5 <= M <= 16 on the 16-row kernel with the tile pair.
// Returns hipErrorInvalidValue for shapes none covers (checked by the
// caller).
template <bool TILED>
hipError_t launch_swiglu_t(bool asym, const void* x, int M, const void* w, const void* s,
                           const void* z, int N2, int K, void* h, hipStream_t stream) {
  const int G = K / kGroup;
  const int I = N2 / 2;
  const int tiles = (I + 15) / 16;
  const uint32_t mask = 0x000F000Fu, cmag = asym ? 0x43004300u : 0x43084308u;
  if (M >= 3) {
    const hipError_t e = launch_xs<TILED, true>(asym, x, M, w, s, z, N2, K, h, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (M <= 4) {
    const int ng = swiglu_wave_ng(M, K);
    if (!ng) return hipErrorInvalidValue;
    const int ks = G / ng;
    const int mm = M == 1 ? 1 : 4;
    const size_t lds = (size_t)ks * (mm * ng * 256 + 2048);
#define QG_SWIGLU_WAVE(A, NGV, MMV)                                                              \
  hipLaunchKernelGGL((qgemv_swiglu_kernel<A, NGV, MMV, TILED>), dim3(tiles), dim3(64 * ks), lds, \
                     stream, (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,       \
                     (const uint16_t*)z, I, K, ks, (uint16_t*)h, mask, cmag)
    if (asym) {
      if (mm == 1) {
        if (ng == 4) QG_SWIGLU_WAVE(true, 4, 1); else if (ng == 8) QG_SWIGLU_WAVE(true, 8, 1);
        else QG_SWIGLU_WAVE(true, 16, 1);
      } else {
        if (ng == 4) QG_SWIGLU_WAVE(true, 4, 4); else QG_SWIGLU_WAVE(true, 8, 4);
      }
    } else {
      if (mm == 1) {
        if (ng == 4) QG_SWIGLU_WAVE(false, 4, 1); else if (ng == 8) QG_SWIGLU_WAVE(false, 8, 1);
        else QG_SWIGLU_WAVE(false, 16, 1);
      } else {
        if (ng == 4) QG_SWIGLU_WAVE(false, 4, 4); else QG_SWIGLU_WAVE(false, 8, 4);
      }
    }
#undef QG_SWIGLU_WAVE
    return hipGetLastError();
  }
  if (G % 4 != 0 || G / 4 > 16) return hipErrorInvalidValue;
  const int ks = G / 4;
  const size_t lds = (size_t)ks * 2 * 4 * 64 * sizeof(float);
  if (asym)
    hipLaunchKernelGGL((qgemv_m16_kernel<true, 4, 2, TILED, true>), dim3(tiles), dim3(64 * ks), lds,
                       stream, (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,
                       (const uint16_t*)z, N2, K, ks, (uint16_t*)h, mask, cmag);
  else
    hipLaunchKernelGGL((qgemv_m16_kernel<false, 4, 2, TILED, true>), dim3(tiles), dim3(64 * ks),
                       lds, stream, (const uint16_t*)x, M, (const uint32_t*)w, (const uint16_t*)s,
                       (const uint16_t*)z, N2, K, ks, (uint16_t*)h, mask, cmag);
  return hipGetLastError();
}

}  // namespace

// LDS per workgroup: x (M*K*2 bytes when staged, <= 48 KiB) + (s, c) pairs
// (G * RW * 128 bytes <= 32 KiB for RW > 1; G * 128 bytes = 64 KiB at the
// API's K limit of 65536 with RW = 1, where x is never staged).
namespace {
template <bool TILED>
hipError_t launch_qgemv_t(bool asym, const void* x, int64_t M, const void* wcodes,
                          const void* wscales, const void* wzeros, int64_t N, int64_t K, void* y,
                          hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  const int G = k / kGroup;
  if (m >= 3) {
    const hipError_t e = launch_xs<TILED, false>(asym, x, m, wcodes, wscales, wzeros, n, k, y, stream);
    if (e != hipErrorNotSupported) return e;
  }
  const int ng = pick_wave_ng(m, n, k);
  if (ng) return launch_wave<TILED>(asym, ng, x, m, wcodes, wscales, wzeros, n, k, y, stream);
  if (m > 4) {
    const int ng16 = pick_m16_ng(k);
    if (ng16) return launch_m16<TILED>(asym, ng16, x, m, wcodes, wscales, wzeros, n, k, y, stream);
  }
  // staged x must leave room for the (s, c) pairs of one row tile in 64 KiB
  const bool xlds = M * K * 2 <= kXldsMaxBytes &&
                    M * K * 2 + M * G * 4 + 16 + (int64_t)G * 128 <= 64 * 1024;
  // 16-byte scale loads need whole 16-byte pieces per row (G % 8 == 0); the
  // cache path stages scales with the generic loop
  const bool svec = (G & 7) == 0;
  if (asym) {
    if (!xlds) return launch_t<true, false, false, TILED>(x, m, wcodes, wscales, wzeros, n, k, y, stream);
    return svec ? launch_t<true, true, true, TILED>(x, m, wcodes, wscales, wzeros, n, k, y, stream)
                : launch_t<true, true, false, TILED>(x, m, wcodes, wscales, wzeros, n, k, y, stream);
  }
  if (!xlds) return launch_t<false, false, false, TILED>(x, m, wcodes, wscales, wzeros, n, k, y, stream);
  return svec ? launch_t<false, true, true, TILED>(x, m, wcodes, wscales, wzeros, n, k, y, stream)
              : launch_t<false, true, false, TILED>(x, m, wcodes, wscales, wzeros, n, k, y, stream);
}

}  // namespace

namespace {

// One lane per 16-byte piece of the tiled output: piece q of tile t, group g,
// quarter b, row r is the 16 bytes at row t*16 + r, byte 64 g + 16 b of the
// canonical codes (zero for rows past N).  64 consecutive lanes write one
// contiguous 1 KiB block.
__global__ __launch_bounds__(256) void tile_codes_kernel(const u32x4* __restrict__ src, int N,
                                                         int K, int64_t pieces,
                                                         u32x4* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= pieces) return;
  const int G = K / kGroup;
  const int r = (int)(q & 15), b = (int)((q >> 4) & 3);
  const int64_t tg = q >> 6;
  const int g = (int)(tg % G);
  const int64_t t = tg / G;
  const int64_t n = t * 16 + r;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (n < N) v = src[(n * (K / 2) + g * 64 + b * 16) / 16];
  dst[q] = v;
}

}  // namespace

QG_DEBUG_TU_SETTER(debug_set_gemv)

hipError_t launch_tile_gemv_codes(const void* codes, int64_t N, int64_t K, void* tiled,
                                  hipStream_t stream) {
  const int64_t pieces = (N + 15) / 16 * 16 * (K / 2) / 16;
  hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                     stream, (const u32x4*)codes, (int)N, (int)K, pieces, (u32x4*)tiled);
  return hipGetLastError();
}

hipError_t launch_qgemv(bool asym, bool tiled, const void* x, int64_t M, const void* wcodes,
                        const void* wscales, const void* wzeros, int64_t N, int64_t K, void* y,
                        hipStream_t stream) {
  return tiled ? launch_qgemv_t<true>(asym, x, M, wcodes, wscales, wzeros, N, K, y, stream)
               : launch_qgemv_t<false>(asym, x, M, wcodes, wscales, wzeros, N, K, y, stream);
}

bool w4a16_group_supported(int64_t K, int64_t group) {
  if (group <= 0 || K % group != 0 || K % kGroup != 0) return false;
  return group == 32 || group == 64 || group % kGroup == 0;
}

hipError_t launch_w4a16_groups(bool asym, bool tiled, const void* x, int64_t M,
                               const void* wcodes, const void* wscales, const void* wzeros,
                               int64_t N, int64_t K, int64_t group, void* y, hipStream_t stream) {
  return tiled ? launch_groups_t<true>(asym, x, (int)M, wcodes, wscales, wzeros, (int)N, (int)K,
                                       (int)group, y, stream)
               : launch_groups_t<false>(asym, x, (int)M, wcodes, wscales, wzeros, (int)N, (int)K,
                                        (int)group, y, stream);
}

bool qgemv_swiglu_supported(int64_t M, int64_t K) {
  const int G = (int)(K / kGroup);
  if (M <= 4) return swiglu_wave_ng((int)M, (int)K) != 0;
  return G % 4 == 0 && G / 4 <= 16;
}

hipError_t launch_qgemv_swiglu(bool asym, bool tiled, const void* x, int64_t M,
                               const void* wcodes, const void* wscales, const void* wzeros,
                               int64_t N2, int64_t K, void* h, hipStream_t stream) {
  return tiled ? launch_swiglu_t<true>(asym, x, (int)M, wcodes, wscales, wzeros, (int)N2, (int)K,
                                       h, stream)
               : launch_swiglu_t<false>(asym, x, (int)M, wcodes, wscales, wzeros, (int)N2, (int)K,
                                        h, stream);
}

}  // namespace qg
