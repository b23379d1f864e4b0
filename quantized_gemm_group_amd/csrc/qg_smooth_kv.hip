// Channel statistics, SmoothQuant factors, static per-channel scales and the
// FP8 E4M3 KV-cache store.
//
// SmoothQuant (《第 1 章：推理加速全景》 section 4.3; 《推理优化与量化算子深度技术调研》
// section 1.5): s_j = max|X_j|^alpha / max|W_j|^(1-alpha) from per-channel
// maxima of calibration activations and of the weights; the folded operands
// are quantized by the group quantizers (qg_quant.hip) with the factors
// applied on load.
//
// KV cache (《推理优化与量化算子深度技术调研》 section 1.6; 《量化与加速》 KV-cache
// section): each new token's keys or values are quantized to E4M3, per token
// and head (scale = absmax over the head dimension / 448) or with static
// per-channel scales, and written into a paged cache at the token's slot.
//
// All kernels here are HBM bound (one read of the operand, at most one byte
// written per element).

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

// ------------------------------------------------------------ channel absmax

// Grid: x = strips of 512 columns (64 lanes x one 8-element vec), y = chunks
// of rows.  The 4 waves of a workgroup walk the rows r0 + w, r0 + w + 4, ...
// of their chunk with 8 rows per wave in flight.  |x| is compared as its IEEE
// bit pattern: for non-negative values the integer order is the numeric order
// (and a NaN, sign cleared, sorts above every number, so it propagates).  The
// waves combine through LDS; one lane per column folds the chunk's maximum
// into the output with an integer atomic max.
constexpr int kAbsWaves = 4;
constexpr int kAbsUnroll = 8;

template <bool BF16>
__global__ __launch_bounds__(64 * kAbsWaves) void channel_absmax_kernel(
    const void* __restrict__ src, int64_t rows, int64_t kvecs, int64_t chunk,
    uint32_t* __restrict__ out) {
  __shared__ uint32_t red[kAbsWaves - 1][8 * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t cv = (int64_t)blockIdx.x * 64 + lane;
  const int64_t r0 = (int64_t)blockIdx.y * chunk;
  const int64_t r1 = r0 + chunk < rows ? r0 + chunk : rows;
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (cv < kvecs) {
    for (int64_t r = r0 + w; r < r1; r += kAbsWaves * kAbsUnroll) {
      if constexpr (BF16) {
        u32x4 d[kAbsUnroll];
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u) {
          const int64_t rr = r + u * kAbsWaves;
          d[u] = rr < r1 ? reinterpret_cast<const u32x4*>(src)[rr * kvecs + cv] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = d[u][e] & 0x7fffu, hi = (d[u][e] >> 16) & 0x7fffu;
            m[2 * e] = m[2 * e] > lo ? m[2 * e] : lo;
            m[2 * e + 1] = m[2 * e + 1] > hi ? m[2 * e + 1] : hi;
          }
      } else {
        u32x4 d[kAbsUnroll][2];
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u) {
          const int64_t rr = r + u * kAbsWaves;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            d[u][h] = rr < r1 ? reinterpret_cast<const u32x4*>(src)[2 * (rr * kvecs + cv) + h]
                              : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t a = d[u][e >> 2][e & 3] & 0x7fffffffu;
            m[e] = m[e] > a ? m[e] : a;
          }
      }
    }
  }
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] <<= 16;    // bf16 magnitude -> fp32 bits, exact
  }
  if (w > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[w - 1][e * 64 + lane] = m[e];
  }
  __syncthreads();
  if (w == 0 && cv < kvecs) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t v = m[e];
#pragma unroll
      for (int q = 0; q < kAbsWaves - 1; ++q) v = v > red[q][e * 64 + lane] ? v : red[q][e * 64 + lane];
      atomicMax(out + cv * 8 + e, v);
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ------------------------------------------------------------ small vectors

// s_j = a^alpha / w^(1 - alpha) in fp64, rounded once to fp32; 1 where a
// statistic is zero (or not a number) or the factor is not a positive normal
// fp32 value.
__global__ __launch_bounds__(256) void smooth_scales_kernel(const float* __restrict__ a,
                                                            const float* __restrict__ w,
                                                            double alpha, int64_t n,
                                                            float* __restrict__ s) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const double av = a[i], wv = w[i];
  float r = 1.f;
  if (av > 0.0 && wv > 0.0) {
    const double v = pow(av, alpha) / pow(wv, 1.0 - alpha);
    const float f = (float)v;
    if (f >= 1.17549435e-38f && f <= 3.40282347e38f) r = f;
  }
  s[i] = r;
}

// Static scales from calibration maxima: absmax / qmax (one fp32 division),
// 1 where that is zero.
__global__ __launch_bounds__(256) void channel_scales_kernel(const float* __restrict__ a,
                                                             float qmax, int64_t n,
                                                             float* __restrict__ s) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = a[i] / qmax;
  s[i] = v == 0.f ? 1.f : v;
}

// ------------------------------------------------------------ KV-cache store

template <bool BF16>
__device__ __forceinline__ void load8(const void* src, int64_t vec, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 w = reinterpret_cast<const u32x4*>(src)[vec];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(src) + 2 * vec;
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// One segment of P = 2^p_log2 lanes per (token, head), lane j of it holding
// elements 8 j .. 8 j + 7 of the head (j < D / 8; the other lanes of the
// segment only join the reduction with zeros); 64 / P segments per wave.
// Per token (PER_CHANNEL false): the segment's absmax gives the scale,
// absmax / 448, 1 when zero, so |x / s| <= 448 (1 + 2^-23), which rounds to
// 448: the conversion never leaves the format's range.  Per channel: x is
// divided by its static scale and clamped to +-448 first, which is the
// saturating encoding.  The codes of token t go to slot slot_mapping[t];
// slots outside [0, num_slots) are skipped.
template <bool BF16, bool PER_CHANNEL>
__global__ __launch_bounds__(256) void kv_store_kernel(const void* __restrict__ src, int nseg,
                                                       int heads, int dvecs, int p_log2,
                                                       const int64_t* __restrict__ slots,
                                                       int64_t num_slots,
                                                       const float* __restrict__ cscale,
                                                       uint8_t* __restrict__ cache,
                                                       float* __restrict__ cache_scales) {
  const int lane = threadIdx.x & 63;
  const int seg = ((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * (64 >> p_log2) + (lane >> p_log2);
  const int j = lane & ((1 << p_log2) - 1);
  const bool live = seg < nseg;
  const bool active = live && j < dvecs;
  const int t = live ? seg / heads : 0;
  const int h = live ? seg - t * heads : 0;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t slot = -1;
  if (live) slot = slots[t];
  if (active) load8<BF16>(src, (int64_t)seg * dvecs + j, v);
  float s = 1.f;
  if constexpr (!PER_CHANNEL) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(v[i]));
    am = wave_max_seg(am, 1 << p_log2);
    s = am / 448.0f;
    if (s == 0.f) s = 1.f;
    // fl32(x / s) as fl32(x * (1/s)_fp64): exact for a normal fp32 quotient
    // (a quotient of 24-bit significands keeps 2^-49 of relative distance
    // from every fp32 rounding midpoint, the fp64 product errs by < 2^-52);
    // subnormal quotients encode to zero either way
    const double r = 1.0 / (double)s;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)((double)v[i] * r);
  } else if (active) {
    const f32x4* p = reinterpret_cast<const f32x4*>(cscale) + 2 * ((int64_t)h * dvecs + j);
    const f32x4 a = p[0], b = p[1];
    const float c[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_fminf(__builtin_fmaxf(v[i] / c[i], -448.f), 448.f);
  }
  if (active && slot >= 0 && slot < num_slots) {
    uint2 out;
    out.x = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0u, false);
    out.x = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], out.x, true);
    out.y = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0u, false);
    out.y = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], out.y, true);
    const int64_t row = slot * heads + h;
    reinterpret_cast<uint2*>(cache)[row * dvecs + j] = out;
    if constexpr (!PER_CHANNEL) {
      if (j == 0) cache_scales[row] = s;
    }
  }
}

inline unsigned blocks256(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_channel_absmax(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                                 bool accumulate, float* out, hipStream_t stream) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  if (!accumulate) hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks256(K)), dim3(256), 0, stream, o, K);
  const int64_t kvecs = K / 8;
  const int64_t strips = (kvecs + 63) / 64;
  // about 1024 workgroups, at least 32 rows (one full round of loads) each
  int64_t ychunks = (1024 + strips - 1) / strips;
  const int64_t ymax = (rows + kAbsWaves * kAbsUnroll - 1) / (kAbsWaves * kAbsUnroll);
  if (ychunks > ymax) ychunks = ymax;
  if (ychunks > 65535) ychunks = 65535;
  if (ychunks < 1) ychunks = 1;
  const int64_t chunk = (rows + ychunks - 1) / ychunks;
  ychunks = (rows + chunk - 1) / chunk;
  const dim3 grid((unsigned)strips, (unsigned)ychunks);
  if (src_dtype == QG_BF16)
    hipLaunchKernelGGL(channel_absmax_kernel<true>, grid, dim3(64 * kAbsWaves), 0, stream, src,
                       rows, kvecs, chunk, o);
  else
    hipLaunchKernelGGL(channel_absmax_kernel<false>, grid, dim3(64 * kAbsWaves), 0, stream, src,
                       rows, kvecs, chunk, o);
  return hipGetLastError();
}

hipError_t launch_smooth_scales(const float* act_absmax, const float* w_absmax, float alpha,
                                int64_t K, float* smooth, hipStream_t stream) {
  hipLaunchKernelGGL(smooth_scales_kernel, dim3(blocks256(K)), dim3(256), 0, stream, act_absmax,
                     w_absmax, (double)alpha, K, smooth);
  return hipGetLastError();
}

hipError_t launch_channel_scales(const float* absmax, int64_t n, float qmax, float* scales,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(channel_scales_kernel, dim3(blocks256(n)), dim3(256), 0, stream, absmax,
                     qmax, n, scales);
  return hipGetLastError();
}

hipError_t launch_kv_cache_store(const void* x, qg_dtype x_dtype, int64_t tokens, int64_t heads,
                                 int64_t head_dim, const int64_t* slot_mapping, int64_t num_slots,
                                 const float* channel_scales, void* cache_codes,
                                 float* cache_scales, hipStream_t stream) {
  const int dvecs = (int)(head_dim / 8);
  int p_log2 = 0;
  while ((1 << p_log2) < dvecs) ++p_log2;
  const int nseg = (int)(tokens * heads);
  const int seg_per_block = 4 * (64 >> p_log2);
  const dim3 grid((unsigned)((nseg + seg_per_block - 1) / seg_per_block));
  uint8_t* cc = reinterpret_cast<uint8_t*>(cache_codes);
  const int hh = (int)heads;
  if (x_dtype == QG_BF16) {
    if (channel_scales)
      hipLaunchKernelGGL((kv_store_kernel<true, true>), grid, dim3(256), 0, stream, x, nseg, hh,
                         dvecs, p_log2, slot_mapping, num_slots, channel_scales, cc, cache_scales);
    else
      hipLaunchKernelGGL((kv_store_kernel<true, false>), grid, dim3(256), 0, stream, x, nseg, hh,
                         dvecs, p_log2, slot_mapping, num_slots, channel_scales, cc, cache_scales);
  } else {
    if (channel_scales)
      hipLaunchKernelGGL((kv_store_kernel<false, true>), grid, dim3(256), 0, stream, x, nseg, hh,
                         dvecs, p_log2, slot_mapping, num_slots, channel_scales, cc, cache_scales);
    else
      hipLaunchKernelGGL((kv_store_kernel<false, false>), grid, dim3(256), 0, stream, x, nseg, hh,
                         dvecs, p_log2, slot_mapping, num_slots, channel_scales, cc, cache_scales);
  }
  return hipGetLastError();
}

}  // namespace qg
